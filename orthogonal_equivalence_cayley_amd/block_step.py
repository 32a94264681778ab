"""One training step over the linears of a LLaMA-style block, through libpoetx.

A step is the whole hot path over one batch: the batched build of every
layer's blocks (both sides), the forward of every layer (keeping Wa and the
permuted input U), the activation-side backward of every layer, and one
batched chain rule through the parameterisation of all layers. The layers a
block computes without depending on each other (q, k, v read the same input;
gate and up too) may run on two HIP streams of default priority, each group of
layers waiting for the one before it (the backward walks the groups in
reverse). The benchmark times this sequence and the full-size parity test
checks its outputs, so both exercise the same calls, launches and streams.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import poetx as _px
from .layer import PoetxLayer, build_many, param_grad_many

# groups of layers with no data dependence between them inside a block
_INDEPENDENT = ({"q", "k", "v"}, {"gate", "up"})


def layer_groups(names: Sequence[str]):
    """Consecutive layers that may run concurrently: [[q, k, v], [o], [gate, up],
    [down]] for a LLaMA block; a layer with no partner forms its own group."""
    groups = []
    for li, name in enumerate(names):
        g = next((s for s in _INDEPENDENT if name in s), None)
        if groups and g is not None and names[groups[-1][-1]] in g:
            groups[-1].append(li)
        else:
            groups.append([li])
    return groups


class BlockStep:
    """Device state of every layer of a block and the step that runs over it.

    layer_inputs: objects with spec (name, m, n, bsz_R, bsz_P), W0, theta_R,
    theta_P, pi_R, pi_P, X and G_Y (host arrays); they are copied to the device
    once. backward=False runs build + forward only. The frozen weight is kept
    with its transpose by default ("dense_t"), so both of its products read it
    K-contiguous."""

    def __init__(self, layer_inputs, k: int, dtype: str = "bf16", *, backward: bool = True,
                 streams: int = 2, weight: str = "dense_t", cayley: str = "neumann",
                 fold: str = "none", index: str = "separate", series: str = "chain",
                 xmem: bool = False):
        if streams not in (1, 2):
            raise ValueError("streams must be 1 or 2")
        self.k, self.dtype, self.backward, self.xmem = k, dtype, backward, xmem
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(tdt).cuda()
        self.names = [inp.spec.name for inp in layer_inputs]
        self.layers, self.bufs = [], []
        for inp in layer_inputs:
            sp = inp.spec
            T = inp.X.shape[0]
            L = PoetxLayer(sp.m, sp.n, sp.bsz_R, sp.bsz_P, k, dtype=dtype, weight=weight,
                           cayley=cayley, fold=fold, index=index, series=series)
            L.set_weight(dev(inp.W0), torch.from_numpy(inp.pi_R), torch.from_numpy(inp.pi_P))
            L.set_theta(torch.from_numpy(inp.theta_R), torch.from_numpy(inp.theta_P))
            b = dict(X=dev(inp.X), Y=torch.empty(T, sp.m, dtype=tdt, device="cuda"),
                     Wa=None if xmem else torch.empty(T, sp.m, dtype=tdt, device="cuda"),
                     U=torch.empty(T, sp.n, dtype=tdt, device="cuda"))
            if backward:
                b.update(G=dev(inp.G_Y), GX=torch.empty(T, sp.n, dtype=tdt, device="cuda"),
                         g=[torch.empty(L.nparam[s], dtype=torch.float32, device="cuda")
                            for s in (0, 1)])
            # workspaces are sized once, before any step
            L.workspace(_px.WS_BUILD)
            L.workspace(_px.WS_FORWARD, T)
            if backward:
                L.workspace(_px.WS_BACKWARD, T)
                L._ws_grad(0)
                L._ws_grad(1)
            self.layers.append(L)
            self.bufs.append(b)
        self.groups = layer_groups(self.names)
        self.side: Optional[torch.cuda.Stream] = torch.cuda.Stream() if streams == 2 else None
        self.two_streams = streams == 2 and any(len(g) > 1 for g in self.groups)

    # ------------------------------------------------------------------ schedule
    def _run_groups(self, order, fn, two: bool) -> None:
        main = torch.cuda.current_stream()
        for grp in order:
            if not two or len(grp) == 1:
                for li in grp:
                    fn(li)
                continue
            self.side.wait_stream(main)
            for j, li in enumerate(grp):
                with torch.cuda.stream(main if j % 2 == 0 else self.side):
                    fn(li)
            main.wait_stream(self.side)

    def _fwd(self, li: int) -> None:
        L, b = self.layers[li], self.bufs[li]
        # the input is kept in the permuted order the backward reads it in
        L.forward(b["X"], Y=b["Y"], Wa=b["Wa"], save=not self.xmem, keep_u=True, U=b["U"])

    def _bwd(self, li: int) -> None:
        L, b = self.layers[li], self.bufs[li]
        L.backward_dq(b["X"], b["G"], G_X=b["GX"])

    def step(self, two: Optional[bool] = None) -> None:
        """One pass of the whole path (asynchronous on the current stream)."""
        two = self.two_streams if two is None else (two and self.side is not None)
        build_many(self.layers)
        self._run_groups(self.groups, self._fwd, two)
        if self.backward:
            # activation path layer by layer, then the chain rule through the
            # parameterisation of all layers in one batched call
            self._run_groups([list(reversed(g)) for g in reversed(self.groups)], self._bwd, two)
            param_grad_many(self.layers, [b["g"] for b in self.bufs])

    # ------------------------------------------------------------------ results
    def outputs(self, li: int) -> dict:
        """Device tensors of layer li after a step: Y, Wa (None with xmem), the
        fp32 blocks Q_R and Q_P and, with the backward, G_X and both packed
        parameter gradients."""
        L, b = self.layers[li], self.bufs[li]
        out = dict(Y=b["Y"], Wa=b["Wa"], QR=L.Q32[0], QP=L.Q32[1])
        if self.backward:
            out.update(G_X=b["GX"], g_theta_R=b["g"][0], g_theta_P=b["g"][1])
        return out
