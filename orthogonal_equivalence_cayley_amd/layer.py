"""One POET-X linear layer on the GPU through libpoetx.

Holds the device buffers of one layer (pre-merged weight, permutations, packed
skew parameters, built blocks, workspaces) and calls the C ABI for build,
forward and backward. torch provides memory and the current stream; all
arithmetic runs in libpoetx's HIP kernels.
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import poetx as _px

_TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}
_PX_DTYPE = {"bf16": _px.POETX_BF16, "f32": _px.POETX_FP32}


def build_many(layers) -> None:
    """Build both sides of every layer in one batched call (one launch per
    block-size class instead of one per side and layer)."""
    items = []
    for L in layers:
        items.extend(L.build_items())
    _px.build_orth_batch(items)


def param_grad_many(layers, g_thetas=None):
    """Chain rule through the parameterisation for every layer after
    backward_dq(): both sides of all layers in one batched call. Returns the
    packed gradients [(g_theta_R, g_theta_P), ...]."""
    items, out = [], []
    for i, L in enumerate(layers):
        g = g_thetas[i] if g_thetas is not None else [
            torch.empty(L.nparam[s], dtype=torch.float32, device=L.device) for s in (0, 1)]
        out.append((g[0], g[1]))
        for side in (_px.SIDE_R, _px.SIDE_P):
            items.append((L.plan, side, L.theta[side], L.dQ[side], g[side], L._ws_grad(side)))
    _px.param_grad_batch(items)
    return out


class PoetxLayer:
    def __init__(self, m: int, n: int, bsz_R: Sequence[int], bsz_P: Sequence[int], k: int,
                 dtype: str = "bf16", device: str = "cuda", weight: str = "dense",
                 cayley: str = "neumann", fold: str = "none", index: str = "separate",
                 series: str = "chain"):
        if dtype not in _TORCH_DTYPE:
            raise ValueError(f"dtype must be one of {sorted(_TORCH_DTYPE)}")
        if weight not in ("dense", "dense_t", "int8", "int8_t"):
            raise ValueError("weight must be 'dense', 'dense_t' (kept with its transpose), "
                             "'int8' (POET-XQ) or 'int8_t' (INT8 kept with its transpose)")
        if cayley not in ("neumann", "exact"):
            raise ValueError("cayley must be 'neumann' (truncated series) or 'exact'")
        if fold not in ("none", "weight"):
            raise ValueError("fold must be 'none' (blocks on the activations) or 'weight'")
        if index not in ("separate", "fused"):
            raise ValueError("index must be 'separate' or 'fused' (index maps inside the block products)")
        if series not in ("chain", "ps"):
            raise ValueError("series must be 'chain' (power chain) or 'ps' (Paterson-Stockmeyer)")
        self.fold, self.index, self.series = fold, index, series
        self.m, self.n, self.k, self.dtype = m, n, k, dtype
        self.weight = weight
        self.device = torch.device(device)
        self.tdtype = _TORCH_DTYPE[dtype]
        self.plan = _px.Plan(m, n, bsz_R, bsz_P, k, _PX_DTYPE[dtype],
                             {"dense": _px.WEIGHT_DENSE, "dense_t": _px.WEIGHT_DENSE_T,
                              "int8": _px.WEIGHT_INT8_ROWS, "int8_t": _px.WEIGHT_INT8_ROWS_T}[weight],
                             _px.CAYLEY_EXACT if cayley == "exact" else _px.CAYLEY_NEUMANN,
                             _px.FOLD_WEIGHT if fold == "weight" else _px.FOLD_NONE,
                             _px.INDEX_FUSED if index == "fused" else _px.INDEX_SEPARATE,
                             _px.SERIES_PS if series == "ps" else _px.SERIES_CHAIN)
        self.nparam = (self.plan.param_count(_px.SIDE_R), self.plan.param_count(_px.SIDE_P))
        self.nelem = (self.plan.block_elems(_px.SIDE_R), self.plan.block_elems(_px.SIDE_P))
        self._ws = {}
        self.Wt = None
        self.pi_R = self.pi_P = None
        self.theta = [None, None]
        self.Q32 = [torch.empty(self.nelem[s], dtype=torch.float32, device=self.device) for s in (0, 1)]
        if dtype == "bf16":
            self.Qact = [torch.empty(self.nelem[s], dtype=torch.bfloat16, device=self.device) for s in (0, 1)]
        else:
            self.Qact = self.Q32
        self.Wa = None
        self.U = None
        self.dQ = [torch.empty(self.nelem[s], dtype=torch.float32, device=self.device) for s in (0, 1)]

    # ------------------------------------------------------------------ setup
    def workspace(self, kind: int, T: int = 0) -> torch.Tensor:
        need = self.plan.workspace_size(T, kind)
        cur = self._ws.get(kind)
        if cur is None or cur.numel() < need:
            cur = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
            self._ws[kind] = cur
        return cur

    def set_weight(self, W0: torch.Tensor, pi_R: torch.Tensor, pi_P: torch.Tensor) -> None:
        """Pre-merge the permutations into W0 (once per inner loop); with an INT8
        weight, quantise in the same pass."""
        assert W0.shape == (self.m, self.n) and W0.dtype == self.tdtype and W0.is_contiguous()
        self.pi_R = pi_R.to(device=self.device, dtype=torch.int32).contiguous()
        self.pi_P = pi_P.to(device=self.device, dtype=torch.int32).contiguous()
        if self.weight in ("int8", "int8_t"):
            self.Wt = torch.empty(self.plan.weight_bytes(), dtype=torch.uint8, device=self.device)
            self.plan.quantize_weight(W0, self.pi_R, self.pi_P, self.Wt)
        elif self.weight == "dense_t":
            # Wt [m, n] then its transpose in one buffer; self.Wt views the first part
            self._wbuf = torch.empty(self.plan.weight_bytes(), dtype=torch.uint8, device=self.device)
            self.Wt = self._wbuf[:W0.numel() * W0.element_size()].view(self.tdtype).view(self.m, self.n)
            self.plan.permute_weight(W0, self.pi_R, self.pi_P, self.Wt)
        else:
            self.Wt = torch.empty_like(W0)
            self.plan.permute_weight(W0, self.pi_R, self.pi_P, self.Wt)

    def int8_weight(self):
        """(q [m, n] int8, s [m] fp32) views of an INT8 Wt (rows in permuted order)."""
        assert self.weight in ("int8", "int8_t")
        mn = self.m * self.n
        off = (mn + 255) // 256 * 256
        q = self.Wt[:mn].view(torch.int8).view(self.m, self.n)
        s = self.Wt[off:off + 4 * self.m].view(torch.float32)
        return q, s

    def merge(self, W_out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """End of an inner loop: R W0 P in the original coordinates, from the
        blocks of the last build(). Start the next loop with
        set_weight(W_new, new permutations) and set_theta(zeros)."""
        if W_out is None:
            W_out = torch.empty(self.m, self.n, dtype=self.tdtype, device=self.device)
        ws = self.workspace(_px.WS_MERGE)
        self.plan.merge_weight(self.Wt, self.pi_R, self.pi_P, self.Q32[0], self.Q32[1], W_out,
                               ws, ws.numel())
        return W_out

    def set_theta(self, theta_R: torch.Tensor, theta_P: torch.Tensor) -> None:
        self.theta = [theta_R.to(device=self.device, dtype=torch.float32).contiguous(),
                      theta_P.to(device=self.device, dtype=torch.float32).contiguous()]
        assert self.theta[0].numel() == self.nparam[0] and self.theta[1].numel() == self.nparam[1]

    # ------------------------------------------------------------------ calls
    def build(self) -> None:
        """Build both sides' blocks (one batched call)."""
        build_many([self])

    def build_side(self, side: int) -> None:
        """Build one side through the single-side entry point."""
        ws = self.workspace(_px.WS_BUILD)
        qa = self.Qact[side] if self.dtype == "bf16" else None
        self.plan.build_orth(side, self.theta[side], self.Q32[side], qa, ws, ws.numel())

    def build_items(self):
        """(plan, side, theta, Q_f32, Q_act, ws) for both sides, for build_many()."""
        out = []
        for side in (_px.SIDE_R, _px.SIDE_P):
            qa = self.Qact[side] if self.dtype == "bf16" else None
            ws = self.workspace(_px.WS_BUILD) if side == _px.SIDE_R else self._ws_build_p()
            out.append((self.plan, side, self.theta[side], self.Q32[side], qa, ws))
        return out

    def _ws_build_p(self) -> torch.Tensor:
        # a second build workspace so both sides of one layer can share a batch
        need = self.plan.workspace_size(0, _px.WS_BUILD)
        cur = self._ws.get("build_p")
        if cur is None or cur.numel() < need:
            cur = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
            self._ws["build_p"] = cur
        return cur

    def _ws_grad(self, side: int) -> torch.Tensor:
        need = self.plan.workspace_size(0, _px.WS_PARAM_GRAD)
        key = ("grad", side)
        cur = self._ws.get(key)
        if cur is None or cur.numel() < need:
            cur = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
            self._ws[key] = cur
        return cur

    def forward(self, X: Optional[torch.Tensor], Y: Optional[torch.Tensor] = None,
                Wa: Optional[torch.Tensor] = None, save: bool = True, keep_u: bool = False,
                U: Optional[torch.Tensor] = None) -> torch.Tensor:
        """save: keep Wa for the backward (POET-Xfast); else it is recomputed.
        keep_u: keep the input in permuted order, U = X Pi_P^T (in U if given),
        which the backward then reads instead of gathering X again.
        X None: U already holds X Pi_P^T (gather_u) and the forward skips its
        gather (keep_u is implied)."""
        if X is None:
            assert U is not None, "forward without X needs the gathered input U"
            keep_u = True
            T = U.shape[0]
            assert U.shape == (T, self.n) and U.dtype == self.tdtype and U.is_contiguous()
        else:
            T = X.shape[0]
            assert X.shape == (T, self.n) and X.dtype == self.tdtype and X.is_contiguous()
        if Y is None:
            Y = torch.empty(T, self.m, dtype=self.tdtype, device=self.device)
        if save and Wa is None:
            Wa = torch.empty(T, self.m, dtype=self.tdtype, device=self.device)
        if keep_u and U is None:
            U = torch.empty(T, self.n, dtype=self.tdtype, device=self.device)
        ws = self.workspace(_px.WS_FORWARD, T)
        self.plan.forward(T, X, self.Wt, self.pi_R, self.pi_P, self.Qact[0], self.Qact[1], Y,
                          Wa if save else None, ws, ws.numel(), U_saved=U if keep_u else None)
        self.Wa = Wa if save else None
        self.U = U if keep_u else None
        return Y

    def gather_u(self, X: torch.Tensor, U: Optional[torch.Tensor] = None) -> torch.Tensor:
        """U = X Pi_P^T, the input in the permuted order forward(None, U=U) takes."""
        T = X.shape[0]
        assert X.shape == (T, self.n) and X.dtype == self.tdtype and X.is_contiguous()
        if U is None:
            U = torch.empty(T, self.n, dtype=self.tdtype, device=self.device)
        self.plan.gather_cols(T, self.n, X, self.pi_P, U)
        return U

    def _check_saved(self, T: int) -> None:
        # no saved Wa (forward(save=False)): the backward recomputes it (POET-Xmem)
        assert self.Wa is None or self.Wa.shape[0] == T, "saved Wa is from another batch"
        assert self.U is None or self.U.shape[0] == T, "kept U is from another batch"

    def backward(self, X: Optional[torch.Tensor], G_Y: torch.Tensor, G_X: Optional[torch.Tensor] = None,
                 g_theta: Optional[Sequence[torch.Tensor]] = None):
        """X may be None when the forward kept U."""
        T = G_Y.shape[0]
        self._check_saved(T)
        assert G_Y.shape == (T, self.m) and G_Y.dtype == self.tdtype and G_Y.is_contiguous()
        if G_X is None:
            G_X = torch.empty(T, self.n, dtype=self.tdtype, device=self.device)
        if g_theta is None:
            g_theta = [torch.empty(self.nparam[s], dtype=torch.float32, device=self.device) for s in (0, 1)]
        ws = self.workspace(_px.WS_BACKWARD, T)
        self.plan.backward(T, X, self.Wt, self.pi_R, self.pi_P, self.theta[0], self.theta[1],
                           self.Qact[0], self.Qact[1], self.Wa, G_Y, G_X, g_theta[0], g_theta[1],
                           ws, ws.numel(), U_saved=self.U)
        return G_X, g_theta[0], g_theta[1]

    def backward_dq(self, X: Optional[torch.Tensor], G_Y: torch.Tensor,
                    G_X: Optional[torch.Tensor] = None):
        """Activation path of the backward: returns G_X and leaves dL/dQ of both
        sides in self.dQ for param_grad_many(). X may be None when the forward
        kept U."""
        T = G_Y.shape[0]
        self._check_saved(T)
        assert G_Y.shape == (T, self.m) and G_Y.dtype == self.tdtype and G_Y.is_contiguous()
        if G_X is None:
            G_X = torch.empty(T, self.n, dtype=self.tdtype, device=self.device)
        ws = self.workspace(_px.WS_BACKWARD, T)
        self.plan.backward_dq(T, X, self.Wt, self.pi_R, self.pi_P, self.Qact[0], self.Qact[1],
                              self.Wa, G_Y, G_X, self.dQ[0], self.dQ[1], ws, ws.numel(),
                              U_saved=self.U)
        return G_X
