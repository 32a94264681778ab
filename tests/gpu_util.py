"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
run the layer through libpoetx, and bring results back as float64 arrays."""
import sys

import numpy as np


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def device_ready() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def to_dev(a: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


def to_np(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def make_layer(inp, k: int, dtype: str, weight: str = "dense", fold: str = "none",
               index: str = "separate"):
    import torch
    from orthogonal_equivalence_cayley_amd import PoetxLayer
    sp = inp.spec
    layer = PoetxLayer(sp.m, sp.n, sp.bsz_R, sp.bsz_P, k, dtype=dtype, weight=weight, fold=fold,
                       index=index)
    layer.set_weight(to_dev(inp.W0, dtype), torch.from_numpy(inp.pi_R), torch.from_numpy(inp.pi_P))
    layer.set_theta(torch.from_numpy(inp.theta_R), torch.from_numpy(inp.theta_P))
    return layer


def run_layer(inp, k: int, dtype: str, backward: bool = True, layer=None):
    """Build + forward (+ backward) on the GPU; returns a dict of float64 arrays."""
    import torch
    if layer is None:
        layer = make_layer(inp, k, dtype)
    layer.build()
    X = to_dev(inp.X, dtype)
    Y = layer.forward(X, save=True)
    out = dict(Y=Y, Wa=layer.Wa, QR=layer.Q32[0], QP=layer.Q32[1], Wt=layer.Wt)
    if dtype == "bf16":
        out.update(QRa=layer.Qact[0], QPa=layer.Qact[1])
    if backward:
        G = to_dev(inp.G_Y, dtype)
        G_X, gR, gP = layer.backward(X, G)
        out.update(G_X=G_X, g_theta_R=gR, g_theta_P=gP)
    torch.cuda.synchronize()
    return {k_: to_np(v) for k_, v in out.items()}, layer


def blocks_concat(Qs) -> np.ndarray:
    return np.concatenate([q.reshape(-1) for q in Qs])
