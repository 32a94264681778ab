"""GPU parity at the five workloads' full sizes, through the same library calls
(and therefore the same kernels and launch shapes) the benchmark times.

The three single-layer workloads are compared with the full float64 oracle.
For the 7-linear blocks at hidden 2048 and 4096 (16384 tokens) every layer is
checked on sampled outputs the oracle computes one by one: 48 token rows of
Y, Wa and G_X (rows are independent; the first and the last row are always
included), all blocks of Q, and the packed parameter gradient of the first and
the last block of each side (a full reduction over all tokens; the last block
is the 256-wide tail where the side has one).
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import blocks_concat, device_ready, log, run_layer, to_dev

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not device_ready():
        pytest.skip("no GPU")


def _check(name, got, want, tol):
    err = oracle.rel_fro(got, want)
    log(f"  {name}: rel_fro={err:.3e} (tol {tol:g})")
    assert err <= tol, (name, err)


@pytest.mark.parametrize("cid", [1, 2, 3])
def test_single_layer_workload_full(cid):
    w = workloads.WORKLOADS[cid]
    inp = workloads.layer_inputs(w, 0)
    log(f"{w.name}: T={w.T} m={inp.spec.m} n={inp.spec.n}")
    got, _ = run_layer(inp, w.k, w.dtype, backward=w.backward)
    ref = oracle.layer_reference(inp, w.k, backward_pass=w.backward)
    tol = TOL_F32 if w.dtype == "f32" else TOL_BF16
    _check("Q_R", got["QR"], blocks_concat(ref["QR"]), TOL_F32)
    _check("Q_P", got["QP"], blocks_concat(ref["QP"]), TOL_F32)
    _check("Wa", got["Wa"], ref["Wa"], tol)
    _check("Y", got["Y"], ref["Y"], tol)
    if w.backward:
        _check("G_X", got["G_X"], ref["G_X"], tol)
        _check("g_theta_R", got["g_theta_R"], ref["g_theta_R"], tol)
        _check("g_theta_P", got["g_theta_P"], ref["g_theta_P"], tol)


def test_exact_cayley_workload_full():
    """Exact-Cayley mode at the full size of the 5632 x 2048 workload (8192
    tokens, forward and backward), against the oracle's solve-based transform
    and its closed-form gradient. The batched fp32 products of the transform
    then run over both sides' 30 blocks in single launches."""
    import torch
    from orthogonal_equivalence_cayley_amd import PoetxLayer
    w = workloads.WORKLOADS[3]
    inp = workloads.layer_inputs(w, 0)
    sp = inp.spec
    log(f"{w.name} exact: T={w.T} m={sp.m} n={sp.n}")
    L = PoetxLayer(sp.m, sp.n, sp.bsz_R, sp.bsz_P, w.k, dtype=w.dtype, cayley="exact")
    L.set_weight(to_dev(inp.W0, w.dtype), torch.from_numpy(inp.pi_R), torch.from_numpy(inp.pi_P))
    L.set_theta(torch.from_numpy(inp.theta_R), torch.from_numpy(inp.theta_P))
    got, _ = run_layer(inp, w.k, w.dtype, backward=w.backward, layer=L)
    ref = oracle.layer_reference(inp, None, backward_pass=w.backward)
    _check("Q_R", got["QR"], blocks_concat(ref["QR"]), TOL_F32)
    _check("Q_P", got["QP"], blocks_concat(ref["QP"]), TOL_F32)
    for key in ("Wa", "Y", "G_X", "g_theta_R", "g_theta_P"):
        _check(key, got[key], ref[key], TOL_BF16)


def _sample_rows(T, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, 46, replace=False)]))


@pytest.mark.parametrize("cid,li", [(4, i) for i in range(7)] + [(5, i) for i in range(7)])
def test_block_workload_layer_sampled(cid, li):
    w = workloads.WORKLOADS[cid]
    inp = workloads.layer_inputs(w, li)
    sp = inp.spec
    log(f"{w.name} layer {sp.name}: T={w.T} m={sp.m} n={sp.n}")
    got, layer = run_layer(inp, w.k, w.dtype, backward=True)
    del layer
    QR = oracle.build_orth(inp.theta_R, sp.bsz_R, w.k)
    QP = oracle.build_orth(inp.theta_P, sp.bsz_P, w.k)
    _check("Q_R", got["QR"], blocks_concat(QR), TOL_F32)
    _check("Q_P", got["QP"], blocks_concat(QP), TOL_F32)
    Wt = oracle.permute_weight(inp.W0, inp.pi_R, inp.pi_P)
    rows = _sample_rows(w.T, 100 * cid + li)
    Yr, War = oracle.forward(inp.X[rows], Wt, inp.pi_R, inp.pi_P, QR, QP, sp.bsz_R, sp.bsz_P)
    _check("Y rows", got["Y"][rows], Yr, TOL_BF16)
    _check("Wa rows", got["Wa"][rows], War, TOL_BF16)
    Gr = oracle.backward_rows(inp.G_Y[rows], Wt, inp.pi_R, inp.pi_P, QR, QP, sp.bsz_R, sp.bsz_P)
    _check("G_X rows", got["G_X"][rows], Gr, TOL_BF16)
    for side, bsz, g in (("R", sp.bsz_R, got["g_theta_R"]), ("P", sp.bsz_P, got["g_theta_P"])):
        offs = np.cumsum([0] + [b * (b - 1) // 2 for b in bsz])
        for j in sorted({0, len(bsz) - 1}):
            want = oracle.theta_grad_block(side, j, inp.X, Wt, inp.pi_R, inp.pi_P, inp.theta_R,
                                           inp.theta_P, QR, QP, inp.G_Y, sp.bsz_R, sp.bsz_P, w.k)
            _check(f"g_theta_{side}[block {j}]", g[offs[j]:offs[j + 1]], want, TOL_BF16)


def test_merge_full_size():
    """Merge of the 5632 x 2048 layer (b = 256 on both sides) at its real shape
    against the dense float64 merge."""
    import torch
    w = workloads.WORKLOADS[3]
    inp = workloads.layer_inputs(w, 0, T=1)
    from gpu_util import make_layer, to_np
    L = make_layer(inp, w.k, w.dtype)
    L.build()
    W = L.merge()
    torch.cuda.synchronize()
    sp = inp.spec
    want = oracle.merge_weight(inp.W0, inp.theta_R, inp.theta_P, inp.pi_R, inp.pi_P, sp.bsz_R,
                               sp.bsz_P, w.k)
    _check("W_new", to_np(W), want, 4e-3)


def test_int8_weight_full_size():
    """POET-XQ on the 5632 x 2048 layer at 8192 tokens (build, forward,
    backward) against the full oracle on the dequantised weight."""
    import dataclasses
    import torch
    from gpu_util import make_layer, to_dev, to_np
    w = workloads.WORKLOADS[3]
    inp = workloads.layer_inputs(w, 0)
    L = make_layer(inp, w.k, "bf16", weight="int8")
    L.build()
    X, G = to_dev(inp.X, "bf16"), to_dev(inp.G_Y, "bf16")
    Y = L.forward(X)
    G_X, gR, gP = L.backward(X, G)
    torch.cuda.synchronize()
    q, s = oracle.quantize_rows(inp.W0)
    ref = oracle.layer_reference(dataclasses.replace(inp, W0=oracle.dequantize_rows(q, s)), w.k)
    _check("Y", to_np(Y), ref["Y"], TOL_BF16)
    _check("G_X", to_np(G_X), ref["G_X"], TOL_BF16)
    _check("g_theta_R", to_np(gR), ref["g_theta_R"], TOL_BF16)
    _check("g_theta_P", to_np(gP), ref["g_theta_P"], TOL_BF16)
