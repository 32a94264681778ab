"""Plans with POETX_INDEX_FUSED: index mapping fused with the block products
(one pass over 32-row panels of whole token rows; sides of 256-wide blocks up
to 2048 features).

Every side of these layers that the fused pass takes runs through it: the
forward's gather + P blocks and R blocks + scatter, the backward's gather + R
blocks and P blocks + scatter, and the POET-Xmem recomputation. Results go
against the float64 oracle (ragged token counts, an odd number of blocks, a
side too wide for the fused pass next to one it takes). The fused forward's
multiplies take the same operands in the same order as the separate gather
followed by the block product, so the two give the same bits.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import blocks_concat, device_ready, log, make_layer, to_dev, to_np

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not device_ready():
        pytest.skip("no GPU")


CASES = [
    dict(m=256, n=256, bR=(256,), bP=(256,), T=1),
    dict(m=512, n=768, bR=(256, 256), bP=(256, 256, 256), T=33),
    dict(m=768, n=512, bR=(256,) * 3, bP=(256,) * 2, T=95),
    dict(m=2048, n=2048, bR=(256,) * 8, bP=(256,) * 8, T=1000),
    # R side 2304 wide: separate kernels there, the fused pass on the P side
    dict(m=2304, n=512, bR=(256,) * 9, bP=(256, 256), T=200),
    # P side 2560 wide: the other way round
    dict(m=512, n=2560, bR=(256, 256), bP=(256,) * 10, T=64),
]


@pytest.mark.parametrize("save", [True, False])
@pytest.mark.parametrize("c", CASES, ids=lambda c: f"{c['m']}x{c['n']}-T{c['T']}")
def test_fused_layer_against_oracle(c, save):
    import torch
    inp = workloads.small_case(c["m"], c["n"], c["bR"], c["bP"], T=c["T"], seed=c["m"] + 3 * c["T"],
                               dtype="bf16", theta_std=0.01)
    log(f"fused layer {c} save={save}")
    L = make_layer(inp, 4, "bf16", index="fused")
    L.build()
    X, G = to_dev(inp.X, "bf16"), to_dev(inp.G_Y, "bf16")
    Y = L.forward(X, save=save)
    Wa = L.Wa
    G_X, gR, gP = L.backward(X, G)
    torch.cuda.synchronize()
    ref = oracle.layer_reference(inp, 4)
    got = dict(Y=to_np(Y), G_X=to_np(G_X), g_theta_R=to_np(gR), g_theta_P=to_np(gP),
               QR=to_np(L.Q32[0]), QP=to_np(L.Q32[1]))
    for key in ("QR", "QP"):
        err = oracle.rel_fro(got[key], blocks_concat(ref[key]))
        assert err <= TOL_F32, (key, err)
    keys = ["Y", "G_X", "g_theta_R", "g_theta_P"]
    if save:
        got["Wa"] = to_np(Wa)
        keys.append("Wa")
    for key in keys:
        err = oracle.rel_fro(got[key], ref[key])
        log(f"  {key}: rel_fro={err:.3e}")
        assert err <= TOL_BF16, (key, err)


@pytest.mark.parametrize("T", [1, 31, 32, 33, 700])
def test_fused_gather_matches_separate_gather(T):
    """Forward from X (gather fused into the P blocks, U kept) against the
    forward from U = poetx_gather_cols(X) (separate block product): U, Wa and Y
    bit for bit."""
    import torch
    inp = workloads.small_case(512, 768, (256, 256), (256,) * 3, T=T, seed=T + 5, dtype="bf16",
                               theta_std=0.01)
    L = make_layer(inp, 4, "bf16", index="fused")
    L.build()
    X = to_dev(inp.X, "bf16")
    U1 = torch.empty_like(X)
    Y1 = L.forward(X, save=True, keep_u=True, U=U1).clone()
    Wa1 = L.Wa.clone()
    U2 = L.gather_u(X)
    Y2 = L.forward(None, save=True, U=U2).clone()
    Wa2 = L.Wa.clone()
    torch.cuda.synchronize()
    assert torch.equal(U1.view(torch.int16), U2.view(torch.int16))
    assert torch.equal(Wa1.view(torch.int16), Wa2.view(torch.int16))
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    want = X.cpu()[:, torch.from_numpy(inp.pi_P).long()]
    assert torch.equal(U1.cpu().view(torch.int16), want.contiguous().view(torch.int16))


@pytest.mark.parametrize("save", [True, False])
def test_fused_plan_matches_separate_plan(save):
    """The fused passes multiply the same operands in the same order as the
    separate gather, block product and scatter: a plan with fused index passes
    and one without give the same bits for every output."""
    import torch
    inp = workloads.small_case(768, 1024, (256,) * 3, (256,) * 4, T=333, seed=9, dtype="bf16",
                               theta_std=0.01)
    out = []
    for index in ("fused", "separate"):
        L = make_layer(inp, 4, "bf16", index=index)
        L.build()
        X, G = to_dev(inp.X, "bf16"), to_dev(inp.G_Y, "bf16")
        Y = L.forward(X, save=save)
        G_X, gR, gP = L.backward(X, G)
        torch.cuda.synchronize()
        out.append([Y, G_X, gR, gP] + ([L.Wa] if save else []))
    for a, b in zip(*out):
        va = a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32)
        vb = b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)
        assert torch.equal(va, vb)
