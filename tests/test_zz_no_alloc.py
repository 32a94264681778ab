"""poetx_forward_noalloc: the forward whose workspace is the library's static
device array (for callers that cannot allocate), through the C ABI, against
poetx_forward with a caller workspace. Same kernels, so the same bits: two
calls in a row, the second with a smaller input and another plan, and a call
whose workspace would not fit, which must be refused before any launch."""
import pytest

import workloads
from gpu_util import device_ready, log, make_layer, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not device_ready():
        pytest.skip("no GPU")


def _bits(t):
    import torch
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu()


def _one(c, T, seed):
    import torch
    from orthogonal_equivalence_cayley_amd import poetx as px
    inp = workloads.small_case(c[0], c[1], c[2], c[3], T=T, seed=seed, dtype=c[4], theta_std=0.01)
    log(f"noalloc {c[:2]} {c[4]} T={T}")
    L = make_layer(inp, 4, c[4])
    L.build()
    X = to_dev(inp.X, c[4])
    Y1 = L.forward(X, save=True).clone()
    Wa1 = L.Wa.clone()
    Y2, Wa2 = torch.empty_like(Y1), torch.empty_like(Wa1)
    U2 = torch.empty_like(X)
    L.plan.forward_noalloc(T, X, L.Wt, L.pi_R, L.pi_P, L.Qact[0], L.Qact[1], Y2, Wa2, U_saved=U2)
    torch.cuda.synchronize()
    assert torch.equal(_bits(Y1), _bits(Y2))
    assert torch.equal(_bits(Wa1), _bits(Wa2))
    want_u = X.cpu()[:, torch.from_numpy(inp.pi_P).long()].contiguous()
    assert torch.equal(_bits(U2), _bits(want_u))
    return L


def test_forward_noalloc_matches_forward():
    from orthogonal_equivalence_cayley_amd import poetx as px
    # first call: fused index passes on both sides (bf16, blocks of 256)
    _one((512, 768, (256, 256), (256,) * 3, "bf16"), 900, 1)
    # second call on the same array: fewer tokens, separate kernels on the
    # 2304-wide side, and an fp32 plan after it
    _one((2304, 512, (256,) * 9, (256, 256), "bf16"), 130, 2)
    L = _one((96, 80, (32, 64), (48, 32), "f32"), 17, 3)
    # a workspace larger than the array is refused on the host
    cap = px.LIB.poetx_forward_noalloc_max_bytes()
    T = cap // (4 * (L.m + L.n)) + 1
    assert L.plan.workspace_size(T, px.WS_FORWARD) > cap
    A = 1 << 20
    st = px.LIB.poetx_forward_noalloc(L.plan.handle, T, A, A, A, A, A, A, A, None, None, None)
    assert st == px.POETX_ERR_WORKSPACE
