"""GPU parity of libpoetx against the float64 oracle on seeded inputs, at sizes
the oracle finishes in seconds (several tiles, ragged tails, edge cases).

Tolerances (relative Frobenius error against the float64 oracle):
  index paths (gather, scatter, weight pre-merge): bit-exact;
  fp32 mode: 1e-5 for Q, Y, Wa, G_X and both parameter gradients;
  bf16 inputs with fp32 accumulation: 2e-2.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import blocks_concat, device_ready, log, make_layer, run_layer, to_dev, to_np

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not device_ready():
        pytest.skip("no GPU")


def _px():
    from orthogonal_equivalence_cayley_amd import poetx
    return poetx


def _plan(dtype):
    px = _px()
    return px.Plan(32, 32, (16, 16), (16, 16), 1, px.POETX_BF16 if dtype == "bf16" else px.POETX_FP32)


def _bits(t):
    import torch
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu()


# ---------------------------------------------------------------- index paths

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dim", [16, 37, 2048, 5632, 9000, 11008, 16384, 40000])
@pytest.mark.parametrize("T", [1, 9, 130])
def test_gather_scatter_bitexact(dtype, dim, T):
    import torch
    log(f"gather/scatter dtype={dtype} dim={dim} T={T}")
    rng = np.random.default_rng(dim * 7 + T)
    x = rng.standard_normal((T, dim)).astype(np.float32)
    idx = rng.permutation(dim).astype(np.int32)
    X = to_dev(x, dtype)
    I = torch.from_numpy(idx).cuda()
    out = torch.empty_like(X)
    back = torch.empty_like(X)
    p = _plan(dtype)
    p.gather_cols(T, dim, X, I, out)
    p.scatter_cols(T, dim, out, I, back)
    torch.cuda.synchronize()
    Xc = X.cpu()
    assert torch.equal(_bits(out), _bits(Xc[:, torch.from_numpy(idx).long()].contiguous()))
    assert torch.equal(_bits(back), _bits(Xc))


@pytest.mark.parametrize("dtype,m,n", [("bf16", 2048, 2048), ("bf16", 5632, 2048), ("bf16", 80, 11008),
                                        ("f32", 37, 53)])
def test_permute_weight_bitexact(dtype, m, n):
    import torch
    log(f"permute_weight {dtype} {m}x{n}")
    rng = np.random.default_rng(m + n)
    W0 = rng.standard_normal((m, n)).astype(np.float32)
    piR, piP = rng.permutation(m).astype(np.int32), rng.permutation(n).astype(np.int32)
    px = _px()
    p = px.Plan(m, n, (m,), (n,), 0, px.POETX_BF16 if dtype == "bf16" else px.POETX_FP32)
    Wd = to_dev(W0, dtype)
    Wt = torch.empty_like(Wd)
    p.permute_weight(Wd, torch.from_numpy(piR).cuda(), torch.from_numpy(piP).cuda(), Wt)
    torch.cuda.synchronize()
    want = Wd.cpu()[torch.from_numpy(piR).long()][:, torch.from_numpy(piP).long()].contiguous()
    assert torch.equal(_bits(Wt), _bits(want))


# ---------------------------------------------------------------- build

@pytest.mark.parametrize("dtype,bsz,k,std", [
    ("f32", (32,) * 8, 3, 0.01),
    ("f32", (5, 1, 17, 64), 0, 0.05),
    ("f32", (7, 33), 6, 0.05),
    ("bf16", (256,) * 3, 4, 0.01),
    ("bf16", (512, 512, 256), 5, 0.005),
    # split chains with eight waves for blocks between 256 and 512 that are not
    # 512 (the generic K loop), mixed in one launch
    ("bf16", (384, 288, 320, 448), 4, 0.01),
    ("bf16", (16, 48), 2, 0.05),
])
def test_build_orth(dtype, bsz, k, std):
    import torch
    log(f"build_orth {dtype} {bsz} k={k}")
    inp = workloads.small_case(sum(bsz), 16, bsz, (16,), T=1, seed=len(bsz) + k, dtype=dtype,
                               theta_std=std)
    layer = make_layer(inp, k, dtype)
    layer.build()
    torch.cuda.synchronize()
    want = blocks_concat(oracle.build_orth(inp.theta_R, bsz, k))
    got = layer.Q32[0].cpu().numpy().astype(np.float64)
    assert oracle.rel_fro(got, want) <= TOL_F32
    if dtype == "bf16":
        # the bf16 copy is the fp32 block rounded to nearest: within half a bf16 ulp
        qa = layer.Qact[0].float().cpu().numpy().astype(np.float64)
        assert np.all(np.abs(qa - want) <= np.abs(want) * 2.0 ** -8 + 1e-6)


@pytest.mark.parametrize("k", list(range(9)))
@pytest.mark.parametrize("dtype,bsz", [("f32", (64, 33)), ("bf16", (256, 96))])
def test_build_orth_every_k(dtype, bsz, k):
    """The power-chain build for every k from 0 to 8 (fp32 chains; split bf16
    chains for the bf16 plan) against the oracle's series."""
    import torch
    log(f"build_orth chain {dtype} {bsz} k={k}")
    inp = workloads.small_case(sum(bsz), 16, bsz, (16,), T=1, seed=100 + k, dtype=dtype, theta_std=0.02)
    layer = make_layer(inp, k, dtype)
    layer.build()
    torch.cuda.synchronize()
    want = blocks_concat(oracle.build_orth(inp.theta_R, bsz, k))
    got = layer.Q32[0].cpu().numpy().astype(np.float64)
    assert oracle.rel_fro(got, want) <= TOL_F32


# ---------------------------------------------------------------- whole layer

def _compare(got, ref, keys, tol, tag):
    for key in keys:
        r = ref[key]
        if key in ("QR", "QP"):
            r = blocks_concat(r)
        err = oracle.rel_fro(got[key], r)
        log(f"  {tag} {key}: rel_fro={err:.3e}")
        assert err <= tol, (key, err)


def test_layer_fp32_small_config():
    w = workloads.WORKLOADS[1]
    inp = workloads.layer_inputs(w, 0)
    log(f"layer fp32 {w.name}")
    got, _ = run_layer(inp, w.k, "f32")
    ref = oracle.layer_reference(inp, w.k)
    _compare(got, ref, ["QR", "QP", "Wa", "Y", "G_X", "g_theta_R", "g_theta_P"], TOL_F32, "cfg1")


@pytest.mark.parametrize("case", [
    dict(m=12, n=9, bR=(5, 7), bP=(4, 1, 4), T=7, k=0),
    dict(m=70, n=45, bR=(30, 40), bP=(45,), T=1, k=5),
    dict(m=96, n=130, bR=(32, 64), bP=(65, 65), T=130, k=2),
    dict(m=64, n=64, bR=(64,), bP=(16, 16, 32), T=257, k=1),
])
def test_layer_fp32_ragged(case):
    inp = workloads.small_case(case["m"], case["n"], case["bR"], case["bP"], T=case["T"],
                               seed=case["m"] + case["T"], dtype="f32", theta_std=0.05)
    log(f"layer fp32 ragged {case}")
    got, _ = run_layer(inp, case["k"], "f32")
    ref = oracle.layer_reference(inp, case["k"])
    _compare(got, ref, ["QR", "QP", "Wa", "Y", "G_X", "g_theta_R", "g_theta_P"], TOL_F32, "ragged")


@pytest.mark.parametrize("case", [
    dict(m=512, n=256, bR=(256, 256), bP=(128, 128), T=300, k=4),
    dict(m=384, n=320, bR=(128, 256), bP=(64, 256), T=77, k=3),
    dict(m=2048, n=512, bR=(512,) * 3 + (256, 256), bP=(512,), T=1000, k=5),
    # blocks of 512 only: the block products with two workgroups per block and
    # the split chains with eight waves (ragged and whole row tiles)
    dict(m=1024, n=1024, bR=(512, 512), bP=(512, 512), T=130, k=4),
    dict(m=768, n=736, bR=(384, 384), bP=(448, 288), T=100, k=3),
    dict(m=512, n=1536, bR=(512,), bP=(512,) * 3, T=64, k=5),
    dict(m=256, n=256, bR=(256,), bP=(256,), T=1, k=4),
    # frozen-weight product on whole 256 x 256 tiles with one 64-deep stage
    # (K = n = 64) and 1088 tiles on 256 workgroups
    dict(m=4352, n=64, bR=(256,) * 17, bP=(64,), T=16384, k=2),
    # the same kernel with three 64-deep stages per tile and 320 tiles (some
    # workgroups take a second tile), and with two stages on exactly 256 tiles
    dict(m=1280, n=192, bR=(256,) * 5, bP=(64, 128), T=16384, k=3),
    dict(m=1024, n=128, bR=(256,) * 4, bP=(128,), T=16384, k=2),
    dict(m=48, n=32, bR=(16, 32), bP=(32,), T=5, k=0),
    # split chains over blocks that are multiples of 32 but not of 64, alone and
    # mixed with other sizes in one launch
    dict(m=256, n=288, bR=(96, 160), bP=(224, 64), T=200, k=4),
    dict(m=320, n=96, bR=(192, 64, 64), bP=(96,), T=64, k=3),
    # the token reduction dQ per run of equal blocks: 21 blocks of 512 on
    # 256 x 256 tiles (three splits) beside one block of 256 with its own split
    # count, as on an 11008-wide side; four blocks of 768 on the large tiles too
    dict(m=11008, n=512, bR=(512,) * 21 + (256,), bP=(512,), T=1024, k=4),
    dict(m=3072, n=256, bR=(768,) * 4, bP=(256,), T=640, k=3),
])
def test_layer_bf16_small(case):
    inp = workloads.small_case(case["m"], case["n"], case["bR"], case["bP"], T=case["T"],
                               seed=case["n"] + case["T"], dtype="bf16", theta_std=0.01)
    log(f"layer bf16 {case}")
    got, _ = run_layer(inp, case["k"], "bf16")
    ref = oracle.layer_reference(inp, case["k"])
    _compare(got, ref, ["QR", "QP"], TOL_F32, "bf16")
    _compare(got, ref, ["Wa", "Y", "G_X", "g_theta_R", "g_theta_P"], TOL_BF16, "bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identity_permutations(dtype):
    """pi_R and pi_P the identity: the gather and the scatter copy rows
    unchanged (U = X bit for bit) and the layer matches the oracle."""
    import torch
    inp = workloads.small_case(512, 256, (256, 256), (128, 128), T=200, seed=31, dtype=dtype,
                               theta_std=0.01 if dtype == "bf16" else 0.05)
    inp.pi_R = np.arange(512, dtype=inp.pi_R.dtype)
    inp.pi_P = np.arange(256, dtype=inp.pi_P.dtype)
    log(f"identity permutations {dtype}")
    L = make_layer(inp, 4, dtype)
    L.build()
    X = to_dev(inp.X, dtype)
    U = L.gather_u(X)
    torch.cuda.synchronize()
    assert torch.equal(_bits(U), _bits(X))
    got, _ = run_layer(inp, 4, dtype)
    ref = oracle.layer_reference(inp, 4)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    _compare(got, ref, ["QR", "QP"], TOL_F32, "identity")
    _compare(got, ref, ["Wa", "Y", "G_X", "g_theta_R", "g_theta_P"], tol, "identity")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_theta_zero_gives_plain_linear(dtype):
    inp = workloads.small_case(256, 128, (128, 128), (128,), T=64, seed=3, dtype=dtype)
    inp.theta_R[:] = 0.0
    inp.theta_P[:] = 0.0
    log(f"theta=0 {dtype}")
    got, _ = run_layer(inp, 4, dtype, backward=False)
    want = inp.X.astype(np.float64) @ inp.W0.astype(np.float64).T
    assert oracle.rel_fro(got["Y"], want) <= (TOL_F32 if dtype == "f32" else TOL_BF16)
    assert np.array_equal(got["QR"], blocks_concat([np.eye(128)] * 2))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_tokens(dtype):
    import torch
    inp = workloads.small_case(64, 32, (32, 32), (32,), T=3, seed=5, dtype=dtype)
    layer = make_layer(inp, 2, dtype)
    layer.build()
    X = to_dev(inp.X[:0], dtype)
    Y = layer.forward(X, save=True)
    G_X, gR, gP = layer.backward(X, to_dev(inp.G_Y[:0], dtype))
    torch.cuda.synchronize()
    assert Y.shape == (0, 64) and G_X.shape == (0, 32)
    assert float(gR.abs().max()) == 0.0 and float(gP.abs().max()) == 0.0


def test_backward_deterministic():
    import torch
    inp = workloads.small_case(512, 256, (256, 256), (256,), T=2000, seed=9, dtype="bf16")
    layer = make_layer(inp, 4, "bf16")
    layer.build()
    X, G = to_dev(inp.X, "bf16"), to_dev(inp.G_Y, "bf16")
    layer.forward(X)
    a = [t.clone() for t in layer.backward(X, G)]
    b = [t.clone() for t in layer.backward(X, G)]
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_build_batch_matches_single_side_builds():
    """One batched build over several layers (supported and generic block sizes,
    bf16 and fp32 plans) gives the same blocks as the single-side entry point,
    and both match the oracle."""
    import torch
    from orthogonal_equivalence_cayley_amd import build_many
    specs = [
        ("bf16", workloads.small_case(512, 256, (256, 256), (128, 128), T=1, seed=1, dtype="bf16", theta_std=0.01), 4),
        ("bf16", workloads.small_case(1024, 512, (512, 256, 256), (512,), T=1, seed=2, dtype="bf16", theta_std=0.005), 4),
        ("f32", workloads.small_case(70, 64, (30, 40), (64,), T=1, seed=3, dtype="f32", theta_std=0.05), 4),
    ]
    layers = [make_layer(inp, k, dt) for dt, inp, k in specs]
    build_many(layers)
    torch.cuda.synchronize()
    batch = [[L.Q32[s].clone() for s in (0, 1)] for L in layers]
    for L in layers:
        L.build_side(0)
        L.build_side(1)
    torch.cuda.synchronize()
    for (dt, inp, k), L, qb in zip(specs, layers, batch):
        for s, bsz, th in ((0, inp.spec.bsz_R, inp.theta_R), (1, inp.spec.bsz_P, inp.theta_P)):
            assert torch.equal(qb[s], L.Q32[s])
            want = blocks_concat(oracle.build_orth(th, bsz, k))
            assert oracle.rel_fro(qb[s].cpu().numpy().astype(np.float64), want) <= TOL_F32


def test_backward_split_matches_backward():
    """backward_dq per layer + one param_grad_batch over all layers gives the
    same results as poetx_backward per layer (same kernels, bit for bit)."""
    import torch
    from orthogonal_equivalence_cayley_amd import param_grad_many
    cases = [
        (workloads.small_case(512, 256, (256, 256), (128, 128), T=300, seed=21, dtype="bf16", theta_std=0.01), 4, "bf16"),
        (workloads.small_case(256, 512, (256,), (256, 128, 128), T=130, seed=22, dtype="bf16", theta_std=0.01), 3, "bf16"),
        (workloads.small_case(70, 45, (30, 40), (45,), T=9, seed=23, dtype="f32", theta_std=0.05), 4, "f32"),
    ]
    layers, ref = [], []
    for inp, k, dt in cases:
        L = make_layer(inp, k, dt)
        L.build()
        X, G = to_dev(inp.X, dt), to_dev(inp.G_Y, dt)
        L.forward(X)
        gx, gr, gp = L.backward(X, G)
        ref.append((gx.clone(), gr.clone(), gp.clone()))
        L.backward_dq(X, G)
        layers.append(L)
    grads = param_grad_many(layers)
    torch.cuda.synchronize()
    for (gx, gr, gp), (g2r, g2p) in zip(ref, grads):
        assert torch.equal(gr, g2r) and torch.equal(gp, g2p)


@pytest.mark.parametrize("case", [
    ("bf16", dict(m=512, n=256, bR=(256, 256), bP=(128, 128), T=300, k=4)),
    ("bf16", dict(m=256, n=768, bR=(256,), bP=(512, 256), T=1000, k=3)),
    ("bf16", dict(m=1024, n=512, bR=(512, 512), bP=(512,), T=200, k=4)),
    ("f32", dict(m=96, n=130, bR=(32, 64), bP=(65, 65), T=130, k=2)),
])
def test_xmem_recompute_matches_saved(case):
    """Backward without a saved Wa (recomputed from X) gives the saved path's
    results bit for bit, and both match the oracle."""
    import torch
    dt, c = case
    inp = workloads.small_case(c["m"], c["n"], c["bR"], c["bP"], T=c["T"], seed=c["m"] + 7,
                               dtype=dt, theta_std=0.01 if dt == "bf16" else 0.05)
    log(f"xmem {dt} {c}")
    L = make_layer(inp, c["k"], dt)
    L.build()
    X, G = to_dev(inp.X, dt), to_dev(inp.G_Y, dt)
    L.forward(X, save=True)
    saved = [t.clone() for t in L.backward(X, G)]
    Y = L.forward(X, save=False)
    assert L.Wa is None
    mem = [t.clone() for t in L.backward(X, G)]
    torch.cuda.synchronize()
    for u, v in zip(saved, mem):
        assert torch.equal(u, v)
    ref = oracle.layer_reference(inp, c["k"])
    tol = TOL_BF16 if dt == "bf16" else TOL_F32
    got = dict(Y=to_np(Y), G_X=to_np(mem[0]), g_theta_R=to_np(mem[1]), g_theta_P=to_np(mem[2]))
    _compare(got, ref, ["Y", "G_X", "g_theta_R", "g_theta_P"], tol, "xmem")


@pytest.mark.parametrize("dt, c", [
    ("bf16", dict(m=512, n=256, bR=(256, 256), bP=(128, 128), T=300, k=4)),
    ("f32", dict(m=70, n=45, bR=(30, 40), bP=(45,), T=9, k=3)),
])
def test_forward_from_gathered_input(dt, c):
    """forward(None, U=gather_u(X)) skips its gather and gives forward(X)'s Y,
    Wa, U and backward bit for bit."""
    import torch
    inp = workloads.small_case(c["m"], c["n"], c["bR"], c["bP"], T=c["T"], seed=c["m"] + 31,
                               dtype=dt, theta_std=0.01 if dt == "bf16" else 0.05)
    log(f"forward from U {dt} {c}")
    L = make_layer(inp, c["k"], dt)
    L.build()
    X, G = to_dev(inp.X, dt), to_dev(inp.G_Y, dt)
    Y1 = L.forward(X, keep_u=True).clone()
    Wa1, U1 = L.Wa.clone(), L.U.clone()
    g1 = [t.clone() for t in L.backward(X, G)]
    U = L.gather_u(X)
    Y2 = L.forward(None, U=U)
    torch.cuda.synchronize()
    assert torch.equal(U, U1) and torch.equal(Y2, Y1) and torch.equal(L.Wa, Wa1)
    g2 = [t.clone() for t in L.backward(None, G)]
    torch.cuda.synchronize()
    for u, v in zip(g1, g2):
        assert torch.equal(u, v)


def test_two_streams_match_one_stream():
    """Two layers' forward and backward issued on two HIP streams at once (each
    call with its own workspace, as the header allows) give the one-stream
    results bit for bit: the library keeps no state shared between calls."""
    import torch
    from orthogonal_equivalence_cayley_amd import build_many, param_grad_many
    specs = [workloads.small_case(512, 256, (256, 256), (128, 128), T=600, seed=41 + i, dtype="bf16",
                                  theta_std=0.01) for i in range(2)]
    layers = [make_layer(inp, 4, "bf16") for inp in specs]
    X = [to_dev(inp.X, "bf16") for inp in specs]
    G = [to_dev(inp.G_Y, "bf16") for inp in specs]
    outs = [dict(Y=torch.empty(600, 512, dtype=torch.bfloat16, device="cuda"),
                 GX=torch.empty(600, 256, dtype=torch.bfloat16, device="cuda"),
                 g=[torch.empty(L.nparam[s], dtype=torch.float32, device="cuda") for s in (0, 1)])
            for L in layers]

    def run(two):
        main = torch.cuda.current_stream()
        side = torch.cuda.Stream() if two else main
        build_many(layers)
        side.wait_stream(main)
        for i, L in enumerate(layers):
            with torch.cuda.stream(side if (two and i == 1) else main):
                L.forward(X[i], Y=outs[i]["Y"])
        for i, L in enumerate(layers):
            with torch.cuda.stream(side if (two and i == 1) else main):
                L.backward_dq(X[i], G[i], G_X=outs[i]["GX"])
        main.wait_stream(side)
        param_grad_many(layers, [o["g"] for o in outs])
        torch.cuda.synchronize()
        return [[o["Y"].clone(), o["GX"].clone(), o["g"][0].clone(), o["g"][1].clone()] for o in outs]

    one = run(False)
    for _ in range(2):
        two = run(True)
        for a, b in zip(one, two):
            for u, v in zip(a, b):
                assert torch.equal(u, v)
    ref = oracle.layer_reference(specs[1], 4)
    _compare(dict(Y=to_np(one[1][0]), G_X=to_np(one[1][1])), ref, ["Y", "G_X"], TOL_BF16, "streams")


# ---------------------------------------------------------------- outer loop

@pytest.mark.parametrize("dt, c", [
    ("f32", dict(m=96, n=130, bR=(32, 64), bP=(65, 65), k=2)),
    ("f32", dict(m=12, n=9, bR=(5, 7), bP=(4, 1, 4), k=0)),
    ("bf16", dict(m=512, n=256, bR=(256, 256), bP=(128, 128), k=4)),
    ("bf16", dict(m=768, n=1024, bR=(512, 256), bP=(256,) * 4, k=3)),
])
def test_merge_weight(dt, c):
    """R W0 P from the built blocks, in the original coordinates."""
    import torch
    inp = workloads.small_case(c["m"], c["n"], c["bR"], c["bP"], T=1, seed=c["n"] + 3, dtype=dt,
                               theta_std=0.05 if dt == "f32" else 0.01)
    log(f"merge {dt} {c}")
    L = make_layer(inp, c["k"], dt)
    L.build()
    W = L.merge()
    torch.cuda.synchronize()
    want = oracle.merge_weight(inp.W0, inp.theta_R, inp.theta_P, inp.pi_R, inp.pi_P, c["bR"], c["bP"],
                               c["k"])
    err = oracle.rel_fro(to_np(W), want)
    log(f"  rel_fro={err:.3e}")
    # fp32: accumulation only; bf16: one rounding of the result (<= 2^-9 per element)
    assert err <= (TOL_F32 if dt == "f32" else 4e-3)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_outer_loop_keeps_the_layer(dt):
    """merge, then theta = 0 and new permutations: the layer computes the same
    map (up to the rounding of the merged weight)."""
    import torch
    inp = workloads.small_case(512, 256, (256, 256), (128, 128), T=300, seed=17, dtype=dt,
                               theta_std=0.05 if dt == "f32" else 0.01)
    L = make_layer(inp, 4, dt)
    L.build()
    X = to_dev(inp.X, dt)
    Y1 = L.forward(X, save=False).clone()
    W = L.merge()
    rng = np.random.default_rng(99)
    pR = rng.permutation(512).astype(np.int32)
    pP = rng.permutation(256).astype(np.int32)
    L.set_weight(W, torch.from_numpy(pR), torch.from_numpy(pP))
    L.set_theta(torch.zeros(L.nparam[0]), torch.zeros(L.nparam[1]))
    L.build()
    Y2 = L.forward(X, save=False)
    torch.cuda.synchronize()
    ref = oracle.layer_reference(inp, 4, backward_pass=False)["Y"]
    tol = TOL_F32 if dt == "f32" else TOL_BF16
    assert oracle.rel_fro(to_np(Y1), ref) <= tol
    assert oracle.rel_fro(to_np(Y2), ref) <= tol
    assert oracle.rel_fro(to_np(Y2), to_np(Y1)) <= tol


# ---------------------------------------------------------------- INT8 frozen weight

def _int8_inputs(m, n, bR, bP, T, seed):
    inp = workloads.small_case(m, n, bR, bP, T=T, seed=seed, dtype="bf16", theta_std=0.01)
    inp.W0[5] = 0.0                       # a zero row: scale 0
    inp.W0[7, 3] = 40.0                   # a row with one large entry (bf16-exact)
    return inp


def _dequantized(inp):
    import dataclasses
    q, s = oracle.quantize_rows(inp.W0)
    return dataclasses.replace(inp, W0=oracle.dequantize_rows(q, s)), q, s


@pytest.mark.parametrize("m, n", [(512, 768), (256, 256), (1024, 512)])
def test_quantize_weight_bitexact(m, n):
    import torch
    inp = _int8_inputs(m, n, (256,) * (m // 256), (256,) * (n // 256), T=1, seed=m + n)
    log(f"quantize {m}x{n}")
    L = make_layer(inp, 2, "bf16", weight="int8")
    q, s = L.int8_weight()
    torch.cuda.synchronize()
    q0, s0 = oracle.quantize_rows(inp.W0)
    assert np.array_equal(q.cpu().numpy(), q0[inp.pi_R][:, inp.pi_P])
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s0[inp.pi_R].view(np.uint32))


@pytest.mark.parametrize("case", [
    dict(m=512, n=256, bR=(256, 256), bP=(256,), T=300, k=4),
    dict(m=256, n=768, bR=(256,), bP=(512, 256), T=1000, k=3),
    dict(m=512, n=512, bR=(128, 128, 256), bP=(256, 256), T=77, k=2),
])
@pytest.mark.parametrize("save", [True, False])
def test_layer_int8_weight(case, save):
    """POET-XQ: forward and backward with the INT8 weight against the oracle on
    the dequantised weight (saved Wa and recomputed Wa)."""
    import torch
    c = case
    inp = _int8_inputs(c["m"], c["n"], c["bR"], c["bP"], T=c["T"], seed=c["T"])
    log(f"int8 layer {c} save={save}")
    L = make_layer(inp, c["k"], "bf16", weight="int8")
    L.build()
    X, G = to_dev(inp.X, "bf16"), to_dev(inp.G_Y, "bf16")
    Y = L.forward(X, save=save)
    G_X, gR, gP = L.backward(X, G)
    torch.cuda.synchronize()
    deq, _, _ = _dequantized(inp)
    ref = oracle.layer_reference(deq, c["k"])
    got = dict(Y=to_np(Y), G_X=to_np(G_X), g_theta_R=to_np(gR), g_theta_P=to_np(gP))
    _compare(got, ref, ["Y", "G_X", "g_theta_R", "g_theta_P"], TOL_BF16, "int8")


@pytest.mark.parametrize("size", ["small", "whole_tiles"])
@pytest.mark.parametrize("save", [True, False])
def test_int8_weight_kept_with_transpose(save, size):
    """POETX_WEIGHT_INT8_ROWS_T: quantize_weight also writes qT (the exact
    transpose of q), and every output equals the INT8_ROWS plan's bit for bit
    (the backward's weight product reads qT K-contiguous, same MFMA order).
    whole_tiles: 1024 x 1024 at 16384 tokens, on whole 256 x 256 tiles with at
    least one tile per CU (the int8_t plan's backward on the NT kernel, the int8
    plan's on the NN kernel)."""
    import torch
    if size == "small":
        m, n, T = 512, 768, 333
        inp = _int8_inputs(m, n, (256, 256), (256,) * 3, T=T, seed=12)
    else:
        m, n, T = 1024, 1024, 16384
        inp = _int8_inputs(m, n, (256,) * 4, (256,) * 4, T=T, seed=13)
    outs = []
    for weight in ("int8", "int8_t"):
        L = make_layer(inp, 4, "bf16", weight=weight)
        L.build()
        X, G = to_dev(inp.X, "bf16"), to_dev(inp.G_Y, "bf16")
        Y = L.forward(X, save=save)
        G_X, gR, gP = L.backward(X, G)
        torch.cuda.synchronize()
        outs.append([Y, G_X, gR, gP])
        if weight == "int8_t":
            q, _ = L.int8_weight()
            mn = m * n
            off = ((mn + 255) // 256 * 256 + 4 * m + 255) // 256 * 256
            assert L.plan.weight_bytes() == off + mn
            qT = L.Wt[off:off + mn].view(torch.int8).view(n, m)
            assert torch.equal(qT.cpu(), q.cpu().t().contiguous())
    for a, b in zip(*outs):
        assert torch.equal(_bits(a), _bits(b))


def test_merge_int8_weight():
    import torch
    inp = _int8_inputs(512, 256, (256, 256), (256,), T=1, seed=3)
    L = make_layer(inp, 4, "bf16", weight="int8")
    L.build()
    W = L.merge()
    torch.cuda.synchronize()
    deq, _, _ = _dequantized(inp)
    want = oracle.merge_weight(deq.W0, inp.theta_R, inp.theta_P, inp.pi_R, inp.pi_P, (256, 256),
                               (256,), 4)
    assert oracle.rel_fro(to_np(W), want) <= 4e-3


# ---------------------------------------------------------------- exact Cayley transform

@pytest.mark.parametrize("dt, c", [
    ("f32", dict(m=96, n=130, bR=(32, 64), bP=(65, 65), T=130, std=0.03)),
    ("f32", dict(m=70, n=45, bR=(30, 40), bP=(45,), T=9, std=0.05)),
    ("bf16", dict(m=512, n=256, bR=(256, 256), bP=(128, 128), T=300, std=0.01)),
    # generators near and far past ||S||_2 = 1, where no truncated series converges
    ("f32", dict(m=128, n=96, bR=(64, 64), bP=(32, 64), T=50, std=0.06)),
    ("f32", dict(m=96, n=130, bR=(32, 64), bP=(65, 65), T=40, std=0.25)),
    ("f32", dict(m=64, n=32, bR=(32, 32), bP=(32,), T=20, std=2.0)),
    ("bf16", dict(m=256, n=512, bR=(256,), bP=(256, 256), T=200, std=0.06)),
])
def test_exact_cayley_layer(dt, c):
    """Exact-Cayley mode: blocks, forward and backward against the oracle's
    solve-based transform and its closed-form gradient."""
    import torch
    from orthogonal_equivalence_cayley_amd import PoetxLayer
    inp = workloads.small_case(c["m"], c["n"], c["bR"], c["bP"], T=c["T"], seed=c["T"] + 1, dtype=dt,
                               theta_std=c["std"])
    sp = inp.spec
    S = oracle.skew_from_packed(inp.theta_R[:sp.bsz_R[0] * (sp.bsz_R[0] - 1) // 2], sp.bsz_R[0])
    log(f"exact cayley {dt} {c}: ||S||_2 of the first R block {np.linalg.norm(S, 2):.3f}")
    L = PoetxLayer(sp.m, sp.n, sp.bsz_R, sp.bsz_P, 4, dtype=dt, cayley="exact")
    L.set_weight(to_dev(inp.W0, dt), torch.from_numpy(inp.pi_R), torch.from_numpy(inp.pi_P))
    L.set_theta(torch.from_numpy(inp.theta_R), torch.from_numpy(inp.theta_P))
    got, _ = run_layer(inp, 4, dt, layer=L)
    ref = oracle.layer_reference(inp, None)
    _compare(got, ref, ["QR", "QP"], TOL_F32, "exact")
    keys = ["Wa", "Y", "G_X", "g_theta_R", "g_theta_P"]
    _compare(got, ref, keys, TOL_F32 if dt == "f32" else TOL_BF16, "exact")


# ---------------------------------------------------------------- blocks folded into the weight

@pytest.mark.parametrize("dt, c", [
    ("bf16", dict(m=256, n=512, bR=(256,), bP=(256, 128, 128), T=600, k=4)),   # T >= m, n: both folds
    ("bf16", dict(m=512, n=256, bR=(256, 256), bP=(256,), T=384, k=3)),        # T < m: backward fold only
    ("f32", dict(m=64, n=45, bR=(30, 34), bP=(45,), T=100, k=2)),              # generic fp32 products
])
@pytest.mark.parametrize("save", [True, False])
def test_layer_with_folded_blocks(dt, c, save):
    """Plans with the weight-side fold: with T >= m (T >= n) the P (R) blocks
    are folded into the frozen weight instead of being applied to T rows;
    results against the oracle."""
    import torch
    inp = workloads.small_case(c["m"], c["n"], c["bR"], c["bP"], T=c["T"], seed=c["T"] + c["m"], dtype=dt,
                               theta_std=0.01 if dt == "bf16" else 0.05)
    log(f"folded {dt} {c} save={save}")
    L = make_layer(inp, c["k"], dt, fold="weight")
    L.build()
    X, G = to_dev(inp.X, dt), to_dev(inp.G_Y, dt)
    Y = L.forward(X, save=save)
    Wa = L.Wa
    G_X, gR, gP = L.backward(X, G)
    torch.cuda.synchronize()
    ref = oracle.layer_reference(inp, c["k"])
    got = dict(Y=to_np(Y), G_X=to_np(G_X), g_theta_R=to_np(gR), g_theta_P=to_np(gP))
    keys = ["Y", "G_X", "g_theta_R", "g_theta_P"]
    if save:
        got["Wa"] = to_np(Wa)
        keys.append("Wa")
    _compare(got, ref, keys, TOL_F32 if dt == "f32" else TOL_BF16, "folded")


@pytest.mark.parametrize("save", [True, False])
def test_kept_input_permutation_matches_gathering(save):
    """A backward that reads the U = X Pi_P^T the forward kept (X not passed)
    gives the same results, bit for bit, as one that gathers X again."""
    import torch
    inp = workloads.small_case(256, 512, (256,), (256, 256), T=700, seed=44, dtype="bf16",
                               theta_std=0.01)
    L = make_layer(inp, 4, "bf16")
    L.build()
    X, G = to_dev(inp.X, "bf16"), to_dev(inp.G_Y, "bf16")
    L.forward(X, save=save)
    a = [t.clone() for t in L.backward(X, G)]
    L.forward(X, save=save, keep_u=True)
    b = [t.clone() for t in L.backward(None, G)]
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("dt, c", [
    ("bf16", dict(m=768, n=512, bR=(256,) * 3, bP=(256, 256), T=300)),
    ("f32", dict(m=37, n=53, bR=(37,), bP=(20, 33), T=41)),
])
def test_weight_kept_with_transpose(dt, c):
    """POETX_WEIGHT_DENSE_T: permute_weight also writes WtT (bit-exact
    transpose), and the backward that reads it gives the oracle's results."""
    import torch
    inp = workloads.small_case(c["m"], c["n"], c["bR"], c["bP"], T=c["T"], seed=c["m"] + 11, dtype=dt,
                               theta_std=0.01 if dt == "bf16" else 0.05)
    log(f"dense_t {dt} {c}")
    L = make_layer(inp, 3, dt, weight="dense_t")
    D = make_layer(inp, 3, dt)
    torch.cuda.synchronize()
    m, n = c["m"], c["n"]
    es = 2 if dt == "bf16" else 4
    off = (m * n * es + 255) // 256 * 256
    WtT = L._wbuf[off:off + m * n * es].view(L.tdtype).view(n, m)
    assert torch.equal(_bits(L.Wt), _bits(D.Wt))
    assert torch.equal(_bits(WtT), _bits(D.Wt.t().contiguous()))
    got, _ = run_layer(inp, 3, dt, layer=L)
    ref = oracle.layer_reference(inp, 3)
    _compare(got, ref, ["Wa", "Y", "G_X", "g_theta_R", "g_theta_P"], TOL_F32 if dt == "f32" else TOL_BF16,
             "dense_t")



@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("k", [0, 1, 2, 3, 4, 5, 6, 7, 8, 12, 32])
def test_paterson_stockmeyer_build(dt, k):
    """POETX_SERIES_PS builds the same Q = sum_j c_j S^j as the power chain:
    against the oracle's build at 1e-5 for every k the plans take a few of
    (including k = 0, where Q = I + S, and the largest, 32), blocks of 32, 96,
    256 and 512."""
    import torch
    from orthogonal_equivalence_cayley_amd import PoetxLayer
    bsz = (32, 96, 256, 512) if dt == "f32" else (256, 512, 32, 96)
    n = sum(bsz)
    rng = np.random.default_rng(100 + k)
    npar = sum(b * (b - 1) // 2 for b in bsz)
    theta = (rng.standard_normal(npar) * 0.005).astype(np.float32)
    log(f"PS build {dt} k={k}")
    L = PoetxLayer(n, n, bsz, bsz, k, dtype=dt, series="ps")
    L.set_theta(torch.from_numpy(theta), torch.from_numpy(theta))
    L.build()
    torch.cuda.synchronize()
    want = blocks_concat(oracle.build_orth(theta, bsz, k))
    for side in (0, 1):
        err = oracle.rel_fro(to_np(L.Q32[side]), want)
        log(f"  side {side}: rel_fro={err:.3e}")
        assert err <= TOL_F32, (side, err)
    if dt == "bf16":
        # the activation copy is the round-to-nearest-even bf16 of the fp32 Q
        assert torch.equal(L.Qact[0].view(torch.int16).cpu(),
                           L.Q32[0].to(torch.bfloat16).view(torch.int16).cpu())


def test_paterson_stockmeyer_layer():
    """A whole layer (build, forward, backward) with the Paterson-Stockmeyer
    build against the oracle."""
    inp = workloads.small_case(512, 768, (256, 256), (256,) * 3, T=150, seed=77, dtype="bf16",
                               theta_std=0.01)
    import torch
    from orthogonal_equivalence_cayley_amd import PoetxLayer
    sp = inp.spec
    L = PoetxLayer(sp.m, sp.n, sp.bsz_R, sp.bsz_P, 4, dtype="bf16", series="ps")
    L.set_weight(to_dev(inp.W0, "bf16"), torch.from_numpy(inp.pi_R), torch.from_numpy(inp.pi_P))
    L.set_theta(torch.from_numpy(inp.theta_R), torch.from_numpy(inp.theta_P))
    got, _ = run_layer(inp, 4, "bf16", layer=L)
    ref = oracle.layer_reference(inp, 4)
    _compare(got, ref, ["QR", "QP"], TOL_F32, "ps")
    _compare(got, ref, ["Wa", "Y", "G_X", "g_theta_R", "g_theta_P"], TOL_BF16, "ps")


@pytest.mark.parametrize("T", [1, 63, 64, 65, 1000, 4097])
@pytest.mark.parametrize("save", [True, False])
def test_backward_token_tiles(T, save):
    """Backward of sides of 256-wide blocks at token counts around the 64-token
    tile of the dL/dQ reduction and its splits, and with a ragged tail, against
    the oracle (save=False: POET-Xmem recomputation)."""
    inp = workloads.small_case(512, 768, (256, 256), (256,) * 3, T=T, seed=T + 3, dtype="bf16",
                               theta_std=0.01)
    log(f"backward T={T} save={save}")
    L = make_layer(inp, 4, "bf16")
    L.build()
    import torch
    X, G = to_dev(inp.X, "bf16"), to_dev(inp.G_Y, "bf16")
    L.forward(X, save=save)
    G_X, gR, gP = L.backward(X, G)
    torch.cuda.synchronize()
    ref = oracle.layer_reference(inp, 4)
    got = dict(G_X=to_np(G_X), g_theta_R=to_np(gR), g_theta_P=to_np(gP))
    _compare(got, ref, ["G_X", "g_theta_R", "g_theta_P"], TOL_BF16, "backward")
