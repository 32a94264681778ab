"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties the oracle to something other than itself: a closed form, an
invariant, a textbook routine (scipy solve, block_diag, SVD), explicit
permutation matrices, or finite differences. A dropped term, a wrong sign or
index, or a transposed operand anywhere in the oracle fails at least one.

Citations
  [PX]   page "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
         Transformation" (gist.science), section "Résumé technique".
  [Pion] page "Pion：保持谱稳定的大语言模型训练优化器", section "数学原理".
"""
import numpy as np
import pytest
import scipy.linalg

import oracle
import workloads


def _rand_skew(b, scale, seed):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((b, b)) * scale
    return np.triu(A, 1) - np.triu(A, 1).T


# --------------------------------------------------------------------------
# packed storage ([PX] §2.D: b(b-1)/2 parameters per block)

def test_packed_order_b3():
    S = oracle.skew_from_packed(np.array([1.5, -2.0, 0.25]), 3)
    want = np.array([[0.0, 1.5, -2.0],
                     [-1.5, 0.0, 0.25],
                     [2.0, -0.25, 0.0]])
    assert np.array_equal(S, want)
    assert np.array_equal(oracle.packed_upper(S), [1.5, -2.0, 0.25])


@pytest.mark.parametrize("b", [2, 3, 32, 256, 512])
def test_parameter_count(b):
    th = np.arange(b * (b - 1) // 2, dtype=np.float64)
    S = oracle.skew_from_packed(th, b)
    assert np.array_equal(S, -S.T)
    assert oracle.packed_upper(S).size == b * (b - 1) // 2


def test_workload_parameter_totals():
    # 7 hidden-2048 linears with b=256: 5 026 560 skew parameters;
    # 7 hidden-4096 linears with b=512 (+ one 256 tail): 19 851 136.
    for cid, want in ((4, 5026560), (5, 19851136)):
        w = workloads.WORKLOADS[cid]
        got = sum(workloads.n_params(l.bsz_R) + workloads.n_params(l.bsz_P) for l in w.layers)
        assert got == want
        for l in w.layers:
            assert sum(l.bsz_R) == l.m and sum(l.bsz_P) == l.n


# --------------------------------------------------------------------------
# Cayley-Neumann blocks ([PX] §2.D; orthogonality Q^T Q = I from [Pion] 数学原理)

@pytest.mark.parametrize("k", [0, 1, 2, 3, 4, 5])
@pytest.mark.parametrize("b", [4, 32])
def test_orthogonality_defect_closed_form(b, k):
    # (I+S) N_k with N_k = (I-S)^{-1}(I - S^{k+1}) gives
    # Q^T Q = (I - (-S)^{k+1})(I - S^{k+1}) exactly.
    S = _rand_skew(b, 0.3 / np.sqrt(b), seed=b * 10 + k)
    Q = oracle.neumann_cayley(S, k)
    I = np.eye(b)
    Sk1 = np.linalg.matrix_power(S, k + 1)
    mSk1 = np.linalg.matrix_power(-S, k + 1)
    want = (I - mSk1) @ (I - Sk1)
    assert np.max(np.abs(Q.T @ Q - want)) < 1e-13
    # and the defect is of the order ||S||^(k+1)
    nS = np.linalg.norm(S, 2)
    assert np.linalg.norm(Q.T @ Q - I, 2) <= 2.0 * nS ** (k + 1) + nS ** (2 * k + 2) + 1e-14


@pytest.mark.parametrize("k", [0, 1, 3, 4, 5, 8])
def test_convergence_to_exact_cayley(k):
    # Q_k - Q_inf = -Q_inf S^{k+1}; S is normal so ||Q_k - Q_inf||_2 = ||S||_2^{k+1}
    b = 32
    S = _rand_skew(b, 0.5 / np.sqrt(b), seed=77 + k)
    I = np.eye(b)
    Qinf = scipy.linalg.solve(I - S, I + S)
    Qk = oracle.neumann_cayley(S, k)
    Sk1 = np.linalg.matrix_power(S, k + 1)
    assert np.max(np.abs((Qk - Qinf) + Qinf @ Sk1)) < 1e-13
    nS = np.linalg.norm(S, 2)
    assert abs(np.linalg.norm(Qk - Qinf, 2) - nS ** (k + 1)) <= 1e-10 * max(nS ** (k + 1), 1e-300) + 1e-15


def test_neumann_limit_is_orthogonal():
    b = 64
    S = _rand_skew(b, 0.3 / np.sqrt(b), seed=5)
    Q = oracle.neumann_cayley(S, 60)
    assert np.max(np.abs(Q.T @ Q - np.eye(b))) < 1e-14
    assert np.max(np.abs(Q - scipy.linalg.solve(np.eye(b) - S, np.eye(b) + S))) < 1e-14


@pytest.mark.parametrize("k", [0, 1, 2, 3, 4, 5, 9])
def test_two_by_two_closed_form(k):
    t = 0.37
    S = np.array([[0.0, t], [-t, 0.0]])          # S^2 = -t^2 I
    a = sum((-t * t) ** (j // 2) for j in range(0, k + 1, 2))   # even powers
    c = sum((-t * t) ** (j // 2) for j in range(1, k + 1, 2))   # odd powers (times S)
    # (I + S)(a I + c S) = (a - c t^2) I + (a + c) S
    want = np.array([[a - c * t * t, (a + c) * t], [-(a + c) * t, a - c * t * t]])
    Q = oracle.neumann_cayley(S, k)
    assert np.max(np.abs(Q - want)) < 1e-15
    # textbook rotation for the exact transform
    Qinf = oracle.neumann_cayley(S, 200)
    cth, sth = (1 - t * t) / (1 + t * t), 2 * t / (1 + t * t)
    assert np.max(np.abs(Qinf - np.array([[cth, sth], [-sth, cth]]))) < 1e-15


def test_build_orth_block_layout():
    bsz = (3, 5, 2)
    rng = np.random.default_rng(3)
    th = rng.standard_normal(workloads.n_params(bsz)) * 0.1
    Qs = oracle.build_orth(th, bsz, 3)
    off = 0
    for b, Q in zip(bsz, Qs):
        cnt = b * (b - 1) // 2
        assert Q.shape == (b, b)
        assert np.allclose(Q, oracle.neumann_cayley(oracle.skew_from_packed(th[off:off + cnt], b), 3))
        off += cnt


# --------------------------------------------------------------------------
# structure: blocks, permutations, input-centric = materialised ([PX] §2.A-§2.C)

def _materialise(inp, k):
    sp = inp.spec
    QR = oracle.build_orth(inp.theta_R, sp.bsz_R, k)
    QP = oracle.build_orth(inp.theta_P, sp.bsz_P, k)
    PiR = np.eye(sp.m)[inp.pi_R]                # (Pi v)_i = v[pi[i]]
    PiP = np.eye(sp.n)[inp.pi_P]
    R = PiR.T @ scipy.linalg.block_diag(*QR) @ PiR
    P = PiP.T @ scipy.linalg.block_diag(*QP) @ PiP
    return R, P, QR, QP


def test_blocks_equal_block_diag():
    bsz = (4, 7, 5)
    rng = np.random.default_rng(11)
    Qs = [rng.standard_normal((b, b)) for b in bsz]
    A = rng.standard_normal((9, sum(bsz)))
    D = scipy.linalg.block_diag(*Qs)
    assert np.max(np.abs(oracle.apply_blocks_T(A, Qs, bsz) - A @ D.T)) < 1e-13
    assert np.max(np.abs(oracle.apply_blocks(A, Qs, bsz) - A @ D)) < 1e-13


def test_gather_is_permutation_matrix():
    inp = workloads.small_case(6, 8, (3, 3), (4, 4), T=5, seed=2)
    PiP = np.eye(8)[inp.pi_P]
    Wt = oracle.permute_weight(inp.W0, inp.pi_R, inp.pi_P)
    # with identity blocks the forward is exactly Y Pi_R^T = X Pi_P^T Wt^T
    I3, I4 = [np.eye(3)] * 2, [np.eye(4)] * 2
    Y, Wa = oracle.forward(inp.X, Wt, inp.pi_R, inp.pi_P, I3, I4, (3, 3), (4, 4))
    assert np.array_equal(Wa, (inp.X.astype(np.float64) @ PiP.T) @ Wt.T)
    PiR = np.eye(6)[inp.pi_R]
    assert np.array_equal(Y, Wa @ PiR)
    assert np.array_equal(Wt, PiR @ inp.W0.astype(np.float64) @ PiP.T)


@pytest.mark.parametrize("case", [
    dict(m=12, n=8, bR=(4, 4, 4), bP=(4, 4), k=3),
    dict(m=12, n=8, bR=(5, 3, 4), bP=(2, 6), k=2),
    dict(m=7, n=9, bR=(7,), bP=(1, 8), k=0),
])
def test_input_centric_equals_materialised(case):
    inp = workloads.small_case(case["m"], case["n"], case["bR"], case["bP"], T=6, seed=19, theta_std=0.2)
    k = case["k"]
    R, P, QR, QP = _materialise(inp, k)
    W = R @ inp.W0.astype(np.float64) @ P
    want = inp.X.astype(np.float64) @ W.T              # y = R W0 P x per token
    Wt = oracle.permute_weight(inp.W0, inp.pi_R, inp.pi_P)
    Y, _ = oracle.forward(inp.X, Wt, inp.pi_R, inp.pi_P, QR, QP, case["bR"], case["bP"])
    assert oracle.rel_fro(Y, want) < 1e-14


def test_theta_zero_is_plain_linear():
    inp = workloads.small_case(24, 16, (8, 8, 8), (8, 8), T=10, seed=4)
    z = lambda bsz: np.zeros(workloads.n_params(bsz))
    QR = oracle.build_orth(z((8, 8, 8)), (8, 8, 8), 4)
    QP = oracle.build_orth(z((8, 8)), (8, 8), 4)
    for Q in QR + QP:
        assert np.array_equal(Q, np.eye(8))
    Wt = oracle.permute_weight(inp.W0, inp.pi_R, inp.pi_P)
    Y, _ = oracle.forward(inp.X, Wt, inp.pi_R, inp.pi_P, QR, QP, (8, 8, 8), (8, 8))
    assert np.max(np.abs(Y - inp.X.astype(np.float64) @ inp.W0.astype(np.float64).T)) < 1e-13


def test_spectrum_preserved():
    # [PX] §1 / [Pion] 数学原理: orthogonal equivalence keeps the singular values
    inp = workloads.small_case(16, 12, (4, 4, 8), (6, 6), T=2, seed=8, theta_std=0.05)
    W0 = inp.W0.astype(np.float64)
    s0 = np.linalg.svd(W0, compute_uv=False)
    R, P, _, _ = _materialise(inp, 80)           # Neumann limit (||S|| < 1)
    s = np.linalg.svd(R @ W0 @ P, compute_uv=False)
    assert np.max(np.abs(s - s0)) / s0[0] < 1e-12
    # truncated series: off only by the orthogonality defect
    R3, P3, _, _ = _materialise(inp, 3)
    s3 = np.linalg.svd(R3 @ W0 @ P3, compute_uv=False)
    dR = np.linalg.norm(R3.T @ R3 - np.eye(16), 2)
    dP = np.linalg.norm(P3.T @ P3 - np.eye(12), 2)
    assert np.max(np.abs(s3 - s0)) / s0[0] <= dR + dP + 1e-12
    assert np.max(np.abs(s3 - s0)) / s0[0] > 1e-8       # and not exact


# --------------------------------------------------------------------------
# backward

def _loss(inp, thR, thP, X, k):
    sp = inp.spec
    QR = oracle.build_orth(thR, sp.bsz_R, k)
    QP = oracle.build_orth(thP, sp.bsz_P, k)
    Wt = oracle.permute_weight(inp.W0, inp.pi_R, inp.pi_P)
    Y, _ = oracle.forward(X, Wt, inp.pi_R, inp.pi_P, QR, QP, sp.bsz_R, sp.bsz_P)
    return float(np.sum(Y * inp.G_Y.astype(np.float64)))


@pytest.mark.parametrize("k", [0, 1, 3, 4])
def test_backward_matches_finite_differences(k):
    inp = workloads.small_case(10, 9, (4, 6), (5, 1, 3), T=4, seed=31 + k, theta_std=0.3)
    thR = inp.theta_R.astype(np.float64)
    thP = inp.theta_P.astype(np.float64)
    X = inp.X.astype(np.float64)
    ref = oracle.layer_reference(
        type("I", (), dict(spec=inp.spec, theta_R=thR, theta_P=thP, W0=inp.W0, pi_R=inp.pi_R,
                           pi_P=inp.pi_P, X=X, G_Y=inp.G_Y))(), k)
    h = 1e-6

    def fd(vec, setter):
        g = np.zeros_like(vec)
        for i in range(vec.size):
            e = np.zeros_like(vec)
            e.flat[i] = h
            g.flat[i] = (setter(vec + e) - setter(vec - e)) / (2 * h)
        return g

    gR = fd(thR, lambda v: _loss(inp, v, thP, X, k))
    gP = fd(thP, lambda v: _loss(inp, thR, v, X, k))
    gX = fd(X, lambda v: _loss(inp, thR, thP, v, k))
    assert oracle.rel_fro(ref["g_theta_R"], gR) < 1e-7
    assert oracle.rel_fro(ref["g_theta_P"], gP) < 1e-7
    assert oracle.rel_fro(ref["G_X"], gX) < 1e-7


def test_cnp_gradient_exact_cayley_limit():
    # dQ_inf = (I + Q_inf) dS (I - S)^{-1}  =>  dL/dS = (I + Q_inf)^T G (I + S)^{-1}
    b = 16
    S = _rand_skew(b, 0.4 / np.sqrt(b), seed=123)
    G = np.random.default_rng(9).standard_normal((b, b))
    I = np.eye(b)
    Qinf = scipy.linalg.solve(I - S, I + S)
    want = (I + Qinf).T @ G @ np.linalg.inv(I + S)
    got = oracle.cnp_backward(G, S, 90)
    assert oracle.rel_fro(got, want) < 1e-12


def test_cnp_gradient_k0_is_identity_map():
    # k = 0: Q = I + S, so dL/dS = G exactly
    b = 6
    S = _rand_skew(b, 0.2, seed=1)
    G = np.random.default_rng(2).standard_normal((b, b))
    assert np.array_equal(oracle.cnp_backward(G, S, 0), G)


def test_cnp_coefficients():
    assert oracle.cnp_coefficients(0) == [1.0, 1.0]
    assert oracle.cnp_coefficients(3) == [1.0, 2.0, 2.0, 2.0, 1.0]


# --------------------------------------------------------------------------
# restricted forms used for sampled checks at full size agree with the full oracle

def test_restricted_forms_match_full_oracle():
    inp = workloads.small_case(24, 20, (8, 16), (4, 12, 4), T=9, seed=61, theta_std=0.1)
    k = 3
    ref = oracle.layer_reference(inp, k)
    sp = inp.spec
    rows = [0, 4, 8]
    Yr = oracle.forward_rows(inp.X[rows], ref["Wt"], inp.pi_R, inp.pi_P, ref["QR"], ref["QP"],
                             sp.bsz_R, sp.bsz_P)
    assert np.max(np.abs(Yr - ref["Y"][rows])) < 1e-14
    Gr = oracle.backward_rows(inp.G_Y[rows], ref["Wt"], inp.pi_R, inp.pi_P, ref["QR"], ref["QP"],
                              sp.bsz_R, sp.bsz_P)
    assert np.max(np.abs(Gr - ref["G_X"][rows])) < 1e-13
    offs = {"R": np.cumsum([0] + [b * (b - 1) // 2 for b in sp.bsz_R]),
            "P": np.cumsum([0] + [b * (b - 1) // 2 for b in sp.bsz_P])}
    for side, nb, full in (("R", 2, ref["g_theta_R"]), ("P", 3, ref["g_theta_P"])):
        for j in range(nb):
            g = oracle.theta_grad_block(side, j, inp.X, ref["Wt"], inp.pi_R, inp.pi_P, inp.theta_R,
                                        inp.theta_P, ref["QR"], ref["QP"], inp.G_Y, sp.bsz_R,
                                        sp.bsz_P, k)
            assert np.max(np.abs(g - full[offs[side][j]:offs[side][j + 1]])) < 1e-12


# --------------------------------------------------------------------------
# merge at the end of an inner loop

def test_merge_two_by_two_by_hand():
    # one 2x2 block per side, identity permutations, k = 0: Q = I + S, so
    # R = [[1, a], [-a, 1]] and P = [[1, c], [-c, 1]]
    a, c = 0.3, -0.7
    W0 = np.array([[2.0, -1.0], [0.5, 3.0]])
    got = oracle.merge_weight(W0, [a], [c], [0, 1], [0, 1], (2,), (2,), 0)
    w11, w12, w21, w22 = 2.0, -1.0, 0.5, 3.0
    RW = np.array([[w11 + a * w21, w12 + a * w22], [w21 - a * w11, w22 - a * w12]])
    want = np.array([[RW[0, 0] - c * RW[0, 1], c * RW[0, 0] + RW[0, 1]],
                     [RW[1, 0] - c * RW[1, 1], c * RW[1, 0] + RW[1, 1]]])
    assert np.max(np.abs(got - want)) < 1e-15
    # swapping both coordinates of a side (pi = [1, 0]) swaps the roles of the
    # two rows (columns): R' = Pi^T R Pi with R' = [[1, -a], [a, 1]]
    got2 = oracle.merge_weight(W0, [a], [0.0], [1, 0], [0, 1], (2,), (2,), 0)
    R2 = np.array([[1.0, -a], [a, 1.0]])
    assert np.max(np.abs(got2 - R2 @ W0)) < 1e-15


@pytest.mark.parametrize("case", [
    dict(m=12, n=8, bR=(4, 4, 4), bP=(4, 4), k=3),
    dict(m=10, n=9, bR=(3, 7), bP=(2, 7), k=1),
])
def test_merge_is_the_layer_map_and_survives_resampling(case):
    inp = workloads.small_case(case["m"], case["n"], case["bR"], case["bP"], T=7, seed=31, theta_std=0.2)
    k, bR, bP = case["k"], case["bR"], case["bP"]
    QR = oracle.build_orth(inp.theta_R, bR, k)
    QP = oracle.build_orth(inp.theta_P, bP, k)
    Wt = oracle.permute_weight(inp.W0, inp.pi_R, inp.pi_P)
    Y, _ = oracle.forward(inp.X, Wt, inp.pi_R, inp.pi_P, QR, QP, bR, bP)
    Wn = oracle.merge_weight(inp.W0, inp.theta_R, inp.theta_P, inp.pi_R, inp.pi_P, bR, bP, k)
    # the input-centric forward computes x -> W_new x
    assert oracle.rel_fro(inp.X.astype(np.float64) @ Wn.T, Y) < 1e-14
    # next inner loop: theta = 0 and fresh permutations give the same layer
    rng = np.random.default_rng(5)
    pR, pP = rng.permutation(case["m"]), rng.permutation(case["n"])
    I_R = oracle.build_orth(np.zeros(workloads.n_params(bR)), bR, k)
    I_P = oracle.build_orth(np.zeros(workloads.n_params(bP)), bP, k)
    Y2, _ = oracle.forward(inp.X, oracle.permute_weight(Wn, pR, pP), pR, pP, I_R, I_P, bR, bP)
    assert oracle.rel_fro(Y2, Y) < 1e-14
    # theta = 0 merges to W0 itself
    W00 = oracle.merge_weight(inp.W0, np.zeros(workloads.n_params(bR)), np.zeros(workloads.n_params(bP)),
                              inp.pi_R, inp.pi_P, bR, bP, k)
    assert np.array_equal(W00, inp.W0.astype(np.float64))


def test_merge_preserves_the_spectrum_in_the_cayley_limit():
    inp = workloads.small_case(16, 12, (4, 4, 8), (6, 6), T=2, seed=8, theta_std=0.05)
    W0 = inp.W0.astype(np.float64)
    Wn = oracle.merge_weight(W0, inp.theta_R, inp.theta_P, inp.pi_R, inp.pi_P, (4, 4, 8), (6, 6), 80)
    s0 = np.linalg.svd(W0, compute_uv=False)
    s = np.linalg.svd(Wn, compute_uv=False)
    assert np.max(np.abs(s - s0)) / s0[0] < 1e-12
    assert oracle.rel_fro(Wn, W0) > 1e-3      # and the weight did change


# --------------------------------------------------------------------------
# INT8 frozen weight

def test_quantize_rows_bounds_and_grid():
    rng = np.random.default_rng(12)
    W = (rng.standard_normal((40, 70)) * rng.uniform(0.01, 3.0, size=(40, 1))).astype(np.float32)
    W[3] = 0.0                                          # an all-zero row
    q, s = oracle.quantize_rows(W)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    amax = np.abs(W).max(axis=1)
    # the largest entry of every non-zero row maps to +-127 and the scale is amax / 127
    for i in range(40):
        if amax[i] == 0:
            assert s[i] == 0 and np.all(q[i] == 0)
            continue
        assert np.abs(q[i]).max() == 127
        assert abs(float(s[i]) * 127 - float(amax[i])) <= 1e-6 * float(amax[i])
    # every entry within half a step of its grid point (plus float32 rounding)
    err = np.abs(oracle.dequantize_rows(q, s) - W.astype(np.float64))
    assert np.all(err <= 0.5 * s[:, None].astype(np.float64) * (1 + 1e-5) + 1e-12)
    # values already on the grid come back exactly
    W2 = (np.arange(-127, 128, dtype=np.float32) * np.float32(0.25))[None, :].repeat(2, 0)
    q2, s2 = oracle.quantize_rows(W2)
    assert np.array_equal(q2[0], np.arange(-127, 128).astype(np.int8))
    assert np.array_equal(oracle.dequantize_rows(q2, s2), W2.astype(np.float64))


def test_quantize_rows_commutes_with_row_and_column_permutations():
    # one scale per row: permuting rows permutes (q, s); permuting columns only
    # permutes q, so quantising W0 and then pre-merging equals quantising Wt
    rng = np.random.default_rng(4)
    W = rng.standard_normal((16, 24)).astype(np.float32)
    pr, pc = rng.permutation(16), rng.permutation(24)
    q, s = oracle.quantize_rows(W)
    q2, s2 = oracle.quantize_rows(W[pr][:, pc])
    assert np.array_equal(q2, q[pr][:, pc]) and np.array_equal(s2, s[pr])


# --------------------------------------------------------------------------
# exact Cayley transform

def test_exact_cayley_two_by_two_closed_form():
    # S = [[0, a], [-a, 0]]: (I+S)(I-S)^{-1} = [[1-a^2, 2a], [-2a, 1-a^2]] / (1+a^2)
    for a in (0.1, -0.7, 2.5):
        S = np.array([[0.0, a], [-a, 0.0]])
        want = np.array([[1 - a * a, 2 * a], [-2 * a, 1 - a * a]]) / (1 + a * a)
        assert np.max(np.abs(oracle.exact_cayley(S) - want)) < 1e-15


def test_exact_cayley_is_orthogonal_and_the_neumann_limit():
    b = 48
    S = _rand_skew(b, 0.25 / np.sqrt(b), seed=5)      # ||S||_2 about 0.5
    Q = oracle.exact_cayley(S)
    assert np.max(np.abs(Q.T @ Q - np.eye(b))) < 1e-13
    assert np.max(np.abs(Q - oracle.neumann_cayley(S, 120))) < 1e-13
    # also for a generator far outside the Neumann series' radius
    S2 = _rand_skew(b, 3.0 / np.sqrt(b), seed=6)
    Q2 = oracle.exact_cayley(S2)
    assert np.max(np.abs(Q2.T @ Q2 - np.eye(b))) < 1e-12
    assert np.linalg.det(Q2) > 0


def test_exact_cayley_gradient_finite_differences():
    b = 7
    S = _rand_skew(b, 0.8 / np.sqrt(b), seed=41)
    G = np.random.default_rng(2).standard_normal((b, b))
    got = oracle.cayley_backward_exact(G, S)
    h = 1e-6
    for (i, j) in [(0, 1), (2, 5), (6, 3), (4, 4)]:
        E = np.zeros((b, b))
        E[i, j] = 1.0
        fd = (np.sum(G * oracle.exact_cayley(S + h * E)) - np.sum(G * oracle.exact_cayley(S - h * E))) / (2 * h)
        assert abs(fd - got[i, j]) <= 1e-7 * max(1.0, abs(fd))


def test_exact_layer_theta_gradient_finite_differences():
    inp = workloads.small_case(8, 6, (3, 5), (6,), T=4, seed=13, theta_std=0.3)
    sp = inp.spec
    ref = oracle.layer_reference(inp, None)
    h = 1e-6
    for side, th in (("R", inp.theta_R), ("P", inp.theta_P)):
        for idx in (0, len(th) - 1):
            tp = np.array(th, dtype=np.float64)
            tm = tp.copy()
            tp[idx] += h
            tm[idx] -= h
            vals = []
            for t in (tp, tm):
                import dataclasses
                mod = dataclasses.replace(inp, theta_R=t if side == "R" else inp.theta_R,
                                          theta_P=t if side == "P" else inp.theta_P)
                Y = oracle.layer_reference(mod, None, backward_pass=False)["Y"]
                vals.append(float(np.sum(Y * inp.G_Y.astype(np.float64))))
            fd = (vals[0] - vals[1]) / (2 * h)
            g = ref["g_theta_R" if side == "R" else "g_theta_P"][idx]
            assert abs(fd - g) <= 1e-6 * max(1.0, abs(fd))
