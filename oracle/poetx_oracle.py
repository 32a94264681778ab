"""Plain float64 NumPy oracle of the POET-X orthogonal-equivalence layer.

TEST INFRASTRUCTURE. This module is the checker, not the product: only
tests/, the smoke check and the benchmark's cpu_baseline leg may import it.
It shares no code with the HIP library (no kernels, tables or helpers), and
nothing here is tuned: every step is written as the definition reads, one
library primitive (matmul, indexing) per step, in float64. (`precision`
switches the float type, for timing the same steps in float32 as a CPU
throughput figure; every check uses float64.)

Citations
  [PX]   page "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
         Transformation" (gist.science, French), section "Résumé technique".
  [Pion] page "Pion：保持谱稳定的大语言模型训练优化器" (zingnex.cn),
         section "数学原理".

Conventions (readings of the pages, which print no equations)
  * Row form: activations are [T, features]; one token x in R^n maps to
    y = R W0 P x in R^m, so Y = X P^T W0^T R^T.
  * Orthogonal side matrices: P = Pi_P^T D_P Pi_P and R = Pi_R^T D_R Pi_R,
    with (Pi v)_i = v[pi[i]] and D = blockdiag(Q_1, Q_2, ...) over contiguous
    blocks in permuted index space ([PX] §2.B permutations held as index
    arrays; §2.C block-diagonal matrices handled block by block).
  * Each block Q = (I + S)(I - S)^{-1} with the inverse replaced by the
    truncated Neumann series sum_{j=0..k} S^j ([PX] §2.D, Cayley-Neumann
    parameterisation). k = 0 gives Q = I + S.
  * S is skew-symmetric; only its strict upper triangle is stored, row-major
    (numpy.triu_indices(b, 1) order), S[i, j] = +theta, S[j, i] = -theta
    ([PX] §2.D, b(b-1)/2 parameters per block). Blocks' parameters are
    concatenated in block order.
  * Pre-merge ([PX] §2.B, "Réduction"): Wt = Pi_R W0 Pi_P^T, i.e.
    Wt[i, j] = W0[pi_R[i], pi_P[j]]; the forward then needs one gather and
    one scatter.
  * Backward ([PX] §2.E, POET-Xfast keeps one extra activation): the saved
    activation is Wa, the output of the W0 product. Gradients are those of
    the truncated Q the forward uses.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import contextlib

import numpy as np

__all__ = [
    "skew_from_packed", "packed_upper", "neumann_cayley", "build_orth",
    "block_offsets", "apply_blocks_T", "apply_blocks", "permute_weight",
    "forward", "forward_rows", "cnp_backward", "backward", "cnp_coefficients",
    "rel_fro", "layer_reference", "backward_rows", "theta_grad_block", "side_matrix",
    "merge_weight", "quantize_rows", "dequantize_rows", "exact_cayley", "cayley_backward_exact",
    "precision",
]



_DT = np.float64   # the float type of every step (float64 unless `precision` says otherwise)


@contextlib.contextmanager
def precision(dtype):
    """Run the oracle's steps in another float type while the context lasts
    (float32 for a CPU throughput figure); checks use the float64 default."""
    global _DT
    old, _DT = _DT, np.dtype(dtype).type
    try:
        yield
    finally:
        _DT = old


def rel_fro(a, ref) -> float:
    """Relative Frobenius error ||a - ref|| / ||ref|| (0 when both vanish)."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(a - ref)
    if den == 0.0:
        return float(num)
    return float(num / den)


def block_offsets(bsz: Sequence[int]) -> List[int]:
    """Start index of each block in permuted index space (blocks contiguous)."""
    off, out = 0, []
    for b in bsz:
        out.append(off)
        off += int(b)
    return out


def skew_from_packed(theta_blk: np.ndarray, b: int) -> np.ndarray:
    """[PX] §2.D: the skew generator from its stored strict upper triangle."""
    theta_blk = np.asarray(theta_blk, dtype=_DT)
    assert theta_blk.shape == (b * (b - 1) // 2,)
    S = np.zeros((b, b), dtype=_DT)
    iu = np.triu_indices(b, 1)
    S[iu] = theta_blk
    S[(iu[1], iu[0])] = -theta_blk
    return S


def packed_upper(M: np.ndarray) -> np.ndarray:
    """Strict upper triangle of a square matrix, row-major."""
    b = M.shape[0]
    return np.asarray(M, dtype=_DT)[np.triu_indices(b, 1)]


def neumann_cayley(S: np.ndarray, k: int) -> np.ndarray:
    """[PX] §2.D: Cayley transform (I+S)(I-S)^{-1} with the inverse replaced by
    the Neumann series I + S + ... + S^k; powers by repeated multiplication."""
    b = S.shape[0]
    I = np.eye(b, dtype=_DT)
    N = I.copy()
    Pj = I.copy()
    for _ in range(k):
        Pj = Pj @ S
        N = N + Pj
    return (I + S) @ N


def exact_cayley(S: np.ndarray) -> np.ndarray:
    """The Cayley transform itself, Q = (I+S)(I-S)^{-1}, by a linear solve: the
    map [PX] §2.D's Neumann series approximates (exact-Cayley mode)."""
    I = np.eye(S.shape[0], dtype=_DT)
    return (I + S) @ np.linalg.solve(I - S, I)


def cayley_backward_exact(G: np.ndarray, S: np.ndarray) -> np.ndarray:
    """Gradient w.r.t. S of <G, Q(S)> for the exact transform. With
    N = (I-S)^{-1}: dN = N dS N, so dQ = dS N + (I+S) N dS N = (I+Q) dS N and
    dL/dS = (I+Q)^T G N^T."""
    I = np.eye(S.shape[0], dtype=_DT)
    N = np.linalg.solve(I - S, I)
    Q = (I + S) @ N
    return (I + Q).T @ G @ N.T


def build_orth(theta: np.ndarray, bsz: Sequence[int], k) -> List[np.ndarray]:
    """Packed parameters of all blocks of one side -> list of orthogonal blocks
    (k = None: the exact transform instead of the truncated series)."""
    theta = np.asarray(theta, dtype=_DT)
    out, off = [], 0
    for b in bsz:
        cnt = b * (b - 1) // 2
        S = skew_from_packed(theta[off:off + cnt], b)
        out.append(exact_cayley(S) if k is None else neumann_cayley(S, k))
        off += cnt
    assert off == theta.shape[0]
    return out


def apply_blocks_T(A: np.ndarray, Qs: Sequence[np.ndarray], bsz: Sequence[int]) -> np.ndarray:
    """[PX] §2.C, row form of D x: each block separately, out[:, blk] = A[:, blk] Q^T."""
    out = np.empty((A.shape[0], sum(bsz)), dtype=_DT)
    for off, b, Q in zip(block_offsets(bsz), bsz, Qs):
        out[:, off:off + b] = A[:, off:off + b] @ Q.T
    return out


def apply_blocks(A: np.ndarray, Qs: Sequence[np.ndarray], bsz: Sequence[int]) -> np.ndarray:
    """Row form of D^T g: out[:, blk] = A[:, blk] Q (used by the backward)."""
    out = np.empty((A.shape[0], sum(bsz)), dtype=_DT)
    for off, b, Q in zip(block_offsets(bsz), bsz, Qs):
        out[:, off:off + b] = A[:, off:off + b] @ Q
    return out


def permute_weight(W0: np.ndarray, pi_R: np.ndarray, pi_P: np.ndarray) -> np.ndarray:
    """[PX] §2.B: fold both permutations into W once: Wt[i, j] = W0[pi_R[i], pi_P[j]]."""
    W0 = np.asarray(W0, dtype=_DT)
    return W0[np.asarray(pi_R)][:, np.asarray(pi_P)]


def forward(X, Wt, pi_R, pi_P, QR, QP, bsz_R, bsz_P) -> Tuple[np.ndarray, np.ndarray]:
    """[PX] §2.A input-centric layer: the orthogonal factors act on activations,
    R W0 P is never formed. Returns (Y, Wa) with Wa the saved activation."""
    X = np.asarray(X, dtype=_DT)
    Wt = np.asarray(Wt, dtype=_DT)
    U = X[:, np.asarray(pi_P)]                 # gather: U = X Pi_P^T
    V = apply_blocks_T(U, QP, bsz_P)           # V = U D_P^T
    Wa = V @ Wt.T                              # Wa = V Wt^T
    Z = apply_blocks_T(Wa, QR, bsz_R)          # Z = Wa D_R^T
    Y = np.empty_like(Z)
    Y[:, np.asarray(pi_R)] = Z                 # scatter: Y = Z Pi_R
    return Y, Wa


def forward_rows(X_rows, Wt, pi_R, pi_P, QR, QP, bsz_R, bsz_P) -> np.ndarray:
    """Forward for a subset of token rows (each row is independent)."""
    return forward(X_rows, Wt, pi_R, pi_P, QR, QP, bsz_R, bsz_P)[0]


def cnp_coefficients(k: int) -> List[float]:
    """Coefficients c_j of S^j in Q = (I+S) sum_{j<=k} S^j = sum_{j<=k+1} c_j S^j."""
    c = [0.0] * (k + 2)
    for j in range(k + 1):          # (I + S) * S^j contributes S^j and S^{j+1}
        c[j] += 1.0
        c[j + 1] += 1.0
    return c


def cnp_backward(G: np.ndarray, S: np.ndarray, k: int) -> np.ndarray:
    """Gradient w.r.t. S of <G, Q(S)> for the truncated Q, by the product rule on
    each power: d(S^j) = sum_{a<j} S^a dS S^{j-1-a}, so the gradient is
    sum_j c_j sum_{a<j} (S^T)^a G (S^T)^{j-1-a}. Direct double sum."""
    c = cnp_coefficients(k)
    b = S.shape[0]
    St = S.T
    pw = [np.eye(b, dtype=_DT)]
    for _ in range(k + 1):
        pw.append(pw[-1] @ St)
    Sbar = np.zeros((b, b), dtype=_DT)
    for j in range(1, k + 2):
        for a in range(j):
            Sbar += c[j] * (pw[a] @ G @ pw[j - 1 - a])
    return Sbar


def _theta_grad(dQs, theta, bsz, k) -> np.ndarray:
    """Map each block's dL/dQ to the packed parameters: dL/dtheta_(i,j) =
    Sbar[i, j] - Sbar[j, i] since S[i, j] = theta and S[j, i] = -theta."""
    theta = np.asarray(theta, dtype=_DT)
    out, off = [], 0
    for b, G in zip(bsz, dQs):
        cnt = b * (b - 1) // 2
        S = skew_from_packed(theta[off:off + cnt], b)
        Sbar = cayley_backward_exact(G, S) if k is None else cnp_backward(G, S, k)
        out.append(packed_upper(Sbar - Sbar.T))
        off += cnt
    return np.concatenate(out) if out else np.zeros(0)


def backward(X, Wt, pi_R, pi_P, theta_R, theta_P, QR, QP, Wa, G_Y, bsz_R, bsz_P, k):
    """Gradients of L = <G_Y, Y> w.r.t. X, theta_R and theta_P, following the
    forward's steps in reverse (W0 is frozen, so it gets no gradient).
    Returns (G_X, g_theta_R, g_theta_P, dQ_R, dQ_P)."""
    X = np.asarray(X, dtype=_DT)
    Wt = np.asarray(Wt, dtype=_DT)
    Wa = np.asarray(Wa, dtype=_DT)
    G_Y = np.asarray(G_Y, dtype=_DT)
    pi_R = np.asarray(pi_R)
    pi_P = np.asarray(pi_P)
    G_Z = G_Y[:, pi_R]                                   # undo the scatter
    dQ_R = [G_Z[:, o:o + b].T @ Wa[:, o:o + b] for o, b in zip(block_offsets(bsz_R), bsz_R)]
    G_Wa = apply_blocks(G_Z, QR, bsz_R)
    G_V = G_Wa @ Wt
    U = X[:, pi_P]
    dQ_P = [G_V[:, o:o + b].T @ U[:, o:o + b] for o, b in zip(block_offsets(bsz_P), bsz_P)]
    G_U = apply_blocks(G_V, QP, bsz_P)
    G_X = np.empty_like(G_U)
    G_X[:, pi_P] = G_U                                   # undo the gather
    g_R = _theta_grad(dQ_R, theta_R, bsz_R, k)
    g_P = _theta_grad(dQ_P, theta_P, bsz_P, k)
    return G_X, g_R, g_P, dQ_R, dQ_P


def layer_reference(inp, k, backward_pass: bool = True):
    """Whole layer on one set of inputs (a workloads.LayerInputs-like object;
    k = None: exact Cayley transform). Returns a dict with Q blocks, Wt, Y, Wa
    and, if asked, the gradients."""
    sp = inp.spec
    QR = build_orth(inp.theta_R, sp.bsz_R, k)
    QP = build_orth(inp.theta_P, sp.bsz_P, k)
    Wt = permute_weight(inp.W0, inp.pi_R, inp.pi_P)
    Y, Wa = forward(inp.X, Wt, inp.pi_R, inp.pi_P, QR, QP, sp.bsz_R, sp.bsz_P)
    out = dict(QR=QR, QP=QP, Wt=Wt, Y=Y, Wa=Wa)
    if backward_pass:
        G_X, gR, gP, dQR, dQP = backward(inp.X, Wt, inp.pi_R, inp.pi_P, inp.theta_R, inp.theta_P,
                                         QR, QP, Wa, inp.G_Y, sp.bsz_R, sp.bsz_P, k)
        out.update(G_X=G_X, g_theta_R=gR, g_theta_P=gP, dQ_R=dQR, dQ_P=dQP)
    return out


def backward_rows(G_Y_rows, Wt, pi_R, pi_P, QR, QP, bsz_R, bsz_P) -> np.ndarray:
    """G_X for a subset of token rows: each row of G_X depends only on the same
    row of G_Y (the backward steps of the activation path, restricted to rows)."""
    G_Y_rows = np.asarray(G_Y_rows, dtype=_DT)
    G_Z = G_Y_rows[:, np.asarray(pi_R)]
    G_Wa = apply_blocks(G_Z, QR, bsz_R)
    G_V = G_Wa @ np.asarray(Wt, dtype=_DT)
    G_U = apply_blocks(G_V, QP, bsz_P)
    G_X = np.empty_like(G_U)
    G_X[:, np.asarray(pi_P)] = G_U
    return G_X


def theta_grad_block(side, j, X, Wt, pi_R, pi_P, theta_R, theta_P, QR, QP, G_Y, bsz_R, bsz_P, k):
    """Packed gradient of one block (side "R" or "P", block index j) over all
    tokens, computing only the columns that block's dL/dQ needs."""
    X = np.asarray(X, dtype=_DT)
    Wt = np.asarray(Wt, dtype=_DT)
    G_Y = np.asarray(G_Y, dtype=_DT)
    pi_R = np.asarray(pi_R)
    pi_P = np.asarray(pi_P)
    if side == "R":
        off, b = block_offsets(bsz_R)[j], bsz_R[j]
        U = X[:, pi_P]
        V = apply_blocks_T(U, QP, bsz_P)
        Wa_blk = V @ Wt[off:off + b].T                  # columns of Wa in block j
        G_Z_blk = G_Y[:, pi_R[off:off + b]]
        dQ = G_Z_blk.T @ Wa_blk
        theta, bsz = theta_R, bsz_R
    else:
        off, b = block_offsets(bsz_P)[j], bsz_P[j]
        G_Wa = apply_blocks(G_Y[:, pi_R], QR, bsz_R)
        G_V_blk = G_Wa @ Wt[:, off:off + b]             # columns of G_V in block j
        U_blk = X[:, pi_P[off:off + b]]
        dQ = G_V_blk.T @ U_blk
        theta, bsz = theta_P, bsz_P
    poff = sum(bb * (bb - 1) // 2 for bb in bsz[:j])
    S = skew_from_packed(np.asarray(theta, dtype=_DT)[poff:poff + b * (b - 1) // 2], b)
    Sbar = cayley_backward_exact(dQ, S) if k is None else cnp_backward(dQ, S, k)
    return packed_upper(Sbar - Sbar.T)


def side_matrix(Qs: Sequence[np.ndarray], bsz: Sequence[int], pi) -> np.ndarray:
    """Dense side matrix Pi^T D Pi: D = blockdiag(Qs) ([PX] §2.C) and Pi the
    permutation matrix with (Pi v)_i = v[pi[i]] ([PX] §2.B), i.e. the rows of
    the identity taken in the order pi."""
    dim = sum(bsz)
    D = np.zeros((dim, dim), dtype=_DT)
    for off, b, Q in zip(block_offsets(bsz), bsz, Qs):
        D[off:off + b, off:off + b] = Q
    Pi = np.eye(dim, dtype=_DT)[np.asarray(pi)]
    return Pi.T @ D @ Pi


def merge_weight(W0, theta_R, theta_P, pi_R, pi_P, bsz_R, bsz_P, k: int) -> np.ndarray:
    """End of an inner loop: the orthogonal factors the loop trained are folded
    into the weight, W_new = R W0 P (the two-sided orthogonal update of
    [Pion] §数学原理; the inner loop of [PX] §2.B keeps W fixed while R and P
    change). Dense materialised matrices, float64; the next loop starts from
    W_new with theta = 0 and new permutations."""
    R = side_matrix(build_orth(theta_R, bsz_R, k), bsz_R, pi_R)
    P = side_matrix(build_orth(theta_P, bsz_P, k), bsz_P, pi_P)
    return R @ np.asarray(W0, dtype=_DT) @ P


def quantize_rows(W) -> Tuple[np.ndarray, np.ndarray]:
    """INT8 storage of the frozen weight (POET-XQ, [PX] §2.E "Quantification":
    the base weights are kept in INT8 and dequantised on the fly). The pages do
    not give the scheme; the one used here is symmetric, one scale per output
    row, every step in float32 with round-to-nearest-even, as written:
      amax = max_j |W[i, j]|,  inv = 127 / amax,  q = clamp(rint(W * inv), -127, 127),
      s = amax / 127   (amax = 0 gives s = 0 and q = 0).
    Returns (q int8 [m, n], s float32 [m])."""
    W = np.asarray(W, dtype=np.float32)
    amax = np.max(np.abs(W), axis=1)
    nz = amax > 0
    inv = np.zeros_like(amax)
    inv[nz] = np.float32(127.0) / amax[nz]
    q = np.clip(np.rint(W * inv[:, None]), -127, 127).astype(np.int8)
    s = np.zeros_like(amax)
    s[nz] = amax[nz] / np.float32(127.0)
    return q, s.astype(np.float32)


def dequantize_rows(q, s) -> np.ndarray:
    """The weight the quantised layer computes with: W[i, j] = s[i] * q[i, j]
    (float64; the product of an int8 and a float32 is exact in float64)."""
    return np.asarray(s, dtype=np.float64)[:, None] * np.asarray(q, dtype=np.float64)
