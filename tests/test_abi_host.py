"""Host-only checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments with the documented status codes before any
device call (none of these calls reaches a GPU)."""
import ctypes
import os
import re

import pytest

from orthogonal_equivalence_cayley_amd import poetx as px

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "poetx.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(poetx_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(px.EXPORTED)
    lib = ctypes.CDLL(px.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def _plan(**kw):
    args = dict(m=64, n=48, bsz_R=(32, 32), bsz_P=(16, 32), k=3, dtype=px.POETX_FP32)
    args.update(kw)
    return px.Plan(**args)


def test_plan_counts():
    p = _plan()
    assert p.param_count(px.SIDE_R) == 2 * 32 * 31 // 2
    assert p.param_count(px.SIDE_P) == 16 * 15 // 2 + 32 * 31 // 2
    assert p.block_elems(px.SIDE_R) == 2 * 32 * 32
    assert p.block_elems(px.SIDE_P) == 16 * 16 + 32 * 32
    assert p.param_count(7) == -1


@pytest.mark.parametrize("kw, status", [
    (dict(bsz_R=(32, 31)), px.POETX_ERR_SHAPE),
    (dict(bsz_P=(48, 0)), px.POETX_ERR_SHAPE),
    (dict(k=-1), px.POETX_ERR_SHAPE),
    (dict(k=33), px.POETX_ERR_SHAPE),
    (dict(dtype=5), px.POETX_ERR_DTYPE),
    (dict(dtype=px.POETX_BF16, bsz_P=(24, 24)), px.POETX_ERR_UNSUPPORTED),
    (dict(dtype=px.POETX_BF16, m=40, bsz_R=(40,)), px.POETX_ERR_UNSUPPORTED),
])
def test_plan_rejects(kw, status):
    with pytest.raises(px.PoetxError) as e:
        _plan(**kw)
    assert e.value.status == status


def test_plan_accepts_ragged_fp32_and_bf16_multiples_of_16():
    _plan(bsz_R=(5, 27, 32), dtype=px.POETX_FP32)
    _plan(bsz_R=(48, 16), bsz_P=(16, 32), dtype=px.POETX_BF16)


def test_null_desc():
    h = ctypes.c_void_p()
    assert px.LIB.poetx_plan_create(None, ctypes.byref(h)) == px.POETX_ERR_INVALID_ARG


def test_workspace_sizes():
    p = _plan()
    b = p.workspace_size(0, px.WS_BUILD)
    assert b >= 3 * 4 * p.block_elems(px.SIDE_P)
    f1, f2 = p.workspace_size(10, px.WS_FORWARD), p.workspace_size(1000, px.WS_FORWARD)
    assert 0 < f1 < f2
    assert p.workspace_size(10, px.WS_BACKWARD) > 0
    assert p.workspace_size(10, 9) == 0
    assert p.workspace_size(-1, px.WS_FORWARD) == 0


def test_status_strings():
    for s in range(8):
        assert isinstance(px.status_string(s), str) and px.status_string(s)


# Argument errors are returned before anything is launched, so fake addresses
# are safe here.
A = 0x10000


def test_forward_argument_errors():
    p = _plan()
    ws = p.workspace_size(4, px.WS_FORWARD)
    call = lambda **kw: px.LIB.poetx_forward(
        p.handle, kw.get("T", 4), kw.get("X", A), A, A, A, A, A, kw.get("Y", A), None,
        kw.get("U", None), kw.get("ws", A), kw.get("wsb", ws), None)
    assert call(T=0) == px.POETX_OK                      # T = 0 is a no-op
    assert call(T=-1) == px.POETX_ERR_INVALID_ARG
    assert call(X=None) == px.POETX_ERR_INVALID_ARG
    # X = NULL is accepted when U_saved holds the gathered input (the later
    # checks then decide)
    assert call(X=None, U=A + 4) == px.POETX_ERR_ALIGNMENT
    assert call(X=None, U=A, wsb=ws - 1) == px.POETX_ERR_WORKSPACE
    assert call(Y=A + 8) == px.POETX_ERR_ALIGNMENT
    assert call(wsb=ws - 1) == px.POETX_ERR_WORKSPACE
    assert call(ws=None) == px.POETX_ERR_WORKSPACE
    assert call(U=A + 4) == px.POETX_ERR_ALIGNMENT
    assert px.LIB.poetx_forward(None, 4, A, A, A, A, A, A, A, None, None, A, ws, None) == \
        px.POETX_ERR_INVALID_ARG


def test_backward_and_build_argument_errors():
    p = _plan()
    wsb = p.workspace_size(4, px.WS_BACKWARD)
    #       h, T, X, Wt, piR, piP, thR, thP, QR, QP, Wa, U, GY, GX, gR, gP, ws, wsb, stream
    args = [p.handle, 4, A, A, A, A, A, A, A, A, A, None, A, A, A, A, A, wsb, None]
    # Wa_saved and U_saved may be missing (recomputed / gathered); G_Y may not,
    # nor both X and U_saved
    for idx, val in ((12, None), (2, None), (10, None)):
        bad = list(args)
        bad[idx] = val
        if idx == 10:
            bad[12] = None
        assert px.LIB.poetx_backward(*bad) == px.POETX_ERR_INVALID_ARG, idx
    bad = list(args)
    bad[3] = A + 4
    assert px.LIB.poetx_backward(*bad) == px.POETX_ERR_ALIGNMENT
    bad = list(args)
    bad[11] = A + 4
    assert px.LIB.poetx_backward(*bad) == px.POETX_ERR_ALIGNMENT
    bad = list(args)
    bad[17] = 16
    assert px.LIB.poetx_backward(*bad) == px.POETX_ERR_WORKSPACE
    bw = p.workspace_size(0, px.WS_BUILD)
    assert px.LIB.poetx_build_orth(p.handle, 3, A, A, None, A, bw, None) == px.POETX_ERR_INVALID_ARG
    assert px.LIB.poetx_build_orth(p.handle, 0, A, A, None, A, bw - 1, None) == px.POETX_ERR_WORKSPACE
    assert px.LIB.poetx_build_orth(p.handle, 0, A + 2, A, None, A, bw, None) == px.POETX_ERR_ALIGNMENT
    assert px.LIB.poetx_permute_weight(p.handle, A, A, A, A, None) == px.POETX_ERR_INVALID_ARG
    assert px.LIB.poetx_gather_cols(p.handle, 3, 5, A, A, A, None) == px.POETX_ERR_INVALID_ARG
    assert px.LIB.poetx_gather_cols(p.handle, 0, 5, A, A, A + 1, None) == px.POETX_OK
    assert px.LIB.poetx_scatter_cols(p.handle, 3, 5, A, A + 8, A + 16, None) == px.POETX_ERR_ALIGNMENT


def test_bench_traffic_record_is_valid_or_marked_stale():
    """bench.py reports the dominant kernel's HBM traffic from a committed
    counter record only while the kernel source matches it."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    import glob
    for path in glob.glob(os.path.join(ROOT, "profiles", "*_traffic.md")):
        name = os.path.basename(path)[:-len("_traffic.md")]
        kernel = next(k for k in bench.TRAFFIC_SOURCES if name.startswith(k + "_"))
        workload = name[len(kernel) + 1:]
        rec, why = bench.load_traffic(kernel, workload)
        if rec is None:
            assert why
            continue
        for key in ("traffic_bytes_per_launch", "algorithmic_bytes_per_launch", "copy_fetch_factor",
                    "copy_write_factor", "source_sha256"):
            assert key in rec
        assert rec["kernel"] == kernel and rec["workload"] == workload
        assert rec["traffic_bytes_per_launch"] >= rec["write_bytes_per_launch"] > 0
    rec2, why2 = bench.load_traffic("w0_gemm_nt_lds", "no-such-workload")
    assert rec2 is None and why2


def test_merge_argument_errors():
    p = _plan()
    wsb = p.workspace_size(0, px.WS_MERGE)
    assert wsb >= 2 * 64 * 48 * 4 + (64 + 48) * 4      # fp32: two fp32 products, inverse perms
    args = [p.handle, A, A + 16, A + 32, A + 48, A + 64, A + 80, A + 96, wsb, None]
    bad = list(args)
    bad[6] = None
    assert px.LIB.poetx_merge_weight(*bad) == px.POETX_ERR_INVALID_ARG
    bad = list(args)
    bad[6] = args[1]                      # W_out aliasing Wt
    assert px.LIB.poetx_merge_weight(*bad) == px.POETX_ERR_INVALID_ARG
    bad = list(args)
    bad[4] = A + 4
    assert px.LIB.poetx_merge_weight(*bad) == px.POETX_ERR_ALIGNMENT
    bad = list(args)
    bad[8] = wsb - 1
    assert px.LIB.poetx_merge_weight(*bad) == px.POETX_ERR_WORKSPACE
    assert px.LIB.poetx_merge_weight(None, *args[1:]) == px.POETX_ERR_INVALID_ARG


def test_int8_weight_plans():
    bf, f32 = px.POETX_BF16, px.POETX_FP32
    p = px.Plan(512, 256, (256, 256), (256,), 4, bf, px.WEIGHT_INT8_ROWS)
    assert p.weight_bytes() == 512 * 256 + 4 * 512          # 131072 is a multiple of 256
    p2 = px.Plan(256, 512, (256,), (256, 256), 4, bf, px.WEIGHT_INT8_ROWS)
    assert p2.weight_bytes() == 256 * 512 + 4 * 256
    assert px.Plan(512, 256, (256, 256), (256,), 4, bf).weight_bytes() == 512 * 256 * 2
    for args, status in [((512, 256, (256, 256), (256,), 4, f32, 1), px.POETX_ERR_UNSUPPORTED),
                         ((384, 256, (256, 128), (256,), 4, bf, 1), px.POETX_ERR_UNSUPPORTED),
                         ((512, 256, (256, 256), (256,), 4, bf, 7), px.POETX_ERR_INVALID_ARG)]:
        with pytest.raises(px.PoetxError) as e:
            px.Plan(*args)
        assert e.value.status == status
    dense = px.Plan(512, 256, (256, 256), (256,), 4, bf)
    assert px.LIB.poetx_quantize_weight(dense.handle, A, A + 16, A + 32, A + 48, None) == \
        px.POETX_ERR_UNSUPPORTED
    assert px.LIB.poetx_permute_weight(p.handle, A, A + 16, A + 32, A + 48, None) == \
        px.POETX_ERR_UNSUPPORTED
    assert px.LIB.poetx_quantize_weight(p.handle, A, A + 16, A + 32, A, None) == \
        px.POETX_ERR_INVALID_ARG
    assert px.LIB.poetx_quantize_weight(p.handle, A, A + 16, A + 36, A + 48, None) == \
        px.POETX_ERR_ALIGNMENT


def test_cayley_mode_validation():
    px.Plan(64, 48, (32, 32), (16, 32), 3, px.POETX_FP32, px.WEIGHT_DENSE, px.CAYLEY_EXACT)
    with pytest.raises(px.PoetxError) as e:
        px.Plan(64, 48, (32, 32), (16, 32), 3, px.POETX_FP32, px.WEIGHT_DENSE, 9)
    assert e.value.status == px.POETX_ERR_INVALID_ARG
    ex = px.Plan(64, 48, (32, 32), (16, 32), 3, px.POETX_FP32, px.WEIGHT_DENSE, px.CAYLEY_EXACT)
    nm = px.Plan(64, 48, (32, 32), (16, 32), 3, px.POETX_FP32)
    # the doubling build keeps two more block arrays
    assert ex.workspace_size(0, px.WS_BUILD) > nm.workspace_size(0, px.WS_BUILD)


def test_fold_option():
    """The weight-side fold is a plan option, off by default: without it the
    forward workspace holds the activation-side V at every T and no folded
    weight; with it (T >= m) the folded m x n weight replaces V."""
    bf = px.POETX_BF16
    args = (256, 512, (256,), (256, 256), 4, bf, px.WEIGHT_DENSE, px.CAYLEY_NEUMANN)
    none = px.Plan(*args)
    fold = px.Plan(*args, px.FOLD_WEIGHT)
    T = 600
    U = V = T * 512 * 2
    Wa = Z = T * 256 * 2
    assert none.workspace_size(T, px.WS_FORWARD) >= U + V + Wa + Z
    assert fold.workspace_size(T, px.WS_FORWARD) < none.workspace_size(T, px.WS_FORWARD)
    # below the fold threshold both plans lay out the same workspace
    assert fold.workspace_size(100, px.WS_FORWARD) == none.workspace_size(100, px.WS_FORWARD)
    with pytest.raises(px.PoetxError) as e:
        px.Plan(*args, 2)
    assert e.value.status == px.POETX_ERR_INVALID_ARG


def test_dense_weight_with_transpose_bytes():
    """POETX_WEIGHT_DENSE_T keeps WtT [n, m] after Wt at a 256-byte boundary."""
    bf, f32 = px.POETX_BF16, px.POETX_FP32
    p = px.Plan(512, 256, (256, 256), (256,), 4, bf, px.WEIGHT_DENSE_T)
    assert p.weight_bytes() == 2 * (512 * 256 * 2)
    q = px.Plan(37, 53, (37,), (53,), 2, f32, px.WEIGHT_DENSE_T)
    off = (37 * 53 * 4 + 255) // 256 * 256
    assert q.weight_bytes() == off + 37 * 53 * 4
    with pytest.raises(px.PoetxError) as e:
        px.Plan(37, 53, (37,), (53,), 2, f32, 4)
    assert e.value.status == px.POETX_ERR_INVALID_ARG


def test_int8_weight_with_transpose_bytes():
    """POETX_WEIGHT_INT8_ROWS_T: q [m, n], the row scales, then qT [n, m], each
    at a 256-byte boundary; the same shape rules as POETX_WEIGHT_INT8_ROWS."""
    bf = px.POETX_BF16
    p = px.Plan(512, 768, (256, 256), (256,) * 3, 4, bf, px.WEIGHT_INT8_ROWS_T)
    mn = 512 * 768
    off = ((mn + 255) // 256 * 256 + 4 * 512 + 255) // 256 * 256
    assert p.weight_bytes() == off + mn
    for args in [(512, 256, (256, 256), (256,), 4, px.POETX_FP32),     # fp32 activations
                 (256, 320, (256,), (320,), 4, bf)]:                    # n not a multiple of 256
        with pytest.raises(px.PoetxError) as e:
            px.Plan(*args, px.WEIGHT_INT8_ROWS_T)
        assert e.value.status == px.POETX_ERR_UNSUPPORTED
    A = 1 << 20
    assert px.LIB.poetx_permute_weight(p.handle, A, A + 16, A + 32, A + 48, None) == \
        px.POETX_ERR_UNSUPPORTED


def test_forward_noalloc_host_checks():
    """The allocation-free forward checks its arguments and its size limit on
    the host, before the device is touched."""
    p = _plan()
    A = 1 << 20
    f = px.LIB.poetx_forward_noalloc
    assert px.LIB.poetx_forward_noalloc_max_bytes() == 64 << 20
    assert f(None, 4, A, A, A, A, A, A, A, None, None, None) == px.POETX_ERR_INVALID_ARG
    assert f(p.handle, -1, A, A, A, A, A, A, A, None, None, None) == px.POETX_ERR_INVALID_ARG
    assert f(p.handle, 0, None, None, None, None, None, None, None, None, None, None) == px.POETX_OK
    assert f(p.handle, 4, None, A, A, A, A, A, A, None, None, None) == px.POETX_ERR_INVALID_ARG
    assert f(p.handle, 4, A + 8, A, A, A, A, A, A, None, None, None) == px.POETX_ERR_ALIGNMENT
    T = (64 << 20) // (4 * (64 + 48)) + 1
    assert p.workspace_size(T, px.WS_FORWARD) > 64 << 20
    assert f(p.handle, T, A, A, A, A, A, A, A, None, None, None) == px.POETX_ERR_WORKSPACE


def test_index_option():
    bf = px.POETX_BF16
    args = (256, 512, (256,), (256, 256), 4, bf, px.WEIGHT_DENSE, px.CAYLEY_NEUMANN, px.FOLD_NONE)
    sep = px.Plan(*args)
    fus = px.Plan(*args, px.INDEX_FUSED)
    # the fused backward keeps bf16 transposes of both sides' blocks
    assert fus.workspace_size(100, px.WS_BACKWARD) > sep.workspace_size(100, px.WS_BACKWARD)
    with pytest.raises(px.PoetxError) as e:
        px.Plan(*args, 2)
    assert e.value.status == px.POETX_ERR_INVALID_ARG


def test_series_option():
    """Paterson-Stockmeyer builds keep the powers S^2 .. S^s and a B buffer:
    at k = 4 the step is s = 2 (S^2 and B), so the build workspace grows by two
    block arrays; bad values are refused."""
    f32 = px.POETX_FP32
    args = (64, 48, (32, 32), (16, 32), 4, f32, px.WEIGHT_DENSE, px.CAYLEY_NEUMANN, px.FOLD_NONE,
            px.INDEX_SEPARATE)
    chain = px.Plan(*args)
    ps = px.Plan(*args, px.SERIES_PS)
    ne = max(chain.block_elems(px.SIDE_R), chain.block_elems(px.SIDE_P))
    grow = ps.workspace_size(0, px.WS_BUILD) - chain.workspace_size(0, px.WS_BUILD)
    assert 2 * 4 * ne <= grow <= 2 * 4 * ne + 256
    with pytest.raises(px.PoetxError) as e:
        px.Plan(*args, 2)
    assert e.value.status == px.POETX_ERR_INVALID_ARG
