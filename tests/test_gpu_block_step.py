"""Full-size parity of the benchmarked step.

The step the benchmark times (orthogonal_equivalence_cayley_amd.block_step:
one batched build over all 14 sides, the forward of the 7 linears with Wa and
the permuted input kept, their activation-side backward, then one batched
chain rule through the parameterisation; independent layers on two HIP
streams) runs at the real sizes of the hidden-2048 and hidden-4096 blocks
(16384 tokens). Every element of Y, Wa and G_X, every block of Q and every
packed parameter gradient of every layer is compared with the full float64
oracle of that layer. At hidden 2048 the variants the benchmark also times run
beside the default input-centric order and are checked against the same
oracle results: the fold of the blocks into the weight, POET-Xmem (Wa not
kept: the backward recomputes it), the Paterson-Stockmeyer build and the
index maps fused into the block products.

The step runs twice before the comparison, so the checked outputs are those
of a step that reuses every workspace of the one before.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import blocks_concat, device_ready, log, to_np

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not device_ready():
        pytest.skip("no GPU")


# variants of the step at hidden 2048, as BlockStep options
_VARIANTS = {
    "fold": dict(fold="weight"),
    "xmem": dict(xmem=True),
    "ps": dict(series="ps"),
    "fused": dict(index="fused"),
}


def _run(cid, **opts):
    import torch
    from orthogonal_equivalence_cayley_amd.block_step import BlockStep
    w = workloads.WORKLOADS[cid]
    log(f"{w.name}: step with {opts or 'the default options'}, T={w.T}, two streams")
    blk = BlockStep(workloads.workload_layers(w), w.k, w.dtype, backward=w.backward, streams=2, **opts)
    for _ in range(2):
        blk.step()
    torch.cuda.synchronize()
    return blk


@pytest.fixture(scope="module", params=[4, 5], ids=["h2048", "h4096"])
def steps(request):
    import torch
    cid = request.param
    out = {"default": _run(cid)}
    if cid == 4:
        for name, opts in _VARIANTS.items():
            out[name] = _run(cid, **opts)
    yield cid, out
    del out
    torch.cuda.empty_cache()


def _check(name, got, want, tol):
    err = oracle.rel_fro(got, want)
    log(f"  {name}: rel_fro={err:.3e} (tol {tol:g})")
    assert err <= tol, (name, err)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("li", range(7))
def test_block_step_layer_full(steps, li):
    cid, runs = steps
    w = workloads.WORKLOADS[cid]
    inp = workloads.layer_inputs(w, li)
    sp = inp.spec
    log(f"{w.name} layer {sp.name} {sp.m}x{sp.n}: float64 oracle at T={w.T}")
    ref = oracle.layer_reference(inp, w.k, backward_pass=True)
    for variant, blk in runs.items():
        got = {k: to_np(v) for k, v in blk.outputs(li).items() if v is not None}
        log(f" {variant}")
        _check("Q_R", got["QR"], blocks_concat(ref["QR"]), TOL_F32)
        _check("Q_P", got["QP"], blocks_concat(ref["QP"]), TOL_F32)
        for key in ("Wa", "Y", "G_X", "g_theta_R", "g_theta_P"):
            if key == "Wa" and key not in got:   # POET-Xmem keeps no Wa
                continue
            _check(key, got[key], ref[key], TOL_BF16)
        # every block's gradient on its own, so that no block can hide in the
        # norm of the whole side
        for side, bsz in (("R", sp.bsz_R), ("P", sp.bsz_P)):
            g, r = got[f"g_theta_{side}"], ref[f"g_theta_{side}"]
            offs = np.cumsum([0] + [b * (b - 1) // 2 for b in bsz])
            worst = max(oracle.rel_fro(g[offs[j]:offs[j + 1]], r[offs[j]:offs[j + 1]])
                        for j in range(len(bsz)))
            log(f"  g_theta_{side} worst block: rel_fro={worst:.3e}")
            assert worst <= TOL_BF16, (side, worst)
