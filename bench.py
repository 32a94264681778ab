#!/usr/bin/env python3
"""Benchmark of the POET-X layer on one MI355X through libpoetx.

One step = one pass of the whole path over the workload: build of every
layer's Cayley-Neumann blocks (both sides), the input-centric forward of every
layer (saving Wa), and the backward of every layer (gradients w.r.t. X and
both sides' packed skew parameters). Every block product runs on the
activations, in the stage order of the input-centric method; --fold times the
variant that folds one side's blocks into the weight where the batch is large.
The default workload is the seven linears of a LLaMA-style block at hidden 2048
(q, k, v, o 2048x2048; gate, up 5632x2048; down 2048x5632), b = 256, k = 4,
bf16 activations and weights, fp32 skew parameters, 16384 tokens, every layer
independently seeded. Inputs are
synthetic (workloads.py) and resident in HBM before the timed region. The
layers a LLaMA block computes independently (q, k, v; gate, up) run on two HIP
streams by default (--streams 1: layer by layer on one stream); the per-stage
diagnostic pass always runs layer by layer.

Prints one JSON line. `roofline` covers the kernel with the largest share of
the step, timed live with HIP events on the stream it runs on; `cpu_baseline`
times the float64 oracle on a bounded sample of the same workload. With two
streams a frozen-weight launch shares the chip with the other stream's work, so
its live rate is below its rate alone, which `frac_isolated` gives (from the
per-stage pass).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15        # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12         # MI355X HBM3E, B/s
PEAK_F32 = 157.3e12       # MI355X fp32 (vector or matrix), FLOP/s
METRIC = "POET-X layer fwd+bwd tokens/s and % bf16 MFMA peak at hidden 2048, 1 GPU"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def ps_products(d: int) -> int:
    """Products of the Paterson-Stockmeyer evaluation of a degree-d polynomial
    (the step with the fewest: s - 1 powers and d // s recurrence products, one
    less when d % s == 0)."""
    return min((s - 1) + d // s - (1 if d % s == 0 else 0) for s in range(1, min(d, 8) + 1))


def ns_steps(w) -> float:
    """Mean Newton-Schulz step count of the exact transform over the workload's
    blocks, by the library's rule: c = max row sum of |S|, rho = c^2 / (2 + c^2),
    the least j with rho^(2^j) <= 2^-30 (at most 28)."""
    import numpy as np
    import workloads
    steps = []
    for li in range(len(w.layers)):
        inp = workloads.layer_inputs(w, li, T=0, draw_grad=False)
        for theta, bsz in ((inp.theta_R, inp.spec.bsz_R), (inp.theta_P, inp.spec.bsz_P)):
            off = 0
            for b in bsz:
                npar = b * (b - 1) // 2
                S = np.zeros((b, b))
                S[np.triu_indices(b, 1)] = theta[off:off + npar]
                S = S - S.T
                off += npar
                c = np.abs(S).sum(1).max()
                j = 0
                if c > 0:
                    rho = c * c / (2 + c * c)
                    need = 30 * np.log(2) / -np.log(rho)
                    while j < 28 and 2.0 ** j < need:
                        j += 1
                steps.append(j)
    return float(np.mean(steps))


def stage_flops(w, T, xmem=False, exact=False, fold=False, int8=False, series="chain", nsj=0.0):
    """Flops each stage executes in one step of the workload. Input-centric
    (the default): 2 T sum(b^2) per side and pass for the block products. With
    --fold, a side folded into the weight costs 2 m sum(b_P^2) (forward, T >= m)
    or 2 n sum(b_R^2) (backward, T >= n) instead. With xmem, the backward's
    recomputation of the P blocks and the Wt product counts too."""
    f = dict(w0_fwd=0.0, w0_bwd=0.0, block_fwd=0.0, block_bwd=0.0, dq=0.0, build=0.0, cnp_bwd=0.0)
    for sp in w.layers:
        sqR = sum(b * b for b in sp.bsz_R)
        sqP = sum(b * b for b in sp.bsz_P)
        cube = sum(b ** 3 for b in sp.bsz_R) + sum(b ** 3 for b in sp.bsz_P)
        fold_f = fold and not int8 and T >= sp.m
        fold_b = fold and not int8 and T >= sp.n
        p_fwd = 2.0 * (sp.m if fold_f else T) * sqP
        f["w0_fwd"] += 2.0 * T * sp.m * sp.n
        f["block_fwd"] += p_fwd + 2.0 * T * sqR
        nprod = 2 * nsj if exact else (ps_products(w.k + 1) if series == "ps" else w.k)
        f["build"] += 2.0 * nprod * cube
        if w.backward:
            f["w0_bwd"] += 2.0 * T * sp.m * sp.n
            f["block_bwd"] += 2.0 * (sp.n if fold_b else T) * sqR + 2.0 * T * sqP
            f["dq"] += 2.0 * T * (sqR + sqP)
            f["cnp_bwd"] += 2.0 * (2 * nsj + 2 if exact else 2 * w.k) * cube
            if xmem:
                f["w0_fwd"] += 2.0 * T * sp.m * sp.n
                f["block_fwd"] += p_fwd
    return f


def w0_bytes_per_step(w, T, int8=False):
    """Algorithmic HBM bytes of the frozen-weight products of one pass over all
    layers: each reads its activation operand and Wt once and writes its output
    once (same for the forward and the backward form; an INT8 Wt is one byte per
    element plus one fp32 scale per row)."""
    el = 2 if w.dtype == "bf16" else 4
    wb = (lambda sp: sp.m * sp.n + 4 * sp.m) if int8 else (lambda sp: el * sp.m * sp.n)
    return sum(el * (T * sp.n + T * sp.m) + wb(sp) for sp in w.layers)


def kernel_source_digest(path: str) -> str:
    with open(os.path.join(ROOT, path), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


# HBM traffic of the dominant kernel comes from two rocprofv3 counter runs
# (FETCH_SIZE, then WRITE_SIZE) of this script with --copy-calibration, kept as
# a JSON block in a text summary under profiles/. The counters are scaled by
# what they read for a plain copy of known size. The figure is used only while
# the kernel's source is the one the counters were taken on.
TRAFFIC_SOURCES = {"w0_gemm_nn_lds": "orthogonal_equivalence_cayley_amd/csrc/k_gemm_lds.hip",
                   "w0_gemm_nt_lds": "orthogonal_equivalence_cayley_amd/csrc/k_gemm_lds.hip",
                   "w0_gemm_nt_pipe": "orthogonal_equivalence_cayley_amd/csrc/k_gemm_w0.hip"}


def load_traffic(kernel: str, workload: str, fold: bool = False):
    suffix = "_fold" if fold else ""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}{suffix}_traffic.md")
    try:
        with open(path) as f:
            m = re.search(r"```json\n(.*?)\n```", f.read(), re.S)
        rec = json.loads(m.group(1))
        if rec.get("source_sha256") != kernel_source_digest(TRAFFIC_SOURCES[kernel]):
            return None, "kernel source changed since the counters were taken"
        return rec, None
    except (OSError, AttributeError, ValueError, KeyError) as e:
        return None, f"no traffic record ({type(e).__name__})"


def copy_calibration(mib: int, reps: int = 3) -> None:
    """A plain device copy of known size, for scaling the FETCH_SIZE and
    WRITE_SIZE counters: each launch reads and writes exactly `mib` MiB."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_seconds(w, tokens: int, dtype):
    """Seconds per step of the oracle on the workload's own layers, every layer
    at `tokens` tokens (build + forward + backward) in float type `dtype`. At
    the workload's full T the figure is measured; below it the oracle also runs
    at 0 tokens (the build and the chain rule, which do not depend on T) and
    the per-token part is scaled to the full T. Returns (seconds, measured
    seconds, full)."""
    import oracle
    import workloads
    tokens = min(tokens, w.T)
    full = tokens == w.T
    fixed = per_tok = measured = 0.0
    with oracle.precision(dtype):
        for li in range(len(w.layers)):
            inp = workloads.layer_inputs(w, li, T=tokens, draw_grad=w.backward)
            for T in ((tokens,) if full else (0, tokens)):
                sub = type("I", (), dict(spec=inp.spec, W0=inp.W0, theta_R=inp.theta_R,
                                         theta_P=inp.theta_P, pi_R=inp.pi_R, pi_P=inp.pi_P,
                                         X=inp.X[:T], G_Y=None if inp.G_Y is None else inp.G_Y[:T]))()
                t0 = time.perf_counter()
                oracle.layer_reference(sub, w.k, backward_pass=w.backward)
                dt = time.perf_counter() - t0
                measured += dt
                if T == 0:
                    t_fixed = dt
                elif not full:
                    per_tok += max(dt - t_fixed, 0.0) / tokens
            if not full:
                fixed += t_fixed
            del inp
    return (measured if full else fixed + per_tok * w.T), measured, full


def cpu_baseline(w, tokens: int):
    """The float64 oracle on the workload's own layers, every layer at `tokens`
    tokens (build + forward + backward), measured at the workload's full T or
    scaled from a sample (which the sample states); beside it the same steps in
    float32 on a quarter of those tokens, as a CPU throughput figure."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    est, measured, full = _oracle_seconds(w, tokens, np.float64)
    what = "build + forward + backward" if w.backward else "build + forward"
    tokens = min(tokens, w.T)
    sample = (f"float64 NumPy oracle, {what} of all {len(w.layers)} layers on their own inputs at "
              f"the full {w.T} tokens: {est:.1f} s per step, measured" if full else
              f"float64 NumPy oracle, {what} of all {len(w.layers)} layers on their own inputs at 0 "
              f"and {tokens} tokens; the per-token part scaled to {w.T} tokens (est. {est:.1f} s "
              f"per step; {measured:.1f} s measured)")
    t32 = max(1, tokens // 4)
    est32, meas32, full32 = _oracle_seconds(w, t32, np.float32)
    return {
        "value": w.T / est, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
        "sample": sample, "seconds_per_step": est, "measured": full,
        "cpu_count": os.cpu_count(), "cpu_model": cpu_model(),
        "fp32": {"value": w.T / est32, "unit": "tokens/s", "seconds_per_step": est32,
                 "sample": (f"the same oracle steps in float32, at 0 and {t32} tokens per layer, the "
                            f"per-token part scaled to {w.T} tokens ({meas32:.1f} s measured)"
                            if not full32 else f"the same oracle steps in float32 at the full {w.T} "
                            f"tokens, measured")},
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=4, help="workload id in workloads.WORKLOADS")
    ap.add_argument("--cpu-tokens", type=int, default=None,
                    help="tokens per layer of the oracle's timed sample (default: the full batch "
                         "at hidden 2048 and below, a quarter of it at hidden 4096)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stages", action="store_true", help="skip the per-stage timing pass")
    ap.add_argument("--streams", type=int, default=2, choices=(1, 2),
                    help="2: layers a llama block computes independently (q, k, v; gate, up) run on "
                         "two HIP streams")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB three times (for counter runs)")
    ap.add_argument("--merge", action="store_true",
                    help="also time the end-of-inner-loop merge W <- R W0 P of every layer")
    ap.add_argument("--exact", action="store_true",
                    help="exact Cayley transform (reference build and gradient) instead of the series")
    ap.add_argument("--xq", action="store_true",
                    help="POET-XQ: frozen weight stored as INT8 (one scale per row)")
    ap.add_argument("--xmem", action="store_true",
                    help="POET-Xmem: keep no Wa; the backward recomputes it from X")
    ap.add_argument("--series", choices=("chain", "ps"), default="chain",
                    help="build: power chain (default) or Paterson-Stockmeyer")
    ap.add_argument("--index", choices=("separate", "fused"), default="separate",
                    help="fused: index maps inside the block products (sides of 256-wide blocks up to 2048)")
    ap.add_argument("--fold", action="store_true",
                    help="variant: fold the P blocks into the weight in the forward (T >= m) and the R "
                         "blocks in the backward (T >= n) instead of applying them to the activations")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(across GPUs it would shard by tokens, each GPU holding every layer's blocks).", file=sys.stderr)
        return 2

    import torch

    import workloads
    from orthogonal_equivalence_cayley_amd import build_many, poetx
    from orthogonal_equivalence_cayley_amd.block_step import BlockStep

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = workloads.WORKLOADS[args.workload]
    T = w.T
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    log(f"bench: {w.name} T={T} layers={len(w.layers)} k={w.k}")
    blk = BlockStep([workloads.layer_inputs(w, li, draw_grad=w.backward) for li in range(len(w.layers))],
                    w.k, w.dtype, backward=w.backward, streams=args.streams,
                    weight="int8_t" if args.xq else "dense_t", cayley="exact" if args.exact else "neumann",
                    fold="weight" if args.fold else "none", series=args.series, xmem=args.xmem,
                    index=args.index)
    layers = blk.layers
    step = blk.step
    torch.cuda.synchronize()
    log("bench: inputs resident")

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("bench: warmup done")

    # timed region: HIP events around the frozen-weight GEMMs only (two
    # launches per layer), everything else untouched
    poetx.timing_reset()
    poetx.timing_enable(["w0_fwd", "w0_bwd"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    poetx.timing_enable([])
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    w0 = {s: poetx.timing_read(s) for s in ("w0_fwd", "w0_bwd")}
    poetx.timing_reset()
    log(f"bench: {ms_per_step:.3f} ms/step")

    xmem = bool(args.xmem and w.backward)
    flops = stage_flops(w, T, xmem, args.exact, args.fold, args.xq, args.series,
                        ns_steps(w) if args.exact else 0.0)
    merge = None
    if args.merge:
        # outer loop: fold the trained factors of every layer into its weight
        # (once per inner loop; fp32 block products on both sides)
        outs = [torch.empty(L.m, L.n, dtype=tdt, device="cuda") for L in layers]
        for L in layers:
            L.workspace(poetx.WS_MERGE)
        build_many(layers)
        for L, o in zip(layers, outs):
            L.merge(o)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record()
        for _ in range(reps):
            for L, o in zip(layers, outs):
                L.merge(o)
        e1.record()
        torch.cuda.synchronize()
        mms = e0.elapsed_time(e1) / reps
        mfl = sum(2.0 * sp.n * sum(b * b for b in sp.bsz_R) + 2.0 * sp.m * sum(b * b for b in sp.bsz_P)
                  for sp in w.layers)
        merge = {"ms_all_layers": mms, "tflops": mfl / (mms * 1e-3) / 1e12,
                 "fp32_frac": mfl / (mms * 1e-3) / PEAK_F32, "flops": mfl}
        del outs
    stages = {}
    if not args.no_stages:
        # separate diagnostic pass: every stage bracketed by events, layer by
        # layer on one stream
        poetx.timing_enable(list(poetx.STAGES))
        n_diag = max(2, min(5, args.steps))
        for _ in range(n_diag):
            step(False)
        torch.cuda.synchronize()
        poetx.timing_enable([])
        recorded = {s: poetx.timing_read(s) for s in poetx.STAGES}
        # where the backward's block products and dL/dQ reductions run as one
        # pass (sides of 256-wide blocks), their time is recorded under block_bwd
        sflops = dict(flops)
        if recorded["dq"][1] == 0:
            sflops["block_bwd"] = sflops.get("block_bwd", 0.0) + sflops.get("dq", 0.0)
        # bf16 plans run every product of the build and chain-rule chains as
        # three bf16 MFMAs on split operands (blocks that are multiples of 32 up
        # to 512): the matrix cores then run 3x the products' flops
        split = (w.dtype == "bf16" and not args.exact and args.series == "chain" and
                 all(b % 32 == 0 and b <= 512 for sp in w.layers for b in sp.bsz_R + sp.bsz_P))
        for s in poetx.STAGES:
            ms, cnt = recorded[s]
            if cnt:
                stages[s] = {"ms_per_step": ms / n_diag,
                             "tflops": sflops.get(s, 0.0) / (ms / n_diag * 1e-3) / 1e12 if ms else None}
                if split and s in ("build", "cnp_bwd") and ms:
                    stages[s]["mfma_tflops_bf16"] = 3.0 * stages[s]["tflops"]
                    stages[s]["frac_of_bf16_peak"] = 3.0 * stages[s]["tflops"] * 1e12 / PEAK_BF16
        poetx.timing_reset()

    # dominant kernel: the frozen-weight product with the largest time share.
    # The forward is always the K-contiguous (NT) kernel; the backward is too
    # only in the fold variant, which folds D_R into a transposed weight (T >= n,
    # whole 256-wide tiles of n, R blocks multiples of 64; not for INT8 weights).
    folded_t = (args.fold and not args.xq and w.dtype == "bf16" and
                all(T >= sp.n and sp.n % 256 == 0 and all(b % 64 == 0 for b in sp.bsz_R)
                    for sp in w.layers))
    # With the weight kept beside its transpose (dense or INT8; the default
    # here) the backward reads it K-contiguous: the NT kernel as well.
    nt_bwd = folded_t or (not args.fold and w.dtype == "bf16")
    # NT products on whole 256 x 256 tiles with at least one tile per CU run the
    # dedicated frozen-weight kernel (k_gemm_w0.hip); an INT8 weight (--xq) is
    # widened exactly to bf16 first (a pass inside the same stage) and takes
    # the same kernels, its row scales applied in the forward's epilogue
    pipe = (w.dtype == "bf16" and T % 256 == 0 and
            all(sp.m % 256 == 0 and sp.n % 256 == 0 and (T // 256) * (min(sp.m, sp.n) // 256) >= 256
                for sp in w.layers))
    nt_name = "w0_gemm_nt_pipe" if pipe else "w0_gemm_nt_lds"
    stage_kernel = {"w0_fwd": nt_name, "w0_bwd": nt_name if nt_bwd else "w0_gemm_nn_lds"}
    per_kernel = {}
    for st, kname in stage_kernel.items():
        ms_s, n_s = w0[st]
        if n_s == 0:
            continue
        tot = per_kernel.setdefault(kname, [0.0, 0, 0.0, []])
        tot[0] += ms_s
        tot[1] += n_s
        tot[2] += flops[st] * args.steps
        tot[3].append(st)
    kernel = max(per_kernel, key=lambda k: per_kernel[k][0])
    ms_tot, launches, kflops, kstages = per_kernel[kernel]
    dom = kstages[0]
    flops_per_launch = kflops / launches
    avg_s = ms_tot / launches * 1e-3
    achieved = flops_per_launch / avg_s
    traffic, traffic_note = None, None
    rec, why = load_traffic(kernel, w.name, args.fold) if not (xmem or args.xq or args.exact) else \
        (None, "counters taken on the dense Xfast step only")
    if rec is not None:
        traffic = rec["traffic_bytes_per_launch"]
        traffic_note = (f"HBM bytes per launch, rocprofv3 FETCH_SIZE + WRITE_SIZE scaled by a plain "
                        f"copy; algorithmic {rec['algorithmic_bytes_per_launch']:.4g}")
    else:
        traffic_note = why
    gemm_keys = ("w0_fwd", "w0_bwd", "block_fwd", "block_bwd", "dq")
    gemm_frac = None
    if stages:
        gt = sum(stages[s]["ms_per_step"] for s in gemm_keys if s in stages) * 1e-3
        gemm_frac = sum(flops[s] for s in gemm_keys) / gt / PEAK_BF16 if gt else None
    # the dominant kernel alone (per-stage pass, one stream): its stages' flops
    # over their event time
    frac_isolated = None
    if stages and all(st in stages for st in kstages):
        t_iso = sum(stages[st]["ms_per_step"] for st in kstages) * 1e-3
        frac_isolated = sum(flops[st] for st in kstages) / t_iso / PEAK_BF16 if t_iso else None
    w0_total_frac = (flops["w0_fwd"] + flops["w0_bwd"]) / (
        (w0["w0_fwd"][0] + w0["w0_bwd"][0]) / args.steps * 1e-3) / PEAK_BF16

    out = {
        "metric": METRIC,
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "tokens": T, "k": w.k,
            "layers": [f"{sp.name} {sp.m}x{sp.n}" for sp in w.layers],
            "block_size": max(max(sp.bsz_R) for sp in w.layers),
            "passes": "build+forward+backward" if w.backward else "build+forward",
            "saved_activation": ("none (POET-Xmem: recomputed)" if xmem else "Wa (POET-Xfast)")
            + "; layer input kept as U = X Pi_P^T",
            "frozen_weight": "int8, one fp32 scale per row (POET-XQ), kept with its transpose" if args.xq
            else f"{w.dtype}, kept with its transpose",
            "orthogonal_map": "exact Cayley (Newton-Schulz inverse, closed-form gradient)" if args.exact
            else f"Cayley-Neumann, k = {w.k}" + (", Paterson-Stockmeyer build" if args.series == "ps"
                                                   else ", power-chain build"),
            "block_products": ("fold variant: P blocks folded into the weight in the forward where "
                               "T >= m, R blocks in the backward where T >= n, the other side on the "
                               "activations" if args.fold else
                               "on the activations (input-centric order: gather, P blocks, Wt product, "
                               "R blocks, scatter; the backward in reverse)"),
            "fold": bool(args.fold),
            "index_maps": ("fused into the block products (sides up to 2048 features)" if args.index == "fused"
                           else "separate gather and scatter passes"),
            "streams": args.streams,
            "schedule": ("independent layers (q, k, v; gate, up) on two HIP streams, in block order; "
                         "backward in reverse" if blk.two_streams
                         else "layer by layer on one stream"),
        },
        "roofline": {
            "kernel": kernel, "bound": "mfma", "achieved": achieved / 1e12, "peak": PEAK_BF16 / 1e12,
            "unit": "TFLOP/s", "frac": achieved / PEAK_BF16, "traffic": traffic,
            "launches": launches, "avg_launch_us": avg_s * 1e6,
            "flops_per_launch": flops_per_launch,
            "algorithmic_bytes_per_launch": w0_bytes_per_step(w, T, args.xq) * args.steps
            * sum(2 if (xmem and st == "w0_fwd") else 1 for st in kstages) / launches,
            "stages": kstages,
            "traffic_note": traffic_note,
            "frac_isolated": frac_isolated,
        },
        "tflops_per_step": sum(flops.values()) / (ms_per_step * 1e-3) / 1e12,
        "w0_gemm_mfma_frac": w0_total_frac,
        "gemm_stage_mfma_frac": gemm_frac,
        "stages": stages,
    }
    if merge is not None:
        out["merge"] = merge
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        tok = args.cpu_tokens
        if tok is None:
            # the full batch up to hidden 2048 (about 20 s of float64 work on 16
            # cores); a quarter of it at hidden 4096
            tok = w.T if min(min(sp.m, sp.n) for sp in w.layers) <= 2048 else w.T // 4
        out["cpu_baseline"] = cpu_baseline(w, tok)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
