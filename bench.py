#!/usr/bin/env python3
"""Benchmark of the POET-X layer on one MI355X through libpoetx.

One step = one pass of the whole path over the workload: build of every
layer's Cayley-Neumann blocks (both sides), the input-centric forward of every
layer (saving Wa), and the backward of every layer (gradients w.r.t. X and
both sides' packed skew parameters). The default workload is the seven
linears of a LLaMA-style block at hidden 2048 (q, k, v, o 2048x2048; gate, up
5632x2048; down 2048x5632), b = 256, k = 4, bf16 activations and weights, fp32
skew parameters, 16384 tokens, every layer independently seeded. Inputs are
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


def stage_flops(w, T, xmem=False, exact=False):
    """Algorithmic flops per stage for one step of the workload (with xmem, the
    backward's recomputation of the P blocks and the Wt product counts too)."""
    f = dict(w0_fwd=0.0, w0_bwd=0.0, block_fwd=0.0, block_bwd=0.0, dq=0.0, build=0.0, cnp_bwd=0.0)
    for sp in w.layers:
        sq = sum(b * b for b in sp.bsz_R) + sum(b * b for b in sp.bsz_P)
        cube = sum(b ** 3 for b in sp.bsz_R) + sum(b ** 3 for b in sp.bsz_P)
        f["w0_fwd"] += 2.0 * T * sp.m * sp.n
        f["block_fwd"] += 2.0 * T * sq
        f["build"] += 2.0 * (11 if exact else w.k) * cube
        if w.backward:
            f["w0_bwd"] += 2.0 * T * sp.m * sp.n
            f["block_bwd"] += 2.0 * T * sq
            f["dq"] += 2.0 * T * sq
            f["cnp_bwd"] += 2.0 * (13 if exact else 2 * w.k) * cube
            if xmem:
                f["w0_fwd"] += 2.0 * T * sp.m * sp.n
                f["block_fwd"] += 2.0 * T * sum(b * b for b in sp.bsz_P)
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
                   "w0_gemm_nt_lds": "orthogonal_equivalence_cayley_amd/csrc/k_gemm_lds.hip"}


def load_traffic(kernel: str, workload: str):
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
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


def cpu_baseline(w, tokens: int):
    """float64 oracle on the workload's own layers: build + forward + backward at
    0 and `tokens` tokens per layer, extrapolated linearly to the full T."""
    import numpy as np
    import oracle
    import workloads
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    fixed = per_tok = 0.0
    for li in range(len(w.layers)):
        inp = workloads.layer_inputs(w, li, T=tokens)
        for T in (0, tokens):
            sub = type("I", (), dict(spec=inp.spec, W0=inp.W0, theta_R=inp.theta_R,
                                     theta_P=inp.theta_P, pi_R=inp.pi_R, pi_P=inp.pi_P,
                                     X=inp.X[:T], G_Y=inp.G_Y[:T]))()
            t0 = time.perf_counter()
            oracle.layer_reference(sub, w.k, backward_pass=w.backward)
            dt = time.perf_counter() - t0
            if T == 0:
                t_fixed = dt
            else:
                per_tok += max(dt - t_fixed, 0.0) / tokens
        fixed += t_fixed
    est = fixed + per_tok * w.T
    return {
        "value": w.T / est, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"float64 NumPy oracle on all {len(w.layers)} layers' own inputs: build + forward + "
                   f"backward at 0 and {tokens} tokens per layer, extrapolated linearly to "
                   f"{w.T} tokens (est. {est:.1f} s per step)"),
        "seconds_per_step_est": est,
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=4, help="workload id in workloads.WORKLOADS")
    ap.add_argument("--cpu-tokens", type=int, default=256)
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
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(across GPUs it would shard by tokens, each GPU holding every layer's blocks).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import workloads
    from orthogonal_equivalence_cayley_amd import PoetxLayer, build_many, param_grad_many, poetx

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = workloads.WORKLOADS[args.workload]
    T = w.T
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(tdt).cuda()

    log(f"bench: {w.name} T={T} layers={len(w.layers)} k={w.k}")
    layers, bufs = [], []
    for li in range(len(w.layers)):
        inp = workloads.layer_inputs(w, li, draw_grad=w.backward)
        sp = inp.spec
        L = PoetxLayer(sp.m, sp.n, sp.bsz_R, sp.bsz_P, w.k, dtype=w.dtype,
                       weight="int8" if args.xq else "dense",
                       cayley="exact" if args.exact else "neumann")
        L.set_weight(dev(inp.W0), torch.from_numpy(inp.pi_R), torch.from_numpy(inp.pi_P))
        L.set_theta(torch.from_numpy(inp.theta_R), torch.from_numpy(inp.theta_P))
        b = dict(X=dev(inp.X), Y=torch.empty(T, sp.m, dtype=tdt, device="cuda"),
                 Wa=None if args.xmem else torch.empty(T, sp.m, dtype=tdt, device="cuda"),
                 U=torch.empty(T, sp.n, dtype=tdt, device="cuda"))
        if w.backward:
            b.update(G=dev(inp.G_Y), GX=torch.empty(T, sp.n, dtype=tdt, device="cuda"),
                     g=[torch.empty(L.nparam[s], dtype=torch.float32, device="cuda") for s in (0, 1)])
        L.workspace(poetx.WS_BUILD)
        L.workspace(poetx.WS_FORWARD, T)
        if w.backward:
            L.workspace(poetx.WS_BACKWARD, T)
            L._ws_grad(0)
            L._ws_grad(1)
        layers.append(L)
        bufs.append(b)
        del inp
    torch.cuda.synchronize()
    log("bench: inputs resident")

    # groups of layers with no data dependence between them in a llama block:
    # q, k, v read the same input; gate and up too (o follows the attention,
    # down the gated product). With --streams 2 the members of a group alternate
    # between the main stream and a side stream, and each group waits for the one
    # before it (the backward walks the groups in reverse).
    indep = ({"q", "k", "v"}, {"gate", "up"})
    groups = []
    for li, sp in enumerate(w.layers):
        g = next((s for s in indep if sp.name in s), None)
        if groups and g is not None and w.layers[groups[-1][-1]].name in g:
            groups[-1].append(li)
        else:
            groups.append([li])
    side = torch.cuda.Stream() if args.streams == 2 else None

    def run_groups(order, fn, two):
        main = torch.cuda.current_stream()
        for grp in order:
            if not two or len(grp) == 1:
                for li in grp:
                    fn(li)
                continue
            side.wait_stream(main)
            for j, li in enumerate(grp):
                with torch.cuda.stream(main if j % 2 == 0 else side):
                    fn(li)
            main.wait_stream(side)

    def fwd(li):
        L, b = layers[li], bufs[li]
        # the input is kept in the permuted order the backward reads it in
        L.forward(b["X"], Y=b["Y"], Wa=b["Wa"], save=not args.xmem, keep_u=True, U=b["U"])

    def bwd(li):
        L, b = layers[li], bufs[li]
        L.backward_dq(b["X"], b["G"], G_X=b["GX"])

    def step(two=side is not None):
        build_many(layers)
        run_groups(groups, fwd, two)
        if w.backward:
            # activation path layer by layer, then the chain rule through the
            # parameterisation of all layers in one batched call
            run_groups([list(reversed(g)) for g in reversed(groups)], bwd, two)
            param_grad_many(layers, [b["g"] for b in bufs])

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
    flops = stage_flops(w, T, xmem, args.exact)
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
        for s in poetx.STAGES:
            ms, cnt = poetx.timing_read(s)
            if cnt:
                stages[s] = {"ms_per_step": ms / n_diag,
                             "tflops": flops.get(s, 0.0) / (ms / n_diag * 1e-3) / 1e12 if ms else None}
        poetx.timing_reset()

    # dominant kernel: the frozen-weight product with the largest time share.
    # The forward is always the K-contiguous (NT) kernel; the backward is too
    # when the library folds D_R into a transposed weight (T >= n, whole
    # 256-wide tiles of n, R blocks multiples of 64; not for INT8 weights).
    folded_t = (not args.xq and all(T >= sp.n and sp.n % 256 == 0 and all(b % 64 == 0 for b in sp.bsz_R)
                                    for sp in w.layers) and w.dtype == "bf16")
    stage_kernel = {"w0_fwd": "w0_gemm_nt_lds", "w0_bwd": "w0_gemm_nt_lds" if folded_t else "w0_gemm_nn_lds"}
    if args.xq:
        stage_kernel = {k: v.replace("w0_", "w0q_") for k, v in stage_kernel.items()}
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
    rec, why = load_traffic(kernel, w.name) if not (xmem or args.xq) else \
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
            "frozen_weight": "int8, one fp32 scale per row (POET-XQ)" if args.xq else w.dtype,
            "orthogonal_map": "exact Cayley (doubling build, closed-form gradient)" if args.exact
            else f"Cayley-Neumann, k = {w.k}",
            "streams": args.streams,
            "schedule": ("independent layers (q, k, v; gate, up) on two HIP streams, in block order; "
                         "backward in reverse" if args.streams == 2 and any(len(g) > 1 for g in groups)
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
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_tokens)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
