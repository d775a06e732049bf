"""Benchmark of the pruned MoE expert backward on one MI355X.

One step = one pass of the whole hot path over one batch: LRM score ->
per-expert top-quota select -> compaction -> the fused varlen grouped GEMM for
dW and dphi, in one library call (lrmoe_pruned_backward; the gather also
writes the GEMM's operand planes).
Inputs are resident in HBM before timing starts; outputs are preallocated.

Prints ONE JSON line.  value = kept pairs per second of the whole path over
the timed steps.  `roofline` is for the dominant kernel, the fused grouped
GEMM: HIP events recorded by the library around that launch, on the stream it
launches on, in every timed step (the only events in the timed region).
`kernels` gives every kernel's time and rate from a separate pass with events
around each kernel; `cpu_baseline` times the CPU oracle on the host cores.

The default workload is the largest single-GPU one: the GLM4.5-106B-A12B-shaped
20x batch-pressure share (655360 routed pairs, 24 GiB token-buffer budget).

Usage: python bench.py [--gpus 1] [--steps 1000] [--warmup 50] [--config 4]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, TFLOP/s

# Sources that define the grouped GEMM kernel and its launch; HBM counters
# taken on another version of them are not reported.
GEMM_SOURCES = ("pruned_expert_backward_amd/csrc/grouped_gemm.hip",
                "pruned_expert_backward_amd/csrc/lrmoe_internal.h",
                "pruned_expert_backward_amd/csrc/api.cpp")
COUNTERS_GLOB = "profiles/grouped_backward_kernel.*.counters.txt"
COPY_BYTES = 1 << 30           # plain copy used to calibrate FETCH_SIZE / WRITE_SIZE


def algorithmic_bytes(p, M, score_mode="lrm"):
    """Bytes the method must move in score + select + compaction (each row
    read or written once): score reads every g and phi row plus alpha and
    writes R (gradient-only rules: g rows only; given random scores: none);
    select reads R and writes the keep flag; compaction reads and writes the
    kept rows, alpha and perm, and zeroes dropped dphi rows."""
    es = 2 if p.dtype == "bf16" else 4
    P = p.P
    score = {"lrm": P * (es * (p.d_out + p.d_in) + 8),
             "random": 0}.get(score_mode, P * (es * p.d_out + 4))
    select = P * 5
    compact = M * (2 * es * (p.d_out + p.d_in) + 12) + (P - M) * 4 * p.d_in
    return score + select + compact


def gemm_flops(p, M):
    return 4.0 * M * p.d_out * p.d_in   # dW and dphi, 2*M*d_out*d_in each


def gemm_floor_bytes(p, M):
    es = 2 if p.dtype == "bf16" else 4
    return (M * es * (p.d_out + p.d_in) + p.E * p.d_out * p.d_in * es
            + p.E * p.d_out * p.d_in * 4 + M * p.d_in * 4)


def gemm_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_counters(workload: str, dw_mode: str, leg: str = "down"):
    """Counters of the grouped GEMM from a committed rocprofv3 summary:
    HBM bytes per launch (FETCH_SIZE and WRITE_SIZE, KiB per dispatch, each
    scaled by bytes / counter of a plain copy of known size) and the MFMA
    busy fraction.  (None, None) when no summary was taken on this workload,
    dW mode and leg (the down projection, or the gate/up one), or the kernel
    sources changed since."""
    import glob
    sha = gemm_sources_sha256()
    for path in sorted(glob.glob(os.path.join(ROOT, COUNTERS_GLOB))):
        kv = {}
        with open(path) as f:
            for line in f:
                line = line.strip()
                if line and not line.startswith("#") and "=" in line:
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        try:
            if (kv["workload"] != workload or kv["dw_mode"] != dw_mode
                    or kv.get("leg", "down") != leg or kv["kernel_sources_sha256"] != sha):
                continue
            fetch = (float(kv["gemm_fetch_kib"]) * float(kv["copy_bytes"])
                     / float(kv["copy_fetch_kib"]))
            write = (float(kv["gemm_write_kib"]) * float(kv["copy_bytes"])
                     / float(kv["copy_write_kib"]))
            busy = float(kv["mfma_busy_frac"]) if "mfma_busy_frac" in kv else None
        except (KeyError, ValueError, ZeroDivisionError):
            continue
        return fetch + write, busy
    return None, None


def copy_calibration(reps: int = 10):
    """A plain device copy of COPY_BYTES, for scaling the HBM counters."""
    import torch
    dev = torch.device("cuda:0")
    n = COPY_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES,
                      "reps": reps, "GBps_read_plus_write": 2 * COPY_BYTES * reps / el / 1e9}),
          flush=True)


def stats_us(d: list):
    """Mean, median, p10 and p90 of per-launch durations (microseconds)."""
    if not d:
        return None
    s = sorted(d)
    pick = lambda f: s[min(len(s) - 1, int(f * (len(s) - 1) + 0.5))]
    return {"mean": sum(s) / len(s), "median": pick(0.5), "p10": pick(0.1), "p90": pick(0.9),
            "launches": len(s)}


def cpu_baseline(p, budget_s: float = 12.0, chain: bool = False):
    """The oracle as it stands on the host cores: whole path on the same
    workload (with chain, the MLP chain through the gate/up projection),
    repeated while under the time budget."""
    from oracle import lrmoe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    runs, t0 = 0, time.perf_counter()
    M = 0
    while True:
        glu = (p.glu.a, p.glu.b, p.gate_up.x, p.gate_up.W2) if chain else None
        out = O.pruned_backward(p.counts, p.policy, p.alpha, p.g, p.phi, p.W, p.row_index,
                                p.dtype, glu=glu)
        M = int(out["seg"][-1])
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or runs >= 200:
            break
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                         None)
    except OSError:  # pragma: no cover
        pass
    return dict(value=M * runs / el, unit="kept pairs/s", cores=int(threads), kind="oracle",
                sample=f"{runs} full pass(es) of the same workload ({p.name}, P={p.P}, M={M}), "
                       f"{el:.1f} s, numpy float64",
                host_cpus=os.cpu_count(), cpu_model=model)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=4,
                    help="workload (4: GLM4.5 20x batch-pressure share, the largest)")
    ap.add_argument("--dw-mode", choices=["exact", "bf16", "f16"], default="f16",
                    help="weight-gradient folding of alpha: exact (bf16 hi + lo, two "
                         "passes), bf16 (one rounding), f16 (one pass on float16 planes)")
    ap.add_argument("--score-mode", choices=["lrm", "grad-sqnorm", "grad-l1", "random"],
                    default="lrm", help="scoring rule (the method, or an ablation baseline)")
    ap.add_argument("--path", choices=["compacted", "masked-dense", "glu-chain"],
                    default="compacted",
                    help="masked-dense: the zero-masked alternative (alpha := 0 on dropped "
                         "pairs, GEMMs over every routed pair), for the A/B against compaction; "
                         "glu-chain (a config with a gate/up projection): the expert MLP "
                         "chained on the compacted layout, down GEMM with the SiLU-GLU "
                         "backward in its epilogue, then the gate/up GEMM")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path shards by expert across GPUs but no multi-GPU run is implemented.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from pruned_expert_backward_amd import lrmoe, workloads

    chain = args.path == "glu-chain"
    if chain and "gate_up" not in workloads.CONFIGS[args.config]:
        print("bench.py: the glu-chain path needs a config with a gate/up projection",
              file=sys.stderr)
        sys.exit(2)
    p = workloads.config(args.config, glu=chain)
    q = lrmoe.plan_quota(p.counts, p.policy)
    M = sum(q)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dtc = lrmoe.BF16 if p.dtype == "bf16" else lrmoe.F32
    mode = {"exact": lrmoe.DW_EXACT, "bf16": lrmoe.DW_BF16, "f16": lrmoe.DW_F16}[args.dw_mode]
    smode = {"lrm": lrmoe.SCORE_LRM, "grad-sqnorm": lrmoe.SCORE_GRAD_SQNORM,
             "grad-l1": lrmoe.SCORE_GRAD_L1, "random": lrmoe.SCORE_LRM}[args.score_mode]
    plan = lrmoe.Plan(p.counts, q, p.d_out, p.d_in, dtc, T=p.T, dw_mode=mode, score_mode=smode)

    def d(a):
        if a is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if a.dtype == np.uint16 else t).to(dev)

    alpha, g, phi, W, row = d(p.alpha), d(p.g), d(p.phi), d(p.W), d(p.row_index)
    out = lrmoe.alloc_select_outputs(plan, dev, zero_target=not chain)
    dW = torch.empty((p.E, p.d_out, p.d_in), dtype=torch.float32, device=dev)
    ws = lrmoe.workspace(plan, dev)
    stream = torch.cuda.current_stream()
    gu = p.gate_up
    if gu is not None:
        # second projection (gate/up) on the same keep set: gather its rows
        # with the down projection's perm, then its own grouped backward
        plan2 = lrmoe.Plan(p.counts, q, gu.d_out, gu.d_in, dtc, T=p.P, dw_mode=mode)
        g2, x, W2 = d(gu.g2), d(gu.x), d(gu.W2)
        out2 = dict(g_c=torch.empty((M, gu.d_out), dtype=g2.dtype, device=dev),
                    phi_c=torch.empty((M, gu.d_in), dtype=x.dtype, device=dev),
                    alpha_c=torch.empty((M,), dtype=torch.float32, device=dev),
                    dphi=torch.empty((p.P, gu.d_in), dtype=torch.float32, device=dev))
        dW2 = torch.empty((p.E, gu.d_out, gu.d_in), dtype=torch.float32, device=dev)
        ws2 = lrmoe.workspace(plan2, dev)
        if chain:   # gate/up output gradient comes from the down GEMM, already compacted
            act_a, act_b = d(p.glu.a), d(p.glu.b)
            out2["g_c"] = None
            # float32 hand-off (bf16 in the single-rounding mode)
            dgu = torch.empty((M, gu.d_out), dtype=lrmoe.glu_grad_dtype(plan), device=dev)

    given_scores = None
    if args.score_mode == "random":   # random dropping: seeded scores drawn once, as input
        gen = torch.Generator(device=dev)
        gen.manual_seed(2024)
        given_scores = torch.rand(p.P, generator=gen, device=dev, dtype=torch.float32)

    dense_path = args.path == "masked-dense"
    # the whole path in one call, except where the step needs the separate
    # calls: given scores (random rule), the MLP chain
    whole = not dense_path and not chain and given_scores is None
    out["dW"] = dW
    if dense_path:
        if gu is not None or p.T != p.P or given_scores is not None:
            print("bench.py: the masked-dense path runs one projection with one g row per "
                  "pair and a computed score", file=sys.stderr)
            sys.exit(2)
        dense = lrmoe.Plan(p.counts, p.counts, p.d_out, p.d_in, dtc, dw_mode=mode)
        dws = lrmoe.workspace(dense, dev)
        sel = dict(scores=torch.empty(p.P, dtype=torch.float32, device=dev),
                   keep=torch.empty(p.P, dtype=torch.uint8, device=dev),
                   seg_offsets=torch.empty(p.E + 1, dtype=torch.int32, device=dev),
                   perm=torch.empty(M, dtype=torch.int32, device=dev))
        am = torch.empty(p.P, dtype=torch.float32, device=dev)
        pid = torch.empty(p.P, dtype=torch.int32, device=dev)
        dphi_full = torch.empty((p.P, p.d_in), dtype=torch.float32, device=dev)

    def step(ssc_t=None, gb_t=None, gu_t=None, gu_events=None):
        if dense_path:   # same selection, no compaction, GEMMs over all P pairs
            if gu_events is not None:
                gu_events[0].record(stream)
            lrmoe.score_select(plan, alpha, g, phi, out=sel, ws=ws)
            lrmoe.mask_alpha(sel["keep"], alpha, am, pid)
            if gu_events is not None:
                gu_events[1].record(stream)
            lrmoe.grouped_backward(dense, pid, am, g, phi, W, dW=dW, dphi=dphi_full, ws=dws,
                                   timing=gb_t)
            return
        if whole:
            lrmoe.pruned_backward(plan, alpha, g, phi, W, g_row_index=row, out=out, ws=ws,
                                  timing=ssc_t)
        else:
            lrmoe.score_select_compact(plan, alpha, g, phi, g_row_index=row, out=out, ws=ws,
                                       scores=given_scores, timing=ssc_t)
        if chain:
            lrmoe.grouped_backward_glu(plan, out["perm"], out["alpha_c"], out["g_c"],
                                       out["phi_c"], W, act_a, act_b, dW=dW, dgu_c=dgu, ws=ws,
                                       timing=gb_t)
            if gu_events is not None:
                gu_events[0].record(stream)
            lrmoe.gather_compact(plan2, out["perm"], out["keep"], alpha, None, x, out=out2)
            if gu_events is not None:
                gu_events[1].record(stream)
            if dgu.dtype == torch.float32:
                lrmoe.grouped_backward_gate_up(plan2, out["perm"], out2["alpha_c"], dgu,
                                               out2["phi_c"], W2, dW=dW2, dx=out2["dphi"],
                                               ws=ws2, timing=gu_t)
            else:
                lrmoe.grouped_backward(plan2, out["perm"], out2["alpha_c"], dgu, out2["phi_c"],
                                       W2, dW=dW2, dphi=out2["dphi"], ws=ws2, timing=gu_t)
            return
        if not whole:
            lrmoe.grouped_backward(plan, out["perm"], out["alpha_c"], out["g_c"], out["phi_c"],
                                   W, dW=dW, dphi=out["dphi"], ws=ws, timing=gb_t)
        if gu is not None:   # gather (with operand planes) + grouped GEMM in one call
            out2["dW"] = dW2
            lrmoe.gather_backward(plan2, out["perm"], out["keep"], alpha, g2, x, W2, out=out2,
                                  ws=ws2, timing=gu_t)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Timed region: whole steps.  The only events in it bracket the dominant
    # kernel (the grouped GEMM launch; in the MLP chain the larger gate/up
    # one), recorded by the library on the stream it launches on; events
    # around every kernel would add gaps to the step.
    # the dominant GEMM: the gate/up projection's where there is one (the
    # larger), else the down projection's
    gemm_slot = 1 if chain or not (whole or gu is not None) else 3
    gemm_timer = lrmoe.KernelTimer(args.steps, slots=(gemm_slot,))
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if gu is not None:
            step(gu_t=gemm_timer)
        elif whole:
            step(ssc_t=gemm_timer)
        else:
            step(gb_t=gemm_timer)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gemm_live = stats_us(gemm_timer.durations_us(gemm_slot))
    gemm_timer.close()

    # Per-kernel breakdown: a separate pass after the timed region, with HIP
    # events around every kernel.
    nb = min(args.steps, 200)
    ssc_timer = lrmoe.KernelTimer(nb)
    gb_timer = lrmoe.KernelTimer(nb)
    if gu is not None or dense_path:
        gu_timer = lrmoe.KernelTimer(nb)
        gu_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(nb)]
    for i in range(nb):
        step(ssc_timer, gb_timer, gu_timer if gu is not None else None,
             gu_ev[i] if (gu is not None or dense_path) else None)
    torch.cuda.synchronize()

    # Cold passes: before each step, evict L2 and the 256 MB MALL, then time
    # score, select and gather again.  "read": a 512 MiB buffer is summed, so
    # the caches hold clean lines only (the kernels' own cost from HBM).
    # "write": a 512 MiB buffer is filled, so its dirty lines are written
    # back while the timed kernels run -- what a kernel pays after a
    # write-heavy one.
    cold = {}
    if not dense_path:
        nc = min(nb, 50)
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        flush_r = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        sink = torch.empty(1, dtype=torch.float32, device=dev)
        for how in ("read", "write"):
            cold_timer = lrmoe.KernelTimer(nc)
            for i in range(nc):
                if how == "read":
                    torch.sum(flush_r, dim=0, keepdim=True, out=sink)
                else:
                    flush.fill_(i & 0xFF)
                step(cold_timer, None, None, None)
            torch.cuda.synchronize()
            st = {n: stats_us(cold_timer.durations_us(slot))
                  for n, slot in (("lrm_score", 0), ("select_scan", 1), ("gather", 2))}
            cold[how] = {n: v for n, v in st.items() if v is not None}
            cold_timer.close()
        del flush, flush_r

    es = 2 if p.dtype == "bf16" else 4
    P, d_o, d_i = p.P, p.d_out, p.d_in
    if whole:   # one call, its slots: score, select, gather (+ planes), GEMM, reduction
        dist = {"lrm_score": stats_us(ssc_timer.durations_us(0)),
                "select_scan": stats_us(ssc_timer.durations_us(1)),
                "gather": stats_us(ssc_timer.durations_us(2)),
                "operand_prologue": stats_us(ssc_timer.durations_us(5)),
                "grouped_gemm": stats_us(ssc_timer.durations_us(3)),
                "splitk_reduce": stats_us(ssc_timer.durations_us(4))}
    else:
        dist = {"lrm_score": stats_us(ssc_timer.durations_us(0)),
                "select_scan": stats_us(ssc_timer.durations_us(1)),
                "gather": stats_us(ssc_timer.durations_us(2)),
                "operand_prologue": stats_us(gb_timer.durations_us(0)),
                "grouped_gemm": stats_us(gb_timer.durations_us(1)),
                "splitk_reduce": stats_us(gb_timer.durations_us(2))}
    us = {k: (v["mean"] if v else None) for k, v in dist.items()}
    # algorithmic bytes (HBM-bound kernels) and FLOP (the GEMM) per launch
    score_bytes = (P * (es * (d_o + d_i) + 8) if args.score_mode == "lrm"
                   else P * (es * d_o + 4))   # gradient-only rules read no phi, no alpha
    # the dropped pairs' dphi rows: zeroed by the gather, except for large fills
    # in the one-call path, whose grouped GEMM launch clears them beside its tiles
    zero_bytes = 0 if chain or dense_path else (P - M) * 4 * d_i
    zero_in_gemm = whole and lrmoe.zero_fill_in_gemm(plan)
    work = {"lrm_score": score_bytes,
            "select_scan": P * 5,
            "gather": M * (2 * es * (d_o + d_i) + 12) + (0 if zero_in_gemm else zero_bytes),
            "grouped_gemm": gemm_flops(p, p.P if dense_path else M)}
    kernels = {}
    for name, t in us.items():
        if t is None:
            continue
        k = {"us": t, "us_median": dist[name]["median"], "us_p10": dist[name]["p10"],
             "us_p90": dist[name]["p90"]}
        if name == "grouped_gemm":
            k.update(algorithmic_flops=work[name], TFLOPs=work[name] / t / 1e6,
                     mfma_frac=work[name] / t / 1e6 / MFMA_BF16_PEAK_TFLOPS)
            if zero_in_gemm:
                k.update(zero_fill_bytes=zero_bytes)
        elif name in work:
            k.update(algorithmic_bytes=work[name], GBps=work[name] / t / 1e3,
                     hbm_frac=work[name] / t / 1e3 / HBM_PEAK_GBS)
        kernels[name] = k
    if whole and p.dtype == "bf16" and "gather" in kernels:
        # what the gather writes beyond the method's bytes: the GEMM's operand
        # planes (alpha times the narrower operand, hi + lo in exact mode; in
        # the float16 mode the scaled float16 planes: both operands when the
        # narrower one is wider than 1024, else only the one with alpha, the
        # GEMM converting the other in registers)
        if args.dw_mode == "f16":
            plane_cols = d_o + d_i if min(d_o, d_i) > 1024 else min(d_o, d_i)
        else:
            plane_cols = min(d_o, d_i) * (2 if args.dw_mode == "exact" else 1)
        kernels["gather"]["gemm_plane_bytes"] = M * plane_cols * 2
    ssc_us = sum(us[n] for n in ("lrm_score", "select_scan", "gather") if us[n] is not None)
    nbytes = algorithmic_bytes(p, M, args.score_mode)
    if chain or zero_in_gemm:   # no dphi rows to zero in the original layout, or
        nbytes -= (P - M) * 4 * d_i   # they are zeroed inside the GEMM launch
    dominant_flops = 4.0 * M * gu.d_out * gu.d_in if gu is not None else work["grouped_gemm"]
    gemm_tf = dominant_flops / gemm_live["mean"] / 1e6
    # MFMA work the kernel executes: products of split operands cost one MFMA
    # pass per term (exact mode: alpha * (narrower operand) as hi + lo).
    terms_dw = 1 + (args.dw_mode == "exact" or p.dtype != "bf16") + (p.dtype != "bf16")
    terms_dp = 1 if p.dtype == "bf16" else 3
    if chain:   # gate/up on the float32 hand-off: alpha * dgu (hi + lo unless single
        # rounding) feeds both products
        terms_dw = terms_dp = 1 if args.dw_mode == "bf16" else 2
    if gu is not None:
        exec_flops = 2.0 * M * gu.d_out * gu.d_in * (terms_dw + terms_dp)
    else:
        Mx = p.P if dense_path else M
        exec_flops = 2.0 * Mx * p.d_out * p.d_in * (terms_dw + terms_dp)
    # committed counters of the dominant launch (the gate/up leg where there is one)
    traffic, mfma_busy = (None, None) if chain or dense_path else read_counters(
        p.name, args.dw_mode, "gate_up" if gu is not None else "down")
    roof = dict(kernel="grouped_backward_kernel", bound="mfma", achieved=gemm_tf,
                peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s", frac=gemm_tf / MFMA_BF16_PEAK_TFLOPS,
                mfma_executed_TFLOPs=exec_flops / gemm_live["mean"] / 1e6,
                launch_us_mean=gemm_live["mean"], launch_us_median=gemm_live["median"],
                launches=gemm_live["launches"],
                traffic=traffic, traffic_unit="bytes per launch",
                mfma_busy_frac=mfma_busy,
                algorithmic_bytes_floor=gemm_floor_bytes(p, M) + (zero_bytes if zero_in_gemm else 0))
    if traffic is not None:   # the launch's measured HBM traffic per second of its duration
        roof["traffic_GBps"] = traffic / gemm_live["mean"] / 1e3
        roof["traffic_hbm_frac"] = roof["traffic_GBps"] / HBM_PEAK_GBS
    if zero_in_gemm:
        roof["zero_fill_bytes"] = zero_bytes
        roof["zero_fill_note"] = ("the launch also clears the dropped pairs' dphi rows "
                                  "(zero_fill_bytes of stores beside the tiles), which the "
                                  "gather would otherwise write")
    if gu is not None:
        roof["note"] = "the gate/up projection's grouped GEMM (its flops 4 M d_out2 d_in2)"
        es2 = 2
        gu_zero = (0 if chain or not lrmoe.zero_fill_in_gemm(plan2)
                   else (P - M) * 4 * gu.d_in)   # cleared in that launch
        roof["algorithmic_bytes_floor"] = (M * es2 * (gu.d_out + gu.d_in)
                                           + p.E * gu.d_out * gu.d_in * (es2 + 4)
                                           + M * gu.d_in * 4 + gu_zero)
        roof.pop("zero_fill_bytes", None)
        roof.pop("zero_fill_note", None)
        if gu_zero:
            roof["zero_fill_bytes"] = gu_zero
    rec = {
        "metric": "kept pairs/s + grouped-GEMM TFLOP/s (% MFMA peak), score/compact % HBM BW",
        "value": M * args.steps / elapsed,
        "unit": "kept pairs/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if p.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": p.name + ("+masked-dense" if dense_path else ""),
                   **({"chain": "down GEMM + SiLU-GLU epilogue -> gather x -> gate/up GEMM"}
                      if chain else {}),
                   "P": p.P, "E": p.E, "d_out": p.d_out, "d_in": p.d_in,
                   "kept_pairs": M, "policy": list(p.policy), "dw_mode": args.dw_mode,
                   "score_mode": args.score_mode,
                   "parallelism": "single GPU (one expert-parallel rank's share)"},
        "roofline": roof,
        "score_select_compact": {"us": ssc_us, "algorithmic_bytes": nbytes,
                                 "GBps": nbytes / ssc_us / 1e3 if ssc_us else None,
                                 "hbm_frac": nbytes / ssc_us / 1e3 / HBM_PEAK_GBS if ssc_us else None},
        "score_select_compact_cold": None if not cold else {
            how: {"us": sum(v["mean"] for v in c.values()),
                  "kernels_us": {k: v["mean"] for k, v in c.items()},
                  "GBps": nbytes / sum(v["mean"] for v in c.values()) / 1e3,
                  "hbm_frac": nbytes / sum(v["mean"] for v in c.values()) / 1e3 / HBM_PEAK_GBS}
            for how, c in cold.items()},
        "score_select_compact_cold_note": ("before each of these steps a 512 MiB buffer is "
                                           "read (clean eviction of L2 and MALL) or written "
                                           "(its dirty lines are written back while the "
                                           "kernels run)") if cold else None,
        "score_select_compact_note": ("the gather also writes the GEMM's operand planes "
                                      "(kernels.gather.gemm_plane_bytes), which the operand "
                                      "prologue would otherwise write; they are not counted "
                                      "in algorithmic_bytes") if whole and p.dtype == "bf16"
                                     else None,
        "kernels": kernels,
        "kernels_note": f"separate pass of {nb} steps after the timed region, HIP events "
                        "around every kernel",
    }
    if gu is not None:
        if chain:
            gd = stats_us([a.elapsed_time(b) * 1e3 for a, b in gu_ev])
            gg = stats_us(gu_timer.durations_us(1))
            gpro, gred = gu_timer.mean_us(0), gu_timer.mean_us(2)
        else:   # lrmoe_gather_backward slots: gather 2, GEMM 3, reduction 4
            gd = stats_us(gu_timer.durations_us(2))
            gg = stats_us(gu_timer.durations_us(3))
            gpro, gred = gu_timer.mean_us(5), gu_timer.mean_us(4)
        if chain:   # x rows and alpha only: the gate/up gradient is already compacted
            gbytes = M * (2 * es * gu.d_in + 12) + (P - M) * 4 * gu.d_in
        else:   # its dropped dphi rows: in the gather unless cleared in the GEMM launch
            gbytes = M * (2 * es * (gu.d_out + gu.d_in) + 12) + (
                0 if lrmoe.zero_fill_in_gemm(plan2) else (P - M) * 4 * gu.d_in)
        gfl = 4.0 * M * gu.d_out * gu.d_in
        rec["gate_up"] = {
            "d_out": gu.d_out, "d_in": gu.d_in,
            "gather_compact": {"us": gd["mean"], "us_median": gd["median"],
                               "algorithmic_bytes": gbytes, "GBps": gbytes / gd["mean"] / 1e3,
                               "hbm_frac": gbytes / gd["mean"] / 1e3 / HBM_PEAK_GBS},
            "grouped_gemm": {"us": gg["mean"], "us_median": gg["median"],
                             "algorithmic_flops": gfl, "TFLOPs": gfl / gg["mean"] / 1e6,
                             "mfma_frac": gfl / gg["mean"] / 1e6 / MFMA_BF16_PEAK_TFLOPS,
                             **({} if chain or not lrmoe.zero_fill_in_gemm(plan2) else
                                {"zero_fill_bytes": (P - M) * 4 * gu.d_in})},
            "operand_prologue_us": gpro, "splitk_reduce_us": gred}
        gu_timer.close()
    if dense_path:
        sd = stats_us([a.elapsed_time(b) * 1e3 for a, b in gu_ev])
        rec["masked_dense"] = {
            "note": "same selection, alpha := 0 on dropped pairs, grouped GEMMs over all P "
                    "routed pairs of the uncompacted g and phi; value counts kept pairs, so it "
                    "compares directly with the compacted path",
            "score_select_mask_us": sd["mean"],
            "gemm_executed_flops": gemm_flops(p, P), "gemm_kept_flops": gemm_flops(p, M)}
        gu_timer.close()
    ssc_timer.close()
    gb_timer.close()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(p, chain=chain)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
