#!/usr/bin/env python3
"""Throughput of causal, normalized Hedgehog linear attention on one MI355X.

One step = one hm_linattn_fwd over the Pythia-1B-shaped layer (B=8, H=16,
n=2048, d=128, f=64, dv=128, bf16 in, float32 accumulation, identity decay):
featurize q and k, intra- and inter-chunk products, state passing, normalize.
Prints ONE JSON line.  Beside the headline prefill number it reports:
  * roofline: the prefill kernel against HBM bandwidth (it is HBM-bound:
    ~96 flop/byte against a ridge of ~315), from HIP-event timing of the
    launches on the stream they run on;
  * mfma: executed and algorithmic bf16 MFMA rates against the dense peak;
  * decode: the decode step at B=256, H=16 (state [128 x 129] float32 per head,
    4096-token prefix, 512 steps) against HBM bandwidth;
  * prefill_extra: the gated layer, the rotary encoding of 32 and of all 128
    features, the short conv and the stage-2 chain, a training step (forward
    that saves + backward), the Mamba-decay workloads (n=8192 and n=131072), the
    per-channel-decay scan on the same layer (ALU-bound) and its decode step;
  * distribution: median / p10 / p90 of single calls, warm and with the caches
    overwritten before each call (cold);
  * cpu_baseline: the float64 CPU oracle timed on a bounded sample.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-extra]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
MFMA_FLOP = 16 * 16 * 32 * 2   # one v_mfma_f32_16x16x32_bf16
METRIC = "prefill tokens/s + % bf16 MFMA peak; decode tokens/s + % HBM BW (1 MI355X)"
KERNEL_SOURCES = ["hm_device.hpp", "hm_prefill.hpp", "hm_step.hpp", "hm_abi.hip"]  # kernels and launch plans
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "selective_state_space_hm_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def prefill_bytes(B, H, n, d, f, dv, decay, elem=2, gate=False):
    """Algorithmic HBM bytes of one prefill: q, k, v read once, o written once,
    dt read once (decay only), the gate read once (gated only), W_q and W_k read once."""
    per_token_head = elem * (2 * d + 2 * dv + (dv if gate else 0)) + (4 if decay else 0)
    return B * H * n * per_token_head + 2 * d * f * elem + (H * 4 if decay else 0)


def prefill_flops_algorithmic(B, H, n, d, f, dv):
    """Chunk-independent work per token-head: featurize q and k (2 x 2df) and the
    state update plus read-out with the denominator column (2 x 2F(dv+1))."""
    F = 2 * f
    return B * H * n * (4 * d * f + 4 * F * (dv + 1))


def segment_pass_split(B, H, nseg, per, dv, dsplit):
    """Column split of the segment pass, as the library chooses it.  When its items
    fill at most half the chip it cuts each segment into 4 or 2 slots (a divisor
    of the segment's chunks) and keeps the full pass's columns; otherwise it takes
    the widest column split of 4 or 2 (32 columns at least) that keeps the pass
    within 256 workgroups."""
    items = B * H * (nseg - 1) * dsplit
    for cand in (4, 2):
        if per % cand == 0 and items * cand <= 256:
            return dsplit
    for cand in (4, 2):
        if cand > dsplit and dv % cand == 0 and dv // cand >= 32 and B * H * (nseg - 1) * cand <= 256:
            return cand
    return dsplit


def prefill_mfma_count(plan, B, H, n, d, f, dv):
    """MFMA instructions (16x16x32 bf16) the prefill kernels issue, from the loop
    structure of the chunk kernel, per 64-token chunk and workgroup:
      feature waves: featurize q and k, phi(k)^T re-layout, the ten causal score
      tiles, the z update (ones-column products);
      state waves: v re-layout, inter read-out, intra read-out, state update.
    The segment pass featurizes k only and updates the state only."""
    chunk, segments, dsplit = plan
    C = chunk
    NCT, NFH, NFT = C // 16, f // 16, 2 * f // 16
    KD, KF, KC = d // 32, NFT // 2, NCT // 2
    vt = dv // dsplit // 16                        # value tiles per workgroup
    intra_steps = sum(bt // 2 + 1 for bt in range(NCT))
    full = (2 * NCT * NFH * KD + NCT * NFT + sum(NCT - a for a in range(NCT)) * KF + NFT * KC
            + vt * NCT + vt * NCT * KF + vt * NFT * KC + vt * intra_steps)
    chunks = (n + C - 1) // C
    per = -(-chunks // segments)
    nseg = -(-chunks // per)
    ls = segment_pass_split(B, H, nseg, per, dv, dsplit)
    vtl = dv // ls // 16
    local = NCT * NFH * KD + NCT * NFT + NFT * KC + vtl * NCT + vtl * NFT * KC
    local_chunks = per * (nseg - 1)
    return B * H * (dsplit * full * chunks + ls * local * local_chunks)


def time_launches(fn, steps, warmup, torch):
    """Average ms per call of fn(), HIP events on torch's current stream (the stream
    the library launches on), bracketed by device synchronization."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return s.elapsed_time(e) / steps, wall


def step_distribution(fn, reps, torch, flush=None):
    """Per-call GPU times (ms) of fn(), each call bracketed by its own HIP events:
    median, p10 and p90.  With `flush`, it runs before every call and overwrites
    L2 and the 256 MB MALL (a cold start for the call's inputs)."""
    times = []
    for _ in range(reps):
        if flush is not None:
            flush()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        e.synchronize()
        times.append(s.elapsed_time(e))
    times.sort()
    pick = lambda q: times[min(len(times) - 1, int(q * (len(times) - 1) + 0.5))]
    return {"median_ms": pick(0.5), "p10_ms": pick(0.1), "p90_ms": pick(0.9), "reps": reps}


def cpu_baseline(case, budget_s=12.0):
    """The float64 oracle's recurrent form on the same inputs, all (b, h) at once,
    token slices continued through the carried state until the time budget is used."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import hm_oracle as orc
    from selective_state_space_hm_amd import inputs

    f64 = inputs.to_f64
    q, k, v = f64(case.q), f64(case.k), f64(case.v)
    wq, wk = f64(case.w_q), f64(case.w_k)
    S = z = None
    done, t0 = 0, time.perf_counter()
    with threadpool_limits(limits=1):
        while done < case.n and time.perf_counter() - t0 < budget_s:
            sl = slice(done, min(case.n, done + 64))
            _, S, z = orc.forward(q[:, :, sl], k[:, :, sl], v[:, :, sl], wq, wk, None, None, S, z)
            done = sl.stop
    el = time.perf_counter() - t0
    return {"value": case.B * done / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"recurrent float64 oracle, all {case.B}x{case.H} (b,h) of the B=8 H=16 d=128 f=64 layer, "
                      f"first {done} of {case.n} tokens in {el:.1f} s on 1 thread (BLAS limited to 1); "
                      f"host has {len(os.sched_getaffinity(0))} cores"}


def hbm_traffic(key):
    """HBM bytes per launch from committed rocprofv3 counter runs (profiles/), if
    they were taken on the current kernel sources; otherwise None."""
    try:
        with open(PROFILE_COUNTERS) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_hash") != kernel_hash():
        return None
    return rec.get(key)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU raises its clocks over the first ~20 ms of sustained work; the default
    # warm-up (about 30 ms of launches) times the steady state.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip decode and the decay workloads")
    ap.add_argument("--part", choices=["all", "decode", "copy"], default="all",
                    help="decode: only the decode benchmark; copy: one 256 MiB device copy, the "
                         "reference run that calibrates rocprofv3's FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--segments", type=int, default=0)
    ap.add_argument("--dsplit", type=int, default=0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the workload is the single-GPU hot path and this build "
              "has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from selective_state_space_hm_amd import hm, inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.part == "copy":
        a = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] copied 3 x 256 MiB")
        return
    if args.part == "decode":
        ws = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
        print(json.dumps({"decode": bench_decode(torch, hm, inputs, dev, ws)}), flush=True)
        return
    log("[bench] generating the B=8 H=16 n=2048 layer")
    case = inputs.pythia1b()
    g = {k: getattr(case, k).to(dev) for k in ("q", "k", "v", "w_q", "w_k")}
    o = torch.empty_like(g["v"])
    plan = hm.hm_linattn_fwd_plan(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], segments=args.segments,
                                  dsplit=args.dsplit)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=dev)

    def step():
        hm.hm_linattn_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], o=o, segments=args.segments,
                          dsplit=args.dsplit, workspace=ws)

    log(f"[bench] prefill plan (chunk, segments, dsplit) = {plan}; timing {args.steps} steps")
    ms, wall = time_launches(step, args.steps, args.warmup, torch)
    # per-call spread, warm (back to back) and cold (caches overwritten before each call)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    dist = {"warm": step_distribution(step, 50, torch),
            "cold": step_distribution(step, 50, torch, flush=lambda: scratch.fill_(1)),
            "note": "single calls, each between its own event pair with the host waiting in between (so "
                    "each includes the gap between its two launches and the GPU idles between calls); cold: a "
                    "512 MiB fill before each call evicts L2 and the MALL, whose dirty lines are written back "
                    "while the call runs. The headline value times back-to-back calls on the same inputs"}
    del scratch
    B, H, n, d, f, dv = case.B, case.H, case.n, case.d, case.f, case.dv
    tokens = B * n
    nbytes = prefill_bytes(B, H, n, d, f, dv, False)
    achieved = nbytes / (ms * 1e-3) / 1e9
    mfma = prefill_mfma_count(plan, B, H, n, d, f, dv) * MFMA_FLOP
    algo = prefill_flops_algorithmic(B, H, n, d, f, dv)
    traffic = hbm_traffic("prefill_bytes_per_launch")
    result = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q, k, v; W ~ N(0, 1/d))",
        "config": {"workload": "Pythia-1B-shaped layer prefill, identity decay", "B": B, "H": H, "seq_len": n,
                   "d": d, "f": f, "dv": dv, "global_batch": B,
                   "plan": {"chunk": plan[0], "segments": plan[1], "dsplit": plan[2]}},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "hm_linattn_fwd: fwd_kernel<bf16,128,64,128,false,FULL>"
                               + (" + segment pass" if plan[1] > 1 else "")
                               + (" + combine_kernel" if plan[1] > 2 else ""),
                     "algorithmic_bytes_per_launch": nbytes},
        "mfma": {"executed_tflops": mfma / (ms * 1e-3) / 1e12,
                 "executed_frac": mfma / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                 "algorithmic_tflops": algo / (ms * 1e-3) / 1e12,
                 "algorithmic_frac": algo / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                 "peak_tflops": BF16_PEAK_TFLOPS},
        "wall_s_timed": wall,
        "distribution": dist,
    }
    if not args.no_extra:
        extra = []
        # the same layer with the mixer's gate branch fused into the output store
        gate = inputs.gate(case.v.shape, torch.bfloat16).to(dev)
        log("[bench] gated prefill, same layer")

        def stepg():
            hm.hm_linattn_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], o=o, workspace=ws, gate=gate)

        msg, _ = time_launches(stepg, 50, 200, torch)
        bg = prefill_bytes(B, H, n, d, f, dv, False, gate=True)
        extra.append({"workload": f"{case.name} B={B} H={H} n={n}, identity decay, o * SiLU(gate)", "ms": msg,
                      "tokens_per_s": tokens / (msg * 1e-3), "achieved_GBs": bg / (msg * 1e-3) / 1e9,
                      "hbm_frac": bg / (msg * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      "plan": {"chunk": plan[0], "segments": plan[1], "dsplit": plan[2]}})
        # the rotary encoding of the features on the same layer: a quarter of the
        # features turned (Pythia's rotary share) and all of them
        pos0 = torch.zeros(B, dtype=torch.int64, device=dev)
        for dims in (32, 128):
            log(f"[bench] rotary prefill dims={dims}, same layer")

            def stepr():
                hm.hm_linattn_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], o=o, workspace=ws, rope_dims=dims,
                                  rope_pos0=pos0)

            msr, _ = time_launches(stepr, 50, 200, torch)
            br = prefill_bytes(B, H, n, d, f, dv, False)
            extra.append({"workload": f"{case.name} B={B} H={H} n={n}, identity decay, rotary encoding of "
                                      f"{dims} of {2 * f} features", "ms": msr, "tokens_per_s": tokens / (msr * 1e-3),
                          "achieved_GBs": br / (msr * 1e-3) / 1e9, "hbm_frac": br / (msr * 1e-3) / 1e9 / HBM_PEAK_GBS})
        # the mixer's short causal conv (K = 4) on q, alone and as part of the
        # stage-2 chain conv(q), conv(k) -> gated prefill
        cw = (torch.randn((d, 4), generator=torch.Generator().manual_seed(1)) / 2).to(dev)
        qc, kc = torch.empty_like(g["q"]), torch.empty_like(g["k"])

        def stepc():
            hm.hm_causal_conv(g["q"], cw, y=qc)

        msc, _ = time_launches(stepc, 50, 200, torch)
        bc = 2 * B * H * n * d * 2 + d * 4 * 4
        extra.append({"workload": f"short causal conv K=4 over q, B={B} H={H} n={n} d={d} bf16", "ms": msc,
                      "achieved_GBs": bc / (msc * 1e-3) / 1e9, "hbm_frac": bc / (msc * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      "kernel": "hm::conv_kernel<bf16,4>", "algorithmic_bytes_per_launch": bc})

        def stepm():
            hm.hm_causal_conv(g["q"], cw, y=qc)
            hm.hm_causal_conv(g["k"], cw, y=kc)
            hm.hm_linattn_fwd(qc, kc, g["v"], g["w_q"], g["w_k"], o=o, workspace=ws, gate=gate)

        msm, _ = time_launches(stepm, 50, 200, torch)
        extra.append({"workload": f"stage-2 mixer chain: conv(q), conv(k), gated prefill, B={B} H={H} n={n}",
                      "ms": msm, "tokens_per_s": tokens / (msm * 1e-3)})
        del gate, qc, kc
        # training step of the same layer: forward that saves, then the backward pass
        d_o = torch.randn(case.v.shape, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(dev)
        save = torch.empty(hm.save_size(g["q"], g["v"], g["w_q"]), dtype=torch.uint8, device=dev)
        bws = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

        def stept():
            hm.hm_linattn_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], o=o, workspace=ws, save=save)

        def stepb():
            hm.hm_linattn_bwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], d_o, save, workspace=bws)

        def steptb():
            stept()
            stepb()

        log("[bench] training forward + backward, same layer")
        msf, _ = time_launches(stept, 50, 100, torch)
        msb, _ = time_launches(stepb, 50, 100, torch)
        mst, _ = time_launches(steptb, 50, 100, torch)
        extra.append({"workload": f"training step (forward saving for the backward, then hm_linattn_bwd), "
                                  f"B={B} H={H} n={n}, identity decay", "ms": mst, "tokens_per_s": tokens / (mst * 1e-3),
                      "forward_ms": msf, "backward_ms": msb})
        del d_o, save, bws
    del g, o

    if not args.no_extra:
        for maker in (inputs.mamba_decay, inputs.long_context):
            c = maker()
            log(f"[bench] {c.name} n={c.n}")
            gg = {k: getattr(c, k).to(dev) for k in ("q", "k", "v", "w_q", "w_k", "dt", "a_log")}
            oo = torch.empty_like(gg["v"])
            pl = hm.hm_linattn_fwd_plan(gg["q"], gg["k"], gg["v"], gg["w_q"], gg["w_k"], gg["dt"], gg["a_log"])
            steps = 50 if c.n <= 8192 else 10

            def stepx():
                hm.hm_linattn_fwd(gg["q"], gg["k"], gg["v"], gg["w_q"], gg["w_k"], gg["dt"], gg["a_log"], o=oo,
                                  workspace=ws)

            msx, _ = time_launches(stepx, steps, 4 * steps, torch)
            bx = prefill_bytes(c.B, c.H, c.n, c.d, c.f, c.dv, True)
            extra.append({"workload": f"{c.name} B={c.B} H={c.H} n={c.n} Mamba decay", "ms": msx,
                          "tokens_per_s": c.B * c.n / (msx * 1e-3), "achieved_GBs": bx / (msx * 1e-3) / 1e9,
                          "hbm_frac": bx / (msx * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          "plan": {"chunk": pl[0], "segments": pl[1], "dsplit": pl[2]}})
            del gg, oo
        extra.append(bench_pc_prefill(torch, hm, inputs, dev))
        result["prefill_extra"] = extra
        result["decode"] = bench_decode(torch, hm, inputs, dev, ws)
        result["decode"]["per_channel_step"] = bench_pc_decode(torch, hm, inputs, dev)

    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(result), flush=True)


# VALU issue per (token, channel, state) of the per-channel scan: one quarter-rate
# exp2 (4 lane-slots of 16) and seven full-rate FMA/MUL ops; a SIMD issues 16
# lane-ops per clock, 1024 SIMDs at 2.4 GHz.
PC_SIMD_CYCLES_PER_ELEM = 7 / 16 + 1 / 4
SIMD_CLOCKS_PER_S = 1024 * 2.4e9


def bench_pc_prefill(torch, hm, inputs, dev):
    """Per-channel-decay prefill on the Pythia-1B-shaped layer (bf16, dt [B,H,n,dv])."""
    c = inputs.make_pc("pc-pythia1b", 8, 16, 2048, 128, 64, 128, torch.bfloat16)
    log(f"[bench] per-channel decay prefill B={c.B} H={c.H} n={c.n}")
    g = {k: getattr(c, k).to(dev) for k in ("q", "k", "v", "w_q", "w_k", "dt", "a_log")}
    o = torch.empty_like(g["v"])

    def step():
        hm.hm_linattn_pc_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], o=o)

    ms, _ = time_launches(step, 10, 20, torch)
    elems = c.B * c.H * c.n * c.dv * 2 * c.f
    alu_s = elems * PC_SIMD_CYCLES_PER_ELEM / SIMD_CLOCKS_PER_S
    return {"workload": f"per-channel decay (A_log [H,dv,2f], dt [B,H,n,dv]) B={c.B} H={c.H} n={c.n}, element-wise scan",
            "ms": ms, "tokens_per_s": c.B * c.n / (ms * 1e-3),
            "roofline": {"bound": "alu", "achieved_elems_per_s": elems / (ms * 1e-3),
                         "alu_time_ms": alu_s * 1e3, "frac": alu_s / (ms * 1e-3),
                         "model": "1 exp2 (quarter rate) + 7 full-rate VALU ops per (token, channel, state)"},
            "kernel": "hm::pc_fwd_kernel<bf16,128,64,128,64,8>"}


def bench_pc_decode(torch, hm, inputs, dev):
    """Per-channel-decay decode step, B=256 H=16 (state 2 x [128 x 128] fp32 per head)."""
    B, H, d, f, dv, steps = 256, 16, 128, 64, 128, 256
    c = inputs.make_pc("pc-decode", B, H, 1, d, f, dv, torch.bfloat16)
    log(f"[bench] per-channel decode B={B} H={H}: {steps} steps")
    g = {k: getattr(c, k).to(dev) for k in ("q", "k", "v", "w_q", "w_k", "dt", "a_log")}
    q1, k1, v1, dt1 = (g["q"][:, :, 0].contiguous(), g["k"][:, :, 0].contiguous(), g["v"][:, :, 0].contiguous(),
                       g["dt"][:, :, 0].contiguous())
    state = torch.zeros((B, H, hm.state_numel_pc(f, dv)), dtype=torch.float32, device=dev)
    o = torch.empty((B, H, dv), dtype=torch.bfloat16, device=dev)

    def run_all():
        for _ in range(steps):
            hm.hm_linattn_pc_step(q1, k1, v1, g["w_q"], g["w_k"], state, dt1, g["a_log"], o=o)

    run_all()
    torch.cuda.synchronize()
    ms = time_launches(run_all, 1, 0, torch)[0] / steps
    nbytes = B * H * (2 * 2 * dv * 2 * f * 4 + 2 * (2 * d + 2 * dv) + 4 * dv) + H * dv * 2 * f * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"per-channel decode B={B} H={H} d={d} f={f} dv={dv}, state 2 x [{dv}x{2 * f}] fp32",
            "ms_per_step": ms, "tokens_per_s": B / (ms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": nbytes},
            "kernel": "hm::pc_step_kernel<bf16,128,64,128>"}


def bench_decode(torch, hm, inputs, dev, ws):
    dc = inputs.decode_setup()
    log(f"[bench] decode B={dc.B} H={dc.H}: prefix {dc.prefix} tokens, {dc.steps} steps")
    wq, wk, a_log = dc.w_q.to(dev), dc.w_k.to(dev), dc.a_log.to(dev)
    state = torch.empty((dc.B, dc.H, hm.state_numel(dc.f, dc.dv)), dtype=torch.float32, device=dev)
    pk, pv, pdt = dc.prefix_k.to(dev), dc.prefix_v.to(dev), dc.prefix_dt.to(dev)
    hm.hm_linattn_fwd(pk, pk, pv, wq, wk, pdt, a_log, s_final=state, workspace=ws)  # prefill -> decode handoff
    del pk, pv, pdt
    qs, ks, vs, dts = [], [], [], []
    for t in range(dc.steps):
        q, k, v, dt = inputs.decode_step_inputs(dc, t)
        qs.append(q)
        ks.append(k)
        vs.append(v)
        dts.append(dt)
    Q = torch.stack(qs).to(dev)
    K = torch.stack(ks).to(dev)
    V = torch.stack(vs).to(dev)
    DT = torch.stack(dts).to(dev)
    O = torch.empty((dc.steps, dc.B, dc.H, dc.dv), dtype=torch.bfloat16, device=dev)
    base = state.clone()

    def run_all():
        for t in range(dc.steps):
            hm.hm_linattn_step(Q[t], K[t], V[t], wq, wk, state, DT[t], a_log, o=O[t])

    state.copy_(base)
    run_all()                       # warm-up pass over all steps
    state.copy_(base)
    torch.cuda.synchronize()
    ms_all, _ = time_launches(run_all, 1, 0, torch)
    ms = ms_all / dc.steps
    # the stage-2 step: q, k through the fused short conv (K = 4), output gated
    g2 = torch.Generator().manual_seed(3)
    cw = [(torch.randn((dc.d, 4), generator=g2) / 2).to(dev) for _ in range(2)]
    cst = [torch.zeros((dc.B, dc.H, 3, dc.d), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    G = (torch.randn((dc.steps, dc.B, dc.H, dc.dv), generator=g2)).to(torch.bfloat16).to(dev)

    def run_all2():
        for t in range(dc.steps):
            hm.hm_linattn_step(Q[t], K[t], V[t], wq, wk, state, DT[t], a_log, o=O[t], gate=G[t],
                               conv=(cw[0], cw[1], None, None, cst[0], cst[1]))

    state.copy_(base)
    run_all2()
    state.copy_(base)
    torch.cuda.synchronize()
    ms2 = time_launches(run_all2, 1, 0, torch)[0] / dc.steps
    # the same steps with the rotary encoding of all features at each row's position
    P0 = torch.full((dc.B,), dc.prefix, dtype=torch.int64, device=dev)
    POS = P0[None, :] + torch.arange(dc.steps, dtype=torch.int64, device=dev)[:, None]

    def run_all3():
        for t in range(dc.steps):
            hm.hm_linattn_step(Q[t], K[t], V[t], wq, wk, state, DT[t], a_log, o=O[t], rope_dims=2 * dc.f,
                               rope_pos=POS[t])

    state.copy_(base)
    run_all3()
    state.copy_(base)
    torch.cuda.synchronize()
    ms3 = time_launches(run_all3, 1, 0, torch)[0] / dc.steps
    F = 2 * dc.f
    per_bh = 2 * (F * dc.dv + F) * 4 + 2 * (2 * dc.d + 2 * dc.dv) + 4
    nbytes = dc.B * dc.H * per_bh + 2 * dc.d * dc.f * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"decode B={dc.B} H={dc.H} d={dc.d} f={dc.f} dv={dc.dv}, state [{F}x{dc.dv + 1}] fp32, "
                        f"{dc.prefix}-token prefix, {dc.steps} steps, Mamba decay",
            "tokens_per_s": dc.B / (ms * 1e-3), "ms_per_step": ms,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": hbm_traffic("decode_bytes_per_launch"),
                         "kernel": "hm::step_kernel<bf16,128,64,128,true>", "algorithmic_bytes_per_launch": nbytes},
            "stage2_step": {"workload": "same steps with q, k through the fused short conv (K=4, state in place) "
                                        "and the output gated", "ms_per_step": ms2,
                            "tokens_per_s": dc.B / (ms2 * 1e-3)},
            "rotary_step": {"workload": f"same steps with the rotary encoding of all {F} features",
                            "ms_per_step": ms3, "tokens_per_s": dc.B / (ms3 * 1e-3)}}


if __name__ == "__main__":
    main()
