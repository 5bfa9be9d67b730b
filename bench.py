#!/usr/bin/env python3
"""Throughput of causal, normalized Hedgehog linear attention on one MI355X.

One step = one hm_linattn_fwd over the largest prefill workload that fits one
GPU, the long-context layer: B=1, H=16, n=131072, d=128, f=64, dv=128, bf16 in,
float32 accumulation, Mamba-style decay (dt ~ N(0,1), A_log ~ U(0, ln 16)):
featurize q and k, intra- and inter-chunk products, state passing (segment pass,
composition, full pass), normalize.  Prints ONE JSON line.  Beside the headline:
  * roofline: the call against HBM bandwidth (it is HBM-bound: ~96 flop/byte
    against a ridge of ~315), from HIP-event timing on the launch stream;
  * mfma: executed and algorithmic bf16 MFMA rates against the dense peak;
  * configs: the same blocks for the Pythia-1B-shaped layer (B=8, H=16, n=2048,
    identity decay) and the Mamba-decay layer (B=2, H=16, n=8192), and the tiny
    float32 case (B=1, H=2, n=256); each prefill config with its per-call spread
    (warm, and cold with L2 and the MALL overwritten before each call);
  * featurize: the standalone Hedgehog featurizer on the Pythia layer's q;
  * prefill_extra: the gated layer, the rotary encoding of 32 and of all 128
    features, the short conv and the stage-2 chain, a training step (forward that
    saves + backward, with the backward's roofline), the per-channel-decay scan;
  * decode: the decode step at B=256, H=16 (state [128 x 129] float32 per head,
    4096-token prefix, 512 steps) against HBM bandwidth, and its variants;
  * cpu_baseline: the float64 CPU oracle on the same inputs, on all host cores (a
    process pool over heads) and on one thread, per config, on bounded samples.

Clock warm-up: before every timed loop the call runs back to back for at least
--warmup-ms of wall time (and at least --warmup calls), so that the timed steps
see the GPU's sustained clock rather than its ramp; the time spent is reported.

  python bench.py [--steps K] [--warmup W] [--warmup-ms T] [--gpus 1] [--no-cpu-baseline] [--no-extra]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import multiprocessing as mp
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
MFMA_FLOP = 16 * 16 * 32 * 2   # one v_mfma_f32_16x16x32_bf16
METRIC = "prefill tokens/s + % bf16 MFMA peak; decode tokens/s + % HBM BW (1 MI355X)"
KERNEL_SOURCES = ["hm_device.hpp", "hm_prefill.hpp", "hm_step.hpp", "hm_cp.hpp", "hm_abi.hip"]  # kernels and plans
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters.json")
CPU_WORKERS_MAX = 12           # oracle processes: the GPU machine allows 16 processes per GPU


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "selective_state_space_hm_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------- work models
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


def backward_bytes(B, H, n, d, dv, decay, elem=2):
    """Algorithmic HBM bytes of the backward pass: q, k, v and dO read once, dq, dk,
    dv written once (and dt read, d dt written, with decay); the float32 weight
    gradients are negligible."""
    return B * H * n * (elem * (3 * d + 4 * dv) + (8 if decay else 0))


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
    structure of the chunk kernel, per 64-token block and workgroup:
      feature waves: featurize q and k, phi(k)^T re-layout, the ten causal score
      tiles, the z update (ones-column products);
      state waves: v re-layout, inter read-out, intra read-out, state update;
    with 128-token chunks the second block of each chunk adds the 16 off-diagonal
    score tiles and their share of the intra read-out.  The segment pass (64-token
    blocks at any chunk length) featurizes k only and updates the state only."""
    chunk, segments, dsplit = plan
    C = 64
    NCT, NFH, NFT = C // 16, f // 16, 2 * f // 16
    KD, KF, KC = d // 32, NFT // 2, NCT // 2
    vt = dv // dsplit // 16                        # value tiles per workgroup
    intra_steps = sum(bt // 2 + 1 for bt in range(NCT))
    full = (2 * NCT * NFH * KD + NCT * NFT + sum(NCT - a for a in range(NCT)) * KF + NFT * KC
            + vt * NCT + vt * NCT * KF + vt * NFT * KC + vt * intra_steps)
    offdiag = NCT * NCT * KF + vt * NCT * KC
    chunks = (n + chunk - 1) // chunk
    per = -(-chunks // segments)
    nseg = -(-chunks // per)
    seg_len = per * chunk
    full_total = 0
    for sgi in range(nseg):
        blocks = -(-min(seg_len, n - sgi * seg_len) // C)
        full_total += blocks * full + (blocks // 2 if chunk == 128 else 0) * offdiag
    ls = segment_pass_split(B, H, nseg, per, dv, dsplit)
    vtl = dv // ls // 16
    local = NCT * NFH * KD + NCT * NFT + NFT * KC + vtl * NCT + vtl * NFT * KC
    local_blocks = (seg_len // C) * (nseg - 1)
    return B * H * (dsplit * full_total + ls * local * local_blocks)



# ---------------------------------------------------------------- timing
def clock_warmup(fn, torch, min_calls, min_ms):
    """Run fn() back to back until at least min_calls calls and min_ms of wall time
    have passed (the GPU raises its clock over the first ~20 ms of sustained work).
    Returns the milliseconds spent."""
    t0 = time.perf_counter()
    calls = 0
    while calls < min_calls or (time.perf_counter() - t0) * 1e3 < min_ms:
        fn()
        calls += 1
        if calls % 16 == 0:
            torch.cuda.synchronize()   # keep the host from running far ahead of the GPU
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3


def time_launches(fn, steps, warmup, torch, warmup_ms=0.0):
    """Average ms per call of fn(), HIP events on torch's current stream (the stream
    the library launches on), bracketed by device synchronization, after the clock
    warm-up.  Returns (ms, wall seconds of the timed region, warm-up ms)."""
    wu = clock_warmup(fn, torch, warmup, warmup_ms)
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return s.elapsed_time(e) / steps, wall, wu


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
    return rec.get("bytes_per_launch", {}).get(key)


def cp_mfma_count(B, H, n, d, f, dv, C):
    """MFMA instructions (16x16x32 bf16) of the chunk-parallel path, from its loop
    structure: per 64-token block of the local pass, the k projection (4 token tiles x
    f/16 feature tiles x d/32 K-steps) and the local state (2f/16 x dv/16 tiles, 2
    K-steps); per 64-query block of the output pass, the q projection, the read-out of
    the start state (4 x dv/16 tiles, 2f/32 K-steps) and, per key block up to its own,
    the k projection, 16 score tiles (2f/32 K-steps) and the weighted scores times V
    (4 x dv/16 tiles, 2 K-steps)."""
    F = 2 * f
    proj = 4 * (f // 16) * max(1, d // 32)
    local_blk = proj + (F // 16) * (dv // 16) * 2
    per_kb = proj + 16 * (F // 32) + 4 * (dv // 16) * 2
    total = 0
    for c0 in range(0, n, C):
        nb = -(-min(C, n - c0) // 64)
        total += nb * local_blk
        total += sum(proj + 4 * (dv // 16) * (F // 32) + (qb + 1) * per_kb for qb in range(nb))
    return B * H * total


def is_cp_plan(plan):
    """Chunk 256 runs on the chunk-parallel path (so do sizes without a fused kernel,
    which no benchmarked workload has)."""
    return plan[0] == 256


def kernel_names(plan, decay, d, f, dv, elem):
    chunk, segs, dsplit = plan
    if is_cp_plan(plan):
        return f"hm_linattn_fwd (chunk-parallel, chunk {chunk}): cp_local_kernel + cp_scan_kernel + cp_out_kernel"
    dw = dv // dsplit
    name = f"fwd_kernel<{'bf16' if elem == 2 else 'float'},{d},{f},{dw},{'true' if decay else 'false'},FULL>"
    return "hm_linattn_fwd: " + name + (" + segment pass" if segs > 1 else "") + \
        (" + combine_kernel" if segs > 2 else "")


def prefill_block(torch, hm, case, dev, ws, steps, warmup, warmup_ms, key, chunk=0, distribution=True):
    """Time hm_linattn_fwd on one workload; the roofline, MFMA and spread blocks."""
    g = {k: (None if getattr(case, k) is None else getattr(case, k).to(dev))
         for k in ("q", "k", "v", "w_q", "w_k", "dt", "a_log")}
    o = torch.empty_like(g["v"])
    args = (g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"])
    plan = hm.hm_linattn_fwd_plan(*args, chunk=chunk)
    st, need = hm.call_workspace_size(hm.fwd_args(*args, o=o, chunk=chunk))
    if need > ws.numel():  # the chunk-parallel path keeps every chunk's state
        ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def step():
        hm.hm_linattn_fwd(*args, o=o, workspace=ws, chunk=chunk)

    log(f"[bench] {case.name} B={case.B} H={case.H} n={case.n}: plan {plan}, {steps} timed steps")
    ms, wall, wu = time_launches(step, steps, warmup, torch, warmup_ms)
    B, H, n, d, f, dv = case.B, case.H, case.n, case.d, case.f, case.dv
    decay = case.dt is not None
    elem = 2 if case.dtype == torch.bfloat16 else 4
    nbytes = prefill_bytes(B, H, n, d, f, dv, decay, elem)
    achieved = nbytes / (ms * 1e-3) / 1e9
    out = {"workload": f"{case.name} B={B} H={H} n={n} d={d} f={f} dv={dv}, "
                       + ("Mamba decay" if decay else "identity decay"),
           "ms": ms, "tokens_per_s": B * n / (ms * 1e-3), "wall_s_timed": wall, "clock_warmup_ms": wu,
           "plan": {"chunk": plan[0], "segments": plan[1], "dsplit": plan[2]},
           "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": achieved / HBM_PEAK_GBS, "traffic": hbm_traffic(key),
                        "kernel": kernel_names(plan, decay, d, f, dv, elem), "algorithmic_bytes_per_launch": nbytes}}
    if elem == 2:
        cp = is_cp_plan(plan)
        mfma = (cp_mfma_count(B, H, n, d, f, dv, plan[0]) if cp else prefill_mfma_count(plan, B, H, n, d, f, dv)) \
            * MFMA_FLOP
        algo = prefill_flops_algorithmic(B, H, n, d, f, dv)
        out["mfma"] = {"executed_tflops": mfma / (ms * 1e-3) / 1e12,
                       "executed_frac": mfma / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                       "algorithmic_tflops": algo / (ms * 1e-3) / 1e12,
                       "algorithmic_frac": algo / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                       "peak_tflops": BF16_PEAK_TFLOPS, "executed_mfma_per_call": mfma // MFMA_FLOP}
    if distribution:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        reps = 50 if ms < 1.0 else 20
        out["distribution"] = {
            "warm": step_distribution(step, reps, torch),
            "cold": step_distribution(step, reps, torch, flush=lambda: scratch.fill_(1)),
            "note": "single calls, each between its own event pair with the host waiting in between (so each "
                    "includes the gaps between its launches and the GPU idles between calls); cold: a 512 MiB "
                    "fill before each call evicts L2 and the MALL, whose dirty lines are written back while the "
                    "call runs. The main figure times back-to-back calls on the same inputs"}
        del scratch
    return out


# ---------------------------------------------------------------- CPU baseline
def _bf16_bits_to_f64(bits):
    import numpy as np
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _oracle_worker(job):
    """One group of (b, h) rows: the oracle's recurrent form over successive 64-token
    slices, carrying its state, until the time budget is spent.  Inputs arrive as
    raw bf16 bits (converted exactly to float64 here).  Returns tokens processed."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import hm_oracle as orc
    q, k, v, wq, wk, dt, a_log, budget = job
    q, k, v, wq, wk = (_bf16_bits_to_f64(x) for x in (q, k, v, wq, wk))
    S = z = None
    done, t0 = 0, time.perf_counter()
    with threadpool_limits(limits=1):
        while done < q.shape[2] and time.perf_counter() - t0 < budget:
            sl = slice(done, min(q.shape[2], done + 64))
            _, S, z = orc.forward(q[:, :, sl], k[:, :, sl], v[:, :, sl], wq, wk,
                                  None if dt is None else dt[:, :, sl], a_log, S, z)
            done = sl.stop
    return done, time.perf_counter() - t0


def _bits(t, torch):
    return t.contiguous().view(torch.int16).numpy().view("uint16")


def cpu_oracle_rate(case, torch, budget, workers, cap):
    """Token throughput of the recurrent float64 oracle on the first `cap` tokens of
    every (b, h) of `case`: the (b, h) rows are split into `workers` groups, one
    process each (1 thread each), or run vectorized in this process when workers
    is 1.  All groups run for the same time budget; the rate counts the tokens
    every group reached."""
    import numpy as np
    n = min(case.n, cap)
    rows = [(b, h) for b in range(case.B) for h in range(case.H)]
    groups = [list(x) for x in np.array_split(np.arange(len(rows)), min(workers, len(rows)))]
    jobs = []
    for grp in groups:
        bs = [rows[i][0] for i in grp]
        hs = [rows[i][1] for i in grp]
        sel = lambda t: t[bs, hs][None, :, :n]
        dt = None if case.dt is None else case.dt[bs, hs][None, :, :n].double().numpy()
        al = None if case.a_log is None else case.a_log[hs].double().numpy()
        jobs.append((_bits(sel(case.q), torch), _bits(sel(case.k), torch), _bits(sel(case.v), torch),
                     _bits(case.w_q, torch), _bits(case.w_k, torch), dt, al, budget))
    if len(jobs) == 1:
        res = [_oracle_worker(jobs[0])]
    else:
        with mp.get_context("spawn").Pool(len(jobs)) as pool:
            res = pool.map(_oracle_worker, jobs)
    tokens = min(r[0] for r in res)
    el = max(r[1] for r in res)
    # every group covers its rows for `tokens` positions; positions are counted per batch row
    return case.B * tokens / el, tokens, el, len(jobs)


def cpu_prefix_and_steps(torch, budget, workers):
    """Decode workload on the CPU oracle: (a) the closed-form prefix state of the
    4096-token prefix (featurize, then one DGEMM per head) for as many sequences as
    the budget allows, (b) recurrent decode steps over a sample of sequences."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import hm_oracle as orc
    from selective_state_space_hm_amd import inputs
    dc = inputs.decode_setup(B=8)     # the first 8 sequences of the B=256 draw order would differ: own sample
    f64 = inputs.to_f64
    wq, wk, al = f64(dc.w_q), f64(dc.w_k), f64(dc.a_log)
    with threadpool_limits(limits=workers):
        t0, nseq = time.perf_counter(), 0
        S = z = None
        while nseq < dc.B and time.perf_counter() - t0 < budget:
            b = slice(nseq, nseq + 1)
            pk = orc.hedgehog_features(f64(dc.prefix_k[b]), wk)
            Sb, zb = orc.prefix_state(pk, f64(dc.prefix_v[b]), orc.log_decay(f64(dc.prefix_dt[b]), al))
            S = Sb if S is None else np.concatenate([S, Sb])
            z = zb if z is None else np.concatenate([z, zb])
            nseq += 1
        el_prefix = time.perf_counter() - t0
        t0, steps = time.perf_counter(), 0
        while steps < dc.steps and time.perf_counter() - t0 < budget:
            q, k, v, dt = inputs.decode_step_inputs(dc, steps)
            _, S, z = orc.step(S, z, f64(q[:nseq]), f64(k[:nseq]), f64(v[:nseq]), wq, wk, f64(dt[:nseq]), al)
            steps += 1
        el_steps = time.perf_counter() - t0
    return {"prefix_states_per_s": nseq * dc.H / el_prefix, "prefix_sample": f"{nseq} sequences x {dc.H} heads, "
            f"4096-token prefix, closed form (featurize + one DGEMM per head), {el_prefix:.1f} s, BLAS threads {workers}",
            "decode_tokens_per_s": nseq * steps / el_steps,
            "decode_sample": f"{steps} recurrent steps over {nseq} sequences x {dc.H} heads in {el_steps:.1f} s"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(torch, inputs, headline_case, budget=3.0):
    """The float64 oracle (recurrent form) on the same seeded inputs: the headline
    workload on all host cores (processes over heads, up to 12) and on one thread,
    then the other measured workloads on all cores, each on a bounded sample."""
    cores = len(os.sched_getaffinity(0))
    workers = max(1, min(CPU_WORKERS_MAX, cores))
    log(f"[bench] CPU oracle: {workers} processes, headline sample")
    rate, tok, el, used = cpu_oracle_rate(headline_case, torch, budget, workers, cap=16384)
    rate1, tok1, el1, _ = cpu_oracle_rate(headline_case, torch, budget, 1, cap=16384)
    out = {"value": rate, "unit": "tokens/s", "cores": used, "kind": "oracle",
           "sample": f"recurrent float64 oracle, all {headline_case.B}x{headline_case.H} (b,h) of the "
                     f"{headline_case.name} workload split over {used} processes of 1 thread, the first {tok} of "
                     f"{headline_case.n} tokens of every head in {el:.1f} s",
           "cpu_model": cpu_model(), "host_cores": cores,
           "one_thread": {"value": rate1, "unit": "tokens/s", "cores": 1,
                          "sample": f"same oracle, all (b,h) vectorized in one process of 1 thread, first {tok1} "
                                    f"tokens in {el1:.1f} s"},
           "configs": []}
    for maker in (inputs.pythia1b, inputs.mamba_decay):
        c = maker()
        log(f"[bench] CPU oracle: {c.name}")
        r, t, e, u = cpu_oracle_rate(c, torch, budget, workers, cap=4096)
        out["configs"].append({"workload": f"{c.name} B={c.B} H={c.H} n={c.n}", "value": r, "unit": "tokens/s",
                               "cores": u, "sample": f"first {t} tokens of every (b,h) in {e:.1f} s"})
        del c
    log("[bench] CPU oracle: decode")
    dec = cpu_prefix_and_steps(torch, budget, workers)
    dec["workload"] = "decode B=256 H=16 d=128 f=64 dv=128, 4096-token prefix (sampled sequences)"
    dec["cores"] = workers
    out["configs"].append(dec)
    return out


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--warmup-ms", type=float, default=250.0,
                    help="least wall time of back-to-back calls before each timed loop (clock ramp)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="headline and the other prefill configs only")
    ap.add_argument("--part", choices=["all", "headline", "pythia", "decay", "decode", "pc", "copy"], default="all",
                    help="headline/pythia/decay: one prefill config only (for profiling runs); decode: only the "
                         "decode benchmark; pc: only the per-channel-decay prefill and decode; copy: one 256 MiB "
                         "device copy, the reference run that calibrates rocprofv3's FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--chunk", type=int, default=0)
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
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
    if args.part == "decode":
        print(json.dumps({"decode": bench_decode(torch, hm, inputs, dev, ws)}), flush=True)
        return
    if args.part == "pc":
        print(json.dumps({"pc_prefill": bench_pc_prefill(torch, hm, inputs, dev, args),
                          "pc_long": bench_pc_long(torch, hm, inputs, dev, args),
                          "pc_decode": bench_pc_decode(torch, hm, inputs, dev)}), flush=True)
        return
    if args.part in ("pythia", "decay"):
        c = inputs.pythia1b() if args.part == "pythia" else inputs.mamba_decay()
        r = prefill_block(torch, hm, c, dev, ws, args.steps, args.warmup, args.warmup_ms, args.part,
                          args.chunk, distribution=False)
        print(json.dumps(r), flush=True)
        return

    log("[bench] generating the long-context workload B=1 H=16 n=131072")
    case = inputs.long_context()
    head = prefill_block(torch, hm, case, dev, ws, args.steps, args.warmup, args.warmup_ms,
                         "headline" if args.chunk in (0, 64) else f"headline_c{args.chunk}", args.chunk,
                         distribution=args.part == "all")
    result = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q, k, v; W ~ N(0, 1/d); dt ~ N(0,1); A_log ~ U(0, ln 16))",
        "config": {"workload": "long-context prefill, Mamba decay", "B": case.B, "H": case.H, "seq_len": case.n,
                   "d": case.d, "f": case.f, "dv": case.dv, "global_batch": case.B, "plan": head["plan"]},
        "roofline": head["roofline"],
        "mfma": head["mfma"],
        "clock_warmup_ms": head["clock_warmup_ms"],
        "wall_s_timed": head["wall_s_timed"],
    }
    if "distribution" in head:
        result["distribution"] = head["distribution"]
    if args.part == "all" and args.chunk == 0:
        # chunk-length sweep of the headline workload: time, HBM fraction and both MFMA fractions
        sweep = []
        for ch in (64, 128, 256):
            r = prefill_block(torch, hm, case, dev, ws, args.steps, args.warmup, args.warmup_ms,
                              "headline" if ch == 64 else f"headline_c{ch}", ch, distribution=False)
            sweep.append({"chunk": ch, "ms": r["ms"], "tokens_per_s": r["tokens_per_s"], "plan": r["plan"],
                          "hbm_frac": r["roofline"]["frac"], "traffic": r["roofline"]["traffic"],
                          "mfma_executed_frac": r["mfma"]["executed_frac"],
                          "mfma_algorithmic_frac": r["mfma"]["algorithmic_frac"],
                          "executed_mfma_per_call": r["mfma"]["executed_mfma_per_call"]})
        result["chunk_sweep"] = sweep
    if args.part == "headline":
        print(json.dumps(result), flush=True)
        return
    configs = []
    for maker, key in ((inputs.pythia1b, "pythia"), (inputs.mamba_decay, "decay")):
        c = maker()
        configs.append(prefill_block(torch, hm, c, dev, ws, max(args.steps, 100), args.warmup, args.warmup_ms, key))
        del c
    tiny = inputs.tiny()
    configs.append(prefill_block(torch, hm, tiny, dev, ws, max(args.steps, 100), args.warmup, args.warmup_ms, "tiny",
                                 distribution=False))
    configs[-1]["note"] = "512 token-heads: one launch of one workgroup per head, bound by launch latency"
    result["configs"] = configs
    if not args.no_extra:
        result["featurize"] = bench_featurize(torch, hm, inputs, dev, args)
        result["prefill_extra"] = bench_prefill_extra(torch, hm, inputs, dev, ws, args)
        result["prefill_extra"].append(bench_pc_prefill(torch, hm, inputs, dev, args))
        result["prefill_extra"].append(bench_pc_long(torch, hm, inputs, dev, args))
        result["decode"] = bench_decode(torch, hm, inputs, dev, ws)
        result["decode"]["per_channel_step"] = bench_pc_decode(torch, hm, inputs, dev)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(torch, inputs, case)
    print(json.dumps(result), flush=True)


def bench_featurize(torch, hm, inputs, dev, args):
    """The standalone featurizer (K1) on the Pythia layer's q: bf16 in, bf16 phi out."""
    c = inputs.pythia1b()
    q, w = c.q.to(dev), c.w_q.to(dev)
    phi = torch.empty((c.B, c.H, c.n, 2 * c.f), dtype=torch.bfloat16, device=dev)

    def step():
        hm.hm_featurize(q, w, phi=phi)

    ms, _, wu = time_launches(step, 100, args.warmup, torch, args.warmup_ms)
    nbytes = c.B * c.H * c.n * (2 * c.d + 2 * 2 * c.f) + c.d * c.f * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"hm_featurize of q, B={c.B} H={c.H} n={c.n} d={c.d} f={c.f}, bf16 phi", "ms": ms,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": nbytes},
            "kernel": "hm::featurize_kernel<bf16,bf16,128,64>", "clock_warmup_ms": wu}


def bench_prefill_extra(torch, hm, inputs, dev, ws, args):
    case = inputs.pythia1b()
    g = {k: getattr(case, k).to(dev) for k in ("q", "k", "v", "w_q", "w_k")}
    o = torch.empty_like(g["v"])
    B, H, n, d, f, dv = case.B, case.H, case.n, case.d, case.f, case.dv
    tokens = B * n
    plan = hm.hm_linattn_fwd_plan(g["q"], g["k"], g["v"], g["w_q"], g["w_k"])
    extra = []
    tl = lambda fn, steps=50: time_launches(fn, steps, args.warmup, torch, args.warmup_ms)[0]
    # the same layer with the mixer's gate branch fused into the output store
    gate = inputs.gate(case.v.shape, torch.bfloat16).to(dev)
    log("[bench] gated prefill, Pythia layer")
    msg = tl(lambda: hm.hm_linattn_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], o=o, workspace=ws, gate=gate))
    bg = prefill_bytes(B, H, n, d, f, dv, False, gate=True)
    extra.append({"workload": f"{case.name} B={B} H={H} n={n}, identity decay, o * SiLU(gate)", "ms": msg,
                  "tokens_per_s": tokens / (msg * 1e-3), "achieved_GBs": bg / (msg * 1e-3) / 1e9,
                  "hbm_frac": bg / (msg * 1e-3) / 1e9 / HBM_PEAK_GBS,
                  "plan": {"chunk": plan[0], "segments": plan[1], "dsplit": plan[2]}})
    # the rotary encoding of the features: a quarter of them turned (Pythia's rotary share) and all
    pos0 = torch.zeros(B, dtype=torch.int64, device=dev)
    for dims in (32, 128):
        log(f"[bench] rotary prefill dims={dims}, Pythia layer")
        msr = tl(lambda: hm.hm_linattn_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], o=o, workspace=ws,
                                           rope_dims=dims, rope_pos0=pos0))
        br = prefill_bytes(B, H, n, d, f, dv, False)
        extra.append({"workload": f"{case.name} B={B} H={H} n={n}, identity decay, rotary encoding of "
                                  f"{dims} of {2 * f} features", "ms": msr, "tokens_per_s": tokens / (msr * 1e-3),
                      "achieved_GBs": br / (msr * 1e-3) / 1e9, "hbm_frac": br / (msr * 1e-3) / 1e9 / HBM_PEAK_GBS})
    # the mixer's short causal conv (K = 4) on q, alone and in the stage-2 chain
    cw = (torch.randn((d, 4), generator=torch.Generator().manual_seed(1)) / 2).to(dev)
    qc, kc = torch.empty_like(g["q"]), torch.empty_like(g["k"])
    msc = tl(lambda: hm.hm_causal_conv(g["q"], cw, y=qc))
    bc = 2 * B * H * n * d * 2 + d * 4 * 4
    extra.append({"workload": f"short causal conv K=4 over q, B={B} H={H} n={n} d={d} bf16", "ms": msc,
                  "achieved_GBs": bc / (msc * 1e-3) / 1e9, "hbm_frac": bc / (msc * 1e-3) / 1e9 / HBM_PEAK_GBS,
                  "kernel": "hm::conv_kernel<bf16,4>", "algorithmic_bytes_per_launch": bc})

    def stepm():
        hm.hm_causal_conv(g["q"], cw, y=qc)
        hm.hm_causal_conv(g["k"], cw, y=kc)
        hm.hm_linattn_fwd(qc, kc, g["v"], g["w_q"], g["w_k"], o=o, workspace=ws, gate=gate)

    msm = tl(stepm)
    extra.append({"workload": f"stage-2 mixer chain: conv(q), conv(k), gated prefill, B={B} H={H} n={n}",
                  "ms": msm, "tokens_per_s": tokens / (msm * 1e-3), "vs_gated_prefill": msm / msg})
    del gate, qc, kc
    # training step: forward that saves, then the backward pass
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

    log("[bench] training forward + backward, Pythia layer")
    msf, msb, mst = tl(stept), tl(stepb), tl(steptb)
    bb = backward_bytes(B, H, n, d, dv, False)
    flops_b = 2 * prefill_flops_algorithmic(B, H, n, d, f, dv)
    extra.append({"workload": f"training step (forward saving for the backward, then hm_linattn_bwd), "
                              f"B={B} H={H} n={n}, identity decay", "ms": mst, "tokens_per_s": tokens / (mst * 1e-3),
                  "forward_ms": msf, "backward_ms": msb,
                  "backward_roofline": {"bound": "hbm", "achieved": bb / (msb * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                                        "unit": "GB/s", "frac": bb / (msb * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                        "algorithmic_bytes_per_launch": bb,
                                        "algorithmic_flops": flops_b,
                                        "model": "q, k, v, dO read once and dq, dk, dv written once (1792 B per "
                                                 "token-head); flops twice the forward's algorithmic count"},
                  "save_bytes": save.numel()})
    return extra


# VALU issue per (token, channel, state) of the per-channel scan: one quarter-rate
# exp2 (4 lane-slots of 16) and seven full-rate FMA/MUL ops; a SIMD issues 16
# lane-ops per clock, 1024 SIMDs at 2.4 GHz.
PC_SIMD_CYCLES_PER_ELEM = 7 / 16 + 1 / 4
SIMD_CLOCKS_PER_S = 1024 * 2.4e9


def bench_pc_prefill(torch, hm, inputs, dev, args):
    """Per-channel-decay prefill on the Pythia-1B-shaped layer (bf16, dt [B,H,n,dv])."""
    c = inputs.make_pc("pc-pythia1b", 8, 16, 2048, 128, 64, 128, torch.bfloat16)
    log(f"[bench] per-channel decay prefill B={c.B} H={c.H} n={c.n}")
    g = {k: getattr(c, k).to(dev) for k in ("q", "k", "v", "w_q", "w_k", "dt", "a_log")}
    o = torch.empty_like(g["v"])

    def step():
        hm.hm_linattn_pc_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], o=o)

    ms = time_launches(step, 10, 4, torch, args.warmup_ms)[0]
    elems = c.B * c.H * c.n * c.dv * 2 * c.f
    alu_s = elems * PC_SIMD_CYCLES_PER_ELEM / SIMD_CLOCKS_PER_S
    return {"workload": f"per-channel decay (A_log [H,dv,2f], dt [B,H,n,dv]) B={c.B} H={c.H} n={c.n}, element-wise scan",
            "ms": ms, "tokens_per_s": c.B * c.n / (ms * 1e-3),
            "roofline": {"bound": "alu", "achieved_elems_per_s": elems / (ms * 1e-3),
                         "alu_time_ms": alu_s * 1e3, "frac": alu_s / (ms * 1e-3),
                         "model": "1 exp2 (quarter rate) + 7 full-rate VALU ops per (token, channel, state)"},
            "kernel": "hm::pc_fwd_kernel<bf16,128,64,128,64,8>"}


def bench_pc_long(torch, hm, inputs, dev, args):
    """Per-channel-decay prefill on the long-context shape (B=1, H=16, n=131072, bf16):
    32 workgroups cover the sequence unsplit; the automatic plan scans it in segments
    (segment pass, element-wise composition, full pass).  Both timed."""
    c = inputs.make_pc("pc-long", 1, 16, 131072, 128, 64, 128, torch.bfloat16, seed=0)
    log(f"[bench] per-channel decay prefill B={c.B} H={c.H} n={c.n}: segmented and unsplit")
    g = {k: getattr(c, k).to(dev) for k in ("q", "k", "v", "w_q", "w_k", "dt", "a_log")}
    o = torch.empty_like(g["v"])
    plan = hm.hm_linattn_pc_plan(g["q"], g["v"], g["w_q"])
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=dev)

    def run(segments):
        return lambda: hm.hm_linattn_pc_fwd(g["q"], g["k"], g["v"], g["w_q"], g["w_k"], g["dt"], g["a_log"], o=o,
                                            segments=segments, workspace=ws)

    ms_seg = time_launches(run(0), 5, 2, torch, args.warmup_ms)[0]
    ms_one = time_launches(run(1), 2, 1, torch, 0.0)[0]
    elems = c.B * c.H * c.n * c.dv * 2 * c.f
    alu_s = elems * PC_SIMD_CYCLES_PER_ELEM / SIMD_CLOCKS_PER_S
    seg_len = -(-(-(-c.n // 64)) // plan) * 64
    work = (c.n + (plan - 1) * seg_len) / c.n  # scan work of both passes over the method's
    return {"workload": f"per-channel decay long context B={c.B} H={c.H} n={c.n} d={c.d} f={c.f} dv={c.dv} bf16",
            "segments": plan, "ms": ms_seg, "tokens_per_s": c.B * c.n / (ms_seg * 1e-3),
            "ms_unsplit": ms_one, "speedup_vs_unsplit": ms_one / ms_seg,
            "roofline": {"bound": "alu", "alu_time_ms": alu_s * 1e3, "frac": alu_s / (ms_seg * 1e-3),
                         "scan_work_over_method": work,
                         "model": "1 exp2 (quarter rate) + 7 full-rate VALU ops per (token, channel, state) of "
                                  "the method; the segment pass repeats the scan of all segments but the last"},
            "kernels": "hm::pc_fwd_kernel<...,LOCAL> + pc_combine_kernel + hm::pc_fwd_kernel<...>"}


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
    ms_all, _, _ = time_launches(run_all, 1, 0, torch)
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
                         "frac": gbs / HBM_PEAK_GBS, "traffic": hbm_traffic("decode"),
                         "kernel": "hm::step_kernel<bf16,128,64,128,true>", "algorithmic_bytes_per_launch": nbytes},
            "stage2_step": {"workload": "same steps with q, k through the fused short conv (K=4, state in place) "
                                        "and the output gated", "ms_per_step": ms2,
                            "tokens_per_s": dc.B / (ms2 * 1e-3)},
            "rotary_step": {"workload": f"same steps with the rotary encoding of all {F} features",
                            "ms_per_step": ms3, "tokens_per_s": dc.B / (ms3 * 1e-3)}}


if __name__ == "__main__":
    main()
