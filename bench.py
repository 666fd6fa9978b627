#!/usr/bin/env python3
"""Benchmark of the Lightning Attention forward pass (prefill) on one MI355X.

One step = one full forward pass (every kernel of the path) over the
MiniMax-layer workload: batch 4, 64 heads, 8192 tokens, head_dim 128, block
256, bf16 in / fp32 accumulation / bf16 out, synthetic N(0,1) inputs already
resident in HBM.  Prints ONE JSON line on stdout.

Also reported in the same line (extra keys): per-kernel times from HIP events
recorded on the library's stream, the tiny fp32 case and two fp32 layer
shapes, the decode step's achieved GB/s (256 sequences x 64 heads, fp32
state, 128 steps), the state-handoff, rotary and indexed-decode variants, the
1,048,576-token prefill, the packed workloads, and the CPU oracle: timed on
the headline workload (`cpu_baseline`) and on every workload
(`cpu_baseline_per_workload`), with the CPU model and thread count.
"""
import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 (vector and MFMA), TFLOP/s
METRIC = "prefill tokens/s + TFLOP/s (% bf16 MFMA peak) at 64 heads, d=128; decode GB/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles created through the HIP runtime (for the library's
    stage markers, recorded on the stream the kernels run on)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.lib.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            out.append(e.value)
        return out

    def ms(self, a, b):
        f = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(f), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return f.value

    def destroy(self, evs):
        for e in evs:
            self.lib.hipEventDestroy(e)


def profiled_traffic(workload_name):
    """HBM bytes per launch of the fused kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, or None when that summary is for another
    workload or the kernel source changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"k_fused_dma_{workload_name}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.strip().split(":")[0] in ("traffic_bytes_per_launch", "source_sha256"):
            k, v = line.strip().split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in ("la_prefill.hip", "la_common.h"):
        with open(os.path.join(ROOT, "linear_attention_attn_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if fields.get("source_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in fields:
        return None
    return float(fields["traffic_bytes_per_launch"])


STAGES = ["tables", "summary", "scan", "fused"]


def stage_times(hip, evs, used, steps):
    """Mean ms per stage from the library's stage events (stage j runs from
    event j to event j + 1); a stage whose opening event was not recorded
    launched nothing and counts 0.  events_total spans the recorded ones."""
    out = {}
    for j, n in enumerate(STAGES):
        out[n] = (sum(hip.ms(e[j], e[j + 1]) for e in evs) / steps) if used[j] else 0.0
    first = used.index(True)
    out["events_total"] = sum(hip.ms(e[first], e[4]) for e in evs) / steps
    return out


def prefill_flops_per_head_token(d, B):
    """Algorithmic work: 2d^2 (Q S) + 2d^2 (K^T V) + 2d(B+1) (causal half of the
    intra-block Q K^T and P V, diagonal included)."""
    return 4 * d * d + 2 * d * (B + 1)


def bench_prefill(w, steps, warmup, dev, traced=True):
    import torch
    import linear_attention_attn_amd as la
    import synth

    q, k, v = synth.prefill_inputs(w.batch, w.heads, w.seq_len, w.head_dim, w.dtype, w.cid, dev)
    o = torch.empty_like(q)
    code = la.LA_DTYPE_BF16 if w.dtype == "bf16" else la.LA_DTYPE_F32
    nbytes = la.lightning_attn_fwd_workspace_size(w.batch, w.heads, w.seq_len, w.head_dim,
                                                  w.block_size, 0, code)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (q, k, v, o, w.batch, w.heads, w.seq_len, w.head_dim, w.block_size, None, code, ws,
            nbytes, stream)

    def step():
        st = la.lightning_attn_fwd(*args)
        if st != la.LA_OK:
            raise la.LightningAttnError(st, "lightning_attn_fwd")

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    chunk = la.lightning_attn_fwd_chunk_tokens(w.batch, w.heads, w.seq_len, w.head_dim,
                                               w.block_size, 0, code)
    # dense input builds no tables; one chunk per sequence runs no summaries
    # or scan: only the events around stages that launch work are recorded
    used = [False, True, True, True, True] if chunk < w.seq_len else [False, False, False, True, True]
    hip = HipEvents()
    evs = [hip.create(la.LA_FWD_NUM_EVENTS) for _ in range(steps)] if traced else None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if traced:
            rec = [e if u else None for e, u in zip(evs[i], used)]
            st = la.lightning_attn_fwd_traced(*args, rec, la.LA_FWD_NUM_EVENTS)
            if st != la.LA_OK:
                raise la.LightningAttnError(st, "lightning_attn_fwd_traced")
        else:
            step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stage = None
    if traced:
        stage = stage_times(hip, evs, used, steps)
        for e in evs:
            hip.destroy(e)
    del q, k, v, o, ws
    torch.cuda.empty_cache()
    return (t1 - t0) * 1000.0 / steps, stage, chunk, nbytes


def bench_prefill_varlen(w, steps, warmup, dev):
    """The packed workload (sequences of the log-uniform lengths back to back,
    cu_seqlens offsets) through lightning_attn_fwd_traced; returns (ms per
    step, per-kernel ms, chunk tokens, total tokens)."""
    import torch
    import linear_attention_attn_amd as la
    import synth

    lengths = synth.varlen_lengths(w.batch, w.len_seed, w.len_lo, w.len_hi)
    q, k, v, cu = synth.varlen_inputs(lengths, w.heads, w.head_dim, w.dtype, w.cid, dev)
    T = int(cu[-1])
    cud = torch.tensor(cu, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    code = la.LA_DTYPE_BF16 if w.dtype == "bf16" else la.LA_DTYPE_F32
    nbytes = la.lightning_attn_fwd_workspace_size(w.batch, w.heads, T, w.head_dim, w.block_size, 1, code)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (q, k, v, o, w.batch, w.heads, T, w.head_dim, w.block_size, cud, code, ws, nbytes, stream)
    for _ in range(warmup):
        st = la.lightning_attn_fwd(*args)
        if st != la.LA_OK:
            raise la.LightningAttnError(st, "lightning_attn_fwd")
    torch.cuda.synchronize()
    hip = HipEvents()
    evs = [hip.create(la.LA_FWD_NUM_EVENTS) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        st = la.lightning_attn_fwd_traced(*args, evs[i], la.LA_FWD_NUM_EVENTS)
        if st != la.LA_OK:
            raise la.LightningAttnError(st, "lightning_attn_fwd_traced")
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stage = stage_times(hip, evs, [True] * la.LA_FWD_NUM_EVENTS, steps)
    for e in evs:
        hip.destroy(e)
    chunk = la.lightning_attn_fwd_chunk_tokens(w.batch, w.heads, T, w.head_dim, w.block_size, 1, code)
    del q, k, v, o, ws, cud
    torch.cuda.empty_cache()
    return (t1 - t0) * 1000.0 / steps, stage, chunk, T


def bench_prefill_state(w, steps, warmup, dev, rope=False):
    """The prefill workload through lightning_attn_fwd_state, each sequence
    starting from a state and returning its final state (in place); with
    rope, through lightning_attn_fwd_rope instead (q and k rotated on half
    the head dims, base 10,000, positions from 0, no states)."""
    import torch
    import linear_attention_attn_amd as la
    import synth

    q, k, v = synth.prefill_inputs(w.batch, w.heads, w.seq_len, w.head_dim, w.dtype, w.cid, dev)
    o = torch.empty_like(q)
    S = synth.decode_state(w.batch, w.heads, w.head_dim, w.cid, dev)
    code = la.LA_DTYPE_BF16 if w.dtype == "bf16" else la.LA_DTYPE_F32
    nbytes = la.lightning_attn_fwd_workspace_size(w.batch, w.heads, w.seq_len, w.head_dim,
                                                  w.block_size, 0, code)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def with_state():
        if rope:
            st = la.lightning_attn_fwd_rope(q, k, v, o, w.batch, w.heads, w.seq_len, w.head_dim,
                                            w.block_size, None, code, w.head_dim // 2, 1e4, None,
                                            None, None, ws, nbytes, stream)
        else:
            st = la.lightning_attn_fwd_state(q, k, v, o, w.batch, w.heads, w.seq_len, w.head_dim,
                                             w.block_size, None, code, S, S, ws, nbytes, stream)
        if st != la.LA_OK:
            raise la.LightningAttnError(st, "lightning_attn_fwd_state")

    def plain():
        st = la.lightning_attn_fwd(q, k, v, o, w.batch, w.heads, w.seq_len, w.head_dim,
                                   w.block_size, None, code, ws, nbytes, stream)
        if st != la.LA_OK:
            raise la.LightningAttnError(st, "lightning_attn_fwd")

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    # alternate the two so that both see the same clocks
    ms_plain, ms_state = [], []
    for _ in range(2):
        ms_plain.append(timed(plain))
        ms_state.append(timed(with_state))
    del q, k, v, o, S, ws
    torch.cuda.empty_cache()
    return min(ms_state), min(ms_plain)


def bench_decode(w, reps, dev):
    import torch
    import linear_attention_attn_amd as la
    import synth

    S = synth.decode_state(w.batch, w.heads, w.head_dim, w.cid, dev)
    ins = [synth.decode_step_inputs(w.batch, w.heads, w.head_dim, w.dtype, w.cid, t, dev)
           for t in range(w.steps)]
    o = torch.empty_like(ins[0][0])
    stream = torch.cuda.current_stream(dev).cuda_stream
    code = la.LA_DTYPE_BF16 if w.dtype == "bf16" else la.LA_DTYPE_F32

    def run_all():
        for q, k, v in ins:
            st = la.lightning_attn_decode(q, k, v, S, o, w.batch, w.heads, w.head_dim, code, stream)
            if st != la.LA_OK:
                raise la.LightningAttnError(st, "lightning_attn_decode")

    run_all()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(reps):
        a.record()
        run_all()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / w.steps
        best = ms if best is None else min(best, ms)
    units = w.batch * w.heads
    d = w.head_dim
    bytes_step = units * (8 * d * d + 8 * d)   # fp32 state read+write; bf16 q, k, v, o
    del S, ins, o
    torch.cuda.empty_cache()
    return best, bytes_step / (best * 1e-3) / 1e9, units / (best * 1e-3)


def bench_decode_indexed(w, reps, dev, pad_rows=64):
    """The decode workload over an indexed state table: a pool of twice as
    many states, rows mapped to shuffled slots, and the same with the batch
    padded by pad_rows padding rows (slot -1)."""
    import numpy as np
    import torch
    import linear_attention_attn_amd as la
    import synth

    pool = synth.decode_state(2 * w.batch, w.heads, w.head_dim, w.cid, dev)
    rng = np.random.default_rng(w.cid)
    live = rng.permutation(2 * w.batch)[:w.batch].astype(np.int32)
    padded = np.full(w.batch + pad_rows, -1, np.int32)
    where = np.sort(rng.permutation(w.batch + pad_rows)[:w.batch])
    padded[where] = live
    code = la.LA_DTYPE_BF16 if w.dtype == "bf16" else la.LA_DTYPE_F32
    stream = torch.cuda.current_stream(dev).cuda_stream
    out = {}
    for name, sl in (("shuffled", live), ("padded", padded)):
        rows = len(sl)
        slots = torch.tensor(sl, device=dev)
        ins = [tuple(torch.nn.functional.pad(x, (0, 0, 0, 0, 0, rows - w.batch)).contiguous() for x in
                     synth.decode_step_inputs(w.batch, w.heads, w.head_dim, w.dtype, w.cid, t, dev))
               for t in range(w.steps)]
        o = torch.empty_like(ins[0][0])

        def run_all():
            for q, k, v in ins:
                st = la.lightning_attn_decode_indexed(q, k, v, pool, 2 * w.batch, slots, o, rows,
                                                      w.heads, w.head_dim, code, stream)
                if st != la.LA_OK:
                    raise la.LightningAttnError(st, "lightning_attn_decode_indexed")

        run_all()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        best = None
        for _ in range(reps):
            a.record()
            run_all()
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / w.steps
            best = ms if best is None else min(best, ms)
        live_bytes = w.batch * w.heads * (8 * w.head_dim ** 2 + 8 * w.head_dim)
        out[name] = {"rows": rows, "live_rows": w.batch, "ms_per_step": best,
                     "gbs_live": live_bytes / (best * 1e-3) / 1e9}
        del ins, o
    del pool
    torch.cuda.empty_cache()
    return out


def copy_calibration(dev, nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of known size (reads nbytes, writes nbytes)."""
    import torch
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(reps):
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_read": nbytes, "bytes_written": nbytes, "ms": best,
            "gbs_read_plus_write": 2 * nbytes / (best * 1e-3) / 1e9}


def cpu_info():
    """The host's CPU model, the cores this process may run on and the
    thread count the oracle uses: OMP_NUM_THREADS when it is set (the GPU
    box sets it to the CPU share of one GPU, which a run must not exceed),
    else every core in the affinity mask."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    try:
        threads = min(affinity, int(omp)) if omp else affinity
    except ValueError:
        threads = affinity
    return {"cpu_model": model, "cores_in_affinity": affinity, "omp_num_threads": omp,
            "threads": max(1, threads)}


def cpu_baseline(w, target_s, info):
    """The oracle (recurrent form, fp64, OpenMP over units) on the headline
    prefill workload: the whole workload, repeated to fill about target_s
    seconds when one run is shorter (else the largest prefix of its units
    that fits).  Scaled to tokens/s."""
    import torch

    import oracle
    import synth

    threads = info["threads"]
    oracle.build(force=False)
    n, d = w.seq_len, w.head_dim
    total = w.batch * w.heads

    def sample(units):
        nb = max(1, -(-units // w.heads))
        nh = min(units, w.heads)
        q, k, v = synth.prefill_inputs(nb, nh, n, d, w.dtype, w.cid, "cpu",
                                       heads_subset=list(range(nh)))
        return [x.to(torch.float32).reshape(nb * nh, n, d)[:units].numpy() for x in (q, k, v)]

    def run(q, k, v):
        t0 = time.perf_counter()
        oracle.causal_linear_attention(q, k, v, "recurrent", nthreads=threads)
        return time.perf_counter() - t0

    # probe with one unit per thread, then size the sample for ~target_s
    units = min(threads, total)
    dt = run(*sample(units))
    per_round = dt / units * threads                 # seconds per `threads` units
    units = min(total, max(units, int(target_s / max(per_round, 1e-6)) * threads))
    q, k, v = sample(units)
    reps = 1
    dt = run(q, k, v)
    if units == total:
        reps = max(1, min(20, int(target_s / max(dt, 1e-6))))
        for _ in range(reps - 1):
            dt += run(q, k, v)
    dt /= reps
    tok_s = units * n / w.heads / dt                 # tokens carrying all heads
    what = ("the whole workload" if units == total
            else f"{units} of {total} (sequence, head) units")
    return {"value": tok_s, "unit": "tokens/s", "cores": min(threads, units), "kind": "oracle",
            "sample": f"recurrent fp64 form on {what} ({units} units x {n} tokens, d={d}), "
                      f"mean of {reps} run(s) of {dt:.2f} s; tokens/s = head-tokens / {w.heads} heads / time",
            "seconds": dt * reps, "cpu_model": info["cpu_model"],
            "cores_in_affinity": info["cores_in_affinity"], "omp_num_threads": info["omp_num_threads"]}


def cpu_baseline_configs(dev, info):
    """The oracle timed on every workload, beside the GPU figures of the same
    run (a baseline only): the tiny fp32 case (naive and recurrent forms), the
    MiniMax layer, both packed workloads and the decode workload in full,
    and the 1M-token prefill on heads 0 and 63 at full length (two units, so
    two cores) with a labelled extrapolation to all 64 heads.  Inputs are the
    workloads' own (generated on the GPU, copied to the host)."""
    import numpy as np
    import torch

    import oracle
    import synth

    threads = info["threads"]
    oracle.build(force=False)
    out = {"cpu_model": info["cpu_model"], "cores_in_affinity": info["cores_in_affinity"],
           "omp_num_threads": info["omp_num_threads"]}
    f32 = lambda x: x.to("cpu").to(torch.float32).numpy()

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    # tiny fp32: naive and recurrent in full
    w = synth.WORKLOADS["tiny_f32"]
    q, k, v = (f32(x) for x in synth.prefill_inputs(w.batch, w.heads, w.seq_len, w.head_dim, w.dtype,
                                                     w.cid, dev))
    units = w.batch * w.heads
    tn = timed(lambda: oracle.causal_linear_attention(q, k, v, "naive", nthreads=threads))
    tr = timed(lambda: oracle.causal_linear_attention(q, k, v, "recurrent", nthreads=threads))
    out["tiny_f32"] = {"sample": "whole workload", "threads": min(threads, units),
                       "naive_s": tn, "recurrent_s": tr,
                       "tokens_per_s_recurrent": w.batch * w.seq_len / tr}
    log(json.dumps({"cpu tiny_f32": out["tiny_f32"]}))

    # MiniMax layer in full
    w = synth.WORKLOADS["minimax_layer"]
    q, k, v = (f32(x) for x in synth.prefill_inputs(w.batch, w.heads, w.seq_len, w.head_dim, w.dtype,
                                                     w.cid, dev))
    t = timed(lambda: oracle.causal_linear_attention(q, k, v, "recurrent", nthreads=threads))
    out["minimax_layer"] = {"sample": "whole workload", "threads": min(threads, w.batch * w.heads),
                            "seconds": t, "tokens_per_s": w.batch * w.seq_len / t}
    del q, k, v
    log(json.dumps({"cpu minimax_layer": out["minimax_layer"]}))

    # 1M tokens: heads 0 and 63 at full length, one core each
    w = synth.WORKLOADS["long_1m"]
    q, k, v = (f32(x)[0] for x in synth.prefill_inputs(w.batch, w.heads, w.seq_len, w.head_dim, w.dtype,
                                                        w.cid, dev, heads_subset=[0, 63]))
    t = timed(lambda: oracle.causal_linear_attention(q, k, v, "recurrent", nthreads=min(2, threads)))
    ht = 2 * w.seq_len / t
    out["long_1m"] = {"sample": "heads 0 and 63 at full length (2 units on 2 cores)",
                      "threads": min(2, threads), "seconds": t, "head_tokens_per_s": ht,
                      "extrapolated_tokens_per_s_all_heads": ht / w.heads * min(threads, w.heads) / 2,
                      "extrapolation": f"EXTRAPOLATED, not measured: head-token rate of the 2 measured "
                                       f"units x {min(threads, w.heads)} / 2 cores (all {w.heads} heads "
                                       f"as independent units on {min(threads, w.heads)} threads), "
                                       f"/ {w.heads} heads per token"}
    del q, k, v
    log(json.dumps({"cpu long_1m": out["long_1m"]}))

    # the packed workloads in full, in groups of 8 heads (host memory)
    for name in ("varlen16", "varlen_short"):
        w = synth.WORKLOADS[name]
        lengths = synth.varlen_lengths(w.batch, w.len_seed, w.len_lo, w.len_hi)
        tot = 0.0
        T = int(synth.cu_from_lengths(lengths)[-1])
        for h0 in range(0, w.heads, 8):
            hs = list(range(h0, min(w.heads, h0 + 8)))
            q, k, v, cu = synth.varlen_inputs(lengths, w.heads, w.head_dim, w.dtype, w.cid, dev,
                                              heads_subset=hs)
            q, k, v = f32(q), f32(k), f32(v)
            tot += timed(lambda: oracle.causal_linear_attention_varlen(q, k, v, cu, "recurrent",
                                                                       nthreads=threads))
            del q, k, v
        out[name] = {"sample": f"whole workload ({T} tokens x {w.heads} heads, 8 heads per call)",
                     "threads": threads, "seconds": tot, "tokens_per_s": T / tot}
        log(json.dumps({f"cpu {name}": out[name]}))

    # decode: every state, all steps
    w = synth.WORKLOADS["decode256"]
    S0 = synth.decode_state(w.batch, w.heads, w.head_dim, w.cid, dev).cpu().numpy()
    units = w.batch * w.heads
    qs, ks, vs = [], [], []
    for t_ in range(w.steps):
        a, b, c = synth.decode_step_inputs(w.batch, w.heads, w.head_dim, w.dtype, w.cid, t_, dev)
        qs.append(f32(a).reshape(units, -1)); ks.append(f32(b).reshape(units, -1))
        vs.append(f32(c).reshape(units, -1))
    Q, K, V = np.stack(qs), np.stack(ks), np.stack(vs)
    del qs, ks, vs
    t = timed(lambda: oracle.decode(Q, K, V, S0.reshape(units, w.head_dim, w.head_dim), nthreads=threads))
    d = w.head_dim
    out["decode256"] = {"sample": f"whole workload ({units} states x {w.steps} steps)", "threads": threads,
                        "seconds": t, "ms_per_step": t * 1e3 / w.steps,
                        "gbs_algorithmic": units * w.steps * (8 * d * d + 8 * d) / t / 1e9}
    log(json.dumps({"cpu decode256": out["decode256"]}))
    del Q, K, V, S0
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU's clocks take tens of milliseconds of sustained load to settle:
    # with a few warm-up steps the first timed steps run measurably slower
    # (about 7% on the MiniMax layer), so the default warm-up is 100 steps
    # (about 45 ms) before 50 timed ones.
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-extras", action="store_true", help="only the headline prefill workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode workload (one line with its figures; for profiling)")
    ap.add_argument("--rope-only", action="store_true",
                    help="only the rotary leg (the MiniMax layer through lightning_attn_fwd_rope, timed "
                         "alternately with the plain call; one line with its figures; for profiling)")
    ap.add_argument("--state-only", action="store_true",
                    help="only the state-handoff leg (the MiniMax layer through lightning_attn_fwd_state, "
                         "timed alternately with the plain call; one line with its figures; for profiling)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--workload", default="minimax_layer",
                    choices=["minimax_layer", "long_1m", "tiny_f32", "minimax_layer_f32", "layer_f32_d64",
                             "varlen16", "varlen_short"],
                    help="dense prefill workload of the headline line")
    ap.add_argument("--calibrate-only", action="store_true",
                    help="only the plain 1 GiB device copy (for the byte-counter calibration)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also time a plain 1 GiB device copy (the reference kernel for the "
                         "HBM byte counters) and report its GB/s")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads shard with no communication). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_attention_attn_amd as la
    import synth

    la.load_library()
    dev = torch.device("cuda:0")
    if args.calibrate_only:
        # the plain device copy alone (the reference kernel for the HBM byte
        # counters), in a process of its own
        print(json.dumps({"copy_calibration": copy_calibration(dev)}), flush=True)
        return
    if args.decode_only:
        wd = synth.WORKLOADS["decode256"]
        dms, dgbs, dtok = bench_decode(wd, 1, dev)
        print(json.dumps({"decode": {"workload": wd.note, "ms_per_step": dms, "gbs": dgbs,
                                     "hbm_frac": dgbs / PEAK_HBM_GBS, "head_steps_per_s": dtok}}),
              flush=True)
        return
    if args.state_only:
        w = synth.WORKLOADS["minimax_layer"]
        sms, pms = bench_prefill_state(w, args.steps, args.warmup, dev)
        print(json.dumps({"state_handoff": {"workload": w.note, "ms_per_step": sms,
                                            "ms_per_step_plain_same_timing": pms,
                                            "overhead_vs_plain": sms / pms - 1.0}}), flush=True)
        return
    if args.rope_only:
        w = synth.WORKLOADS["minimax_layer"]
        rms, pms = bench_prefill_state(w, args.steps, args.warmup, dev, rope=True)
        print(json.dumps({"rope": {"workload": w.note, "ms_per_step": rms,
                                   "ms_per_step_plain_same_timing": pms,
                                   "overhead_vs_plain": rms / pms - 1.0}}), flush=True)
        return
    w = synth.WORKLOADS[args.workload]
    if w.kind == "varlen":
        # one packed workload on its own (for profiling runs): one line with its figures
        vms, vstage, vchunk, vT = bench_prefill_varlen(w, args.steps, args.warmup, dev)
        vbytes = w.heads * vT * 4 * w.head_dim * 2
        print(json.dumps({w.name: {"workload": w.note, "tokens": vT, "ms_per_step": vms,
                                   "hbm_gbs": vbytes / (vms * 1e-3) / 1e9,
                                   "roofline_frac": vbytes / (PEAK_HBM_GBS * 1e9) / (vms * 1e-3),
                                   "kernels_ms": vstage, "chunk_tokens": vchunk}}), flush=True)
        return
    d, B = w.head_dim, w.block_size
    head_tokens = w.batch * w.heads * w.seq_len
    tokens = w.batch * w.seq_len

    log(f"prefill {w.name}: {w.note}")
    ms, stage, chunk, wsb = bench_prefill(w, args.steps, args.warmup, dev)
    t = ms * 1e-3
    flops = head_tokens * prefill_flops_per_head_token(d, B)
    flops_dense = head_tokens * (4 * d * d + 4 * d * B)
    alg_bytes = head_tokens * 4 * d * (2 if w.dtype == "bf16" else 4)
    tflops = flops / t / 1e12
    fused_ms = stage["fused"]
    fused_gbs = alg_bytes / (fused_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": tokens / t,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic: q,k,v ~ N(0,1), q and k scaled by 1/sqrt(d), rounded to bf16",
        "config": {"workload": f"{w.name} ({w.note})", "batch": w.batch, "heads": w.heads,
                   "seq_len": w.seq_len, "head_dim": d, "block_size": B,
                   "chunk_tokens": chunk, "parallelism": "single GPU"},
        "tflops": tflops,
        "mfma_frac": tflops / PEAK_BF16_TFLOPS,
        "tflops_dense_executed": flops_dense / t / 1e12,
        "hbm_gbs_step": alg_bytes / t / 1e9,
        "roofline_frac_step": max(flops / (PEAK_BF16_TFLOPS * 1e12), alg_bytes / (PEAK_HBM_GBS * 1e9)) / t,
        "kernels_ms": stage,
        "workspace_bytes": wsb,
        "roofline": {"bound": "hbm", "kernel": "k_fused (intra-block Q K^T, P V and Q S)",
                     "achieved": fused_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": fused_gbs / PEAK_HBM_GBS, "traffic": profiled_traffic(w.name)},
    }
    log(json.dumps({k: out[k] for k in ("value", "ms_per_step", "tflops", "kernels_ms")}))

    if not args.no_extras:
        for tname, tsteps, twarm in (("tiny_f32", 200, 50), ("minimax_layer_f32", 10, 5),
                                     ("layer_f32_d64", 20, 10)):
            wt = synth.WORKLOADS[tname]
            log(f"prefill {wt.name}: {wt.note}")
            tms, tstage, tchunk, _ = bench_prefill(wt, tsteps, twarm, dev)
            tht = wt.batch * wt.heads * wt.seq_len
            tbytes = tht * 4 * wt.head_dim * 4
            tfl = tht * prefill_flops_per_head_token(wt.head_dim, wt.block_size)
            fused_s = tstage["fused"] * 1e-3
            out[tname] = {"workload": wt.note, "ms_per_step": tms,
                          "tokens_per_s": wt.batch * wt.seq_len / (tms * 1e-3),
                          "hbm_gbs": tbytes / (tms * 1e-3) / 1e9,
                          "tflops": tfl / (tms * 1e-3) / 1e12,
                          "kernels_ms": tstage, "chunk_tokens": tchunk,
                          "fused_hbm_frac": tbytes / fused_s / 1e9 / PEAK_HBM_GBS,
                          "fused_fp32_mfma_frac": tfl / fused_s / 1e12 / PEAK_FP32_TFLOPS,
                          "roofline_frac_step": max(tfl / (PEAK_FP32_TFLOPS * 1e12),
                                                    tbytes / (PEAK_HBM_GBS * 1e9)) / (tms * 1e-3)}
            if tname == "tiny_f32":
                out[tname]["note"] = ("correctness-size case: 2 MB of traffic (0.26 us at 8 TB/s), bound by "
                                      "kernel launch latency")
            log(json.dumps(out[tname]))
        wd = synth.WORKLOADS["decode256"]
        log(f"decode {wd.name}: {wd.note}")
        dms, dgbs, dtok = bench_decode(wd, 5, dev)
        out["decode"] = {"workload": wd.note, "ms_per_step": dms, "gbs": dgbs,
                         "hbm_frac": dgbs / PEAK_HBM_GBS, "head_steps_per_s": dtok}
        log(json.dumps(out["decode"]))
        out["decode_indexed"] = bench_decode_indexed(wd, 5, dev)
        out["decode_indexed"]["workload"] = (f"{wd.note}; states in a pool of {2 * wd.batch} x {wd.heads}, "
                                             "rows on shuffled slots; 'padded' adds 64 padding rows")
        log(json.dumps(out["decode_indexed"]))
        sms, pms = bench_prefill_state(w, args.steps, args.warmup, dev)
        out["state_handoff"] = {
            "workload": f"{w.name} through lightning_attn_fwd_state: every sequence starts from a "
                        "state and returns its final state (in place)",
            "ms_per_step": sms, "tokens_per_s": tokens / (sms * 1e-3),
            "ms_per_step_plain_same_timing": pms,
            "state_bytes": w.batch * w.heads * 2 * 4 * d * d,
            "overhead_vs_plain": sms / pms - 1.0}
        log(json.dumps(out["state_handoff"]))
        rms, pms = bench_prefill_state(w, args.steps, args.warmup, dev, rope=True)
        out["rope"] = {
            "workload": f"{w.name} through lightning_attn_fwd_rope: q and k rotated on the first "
                        "64 of 128 dims (base 10,000) inside the kernels",
            "ms_per_step": rms, "tokens_per_s": tokens / (rms * 1e-3),
            "ms_per_step_plain_same_timing": pms,
            "overhead_vs_plain": rms / pms - 1.0}
        log(json.dumps(out["rope"]))
        wl = synth.WORKLOADS["long_1m"]
        log(f"prefill {wl.name}: {wl.note}")
        lms, lstage, lchunk, _ = bench_prefill(wl, 5, 3, dev)
        lht = wl.batch * wl.heads * wl.seq_len
        lbytes = lht * 4 * wl.head_dim * 2
        out["long_1m"] = {"workload": wl.note, "ms_per_step": lms,
                          "tokens_per_s": wl.seq_len / (lms * 1e-3),
                          "tflops": lht * prefill_flops_per_head_token(wl.head_dim, wl.block_size)
                          / (lms * 1e-3) / 1e12,
                          "hbm_gbs": lbytes / (lms * 1e-3) / 1e9,
                          "roofline_frac": lbytes / (PEAK_HBM_GBS * 1e9) / (lms * 1e-3),
                          "kernels_ms": lstage, "chunk_tokens": lchunk}
        out["long_1m"]["mfma_frac"] = out["long_1m"]["tflops"] / PEAK_BF16_TFLOPS
        log(json.dumps(out["long_1m"]))
        for vname, vsteps in (("varlen16", 10), ("varlen_short", 50)):
            wv = synth.WORKLOADS[vname]
            log(f"prefill {wv.name}: {wv.note}")
            vms, vstage, vchunk, vT = bench_prefill_varlen(wv, vsteps, 5, dev)
            vht = wv.heads * vT
            vbytes = vht * 4 * wv.head_dim * 2
            out[vname] = {"workload": f"{wv.note}, H{wv.heads} d{wv.head_dim}, block {wv.block_size}, "
                                      f"{vT} tokens",
                          "ms_per_step": vms, "tokens_per_s": vT / (vms * 1e-3),
                          "tflops": vht * prefill_flops_per_head_token(wv.head_dim, wv.block_size)
                          / (vms * 1e-3) / 1e12,
                          "hbm_gbs": vbytes / (vms * 1e-3) / 1e9,
                          "roofline_frac": vbytes / (PEAK_HBM_GBS * 1e9) / (vms * 1e-3),
                          "kernels_ms": vstage, "chunk_tokens": vchunk}
            log(json.dumps(out[vname]))

    if args.copy_calibration:
        out["copy_calibration"] = copy_calibration(dev)
        log(json.dumps(out["copy_calibration"]))

    if not args.no_cpu:
        info = cpu_info()
        log("cpu baseline (oracle)", json.dumps(info))
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, info)
        log(json.dumps(out["cpu_baseline"]))
        if not args.no_extras:
            out["cpu_baseline_per_workload"] = cpu_baseline_configs(dev, info)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
