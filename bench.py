#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

Headline (the JSON `value`): decode KV-read bandwidth of the GQA split-KV
decode workload -- batch 32, 64 query heads over 8 KV heads, T = 1,
s_k = 8192, hd = 128, 64 partitions of 128 keys merged by LSE.  One step is
fmha_decode_splitkv followed by fmha_lse_merge on the same stream, with all
inputs resident in HBM.  The 1 GiB of K/V is four times the Infinity Cache,
so every step streams it from HBM.

Also reported on the same line:
  repeats       the timed region measured five more times (median beside
                the contract's single region).
  roofline      the split kernel (the dominant one; its name is the one the
                library's plan query gives): algorithmic bytes per launch /
                its duration, the median of five timings of K back-to-back
                launches with nothing between them, against 8 TB/s.
  cpu_baseline  the fp64 CPU oracle on the host cores, a baseline only: the
                same decode workload (split + merge) as KV-read GB/s, plus
                four fused workloads, each with one thread and with the
                host's share of threads; core count and CPU model recorded.
  ragged_decode the same decode shapes with per-row key counts uniform on
                1..8192 (split + merge), as GB/s of the K/V actually read.
  sharded_decode_one_gpu_share
                one GPU's share of the decode workload sharded over 8 GPUs
                by KV head or by sequence, at its real shape (cold).
  mx_output     the largest causal prefill point with MX-coded output
                (FP8 E4M3 and FP4 E2M1 with E8M0 block scales).
  attainable    what this GPU sustains: a 2 GiB streaming read (plain and
                non-temporal loads) and a bf16 MFMA loop; `roofline` and the
                prefill lines also give their fraction of these.
  prefill       the largest causal MHA prefill point, the sliding-window
                MQA prefill and a long causal GQA prefill (T = s_k = 4096):
                fused-kernel TFLOP/s (algorithmic flops) against the dense
                bf16 MFMA peak and against the roofline (bandwidth for the
                first two, MFMA for the long one), timed from graph replays
                over input replicas rotated through more than the Infinity
                Cache.

Separately, `--grid PATH` times every point of the decode and prefill grids
(cold and hot, with the launch floor of an empty kernel) and writes them to
PATH.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--grid PATH]
"""
import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2516.6    # 256 CU x 2.4 GHz x 4096 flop/clk, dense bf16
METRIC = "decode KV-read GB/s + prefill attn TFLOP/s (bf16), % of MI355X roofline"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    """sha256 over the HIP sources: ties counter results to the code they measured."""
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(ROOT, "head_attention_fmha_amd", "csrc", "*"))):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel_tag):
    """HBM bytes per launch from the committed counter summary, or None when the
    summary is missing or was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_tag}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def decode_bytes(w):
    kv = 4 * w.batch * w.n_kv_h * w.s_k * w.hd               # K + V, bf16
    q = 2 * w.batch * w.T * w.n_h * w.hd
    part_o = 4 * w.batch * w.n_h * w.T * w.n_split * w.hd
    part_l = 4 * w.batch * w.n_h * w.T * w.n_split
    o = 2 * w.batch * w.T * w.n_h * w.hd
    lse = 4 * w.batch * w.n_h * w.T
    split_kernel = kv + q + part_o + part_l                     # reads K, V, Q; writes partials
    merge_kernel = part_o + part_l + o + lse                    # reads partials; writes O, lse
    return kv, split_kernel, merge_kernel


def forward_work(w):
    """Algorithmic (flops, total bytes, K+V bytes) of one fused call: masked
    keys are not work, and K/V bytes count the union of the keys any query
    sees (each read once)."""
    pairs = 0
    union_lo, union_hi = w.s_k, 0
    for i in range(w.T):
        pos = w.s_k - w.T + i
        hi = min(w.s_k, pos + 1) if w.causal else w.s_k
        lo = max(0, pos - w.window + 1) if w.window else 0
        pairs += max(0, hi - lo)
        union_lo, union_hi = min(union_lo, lo), max(union_hi, hi)
    flops = 4.0 * w.hd * w.batch * w.n_h * pairs
    u = max(0, union_hi - union_lo)
    kv = 4 * w.batch * w.n_kv_h * u * w.hd
    byts = 2 * 2 * w.batch * w.T * w.n_h * w.hd + 4 * w.batch * w.n_h * w.T + kv
    return flops, byts, kv


def prefill_work(w):
    """Algorithmic (flops, bytes) of one fused call."""
    flops, byts, _ = forward_work(w)
    return flops, byts


def run_decode(args, torch, fa, I):
    w = I.GQA_SPLITKV_DECODE
    dev = torch.device("cuda:0")
    log(f"decode workload {w.name}: drawing inputs on the device")
    q, k, v = I.make_qkv(w, device="cuda")
    o_part = torch.empty((w.batch, w.n_h, w.T, w.n_split, w.hd), dtype=torch.float32, device=dev)
    lse_part = torch.empty((w.batch, w.n_h, w.T, w.n_split), dtype=torch.float32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.batch, w.n_h, w.T), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def split():
        fa.fmha_decode_splitkv(q, k, v, o_part, lse_part, split_len=w.split_len, scale=w.scale, stream=stream)

    def merge():
        fa.fmha_lse_merge(o_part, lse_part, o, lse, stream=stream)

    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def timed_steps(fn, n):
        """ms per call of n back-to-back calls of fn, between two events on the
        launch stream (nothing else in between)."""
        a, b = E(), E()
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    def step():
        split()
        merge()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed steps: nothing but the two launches between the two events
    ms_per_step = timed_steps(step, args.steps)
    # the same measurement repeated five more times (reported beside it)
    repeats = [timed_steps(step, args.steps) for _ in range(5)]
    # the split kernel alone, back to back without instrumentation between its
    # launches: its duration for the roofline (each launch streams the whole
    # 1 GiB of K/V and writes the partials, as in the step)
    split_reps = [timed_steps(split, args.steps) for _ in range(5)]
    split_ms = sorted(split_reps)[len(split_reps) // 2]
    merge_ms = max(1e-6, sorted(repeats)[len(repeats) // 2] - split_ms)
    kv_bytes, split_bytes, merge_bytes = decode_bytes(w)
    log(f"decode: {ms_per_step * 1e3:.1f} us/step (repeats {', '.join(f'{r * 1e3:.1f}' for r in repeats)}); "
        f"split alone {split_ms * 1e3:.1f} us, merge + launch gap {merge_ms * 1e3:.1f} us")
    res = {
        "w": w, "ms_per_step": ms_per_step, "repeats_ms": repeats, "split_ms": split_ms, "merge_ms": merge_ms,
        "split_reps_ms": split_reps,
        "value": kv_bytes / (ms_per_step * 1e-3) / 1e9,
        "split_gbs": split_bytes / (split_ms * 1e-3) / 1e9,
        "merge_gbs": merge_bytes / (merge_ms * 1e-3) / 1e9,
        "split_bytes": split_bytes, "kv_bytes": kv_bytes,
        "plan": fa.fmha_attention_plan(w.batch, w.n_h, w.n_kv_h, w.T, w.s_k, w.hd, split_len=w.split_len),
    }
    return res


def run_ragged_decode(args, torch, fa, I):
    """Ragged split-KV decode: per-row key counts uniform on 1..8192."""
    w = I.RAGGED_DECODE
    q, k, v = I.make_qkv(w, device="cuda")
    lens = I.ragged_lengths(w.batch, w.s_k)
    seqlens = lens.to("cuda")
    o_part = torch.empty((w.batch, w.n_h, w.T, w.n_split, w.hd), dtype=torch.float32, device="cuda")
    lse_part = torch.empty((w.batch, w.n_h, w.T, w.n_split), dtype=torch.float32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((w.batch, w.n_h, w.T), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        fa.fmha_decode_splitkv_segment(q, k, v, o_part, lse_part, split_len=w.split_len, part_offset=0,
                                       seqlens_k=seqlens, scale=w.scale, stream=stream)
        fa.fmha_lse_merge(o_part, lse_part, o, lse, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / args.steps
    kv_bytes = 4 * int(lens.sum()) * w.n_kv_h * w.hd
    log(f"ragged decode {w.name}: {us:.1f} us/step, {kv_bytes / (us * 1e-6) / 1e9:.0f} GB/s of K/V")
    return {"workload": w.name, "us_per_step": round(us, 2), "kv_gbs": round(kv_bytes / (us * 1e-6) / 1e9, 1),
            "kv_bytes": kv_bytes, "mean_len": round(float(lens.float().mean()), 1),
            "step": "fmha_decode_splitkv_segment (per-row lengths) + fmha_lse_merge"}


SPLIT_DECODE_LEN = 128  # keys per partition when the grid times MQA decode as split-KV + merge
WARM_MS = 30.0  # GPU time replayed before timing: clocks settle under sustained load


def run_shards(torch, fa, I):
    """One GPU's share of the GQA split-KV decode workload sharded over
    I.SHARDS GPUs, at its real shape.  Each share holds 128 MiB of K/V, which
    the Infinity Cache would keep, so K/V replicas are rotated through at
    least 512 MiB (graph-timed, cold).
      by KV head: b32, 8 query heads over one KV head, 8192 keys; split into
        64 partitions of 128 + LSE merge (nothing to exchange);
      by sequence: b32, h64/kv8, 1024 keys; its 8 partitions go to slots
        0..7 of the 64-slot fp32 partial buffer (the other GPUs fill the
        rest); after the exchange, the owner of 8 query heads merges their 64
        slots.  The exchange itself (fp32 partials over xGMI) is not timed."""
    out = []
    for w in (I.HEAD_SHARD_DECODE, I.SEQ_SHARD_DECODE):
        seq = w is I.SEQ_SHARD_DECODE
        n_total = w.n_split * (I.SHARDS if seq else 1)
        q, k, v = I.make_qkv(w, device="cuda")
        kv = 4 * w.batch * w.n_kv_h * w.s_k * w.hd
        reps = max(1, math.ceil(512 * 2**20 / kv))
        ins = [(q, k, v) if r == 0 else (q.clone(), k.clone(), v.clone()) for r in range(reps)]
        o_part = torch.empty((w.batch, w.n_h, 1, n_total, w.hd), dtype=torch.float32, device="cuda")
        lse_part = torch.empty((w.batch, w.n_h, 1, n_total), dtype=torch.float32, device="cuda")
        o = torch.empty_like(q)
        lse = torch.empty((w.batch, w.n_h, 1), dtype=torch.float32, device="cuda")

        def mk(x):
            def step():
                st = torch.cuda.current_stream()
                if seq:
                    fa.fmha_decode_splitkv_segment(x[0], x[1], x[2], o_part, lse_part, split_len=w.split_len,
                                                   part_offset=0, scale=w.scale, stream=st)
                else:
                    fa.fmha_decode_splitkv(x[0], x[1], x[2], o_part, lse_part, split_len=w.split_len, scale=w.scale,
                                           stream=st)
                    fa.fmha_lse_merge(o_part, lse_part, o, lse, stream=st)
            return step
        us = rotated_time_us(torch, [mk(x) for x in ins])
        line = {"workload": w.name, "us_per_step": round(us, 2), "kv_gbs": round(kv / (us * 1e-6) / 1e9, 1),
                "frac_of_hbm_peak": round(kv / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "rotated_replicas": reps}
        if seq:
            # after the exchange: 8 query heads x 64 slots per batch row
            heads = w.n_h // I.SHARDS
            op_own = torch.zeros((w.batch, heads, 1, n_total, w.hd), dtype=torch.float32, device="cuda")
            lp_own = torch.zeros((w.batch, heads, 1, n_total), dtype=torch.float32, device="cuda")
            o_own = torch.empty((w.batch, 1, heads, w.hd), dtype=torch.bfloat16, device="cuda")
            m_us = rotated_time_us(torch, [lambda: fa.fmha_lse_merge(op_own, lp_own, o_own, None,
                                                                      stream=torch.cuda.current_stream())])
            sent = w.batch * w.n_h * w.n_split * (w.hd + 1) * 4 * (I.SHARDS - 1) // I.SHARDS
            line.update({"step": f"fmha_decode_splitkv_segment: {w.n_split} partitions into slots 0..{w.n_split - 1} "
                                 f"of {n_total}", "merge_after_exchange_us": round(m_us, 2),
                         "exchange_bytes_per_gpu": sent})
        else:
            line["step"] = "fmha_decode_splitkv + fmha_lse_merge"
        log(f"shard {w.name}: {us:.2f} us/step, {line['kv_gbs']:.0f} GB/s of K/V"
            + (f", merge after exchange {line['merge_after_exchange_us']:.2f} us" if seq else ""))
        out.append(line)
        del ins, q, k, v, o_part, lse_part
        torch.cuda.empty_cache()
    return out


def graph_time_us(torch, calls, reps):
    """Capture `calls` (one launch each) into one graph, replay it for about
    WARM_MS untimed, then return the mean us per call over `reps` replays."""
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for c in calls:  # warm, outside capture
            c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in calls:
            c()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    g.replay()
    e.record()
    torch.cuda.synchronize()
    for _ in range(max(1, math.ceil(WARM_MS / max(s.elapsed_time(e), 1e-3)))):
        g.replay()
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) * 1e3 / (reps * len(calls))


def rotated_time_us(torch, calls):
    """Mean us per call over the given calls (one per input replica), captured
    at least 32 to a graph -- a graph replay has a fixed cost of its own -- and
    replayed for about 200 calls in all."""
    per_graph = calls * max(1, 32 // len(calls))
    return graph_time_us(torch, per_graph, reps=max(3, 200 // len(per_graph)))


def run_prefill(torch, fa, I):
    out = []
    for w in (I.mha_causal_prefill(128, 512, 512), I.SWA_MQA_PREFILL, I.LONG_PREFILL):
        flops, byts = prefill_work(w)
        foot = 2 * (w.batch * w.T * w.n_h * w.hd * 2) + 2 * (w.batch * w.s_k * w.n_kv_h * w.hd * 2)
        reps = max(1, min(64, math.ceil(512 * 2**20 / foot)))  # rotate >= 512 MiB
        q, k, v = I.make_qkv(w, device="cuda")
        bufs = []
        for r in range(reps):
            qr, kr, vr = (q, k, v) if r == 0 else (q.clone(), k.clone(), v.clone())
            bufs.append((qr, kr, vr, torch.empty_like(qr),
                         torch.empty((w.batch, w.n_h, w.T), dtype=torch.float32, device="cuda")))

        def mk(bf):
            return lambda: fa.fmha_forward(bf[0], bf[1], bf[2], bf[3], bf[4], scale=w.scale,
                                           window=w.window, causal=w.causal,
                                           stream=torch.cuda.current_stream())
        us = rotated_time_us(torch, [mk(bf) for bf in bufs])
        t_roof_us = max(byts / (HBM_PEAK_GBS * 1e9), flops / (MFMA_BF16_PEAK_TFS * 1e12)) * 1e6
        tfs = flops / (us * 1e-6) / 1e12
        plan = fa.fmha_attention_plan(w.batch, w.n_h, w.n_kv_h, w.T, w.s_k, w.hd, window=w.window,
                                      causal=w.causal)
        out.append({"workload": w.name, "us_per_call": round(us, 2), "tflops": round(tfs, 1),
                    "plan": plan,
                    "frac_of_mfma_peak": round(tfs / MFMA_BF16_PEAK_TFS, 4),
                    "frac_of_roofline": round(t_roof_us / us, 4),
                    "roofline_bound": "hbm" if byts / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_BF16_PEAK_TFS * 1e12)
                    else "mfma",
                    "alg_gflop": round(flops / 1e9, 3), "alg_mib": round(byts / 2**20, 2),
                    "rotated_replicas": reps})
        log(f"prefill {w.name}: {us:.2f} us, {tfs:.1f} TFLOP/s, {t_roof_us / us:.1%} of roofline")
        del bufs, q, k, v
        torch.cuda.empty_cache()
    return out


def run_grid(torch, fa, I, path):
    """Every point of the single-head decode, the MQA decode grid, the causal
    MHA prefill grid and the sliding-window MQA prefill, one fmha_forward call
    each, timed from graph replays: cold (input replicas rotated through at
    least 512 MiB, twice the Infinity Cache; the single-head decode point is
    32 KiB and is timed hot only, as latency) and hot (one input set).  The
    launch floor is an empty kernel timed the same way; a point whose
    roofline time is below five floors is flagged launch-bound.  Writes the
    table to `path` as JSON."""
    from head_attention_fmha_amd import peaks
    floor_us = graph_time_us(torch, [lambda: peaks.empty(1, torch.cuda.current_stream())] * 64, reps=50)
    log(f"grid: launch floor (empty kernel) {floor_us:.2f} us")
    points = []
    for w in [I.SINGLE_HEAD_DECODE] + I.MQA_DECODE_GRID + I.MHA_PREFILL_GRID + [I.SWA_MQA_PREFILL]:
        flops, byts, kv = forward_work(w)
        foot = 2 * (w.batch * w.T * w.n_h * w.hd * 2) + 2 * (w.batch * w.s_k * w.n_kv_h * w.hd * 2)
        cold = w is not I.SINGLE_HEAD_DECODE
        reps = max(1, min(64, math.ceil(512 * 2**20 / foot))) if cold else 1
        q, k, v = I.make_qkv(w, device="cuda")
        bufs = []
        for r in range(reps):
            qr, kr, vr = (q, k, v) if r == 0 else (q.clone(), k.clone(), v.clone())
            bufs.append((qr, kr, vr, torch.empty_like(qr),
                         torch.empty((w.batch, w.n_h, w.T), dtype=torch.float32, device="cuda")))

        def mk(bf):
            return lambda: fa.fmha_forward(bf[0], bf[1], bf[2], bf[3], bf[4], scale=w.scale,
                                           window=w.window, causal=w.causal,
                                           stream=torch.cuda.current_stream())
        hot_us = rotated_time_us(torch, [mk(bufs[0])])
        us = rotated_time_us(torch, [mk(bf) for bf in bufs]) if cold else hot_us
        t_roof_us = max(byts / (HBM_PEAK_GBS * 1e9), flops / (MFMA_BF16_PEAK_TFS * 1e12)) * 1e6
        tfs = flops / (us * 1e-6) / 1e12
        # MQA decode also as split-KV into 128-key partitions + LSE merge: its
        # fused call has only 64 workgroups (8 batch rows x 8 tiles of the 128
        # stacked query heads), the split spreads the keys over more
        split_us = None
        if w.n_kv_h == 1 and w.T == 1 and w.s_k > SPLIT_DECODE_LEN:
            ns = fa.n_split_for(w.s_k, SPLIT_DECODE_LEN)
            o_part = torch.empty((w.batch, w.n_h, 1, ns, w.hd), dtype=torch.float32, device="cuda")
            lse_part = torch.empty((w.batch, w.n_h, 1, ns), dtype=torch.float32, device="cuda")

            def mk_split(bf):
                def step():
                    st = torch.cuda.current_stream()
                    fa.fmha_decode_splitkv(bf[0], bf[1], bf[2], o_part, lse_part, split_len=SPLIT_DECODE_LEN,
                                           scale=w.scale, stream=st)
                    fa.fmha_lse_merge(o_part, lse_part, bf[3], bf[4], stream=st)
                return step
            split_us = rotated_time_us(torch, [mk_split(bf) for bf in bufs])
            del o_part, lse_part
        # the one-call workspace entry: few-unit points split over the keys
        # into partitions of at most 128 keys and merged (two launches)
        ws_us = None
        ws_bytes = fa.fmha_forward_ws_size(w.batch, w.n_h, w.n_kv_h, w.T, w.s_k, w.hd, window=w.window,
                                           causal=w.causal)
        if ws_bytes:
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")

            def mk_ws(bf):
                return lambda: fa.fmha_forward_ws(bf[0], bf[1], bf[2], bf[3], bf[4], ws, scale=w.scale,
                                                  window=w.window, causal=w.causal,
                                                  stream=torch.cuda.current_stream())
            ws_us = rotated_time_us(torch, [mk_ws(bf) for bf in bufs]) if cold else \
                rotated_time_us(torch, [mk_ws(bufs[0])])
            del ws
        plan = fa.fmha_attention_plan(w.batch, w.n_h, w.n_kv_h, w.T, w.s_k, w.hd, window=w.window, causal=w.causal)
        pt = {"workload": w.name, "T": w.T, "s_k": w.s_k, "hd": w.hd, "us": round(us, 2), "hot_us": round(hot_us, 2),
              "cold": cold, "kv_gbs": round(kv / (us * 1e-6) / 1e9, 1),
              "total_gbs": round(byts / (us * 1e-6) / 1e9, 1), "tflops": round(tfs, 2),
              "t_roof_us": round(t_roof_us, 3), "frac_of_roofline": round(t_roof_us / us, 4),
              "frac_of_hbm_peak": round(byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
              "frac_of_mfma_peak": round(tfs / MFMA_BF16_PEAK_TFS, 4),
              "launch_bound": t_roof_us < 5 * floor_us, "replicas": reps,
              "workgroups": plan["workgroups"], "row_parallel": plan["row_parallel"]}
        if split_us is not None:
            pt.update({"split_merge_us": round(split_us, 2), "split_len": SPLIT_DECODE_LEN,
                       "split_merge_frac_of_roofline": round(t_roof_us / split_us, 4)})
        pt["kernel"] = plan["kernel"]
        if ws_us is not None:
            pt.update({"ws_us": round(ws_us, 2), "ws_frac_of_roofline": round(t_roof_us / ws_us, 4),
                       "ws_bytes": ws_bytes})
        points.append(pt)
        log(f"grid {w.name}: {us:.2f} us (hot {hot_us:.2f}), {pt['kv_gbs']:.0f} GB/s K+V, "
            f"{pt['total_gbs']:.0f} GB/s total, {tfs:.1f} TFLOP/s, {t_roof_us / us:.1%} of roofline"
            f"{' (launch-bound)' if pt['launch_bound'] else ''}"
            f"{f'; split-KV + merge {split_us:.2f} us' if split_us is not None else ''}"
            f"{f'; fmha_forward_ws {ws_us:.2f} us' if ws_us is not None else ''}")
        del bufs, q, k, v
        torch.cuda.empty_cache()
    with open(path, "w") as f:
        json.dump({"launch_floor_us": round(floor_us, 3), "hbm_peak_gbs": HBM_PEAK_GBS,
                   "mfma_bf16_peak_tflops": MFMA_BF16_PEAK_TFS, "points": points}, f, indent=1)
    log(f"grid: {len(points)} points written to {path}")


def run_small(torch, fa, I, calls=20):
    """The few-unit workloads, each called `calls` times back to back (for
    profiler runs; nothing is reported): the MQA decode at hd 128 and 512
    over 128 and 512 keys through fmha_forward and fmha_forward_ws, and the
    sliding-window MQA prefill."""
    for w in (I.mqa_decode(128, 128), I.mqa_decode(128, 512), I.mqa_decode(512, 128), I.mqa_decode(512, 512),
              I.SWA_MQA_PREFILL):
        q, k, v = I.make_qkv(w, device="cuda")
        o = torch.empty_like(q)
        lse = torch.empty((w.batch, w.n_h, w.T), dtype=torch.float32, device="cuda")
        ws = fa.workspace_for(q, k, window=w.window, causal=w.causal)
        for _ in range(calls):
            fa.fmha_forward(q, k, v, o, lse, scale=w.scale, window=w.window, causal=w.causal)
        if ws is not None:
            for _ in range(calls):
                fa.fmha_forward_ws(q, k, v, o, lse, ws, scale=w.scale, window=w.window, causal=w.causal)
        torch.cuda.synchronize()
        log(f"small {w.name}: {calls} fmha_forward calls" + (f" + {calls} fmha_forward_ws calls" if ws is not None
                                                             else ""))
        del q, k, v, o, lse, ws


def run_mx_output(torch, fa, I):
    """The largest causal MHA prefill point with the output written as MX
    codes (FP8 E4M3, FP4 E2M1) instead of bf16, each timed like the prefill
    lines (graph replays over rotated replicas)."""
    w = I.mha_causal_prefill(128, 512, 512)
    flops, _ = prefill_work(w)
    foot = 2 * (w.batch * w.T * w.n_h * w.hd * 2) + 2 * (w.batch * w.s_k * w.n_kv_h * w.hd * 2)
    reps = max(1, min(64, math.ceil(512 * 2**20 / foot)))
    q, k, v = I.make_qkv(w, device="cuda")
    ins = [(q, k, v) if r == 0 else (q.clone(), k.clone(), v.clone()) for r in range(reps)]
    out = []
    for fmt, name in ((fa.MX_FP8_E4M3, "mxfp8_e4m3"), (fa.MX_FP4_E2M1, "mxfp4_e2m1")):
        cs, ss = fa.mx_shapes(w.batch, w.T, w.n_h, w.hd, fmt)
        bufs = [(x, torch.empty(cs, dtype=torch.uint8, device="cuda"),
                 torch.empty(ss, dtype=torch.uint8, device="cuda")) for x in ins]

        def mk(bf, fmt=fmt):
            return lambda: fa.fmha_forward_mx(bf[0][0], bf[0][1], bf[0][2], bf[1], bf[2], fmt=fmt, scale=w.scale,
                                              causal=True, stream=torch.cuda.current_stream())
        us = rotated_time_us(torch, [mk(bf) for bf in bufs])
        out.append({"workload": w.name, "format": name, "us_per_call": round(us, 2),
                    "tflops": round(flops / (us * 1e-6) / 1e12, 1)})
        log(f"mx output {name} {w.name}: {us:.2f} us")
        del bufs
    del ins, q, k, v
    torch.cuda.empty_cache()
    return out


def run_attainable(torch):
    """What this GPU sustains, for roofline fractions beside the published
    peaks: a streaming read of 2 GiB (8x the Infinity Cache) with plain and
    with non-temporal loads, and a loop of independent bf16 MFMAs."""
    from head_attention_fmha_amd import peaks
    st = torch.cuda.current_stream()

    def timed_ms(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(reps):
            fn()
        b.record(st)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    buf = torch.ones(2 * 2**30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1024 * 4, dtype=torch.float32, device="cuda")
    nbytes = buf.numel()
    plain = nbytes / (timed_ms(lambda: peaks.stream_read(buf, False, sink, st), 10) * 1e-3) / 1e9
    nt = nbytes / (timed_ms(lambda: peaks.stream_read(buf, True, sink, st), 10) * 1e-3) / 1e9
    del buf
    flops = 1024 * 4 * 4096 * 4 * 32768.0
    ms = timed_ms(lambda: peaks.mfma_bf16(1024, 4096, sink, st), 5)
    mfma = flops / (ms * 1e-3) / 1e12
    log(f"attainable: streaming read {plain:.0f} GB/s plain, {nt:.0f} GB/s non-temporal; bf16 MFMA {mfma:.0f} TFLOP/s")
    return {"hbm_read_gbs": round(plain, 1), "hbm_read_nt_gbs": round(nt, 1), "mfma_bf16_tflops": round(mfma, 1),
            "hbm_frac_of_published": round(max(plain, nt) / HBM_PEAK_GBS, 4),
            "mfma_frac_of_published": round(mfma / MFMA_BF16_PEAK_TFS, 4),
            "how": "2 GiB streaming read (16-byte loads, whole chip), plain and non-temporal; 1024 x 4 waves x "
                   "4096 rounds of 4 independent v_mfma_f32_32x32x16_bf16"}


def cpu_model():
    """The host CPU's model name (lscpu), or None."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    for ln in out.splitlines():
        if ln.startswith("Model name:"):
            return ln.split(":", 1)[1].strip()
    return None


def run_cpu_baseline(I, torch, budget_s):
    """The fp64 oracle on the host cores, as a baseline (not a target): the
    GQA split-KV decode workload (split + merge, the bench step) and the
    single-head decode, the largest MQA decode point, the largest causal MHA
    prefill point and the sliding-window prefill (one fused call each), each
    with one thread and with the host's CPU share (at most 16 threads).  Runs
    are repeated up to three times within the budget; the median is reported,
    excluding input generation.  The headline `value` is the decode step with all threads."""
    import oracle
    threads_all = oracle.default_threads()
    decode = I.GQA_SPLITKV_DECODE
    cases = [("decode", decode), ("fused", I.SINGLE_HEAD_DECODE), ("fused", I.mqa_decode(512, 512)),
             ("fused", I.SWA_MQA_PREFILL), ("fused", I.mha_causal_prefill(128, 512, 512))]
    per = []
    t_start = time.perf_counter()
    headline = None
    for kind, w in cases:
        q, k, v = I.make_qkv(w)  # seeded CPU draws (the oracle's own recipe)
        flops, byts, kvb = forward_work(w)
        for threads in (1, threads_all):
            times = []
            for _ in range(3):
                t0 = time.perf_counter()
                if kind == "decode":
                    op, lp = oracle.split(q, k, v, w.scale, w.split_len, threads=threads)
                    oracle.merge(op, lp)
                else:
                    oracle.attention(q, k, v, w.scale, causal=w.causal, window=w.window, threads=threads)
                times.append(time.perf_counter() - t0)
                if time.perf_counter() - t_start > budget_s or times[-1] > budget_s / 8:
                    break
            t = sorted(times)[len(times) // 2]
            rec = {"workload": w.name, "threads": threads, "s": round(t, 6), "runs": len(times),
                   "kv_gbs": round(kvb / t / 1e9, 4), "gflops": round(flops / t / 1e9, 3)}
            per.append(rec)
            log(f"cpu baseline {w.name}, {threads} thread(s): {t:.3f} s")
            if kind == "decode" and threads == threads_all:
                headline = rec
    return {"value": headline["kv_gbs"], "unit": "GB/s", "cores": threads_all, "kind": "oracle",
            "sample": f"{decode.name}: the whole workload (split into {decode.n_split} partitions + LSE merge, "
                      f"fp64), median of {headline['runs']} run(s) of {headline['s']:.2f} s on {threads_all} threads",
            "host_logical_cpus": os.cpu_count(), "host_cpu_model": cpu_model(),
            "threads_note": f"all-core runs use min(os.cpu_count(), 16) = {threads_all} threads, the host share of "
                            f"one GPU",
            "per_workload": per}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-ragged", action="store_true",
                    help="skip the ragged decode line (profiler runs of the headline kernel)")
    ap.add_argument("--no-shards", action="store_true",
                    help="skip the per-GPU share lines of the sharded decode (profiler runs of the headline kernel)")
    ap.add_argument("--cpu-seconds", type=float, default=40.0,
                    help="time budget of the CPU oracle baseline (all its workloads)")
    ap.add_argument("--only-small", action="store_true",
                    help="run only the few-unit workloads (MQA decode, sliding-window prefill) for profiler runs; "
                         "prints no JSON line")
    ap.add_argument("--only-prefill", action="store_true",
                    help="time only the prefill workloads (for profiler runs); prints no JSON line")
    ap.add_argument("--grid", metavar="PATH",
                    help="time every point of the decode and prefill grids, write them to PATH as JSON, "
                         "and print no JSON line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed region, copy 1 GiB twice (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the attention path "
              f"shards by batch, KV head or sequence with no cross-GPU step measured here)", file=sys.stderr)
        sys.exit(2)

    import torch
    import head_attention_fmha_amd as fa
    from head_attention_fmha_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    fa.load_library()

    def calibrate_copy():
        src = torch.empty(2**30, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.grid:
        run_grid(torch, fa, I, args.grid)
        return
    if args.only_small:
        run_small(torch, fa, I)
        return
    if args.only_prefill:
        run_prefill(torch, fa, I)
        if args.calibrate_copy:
            calibrate_copy()
        return
    # the attainable-peak probes run first: a few tens of milliseconds of
    # sustained load that also bring the GPU's clocks to the state every later
    # measurement runs in
    att = run_attainable(torch)
    res = run_decode(args, torch, fa, I)
    if args.calibrate_copy:
        calibrate_copy()
    ragged = None if args.no_ragged else run_ragged_decode(args, torch, fa, I)
    shards = None if args.no_shards else run_shards(torch, fa, I)
    prefill = None if args.no_prefill else run_prefill(torch, fa, I)
    mx_out = None if args.no_prefill else run_mx_output(torch, fa, I)
    cpu = None if args.no_cpu_baseline else run_cpu_baseline(I, torch, args.cpu_seconds)
    best_bw = max(att["hbm_read_gbs"], att["hbm_read_nt_gbs"])
    for p in prefill or []:
        t_att = max(p["alg_mib"] * 2**20 / (best_bw * 1e9), p["alg_gflop"] * 1e9 / (att["mfma_bf16_tflops"] * 1e12))
        p["frac_of_attainable_roofline"] = round(t_att * 1e6 / p["us_per_call"], 4)
    w = res["w"]
    split_us = res["split_ms"] * 1e3
    kernel = res["plan"]["kernel"]
    # counter summaries are keyed by the kernel family and the workload
    split_tag = kernel.split("<")[0] + "_hd128_split_gqa_decode"
    line = {
        "metric": METRIC,
        "value": round(res["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded device draws: Q, K ~ N(0,1), V ~ U(-1,1), bf16)",
        "config": {"workload": w.name, "batch": w.batch, "n_h": w.n_h, "n_kv_h": w.n_kv_h, "T": w.T,
                   "s_k": w.s_k, "hd": w.hd, "split_len": w.split_len, "n_split": w.n_split,
                   "step": "fmha_decode_splitkv + fmha_lse_merge",
                   "split_us": round(split_us, 2), "merge_us": round(res["merge_ms"] * 1e3, 2),
                   "merge_gbs": round(res["merge_gbs"], 1)},
        "repeats": {"ms_per_step": [round(r, 5) for r in res["repeats_ms"]],
                    "median_ms_per_step": round(sorted(res["repeats_ms"])[2], 5),
                    "how": f"the timed region ({args.steps} steps) measured five more times right after it"},
        "roofline": {"kernel": kernel, "bound": "hbm",
                     "achieved": round(res["split_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(res["split_gbs"] / HBM_PEAK_GBS, 4), "traffic": measured_traffic(split_tag),
                     "alg_bytes_per_launch": res["split_bytes"], "launch_us": round(split_us, 2),
                     "launch_us_how": f"median of 5 timings of {args.steps} back-to-back split launches "
                                      f"(no instrumentation between launches)",
                     "frac_of_attainable": round(res["split_gbs"] / best_bw, 4)},
        "attainable": att,
        "cpu_baseline": cpu,
        "prefill": prefill,
        "ragged_decode": ragged,
        "sharded_decode_one_gpu_share": shards,
        "mx_output": mx_out,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
