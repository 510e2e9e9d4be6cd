#!/usr/bin/env python3
"""Benchmark of the paged-KV attention hot path on one MI355X.

One step = one pass of the whole path over one synthetic batch: the cache
write of this step's new tokens (pkv_cache_write), then the varlen attention
forward over the paged cache (pkv_varlen_fwd: the attention kernel and, when
the KV range is split, the log-sum-exp merge kernel). Inputs are resident in
HBM before timing starts. The KV cache is replicated and the replicas are used
in turn, so a step never finds its KV in the 256 MB last-level cache.

Default run (one GPU), the two halves of the headline metric in one process:
paged decode, Llama-3-8B-like GQA (32 query / 8 kv heads, head size 128,
bf16), batch 64, one query token per request, context lengths uniform in
[512, 4096], page size 16, random block table, measured as KV bytes read per
second (GB/s) against the MI355X HBM peak of 8 TB/s; and, nested under
"prefill" in the same JSON line, chunked prefill (batch 8, new tokens uniform
in [128, 2048] on cached contexts uniform in [0, 4096], same heads, page 16,
causal) in TFLOP/s of visible query-key pairs against the 2.5 PFLOP/s bf16
dense MFMA peak. Under "also", the other workloads below (20 timed steps
each, no CPU baseline), each run as a child process.
Other workloads (--workload): chunked_prefill (TFLOP/s against the 2.5 PFLOP/s
bf16 dense MFMA peak), long_decode, long_decode_cascade, fp8_decode,
spec_decode (several new tokens per request; KV GB/s). The
attention variants can be switched on for any workload but the cascade
(--sliding-window W, --softcap C, --sinks, --alibi); bytes and flops then count only
what the window leaves visible.

Prints ONE JSON line. `value` is the whole step (cache write + attention)
replayed in a HIP graph. `roofline.achieved` is the algorithmic bytes (or
flops) per call over the attention's own time: the attention kernel plus its
merge kernel, K calls replayed back to back in a HIP graph and timed by
events around the replay (per-launch event pairs in an eager pass, also
reported, add the dispatch latency to every kernel). The float64 CPU oracle
is timed on the same workload (rank 0, one GPU only) as a reported baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
# fp8-q prefill: Q K^T on the fp8 matrix cores, P V on the bf16 ones, equal
# flops each, so the time at peak is F/2 / 5.0 + F/2 / 2.5 PFLOP/s
FP8_QK_BF16_PV_PEAK_TFLOPS = 1.0 / (0.5 / FP8_PEAK_TFLOPS + 0.5 / BF16_PEAK_TFLOPS)
PREFILL_WORKLOADS = ("chunked_prefill", "fp8kv_prefill", "fp8_prefill", "encoder")

# HBM bytes per launch of the dominant kernel, measured with rocprofv3 counters
# (FETCH_SIZE, WRITE_SIZE) and scaled by the same counters' reading for a plain
# device copy of known size; each entry carries the hash of the kernel sources
# it was taken on and is ignored once those sources change.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.txt")
KERNEL_SOURCES = ["pkv_attn.hip", "pkv_common.h", "pkv_device.h", "pkv_kernels.h"]
DOMINANT_KERNEL = {"paged_decode": "decode_balanced_kernel", "chunked_prefill": "prefill_kernel",
                   "long_decode": "decode_balanced_kernel", "long_decode_cascade": "decode_balanced_kernel",
                   "fp8_decode": "decode_balanced_kernel", "spec_decode": "prefill_kernel",
                   "fp8kv_prefill": "prefill_kernel", "fp8_prefill": "prefill_kernel", "encoder": "prefill_kernel"}

WORKLOADS = {
    "paged_decode": "paged decode, 32/8 heads GQA, head 128, bf16, batch 64, ctx U[512,4096], page 16",
    "chunked_prefill": "chunked prefill, batch 8, new U[128,2048] on cached U[0,4096], 32/8 heads, head 128, "
                       "bf16, page 16, causal",
    "long_decode": "long-context split-KV decode, batch 4, ctx 131072, 64/8 heads, head 128, bf16, page 256",
    "long_decode_cascade": "long decode as cascade: 4 requests share a 32768-token prefix, ctx 131072, "
                           "64/8 heads, head 128, bf16, page 256",
    "fp8_decode": "decode over an fp8 e4m3fn cache, bf16 q, batch 128, ctx U[1024,8192], 32/8 heads, head 128",
    "spec_decode": "multi-token decode (speculative verification), batch 64, q_len U[2,16] on ctx U[512,4096], "
                   "32/8 heads, head 128, bf16, page 16",
    "fp8kv_prefill": "chunked prefill over an fp8 e4m3fn cache, bf16 q, batch 8, new U[128,2048] on cached "
                     "U[0,4096], 32/8 heads, head 128, page 16, causal",
    "encoder": "non-causal encoder attention, flat K/V (no cache), batch 16, lengths U[512,4096], 32 heads MHA, "
               "head 128, bf16",
    "fp8_prefill": "chunked prefill, fp8 e4m3fn q and cache (QK^T on fp8 MFMA, PV on bf16 MFMA), batch 8, new "
                   "U[128,2048] on cached U[0,4096], 32/8 heads, head 128, page 16, causal",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def make(name, bs, over=None):
    import workloads
    if name == "paged_decode":
        return workloads.paged_decode(bs=bs or 16, **(over or {}))
    if name == "chunked_prefill":
        return workloads.chunked_prefill(bs=bs or 16)
    if name == "long_decode":
        return workloads.long_decode()
    if name == "long_decode_cascade":
        return workloads.long_decode(shared_prefix=32768)
    if name == "fp8_decode":
        return workloads.fp8_decode(bs=bs or 16)
    if name == "spec_decode":
        return workloads.spec_decode(bs=bs or 16)
    if name == "encoder":
        return workloads.encoder()
    if name == "fp8kv_prefill":
        return workloads.chunked_prefill(bs=bs or 16, cache_dtype="fp8")
    if name == "fp8_prefill":
        return workloads.chunked_prefill(bs=bs or 16, cache_dtype="fp8", q_dtype="fp8")
    raise SystemExit(f"unknown workload {name}")


def kv_elem_bytes(prob):
    return 1 if prob.cache_dtype == "fp8" else 2


def kv_bytes(prob, unique=False, window=0):
    """Algorithmic KV bytes of one forward: every request with a query token
    reads K and V of all its seq_len positions (cascade: the shared prefix
    once); with a sliding
    window of w keys, of the positions its first query token's window starts
    at onward."""
    per_tok = prob.Hkv * prob.hd * 2 * kv_elem_bytes(prob)
    L = np.where(prob.q_lens > 0, prob.seq_lens, 0).astype(np.int64)  # a request without queries reads nothing
    if window > 0:
        toks = int((L - np.minimum(L, np.maximum(0, prob.ctx_lens.astype(np.int64) - (window - 1)))).sum())
    else:
        toks = int(L.sum())
    if unique and prob.shared_prefix:
        toks -= (prob.B - 1) * prob.shared_prefix
    return toks * per_tok


def visible_keys(prob, window=0):
    """Keys each packed query row sees: ctx + t + 1 (causal) or L, at most
    the window."""
    n = []
    for r in range(prob.B):
        ql, ctx, L = int(prob.q_lens[r]), int(prob.ctx_lens[r]), int(prob.seq_lens[r])
        i = ctx + np.arange(ql, dtype=np.int64)
        vis = i + 1 if prob.causal else np.full(ql, L, np.int64)
        if window > 0:
            vis = vis - np.maximum(0, i - (window - 1))
        n.append(vis)
    return np.concatenate(n) if n else np.zeros(0, np.int64)


def kernel_sources_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_flash_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, block_size):
    """Counter-measured HBM bytes per launch for this workload, or None when
    no entry was taken on the current kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    want = kernel_sources_hash()
    for ln in open(TRAFFIC_FILE):
        f = ln.split("#")[0].split()
        if len(f) == 6 and f[0] == workload and int(f[1]) == block_size and f[5] == want:
            return int(f[3]) + int(f[4])
    return None


def pmc_summary(args):
    """Turn rocprofv3 --pmc CSV output into one traffic.txt line: mean
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the dominant kernel, each
    scaled by true bytes / counter bytes of a plain copy kernel."""
    import csv
    import glob

    def mean_counter(d, counter, name):
        vals = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for row in csv.DictReader(open(f)):
                if row["Counter_Name"] == counter and name in row["Kernel_Name"]:
                    vals.append(float(row["Counter_Value"]))
        if not vals:
            raise SystemExit(f"no {counter} rows for {name} under {d}")
        return sum(vals) / len(vals)
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = args.pmc_summary
    copy_bytes = args.calibrate_bytes
    f_fac = copy_bytes / (1024 * mean_counter(cfetch_dir, "FETCH_SIZE", "copyBuffer"))
    w_fac = copy_bytes / (1024 * mean_counter(cwrite_dir, "WRITE_SIZE", "copyBuffer"))
    kern = DOMINANT_KERNEL[args.workload or "paged_decode"]
    fetch = mean_counter(fetch_dir, "FETCH_SIZE", kern) * 1024 * f_fac
    write = mean_counter(write_dir, "WRITE_SIZE", kern) * 1024 * w_fac
    print(f"{args.workload or 'paged_decode'} {args.block_size} {kern} {int(round(fetch))} {int(round(write))} {kernel_sources_hash()}"
          f"  # copy factors fetch {f_fac:.4f} write {w_fac:.4f}")


def visible_flops(prob, window=0):
    """4 * hd * H * (visible query-key pairs): QK^T and PV, causal (and
    in-window) pairs only."""
    return 4 * prob.hd * prob.H * int(visible_keys(prob, window).sum())


def cascade_sweep():
    """Plain against cascade decode (64/8 heads, head 128, bf16, page 256) on
    batches whose requests share a prefix, each form timed as one HIP graph of
    30 forwards over 3 cache replicas used in turn, and the library's choice
    (pkv_cascade_choose) with its predicted times."""
    import torch

    import paged_kv_cache_flash_amd as pkv
    import workloads
    dev = torch.device("cuda:0")

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)
    for B, L, P in ((4, 131072, 32768), (4, 131072, 49152), (4, 131072, 65536), (4, 131072, 98304),
                    (8, 131072, 98304), (2, 262144, 196608), (8, 65536, 49152), (4, 131072, 8192),
                    (8, 16384, 8192), (16, 8192, 4096), (16, 4096, 512), (32, 8192, 2048), (64, 2048, 1024),
                    (2, 131072, 32768), (2, 131072, 65536), (3, 131072, 65536), (4, 65536, 32768),
                    (4, 32768, 16384), (4, 16384, 8192), (2, 32768, 16384), (8, 32768, 16384), (16, 16384, 8192),
                    (4, 131072, 16384), (3, 65536, 16384)):
        prob = workloads.long_decode(B=B, L=L, shared_prefix=P)
        reps = []
        for _ in range(3):
            kc, vc = prob.empty_cache()
            kc, vc = to_dev(kc), to_dev(vc)
            for c0 in range(0, len(prob.kv_src_k), 1 << 20):
                rr = np.arange(c0, min(len(prob.kv_src_k), c0 + (1 << 20)))
                pkv.pkv_cache_write(to_dev(prob.kv_src_k[rr]), to_dev(prob.kv_src_v[rr]), kc, vc,
                                    to_dev(prob.kv_slots[rr]))
            reps.append((kc, vc))
        q, qsl, sl, bt = to_dev(prob.q), to_dev(prob.query_start_loc), to_dev(prob.seq_lens), to_dev(prob.block_table)
        out = torch.empty_like(q)
        ws = torch.empty(pkv.pkv_varlen_workspace_size(q, reps[0][0], reps[0][1], qsl, sl, bt, prob.max_seqlen_q,
                                                       prob.max_seqlen_k, prob.scale), dtype=torch.uint8, device=dev)
        forms = {
            "plain": lambda i: pkv.pkv_varlen_fwd(q, reps[i % 3][0], reps[i % 3][1], qsl, sl, bt, prob.max_seqlen_q,
                                                  prob.max_seqlen_k, prob.scale, out=out, workspace=ws),
            "cascade": lambda i: pkv.cascade_attention(q, reps[i % 3][0], reps[i % 3][1], qsl, sl, bt, P,
                                                       prob.max_seqlen_q, prob.max_seqlen_k, prob.scale, out=out),
        }
        us = {}
        for name, f in forms.items():
            for i in range(4):
                f(i)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(30):
                    f(i)
            g.replay()
            torch.cuda.synchronize()
            t = time.perf_counter()
            g.replay()
            torch.cuda.synchronize()
            us[name] = (time.perf_counter() - t) / 30 * 1e6
        use, tp, tc = pkv.use_cascade_attention(P, prob.seq_lens, prob.T, prob.H, prob.Hkv, prob.hd)
        print(json.dumps({"batch": B, "seq_len": L, "shared_prefix": P, "plain_us": round(us["plain"], 1),
                          "cascade_us": round(us["cascade"], 1), "model_plain_us": round(tp, 1),
                          "model_cascade_us": round(tc, 1), "chosen": "cascade" if use else "plain",
                          "faster": "cascade" if us["cascade"] < us["plain"] else "plain"}), flush=True)
        del reps


def run_one(args, wl):
    """Time workload `wl` and return its result line (without printing it)."""
    import torch

    import paged_kv_cache_flash_amd as pkv

    dev = torch.device("cuda:0")

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        if a.dtype == np.uint8:
            return torch.from_numpy(a).to(dev).view(torch.float8_e4m3fn)
        return torch.from_numpy(a).to(dev)
    variants = args.sliding_window > 0 or args.softcap > 0 or args.sinks or args.alibi
    if variants and wl == "long_decode_cascade":
        raise SystemExit("bench: the attention variants are not benchmarked on the cascade workload")
    t0 = time.time()
    over = {k: v for k, v in (("B", args.batch), ("H", args.heads), ("Hkv", args.kv_heads)) if v}
    prob = make(wl, args.block_size, over)
    log(f"[bench] workload {wl}: B={prob.B} T={prob.T} sumL={int(prob.seq_lens.sum())} "
        f"H={prob.H} Hkv={prob.Hkv} hd={prob.hd} bs={prob.bs} cache={prob.cache_dtype} "
        f"(generated in {time.time() - t0:.1f}s)")

    # device inputs
    q = to_dev(prob.q)
    qsl = to_dev(prob.query_start_loc)
    seq_lens = to_dev(prob.seq_lens) if prob.paged else None
    bt = to_dev(prob.block_table) if prob.paged else None
    ks = vs = None
    if prob.cache_dtype == "fp8":
        ks = torch.tensor([prob.k_scale], dtype=torch.float32, device=dev)
        vs = torch.tensor([prob.v_scale], dtype=torch.float32, device=dev)
    qs = torch.tensor([prob.q_scale], dtype=torch.float32, device=dev) if prob.q_dtype == "fp8" else None
    reps = []
    if prob.paged:
        new_rows = prob.new_rows
        k_new, v_new, slots_new = to_dev(prob.kv_src_k[new_rows]), to_dev(prob.kv_src_v[new_rows]), \
            to_dev(prob.kv_slots[new_rows])
        cache_bytes = 2 * prob.num_blocks * prob.bs * prob.Hkv * prob.hd * kv_elem_bytes(prob)
        R = args.replicas or max(1, min(8, int(np.ceil(1.5e9 / cache_bytes)) + 1))
        ctx_rows = prob.context_rows()
        kc0, vc0 = prob.empty_cache()
        for _ in range(R):
            kc, vc = to_dev(kc0), to_dev(vc0)
            for c0 in range(0, len(ctx_rows), 1 << 20):
                rr = ctx_rows[c0:c0 + (1 << 20)]
                pkv.pkv_cache_write(to_dev(prob.kv_src_k[rr]), to_dev(prob.kv_src_v[rr]), kc, vc,
                                    to_dev(prob.kv_slots[rr]), ks, vs)
            reps.append((kc, vc))
        del kc0, vc0
    else:
        # flat K/V packed like q: the step is the forward alone (no cache write)
        flat = np.concatenate(prob.pos_rows)
        cache_bytes = 2 * len(flat) * prob.Hkv * prob.hd * kv_elem_bytes(prob)
        R = args.replicas or max(1, min(8, int(np.ceil(1.5e9 / cache_bytes)) + 1))
        for _ in range(R):
            reps.append((to_dev(prob.kv_src_k[flat]), to_dev(prob.kv_src_v[flat])))
    torch.cuda.synchronize()
    log(f"[bench] {R} cache replicas of {cache_bytes / 1e9:.3f} GB resident")

    out = torch.empty(q.shape, dtype=torch.bfloat16 if prob.q_dtype == "fp8" else q.dtype, device=dev)
    lse = torch.empty((prob.H, prob.T), dtype=torch.float32, device=dev)
    cascade = prob.shared_prefix > 0
    W = args.sliding_window
    sinks_h = np.random.default_rng(12345).normal(1.5, 2.0, prob.H).astype(np.float32) if args.sinks else None
    alibi_h = (2.0 ** (-8.0 * (np.arange(prob.H) + 1) / prob.H)).astype(np.float32) if args.alibi else None
    fwd_kw = dict(softmax_scale=prob.scale, causal=prob.causal, k_scale=ks, v_scale=vs, sliding_window=W,
                  softcap=args.softcap, sinks=None if sinks_h is None else to_dev(sinks_h), q_scale=qs,
                  alibi_slopes=None if alibi_h is None else to_dev(alibi_h))
    if not cascade:
        need = pkv.pkv_varlen_workspace_size(q, reps[0][0], reps[0][1], qsl, seq_lens, bt, prob.max_seqlen_q,
                                             prob.max_seqlen_k, prob.scale, prob.causal, args.num_splits, W)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        splits = pkv.pkv_varlen_num_splits(q, reps[0][0], reps[0][1], qsl, seq_lens, bt, prob.max_seqlen_q,
                                           prob.max_seqlen_k, prob.scale, prob.causal, args.num_splits, W)
    else:
        splits = None
        ws = torch.empty(pkv.pkv_cascade_workspace_size(q, reps[0][0], reps[0][1], qsl, seq_lens, bt,
                                                        prob.shared_prefix, prob.max_seqlen_q, prob.max_seqlen_k,
                                                        prob.scale), dtype=torch.uint8, device=dev)

    def step(i, write=True):
        kc, vc = reps[i % R]
        if prob.paged and write:
            pkv.pkv_cache_write(k_new, v_new, kc, vc, slots_new, ks, vs)
        if cascade:
            pkv.cascade_attention(q, kc, vc, qsl, seq_lens, bt, prob.shared_prefix, prob.max_seqlen_q,
                                  prob.max_seqlen_k, prob.scale, k_scale=ks, v_scale=vs, out=out, workspace=ws)
        else:
            pkv.pkv_varlen_fwd(q, kc, vc, qsl, seq_lens, bt, prob.max_seqlen_q, prob.max_seqlen_k, out=out,
                               lse=lse, num_splits=args.num_splits, workspace=ws, **fwd_kw)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Eager timed pass: the K steps launched one by one, with the library's
    # HIP events around each attention kernel and each merge kernel (on the
    # stream they are launched on). Kernel durations come from this pass.
    pkv.timing_enable(True)
    pkv.timing_collect()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t_start) * 1e3 / args.steps
    main_each, merge_each = pkv.timing_collect_calls()
    calls, main_ms, merge_ms = len(main_each), float(sum(main_each)), float(sum(merge_each))
    pkv.timing_enable(False)

    # The cache write on its own: K calls captured in one HIP graph (a call
    # launched eagerly is shorter than its host launch), timed with events
    # around a replay, and its algorithmic bytes (new K and V read, written
    # into the cache, and one int64 slot per token).
    cache_write = None
    if prob.paged and not args.eager:
        cw_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cw_graph):
            for i in range(args.steps):
                kc, vc = reps[(args.warmup + i) % R]
                pkv.pkv_cache_write(k_new, v_new, kc, vc, slots_new, ks, vs)
        cw_graph.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cw_graph.replay()
        e1.record()
        torch.cuda.synchronize()
        cw_us = e0.elapsed_time(e1) * 1e3 / args.steps
        cw_bytes = k_new.numel() * 2 * (k_new.element_size() + reps[0][0].element_size()) + slots_new.numel() * 8
        cache_write = {"tokens": int(k_new.shape[0]), "us_per_call": round(cw_us, 2), "bytes": int(cw_bytes),
                       "GB_per_s": round(cw_bytes / cw_us / 1e3, 1), "launch": "hip_graph"}
        del cw_graph

    # The attention alone (attention kernel + merge kernel, no cache write):
    # the K calls captured in one HIP graph and timed by events around a
    # replay on the launch stream. Back to back in a graph, the calls pay no
    # per-launch event or dispatch latency, so this is the kernels' own time
    # (rocprofv3's kernel durations agree with it); the roofline uses it.
    attn_ms = None
    if not args.eager:
        a_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(a_graph):
            for i in range(args.steps):
                step(args.warmup + i, write=False)
        a_graph.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        a_graph.replay()
        e1.record()
        torch.cuda.synchronize()
        attn_ms = e0.elapsed_time(e1) / args.steps
        del a_graph

    use_graph = not args.eager
    if use_graph:
        # The K timed steps captured into one HIP graph, as a serving engine
        # captures its decode step: one untimed replay, then the timed replay.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(args.warmup + i)
        graph.replay()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t_start) * 1e3 / args.steps
    else:
        ms_step = ms_eager
    log(f"[bench] {args.steps} steps: {ms_step:.4f} ms/step ({'graph' if use_graph else 'eager'}; eager "
        f"{ms_eager:.4f}); attention calls {calls}, main kernel {main_ms / max(calls, 1):.4f} ms avg, "
        f"merge {merge_ms / max(calls, 1):.4f} ms avg"
        + (f"; attention alone in a graph {attn_ms:.4f} ms per call" if attn_ms else ""))
    # per-call attention time for the roofline: the graph-replayed attention
    # when there is one, else the eager events around the kernels
    t_attn_ms = attn_ms if attn_ms else (main_ms + merge_ms) / args.steps

    decode_like = wl not in PREFILL_WORKLOADS
    # the balanced decode runs 1024 or 2048 waves; a plan of fewer splits is
    # the plain decode grid (e.g. a short sliding window)
    kernel_name = DOMINANT_KERNEL[wl]
    if kernel_name == "decode_balanced_kernel" and splits is not None and splits < 1024:
        kernel_name = "decode_kernel"
    # HBM bytes per launch of the dominant kernel from committed counter runs
    # (None unless they were taken on the current kernel sources)
    traffic = None if variants else measured_traffic(wl, prob.bs)
    if decode_like:
        kvb = kv_bytes(prob, unique=cascade, window=W)
        value = kvb / (ms_step * 1e-3) / 1e9
        metric, unit = "paged decode KV GB/s", "GB/s"
        # the attention reads the whole KV once per step (cascade: a prefix
        # launch and a suffix launch per step); its time is the attention
        # kernel plus the split-KV merge kernel, and the dominant kernel alone
        # is reported beside it
        achieved = kvb / (t_attn_ms * 1e-3) / 1e9
        achieved_k = kvb / (main_ms / args.steps * 1e-3) / 1e9
        # every algorithmic byte: K/V, q, out, lse and the block-table entries read
        used_pages = int(((prob.seq_lens.astype(np.int64) + prob.bs - 1) // prob.bs).sum()) if prob.paged else 0
        all_bytes = kvb + prob.T * prob.H * prob.hd * 2 * (1 if prob.q_dtype == "fp8" else 2) \
            + prob.T * prob.H * prob.hd * 2 + prob.T * prob.H * 4 + used_pages * 4
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "timed": ("attention kernel + split-KV merge kernel, " +
                              ("K calls replayed in a HIP graph" if attn_ms else "eager, events around each")),
                    "algorithmic_bytes_per_launch": kvb,
                    "all_algorithmic_bytes_per_launch": int(all_bytes),
                    "achieved_all_bytes": round(all_bytes / (t_attn_ms * 1e-3) / 1e9, 1),
                    "kernel_only": {"kernel": kernel_name, "achieved": round(achieved_k, 1),
                                    "frac": round(achieved_k / HBM_PEAK_GBS, 4)}}
    else:
        fl = visible_flops(prob, W)
        value = fl / (ms_step * 1e-3) / 1e12
        metric, unit = ("causal prefill TFLOP/s" if prob.causal else "non-causal attention TFLOP/s"), "TFLOP/s"
        achieved = fl / (t_attn_ms * 1e-3) / 1e12
        peak = FP8_QK_BF16_PV_PEAK_TFLOPS if prob.q_dtype == "fp8" else BF16_PEAK_TFLOPS
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": round(peak, 1), "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4), "traffic": traffic,
                    "timed": DOMINANT_KERNEL[wl] + (" + split-KV merge kernel" if merge_ms > 0 else "") +
                             (", K calls replayed in a HIP graph" if attn_ms else ", eager, events around each"),
                    "algorithmic_flops_per_launch": fl}

    cpu = None
    if not args.no_cpu_baseline:
        # CPU-baseline leg: the float64 oracle (test infrastructure) on this
        # workload. It first checks sampled rows of the timed output, then is
        # timed on whole requests of the same batch.
        # correctness spot check of the timed configuration against the oracle
        import oracle
        rng = np.random.default_rng(0)
        sample = np.sort(rng.choice(prob.T, size=min(prob.T, 8), replace=False))
        if prob.paged:
            kc_o, vc_o = prob.empty_cache()
            kc_o, vc_o = oracle.cache_write(prob.kv_src_k, prob.kv_src_v, kc_o, vc_o, prob.kv_slots, prob.bs,
                                            k_scale=prob.k_scale, v_scale=prob.v_scale)
            sl_o, bt_o = prob.seq_lens, prob.block_table
        else:
            flat = np.concatenate(prob.pos_rows)
            kc_o, vc_o, sl_o, bt_o = prob.kv_src_k[flat], prob.kv_src_v[flat], None, None
        var_o = dict(window_left=W - 1 if W > 0 else -1, softcap=args.softcap,
                     sinks=None if sinks_h is None else sinks_h.astype(np.float64),
                     alibi=None if alibi_h is None else alibi_h.astype(np.float64))
        ref, ref_lse = oracle.attention(prob.q, kc_o, vc_o, prob.query_start_loc, sl_o, bt_o,
                                        scale=prob.scale, causal=prob.causal, rows=sample, k_scale=prob.k_scale,
                                        v_scale=prob.v_scale, q_scale=prob.q_scale, **var_o)
        tol = 5e-2 if prob.cache_dtype == "fp8" else 1e-2
        o = out.float().cpu().numpy().astype(np.float64)[sample]
        # the bar is tol, widened by half a bf16 ulp only where that rounding
        # of the exact answer alone exceeds tol (|ref| >= 4 at 1e-2)
        half_ulp = np.where(np.abs(ref) > 0, np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 8), 0)
        if not np.all(np.abs(o - ref) <= np.where(half_ulp > tol, tol + half_ulp, tol)):
            raise SystemExit(f"bench: sampled rows differ from the oracle by {np.abs(o - ref).max():.3e}")
        if not cascade:
            lerr = np.abs(lse.cpu().numpy()[:, sample] - ref_lse).max()
            if lerr > 1e-3:
                raise SystemExit(f"bench: sampled lse differs from the oracle by {lerr:.3e}")
        log(f"[bench] sampled rows match the oracle (tolerance {tol})")
        # the oracle as it stands, on whole requests of the same batch, until
        # about --cpu-seconds of CPU work
        nthr = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
        # rows in packed order, a few at a time, until about --cpu-seconds
        done_rows, done_bytes, done_flops, t_cpu = 0, 0, 0, 0.0
        vis = visible_keys(prob, W)
        per_tok_kv = prob.Hkv * prob.hd * 2 * kv_elem_bytes(prob)
        # (a batch the oracle finishes sooner is run again from its first row)
        r0, passes = 0, 0
        while t_cpu < args.cpu_seconds:
            rows = np.arange(r0, min(prob.T, r0 + 16))
            t1 = time.perf_counter()
            oracle.attention(prob.q, kc_o, vc_o, prob.query_start_loc, sl_o, bt_o,
                             scale=prob.scale, causal=prob.causal, rows=rows, k_scale=prob.k_scale,
                             v_scale=prob.v_scale, nthreads=nthr, q_scale=prob.q_scale, **var_o)
            t_cpu += time.perf_counter() - t1
            n_vis = int(vis[rows].sum())
            done_flops += 4 * prob.hd * prob.H * n_vis
            done_bytes += n_vis * per_tok_kv   # keys read for these rows (all kv heads)
            done_rows += len(rows)
            r0 += len(rows)
            if r0 >= prob.T:
                r0, passes = 0, passes + 1
        cpu_val = (done_bytes / t_cpu / 1e9) if decode_like else (done_flops / t_cpu / 1e12)
        what = (f"{passes} passes over all {prob.T} query rows" + (f" and the first {r0} again" if r0 else "")
                if passes else f"first {done_rows} of {prob.T} query rows")
        cpu = {"value": round(cpu_val, 4), "unit": unit, "cores": oracle.num_threads() if nthr <= 0 else nthr,
               "kind": "oracle",
               "sample": f"{what} of the same batch, all heads, float64, {t_cpu:.1f}s"}
        log(f"[bench] oracle: {cpu}")

    desc = WORKLOADS[wl]
    if over or (args.block_size and wl == "paged_decode"):
        desc = (f"paged decode, {prob.H}/{prob.Hkv} heads, head {prob.hd}, bf16, batch {prob.B}, "
                f"ctx U[512,4096], page {prob.bs}")
    if prob.bs != 16 and "page 16" in desc:
        desc = desc.replace("page 16", f"page {prob.bs}")
    if W > 0:
        desc += f", sliding window {W}"
    if args.softcap > 0:
        desc += f", softcap {args.softcap:g}"
    if args.sinks:
        desc += ", sinks"
    if args.alibi:
        desc += ", ALiBi"
    med = float(np.median(main_each)) if main_each else None
    roofline["kernel_ms_mean"] = round(main_ms / max(calls, 1), 5)
    roofline["kernel_ms_median"] = round(med, 5) if med else None
    roofline["kernel_ms_min"] = round(float(min(main_each)), 5) if main_each else None
    roofline["merge_ms_mean"] = round(merge_ms / max(calls, 1), 5)
    roofline["attention_ms_per_call_graph"] = round(attn_ms, 5) if attn_ms else None
    cfg = {"workload": desc, "global_batch": prob.B, "seq_len": prob.max_seqlen_k,
           "num_heads": prob.H, "num_kv_heads": prob.Hkv, "head_size": prob.hd, "block_size": prob.bs if prob.paged else None,
           "kv_cache_dtype": prob.cache_dtype, "num_splits": splits, "cache_replicas": R,
           "launch": "hip_graph" if use_graph else "eager", "ms_per_step_eager": round(ms_eager, 5),
           "parallelism": "single GPU"}
    line = {"metric": metric, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "fp8 QK^T, bf16 PV" if prob.q_dtype == "fp8" else "bf16", "data": "synthetic", "config": cfg, "roofline": roofline,
            "cpu_baseline": cpu, "cache_write": cache_write}
    return line


# The other workloads of the hot path, timed briefly in the default run, each
# in a child process of its own (so that no failure there costs the line
# above): configs 4 and 5, config 4 as a one-launch cascade, multi-token
# decode, the non-causal encoder and windowed decode with sinks.
OTHER_WORKLOADS = (("long_decode", ["--workload", "long_decode"]),
                   ("long_decode_cascade", ["--workload", "long_decode_cascade"]),
                   ("fp8_decode", ["--workload", "fp8_decode"]),
                   ("multi_token_decode", ["--workload", "spec_decode"]),
                   ("encoder", ["--workload", "encoder"]),
                   ("paged_decode_window1024_sinks", ["--workload", "paged_decode", "--sliding-window", "1024",
                                                      "--sinks"]))


def other_workloads():
    import subprocess
    out = {}
    for key, wargs in OTHER_WORKLOADS:
        cmd = [sys.executable, os.path.abspath(__file__), *wargs, "--steps", "20", "--warmup", "5",
               "--no-cpu-baseline"]
        log(f"[bench] {key}: {' '.join(wargs)}")
        try:
            res = subprocess.run(cmd, capture_output=True, text=True, timeout=180)
            rows = [l for l in res.stdout.splitlines() if l.startswith("{")]
            if res.returncode != 0 or not rows:
                tail = (res.stderr or res.stdout).strip().splitlines()[-1:] or [""]
                out[key] = {"error": f"exit {res.returncode}: {tail[0][:200]}"}
                continue
            r = json.loads(rows[-1])
            rf = r["roofline"]
            out[key] = {"metric": r["metric"], "value": r["value"], "unit": r["unit"], "ms_per_step": r["ms_per_step"],
                        "steps": r["steps"], "config": r["config"],
                        "roofline": {k: rf.get(k) for k in ("bound", "achieved", "peak", "unit", "frac", "traffic",
                                                            "attention_ms_per_call_graph")}}
        except Exception as e:  # (a timeout, an unreadable line)
            out[key] = {"error": f"{type(e).__name__}: {e}"[:200]}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, choices=sorted(WORKLOADS),
                    help="one workload only (default: paged decode, with the chunked prefill leg nested)")
    ap.add_argument("--block-size", type=int, default=0,
                    help="page size (default 16; a page as long as the longest request makes the KV contiguous)")
    ap.add_argument("--batch", type=int, default=0, help="paged_decode: requests (default 64)")
    ap.add_argument("--heads", type=int, default=0, help="paged_decode: query heads (default 32)")
    ap.add_argument("--kv-heads", type=int, default=0, help="paged_decode: kv heads (default 8)")
    ap.add_argument("--num-splits", type=int, default=0, help="0 = library's choice")
    ap.add_argument("--sliding-window", type=int, default=0, help="a query sees at most this many keys (0: off)")
    ap.add_argument("--softcap", type=float, default=0.0, help="logits soft cap (0: off)")
    ap.add_argument("--sinks", action="store_true", help="one sink logit per query head (seeded)")
    ap.add_argument("--alibi", action="store_true", help="ALiBi with the geometric slopes 2^(-8 (h + 1) / H)")
    ap.add_argument("--replicas", type=int, default=0, help="KV cache copies used in turn (0 = enough for 1.5 GB)")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches only (default: the timed steps are one captured HIP graph)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle baseline")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (reference for HBM byte counters)")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="only summarise rocprofv3 --pmc output of this workload into a traffic line")
    ap.add_argument("--calibrate-bytes", type=int, default=1 << 30, help="bytes of the copy in the calibration runs")
    ap.add_argument("--cascade-sweep", action="store_true",
                    help="only time plain against cascade decode on shared-prefix batches, next to the library's "
                         "cascade choice (one JSON line per batch)")
    args = ap.parse_args()

    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.cascade_sweep:
        cascade_sweep()
        return
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 3}), flush=True)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the attention shards by request "
              "or kv head with no exchange; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.workload is None:
        # the headline pair: paged decode (KV GB/s against HBM) with the
        # chunked prefill leg (TFLOP/s against bf16 MFMA) nested in its line
        line = run_one(args, "paged_decode")
        pre = run_one(args, "chunked_prefill")
        line["prefill"] = {k: pre[k] for k in ("metric", "value", "unit", "ms_per_step", "higher_is_better",
                                                "dtype", "config", "roofline", "cpu_baseline", "cache_write")}
        line["also"] = other_workloads()
    else:
        line = run_one(args, args.workload)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
