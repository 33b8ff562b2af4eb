#!/usr/bin/env python3
"""Benchmark of the fused attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the Attention layer's forward over one batch of
synthetic input, as the blog post "从零实现 vLLM (1.3)：如何加速 Attention 计算"
walks through it (section Attention 源码分析): store the batch's new K/V into
the paged cache (kv_store_slots), then attention.

* Headline (value): varlen causal prefill, 16 sequences with lengths uniform
  in [128, 4096] (Lq = Lk), 32 query / 8 KV heads, head_dim 128, bf16 inputs,
  bf16 output.  value = algorithmic attention flops of the step / step time,
  in TFLOP/s; algorithmic flops = 4 * d * Hq * (number of visible
  query-key pairs).  Inputs are resident in HBM before timing starts.
* decode (extra object): paged decode, batch 64, contexts uniform in
  [512, 8192], block 256, new token stored first; algorithmic bytes = every
  cached K and V byte read once per KV head; GB/s.  It carries its own
  roofline, the oracle's rate on a sample of the batch (cpu_baseline), and
  the shared-prompt decode variant (64 sequences whose block tables begin
  with the same 8 physical blocks).
* roofline: the prefill kernel alone, timed right after the steps as K
  launches back to back between two HIP events (no store between them; the
  steps themselves carry no events, whose records leave the GPU idle for a
  few microseconds each), against bf16 dense MFMA peak;
  traffic = HBM bytes per launch from the FETCH_SIZE / WRITE_SIZE counter
  runs recorded in profiles/ (null once the kernel sources changed).
* other_prefill: the 32768-token sequence, the prefix-cache batch (32
  sequences, 1-512 new tokens on 1K-16K cached ones, paged) and the
  shared-prompt batch, a few timed steps each, as TFLOP/s against the same
  peak, with recorded traffic and, for the paged batches, the sum over
  sequences of max(flops / MFMA peak, bytes / HBM peak).  They run before
  the headline, which is then timed on a GPU already at its working clock.
* unfused_baseline: the blog's standard three-step method (X and A stored in
  HBM between three kernels) on the same varlen workload, next to the fused
  kernel's time; skipped with --skip-unfused (it needs ~52 GB of workspace).
* cpu_baseline: the fp64 CPU oracle timed on a bounded sample of the same
  workload's rows on this host's cores, scaled to TFLOP/s by the same
  algorithmic flop count.
* env: device, versions, and the GPU clock read (amd-smi / rocm-smi) while
  the headline kernel runs back to back, next to the nominal clock of the
  peak figures.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

# Sources whose hash identifies each kernel; a recorded HBM-traffic figure is
# reported only while these files are unchanged since the counters were taken.
KERNEL_SOURCES = {
    "prefill": ["attention_sdpa_amd/csrc/prefill_mfma.hip", "attention_sdpa_amd/csrc/device_common.h",
                "attention_sdpa_amd/csrc/launch.h"],
    "decode": ["attention_sdpa_amd/csrc/decode.hip", "attention_sdpa_amd/csrc/device_common.h",
               "attention_sdpa_amd/csrc/launch.h"],
}
# per workload: (kernel whose sources the counters describe, counter file)
TRAFFIC_FILES = {"varlen": ("prefill", "profiles/prefill_mfma_varlen16_pmc.md"),
                 "long": ("prefill", "profiles/prefill_mfma_long32k_pmc.md"),
                 "prefix": ("prefill", "profiles/prefill_mfma_prefix32_pmc.md"),
                 "decode": ("decode", "profiles/decode_paged_b64_pmc.md")}


PREFILL_WORKLOADS = {
    "varlen": "varlen causal prefill: 16 sequences, lengths U[128,4096] (Lq = Lk), packed by "
              "cu_seqlens, 32 Q / 8 KV heads, head_dim 128, bf16 in/out, new K/V stored to a "
              "256-token paged cache first",
    "long": "long causal prefill: 1 sequence of 32768 tokens, 32 Q / 8 KV heads, head_dim 128, "
            "bf16 in/out, Q/K ~ N(0, 4), new K/V stored to a 256-token paged cache first",
    "noncausal": "varlen non-causal prefill: the 16-sequence batch of the headline workload "
                 "without the causal mask, bf16 in/out",
    "prefix": "prefix-cache prefill: 32 sequences, new-token lengths U[1,512] attending to cached "
              "prefixes U[1024,16384] plus themselves through a 256-token paged cache (new K/V "
              "stored first), end-aligned causal mask, 32 Q / 8 KV heads, head_dim 128, bf16",
    "shared": "shared-prompt prefill: 32 sequences whose block tables all begin with the same 8 "
              "physical blocks (a 2048-token system prompt stored once), then own cached tokens "
              "U[0,4096] and new tokens U[1,512] through a 256-token paged cache (new K/V stored "
              "first), end-aligned causal mask, 32 Q / 8 KV heads, head_dim 128, bf16",
}
SHARED_DECODE = ("shared-prompt decode: batch 64 whose block tables all begin with the same 8 "
                 "physical blocks (a 2048-token prompt stored once), own cached tokens U[0,6144], "
                 "new token stored first, block 256, 32 Q / 8 KV heads, head_dim 128")


def source_sha(which: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[which]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload: str):
    """HBM bytes per launch measured by the FETCH_SIZE / WRITE_SIZE passes
    recorded in profiles/ for this workload, or None if missing or the
    kernel changed since."""
    which, rel = TRAFFIC_FILES[workload]
    path = os.path.join(ROOT, rel)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.split(":", 1)[0].strip() in ("kernel_source_sha256",
                                                                  "traffic_bytes_per_launch"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256") != source_sha(which):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def visible_pairs(cu_q, cu_k, causal=True) -> int:
    """Number of (query, key) pairs that the causal, end-aligned mask keeps."""
    total = 0
    for b in range(len(cu_q) - 1):
        lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        if not causal:
            total += lq * lk
            continue
        for_i0 = lk - lq + 1     # visible keys of query 0 (may be <= 0)
        # sum_{i=0}^{lq-1} clamp(for_i0 + i, 0, lk)
        for i in range(lq):
            n = for_i0 + i
            total += 0 if n <= 0 else (lk if n > lk else n)
    return total


def timed_loop(step, steps, warmup, torch):
    """W untimed steps, then K timed steps between a device sync on both
    sides; returns the wall time of the K steps in seconds.  Nothing else is
    enqueued between the steps (no events: each one recorded between two
    launches leaves the GPU idle for several microseconds)."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def launch_ms(call, steps, warmup, torch):
    """Average duration in ms of one launch of `call` (an attention entry
    point): W untimed calls, then K calls back to back between two HIP
    events on torch's current stream, which is the stream the library
    launches on."""
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def shared_prefill_workload(workloads, dtype, queries=(1, 512), n_seqs=32, own_hi=4096, seed=1006):
    """The shared-prompt workload: 8 blocks of 256 tokens shared by every block table."""
    return workloads.shared_prefix_prefill(n_seqs=n_seqs, shared_blocks=8, own_lo=0, own_hi=own_hi,
                                           q_lo=queries[0], q_hi=queries[1], hq=32, hkv=8, d=128,
                                           block_size=256, seed=seed, dtype=dtype)


def per_sequence_bound(cu_q, cu_k, hq=32, hkv=8, d=128):
    """Sum over sequences of max(flops_b / MFMA peak, bytes_b / HBM peak), in
    seconds: the roofline of a batch whose sequences differ in arithmetic
    intensity (Q, O and the sequence's K/V moved once, bf16)."""
    t = 0.0
    for b in range(len(cu_q) - 1):
        lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        fl = 4.0 * d * hq * visible_pairs([0, lq], [0, lk], True)
        by = 2.0 * d * (2 * lq * hq + 2 * lk * hkv)
        t += max(fl / (PEAK_BF16_TFLOPS * 1e12), by / (PEAK_HBM_GBS * 1e9))
    return t


def prep_prefix(args, torch, attn, workloads):
    """Prefix-cache prefill: the new tokens' K/V are stored into the paged
    cache, then the new queries attend to prefix + new keys through the
    block table (end-aligned causal mask).  Builds the inputs on the GPU and
    returns the timing run (called later, back to back with the others)."""
    if args.prefill_workload == "shared":
        pp = shared_prefill_workload(workloads, args.torch_dtype)
    else:
        pp = workloads.prefix_prefill(dtype=args.torch_dtype)
    pg = pp.paged
    q = pp.q.cuda()
    kc, vc = pg.k_cache.cuda(), pg.v_cache.cuda()
    kn, vn, slots = pg.k_new.cuda(), pg.v_new.cuda(), pg.slot_mapping.cuda()
    cu_q, cu_k, bt = pp.cu_seqlens_q.cuda(), pg.cu_seqlens_k.cuda(), pg.block_table.cuda()
    out = torch.empty_like(q)

    def call():
        attn.attn_prefill_varlen(q, kc, vc, cu_q, cu_k, pp.max_seqlen_q, pp.max_seqlen_k,
                                 pp.softmax_scale, True, block_table=bt, out=out)

    def step(i):
        attn.kv_store_slots(kn, vn, kc, vc, slots)
        call()

    def go():
        wall = timed_loop(step, args.steps, args.warmup, torch)
        k_ms = launch_ms(call, args.steps, args.warmup, torch)
        pairs = visible_pairs(pp.cu_seqlens_q.tolist(), pg.cu_seqlens_k.tolist(), True)
        flops = 4.0 * 128 * 32 * pairs
        ms_step = wall * 1e3 / args.steps
        total_k = int(pg.cu_seqlens_k[-1])
        bound_s = per_sequence_bound(pp.cu_seqlens_q.tolist(), pg.cu_seqlens_k.tolist())
        return dict(vl=None, flops=flops, ms_step=ms_step, kernel_ms=k_ms,
                    tflops_step=flops / (ms_step * 1e-3) / 1e12,
                    tflops_kernel=flops / (k_ms * 1e-3) / 1e12,
                    total_tokens=int(q.shape[0]),
                    bytes_alg=2.0 * (2 * q.numel() + 2 * total_k * 8 * 128),
                    bound_ms=bound_s * 1e3, unique_kv_bytes=2.0 * 2 * kc.shape[0] * kc.shape[1] * 8 * 128)
    return go


def prep_prefill(args, torch, attn, workloads):
    """Inputs of one prefill workload on the GPU; returns its timing run."""
    if args.prefill_workload in ("prefix", "shared"):
        return prep_prefix(args, torch, attn, workloads)
    if args.prefill_workload == "long":
        vl = workloads.long_prefill(dtype=args.torch_dtype)
    elif args.prefill_workload == "noncausal":
        vl = workloads.varlen_prefill(dtype=args.torch_dtype)
        vl.causal = False
    else:
        vl = workloads.varlen_prefill(dtype=args.torch_dtype)
    cache = workloads.cache_for_varlen(vl, block_size=256, seed=5)
    q, k, v = vl.q.cuda(), vl.k.cuda(), vl.v.cuda()
    cu_q, cu_k = vl.cu_seqlens_q.cuda(), vl.cu_seqlens_k.cuda()
    kc, vc = cache.k_cache.cuda(), cache.v_cache.cuda()
    slots = cache.slot_mapping.cuda()
    out = torch.empty_like(q)

    def enqueue():
        attn.attn_prefill_varlen(q, k, v, cu_q, cu_k, vl.max_seqlen_q, vl.max_seqlen_k,
                                 vl.softmax_scale, vl.causal, out=out)

    def step(i):
        attn.kv_store_slots(k, v, kc, vc, slots)
        enqueue()

    def go():
        wall = timed_loop(step, args.steps, args.warmup, torch)
        k_ms = launch_ms(enqueue, args.steps, args.warmup, torch)
        pairs = visible_pairs(vl.cu_seqlens_q.tolist(), vl.cu_seqlens_k.tolist(), vl.causal)
        flops = 4.0 * 128 * 32 * pairs
        ms_step = wall * 1e3 / args.steps
        lens = (vl.cu_seqlens_q[1:] - vl.cu_seqlens_q[:-1]).tolist()
        return dict(vl=vl, flops=flops, ms_step=ms_step, kernel_ms=k_ms,
                    tflops_step=flops / (ms_step * 1e-3) / 1e12,
                    tflops_kernel=flops / (k_ms * 1e-3) / 1e12,
                    total_tokens=int(vl.q.shape[0]), lens=lens, enqueue=enqueue,
                    bytes_alg=2.0 * (q.numel() + k.numel() + v.numel() + out.numel()))
    return go


def shared_decode_workload(workloads, dtype):
    """Decode over a shared prompt: the shared-prompt builder with one new
    token per sequence (its K/V stored first), 64 sequences."""
    pp = shared_prefill_workload(workloads, dtype, queries=(1, 1), n_seqs=64, own_hi=6144, seed=1007)
    return workloads.Decode(pp.q.view(pp.batch, 32, 128), pp.softmax_scale, pp.paged, "shared_decode")


def prep_decode(args, torch, attn, workloads, shared=False):
    """Inputs of the decode workload on the GPU; returns its timing run."""
    dc = shared_decode_workload(workloads, args.torch_dtype) if shared else \
        workloads.paged_decode(dtype=args.torch_dtype)
    pg = dc.paged
    q = dc.q.cuda()
    kc, vc = pg.k_cache.cuda(), pg.v_cache.cuda()
    kn, vn, slots = pg.k_new.cuda(), pg.v_new.cuda(), pg.slot_mapping.cuda()
    sl, bt = pg.seqlens_k.cuda(), pg.block_table.cuda()
    out = torch.empty_like(q)
    need = attn.attn_decode_workspace_bytes(q.shape[0], 32, 8, 128, bt.shape[1], 256, 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def call():
        attn.attn_decode_paged(q, kc, vc, sl, bt, dc.softmax_scale, workspace=ws, out=out)

    def step(i):
        attn.kv_store_slots(kn, vn, kc, vc, slots)
        call()

    def go():
        wall = timed_loop(step, args.steps, args.warmup, torch)
        k_ms = launch_ms(call, args.steps, args.warmup, torch)
        kv_bytes = float(sum(pg.seqlens_k.tolist())) * 8 * 128 * 2 * 2
        ms_step = wall * 1e3 / args.steps
        return dict(dc=dc, kv_bytes=kv_bytes, ms_step=ms_step, kernel_ms=k_ms,
                    gbs_step=kv_bytes / (ms_step * 1e-3) / 1e9,
                    gbs_kernel=kv_bytes / (k_ms * 1e-3) / 1e9,
                    unique_kv_bytes=2.0 * 2 * kc.shape[0] * kc.shape[1] * 8 * 128)
    return go


def prep_unfused(args, torch, attn, workloads):
    """The unfused three-kernel baseline (X and A stored in HBM between the
    steps) on the headline varlen workload; returns its timing run, which
    takes the fused kernel's time for the comparison."""
    vl = workloads.varlen_prefill()
    q, k, v = vl.q.cuda(), vl.k.cuda(), vl.v.cuda()
    cu_q, cu_k = vl.cu_seqlens_q.cuda(), vl.cu_seqlens_k.cuda()
    out = torch.empty_like(q)
    B = vl.cu_seqlens_q.numel() - 1
    need = attn.attn_unfused_workspace_bytes(B, 32, vl.max_seqlen_q, vl.max_seqlen_k)

    def go(fused_ms):
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")

        def call():
            attn.attn_prefill_unfused(q, k, v, cu_q, cu_k, vl.max_seqlen_q, vl.max_seqlen_k,
                                      vl.softmax_scale, True, workspace=ws, out=out)

        steps, warmup = max(1, min(args.steps, 10)), max(1, min(args.warmup, 2))
        ms = launch_ms(call, steps, warmup, torch)
        lq = (vl.cu_seqlens_q[1:] - vl.cu_seqlens_q[:-1]).tolist()
        lk = (vl.cu_seqlens_k[1:] - vl.cu_seqlens_k[:-1]).tolist()
        pairs_all = float(sum(a * b for a, b in zip(lq, lk)))
        pairs = visible_pairs(vl.cu_seqlens_q.tolist(), vl.cu_seqlens_k.tolist(), True)
        # the round trips the fused kernel avoids, per query head: X written for
        # every (query, key) pair (fp32) and read back for the visible ones, A
        # written (bf16) for every pair and read back
        xa_bytes = 32 * (pairs_all * (4 + 2 + 2) + pairs * 4)
        flops = 4.0 * 128 * 32 * pairs
        del ws
        return {"workload": "the headline varlen causal prefill, unfused: X = s*QK^T (fp32) and "
                            "A = softmax(X) (bf16) stored in HBM between three kernels",
                "kernel_ms": round(ms, 4), "steps": steps,
                "tflops_alg": round(flops / (ms * 1e-3) / 1e12, 2),
                "xa_bytes": xa_bytes, "xa_gbs": round(xa_bytes / (ms * 1e-3) / 1e9, 1),
                "fused_kernel_ms": round(fused_ms, 4), "fused_speedup": round(ms / fused_ms, 2)}
    return go


def host_threads() -> int:
    """CPU threads this process may use (its affinity mask, capped by
    OMP_NUM_THREADS when that is set)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(n, 1)


def cpu_baseline_prefill(vl, seconds: float):
    """Oracle on a bounded, seeded sample of (token, head) rows, time-boxed
    to about `seconds`; TFLOP/s from the same algorithmic flop count."""
    import numpy as np
    import oracle
    q = vl.q.float().numpy()
    k = vl.k.float().numpy()
    v = vl.v.float().numpy()
    cu_q = vl.cu_seqlens_q.numpy()
    cu_k = vl.cu_seqlens_k.numpy()
    hq = q.shape[1]
    total = q.shape[0] * hq
    rng = np.random.default_rng(2024)
    order = rng.permutation(total)
    threads = host_threads()
    oracle.attn_varlen(q, k, v, cu_q, cu_k, vl.softmax_scale, True, rows=order[:64], threads=threads)
    done, flops, t_used, batch = 0, 0.0, 0.0, 256
    seq_of = np.searchsorted(cu_q, np.arange(q.shape[0]), side="right") - 1
    while t_used < seconds and done < total:
        rows = order[done:done + batch]
        t0 = time.perf_counter()
        oracle.attn_varlen(q, k, v, cu_q, cu_k, vl.softmax_scale, True, rows=rows, threads=threads)
        t_used += time.perf_counter() - t0
        tok = rows // hq
        b = seq_of[tok]
        i = tok - cu_q[b]
        lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        nvis = np.clip(lk - lq + i + 1, 0, lk)
        flops += float(4.0 * q.shape[2] * nvis.sum())
        done += rows.size
        batch = min(batch * 2, 8192)
    return dict(value=flops / t_used / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                sample=f"{done} of {total} (token, head) rows drawn at random (seed 2024) from the "
                       f"varlen prefill workload, fp64 3-pass oracle, {t_used:.1f} s wall")


OTHER_PREFILL = ("long", "prefix", "shared")


def prep_other_prefill(args, torch, attn, workloads):
    """Inputs of the 32K-sequence, prefix-cache and shared-prompt prefill
    workloads; returns {workload: timing run} (a few timed steps each)."""
    import copy
    runs = {}
    for w in OTHER_PREFILL:
        a2 = copy.copy(args)
        a2.prefill_workload, a2.steps, a2.warmup = w, max(1, min(args.steps, 20)), max(1, min(args.warmup, 3))
        runs[w] = (a2, prep_prefill(a2, torch, attn, workloads))
    return runs


def other_prefill_entry(args, w, a2, r):
    """The bench-line object of one of the other prefill workloads."""
    e = {"workload": PREFILL_WORKLOADS[w].replace("bf16", args.dtype), "steps": a2.steps,
         "algorithmic_flops": r["flops"], "kernel_ms": round(r["kernel_ms"], 4),
         "tflops": round(r["tflops_kernel"], 2),
         "frac": round(r["tflops_kernel"] / PEAK_BF16_TFLOPS, 4),
         "traffic": recorded_traffic(w) if w in TRAFFIC_FILES and args.dtype == "bf16" else None}
    if "bound_ms" in r:
        # the batch mixes memory- and MFMA-bound sequences: the sum over
        # sequences of max(flops/P, bytes/BW), and the rate it allows
        e["per_sequence_bound"] = {
            "ms": round(r["bound_ms"], 4),
            "tflops": round(r["flops"] / (r["bound_ms"] * 1e-3) / 1e12, 2),
            "frac_of_bound": round(r["bound_ms"] / r["kernel_ms"], 4)}
    if w == "shared":
        e["unique_kv_bytes"] = r["unique_kv_bytes"]
    return e


def cpu_baseline_decode(dc, seconds: float):
    """Oracle decode on seeded random subsets of the batch's sequences (all
    32 query heads of each), time-boxed to about `seconds`; GB/s from the
    same algorithmic byte count (every K and V byte of a sequence once per
    KV head)."""
    import numpy as np
    import oracle
    pg = dc.paged
    q = dc.q.float().numpy()
    k = pg.k_logical.float().numpy()
    v = pg.v_logical.float().numpy()
    cu = pg.cu_seqlens_k.numpy().astype(np.int64)
    B = q.shape[0]
    hkv, d = k.shape[1], k.shape[2]
    rng = np.random.default_rng(2025)
    threads = host_threads()
    t_used, nbytes, nseq, calls = 0.0, 0.0, 0, 0
    while t_used < seconds and calls < 1000:
        sel = np.sort(rng.choice(B, size=min(8, B), replace=False))
        lens = cu[sel + 1] - cu[sel]
        rows = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in sel])
        sub_cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        qs, ks, vs = q[sel], k[rows], v[rows]
        t0 = time.perf_counter()
        oracle.attn_decode(qs, ks, vs, sub_cu, dc.softmax_scale, threads=threads)
        t_used += time.perf_counter() - t0
        nbytes += float(lens.sum()) * hkv * d * 2 * 2
        nseq += sel.size
        calls += 1
    return dict(value=nbytes / t_used / 1e9, unit="GB/s", cores=threads, kind="oracle",
                sample=f"{calls} seeded draws (seed 2025) of 8 of the {B} sequences, all 32 query heads "
                       f"each ({nseq} sequence-calls), fp64 oracle decode, {t_used:.1f} s wall")


def _read_sclk_mhz():
    """Current GPU clock(s) in MHz from amd-smi (one value per XCD, averaged)
    or else rocm-smi; None if neither gives a reading."""
    import re
    import shutil
    import statistics
    import subprocess
    amd = shutil.which("amd-smi") or ("/opt/rocm/bin/amd-smi" if os.path.exists("/opt/rocm/bin/amd-smi") else None)
    if amd:
        try:
            out = subprocess.run([amd, "metric", "--clock", "--json"], capture_output=True, text=True,
                                 timeout=20).stdout
            j = json.loads(out[out.index("{") if out.lstrip().startswith("{") else out.index("["):])
            gpus = j.get("gpu_data", j) if isinstance(j, dict) else j
            clocks = gpus[0]["clock"]
            vals = [float(v["clk"]["value"]) for k, v in clocks.items()
                    if k.startswith("gfx") and isinstance(v, dict) and isinstance(v.get("clk"), dict)]
            if vals:
                return statistics.mean(vals)
        except Exception:
            pass
    smi = shutil.which("rocm-smi") or ("/opt/rocm/bin/rocm-smi" if os.path.exists("/opt/rocm/bin/rocm-smi") else None)
    if smi:
        try:
            out = subprocess.run([smi, "-g", "--json"], capture_output=True, text=True, timeout=20).stdout
            j = json.loads(out[out.index("{"):])
            for card in j.values():
                for key, val in (card.items() if isinstance(card, dict) else []):
                    m = re.search(r"\((\d+)\s*mhz\)", str(val), re.I)
                    if "sclk" in key.lower() and m:
                        return float(m.group(1))
        except Exception:
            pass
    return None


def sample_sclk_mhz(torch, enqueue, seconds=3.0):
    """The GPU clock under load: keep the GPU busy with `enqueue()` launches
    for about `seconds` while a helper thread reads the current clock (MHz;
    median of the readings taken while the work runs), or None."""
    import statistics
    import threading
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    enqueue()
    e1.record()
    e1.synchronize()
    per = max(e0.elapsed_time(e1) * 1e-3, 1e-4)
    readings, done = [], threading.Event()

    def reader():
        time.sleep(0.3)
        while not done.is_set() and len(readings) < 4:
            v = _read_sclk_mhz()
            if v is None or done.is_set():
                return                     # no tool, or the work ended mid-reading
            readings.append(v)

    th = threading.Thread(target=reader, daemon=True)
    th.start()
    # batches of ~50 ms of work, at most two in flight: the GPU stays busy
    # without the host queueing far ahead of it
    t_end = time.perf_counter() + seconds
    prev = None
    while time.perf_counter() < t_end and (th.is_alive() or not readings):
        for _ in range(max(1, int(0.05 / per))):
            enqueue()
        ev = torch.cuda.Event()
        ev.record()
        if prev is not None:
            prev.synchronize()
        prev = ev
        if not th.is_alive():
            break
    torch.cuda.synchronize()
    done.set()
    th.join(timeout=30)
    return round(statistics.median(readings)) if readings else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--skip-cpu", action="store_true", help="omit the CPU oracle baseline")
    ap.add_argument("--only", choices=["all", "prefill", "decode", "unfused"], default="all")
    ap.add_argument("--dtype", choices=["bf16", "fp16"], default="bf16",
                    help="16-bit input (and output) type of every workload")
    ap.add_argument("--skip-other-prefill", action="store_true",
                    help="omit the 32K-sequence and prefix-cache prefill timings of the default run")
    ap.add_argument("--skip-unfused", action="store_true",
                    help="omit the unfused three-kernel baseline (it needs ~52 GB of workspace)")
    ap.add_argument("--prefill-workload", choices=["varlen", "long", "noncausal", "prefix", "shared"],
                    default="varlen",
                    help="prefill workload to time: the varlen 16-sequence batch (headline), the "
                         "32768-token single sequence, the varlen batch without the causal mask, "
                         "the 32-sequence prefix-cache batch through the paged cache, or the "
                         "32-sequence batch sharing a cached 2048-token prompt")
    ap.add_argument("--decode-workload", choices=["random", "shared"], default="random",
                    help="decode workload of --only decode: the batch-64 random-context pool "
                         "(headline) or the batch-64 pool sharing a 2048-token prompt")
    ap.add_argument("--skip-clock", action="store_true", help="omit the sclk reading under load")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain elementwise copy of 1 GiB (read 1 GiB, write 1 GiB), "
                         "the reference for scaling the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU; --gpus {args.gpus} is not supported "
              "(the attention path would shard by KV head or by sequence, with no exchange "
              "between GPUs)", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_sdpa_amd as attn
    import workloads
    args.torch_dtype = torch.float16 if args.dtype == "fp16" else torch.bfloat16

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    attn.load_library()
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = (1 << 30) // 4
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            torch.mul(x, 1.0, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "elementwise copy", "bytes_read": 4 * n,
                          "bytes_written": 4 * n, "launches": 3}), flush=True)
        return

    # Every workload's inputs are built (on the CPU, then copied) before any
    # timing, and the timed sections then run back to back.  After idle
    # time -- such as the seconds the CPU spends building a workload -- the
    # GPU's first ~30 launches run at a lower clock (measured: the varlen
    # kernel ramps from ~720 to ~970 TFLOP/s over its first ~25 ms), which a
    # few milliseconds of warm-up steps do not cover.  The 32K prefill runs
    # first and brings the GPU to its working clock.  W and K are unchanged.
    want_other = args.only == "all" and args.prefill_workload == "varlen" and not args.skip_other_prefill
    want_unfused = args.only in ("all", "prefill", "unfused") and args.prefill_workload == "varlen" and \
        not args.skip_unfused and args.dtype == "bf16"
    other_runs = prep_other_prefill(args, torch, attn, workloads) if want_other else {}
    head_run = prep_prefill(args, torch, attn, workloads) if args.only in ("all", "prefill") else None
    unf_run = prep_unfused(args, torch, attn, workloads) if want_unfused else None
    dec_run = dsh_run = None
    if args.only in ("all", "decode"):
        dec_run = prep_decode(args, torch, attn, workloads,
                              shared=args.only == "decode" and args.decode_workload == "shared")
        if args.only == "all":
            import copy
            a_sh = copy.copy(args)
            a_sh.steps, a_sh.warmup = max(1, min(args.steps, 20)), max(1, min(args.warmup, 3))
            dsh_run = prep_decode(a_sh, torch, attn, workloads, shared=True)
    torch.cuda.synchronize()

    res = {}
    if other_runs:
        other = {}
        for w, (a2, go) in other_runs.items():
            r = go()
            other[w] = other_prefill_entry(args, w, a2, r)
            print(f"[bench] {w} prefill kernel {r['kernel_ms']:.3f} ms, {r['tflops_kernel']:.1f} TFLOP/s",
                  file=sys.stderr, flush=True)
        res["other_prefill"] = other
    if head_run is not None:
        pre = head_run()
        print(f"[bench] prefill step {pre['ms_step']:.3f} ms, kernel {pre['kernel_ms']:.3f} ms, "
              f"{pre['tflops_kernel']:.1f} TFLOP/s kernel", file=sys.stderr, flush=True)
        res["prefill"] = pre
    if unf_run is not None:
        fused_ms = res["prefill"]["kernel_ms"] if "prefill" in res else float("nan")
        unf = unf_run(fused_ms)
        print(f"[bench] unfused baseline {unf['kernel_ms']:.3f} ms "
              f"(fused kernel {fused_ms:.3f} ms), X/A traffic {unf['xa_gbs']:.0f} GB/s",
              file=sys.stderr, flush=True)
        res["unfused"] = unf
    if dec_run is not None:
        dec = dec_run()
        print(f"[bench] decode step {dec['ms_step']:.3f} ms, kernels {dec['kernel_ms']:.3f} ms, "
              f"{dec['gbs_kernel']:.0f} GB/s", file=sys.stderr, flush=True)
        res["decode"] = dec
        if dsh_run is not None:
            ds = dsh_run()
            print(f"[bench] shared-prompt decode kernels {ds['kernel_ms']:.3f} ms, {ds['gbs_kernel']:.0f} GB/s",
                  file=sys.stderr, flush=True)
            res["decode_shared"] = ds
    sclk = None
    if not args.skip_clock and "prefill" in res and "enqueue" in res["prefill"]:
        sclk = sample_sclk_mhz(torch, res["prefill"]["enqueue"])

    line = {
        "metric": "prefill attn TFLOP/s (% MFMA peak); paged decode KV GB/s (% HBM peak)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": args.dtype, "data": "synthetic (seeded; no dataset or weights involved)",
    }
    if "prefill" in res:
        pre = res["prefill"]
        line.update({
            "value": round(pre["tflops_step"], 2), "unit": "TFLOP/s",
            "ms_per_step": round(pre["ms_step"], 4),
            "config": {"workload": PREFILL_WORKLOADS[args.prefill_workload].replace("bf16", args.dtype),
                       "total_tokens": pre["total_tokens"], "algorithmic_flops": pre["flops"],
                       "step": "kv_store_slots + attn_prefill_varlen"},
            "roofline": {"bound": "mfma", "achieved": round(pre["tflops_kernel"], 2),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(pre["tflops_kernel"] / PEAK_BF16_TFLOPS, 4),
                         "traffic": recorded_traffic(args.prefill_workload)
                         if args.prefill_workload in TRAFFIC_FILES and args.dtype == "bf16" else None,
                         "kernel": f"prefill_mfma_kernel<{args.dtype}, true>",
                         "kernel_ms": round(pre["kernel_ms"], 4)},
        })
    if "decode" in res:
        dec = res["decode"]
        dobj = {"workload": "paged decode: batch 64, contexts U[512,8192], block 256, permuted "
                            f"pool, 32 Q / 8 KV heads, head_dim 128, {args.dtype}, new token stored first",
                "metric": "KV GB/s", "value": round(dec["gbs_step"], 1),
                "ms_per_step": round(dec["ms_step"], 4),
                "kv_bytes": dec["kv_bytes"],
                "roofline": {"bound": "hbm", "achieved": round(dec["gbs_kernel"], 1),
                             "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(dec["gbs_kernel"] / PEAK_HBM_GBS, 4),
                             "traffic": recorded_traffic("decode")
                             if args.dtype == "bf16" and not dec["dc"].name.startswith("shared") else None,
                             "kernel": f"decode_split_kernel<{args.dtype}, 128> + decode_combine_kernel<{args.dtype}, 128>",
                             "kernel_ms": round(dec["kernel_ms"], 4)}}
        if dec["dc"].name.startswith("shared"):
            dobj["workload"] = SHARED_DECODE + f", {args.dtype}"
        if not args.skip_cpu:
            dobj["cpu_baseline"] = cpu_baseline_decode(dec["dc"], min(args.cpu_seconds, 10.0))
        if "decode_shared" in res:
            ds = res["decode_shared"]
            dobj["shared_prompt"] = {
                "workload": SHARED_DECODE + f", {args.dtype}",
                "kv_bytes": ds["kv_bytes"], "unique_kv_bytes": ds["unique_kv_bytes"],
                "kernel_ms": round(ds["kernel_ms"], 4), "gbs": round(ds["gbs_kernel"], 1),
                "frac": round(ds["gbs_kernel"] / PEAK_HBM_GBS, 4)}
        if "prefill" in res:
            line["decode"] = dobj
        else:
            line.update({"value": dobj["value"], "unit": "GB/s", "ms_per_step": dobj["ms_per_step"],
                         "config": {"workload": dobj["workload"]},
                         "roofline": dobj["roofline"]})
    props = torch.cuda.get_device_properties(0)
    line["env"] = {"device": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
                   "compute_units": props.multi_processor_count, "hip": torch.version.hip,
                   "torch": torch.__version__,
                   # rocm-smi's current sclk while the headline prefill kernel runs back to back
                   "sclk_mhz_under_load": sclk,
                   "peak_basis": "bf16 dense MFMA 2.5 PFLOP/s = 256 CU x 4096 flop/clk x 2.4 GHz "
                                 "(nominal clock); HBM 8 TB/s"}
    if "unfused" in res:
        line["unfused_baseline"] = res["unfused"]
    if "other_prefill" in res:
        line["other_prefill"] = res["other_prefill"]
    if not args.skip_cpu and "prefill" in res and res["prefill"]["vl"] is not None:
        line["cpu_baseline"] = cpu_baseline_prefill(res["prefill"]["vl"], args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
