"""Seeded random shapes against the fp64 oracle: batch sizes, ragged and
empty sequences, GQA ratios (including groups of 1, 3, 5, 6 and 16),
causal and non-causal, end-aligned key ranges longer than the queries,
contiguous and paged K/V with several block sizes, fp32 and 16-bit
output, and decode item sizes.  Each draw is logged before it runs, so a
failure names its case.  Pages: blog post "从零实现 vLLM (1.3)：如何加速
Attention 计算", sections Prefill and Decode."""
import numpy as np
import pytest
import torch

import attention_sdpa_amd as attn
import oracle
import workloads
from tests.helpers import check_bf16, check_bf16_output, dev, log, np32

pytestmark = pytest.mark.gpu

HEADS = [(8, 8), (16, 4), (12, 3), (10, 2), (6, 1), (9, 3), (32, 8), (64, 4), (16, 16)]


def draw_lengths(rng, n, lo, hi, p_zero=0.1):
    lens = rng.integers(lo, hi + 1, size=n)
    lens[rng.random(n) < p_zero] = 0
    return [int(x) for x in lens]


def check(got, ref, out16, what):
    if out16:
        check_bf16_output(got, ref, what)
    else:
        check_bf16(np32(got), ref, what)


@pytest.mark.parametrize("seed", range(16))
def test_random_prefill(seed):
    rng = np.random.default_rng(5000 + seed)
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    B = int(rng.integers(1, 20))
    lq = draw_lengths(rng, B, 1, 500)
    lq[0] = max(lq[0], 1)
    extra = rng.integers(0, 300, size=B) if rng.random() < 0.5 else np.zeros(B, dtype=np.int64)
    lk = [q + int(e) for q, e in zip(lq, extra)]
    # bound the oracle's work (query-key pairs times heads) to a few seconds
    while sum(q * k for q, k in zip(lq, lk)) * hq > 4e7:
        half = [max(q // 2, 1 if q else 0) for q in lq]
        lk = [h + (k - q) // 2 for h, q, k in zip(half, lq, lk)]
        lq = half
    causal = bool(rng.random() < 0.75)
    paged = bool(rng.random() < 0.5)
    out16 = bool(rng.random() < 0.5)
    bs = int(rng.choice([64, 128, 256]))
    what = (f"random prefill seed={seed} B={B} heads={hq}/{hkv} causal={causal} "
            f"paged={paged}{f' bs={bs}' if paged else ''} out={'bf16' if out16 else 'fp32'}")
    log(f"case {what}")
    base = workloads.varlen(lq, lk, hq, hkv, 128, torch.bfloat16, seed=6000 + seed, causal=causal)
    out_dtype = torch.bfloat16 if out16 else torch.float32
    if paged:
        # the cached part of each sequence is its keys before the queries
        pg = workloads.paged_pool(base.k, base.v, base.cu_seqlens_k,
                                  [k - q for q, k in zip(lq, lk)], bs, seed=7000 + seed, spare_blocks=2)
        kc, vc = dev(pg.k_cache), dev(pg.v_cache)
        attn.kv_store_slots(dev(pg.k_new), dev(pg.v_new), kc, vc, dev(pg.slot_mapping))
        got = attn.attn_prefill_varlen(dev(base.q), kc, vc, dev(base.cu_seqlens_q), dev(pg.cu_seqlens_k),
                                       base.max_seqlen_q, base.max_seqlen_k, base.softmax_scale, causal,
                                       block_table=dev(pg.block_table), out_dtype=out_dtype)
    else:
        got = attn.attn_prefill_varlen(dev(base.q), dev(base.k), dev(base.v), dev(base.cu_seqlens_q),
                                       dev(base.cu_seqlens_k), base.max_seqlen_q, base.max_seqlen_k,
                                       base.softmax_scale, causal, out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref = oracle.attn_varlen(np32(base.q), np32(base.k), np32(base.v), base.cu_seqlens_q.numpy(),
                             base.cu_seqlens_k.numpy(), base.softmax_scale, causal)
    check(got, ref, out16, what)


@pytest.mark.parametrize("seed", range(16))
def test_random_decode(seed):
    rng = np.random.default_rng(8000 + seed)
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    hi = int(rng.choice([300, 1500, 4000]))
    # bound the cache the test builds (sequences x keys x KV heads)
    B = int(rng.integers(1, max(2, min(90, int(4e6 // (hi * hkv))))))
    ctx = draw_lengths(rng, B, 1, hi, p_zero=0.05)
    bs = int(rng.choice([64, 128, 256]))
    split = int(rng.choice([0, 0, 32, 64, 96, 256]))
    out16 = bool(rng.random() < 0.5)
    what = (f"random decode seed={seed} B={B} ctx<={hi} heads={hq}/{hkv} bs={bs} split={split} "
            f"out={'bf16' if out16 else 'fp32'}")
    log(f"case {what}")
    base = workloads.varlen([1] * B, ctx, hq, hkv, 128, torch.bfloat16, seed=9000 + seed)
    mbs = max(1, max((c + bs - 1) // bs for c in ctx))
    pg = workloads.paged_pool(base.k, base.v, base.cu_seqlens_k, [max(c - 1, 0) for c in ctx], bs,
                              seed=9500 + seed, spare_blocks=3, max_blocks_per_seq=mbs)
    kc, vc = dev(pg.k_cache), dev(pg.v_cache)
    attn.kv_store_slots(dev(pg.k_new), dev(pg.v_new), kc, vc, dev(pg.slot_mapping))
    q = base.q.view(B, hq, 128)
    got = attn.attn_decode_paged(dev(q), kc, vc, dev(pg.seqlens_k), dev(pg.block_table), base.softmax_scale,
                                 split_tokens=split, out_dtype=torch.bfloat16 if out16 else torch.float32)
    torch.cuda.synchronize()
    ref = oracle.attn_decode(np32(q), np32(pg.k_logical), np32(pg.v_logical), pg.cu_seqlens_k.numpy(),
                             base.softmax_scale)
    check(got, ref, out16, what)
