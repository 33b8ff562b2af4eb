"""GPU parity of attn_prefill_varlen against the fp64 oracle.

Small cases are compared element by element on every output; the full-size
workloads are compared on sampled rows the oracle computes one by one, in
the same launch configuration the benchmark times.  Pages: blog post
"从零实现 vLLM (1.3)：如何加速 Attention 计算" (sections Prefill, FlashAttention
的最终实现, 计算流程(1-Pass 算法与分块))."""
import numpy as np
import pytest
import torch

import attention_sdpa_amd as attn
import oracle
import workloads
from tests.helpers import (check_bf16, check_bf16_output, check_f16, check_f32, dev, log, np32,
                           oracle_varlen, sample_rows, unit_rows)

pytestmark = pytest.mark.gpu


def run_varlen(vl, out_dtype=torch.float32, causal=None):
    out = attn.attn_prefill_varlen(dev(vl.q), dev(vl.k), dev(vl.v), dev(vl.cu_seqlens_q),
                                   dev(vl.cu_seqlens_k), vl.max_seqlen_q, vl.max_seqlen_k,
                                   vl.softmax_scale, vl.causal if causal is None else causal,
                                   out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


# ---------------------------------------------------------------- fp32 path

def test_fp32_single_head_L256_d64():
    vl = workloads.fp32_single_head()
    log(f"case {vl.name}")
    got = run_varlen(vl)
    check_f32(np32(got), oracle_varlen(vl), vl.name)


def test_fp32_stress_logits_near_700():
    vl = workloads.fp32_stress()
    log(f"case {vl.name}")
    got = np32(run_varlen(vl))
    ref = oracle_varlen(vl)
    check_f32(got, ref, vl.name)
    # row 2 is the [700, 710, 705] example's weights applied to V rows 0..2
    w = np.exp(np.array([-10.0, 0.0, -5.0]))
    w /= w.sum()
    assert np.max(np.abs(got[2, 0] - w @ np32(vl.v)[:3, 0].astype(np.float64))) <= 1e-5


@pytest.mark.parametrize("d", [64, 128])
def test_fp32_varlen_gqa_ragged(d):
    vl = workloads.varlen([1, 130, 7, 64, 200], [1, 130, 7, 64, 200], 4, 2, d, torch.float32,
                          seed=5 + d)
    log(f"case fp32 varlen gqa d={d}")
    check_f32(np32(run_varlen(vl)), oracle_varlen(vl), f"fp32 d{d}")


def test_fp32_prefix_and_noncausal():
    vl = workloads.varlen([3, 40, 1], [50, 40, 9], 2, 1, 64, torch.float32, seed=8)
    log("case fp32 Lq<Lk end-aligned")
    check_f32(np32(run_varlen(vl)), oracle_varlen(vl), "fp32 prefix")
    vl.causal = False
    check_f32(np32(run_varlen(vl)), oracle_varlen(vl), "fp32 non-causal")


# ---------------------------------------------------------------- bf16 path

RAGGED = [1, 31, 32, 33, 63, 64, 65, 127, 129, 257, 500]


@pytest.mark.parametrize("hq,hkv", [(32, 8), (8, 8), (4, 2), (16, 2), (6, 2)])
def test_bf16_varlen_ragged(hq, hkv):
    vl = workloads.varlen(RAGGED, RAGGED, hq, hkv, 128, torch.bfloat16, seed=hq * 10 + hkv)
    log(f"case bf16 varlen ragged hq={hq} hkv={hkv}")
    check_bf16(np32(run_varlen(vl)), oracle_varlen(vl), f"bf16 ragged {hq}/{hkv}")


def test_bf16_output_dtype():
    vl = workloads.varlen([77, 300, 5], [77, 300, 5], 8, 2, 128, torch.bfloat16, seed=3)
    log("case bf16 output")
    got = run_varlen(vl, out_dtype=torch.bfloat16)
    assert got.dtype == torch.bfloat16
    check_bf16_output(got, oracle_varlen(vl), "bf16 out")


def test_bf16_end_aligned_causal_and_noncausal():
    lq = [1, 17, 64, 100, 3, 40]
    lk = [300, 17, 200, 100, 1, 0]   # includes Lq > Lk (rows see no key) and Lk = 0
    vl = workloads.varlen(lq, lk, 8, 2, 128, torch.bfloat16, seed=4)
    log("case bf16 Lq<=Lk end-aligned, empty K")
    got = np32(run_varlen(vl))
    ref = oracle_varlen(vl)
    check_bf16(got, ref, "bf16 end-aligned")
    # rows that see no key are exactly zero
    cu = vl.cu_seqlens_q.tolist()
    assert np.all(got[cu[4]:cu[4] + 2] == 0) and np.all(got[cu[5]:cu[6]] == 0)
    vl.causal = False
    check_bf16(np32(run_varlen(vl)), oracle_varlen(vl), "bf16 non-causal")


def test_bf16_empty_sequences():
    vl = workloads.varlen([0, 50, 0, 3], [0, 50, 10, 3], 4, 4, 128, torch.bfloat16, seed=6)
    log("case bf16 empty sequences")
    check_bf16(np32(run_varlen(vl)), oracle_varlen(vl), "bf16 empty seqs")


def test_bf16_many_sequences():
    """More sequences than the per-workgroup schedule tables hold (1100 >
    1024), so the launch takes the strided unit schedule; lengths include 0."""
    g = np.random.default_rng(11)
    lens = g.integers(0, 41, size=1100)
    lens[::97] = 0
    vl = workloads.varlen(lens, lens, 4, 2, 128, torch.bfloat16, seed=12)
    log("case bf16 1100 sequences (strided schedule)")
    check_bf16(np32(run_varlen(vl)), oracle_varlen(vl), "bf16 1100 seqs")


def test_bf16_loose_max_seqlen():
    """max_seqlen_q / max_seqlen_k far above every actual length: the
    schedule must skip the rows no sequence reaches."""
    vl = workloads.varlen([130, 7, 64, 65], [130, 7, 64, 65], 8, 2, 128, torch.bfloat16, seed=13)
    log("case bf16 loose max_seqlen")
    out = attn.attn_prefill_varlen(dev(vl.q), dev(vl.k), dev(vl.v), dev(vl.cu_seqlens_q),
                                   dev(vl.cu_seqlens_k), 5000, 5000, vl.softmax_scale, True,
                                   out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_bf16(np32(out), oracle_varlen(vl), "bf16 loose max_seqlen")


def test_bf16_one_hot_logits_exact():
    """Logit gap > 100 after scaling: the output equals V of the target key
    to bf16 precision of the inputs (weights are 1 and ~e^-100)."""
    L, d = 70, 128
    q = torch.zeros(L, 1, d)
    q[:, 0, 0] = 1.0
    k = torch.zeros(L, 1, d)
    k[:, 0, 0] = -64.0
    k[5, 0, 0] = 64.0
    g = torch.Generator().manual_seed(2)
    v = torch.randn(L, 1, d, generator=g)
    cu = torch.tensor([0, L], dtype=torch.int32)
    vl = workloads.Varlen(q.bfloat16(), k.bfloat16(), v.bfloat16(), cu, cu.clone(), L, L, 1.0, False)
    log("case bf16 one-hot")
    got = np32(run_varlen(vl))
    assert np.array_equal(got[:, 0], np.broadcast_to(np32(vl.v)[5, 0], (L, d)))


def rising_logits(lens, hq, hkv, d, slope, seed, dtype=torch.bfloat16):
    """Packed bf16 q/k/v whose logits grow by about `slope` per key along
    each sequence (feature 0 of every query is 16, of key j about
    j * slope / (16 * scale)), plus N(0, 1/4) noise in the other features."""
    scale = d ** -0.5
    g = torch.Generator().manual_seed(seed)
    T = sum(lens)
    q = torch.randn(T, hq, d, generator=g) * 0.5
    k = torch.randn(T, hkv, d, generator=g) * 0.5
    v = torch.randn(T, hkv, d, generator=g)
    q[:, :, 0] = 16.0
    pos = torch.cat([torch.arange(L, dtype=torch.float32) for L in lens])
    k[:, :, 0] = (pos * slope / (16.0 * scale))[:, None]
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    return q.to(dtype), k.to(dtype), v.to(dtype), cu, scale


@pytest.mark.parametrize("causal", [True, False])
def test_bf16_rising_logits_rescale_every_tile(causal):
    """Logits rising by ~1 per key, 64 per 64-key tile: past the lazy
    reference's threshold (a scaled rise of 8, 8 / (scale log2 e) ~ 63 logit
    units at d = 128), so the reference and o', d' are rescaled on nearly
    every tile, also while P V products of the step are still in flight."""
    lens = [1000, 333, 700]
    q, k, v, cu, scale = rising_logits(lens, 16, 4, 128, 1.0, 31)
    vl = workloads.Varlen(q, k, v, cu, cu.clone(), max(lens), max(lens), scale, causal)
    log(f"case bf16 rising logits causal={causal}")
    got = np32(run_varlen(vl))
    check_bf16(got, oracle_varlen(vl), f"rising logits causal={causal}")


def test_f16_rising_logits_rescale_every_tile():
    """The same rising logits with fp16 inputs (fp16 weights P, up to 2^8)."""
    lens = [1000, 333, 700]
    q, k, v, cu, scale = rising_logits(lens, 16, 4, 128, 1.0, 37, torch.float16)
    vl = workloads.Varlen(q, k, v, cu, cu.clone(), max(lens), max(lens), scale, True)
    log("case fp16 rising logits")
    check_f16(np32(run_varlen(vl)), oracle_varlen(vl), "fp16 rising logits")


# ---------------------------------------------------------------- paged (prefix cache)

def run_prefix(pp, out_dtype=torch.float32, store=True):
    pg = pp.paged
    kc, vc = dev(pg.k_cache), dev(pg.v_cache)
    if store:
        attn.kv_store_slots(dev(pg.k_new), dev(pg.v_new), kc, vc, dev(pg.slot_mapping))
    out = attn.attn_prefill_varlen(dev(pp.q), kc, vc, dev(pp.cu_seqlens_q), dev(pg.cu_seqlens_k),
                                   pp.max_seqlen_q, pp.max_seqlen_k, pp.softmax_scale, True,
                                   block_table=dev(pg.block_table), out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


def oracle_prefix(pp, rows=None):
    pg = pp.paged
    return oracle.attn_varlen(np32(pp.q), np32(pg.k_logical), np32(pg.v_logical),
                              pp.cu_seqlens_q.numpy(), pg.cu_seqlens_k.numpy(), pp.softmax_scale,
                              True, rows=rows)


@pytest.mark.parametrize("block_size", [64, 256])
def test_bf16_prefix_prefill_paged(block_size):
    pp = workloads.prefix_prefill(n_seqs=6, q_lo=1, q_hi=150, p_lo=0, p_hi=700, hq=8, hkv=2,
                                  block_size=block_size, seed=21 + block_size)
    log(f"case bf16 prefix paged bs={block_size}")
    check_bf16(np32(run_prefix(pp)), oracle_prefix(pp), f"prefix bs{block_size}")


def test_bf16_prefix_long_context():
    """New tokens on cached prefixes of 60K-100K tokens: units that stream
    ~1,500 K/V tiles through the block table."""
    pp = workloads.prefix_prefill(n_seqs=2, q_lo=1, q_hi=40, p_lo=60000, p_hi=100000, hq=32, hkv=8,
                                  block_size=256, seed=27)
    log("case bf16 prefix prefill, 60K-100K cached tokens")
    check_bf16(np32(run_prefix(pp)), oracle_prefix(pp), "prefix long context")


def test_bf16_shared_prefix_blocks():
    """Block tables that share their first physical blocks (one cached prompt
    read by every sequence; the page-table picture of the Prefill section has
    two sequences pointing at the same block) give the oracle's result for the
    logical per-sequence K/V."""
    pp = workloads.shared_prefix_prefill(n_seqs=6, shared_blocks=3, own_lo=0, own_hi=300,
                                         q_lo=1, q_hi=150, hq=8, hkv=2, block_size=64, seed=31)
    assert (pp.paged.block_table[:, :3] == pp.paged.block_table[0, :3]).all()
    log("case bf16 shared prefix blocks")
    check_bf16(np32(run_prefix(pp)), oracle_prefix(pp), "shared prefix")


def test_paged_block_permutation_bit_identical():
    """The same logical K/V laid out in two differently permuted pools gives
    bit-identical outputs (arithmetic order depends on logical positions only),
    and an identity block table equals the contiguous path bit for bit."""
    base = workloads.varlen([40, 300, 129], [300, 300, 500], 8, 2, 128, torch.bfloat16, seed=9)
    outs = []
    for seed in (1, 2):
        pg = workloads.paged_pool(base.k, base.v, base.cu_seqlens_k, [0, 0, 0], 64, seed=seed,
                                  spare_blocks=5)
        pp = workloads.PrefixPrefill(base.q, base.cu_seqlens_q, base.max_seqlen_q, base.max_seqlen_k,
                                     base.softmax_scale, pg)
        outs.append(run_prefix(pp))
    log("case permutation invariance")
    assert torch.equal(outs[0], outs[1])
    contiguous = run_varlen(base)
    assert torch.equal(outs[0], contiguous)


def test_fp32_paged_matches_oracle():
    base = workloads.varlen([5, 70], [90, 70], 2, 2, 64, torch.float32, seed=10)
    pg = workloads.paged_pool(base.k, base.v, base.cu_seqlens_k, [80, 0], 16, seed=3)
    pp = workloads.PrefixPrefill(base.q, base.cu_seqlens_q, base.max_seqlen_q, base.max_seqlen_k,
                                 base.softmax_scale, pg)
    log("case fp32 paged")
    check_f32(np32(run_prefix(pp)), oracle_prefix(pp), "fp32 paged")


def test_bf16_paged_many_sequences():
    """Paged K/V with more sequences than the schedule tables hold (1100 >
    1024): the launch takes the strided unit schedule through the block
    table; cached prefixes include empty ones."""
    pp = workloads.prefix_prefill(n_seqs=1100, q_lo=1, q_hi=24, p_lo=0, p_hi=90, hq=4, hkv=2,
                                  block_size=64, seed=91)
    log("case bf16 paged 1100 sequences (strided schedule)")
    check_bf16(np32(run_prefix(pp)), oracle_prefix(pp), "bf16 paged 1100 seqs")


def bad_block_case(pp, picks):
    """Block table with the (sequence, block index, id) picks applied, and the
    list of (first row, end row) logical ranges they cover."""
    pg = pp.paged
    bt = pg.block_table.clone()
    cu = pg.cu_seqlens_k.tolist()
    bs = pg.block_size
    ranges = []
    for b, i, blk in picks:
        assert cu[b] + bs * i < cu[b + 1], "the pick must be one of the sequence's blocks"
        bt[b, i] = blk
        ranges.append((b, i, cu[b] + bs * i, min(cu[b] + bs * (i + 1), cu[b + 1])))
    return bt, ranges


def test_fp32_paged_block_ids_outside_the_pool():
    """fp32 prefill: a block id outside [0, num_blocks) reads as zero rows."""
    pp = workloads.prefix_prefill(n_seqs=4, q_lo=5, q_hi=40, p_lo=60, p_hi=200, hq=4, hkv=2, d=64,
                                  block_size=16, seed=81, dtype=torch.float32)
    pg = pp.paged
    nb = pg.num_blocks
    bt, ranges = bad_block_case(pp, [(0, 0, -1), (1, 2, nb), (3, 1, nb + 4)])
    k, v = pg.k_logical.clone(), pg.v_logical.clone()
    for _, _, lo, hi in ranges:
        k[lo:hi] = 0
        v[lo:hi] = 0
    kc, vc = dev(pg.k_cache), dev(pg.v_cache)
    attn.kv_store_slots(dev(pg.k_new), dev(pg.v_new), kc, vc, dev(pg.slot_mapping))
    log("case fp32 paged block ids outside the pool")
    got = attn.attn_prefill_varlen(dev(pp.q), kc, vc, dev(pp.cu_seqlens_q), dev(pg.cu_seqlens_k),
                                   pp.max_seqlen_q, pp.max_seqlen_k, pp.softmax_scale, True,
                                   block_table=dev(bt), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.attn_varlen(np32(pp.q), np32(k), np32(v), pp.cu_seqlens_q.numpy(),
                             pg.cu_seqlens_k.numpy(), pp.softmax_scale, True)
    check_f32(np32(got), ref, "fp32 paged bad block ids")


def test_bf16_paged_block_ids_outside_the_pool():
    """Matrix-core prefill: a block id outside [0, num_blocks) is read as
    physical block 0 (the access stays inside the cache), and sequences whose
    tables are valid are unaffected."""
    pp = workloads.prefix_prefill(n_seqs=6, q_lo=20, q_hi=150, p_lo=200, p_hi=700, hq=8, hkv=2,
                                  block_size=64, seed=71)
    pg = pp.paged
    nb = pg.num_blocks
    bt, ranges = bad_block_case(pp, [(1, 0, -1), (1, 3, nb), (4, 1, nb + 9), (5, 2, -7)])
    kc, vc = dev(pg.k_cache), dev(pg.v_cache)
    attn.kv_store_slots(dev(pg.k_new), dev(pg.v_new), kc, vc, dev(pg.slot_mapping))
    # slots of block 0 that no sequence uses hold the NaN sentinel; give them
    # finite values (no valid table reaches them)
    kc[0] = torch.nan_to_num(kc[0], nan=0.25)
    vc[0] = torch.nan_to_num(vc[0], nan=-0.5)
    k0, v0 = kc[0].cpu(), vc[0].cpu()
    k, v = pg.k_logical.clone(), pg.v_logical.clone()
    for _, _, lo, hi in ranges:
        k[lo:hi] = k0[:hi - lo]
        v[lo:hi] = v0[:hi - lo]
    log("case bf16 paged block ids outside the pool")
    got = attn.attn_prefill_varlen(dev(pp.q), kc, vc, dev(pp.cu_seqlens_q), dev(pg.cu_seqlens_k),
                                   pp.max_seqlen_q, pp.max_seqlen_k, pp.softmax_scale, True,
                                   block_table=dev(bt), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.attn_varlen(np32(pp.q), np32(k), np32(v), pp.cu_seqlens_q.numpy(),
                             pg.cu_seqlens_k.numpy(), pp.softmax_scale, True)
    check_bf16(np32(got), ref, "bf16 paged bad block ids")


# ---------------------------------------------------------------- full-size workloads
# The benchmark's workloads in the benchmark's launch configuration (bf16
# output), and again with fp32 output; the varlen and prefix-cache batches
# are compared on every output row, the 32K sequence on every row of every
# 16th (query block, KV head) unit spread over the sequence and all KV heads.

def check_both(got_f32, got_bf16, ref, what):
    """fp32 output to the method's tolerance, bf16 output (the one the
    benchmark times) to the same tolerance plus its own rounding."""
    check_bf16(np32(got_f32).reshape(ref.shape), ref, f"{what} fp32 out")
    check_bf16_output(got_bf16.reshape(ref.shape), ref, f"{what} bf16 out")


def test_full_varlen_prefill_16_seqs():
    vl = workloads.varlen_prefill()
    log(f"case {vl.name} total_q={vl.q.shape[0]} (every row)")
    got32 = run_varlen(vl)
    got16 = run_varlen(vl, out_dtype=torch.bfloat16)
    ref = oracle_varlen(vl)
    check_both(got32, got16, ref, "varlen 16 seqs (all rows)")


def test_full_long_prefill_32k():
    vl = workloads.long_prefill()
    rows = unit_rows(vl.q.shape[0], 32, 8, every=16)
    log(f"case {vl.name}: {rows.size} rows = every 16th (query block, KV head) unit")
    got32 = np32(run_varlen(vl)).reshape(-1, 128)[rows]
    got16 = run_varlen(vl, out_dtype=torch.bfloat16).reshape(-1, 128)[torch.from_numpy(rows).cuda()]
    ref = oracle_varlen(vl, rows=rows)
    check_bf16(got32, ref, "long 32k (1/16 of the units) fp32 out")
    check_bf16_output(got16, ref, "long 32k (1/16 of the units) bf16 out")


def test_full_prefix_prefill_32_seqs():
    pp = workloads.prefix_prefill()
    log(f"case {pp.name} (every row)")
    got32 = run_prefix(pp)
    got16 = run_prefix(pp, out_dtype=torch.bfloat16)
    ref = oracle_prefix(pp)
    check_both(got32, got16, ref, "prefix 32 seqs (all rows)")
