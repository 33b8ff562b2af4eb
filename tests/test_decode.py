"""GPU parity of attn_decode_paged (after kv_store_slots stores the new
token) against the fp64 oracle, which reads the logical per-sequence K/V,
never the paged pool.  Pages: blog post "从零实现 vLLM (1.3)：如何加速
Attention 计算", section Decode."""
import numpy as np
import pytest
import torch

import attention_sdpa_amd as attn
import oracle
import workloads
from tests.golden import load as load_golden
from tests.helpers import check_bf16, check_bf16_output, dev, log, np32

pytestmark = pytest.mark.gpu


def run_decode(dc, split=0, out_dtype=torch.float32):
    pg = dc.paged
    kc, vc = dev(pg.k_cache), dev(pg.v_cache)
    attn.kv_store_slots(dev(pg.k_new), dev(pg.v_new), kc, vc, dev(pg.slot_mapping))
    out = attn.attn_decode_paged(dev(dc.q), kc, vc, dev(pg.seqlens_k), dev(pg.block_table),
                                 dc.softmax_scale, split_tokens=split, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


def oracle_decode(dc):
    pg = dc.paged
    return oracle.attn_decode(np32(dc.q), np32(pg.k_logical), np32(pg.v_logical),
                              pg.cu_seqlens_k.numpy(), dc.softmax_scale)


def make_decode(ctx, hq=32, hkv=8, block_size=256, seed=0, mbs=None):
    """Decode inputs with explicit context lengths."""
    B = len(ctx)
    base = workloads.varlen([1] * B, ctx, hq, hkv, 128, torch.bfloat16, seed)
    mbs = mbs or max(1, max((c + block_size - 1) // block_size for c in ctx))
    pg = workloads.paged_pool(base.k, base.v, base.cu_seqlens_k, [max(c - 1, 0) for c in ctx],
                              block_size, seed + 1, spare_blocks=2, max_blocks_per_seq=mbs)
    return workloads.Decode(base.q.view(B, hq, 128), base.softmax_scale, pg, f"ctx{ctx}")


@pytest.mark.parametrize("slope", [1.0, -1.0])
@pytest.mark.parametrize("split", [0, 256])
def test_decode_monotone_logits(slope, split):
    """Logits rising (or falling) by ~1 per key along each context: rising,
    every chunk raises the running maximum by ~32 and each run's partial
    carries a maximum far above the previous run's, so the merge scales
    all but the last runs' partials by factors that underflow to 0;
    falling, the first chunk holds the maximum."""
    ctx = [6000, 1, 777, 12000]
    B, hq, hkv, d = len(ctx), 32, 8, 128
    scale = d ** -0.5
    g = torch.Generator().manual_seed(41)
    T = sum(ctx)
    q = torch.randn(B, hq, d, generator=g) * 0.5
    k = torch.randn(T, hkv, d, generator=g) * 0.5
    v = torch.randn(T, hkv, d, generator=g)
    q[:, :, 0] = 16.0
    pos = torch.cat([torch.arange(c, dtype=torch.float32) for c in ctx])
    k[:, :, 0] = (pos * slope / (16.0 * scale))[:, None]
    cu_k = torch.tensor([0] + list(np.cumsum(ctx)), dtype=torch.int32)
    mbs = max((c + 255) // 256 for c in ctx)
    pg = workloads.paged_pool(k.bfloat16(), v.bfloat16(), cu_k, [c - 1 for c in ctx], 256, 43,
                              spare_blocks=2, max_blocks_per_seq=mbs)
    dc = workloads.Decode(q.bfloat16(), scale, pg, "monotone logits")
    log(f"case decode monotone logits slope={slope} split={split}")
    check_bf16(np32(run_decode(dc, split)), oracle_decode(dc), f"decode slope {slope} split {split}")


def test_decode_shapes_example():
    """The Decode section's example shapes: q [2, 32, 128] -> o [2, 32, 128]."""
    shp = load_golden("decode_shapes.txt")["q_shape"]
    dc = make_decode([300, 1000], hq=shp[1], hkv=8, seed=1)
    assert list(dc.q.shape) == shp
    log("case decode shapes example")
    got = run_decode(dc)
    assert list(got.shape) == shp
    check_bf16(np32(got), oracle_decode(dc), "decode [2,32,128]")


@pytest.mark.parametrize("split", [0, 32, 64, 256, 1024])
def test_decode_ragged_contexts(split):
    ctx = [1, 2, 63, 64, 65, 255, 256, 257, 1000, 3000]
    dc = make_decode(ctx, seed=7)
    log(f"case decode ragged split={split}")
    check_bf16(np32(run_decode(dc, split)), oracle_decode(dc), f"decode split {split}")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 1), (12, 4), (12, 3), (32, 16), (24, 12), (10, 5)])
def test_decode_group_sizes(hq, hkv):
    dc = make_decode([17, 700, 129], hq=hq, hkv=hkv, block_size=64, seed=hq + hkv)
    log(f"case decode groups {hq}/{hkv}")
    check_bf16(np32(run_decode(dc)), oracle_decode(dc), f"decode {hq}/{hkv}")


@pytest.mark.parametrize("split", [0, 96])
def test_decode_many_short_sequences(split):
    """More sequences than a wavefront scans at once and than there are
    compute units, most far shorter than one run, with empty ones between:
    runs then hold many sequences each and the partial links are short."""
    rng = np.random.default_rng(11)
    ctx = [int(c) for c in rng.integers(0, 120, size=300)]
    ctx[5] = ctx[77] = ctx[299] = 0
    ctx[130] = 2000
    dc = make_decode(ctx, hq=16, hkv=4, block_size=64, seed=12)
    log(f"case decode 300 short sequences split={split}")
    got = np32(run_decode(dc, split))
    ref = oracle_decode(dc)
    for b in (5, 77, 299):
        assert np.all(got[b] == 0)
    check_bf16(got, ref, f"decode 300 short split {split}")


def test_decode_zero_context_and_bf16_output():
    dc = make_decode([0, 90, 513], seed=3)
    log("case decode zero ctx + bf16 out")
    got = run_decode(dc)
    ref = oracle_decode(dc)
    assert np.all(np32(got)[0] == 0)
    check_bf16(np32(got), ref, "decode zero ctx")
    got_b = run_decode(dc, out_dtype=torch.bfloat16)
    check_bf16_output(got_b, ref, "decode bf16 out")


def test_decode_equals_last_prefill_row():
    """Decode of the newest token equals the last row of causal prefill over
    the same context (both on the GPU, through the same paged cache)."""
    ctx = [150, 600, 64]
    dc = make_decode(ctx, hq=8, hkv=2, block_size=64, seed=5)
    dec = np32(run_decode(dc))
    pg = dc.paged
    kc, vc = dev(pg.k_cache), dev(pg.v_cache)
    attn.kv_store_slots(dev(pg.k_new), dev(pg.v_new), kc, vc, dev(pg.slot_mapping))
    q = torch.zeros(sum(ctx), 8, 128, dtype=torch.bfloat16)
    cu = pg.cu_seqlens_k
    for b in range(3):
        q[cu[b + 1] - 1] = dc.q[b]
    pre = attn.attn_prefill_varlen(dev(q), kc, vc, dev(cu), dev(cu), max(ctx), max(ctx),
                                   dc.softmax_scale, True, block_table=dev(pg.block_table),
                                   out_dtype=torch.float32)
    torch.cuda.synchronize()
    last = np32(pre)[[c - 1 for c in cu[1:].tolist()]]
    log("case decode == last prefill row")
    check_bf16(dec, last, "decode vs prefill")


def test_full_paged_decode_64():
    dc = workloads.paged_decode()
    log(f"case {dc.name}")
    ref = oracle_decode(dc)
    got = run_decode(dc)
    check_bf16(np32(got), ref, "decode 64 (all rows)")
    for split in (256, 2048):
        check_bf16(np32(run_decode(dc, split)), ref, f"decode 64 split {split}")


def test_decode_shared_prefix_blocks():
    """Decode over block tables whose first blocks are shared by every
    sequence (one cached prompt stored once): the new token of each sequence
    attends to the prompt, its own cached tokens and itself."""
    pp = workloads.shared_prefix_prefill(n_seqs=8, shared_blocks=4, own_lo=0, own_hi=700,
                                         q_lo=1, q_hi=1, hq=32, hkv=8, block_size=256, seed=41)
    dc = workloads.Decode(pp.q.view(8, 32, 128), pp.softmax_scale, pp.paged, pp.name)
    assert (dc.paged.block_table[:, :4] == dc.paged.block_table[0, :4]).all()
    log("case decode shared prefix blocks")
    for split in (0, 256):
        check_bf16(np32(run_decode(dc, split)), oracle_decode(dc), f"decode shared prefix split {split}")


def test_decode_reused_workspace():
    """One workspace serves calls of different sizes back to back: every word
    the merge reads is written by the same call, so nothing needs clearing
    (it starts as garbage here on purpose)."""
    cases = [make_decode([5000, 3000, 700], seed=21), make_decode([9000], seed=22),
             make_decode([64, 1, 4000, 2500, 0, 128], seed=23), make_decode([5000, 3000, 700], seed=24)]
    need = max(attn.attn_decode_workspace_bytes(dc.q.shape[0], 32, 8, 128,
                                                dc.paged.block_table.shape[1], 256, 0) for dc in cases)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    for i, dc in enumerate(cases * 2):
        pg = dc.paged
        kc, vc = dev(pg.k_cache), dev(pg.v_cache)
        attn.kv_store_slots(dev(pg.k_new), dev(pg.v_new), kc, vc, dev(pg.slot_mapping))
        got = attn.attn_decode_paged(dev(dc.q), kc, vc, dev(pg.seqlens_k), dev(pg.block_table),
                                     dc.softmax_scale, workspace=ws, out_dtype=torch.float32)
        torch.cuda.synchronize()
        log(f"case decode reused workspace call {i}")
        check_bf16(np32(got), oracle_decode(dc), f"decode reused workspace call {i}")


def test_decode_block_ids_outside_the_pool():
    """A block id outside [0, num_blocks) reads as zero rows.  Many short
    sequences put sequence boundaries inside runs, and the bad ids include
    first blocks, which the split kernel requests for the next sequence while
    it finishes the previous one."""
    rng = np.random.default_rng(61)
    ctx = [int(c) for c in rng.integers(100, 900, size=48)]
    dc = make_decode(ctx, block_size=64, seed=62)
    pg = dc.paged
    nb = pg.num_blocks
    bad = [(b, 0, -1 if b % 2 else nb + b) for b in range(0, 48, 3)]
    bad += [(b, (ctx[b] + 63) // 64 // 2, nb) for b in range(1, 48, 5) if (ctx[b] + 63) // 64 > 2]
    # the block of the new token (the last of each context) stays valid
    assert all(i != (ctx[b] - 1) // 64 for b, i, _ in bad)
    bt = pg.block_table.clone()
    k, v = pg.k_logical.clone(), pg.v_logical.clone()
    cu = pg.cu_seqlens_k.tolist()
    for b, i, blk in bad:
        bt[b, i] = blk
        lo, hi = cu[b] + 64 * i, min(cu[b] + 64 * (i + 1), cu[b + 1])
        k[lo:hi] = 0
        v[lo:hi] = 0
    kc, vc = dev(pg.k_cache), dev(pg.v_cache)
    attn.kv_store_slots(dev(pg.k_new), dev(pg.v_new), kc, vc, dev(pg.slot_mapping))
    log("case decode block ids outside the pool")
    got = attn.attn_decode_paged(dev(dc.q), kc, vc, dev(pg.seqlens_k), dev(bt), dc.softmax_scale,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.attn_decode(np32(dc.q), np32(k), np32(v), pg.cu_seqlens_k.numpy(), dc.softmax_scale)
    check_bf16(np32(got), ref, "decode bad block ids")


def test_decode_largest_item_size():
    """split_tokens at the largest multiple of 32 an int holds: every
    sequence is one item, and the item counts and ends (computed in 64 bits)
    do not overflow."""
    dc = make_decode([700, 1, 3000, 257], seed=71)
    log("case decode split_tokens 2147483616")
    check_bf16(np32(run_decode(dc, 2147483616)), oracle_decode(dc), "decode largest item size")


def test_decode_long_context_128k():
    """A 131072-token context beside short ones: a sequence spanning many
    runs (the merge reads dozens of partials) and 512-entry block tables."""
    dc = make_decode([131072, 5, 70000, 300], seed=73)
    assert dc.paged.block_table.shape[1] == 512
    log("case decode 128K context")
    check_bf16(np32(run_decode(dc)), oracle_decode(dc), "decode 128K context")


def test_decode_all_contexts_empty():
    """Every context length 0: the key stream has no item at all, no run is
    used, and every output row is 0."""
    dc = make_decode([0, 0, 0], seed=31, mbs=2)
    log("case decode all contexts empty")
    got = run_decode(dc)
    assert np.all(np32(got) == 0)
