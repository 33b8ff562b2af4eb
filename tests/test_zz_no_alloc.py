"""attn_decode_paged_noalloc (the decode entry point that allocates nothing,
on the library's per-GPU scratch array) against attn_decode_paged on the
same inputs: two calls in a row, the second smaller, so that what the first
call leaves in the scratch cannot leak into the second.  Same kernels, same
run partition: the outputs must be bit-identical, and both within the bf16
tolerance of the oracle."""
import numpy as np
import pytest
import torch

import attention_sdpa_amd as attn
import oracle
import workloads
from tests.helpers import check_bf16, dev, log, np32

pytestmark = pytest.mark.gpu


def decode_pair(dc):
    pg = dc.paged
    kc, vc = dev(pg.k_cache), dev(pg.v_cache)
    attn.kv_store_slots(dev(pg.k_new), dev(pg.v_new), kc, vc, dev(pg.slot_mapping))
    q, sl, bt = dev(dc.q), dev(pg.seqlens_k), dev(pg.block_table)
    ref_out = attn.attn_decode_paged(q, kc, vc, sl, bt, dc.softmax_scale, out_dtype=torch.float32)
    out = torch.full_like(ref_out, float("nan"))
    attn.attn_decode_paged_noalloc(q, kc, vc, sl, bt, dc.softmax_scale, out=out)
    torch.cuda.synchronize()
    return ref_out, out


def oracle_decode(dc):
    pg = dc.paged
    return oracle.attn_decode(np32(dc.q), np32(pg.k_logical), np32(pg.v_logical),
                              pg.cu_seqlens_k.numpy(), dc.softmax_scale)


def test_noalloc_matches_workspace_entry_point_twice():
    big = workloads.paged_decode()                      # batch 64, contexts U[512, 8192]
    small = workloads.paged_decode(batch=5, lo=1, hi=700, hq=8, hkv=2, block_size=64, seed=321)
    for name, dc in (("batch 64", big), ("batch 5, smaller", small)):
        log(f"case noalloc decode {name}")
        ref_out, out = decode_pair(dc)
        assert torch.equal(out, ref_out), f"{name}: differs from attn_decode_paged"
        check_bf16(np32(out), oracle_decode(dc), f"noalloc {name}")


def test_noalloc_layout_follows_the_device_runs():
    """The scratch layout counts the runs this device uses, not the 1024 a
    caller's workspace is sized for: 64 query heads fit (their 1024-run
    layout would not), and so do 1200 sequences at 32 heads (more than the
    992 a 1024-run layout allows)."""
    for name, dc in (("64 query heads", workloads.paged_decode(batch=6, lo=1, hi=900, hq=64, hkv=8,
                                                               block_size=64, seed=331)),
                     ("1200 sequences", workloads.paged_decode(batch=1200, lo=1, hi=40, hq=32, hkv=8,
                                                               block_size=64, seed=332))):
        log(f"case noalloc decode {name}")
        ref_out, out = decode_pair(dc)
        assert torch.equal(out, ref_out), f"{name}: differs from attn_decode_paged"
        check_bf16(np32(out), oracle_decode(dc), f"noalloc {name}")


def test_noalloc_rejects_calls_beyond_the_scratch():
    # 2048 sequences x 32 heads needs more than the 32 MiB scratch: rejected before any launch
    q = torch.zeros(2048, 32, 128, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(1, 256, 8, 128, dtype=torch.bfloat16, device="cuda")
    sl = torch.ones(2048, dtype=torch.int32, device="cuda")
    bt = torch.zeros(2048, 1, dtype=torch.int32, device="cuda")
    with pytest.raises(attn.AttnError) as ei:
        attn.attn_decode_paged_noalloc(q, kc, kc.clone(), sl, bt, 0.088)
    assert ei.value.status == attn.ATTN_ERR_WORKSPACE
