"""The Python binding's argument checks, without a GPU: mismatched dtypes,
shapes, index lengths and devices raise before any pointer reaches the
library (each of these would otherwise make a kernel read past a buffer)."""
import pytest
import torch

import attention_sdpa_amd as attn

bf = torch.bfloat16


def varlen_args(**kw):
    a = dict(q=torch.zeros(10, 4, 128, dtype=bf), k=torch.zeros(12, 2, 128, dtype=bf),
             v=torch.zeros(12, 2, 128, dtype=bf), cu_q=torch.tensor([0, 4, 10], dtype=torch.int32),
             cu_k=torch.tensor([0, 5, 12], dtype=torch.int32))
    a.update(kw)
    return a


def call_varlen(block_table=None, **kw):
    a = varlen_args(**kw)
    return attn.attn_prefill_varlen(a["q"], a["k"], a["v"], a["cu_q"], a["cu_k"], 6, 7, 0.088, True,
                                    block_table=block_table)


def test_varlen_valid_args_reach_the_device_check():
    with pytest.raises(ValueError, match="live on the GPU"):
        call_varlen()


@pytest.mark.parametrize("kw,msg", [
    (dict(q=torch.zeros(10, 4, 128)), "share a dtype"),                          # fp32 q, bf16 k/v
    (dict(v=torch.zeros(12, 2, 128, dtype=torch.float16)), "share a dtype"),
    (dict(v=torch.zeros(11, 2, 128, dtype=bf)), "differ in shape"),              # v shorter than k
    (dict(k=torch.zeros(12, 2, 64, dtype=bf), v=torch.zeros(12, 2, 64, dtype=bf)), "head_dim"),
    (dict(cu_k=torch.tensor([0, 12], dtype=torch.int32)), "cu_seqlens_k has 2 entries"),
    (dict(cu_q=torch.tensor([0], dtype=torch.int32)), "at least 2 entries"),
    (dict(q=torch.zeros(10, 512, dtype=bf)), "q must be"),
])
def test_varlen_mismatches_raise(kw, msg):
    with pytest.raises(ValueError, match=msg):
        call_varlen(**kw)


def test_varlen_index_dtype_and_device():
    with pytest.raises(TypeError, match="int32"):
        call_varlen(cu_k=torch.tensor([0, 5, 12], dtype=torch.int64))
    with pytest.raises(ValueError, match="every tensor must be on"):
        call_varlen(cu_k=torch.zeros(3, dtype=torch.int32, device="meta"))


def test_varlen_paged_block_table_rows():
    kc = torch.zeros(4, 64, 2, 128, dtype=bf)
    bt_short = torch.zeros(1, 4, dtype=torch.int32)          # 2 sequences need 2 rows
    with pytest.raises(ValueError, match="block_table"):
        call_varlen(block_table=bt_short, k=kc, v=kc.clone())
    with pytest.raises(ValueError, match="paged k"):
        call_varlen(block_table=torch.zeros(2, 4, dtype=torch.int32))   # k not 4-D
    with pytest.raises(TypeError, match="block_table must be int32"):
        call_varlen(block_table=torch.zeros(2, 4, dtype=torch.int64), k=kc, v=kc.clone())


def decode_args(**kw):
    a = dict(q=torch.zeros(3, 4, 128, dtype=bf), kc=torch.zeros(5, 64, 2, 128, dtype=bf),
             vc=torch.zeros(5, 64, 2, 128, dtype=bf), sl=torch.tensor([1, 2, 3], dtype=torch.int32),
             bt=torch.zeros(3, 2, dtype=torch.int32))
    a.update(kw)
    return a


def call_decode(**kw):
    a = decode_args(**kw)
    return attn.attn_decode_paged(a["q"], a["kc"], a["vc"], a["sl"], a["bt"], 0.088)


@pytest.mark.parametrize("kw,msg", [
    (dict(vc=torch.zeros(5, 64, 2, 128, dtype=torch.float16)), "share a dtype"),
    (dict(vc=torch.zeros(4, 64, 2, 128, dtype=bf)), "differ in shape"),
    (dict(sl=torch.tensor([1, 2], dtype=torch.int32)), "cache_seqlens has 2 entries"),
    (dict(bt=torch.zeros(2, 2, dtype=torch.int32)), "block_table"),
    (dict(kc=torch.zeros(5, 128, 128, dtype=bf), vc=torch.zeros(5, 128, 128, dtype=bf)), "caches must be"),
])
def test_decode_mismatches_raise(kw, msg):
    with pytest.raises(ValueError, match=msg):
        call_decode(**kw)


def test_decode_valid_args_reach_the_device_check():
    with pytest.raises(ValueError, match="live on the GPU"):
        call_decode()


def test_padded_and_unfused_mismatches_raise():
    q = torch.zeros(2, 8, 4, 128, dtype=bf)
    k = torch.zeros(2, 9, 2, 128, dtype=bf)
    lq = torch.tensor([8, 3], dtype=torch.int32)
    with pytest.raises(ValueError, match="differ in shape"):
        attn.attn_prefill_padded(q, k, k[:, :8].contiguous(), lq, lq, 0.088)
    with pytest.raises(ValueError, match="seqlens_k has 1 entries"):
        attn.attn_prefill_padded(q, k, k.clone(), lq, lq[:1].contiguous(), 0.088)
    with pytest.raises(ValueError, match="share a dtype"):
        attn.attn_prefill_padded(q.float(), k, k.clone(), lq, lq, 0.088)
    a = varlen_args()
    with pytest.raises(ValueError, match="differ in shape"):
        attn.attn_prefill_unfused(a["q"], a["k"], a["v"][:11].contiguous(), a["cu_q"], a["cu_k"], 6, 7, 0.088)
    with pytest.raises(ValueError, match="cu_seqlens_k has 2 entries"):
        attn.attn_prefill_unfused(a["q"], a["k"], a["v"], a["cu_q"], a["cu_k"][:2].contiguous(), 6, 7, 0.088)


def test_kv_store_mismatches_raise():
    k = torch.zeros(3, 2, 128, dtype=bf)
    kc = torch.zeros(4, 64, 2, 128, dtype=bf)
    slots = torch.tensor([0, 1, 2], dtype=torch.int32)
    with pytest.raises(ValueError):
        attn.kv_store_slots(k, k.half(), kc, kc.clone(), slots)
    with pytest.raises(TypeError, match="int32"):
        attn.kv_store_slots(k, k.clone(), kc, kc.clone(), slots.long())
    with pytest.raises(ValueError, match="every tensor must be on"):
        attn.kv_store_slots(k, k.clone(), kc, kc.clone(), torch.zeros(3, dtype=torch.int32, device="meta"))
