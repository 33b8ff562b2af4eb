"""GPU parity of attn_prefill_padded: the padded-batch layout of the blog
post "从零实现 vLLM (1.3)：如何加速 Attention 计算" (section Prefill: a padded
batch and its varlen packing by cu_seqlens give the same outputs on the valid
rows).  The oracle runs on the packed layout; the padded tensors are built
from it by placing each sequence's rows at the start of its padded slot."""
import numpy as np
import pytest
import torch

import attention_sdpa_amd as attn
import oracle
import workloads
from tests.golden import load as load_golden
from tests.helpers import check_bf16, check_f32, dev, log, np32

pytestmark = pytest.mark.gpu

SENTINEL = 1234.5


def to_padded(x, cu, L):
    """[total, H, d] packed by cu -> [B, L, H, d] with the gaps NaN (so a
    kernel that reads a padded row as a key cannot pass)."""
    B = len(cu) - 1
    out = torch.full((B, L) + tuple(x.shape[1:]), float("nan"), dtype=x.dtype)
    for b in range(B):
        out[b, :cu[b + 1] - cu[b]] = x[cu[b]:cu[b + 1]]
    return out


def run_padded(vl, causal=None, out_dtype=torch.float32, mq=None, mk=None):
    cq, ck = vl.cu_seqlens_q.tolist(), vl.cu_seqlens_k.tolist()
    mq = mq or max(1, max(b - a for a, b in zip(cq, cq[1:])))
    mk = mk or max(1, max(b - a for a, b in zip(ck, ck[1:])))
    q = to_padded(vl.q, cq, mq)
    k, v = to_padded(vl.k, ck, mk), to_padded(vl.v, ck, mk)
    lq = torch.tensor([b - a for a, b in zip(cq, cq[1:])], dtype=torch.int32)
    lk = torch.tensor([b - a for a, b in zip(ck, ck[1:])], dtype=torch.int32)
    out = torch.full((len(lq), mq) + tuple(vl.q.shape[1:]), SENTINEL, dtype=out_dtype, device="cuda")
    attn.attn_prefill_padded(dev(q), dev(k), dev(v), dev(lq), dev(lk), vl.softmax_scale,
                             vl.causal if causal is None else causal, out=out)
    torch.cuda.synchronize()
    got = out.cpu()
    valid = torch.cat([got[b, :int(lq[b])] for b in range(len(lq))])
    pad_rows = [got[b, int(lq[b]):] for b in range(len(lq))]
    return np32(valid), pad_rows


def oracle_varlen(vl, causal=None):
    return oracle.attn_varlen(np32(vl.q), np32(vl.k), np32(vl.v), vl.cu_seqlens_q.numpy(),
                              vl.cu_seqlens_k.numpy(), vl.softmax_scale,
                              vl.causal if causal is None else causal)


def assert_pads_untouched(pads):
    for p in pads:
        assert torch.all(p == SENTINEL), "an output row past seqlens_q was written"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_padded_blog_example(dtype):
    """The Prefill section's batch: query lengths 5, 2, 1 against key lengths
    9, 7, 3, padded to 5 and 9 rows."""
    ex = load_golden("varlen_example.txt")
    cq, ck = ex["cu_seqlens_q"], ex["cu_seqlens_k"]
    lq = [b - a for a, b in zip(cq, cq[1:])]
    lk = [b - a for a, b in zip(ck, ck[1:])]
    d = 128 if dtype == torch.bfloat16 else 64
    vl = workloads.varlen(lq, lk, 8, 2, d, dtype, seed=31)
    assert vl.cu_seqlens_q.tolist() == cq and vl.cu_seqlens_k.tolist() == ck
    log(f"case padded blog example {dtype}")
    for causal in (True, False):
        got, pads = run_padded(vl, causal=causal, mq=ex["padded_q_len"][0])
        ref = oracle_varlen(vl, causal=causal)
        (check_bf16 if dtype == torch.bfloat16 else check_f32)(got, ref, f"padded example causal={causal}")
        assert_pads_untouched(pads)


def test_padded_ragged_bf16():
    lq = [1, 63, 64, 65, 200, 0, 130]
    lk = [1, 63, 300, 65, 200, 10, 90]
    vl = workloads.varlen(lq, lk, 32, 8, 128, torch.bfloat16, seed=32)
    log("case padded ragged bf16")
    got, pads = run_padded(vl)
    check_bf16(got, oracle_varlen(vl), "padded ragged")
    assert_pads_untouched(pads)


def test_padded_equals_varlen_bits():
    """The padded entry runs the varlen kernel in place: same inputs, same
    arithmetic order, so the valid rows are bit-identical to the packed call."""
    lq = [40, 300, 7, 129]
    vl = workloads.varlen(lq, lq, 16, 4, 128, torch.bfloat16, seed=33)
    got, _ = run_padded(vl)
    packed = attn.attn_prefill_varlen(dev(vl.q), dev(vl.k), dev(vl.v), dev(vl.cu_seqlens_q),
                                      dev(vl.cu_seqlens_k), vl.max_seqlen_q, vl.max_seqlen_k,
                                      vl.softmax_scale, True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    log("case padded == varlen bits")
    assert np.array_equal(got, np32(packed))


def test_padded_no_keys_at_all():
    """max_seqlen_k = 0: no sequence has a key, so every valid output row is
    0 (and padded rows stay untouched)."""
    q = torch.randn(2, 4, 8, 128).to(torch.bfloat16)
    k = torch.empty(2, 0, 2, 128, dtype=torch.bfloat16)
    lq = torch.tensor([3, 4], dtype=torch.int32)
    lk = torch.tensor([0, 0], dtype=torch.int32)
    out = torch.full((2, 4, 8, 128), SENTINEL, dtype=torch.float32, device="cuda")
    log("case padded no keys")
    attn.attn_prefill_padded(dev(q), dev(k), dev(k), dev(lq), dev(lk), 0.1, True, out=out)
    torch.cuda.synchronize()
    got = out.cpu()
    assert torch.all(got[0, :3] == 0) and torch.all(got[1, :4] == 0)
    assert torch.all(got[0, 3:] == SENTINEL)
