"""GPU parity of the unfused three-kernel baseline attn_prefill_unfused (the
standard method of the blog post "从零实现 vLLM (1.3)：如何加速 Attention
计算", section 标准实现方法: X and A stored between the steps) against the fp64
oracle, and against the fused one-pass kernel on the same inputs."""
import numpy as np
import pytest
import torch

import attention_sdpa_amd as attn
import oracle
import workloads
from tests.helpers import check_bf16, check_bf16_output, dev, log, np32

pytestmark = pytest.mark.gpu


def run_unfused(vl, causal=None, out_dtype=torch.float32, workspace=None):
    out = attn.attn_prefill_unfused(dev(vl.q), dev(vl.k), dev(vl.v), dev(vl.cu_seqlens_q),
                                    dev(vl.cu_seqlens_k), vl.max_seqlen_q, vl.max_seqlen_k,
                                    vl.softmax_scale, vl.causal if causal is None else causal,
                                    workspace=workspace, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


def oracle_varlen(vl, causal=None):
    return oracle.attn_varlen(np32(vl.q), np32(vl.k), np32(vl.v), vl.cu_seqlens_q.numpy(),
                              vl.cu_seqlens_k.numpy(), vl.softmax_scale,
                              vl.causal if causal is None else causal)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 2), (12, 3)])
def test_unfused_ragged(hq, hkv):
    lq = [1, 63, 64, 65, 130, 7]
    vl = workloads.varlen(lq, lq, hq, hkv, 128, torch.bfloat16, seed=hq * 10 + hkv)
    log(f"case unfused ragged {hq}/{hkv}")
    check_bf16(np32(run_unfused(vl)), oracle_varlen(vl), f"unfused ragged {hq}/{hkv}")


def test_unfused_end_aligned_noncausal_empty():
    """Lq < Lk (end-aligned causal), Lq > Lk (rows with no visible key give
    zeros), an empty sequence, and the non-causal form."""
    vl = workloads.varlen([5, 40, 0, 90, 3], [9, 300, 4, 60, 3], 8, 2, 128, torch.bfloat16, seed=3)
    log("case unfused end-aligned / empty / non-causal")
    got = np32(run_unfused(vl))
    ref = oracle_varlen(vl)
    check_bf16(got, ref, "unfused end-aligned causal")
    rows = slice(int(vl.cu_seqlens_q[3]), int(vl.cu_seqlens_q[3]) + 29)   # Lq 90 > Lk 60: first 30 rows see nothing
    assert np.all(got[rows] == 0)
    check_bf16(np32(run_unfused(vl, causal=False)), oracle_varlen(vl, causal=False), "unfused non-causal")


def test_unfused_matches_fused_and_bf16_output():
    """Medium varlen batch: the unfused path and the fused kernel both match
    the oracle; bf16 output within the output-rounding bound."""
    vl = workloads.varlen_prefill(n_seqs=4, lo=128, hi=1500, hq=32, hkv=8, seed=77)
    log("case unfused medium varlen")
    ref = oracle_varlen(vl)
    unf = np32(run_unfused(vl))
    check_bf16(unf, ref, "unfused medium")
    fused = attn.attn_prefill_varlen(dev(vl.q), dev(vl.k), dev(vl.v), dev(vl.cu_seqlens_q),
                                     dev(vl.cu_seqlens_k), vl.max_seqlen_q, vl.max_seqlen_k,
                                     vl.softmax_scale, True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_bf16(np32(fused), ref, "fused medium")
    check_bf16_output(run_unfused(vl, out_dtype=torch.bfloat16), ref, "unfused bf16 out")


def test_unfused_reused_workspace():
    """A workspace left full of another call's X and A does not leak into the
    next call (its contents on entry are ignored)."""
    a = workloads.varlen([200, 50], [200, 50], 8, 2, 128, torch.bfloat16, seed=8)
    b = workloads.varlen([30, 190], [30, 190], 8, 2, 128, torch.bfloat16, seed=9)
    need = attn.attn_unfused_workspace_bytes(2, 8, 200, 200)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    log("case unfused reused workspace")
    for vl in (a, b, a):
        check_bf16(np32(run_unfused(vl, workspace=ws)), oracle_varlen(vl), "unfused reuse")


def test_unfused_sequence_without_keys():
    """A sequence with queries but no keys gives zero rows; its neighbours
    are unaffected."""
    vl = workloads.varlen([4, 6, 3], [5, 0, 3], 8, 2, 128, torch.bfloat16, seed=10)
    log("case unfused sequence without keys")
    for causal in (True, False):
        got = np32(run_unfused(vl, causal=causal))
        assert np.all(got[4:10] == 0)
        check_bf16(got, oracle_varlen(vl, causal=causal), f"unfused no-key sequence causal={causal}")
