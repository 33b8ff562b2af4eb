"""GPU parity for fp16 inputs (the 16-bit type the blog post "从零实现 vLLM
(1.3)：如何加速 Attention 计算" names in its safe-softmax section, where exp
overflows fp16 from x ~ 11): the same kernels as bf16, templated on the
element type, against the fp64 oracle on the same fp16-rounded inputs.  The
bar (max abs 5e-3, mean abs 5e-4) follows from P rounded to fp16 (relative
error 2^-11) with fp32 accumulation."""
import numpy as np
import pytest
import torch

import attention_sdpa_amd as attn
import oracle
import workloads
from tests.helpers import check_f16, check_f16_output, dev, log, np32, oracle_varlen

pytestmark = pytest.mark.gpu
F16 = torch.float16


def run_varlen(vl, causal=None, out_dtype=torch.float32):
    out = attn.attn_prefill_varlen(dev(vl.q), dev(vl.k), dev(vl.v), dev(vl.cu_seqlens_q),
                                   dev(vl.cu_seqlens_k), vl.max_seqlen_q, vl.max_seqlen_k,
                                   vl.softmax_scale, vl.causal if causal is None else causal,
                                   out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 8), (12, 3)])
def test_fp16_varlen_ragged(hq, hkv):
    lq = [1, 63, 64, 65, 200, 7, 129]
    vl = workloads.varlen(lq, lq, hq, hkv, 128, F16, seed=40 + hq)
    log(f"case fp16 varlen {hq}/{hkv}")
    ref = oracle_varlen(vl)
    check_f16(np32(run_varlen(vl)), ref, f"fp16 varlen {hq}/{hkv}")
    check_f16_output(run_varlen(vl, out_dtype=F16), ref, f"fp16 varlen {hq}/{hkv} fp16 out")


def test_fp16_end_aligned_and_noncausal():
    vl = workloads.varlen([5, 40, 90, 1], [9, 300, 60, 1], 8, 2, 128, F16, seed=44)
    log("case fp16 end-aligned / non-causal")
    check_f16(np32(run_varlen(vl)), oracle_varlen(vl), "fp16 end-aligned causal")
    check_f16(np32(run_varlen(vl, causal=False)), oracle_varlen(vl, causal=False), "fp16 non-causal")


def test_fp16_stress_logits_near_700():
    """Logits around 700 (the safe-softmax section's overflow example) with
    fp16 inputs: e^700 overflows any float type, and e^x overflows fp16 from
    x ~ 11; the kernels keep the running maximum in fp32 and P <= 2^8."""
    vl = workloads.fp16_stress()
    log(f"case {vl.name}")
    got = np32(run_varlen(vl))
    ref = oracle_varlen(vl)
    check_f16(got, ref, vl.name)
    # row 2 is the [700, 710, 705] example's weights applied to V rows 0..2
    w = np.exp(np.array([-10.0, 0.0, -5.0]))
    w /= w.sum()
    v = np32(vl.v).astype(np.float64)
    assert np.max(np.abs(got[2, 0] - w @ v[:3, 0])) <= 5e-3


def test_fp16_prefix_prefill_paged():
    pp = workloads.prefix_prefill(n_seqs=4, q_lo=1, q_hi=150, p_lo=10, p_hi=700, hq=16, hkv=4,
                                  block_size=64, seed=45, dtype=F16)
    pg = pp.paged
    kc, vc = dev(pg.k_cache), dev(pg.v_cache)
    attn.kv_store_slots(dev(pg.k_new), dev(pg.v_new), kc, vc, dev(pg.slot_mapping))
    out = attn.attn_prefill_varlen(dev(pp.q), kc, vc, dev(pp.cu_seqlens_q), dev(pg.cu_seqlens_k),
                                   pp.max_seqlen_q, pp.max_seqlen_k, pp.softmax_scale, True,
                                   block_table=dev(pg.block_table), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.attn_varlen(np32(pp.q), np32(pg.k_logical), np32(pg.v_logical),
                             pp.cu_seqlens_q.numpy(), pg.cu_seqlens_k.numpy(), pp.softmax_scale, True)
    log("case fp16 prefix prefill paged")
    check_f16(np32(out), ref, "fp16 prefix paged")


@pytest.mark.parametrize("split", [0, 256])
def test_fp16_decode(split):
    dc = workloads.paged_decode(batch=6, lo=1, hi=3000, hq=32, hkv=8, block_size=256, seed=46,
                                dtype=F16)
    pg = dc.paged
    kc, vc = dev(pg.k_cache), dev(pg.v_cache)
    attn.kv_store_slots(dev(pg.k_new), dev(pg.v_new), kc, vc, dev(pg.slot_mapping))
    ref = oracle.attn_decode(np32(dc.q), np32(pg.k_logical), np32(pg.v_logical),
                             pg.cu_seqlens_k.numpy(), dc.softmax_scale)
    log(f"case fp16 decode split={split}")
    for out_dtype in (torch.float32, F16):
        got = attn.attn_decode_paged(dev(dc.q), kc, vc, dev(pg.seqlens_k), dev(pg.block_table),
                                     dc.softmax_scale, split_tokens=split, out_dtype=out_dtype)
        torch.cuda.synchronize()
        if out_dtype == F16:
            check_f16_output(got, ref, "fp16 decode fp16 out")
        else:
            check_f16(np32(got), ref, "fp16 decode")


def test_fp16_padded():
    lq, lk = [5, 2, 1], [9, 7, 3]
    vl = workloads.varlen(lq, lk, 8, 2, 128, F16, seed=47)
    q = torch.zeros(3, 5, 8, 128, dtype=F16)
    k = torch.full((3, 9, 2, 128), float("nan"), dtype=F16)
    v = k.clone()
    cq, ck = vl.cu_seqlens_q.tolist(), vl.cu_seqlens_k.tolist()
    for b in range(3):
        q[b, :lq[b]] = vl.q[cq[b]:cq[b + 1]]
        k[b, :lk[b]] = vl.k[ck[b]:ck[b + 1]]
        v[b, :lk[b]] = vl.v[ck[b]:ck[b + 1]]
    out = attn.attn_prefill_padded(dev(q), dev(k), dev(v), dev(torch.tensor(lq, dtype=torch.int32)),
                                   dev(torch.tensor(lk, dtype=torch.int32)), vl.softmax_scale, True,
                                   out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = np.concatenate([np32(out[b, :lq[b]]) for b in range(3)])
    log("case fp16 padded")
    check_f16(got, oracle_varlen(vl), "fp16 padded")


def test_full_fp16_varlen_prefill_16_seqs():
    """The headline varlen workload (16 sequences, U[128, 4096]) with fp16
    inputs, in the launch configuration the benchmark times, on sampled rows
    (first, middle and last token of every sequence for three heads, plus
    random rows)."""
    from tests.helpers import sample_rows
    vl = workloads.varlen_prefill(dtype=F16)
    log(f"case fp16 {vl.name}")
    got = run_varlen(vl)
    rows = sample_rows(vl.cu_seqlens_q, 32, 600, seed=3)
    check_f16(np32(got).reshape(-1, 128)[rows], oracle_varlen(vl, rows=rows), "fp16 varlen 16 seqs (sampled)")
    assert torch.isfinite(got).all().item()


def test_full_fp16_paged_decode_64():
    """The decode workload (batch 64, contexts U[512, 8192], block 256,
    permuted pool) with fp16 inputs, every output row."""
    dc = workloads.paged_decode(dtype=F16)
    pg = dc.paged
    kc, vc = dev(pg.k_cache), dev(pg.v_cache)
    attn.kv_store_slots(dev(pg.k_new), dev(pg.v_new), kc, vc, dev(pg.slot_mapping))
    got = attn.attn_decode_paged(dev(dc.q), kc, vc, dev(pg.seqlens_k), dev(pg.block_table),
                                 dc.softmax_scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    log("case fp16 decode 64")
    ref = oracle.attn_decode(np32(dc.q), np32(pg.k_logical), np32(pg.v_logical),
                             pg.cu_seqlens_k.numpy(), dc.softmax_scale)
    check_f16(np32(got), ref, "fp16 decode 64 (all rows)")
