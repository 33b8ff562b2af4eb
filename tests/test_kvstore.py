"""GPU: kv_store_slots is a bit-exact scatter (the store_kvcache step of the
blog post "从零实现 vLLM (1.3)：如何加速 Attention 计算", section Attention 源码
分析), checked against the oracle's numpy scatter on integer views."""
import numpy as np
import pytest
import torch

import attention_sdpa_amd as attn
import oracle
import workloads
from tests.helpers import dev, log

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("case", ["decode_like", "prefix_like"])
def test_kv_store_bit_exact(dtype, case):
    log(f"kv_store {case} {dtype}")
    if case == "decode_like":
        dc = workloads.paged_decode(batch=7, lo=1, hi=700, hq=8, hkv=2, d=128, block_size=64,
                                    seed=11, dtype=dtype, spare_blocks=3)
        pg = dc.paged
    else:
        pp = workloads.prefix_prefill(n_seqs=5, q_lo=1, q_hi=90, p_lo=0, p_hi=300, hq=4, hkv=4,
                                      d=64 if dtype == torch.float32 else 128, block_size=128,
                                      seed=12, dtype=dtype)
        pg = pp.paged
    kc, vc = dev(pg.k_cache), dev(pg.v_cache)
    attn.kv_store_slots(dev(pg.k_new), dev(pg.v_new), kc, vc, dev(pg.slot_mapping))
    torch.cuda.synchronize()
    ref_k, ref_v = _bits(pg.k_cache).copy(), _bits(pg.v_cache).copy()
    oracle.kv_store(_bits(pg.k_new), _bits(pg.v_new), ref_k, ref_v, pg.slot_mapping.numpy())
    assert np.array_equal(_bits(kc), ref_k)
    assert np.array_equal(_bits(vc), ref_v)


def test_kv_store_skips_negative_and_out_of_range_slots():
    log("kv_store negative / out-of-range slots")
    nb, bs, hkv, d = 4, 64, 2, 128
    kc = torch.full((nb, bs, hkv, d), 7, dtype=torch.int16).view(torch.bfloat16)
    vc = torch.full((nb, bs, hkv, d), 9, dtype=torch.int16).view(torch.bfloat16)
    g = torch.Generator().manual_seed(3)
    kn = torch.randn(6, hkv, d, generator=g).to(torch.bfloat16)
    vn = torch.randn(6, hkv, d, generator=g).to(torch.bfloat16)
    slots = torch.tensor([5, -1, 255, nb * bs, 64, -7], dtype=torch.int32)
    kd, vd = dev(kc), dev(vc)
    attn.kv_store_slots(dev(kn), dev(vn), kd, vd, dev(slots))
    torch.cuda.synchronize()
    rk, rv = _bits(kc).copy(), _bits(vc).copy()
    keep = slots.clone()
    keep[keep >= nb * bs] = -1          # the library skips slots beyond the cache
    oracle.kv_store(_bits(kn), _bits(vn), rk, rv, keep.numpy())
    assert np.array_equal(_bits(kd), rk) and np.array_equal(_bits(vd), rv)


def test_kv_store_empty_is_noop():
    kc = torch.zeros(2, 64, 1, 128, dtype=torch.bfloat16, device="cuda")
    e = torch.zeros(0, 1, 128, dtype=torch.bfloat16, device="cuda")
    attn.kv_store_slots(e, e, kc, kc.clone(), torch.zeros(0, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert kc.abs().sum().item() == 0
