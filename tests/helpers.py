"""Shared helpers for the GPU parity tests: device transfer, oracle calls on
the exact inputs the GPU sees, and the tolerances.

Tolerances (fixed by the accuracy targets of this project):
* fp32 inputs: max |gpu - oracle| <= 1e-5;
* bf16 inputs, fp32 output: max abs <= 1e-2 and mean abs <= 1e-3 against the
  fp64 oracle computed on the same bf16-rounded inputs;
* bf16 output: against the oracle rounded to bf16, within 1e-2 plus one
  bf16 ulp of the reference value (both compared values are rounded to bf16,
  each by up to half an ulp; the rounding alone can exceed 1e-2 for |O| >= 2);
* KV store and paging: bit-exact.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 1e-2
BF16_MEAN_ABS = 1e-3


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().cuda()


def oracle_varlen(vl, rows=None, causal=None) -> np.ndarray:
    return oracle.attn_varlen(np32(vl.q), np32(vl.k), np32(vl.v), vl.cu_seqlens_q.numpy(),
                              vl.cu_seqlens_k.numpy(), vl.softmax_scale,
                              vl.causal if causal is None else causal, rows=rows)


def errs(got, ref):
    d = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def check_f32(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx, mean = errs(got, ref)
    log(f"  {what}: fp32 max abs {mx:.3e} mean abs {mean:.3e}")
    assert mx <= F32_MAX_ABS, f"{what}: max abs {mx:.3e} > {F32_MAX_ABS}"


def check_bf16(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx, mean = errs(got, ref)
    log(f"  {what}: bf16 max abs {mx:.3e} mean abs {mean:.3e}")
    assert mx <= BF16_MAX_ABS, f"{what}: max abs {mx:.3e} > {BF16_MAX_ABS}"
    assert mean <= BF16_MEAN_ABS, f"{what}: mean abs {mean:.3e} > {BF16_MEAN_ABS}"


def check_bf16_output(got_bf16: torch.Tensor, ref, what=""):
    """bf16-valued output vs the oracle rounded to bf16 (RNE)."""
    ref = np.asarray(ref, dtype=np.float64)
    ref_b = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    got = got_bf16.detach().double().cpu().numpy()
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mag = np.maximum(np.abs(ref_b), 2.0 ** -126)
    ulp = 2.0 ** (np.floor(np.log2(mag)) - 7)       # bf16: 8 significant bits
    bound = BF16_MAX_ABS + ulp
    diff = np.abs(got - ref_b)
    excess = diff - bound
    mean = float(diff.mean()) if diff.size else 0.0
    log(f"  {what}: bf16-out max |diff| {diff.max():.3e} mean |diff| {mean:.3e} "
        f"(vs unrounded oracle {np.abs(got - ref).mean():.3e}), max excess over bound {excess.max():.3e}")
    assert np.all(excess <= 0), f"{what}: bf16 output outside 1e-2 + 1 ulp"
    assert mean <= BF16_MEAN_ABS, f"{what}: bf16-out mean abs {mean:.3e} > {BF16_MEAN_ABS}"


def unit_rows(total_q: int, hq: int, hkv: int, every: int, block: int = 64) -> np.ndarray:
    """Flat (token * hq + head) rows of every `every`-th (query block, KV
    head) unit of one sequence: block qb of KV head g is taken when
    (qb - 2 g) mod every == 0, so each KV head contributes blocks spread
    evenly over the whole sequence, and each taken unit is complete (all
    `block` positions of all hq / hkv query heads of that KV head)."""
    group = hq // hkv
    rows = []
    for g in range(hkv):
        for qb in range((2 * g) % every, -(-total_q // block), every):
            t = np.arange(qb * block, min((qb + 1) * block, total_q), dtype=np.int64)
            for h in range(g * group, (g + 1) * group):
                rows.append(t * hq + h)
    return np.sort(np.concatenate(rows))


def sample_rows(cu_q: torch.Tensor, hq: int, n: int, seed: int) -> np.ndarray:
    """Flat (token * hq + head) rows: the first and last token of every
    sequence for several heads, plus n random rows."""
    rng = np.random.default_rng(seed)
    cu = cu_q.tolist()
    rows = []
    for b in range(len(cu) - 1):
        if cu[b + 1] > cu[b]:
            for t in (cu[b], cu[b + 1] - 1, (cu[b] + cu[b + 1]) // 2):
                for h in (0, hq // 2, hq - 1):
                    rows.append(t * hq + h)
    total = cu[-1]
    if total > 0:
        rows.extend((rng.integers(0, total, n) * hq + rng.integers(0, hq, n)).tolist())
    return np.unique(np.asarray(rows, dtype=np.int64))


# fp16 inputs: the kernels round P to fp16 (relative error <= 2^-11 per
# weight, doubled at most by the normalisation) and accumulate in fp32, so
# with |V| <= ~5.5 the output error is below 2 * 2^-11 * 5.5 ~ 5.4e-3; the
# bar is half the bf16 one.
F16_MAX_ABS = 5e-3
F16_MEAN_ABS = 5e-4


def check_f16(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx, mean = errs(got, ref)
    log(f"  {what}: fp16 max abs {mx:.3e} mean abs {mean:.3e}")
    assert mx <= F16_MAX_ABS, f"{what}: max abs {mx:.3e} > {F16_MAX_ABS}"
    assert mean <= F16_MEAN_ABS, f"{what}: mean abs {mean:.3e} > {F16_MEAN_ABS}"


def check_f16_output(got_f16: torch.Tensor, ref, what=""):
    """fp16-valued output vs the oracle rounded to fp16 (RNE)."""
    ref = np.asarray(ref, dtype=np.float64)
    ref_h = ref.astype(np.float16).astype(np.float64)
    got = got_f16.detach().double().cpu().numpy()
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mag = np.maximum(np.abs(ref_h), 2.0 ** -14)
    ulp = 2.0 ** (np.floor(np.log2(mag)) - 10)      # fp16: 11 significant bits
    excess = np.abs(got - ref_h) - (F16_MAX_ABS + ulp)
    log(f"  {what}: fp16-out max |diff| {np.abs(got - ref_h).max():.3e}")
    assert np.all(excess <= 0), f"{what}: fp16 output outside 5e-3 + 1 ulp"
