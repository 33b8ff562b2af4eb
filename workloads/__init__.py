"""Seeded synthetic inputs for the attention hot path.

This module only draws numbers and lays them out in memory: sequence
lengths, Q/K/V values, the physical block pool of a paged KV cache, the
block table and the slot mapping.  It holds none of the attention arithmetic,
so that the CPU oracle and the GPU library can both be fed from it without
sharing any computation.

Everything is produced on the CPU with ``torch.Generator().manual_seed(seed)``
and returned as CPU tensors.  bf16 inputs are drawn in float32 and rounded to
bf16 (round-to-nearest-even) before either side sees them; the oracle reads
the exact bf16 values upcast to float32.

Layouts (from the blog post "从零实现 vLLM (1.3)：如何加速 Attention 计算",
sections Prefill and Decode):

* packed varlen q [total_q, Hq, d], k/v [total_k, Hkv, d]; sequence b owns
  rows cu_seqlens[b] .. cu_seqlens[b+1]-1;
* paged caches [num_blocks, block_size, Hkv, d]; block_table [batch,
  max_blocks] int32 of physical block ids, padded with -1;
* slot_mapping [T_new] int32, slot = block_id * block_size + offset.

Cache slots that hold no live token are filled with a NaN sentinel so that a
kernel which reads past a sequence's length cannot go unnoticed.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

BF16_NAN_BITS = 0x7FC1  # quiet NaN pattern used as the "no live token" sentinel


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _randn(g, shape, std, dtype):
    # drawn as one flat vector, then viewed with the requested shape
    n = 1
    for s in shape:
        n *= int(s)
    x = torch.randn(n, generator=g, dtype=torch.float32).view(*shape)
    if std != 1.0:
        x = x * std
    return x.to(dtype)


def _cumsum0(lengths) -> torch.Tensor:
    out = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    if len(lengths):
        out[1:] = torch.cumsum(torch.as_tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return out


def sentinel_like(shape, dtype) -> torch.Tensor:
    """A tensor of the given shape filled with NaN (bf16: a fixed quiet NaN)."""
    if dtype == torch.bfloat16:
        return torch.full(shape, BF16_NAN_BITS, dtype=torch.int16).view(torch.bfloat16)
    return torch.full(shape, float("nan"), dtype=dtype)


@dataclass
class Varlen:
    """A packed variable-length batch (contiguous K/V)."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    cu_seqlens_q: torch.Tensor
    cu_seqlens_k: torch.Tensor
    max_seqlen_q: int
    max_seqlen_k: int
    softmax_scale: float
    causal: bool = True
    name: str = ""

    @property
    def batch(self) -> int:
        return self.cu_seqlens_q.numel() - 1


@dataclass
class Paged:
    """A paged KV cache holding each sequence's first ``prefix_lens[b]`` tokens,
    plus the new tokens still to be stored through ``slot_mapping``.

    ``k_logical``/``v_logical`` [total_k, Hkv, d] hold every token of every
    sequence (prefix and new) in logical order at offsets ``cu_seqlens_k``;
    the oracle reads only these.  ``k_new``/``v_new`` are the rows of the new
    tokens, in order, and ``slot_mapping`` says where each one goes."""
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    k_logical: torch.Tensor
    v_logical: torch.Tensor
    cu_seqlens_k: torch.Tensor
    seqlens_k: torch.Tensor
    prefix_lens: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    slot_mapping: torch.Tensor
    block_size: int
    max_blocks_per_seq: int

    @property
    def num_blocks(self) -> int:
        return self.k_cache.shape[0]


def varlen(lens_q, lens_k, hq, hkv, d, dtype=torch.bfloat16, seed=0,
           q_std=1.0, k_std=1.0, v_std=1.0, scale=None, causal=True, name="") -> Varlen:
    """Packed q/k/v for sequences with the given query/key lengths."""
    lens_q = [int(x) for x in lens_q]
    lens_k = [int(x) for x in lens_k]
    g = _gen(seed)
    tq, tk = sum(lens_q), sum(lens_k)
    q = _randn(g, (tq, hq, d), q_std, dtype)
    k = _randn(g, (tk, hkv, d), k_std, dtype)
    v = _randn(g, (tk, hkv, d), v_std, dtype)
    return Varlen(q, k, v, _cumsum0(lens_q), _cumsum0(lens_k),
                  max(lens_q) if lens_q else 0, max(lens_k) if lens_k else 0,
                  (1.0 / math.sqrt(d)) if scale is None else float(scale), causal, name)


def paged_pool(k_logical, v_logical, cu_seqlens_k, prefix_lens, block_size,
               seed=0, spare_blocks=0, max_blocks_per_seq=None) -> Paged:
    """Lay sequences out in a randomly permuted pool of physical blocks.

    Sequence b needs ceil(Lk_b / block_size) blocks; physical ids come from a
    seeded permutation of the pool and are handed to sequences in order.
    Tokens [0, prefix_lens[b]) are placed in the pool now; the remaining
    tokens become k_new/v_new with their slot_mapping.  Every other slot holds
    the NaN sentinel."""
    g = _gen(seed)
    cu = [int(x) for x in cu_seqlens_k.tolist()]
    batch = len(cu) - 1
    lens = [cu[b + 1] - cu[b] for b in range(batch)]
    prefix = [int(x) for x in torch.as_tensor(prefix_lens).tolist()]
    nblk = [(L + block_size - 1) // block_size for L in lens]
    num_blocks = sum(nblk) + int(spare_blocks)
    mbs = max(nblk) if max_blocks_per_seq is None else int(max_blocks_per_seq)
    perm = torch.randperm(num_blocks, generator=g).to(torch.int32)
    block_table = torch.full((batch, max(mbs, 1)), -1, dtype=torch.int32)
    pos = 0
    for b in range(batch):
        block_table[b, :nblk[b]] = perm[pos:pos + nblk[b]]
        pos += nblk[b]
    hkv, d = k_logical.shape[1], k_logical.shape[2]
    dtype = k_logical.dtype
    k_cache = sentinel_like((num_blocks, block_size, hkv, d), dtype)
    v_cache = sentinel_like((num_blocks, block_size, hkv, d), dtype)
    new_rows, slots = [], []
    for b in range(batch):
        L, P = lens[b], prefix[b]
        j = torch.arange(L)
        phys = block_table[b, (j // block_size)].to(torch.int64)
        off = j % block_size
        # place the prefix tokens
        kp = k_logical[cu[b]:cu[b] + P]
        vp = v_logical[cu[b]:cu[b] + P]
        k_cache[phys[:P], off[:P]] = kp
        v_cache[phys[:P], off[:P]] = vp
        # the rest are new tokens, stored later through slot_mapping
        new_rows.append(torch.arange(cu[b] + P, cu[b] + L))
        slots.append((phys[P:] * block_size + off[P:]).to(torch.int32))
    rows = torch.cat(new_rows) if new_rows else torch.zeros(0, dtype=torch.int64)
    return Paged(k_cache, v_cache, block_table, k_logical, v_logical,
                 torch.as_tensor(cu, dtype=torch.int32), torch.as_tensor(lens, dtype=torch.int32),
                 torch.as_tensor(prefix, dtype=torch.int32),
                 k_logical[rows].contiguous(), v_logical[rows].contiguous(),
                 torch.cat(slots) if slots else torch.zeros(0, dtype=torch.int32),
                 block_size, max(mbs, 1))


# ---------------------------------------------------------------------------
# The five named workloads (and scaled-down versions of them for tests).
# ---------------------------------------------------------------------------

def fp32_single_head(L=256, d=64, seed=1001) -> Varlen:
    """fp32 causal attention: batch 1, one head, L=256, head_dim 64, Q/K/V
    i.i.d. N(0,1), scale 1/sqrt(64)."""
    return varlen([L], [L], 1, 1, d, torch.float32, seed, name="fp32_single_head_L256_d64")


def fp32_stress(L=256, d=64, seed=1001) -> Varlen:
    """The large-logit stress input for the fp32 path.  Every query row is
    (8, 0, ..., 0) and the scale is 1/8, so the scaled logit of key j is
    exactly K[j, 0].  K[0:3, 0] = 700, 710, 705 (the overflow example of the
    safe-softmax section); K[j, 0] = 700 + delta_j for j >= 3 with delta_j
    drawn from N(0, 5^2) and rounded to a 2^-8 grid, so every logit is an
    exact float32.  Other K columns are N(0, 1) (they meet zeros in q).
    V is N(0, 1).  Causal, so row i is a softmax over the prefix 0..i."""
    g = _gen(seed + 500)
    q = torch.zeros(L, 1, d, dtype=torch.float32)
    q[:, 0, 0] = 8.0
    k = _randn(g, (L, 1, d), 1.0, torch.float32)
    delta = torch.round(torch.randn(L, generator=g, dtype=torch.float32) * 5.0 * 256.0) / 256.0
    col = 700.0 + delta
    col[0], col[1], col[2] = 700.0, 710.0, 705.0
    k[:, 0, 0] = col
    v = _randn(g, (L, 1, d), 1.0, torch.float32)
    cu = _cumsum0([L])
    return Varlen(q, k, v, cu, cu.clone(), L, L, 1.0 / 8.0, True, "fp32_stress_L256_d64")


def fp16_stress(L=300, hq=8, hkv=2, d=128, seed=1601) -> Varlen:
    """The large-logit stress input for fp16 inputs (the overflow example of
    the safe-softmax section, with fp16 named as the type that overflows).
    Every query row is (16, 0, ..., 0) and the scale is 1/16, so the scaled
    logit of key j is exactly K[j, 0] (the products are exact in fp32).
    K[0:3, 0] = 700, 710, 705; K[j, 0] = 700 + delta_j for j >= 3 with
    delta_j drawn from N(0, 5^2) and rounded to a 2^-1 grid, so every logit
    is an exact fp16 value.  Other K columns are N(0, 1) (they meet zeros in
    q).  V is N(0, 1).  Causal, one sequence, GQA heads sharing the K
    column."""
    g = _gen(seed)
    q = torch.zeros(L, hq, d, dtype=torch.float32)
    q[:, :, 0] = 16.0
    k = torch.randn(L, hkv, d, generator=g, dtype=torch.float32)
    delta = torch.round(torch.randn(L, generator=g, dtype=torch.float32) * 5.0 * 2.0) / 2.0
    col = 700.0 + delta
    col[0], col[1], col[2] = 700.0, 710.0, 705.0
    k[:, :, 0] = col[:, None]
    v = torch.randn(L, hkv, d, generator=g, dtype=torch.float32)
    cu = _cumsum0([L])
    return Varlen(q.to(torch.float16), k.to(torch.float16), v.to(torch.float16), cu, cu.clone(),
                  L, L, 1.0 / 16.0, True, f"fp16_stress_L{L}")


def varlen_prefill(n_seqs=16, lo=128, hi=4096, hq=32, hkv=8, d=128, seed=1002,
                   dtype=torch.bfloat16) -> Varlen:
    """Varlen causal prefill: n_seqs sequences with lengths uniform in
    [lo, hi], packed via cu_seqlens (Lq = Lk), GQA hq/hkv, Q/K/V N(0,1)."""
    g = _gen(seed)
    lens = torch.randint(lo, hi + 1, (n_seqs,), generator=g).tolist()
    return varlen(lens, lens, hq, hkv, d, dtype, seed + 7,
                  name=f"varlen_prefill_{n_seqs}x[{lo},{hi}]_h{hq}/{hkv}_d{d}")


def long_prefill(L=32768, hq=32, hkv=8, d=128, seed=1005, dtype=torch.bfloat16) -> Varlen:
    """Long-context causal prefill: batch 1, Q/K ~ N(0, 4) (sigma 2, large
    logits that exercise the max rescaling), V ~ N(0, 1)."""
    return varlen([L], [L], hq, hkv, d, dtype, seed, q_std=2.0, k_std=2.0, v_std=1.0,
                  name=f"long_prefill_L{L}_h{hq}/{hkv}_d{d}")


@dataclass
class PrefixPrefill:
    """Prefix-cache prefill: q holds only the new tokens; K/V of the whole
    context come from the paged cache (prefix already cached, new tokens
    stored through slot_mapping first)."""
    q: torch.Tensor
    cu_seqlens_q: torch.Tensor
    max_seqlen_q: int
    max_seqlen_k: int
    softmax_scale: float
    paged: Paged
    name: str = ""

    @property
    def batch(self) -> int:
        return self.cu_seqlens_q.numel() - 1


def prefix_prefill(n_seqs=32, q_lo=1, q_hi=512, p_lo=1024, p_hi=16384, hq=32, hkv=8,
                   d=128, block_size=256, seed=1004, dtype=torch.bfloat16) -> PrefixPrefill:
    """Prefix-cache prefill: new-token lengths uniform in [q_lo, q_hi], cached
    prefixes uniform in [p_lo, p_hi], Lk = prefix + Lq, block size 256."""
    g = _gen(seed)
    lq = torch.randint(q_lo, q_hi + 1, (n_seqs,), generator=g).tolist()
    pre = torch.randint(p_lo, p_hi + 1, (n_seqs,), generator=g).tolist()
    lk = [a + b for a, b in zip(lq, pre)]
    base = varlen(lq, lk, hq, hkv, d, dtype, seed + 7)
    pg = paged_pool(base.k, base.v, base.cu_seqlens_k, pre, block_size, seed + 13)
    return PrefixPrefill(base.q, base.cu_seqlens_q, max(lq), max(lk), base.softmax_scale, pg,
                         f"prefix_prefill_{n_seqs}x(q[{q_lo},{q_hi}]+p[{p_lo},{p_hi}])_bs{block_size}")


def shared_prefix_prefill(n_seqs=6, shared_blocks=3, own_lo=0, own_hi=300, q_lo=1, q_hi=150,
                          hq=8, hkv=2, d=128, block_size=64, seed=0,
                          dtype=torch.bfloat16) -> PrefixPrefill:
    """Sequences that share a cached prompt: every block table begins with the
    same ``shared_blocks`` physical blocks (stored once, read by all), then
    each sequence's own cached tokens (uniform in [own_lo, own_hi]) and its new
    tokens (uniform in [q_lo, q_hi]), which are the queries and are stored
    through slot_mapping.  The logical K/V of every sequence begins with the
    same prompt rows, so the oracle needs no knowledge of the sharing."""
    g = _gen(seed)
    S = shared_blocks * block_size
    own = torch.randint(own_lo, own_hi + 1, (n_seqs,), generator=g).tolist()
    lq = torch.randint(q_lo, q_hi + 1, (n_seqs,), generator=g).tolist()
    lk = [S + o + q for o, q in zip(own, lq)]
    base = varlen(lq, lk, hq, hkv, d, dtype, seed + 7)
    cu = [int(x) for x in base.cu_seqlens_k.tolist()]
    for b in range(1, n_seqs):                        # the same prompt in every sequence
        base.k[cu[b]:cu[b] + S] = base.k[0:S]
        base.v[cu[b]:cu[b] + S] = base.v[0:S]
    own_blocks = [(L - S + block_size - 1) // block_size for L in lk]
    num_blocks = shared_blocks + sum(own_blocks)
    perm = torch.randperm(num_blocks, generator=g).to(torch.int32)
    mbs = shared_blocks + max(own_blocks)
    block_table = torch.full((n_seqs, mbs), -1, dtype=torch.int32)
    pos = shared_blocks
    for b in range(n_seqs):
        block_table[b, :shared_blocks] = perm[:shared_blocks]
        block_table[b, shared_blocks:shared_blocks + own_blocks[b]] = perm[pos:pos + own_blocks[b]]
        pos += own_blocks[b]
    k_cache = sentinel_like((num_blocks, block_size, hkv, d), dtype)
    v_cache = sentinel_like((num_blocks, block_size, hkv, d), dtype)
    j = torch.arange(S)
    shared_phys = perm[:shared_blocks].to(torch.int64)[j // block_size]
    k_cache[shared_phys, j % block_size] = base.k[0:S]
    v_cache[shared_phys, j % block_size] = base.v[0:S]
    new_rows, slots = [], []
    for b in range(n_seqs):
        jj = torch.arange(S, lk[b])
        phys = block_table[b, jj // block_size].to(torch.int64)
        off = jj % block_size
        P = own[b]                                    # own cached tokens: positions S .. S + P
        k_cache[phys[:P], off[:P]] = base.k[cu[b] + S:cu[b] + S + P]
        v_cache[phys[:P], off[:P]] = base.v[cu[b] + S:cu[b] + S + P]
        new_rows.append(torch.arange(cu[b] + S + P, cu[b] + lk[b]))
        slots.append((phys[P:] * block_size + off[P:]).to(torch.int32))
    rows = torch.cat(new_rows)
    pg = Paged(k_cache, v_cache, block_table, base.k, base.v,
               torch.as_tensor(cu, dtype=torch.int32), torch.as_tensor(lk, dtype=torch.int32),
               torch.as_tensor([S + o for o in own], dtype=torch.int32),
               base.k[rows].contiguous(), base.v[rows].contiguous(), torch.cat(slots),
               block_size, mbs)
    return PrefixPrefill(base.q, base.cu_seqlens_q, max(lq), max(lk), base.softmax_scale, pg,
                         f"shared_prefix_{n_seqs}x({S}+[{own_lo},{own_hi}]+[{q_lo},{q_hi}])_bs{block_size}")


@dataclass
class Decode:
    """Single-token decode against a paged cache.  The cache holds the first
    ctx-1 tokens of each sequence; the new token's K/V are stored through
    slot_mapping first, then every one of the ctx tokens is attended to."""
    q: torch.Tensor
    softmax_scale: float
    paged: Paged
    name: str = ""

    @property
    def batch(self) -> int:
        return self.q.shape[0]


def paged_decode(batch=64, lo=512, hi=8192, hq=32, hkv=8, d=128, block_size=256,
                 seed=1003, dtype=torch.bfloat16, spare_blocks=0) -> Decode:
    """Paged-KV decode: context lengths uniform in [lo, hi] (including the new
    token), block size 256, permuted pool, max_blocks_per_seq = ceil(hi/256)."""
    g = _gen(seed)
    ctx = torch.randint(lo, hi + 1, (batch,), generator=g).tolist()
    base = varlen([1] * batch, ctx, hq, hkv, d, dtype, seed + 7)
    mbs = (hi + block_size - 1) // block_size
    pg = paged_pool(base.k, base.v, base.cu_seqlens_k, [c - 1 for c in ctx], block_size,
                    seed + 13, spare_blocks=spare_blocks, max_blocks_per_seq=mbs)
    return Decode(base.q.view(batch, hq, d), base.softmax_scale, pg,
                  f"paged_decode_b{batch}_ctx[{lo},{hi}]_bs{block_size}_h{hq}/{hkv}_d{d}")


def cache_for_varlen(vl: Varlen, block_size=256, seed=0) -> Paged:
    """An empty paged cache sized for a varlen batch, with the slot mapping
    that stores every token of it (the store that precedes prefill)."""
    return paged_pool(vl.k, vl.v, vl.cu_seqlens_k, [0] * vl.batch, block_size, seed)
