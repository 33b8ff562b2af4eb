"""Property tests of the fp64 oracle (CPU only), drawn by hypothesis: facts
the blog post "从零实现 vLLM (1.3)：如何加速 Attention 计算" states or that
follow from the definition of attention, checked on random inputs rather
than on fixed examples.

* 在线 Softmax: the 2-pass online softmax equals the 3-pass safe softmax for
  any input, including shifts far beyond exp's range.
* softmax is shift-invariant, so attention is unchanged when every logit of
  a row moves by the same amount (a Q component that meets a constant K
  column).
* every output row is a convex combination of the visible V rows (rows of A
  are non-negative and sum to 1): it lies inside their per-column range.
* 计算流程 (varlen packing): attention of a packed batch equals attention of
  each sequence on its own; without the causal mask, permuting the keys (and
  their values) changes nothing.
"""
import numpy as np
from hypothesis import given, settings, strategies as st

import oracle

SET = settings(max_examples=60, deadline=None)


def rng_arrays(seed, *shapes):
    g = np.random.default_rng(seed)
    return [g.standard_normal(s).astype(np.float32) for s in shapes]


@SET
@given(st.lists(st.floats(-50, 50), min_size=1, max_size=40), st.floats(-1e6, 1e6))
def test_online_equals_safe_for_any_shift(xs, shift):
    x = np.array(xs, dtype=np.float64) + shift
    safe = oracle.softmax_safe3(x)
    online, _, _ = oracle.softmax_online2(x)
    assert np.all(np.isfinite(safe)) and abs(safe.sum() - 1.0) < 1e-12
    np.testing.assert_allclose(online, safe, rtol=1e-12, atol=1e-300)


@SET
@given(st.integers(1, 12), st.integers(1, 12), st.integers(0, 2**31 - 1), st.booleans(),
       st.floats(-20, 20))
def test_logit_shift_leaves_attention_unchanged(lq, extra, seed, causal, c):
    lk = lq + extra
    d = 8
    q, k, v = rng_arrays(seed, (lq, 1, d), (lk, 1, d), (lk, 1, d))
    cu_q, cu_k = np.array([0, lq], np.int32), np.array([0, lk], np.int32)
    base = oracle.attn_varlen(q, k, v, cu_q, cu_k, 0.5, causal)
    # a new Q component 1 against a constant K column c adds 0.5*c to every logit
    q2 = np.concatenate([q, np.ones((lq, 1, 1), np.float32)], axis=2)
    k2 = np.concatenate([k, np.full((lk, 1, 1), c, np.float32)], axis=2)
    v2 = np.concatenate([v, np.zeros((lk, 1, 1), np.float32)], axis=2)
    shifted = oracle.attn_varlen(q2, k2, v2, cu_q, cu_k, 0.5, causal)[..., :d]
    np.testing.assert_allclose(shifted, base, rtol=1e-11, atol=1e-12)


@SET
@given(st.integers(1, 10), st.integers(0, 10), st.integers(0, 2**31 - 1), st.booleans(),
       st.floats(0.01, 4.0))
def test_output_rows_are_convex_combinations_of_visible_values(lq, extra, seed, causal, scale):
    lk = lq + extra
    d = 6
    q, k, v = rng_arrays(seed, (lq, 2, d), (lk, 1, d), (lk, 1, d))
    q *= 3.0
    o = oracle.attn_varlen(q, k, v, np.array([0, lq], np.int32), np.array([0, lk], np.int32), scale, causal)
    for i in range(lq):
        n_vis = min(lk, lk - lq + i + 1) if causal else lk
        vis = v[:n_vis, 0].astype(np.float64)
        for h in range(2):
            assert np.all(o[i, h] >= vis.min(0) - 1e-12) and np.all(o[i, h] <= vis.max(0) + 1e-12)


@SET
@given(st.lists(st.tuples(st.integers(0, 9), st.integers(0, 9)), min_size=1, max_size=5),
       st.integers(0, 2**31 - 1), st.booleans())
def test_packed_batch_equals_sequences_alone(lens, seed, causal):
    lq = [a for a, _ in lens]
    lk = [a + b for a, b in lens]
    hq, hkv, d = 4, 2, 8
    q, k, v = rng_arrays(seed, (sum(lq), hq, d), (sum(lk), hkv, d), (sum(lk), hkv, d))
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    packed = oracle.attn_varlen(q, k, v, cu_q, cu_k, 0.3, causal)
    for b in range(len(lens)):
        if lq[b] == 0:
            continue
        qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        alone = oracle.attn_varlen(q[qs], k[ks], v[ks], np.array([0, lq[b]], np.int32),
                                   np.array([0, lk[b]], np.int32), 0.3, causal)
        np.testing.assert_array_equal(packed[qs], alone)


@SET
@given(st.integers(1, 8), st.integers(1, 16), st.integers(0, 2**31 - 1))
def test_noncausal_key_permutation_invariance(lq, lk, seed):
    d = 8
    q, k, v = rng_arrays(seed, (lq, 2, d), (lk, 1, d), (lk, 1, d))
    perm = np.random.default_rng(seed + 1).permutation(lk)
    cu_q, cu_k = np.array([0, lq], np.int32), np.array([0, lk], np.int32)
    a = oracle.attn_varlen(q, k, v, cu_q, cu_k, 0.4, False)
    b = oracle.attn_varlen(q, k[perm], v[perm], cu_q, cu_k, 0.4, False)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
