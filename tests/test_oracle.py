"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself: closed forms derived
by hand from the pages' definitions and evaluated in 50-digit decimal
arithmetic, invariants the pages state (blocked == unblocked, varlen ==
padded, rows of A sum to 1), brute force on tiny inputs (numpy with X and A
materialised, torch's CPU fp64 scaled_dot_product_attention with an explicit
boolean mask), and special cases with known answers.  The last test plants
plausible mistakes in copies of oracle.c and checks that these pins catch
every one of them.

Pages: blog post "从零实现 vLLM (1.3)：如何加速 Attention 计算".
"""
import decimal
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.golden import load as load_golden

D = decimal.Decimal
decimal.getcontext().prec = 50


def exact_softmax(x):
    """50-digit decimal softmax by the definition (max subtracted, which does
    not change the value)."""
    xs = [D(repr(float(t))) for t in x]
    m = max(xs)
    e = [(t - m).exp() for t in xs]
    s = sum(e)
    return [float(t / s) for t in e]


def rel_close(a, b, tol):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return np.all(np.abs(a - b) <= tol * np.maximum(np.abs(b), 1e-300))


def to_np(t):
    return t.float().numpy() if t.dtype != torch.float32 else t.numpy()


# ---------------------------------------------------------------------------
# Pin batteries.  Each check_* raises AssertionError on a mismatch; they take
# the oracle library as an argument so the planted-mistake test can run them
# against modified builds.
# ---------------------------------------------------------------------------

def check_overflow_example(orc):
    """Section "安全 Softmax"的提出 / 解决方法: [700, 710, 705]."""
    x = load_golden("safe_softmax_overflow.txt")["x"]
    closed = [math.exp(-10), 1.0, math.exp(-5)]
    s = sum(closed)
    closed = [c / s for c in closed]
    exact = exact_softmax(x)
    assert rel_close(exact, closed, 1e-15)
    got = orc.softmax_safe3(x)
    assert np.all(np.isfinite(got)), got
    assert rel_close(got, exact, 1e-14), (got, exact)
    got2, _, _ = orc.softmax_online2(x)
    assert rel_close(got2, exact, 1e-14), (got2, exact)
    # the max may sit anywhere in the vector: a first element far below the
    # maximum must not leak into the exponent either
    x2 = [0.0, 750.0, 745.0]
    got3 = orc.softmax_safe3(x2)
    assert np.all(np.isfinite(got3)) and rel_close(got3, exact_softmax(x2), 1e-14), got3
    # negative control: the naive formula overflows (e^710 > DBL_MAX)
    with np.errstate(all="ignore"):
        naive = orc.softmax_naive(x)
    assert not np.all(np.isfinite(naive)), naive


def check_online_example(orc):
    """Section 在线 Softmax (2-Pass) worked example [10, 0, 8, 12, 5]: the running
    maxima, the proxy denominators d'_i = sum_{j<=i} e^{x_j - m_i} (evaluated
    from this definition, not from the recurrence the oracle runs), and the
    final result, which must equal the 3-pass result."""
    x = load_golden("online_softmax_example.txt")["x"]
    out, m, dprime = orc.softmax_online2(x)
    assert list(m) == [10.0, 10.0, 10.0, 12.0, 12.0], m
    for i in range(len(x)):
        mi = max(x[: i + 1])
        want = float(sum((D(xj) - D(mi)).exp() for xj in x[: i + 1]))
        assert abs(dprime[i] - want) <= 1e-15 * want, (i, dprime[i], want)
    # spot values of d'_i written out by hand
    assert abs(dprime[1] - (1 + math.exp(-10))) < 1e-15
    assert abs(dprime[4] - (math.exp(-2) + math.exp(-12) + math.exp(-4) + 1 + math.exp(-7))) < 1e-15
    exact = exact_softmax(x)
    assert rel_close(out, exact, 1e-14)
    assert rel_close(orc.softmax_safe3(x), exact, 1e-14)
    assert np.max(np.abs(out - orc.softmax_safe3(x))) < 1e-15


def check_softmax_random(orc):
    rng = np.random.default_rng(5)
    for n, off, sc in [(1, 0, 1), (2, 0, 1), (17, 1000.0, 3.0), (64, -500.0, 10.0), (33, 0.0, 0.01)]:
        x = rng.standard_normal(n) * sc + off
        exact = exact_softmax(x)
        assert rel_close(orc.softmax_safe3(x), exact, 1e-13)
        assert rel_close(orc.softmax_online2(x)[0], exact, 1e-13)
        assert abs(sum(orc.softmax_safe3(x)) - 1) < 1e-14


def brute_numpy(q, k, v, cu_q, cu_k, scale, causal):
    """Materialise X = s Q K^T and A = softmax(X) per sequence and head with
    numpy (section 标准实现方法), visible set aligned to the sequence end."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    out = np.zeros(q.shape, dtype=np.float64)
    hq, hkv = q.shape[1], k.shape[1]
    for b in range(len(cu_q) - 1):
        qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        for h in range(hq):
            g = h * hkv // hq
            X = scale * q[qs, h, :] @ k[ks, g, :].T
            vis = np.ones((lq, lk), dtype=bool)
            if causal:
                vis = np.arange(lk)[None, :] <= (np.arange(lq)[:, None] + lk - lq)
            X = np.where(vis, X, -np.inf)
            for i in range(lq):
                if not vis[i].any():
                    continue
                a = np.exp(X[i] - X[i].max())
                a /= a.sum()
                out[cu_q[b] + i, h] = a @ v[ks, g, :]
    return out


def torch_sdpa_fp64(q, k, v, cu_q, cu_k, scale, causal):
    """torch's CPU fp64 scaled_dot_product_attention, one sequence at a time,
    with an explicit boolean mask (bottom-right aligned)."""
    q, k, v = (torch.as_tensor(np.asarray(t, dtype=np.float64)) for t in (q, k, v))
    hq, hkv = q.shape[1], k.shape[1]
    out = torch.zeros_like(q)
    for b in range(len(cu_q) - 1):
        lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        if lq == 0 or lk == 0:
            continue
        qb = q[cu_q[b]:cu_q[b + 1]].transpose(0, 1)                      # [hq, lq, d]
        kb = k[cu_k[b]:cu_k[b + 1]].transpose(0, 1).repeat_interleave(hq // hkv, 0)
        vb = v[cu_k[b]:cu_k[b + 1]].transpose(0, 1).repeat_interleave(hq // hkv, 0)
        mask = torch.ones(lq, lk, dtype=torch.bool)
        if causal:
            mask = torch.arange(lk)[None, :] <= (torch.arange(lq)[:, None] + lk - lq)
        rows_ok = mask.any(1)
        o = torch.nn.functional.scaled_dot_product_attention(
            qb.contiguous(), kb.contiguous(), vb.contiguous(), attn_mask=mask, scale=scale)
        o = o * rows_ok[None, :, None]
        out[cu_q[b]:cu_q[b + 1]] = o.transpose(0, 1)
    return out.numpy()


def exact_decimal_attention(q, k, v, cu_q, cu_k, scale, causal):
    """50-digit decimal attention on tiny inputs (the exact result)."""
    hq, hkv, d = q.shape[1], k.shape[1], q.shape[2]
    out = np.zeros(q.shape, dtype=np.float64)
    sc = D(repr(float(scale)))
    for b in range(len(cu_q) - 1):
        lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        for i in range(lq):
            nv = min(lk, lk - lq + i + 1) if causal else lk
            if nv <= 0:
                continue
            for h in range(hq):
                g = h * hkv // hq
                qi = [D(repr(float(t))) for t in q[cu_q[b] + i, h]]
                xs = []
                for j in range(nv):
                    kj = [D(repr(float(t))) for t in k[cu_k[b] + j, g]]
                    xs.append(sc * sum(a * c for a, c in zip(qi, kj)))
                m = max(xs)
                e = [(x - m).exp() for x in xs]
                s = sum(e)
                for c in range(d):
                    out[cu_q[b] + i, h, c] = float(sum(
                        e[j] / s * D(repr(float(v[cu_k[b] + j, g, c]))) for j in range(nv)))
    return out


def _np32(vl):
    return to_np(vl.q), to_np(vl.k), to_np(vl.v)


def check_brute_force(orc):
    """Tiny random batches with GQA, Lq < Lk, Lq == Lk, causal and not."""
    cases = [([3, 1, 4], [5, 1, 4], 4, 2, 8, 0.3, True),
             ([2, 6], [2, 6], 2, 2, 4, 0.5, True),
             ([4], [7], 4, 1, 16, 0.25, False),
             ([1, 5], [3, 5], 6, 3, 8, 1.0, True)]
    for i, (lq, lk, hq, hkv, d, sc, causal) in enumerate(cases):
        vl = workloads.varlen(lq, lk, hq, hkv, d, torch.float32, seed=100 + i, scale=sc,
                              causal=causal)
        q, k, v = _np32(vl)
        cu_q, cu_k = vl.cu_seqlens_q.tolist(), vl.cu_seqlens_k.tolist()
        got = orc.attn_varlen(q, k, v, cu_q, cu_k, sc, causal)
        ref1 = brute_numpy(q, k, v, cu_q, cu_k, sc, causal)
        ref2 = torch_sdpa_fp64(q, k, v, cu_q, cu_k, sc, causal)
        assert np.max(np.abs(got - ref1)) < 1e-13, (i, np.max(np.abs(got - ref1)))
        assert np.max(np.abs(got - ref2)) < 1e-13, (i, np.max(np.abs(got - ref2)))


def check_exact_tiny(orc):
    vl = workloads.varlen([3, 2], [4, 2], 2, 1, 3, torch.float32, seed=7, scale=0.7)
    q, k, v = _np32(vl)
    cu_q, cu_k = vl.cu_seqlens_q.tolist(), vl.cu_seqlens_k.tolist()
    got = orc.attn_varlen(q, k, v, cu_q, cu_k, 0.7, True)
    exact = exact_decimal_attention(q, k, v, cu_q, cu_k, 0.7, True)
    assert np.max(np.abs(got - exact)) < 1e-14, np.max(np.abs(got - exact))


def check_rows_of_A(orc):
    """With V = identity (value j is the j-th unit vector), output row i is
    row i of A itself: entries in (0, 1] on the visible keys, exactly 0 on the
    hidden ones, summing to 1 (sections 标准实现方法 second step)."""
    lk, lq = 12, 12
    d = lk
    rng = np.random.default_rng(3)
    q = (rng.standard_normal((lq, 1, d)) * 2).astype(np.float32)
    k = (rng.standard_normal((lk, 1, d)) * 2).astype(np.float32)
    v = np.eye(lk, dtype=np.float32)[:, None, :]
    A = orc.attn_varlen(q, k, v, [0, lq], [0, lk], 1 / math.sqrt(d), True)[:, 0, :]
    for i in range(lq):
        row = A[i]
        assert np.all(row[: i + 1] > 0) and np.all(row[: i + 1] <= 1)
        assert np.all(row[i + 1:] == 0)
        assert abs(row.sum() - 1) < 1e-14
    X = (q[:, 0, :].astype(np.float64) @ k[:, 0, :].T.astype(np.float64)) / math.sqrt(d)
    for i in range(lq):
        assert rel_close(A[i, : i + 1], exact_softmax(X[i, : i + 1]), 1e-13)


def flash_recurrence(q, k, v, scale, n_vis, tile, deferred):
    """The FlashAttention one-pass recurrence (sections FlashAttention 的最终实现
    and 计算流程(1-Pass 算法与分块)) in fp64 for one query row: K/V are cut
    into tiles along the sequence and the state (m, d', o') is updated tile
    by tile.  deferred=False keeps o' normalised at every step as the page's
    recurrence does; deferred=True keeps it unnormalised and divides once."""
    m, dp, o = -np.inf, 0.0, np.zeros(v.shape[1])
    for t0 in range(0, n_vis, tile):
        x = scale * (k[t0:min(t0 + tile, n_vis)] @ q)
        vt = v[t0:min(t0 + tile, n_vis)]
        m_new = max(m, x.max())
        carry = 0.0 if dp == 0.0 else dp * math.exp(m - m_new)
        e = np.exp(x - m_new)
        d_new = carry + e.sum()
        if deferred:
            o = o * (0.0 if dp == 0.0 else math.exp(m - m_new)) + e @ vt
        else:
            o = o * (carry / d_new) + (e @ vt) / d_new
        m, dp = m_new, d_new
    return o / dp if deferred else o


def check_blocked_equals_unblocked(orc):
    L, d = 70, 16
    vl = workloads.varlen([L], [L], 1, 1, d, torch.float32, seed=11, k_std=3.0)
    q, k, v = (a.astype(np.float64) for a in _np32(vl))
    sc = 0.5
    ref = orc.attn_varlen(*_np32(vl), [0, L], [0, L], sc, True)[:, 0, :]
    for tile in (1, 2, 3, 7, 64, L):
        for deferred in (False, True):
            for i in (0, 1, 5, 33, L - 1):
                got = flash_recurrence(q[i, 0], k[:, 0], v[:, 0], sc, i + 1, tile, deferred)
                assert np.max(np.abs(got - ref[i])) < 1e-12, (tile, deferred, i)
    # split-and-merge: two partial states over disjoint key ranges combine
    # into the full result (the same associativity the tiles rely on).
    i = L - 1
    parts = []
    for lo, hi in ((0, 23), (23, 51), (51, L)):
        x = sc * (k[lo:hi, 0] @ q[i, 0])
        m = x.max()
        e = np.exp(x - m)
        parts.append((m, e.sum(), e @ v[lo:hi, 0]))
    M = max(p[0] for p in parts)
    l = sum(p[1] * math.exp(p[0] - M) for p in parts)
    o = sum(p[2] * math.exp(p[0] - M) for p in parts) / l
    assert np.max(np.abs(o - ref[i])) < 1e-12


def check_varlen_equals_padded(orc):
    """Section Prefill: the varlen layout addressed by cu_seqlens gives the
    same outputs as a padded [batch, max_len, H, d] layout with length masks."""
    g = load_golden("varlen_example.txt")
    cu_q, cu_k = g["cu_seqlens_q"], g["cu_seqlens_k"]
    lq = [cu_q[i + 1] - cu_q[i] for i in range(3)]
    lk = [cu_k[i + 1] - cu_k[i] for i in range(3)]
    assert lq == [5, 2, 1] and lk == [9, 7, 3] and max(lq) == g["padded_q_len"][0]
    for d in (8, 128):
        vl = workloads.varlen(lq, lk, 2, 2, d, torch.float32, seed=21 + d)
        q, k, v = _np32(vl)
        got = orc.attn_varlen(q, k, v, cu_q, cu_k, vl.softmax_scale, True)
        # padded layout: zero padding, masks by length and causal alignment
        Pq, Pk = max(lq), max(lk)
        qp = np.zeros((3, Pq, 2, d)); kp = np.zeros((3, Pk, 2, d)); vp = np.zeros((3, Pk, 2, d))
        for b in range(3):
            qp[b, :lq[b]] = q[cu_q[b]:cu_q[b + 1]]
            kp[b, :lk[b]] = k[cu_k[b]:cu_k[b + 1]]
            vp[b, :lk[b]] = v[cu_k[b]:cu_k[b + 1]]
        for b in range(3):
            for h in range(2):
                X = vl.softmax_scale * qp[b, :, h] @ kp[b, :, h].T          # [Pq, Pk]
                i = np.arange(Pq)[:, None]
                j = np.arange(Pk)[None, :]
                valid = (j < lk[b]) & (j <= i + lk[b] - lq[b])
                X = np.where(valid, X, -np.inf)
                for r in range(lq[b]):
                    a = np.exp(X[r] - X[r].max()); a /= a.sum()
                    assert np.max(np.abs(a @ vp[b, :, h] - got[cu_q[b] + r, h])) < 1e-13


def check_special_cases(orc):
    rng = np.random.default_rng(9)
    d = 8
    # Lk = 1: the only key gets weight 1, O = V_0 exactly
    q = rng.standard_normal((1, 2, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, d)).astype(np.float32)
    v = rng.standard_normal((1, 1, d)).astype(np.float32)
    o = orc.attn_varlen(q, k, v, [0, 1], [0, 1], 0.3, True)
    assert np.array_equal(o[0, 0], v[0, 0].astype(np.float64))
    assert np.array_equal(o[0, 1], v[0, 0].astype(np.float64))
    # Q = 0: all logits equal, O_i = mean of the visible V rows (Lq < Lk)
    lq, lk = 4, 10
    q = np.zeros((lq, 1, d), np.float32)
    k = rng.standard_normal((lk, 1, d)).astype(np.float32)
    v = rng.standard_normal((lk, 1, d)).astype(np.float32)
    o = orc.attn_varlen(q, k, v, [0, lq], [0, lk], 0.3, True)
    for i in range(lq):
        want = v[: lk - lq + i + 1, 0].astype(np.float64).mean(0)
        assert np.max(np.abs(o[i, 0] - want)) < 1e-15
    # all V rows equal c: O = c for every row
    v = np.tile(rng.standard_normal((1, 1, d)).astype(np.float32), (lk, 1, 1))
    q = rng.standard_normal((lq, 1, d)).astype(np.float32)
    o = orc.attn_varlen(q, k, v, [0, lq], [0, lk], 0.3, True)
    assert np.max(np.abs(o[:, 0] - v[0, 0])) < 1e-14
    # causal, Lq == Lk: row 0 sees only key 0, O_0 = V_0
    v2 = rng.standard_normal((lq, 1, d)).astype(np.float32)
    o = orc.attn_varlen(q, k[:lq], v2, [0, lq], [0, lq], 0.3, True)
    assert np.array_equal(o[0, 0], v2[0, 0].astype(np.float64))
    # one-hot logits (gap > 100 after scaling): O = V_target exactly
    k1 = np.zeros((6, 1, d), np.float32)
    k1[3, 0, 0] = 1000.0
    q1 = np.zeros((1, 1, d), np.float32)
    q1[0, 0, 0] = 1.0
    v1 = rng.standard_normal((6, 1, d)).astype(np.float32)
    o = orc.attn_varlen(q1, k1, v1, [0, 1], [0, 6], 0.5, True)
    assert np.array_equal(o[0, 0], v1[3, 0].astype(np.float64))
    # a row that sees no key (Lq > Lk under end alignment) is all zeros
    q3 = rng.standard_normal((3, 1, d)).astype(np.float32)
    o = orc.attn_varlen(q3, k[:1], v[:1], [0, 3], [0, 1], 0.3, True)
    assert np.all(o[:2] == 0) and np.array_equal(o[2, 0], v[0, 0].astype(np.float64))


def check_gqa(orc):
    """Query head h reads KV head h // (hq/hkv): equal to hkv = hq with each
    KV head repeated for its group."""
    vl = workloads.varlen([5, 3], [5, 7], 8, 2, 16, torch.float32, seed=31)
    q, k, v = _np32(vl)
    cu_q, cu_k = vl.cu_seqlens_q.tolist(), vl.cu_seqlens_k.tolist()
    got = orc.attn_varlen(q, k, v, cu_q, cu_k, 0.25, True)
    kr = np.ascontiguousarray(np.repeat(k, 4, axis=1))
    vr = np.ascontiguousarray(np.repeat(v, 4, axis=1))
    ref = orc.attn_varlen(q, kr, vr, cu_q, cu_k, 0.25, True)
    assert np.array_equal(got, ref)
    # and each head really reads a different KV head
    assert np.max(np.abs(got[:, 0] - got[:, 4])) > 1e-3


def check_prefix_equals_full(orc):
    """Prefix-cache prefill (section Prefill, prefix cache): with Q = only the
    new tokens and K/V = the whole context, the outputs equal the last Lq
    rows of a full causal prefill over the same context."""
    lk, lq = 23, 6
    full = workloads.varlen([lk], [lk], 4, 2, 16, torch.float32, seed=41)
    q, k, v = _np32(full)
    ref = orc.attn_varlen(q, k, v, [0, lk], [0, lk], 0.25, True)
    got = orc.attn_varlen(np.ascontiguousarray(q[lk - lq:]), k, v, [0, lq], [0, lk], 0.25, True)
    assert np.array_equal(got, ref[lk - lq:])


def check_decode_equals_last_row(orc):
    """Decode section: one new query against all cached tokens equals the
    last row of causal prefill over the same context."""
    lens = [7, 1, 12]
    full = workloads.varlen(lens, lens, 4, 2, 16, torch.float32, seed=51)
    q, k, v = _np32(full)
    cu = full.cu_seqlens_q.tolist()
    ref = orc.attn_varlen(q, k, v, cu, cu, 0.25, True)
    qd = np.ascontiguousarray(np.stack([q[cu[b + 1] - 1] for b in range(3)]))
    got = orc.attn_decode(qd, k, v, cu, 0.25)
    for b in range(3):
        assert np.array_equal(got[b], ref[cu[b + 1] - 1])


def check_stress_rows(orc):
    """The large-logit input: row 2's weights are the closed form of the
    [700, 710, 705] example, every row is finite."""
    st = workloads.fp32_stress()
    q, k, v = _np32(st)
    L = q.shape[0]
    o = orc.attn_varlen(q, k, v, [0, L], [0, L], st.softmax_scale, True)[:, 0, :]
    assert np.all(np.isfinite(o))
    w = [math.exp(-10), 1.0, math.exp(-5)]
    s = sum(w)
    want = sum((w[j] / s) * v[j, 0].astype(np.float64) for j in range(3))
    assert np.max(np.abs(o[2] - want)) < 1e-14
    assert np.array_equal(o[0], v[0, 0].astype(np.float64))
    for i in (17, 100, L - 1):
        x = k[: i + 1, 0, 0].astype(np.float64)
        want = np.asarray(exact_softmax(x)) @ v[: i + 1, 0].astype(np.float64)
        assert np.max(np.abs(o[i] - want)) < 1e-13


def check_row_subset(orc):
    vl = workloads.varlen([9, 4], [9, 11], 4, 2, 8, torch.float32, seed=61)
    q, k, v = _np32(vl)
    cu_q, cu_k = vl.cu_seqlens_q.tolist(), vl.cu_seqlens_k.tolist()
    full = orc.attn_varlen(q, k, v, cu_q, cu_k, 0.3, True)
    rows = np.array([0, 5, 13, 4 * 9 + 3, 4 * 12 + 2])
    sub = orc.attn_varlen(q, k, v, cu_q, cu_k, 0.3, True, rows=rows)
    for r, flat in enumerate(rows):
        assert np.array_equal(sub[r], full[flat // 4, flat % 4])


ALL_CHECKS = [check_overflow_example, check_online_example, check_softmax_random,
              check_brute_force, check_exact_tiny, check_rows_of_A,
              check_blocked_equals_unblocked, check_varlen_equals_padded,
              check_special_cases, check_gqa, check_prefix_equals_full,
              check_decode_equals_last_row, check_stress_rows, check_row_subset]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=[c.__name__ for c in ALL_CHECKS])
def test_oracle_pin(check):
    check(oracle.default())


def test_kv_store_scatter():
    """store_kvcache (section Attention 源码分析): slot = block * block_size +
    offset; negative slots are skipped; every other slot keeps its value."""
    nb, bs, h, d = 3, 4, 2, 2
    kc = np.full((nb, bs, h, d), -1, dtype=np.int16)
    vc = np.full((nb, bs, h, d), -2, dtype=np.int16)
    kn = np.arange(4 * h * d, dtype=np.int16).reshape(4, h, d)
    vn = kn + 100
    slots = [5, -1, 0, 11]   # block 1 offset 1, skip, block 0 offset 0, block 2 offset 3
    oracle.kv_store(kn, vn, kc, vc, slots)
    assert np.array_equal(kc[1, 1], kn[0]) and np.array_equal(vc[1, 1], vn[0])
    assert np.array_equal(kc[0, 0], kn[2]) and np.array_equal(vc[0, 0], vn[2])
    assert np.array_equal(kc[2, 3], kn[3]) and np.array_equal(vc[2, 3], vn[3])
    touched = {(1, 1), (0, 0), (2, 3)}
    for b in range(nb):
        for o in range(bs):
            if (b, o) not in touched:
                assert np.all(kc[b, o] == -1) and np.all(vc[b, o] == -2)


# ---------------------------------------------------------------------------
# Planted mistakes: every one of these edits to oracle.c must be caught.
# ---------------------------------------------------------------------------

MUTANTS = [
    ("causal offset dropped (top-left alignment)",
     "causal ? (lk - lq + i + 1) : lk", "causal ? (i + 1) : lk"),
    ("causal off by one", "causal ? (lk - lq + i + 1) : lk", "causal ? (lk - lq + i) : lk"),
    ("scale dropped", "x[j] = scale * acc;", "x[j] = acc;"),
    ("GQA mapping interleaved", "const int g = h / group;", "const int g = h % hkv;"),
    ("V read in place of K", "const float *kj = k + j * kv_stride", "const float *kj = v + j * kv_stride"),
    ("V rows at the query offsets",
     "v + (int64_t)cu_k[b] * hkv * d,\n                     (int64_t)hkv * d, g,",
     "v + (int64_t)cu_q[b] * hkv * d,\n                     (int64_t)hkv * d, g,"),
    ("online rescale dropped", "d_prev * exp(m_prev - m_i)", "d_prev"),
    ("online max sign", "exp(x[i] - m_i)", "exp(m_i - x[i])"),
    ("denominator without max", "for (int64_t j = 0; j < n_vis; ++j) den += exp(x[j] - m);",
     "for (int64_t j = 0; j < n_vis; ++j) den += exp(x[j]);"),
    ("decode drops the newest key", "h / group, d, lk, scale, x, o + r * d);",
     "h / group, d, lk - 1, scale, x, o + r * d);"),
    ("empty row not zeroed", "for (int c = 0; c < d; ++c) o[c] = 0.0;\n    if (n_vis <= 0) return;",
     "if (n_vis <= 0) return;\n    for (int c = 0; c < d; ++c) o[c] = 0.0;"),
    ("safe3 max pass skipped", "for (int64_t j = 0; j < n; ++j) if (x[j] > m) m = x[j];          /* pass 1 */",
     "m = x[0];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    src = oracle.source_text()
    assert src.count(old) == 1, f"mutation site not unique/present: {name}"
    variant = oracle.build_variant(src.replace(old, new), str(tmp_path))
    failures = []
    for check in ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(variant)
        except (AssertionError, ValueError):
            failures.append(check.__name__)
    assert failures, f"planted mistake '{name}' passed every pin"
