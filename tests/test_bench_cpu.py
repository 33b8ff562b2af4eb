"""Host logic of bench.py (no GPU): the algorithmic pair count behind every
TFLOP/s figure, the per-sequence bound, and the rule that a recorded HBM
traffic figure is reported only while the kernel sources are unchanged."""
import numpy as np

import bench


def brute_pairs(lq, lk, causal):
    """(query, key) pairs the end-aligned causal mask keeps, by enumeration:
    query i of a sequence sees key j iff j <= i + (Lk - Lq)."""
    total = 0
    for a, b in zip(lq, lk):
        for i in range(a):
            for j in range(b):
                if not causal or j <= i + (b - a):
                    total += 1
    return total


def cu(lens):
    return [0] + list(np.cumsum(lens))


def test_visible_pairs_matches_enumeration():
    rng = np.random.default_rng(3)
    for _ in range(40):
        n = int(rng.integers(1, 6))
        lq = [int(x) for x in rng.integers(0, 40, size=n)]
        lk = [int(x) for x in rng.integers(0, 40, size=n)]     # Lq > Lk included: empty rows
        for causal in (True, False):
            assert bench.visible_pairs(cu(lq), cu(lk), causal) == brute_pairs(lq, lk, causal)


def test_visible_pairs_closed_forms():
    # Lq = Lk = L under the causal mask: the lower triangle, L (L + 1) / 2
    for L in (1, 2, 63, 64, 65, 1000):
        assert bench.visible_pairs([0, L], [0, L], True) == L * (L + 1) // 2
    # the 32768-token sequence: 4 * d * Hq * pairs = 8.796e12 flops
    pairs = bench.visible_pairs([0, 32768], [0, 32768], True)
    assert pairs == 32768 * 32769 // 2
    assert 4 * 128 * 32 * pairs == 8796361457664
    # decode (one query attending to Lk keys) and a prefix of P cached keys
    assert bench.visible_pairs([0, 1], [0, 500], True) == 500
    assert bench.visible_pairs([0, 3], [0, 10], True) == 8 + 9 + 10


def test_per_sequence_bound_is_the_larger_roof():
    P = bench.PEAK_BF16_TFLOPS * 1e12
    BW = bench.PEAK_HBM_GBS * 1e9
    for lq, lk in ((1, 4096), (512, 16384), (4096, 4096)):
        fl = 4.0 * 128 * 32 * bench.visible_pairs([0, lq], [0, lk], True)
        by = 2.0 * 128 * (2 * lq * 32 + 2 * lk * 8)
        assert abs(bench.per_sequence_bound([0, lq], [0, lk]) - max(fl / P, by / BW)) < 1e-15
    # a batch is the sum of its sequences
    both = bench.per_sequence_bound([0, 1, 513], [0, 4096, 4096 + 16384])
    one = bench.per_sequence_bound([0, 1], [0, 4096]) + bench.per_sequence_bound([0, 512], [0, 16384])
    assert abs(both - one) < 1e-15


def test_recorded_traffic_needs_matching_sources(tmp_path, monkeypatch):
    sha = bench.source_sha("prefill")                    # the sources as they are
    (tmp_path / "good.md").write_text(f"traffic_bytes_per_launch: 1234\nkernel_source_sha256: {sha}\n")
    (tmp_path / "stale.md").write_text("traffic_bytes_per_launch: 1234\nkernel_source_sha256: 0000\n")
    monkeypatch.setattr(bench, "source_sha", lambda which: sha)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_FILES", {"good": ("prefill", "good.md"), "stale": ("prefill", "stale.md"),
                                                 "missing": ("prefill", "none.md")})
    assert bench.recorded_traffic("good") == 1234.0
    assert bench.recorded_traffic("stale") is None
    assert bench.recorded_traffic("missing") is None


def test_committed_traffic_records_match_the_kernels():
    """Every FETCH_SIZE / WRITE_SIZE record in profiles/ was taken on the
    kernel sources as committed (re-take them after changing a kernel)."""
    for w in bench.TRAFFIC_FILES:
        assert bench.recorded_traffic(w) is not None, w
