"""Host logic of the test helpers: the unit subset used for the 32K-token
parity check covers every KV head and the whole sequence, in whole units."""
import numpy as np

from tests.helpers import unit_rows


def test_unit_rows_cover_heads_and_sequence():
    total, hq, hkv, every = 32768, 32, 8, 16
    rows = unit_rows(total, hq, hkv, every)
    assert rows.size * every == total * hq          # exactly 1/16 of the rows
    tok, head = rows // hq, rows % hq
    g = head // (hq // hkv)
    qb = tok // 64
    assert set(g.tolist()) == set(range(hkv))
    for gg in range(hkv):
        blocks = np.unique(qb[g == gg])
        assert blocks.size == total // 64 // every
        assert blocks.min() < every and blocks.max() >= total // 64 - every   # start to end
        assert np.all(np.diff(blocks) == every)
    # each taken unit is complete: 64 positions x 4 query heads
    units, counts = np.unique(qb * hkv + g, return_counts=True)
    assert np.all(counts == 64 * (hq // hkv))


def test_unit_rows_ragged_tail():
    rows = unit_rows(100, 4, 2, every=1)           # every unit: all rows, tail included
    assert np.array_equal(rows, np.arange(400))
    rows = unit_rows(100, 4, 2, every=2)           # KV head 1 starts at block 2 % 2 = 0
    assert np.array_equal(rows // 4, np.repeat(np.arange(64), 4))
