"""The split rule (oracle.mla_ref.split_table) against a unit-by-unit brute force."""
import numpy as np
import pytest

from oracle import bruteforce as bf
from oracle import mla_ref as ref


def _check(seq_lens, G):
    table, pieces = ref.split_table(seq_lens, G)
    table2, pieces2 = bf.split_table(seq_lens, G)
    assert np.array_equal(table, np.array(table2, dtype=np.int64).reshape(table.shape))
    assert pieces == pieces2
    cap = ref.num_slots(len(seq_lens), G)
    slots = [p[2] for p in pieces]
    assert len(set(slots)) == len(slots) and all(0 <= s < cap for s in slots)
    for b, L in enumerate(seq_lens):
        mine = sorted((p[3], p[4]) for p in pieces if p[0] == b)
        covered = []
        for t0, t1 in mine:
            assert t0 < t1 and t0 % 64 == 0
            covered.extend(range(t0, t1))
        assert covered == list(range(int(L)))
    return table, pieces


@pytest.mark.parametrize("seed", range(12))
def test_random_batches(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    lens = rng.integers(0, 3000, size=B)
    lens[rng.random(B) < 0.2] = 0
    for G in (1, 3, 8, 64, 256, 1000):
        _check(lens, G)


def test_workload_shapes():
    # 64 x 4096 over 256 shares: 4 pieces of 1024 tokens each per sequence
    table, pieces = _check([4096] * 64, 256)
    assert all(t[1] == 4 for t in table) and all(p[4] - p[3] == 1024 for p in pieces)
    # 4 x 131072 over 256 shares: 64 pieces of 2048 tokens
    table, pieces = _check([131072] * 4, 256)
    assert all(t[1] == 64 for t in table) and all(p[4] - p[3] == 2048 for p in pieces)


def test_degenerate():
    table, pieces = _check([0, 0, 0], 4)
    assert pieces == [] and np.all(table == 0)
    _check([1], 1)
    _check([1], 300)
    _check([65, 0, 1, 64, 63], 2)
