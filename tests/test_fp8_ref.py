"""Pins of the oracle's OCP E4M3 reference (oracle/fp8.py)."""
import numpy as np
import pytest
import torch

from oracle import fp8


def test_decode_table_closed_forms():
    t = fp8.e4m3_decode_table()
    assert t[0x7E] == 448.0                 # largest finite magnitude 1.75 * 2^8
    assert t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9             # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9         # largest subnormal
    assert t[0x08] == 2.0 ** -6             # smallest normal
    assert t[0x38] == 1.0                   # exponent field 7 = bias
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)         # positive codes are ordered by value
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])


def test_decode_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t = fp8.e4m3_decode_table()
    same = (t == ref) | (np.isnan(t) & np.isnan(ref))
    assert same.all()


def _sweep():
    rng = np.random.default_rng(7)
    t = fp8.e4m3_decode_table()
    finite = np.sort(np.unique(t[np.isfinite(t)]))
    mids = (finite[1:] + finite[:-1]) / 2              # exact ties between neighbours
    dense = np.linspace(-448, 448, 400001)
    tiny = np.linspace(-2.0 ** -5, 2.0 ** -5, 20001)   # subnormal range and its edge
    rnd = rng.standard_normal(100000) * 50
    x = np.concatenate([finite, mids, dense, tiny, rnd, [0.0, -0.0]])
    x = x[np.abs(x) <= 448]
    return x.astype(np.float32)


def test_encode_matches_torch_cast():
    x = _sweep()
    ours = fp8.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, (x[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_encode_is_nearest_ties_to_even_by_search():
    t = fp8.e4m3_decode_table()
    codes = np.array([c for c in range(256) if np.isfinite(t[c])])
    rng = np.random.default_rng(3)
    finite = np.sort(np.unique(t[codes]))
    mids = (finite[1:] + finite[:-1]) / 2
    x = np.concatenate([rng.uniform(-448, 448, 3000), mids, rng.uniform(-0.02, 0.02, 2000)]).astype(np.float32)
    ours = fp8.e4m3_encode(x)
    for v, got in zip(x.astype(np.float64), ours):
        d = np.abs(t[codes] - v)
        best = codes[d == d.min()]
        vals = {t[c] for c in best}
        if len(vals) > 1:                       # a tie: the even mantissa wins
            best = [c for c in best if (c & 1) == 0]
        if v == 0:
            assert t[got] == 0
        else:
            assert got in best, (v, got, best)


def test_encode_saturates_and_keeps_sign():
    x = np.array([448.0, 460.0, 464.0, 500.0, 1e6, -1e6, np.inf, -np.inf, -0.0, -1e-9, np.nan], np.float32)
    got = fp8.e4m3_encode(x)
    assert list(got[:8]) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE]
    assert got[8] == 0x80 and got[9] == 0x80 and got[10] == 0x7F


def test_quantize_rows():
    rng = np.random.default_rng(11)
    rows = rng.standard_normal((64, 576)).astype(np.float32)
    rows[3] = 0.0
    rows[4] *= 1e-30                               # amax far below 1: inv is large but finite
    codes, scale = fp8.quantize_rows(rows)
    t = fp8.e4m3_decode_table()
    assert scale[3] == 1.0 and np.all(codes[3] == 0)
    for r in (0, 1, 4, 63):
        amax_idx = np.argmax(np.abs(rows[r]))
        assert abs(t[codes[r, amax_idx]]) == 448.0
        deq = t[codes[r]] * np.float64(scale[r])
        assert np.all(np.abs(deq - rows[r]) <= np.abs(rows[r]) * 2.0 ** -4 + np.float64(scale[r]) * 2.0 ** -10)
    # one row equals the row-at-a-time form
    c1, s1 = fp8.quantize_row(rows[1])
    assert np.array_equal(c1, codes[1]) and s1 == scale[1]
