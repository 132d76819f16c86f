"""Pins of the oracle's projections around the decode step (CPU only).

- cache_rows: the new cache row [c | k^R] of a token (page "MLA deep compression", sections
  "Low-rank projection" and "Decoupled RoPE");
- query_rows: the absorbed query (W^UK_i)^T W^Q_i h and the RoPE query (same page, section
  "Absorption: an equivalent rewrite at inference" with W^QK_i = (W^UK_i)^T W^Q_i);
- output_projection / fold_output_weights: y = sum_i W^O_i W^UV_i u_i ("Attention-head anatomy",
  section 5: W^UV folds into W^O).

Each is checked against pure-Python scalar loops (rotations as complex exponentials at arbitrary
positions), against independently pinned oracle functions (project_tiny, absorb_query,
mla_nonabsorbed), and against the explicit products the pages describe (W^QK_i, W^O_i W^UV_i);
planted mistakes must fail.
"""
import cmath
import math

import numpy as np
import pytest

from mla_latent_kv_03_amd import workloads
from oracle import mla_ref as ref

from test_oracle_projections import _matvec, _pairs, _theta


def _rot(vec, pos, base=10000.0):
    th = _theta(len(vec), base)
    out = []
    for m, z in enumerate(_pairs(vec)):
        r = z * cmath.exp(1j * pos * th[m])
        out += [r.real, r.imag]
    return out


def _maxrel(got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    return float(np.max(np.abs(got - want)) / max(1.0, float(np.max(np.abs(want)))))


def _small(seed, n_h=3, d=7, d_c=6, d_h=4, d_r=4, d_v=5):
    rng = np.random.default_rng(seed)
    return dict(h=rng.standard_normal((4, d)), dkv=rng.standard_normal((d_c, d)), kr=rng.standard_normal((d_r, d)),
                q=rng.standard_normal((n_h * d_h, d)), uk=rng.standard_normal((n_h, d_h, d_c)),
                qr=rng.standard_normal((n_h * d_r, d)), uv=rng.standard_normal((n_h, d_v, d_c)),
                o=rng.standard_normal((d, n_h * d_v)), n_h=n_h, d_h=d_h, d_r=d_r, d_v=d_v, d_c=d_c)


POS = [3, 1000, 65535, 131071]


# ------------------------------------------------------------------ cache_rows

def cache_rows_errors(fn, w):
    c, k_r = fn(w["h"], w["dkv"], w["kr"], np.array(POS))
    err = 0.0
    for t in range(len(POS)):
        h = w["h"][t].tolist()
        err = max(err, _maxrel(c[t], _matvec(w["dkv"].tolist(), h)))
        err = max(err, _maxrel(k_r[t], _rot(_matvec(w["kr"].tolist(), h), POS[t])))
    return err


def test_cache_rows_scalar_loops():
    assert cache_rows_errors(ref.cache_rows, _small(1)) <= 1e-12


def test_cache_rows_equal_tiny_layer_projections():
    layer = workloads.tiny_layer(seed=1)
    c, k_r, _, _ = ref.project_tiny(layer["h"], layer, 8, 16, 16)
    c2, k2 = ref.cache_rows(layer["h"], layer["dkv"], layer["kr"], np.arange(layer["L"]))
    assert np.array_equal(c, c2) and np.max(np.abs(k_r - k2)) <= 1e-14


# ------------------------------------------------------------------ query_rows

def query_rows_errors(fn, w):
    n_h, d_h, d_r = w["n_h"], w["d_h"], w["d_r"]
    q_nope, q_pe = fn(w["h"], w["q"], w["uk"], w["qr"], np.array(POS))
    err = 0.0
    for t in range(len(POS)):
        h = w["h"][t].tolist()
        for i in range(n_h):
            # the page's precomputed W^QK_i = (W^UK_i)^T W^Q_i, formed entry by entry
            wq = w["q"][i * d_h:(i + 1) * d_h]
            uk = w["uk"][i]
            wqk = [[sum(uk[k][cc] * wq[k][m] for k in range(d_h)) for m in range(wq.shape[1])]
                   for cc in range(uk.shape[1])]
            err = max(err, _maxrel(q_nope[t, i], _matvec(wqk, h)))
            err = max(err, _maxrel(q_pe[t, i], _rot(_matvec(w["qr"][i * d_r:(i + 1) * d_r].tolist(), h), POS[t])))
    return err


def test_query_rows_scalar_loops():
    assert query_rows_errors(ref.query_rows, _small(2)) <= 1e-12


def test_query_rows_equal_tiny_layer_absorption():
    layer = workloads.tiny_layer(seed=1)
    _, _, q_c, q_r = ref.project_tiny(layer["h"], layer, 8, 16, 16)
    qn, qp = ref.query_rows(layer["h"], layer["q"], layer["uk"], layer["qr"], np.arange(layer["L"]))
    for t in (0, 64, 127):
        assert np.max(np.abs(qn[t] - ref.absorb_query(q_c[t], layer["uk"]))) <= 1e-13
        assert np.max(np.abs(qp[t] - q_r[t])) <= 1e-14


# ------------------------------------------------------------------ output side

def output_errors(proj, fold, w):
    rng = np.random.default_rng(7)
    o = rng.standard_normal((2, w["n_h"], w["d_v"]))
    y = proj(o, w["o"])
    err = 0.0
    for r in range(2):
        want = [sum(w["o"][k][i * w["d_v"] + v] * o[r, i, v] for i in range(w["n_h"]) for v in range(w["d_v"]))
                for k in range(w["o"].shape[0])]
        err = max(err, _maxrel(y[r], want))
    # folded weights: entry (k, i*d_c + c) = sum_v W^O[k, i*d_v + v] W^UV_i[v, c]
    f = fold(w["o"], w["uv"])
    d_c = w["d_c"]
    for i in range(w["n_h"]):
        for k in range(w["o"].shape[0]):
            want = [sum(w["o"][k][i * w["d_v"] + v] * w["uv"][i][v][cc] for v in range(w["d_v"])) for cc in range(d_c)]
            err = max(err, _maxrel(f[k, i * d_c:(i + 1) * d_c], want))
    return err


def test_output_projection_and_fold_scalar_loops():
    assert output_errors(ref.output_projection, ref.fold_output_weights, _small(3)) <= 1e-12


def test_folded_output_equals_plain_attention_then_w_o():
    """The tiny layer: plain multi-head attention with explicit keys and values
    (mla_nonabsorbed), its head outputs through W^O, equals sum_i W^OV_i u_i with u from the
    absorbed form and the folded W^OV."""
    layer = workloads.tiny_layer(seed=1)
    rng = np.random.default_rng(11)
    w_o = rng.standard_normal((64, 8 * 16)) / math.sqrt(8 * 16)
    c, k_r, q_c, q_r = ref.project_tiny(layer["h"], layer, 8, 16, 16)
    t = 127
    o_n, _ = ref.mla_nonabsorbed(c, k_r, q_c[t], q_r[t], layer["uk"], layer["uv"], layer["scale"], t + 1)
    y_plain = ref.output_projection(o_n, w_o)
    _, _, u = ref.mla_absorbed(ref.absorb_query(q_c[t], layer["uk"]), q_r[t], c, k_r, layer["uv"], layer["scale"], t + 1)
    y_fold = ref.fold_output_weights(w_o, layer["uv"]) @ u.reshape(-1)
    assert np.max(np.abs(y_plain - y_fold)) / np.max(np.abs(y_plain)) <= 1e-12


# ------------------------------------------------------------------ planted mistakes

def test_adjacent_mutants_are_caught():
    w = _small(4)

    def rows_rope_off_by_one(h, dkv, kr, pos, base=10000.0):
        return ref.cache_rows(h, dkv, kr, np.asarray(pos) + 1, base)

    def rows_unrotated(h, dkv, kr, pos, base=10000.0):
        c, _ = ref.cache_rows(h, dkv, kr, pos, base)
        return c, np.asarray(h, float) @ np.asarray(kr, float).T

    def query_heads_swapped(h, wq, uk, wqr, pos, base=10000.0):
        return ref.query_rows(h, wq, uk[::-1], wqr, pos, base)

    def query_rope_at_zero(h, wq, uk, wqr, pos, base=10000.0):
        return ref.query_rows(h, wq, uk, wqr, np.zeros_like(pos), base)

    def proj_blocks_reversed(o, w_o):
        return ref.output_projection(np.asarray(o)[..., ::-1, :], w_o)

    def fold_next_head(w_o, w_uv):
        return ref.fold_output_weights(w_o, np.roll(w_uv, 1, axis=0))

    assert cache_rows_errors(rows_rope_off_by_one, w) > 1e-6
    assert cache_rows_errors(rows_unrotated, w) > 1e-6
    assert query_rows_errors(query_heads_swapped, w) > 1e-6
    assert query_rows_errors(query_rope_at_zero, w) > 1e-6
    assert output_errors(proj_blocks_reversed, ref.fold_output_weights, w) > 1e-6
    assert output_errors(ref.output_projection, fold_next_head, w) > 1e-6
