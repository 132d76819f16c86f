"""Pins of the GQLA per-group path of the oracle (CPU only).

The GQLA abstract (chatpaper.ai) states that its weights expose two algebraically equivalent
decoding paths: an MQA-absorb path identical to MLA's and a GQA path with a per-group expanded
cache.  With the heads of a group sharing W^UK_g and W^UV_g, the GQA path over
k_{j,g} = W^UK_g c_j, v_{j,g} = W^UV_g c_j must equal the absorbed decode with
q~_i = (W^UK_g)^T q^C_i and o_i = W^UV_g u_i, and the plain (non-absorbed) attention with
per-head weights repeated over each group.
"""
import numpy as np
import pytest

from oracle import bruteforce as bf
from oracle import mla_ref as ref


def _case(seed, n_h=8, n_g=2, L=40, d_c=24, d_h=6, d_r=4, d_v=5):
    rng = np.random.default_rng(seed)
    return dict(c=rng.standard_normal((L, d_c)), k_r=rng.standard_normal((L, d_r)),
                q_c=rng.standard_normal((n_h, d_h)), q_r=rng.standard_normal((n_h, d_r)),
                uk=rng.standard_normal((n_g, d_h, d_c)) / np.sqrt(d_c), uv=rng.standard_normal((n_g, d_v, d_c)),
                n_h=n_h, n_g=n_g, scale=0.3)


def _per_head(w, n_h):
    return np.repeat(w, n_h // w.shape[0], axis=0)


@pytest.mark.parametrize("seed,n_h,n_g,n_vis", [(1, 8, 2, 40), (2, 8, 8, 17), (3, 6, 1, 1), (4, 16, 4, 33)])
def test_gqa_path_equals_absorbed_path(seed, n_h, n_g, n_vis):
    w = _case(seed, n_h=n_h, n_g=n_g)
    k, v = ref.gqla_expand(w["c"], w["uk"], w["uv"])
    o_g, lse_g = ref.gqla_decode(w["q_c"], w["q_r"], k, v, w["k_r"], w["scale"], n_vis)
    uk_h, uv_h = _per_head(w["uk"], n_h), _per_head(w["uv"], n_h)
    o_a, lse_a, _ = ref.mla_absorbed(ref.absorb_query(w["q_c"], uk_h), w["q_r"], w["c"], w["k_r"], uv_h, w["scale"],
                                     n_vis)
    assert np.max(np.abs(o_g - o_a)) / np.max(np.abs(o_a)) <= 1e-12
    assert np.max(np.abs(lse_g - lse_a)) <= 1e-12


def test_gqa_path_bruteforce():
    w = _case(5, n_h=4, n_g=2, L=7, d_c=5, d_h=3, d_r=2, d_v=3)
    k, v = ref.gqla_expand(w["c"], w["uk"], w["uv"])
    o_g, lse_g = ref.gqla_decode(w["q_c"], w["q_r"], k, v, w["k_r"], w["scale"], 6)
    o_b, lse_b = bf.nonabsorbed_decode(w["c"].tolist(), w["k_r"].tolist(), w["q_c"].tolist(), w["q_r"].tolist(),
                                       _per_head(w["uk"], 4).tolist(), _per_head(w["uv"], 4).tolist(), w["scale"], 6)
    assert np.max(np.abs(o_g - np.array(o_b))) <= 1e-13
    assert np.max(np.abs(lse_g - np.array(lse_b))) <= 1e-13
    # expansion entries by scalar loops
    for j in range(7):
        for g in range(2):
            for kk in range(3):
                assert abs(k[j, g, kk] - sum(w["uk"][g][kk][cc] * w["c"][j][cc] for cc in range(5))) <= 1e-13


def test_gqa_path_mutants_caught():
    w = _case(6)
    k, v = ref.gqla_expand(w["c"], w["uk"], w["uv"])
    want, _ = ref.gqla_decode(w["q_c"], w["q_r"], k, v, w["k_r"], w["scale"], 40)
    o_a, _, _ = ref.mla_absorbed(ref.absorb_query(w["q_c"], _per_head(w["uk"], 8)), w["q_r"], w["c"], w["k_r"],
                                 _per_head(w["uv"], 8), w["scale"], 40)
    assert np.max(np.abs(want - o_a)) <= 1e-12
    # heads interleaved over groups (i % n_g) instead of consecutive blocks (i // per)
    uk_bad = np.tile(w["uk"], (4, 1, 1))
    o_bad, _, _ = ref.mla_absorbed(ref.absorb_query(w["q_c"], uk_bad), w["q_r"], w["c"], w["k_r"],
                                   np.tile(w["uv"], (4, 1, 1)), w["scale"], 40)
    assert np.max(np.abs(want - o_bad)) > 1e-3
    # the expanded value taken from W^UK instead of W^UV (shapes permitting)
    w2 = _case(7, d_v=6)
    k2, _ = ref.gqla_expand(w2["c"], w2["uk"], w2["uv"])
    o_bad2, _ = ref.gqla_decode(w2["q_c"], w2["q_r"], k2, k2, w2["k_r"], w2["scale"], 40)
    o_ok2, _, _ = ref.mla_absorbed(ref.absorb_query(w2["q_c"], _per_head(w2["uk"], 8)), w2["q_r"], w2["c"], w2["k_r"],
                                   _per_head(w2["uv"], 8), w2["scale"], 40)
    assert np.max(np.abs(o_bad2 - o_ok2)) > 1e-3
