"""Planted mistakes in the oracle (CPU only): each mutant must fail at least one pin.

This shows that the pins of tests/test_oracle_identities.py and tests/test_fp8_ref.py
would catch a plausible slip (a dropped term, a wrong sign or index, a transposed
operand, an off-by-one visibility) rather than re-deriving the oracle from itself.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from mla_latent_kv_03_amd import workloads
from oracle import bruteforce as bf
from oracle import fp8
from oracle import mla_ref as ref


def _rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(b), 1e-300)


# ------------------------------------------------------------------ pins as functions of an implementation

def pin_identity(absorbed):
    layer = workloads.tiny_layer(seed=1)
    c, k_r, q_c, q_r = ref.project_tiny(layer["h"], layer, 8, 16, 16)
    qa = ref.absorb_query(q_c[127], layer["uk"])
    o_a, lse_a, _ = absorbed(qa, q_r[127], c, k_r, layer["uv"], layer["scale"], 128)
    o_n, lse_n = ref.mla_nonabsorbed(c, k_r, q_c[127], q_r[127], layer["uk"], layer["uv"], layer["scale"], 128)
    return _rel(o_a, o_n) <= 1e-12 and np.max(np.abs(lse_a - lse_n)) <= 1e-12


def pin_sdpa(absorbed):
    rng = np.random.default_rng(5)
    n_h, L, dc, dr, dv = 4, 40, 24, 8, 12
    qn, qp = rng.standard_normal((n_h, dc)), rng.standard_normal((n_h, dr))
    c, kp = rng.standard_normal((L, dc)), rng.standard_normal((L, dr))
    w = rng.standard_normal((n_h, dv, dc))
    sc = 1 / math.sqrt(dv + dr)
    n_vis = 33
    q = torch.from_numpy(np.concatenate([qn, qp], -1))[None, None]
    k = torch.from_numpy(np.concatenate([c, kp], -1)[:n_vis])[None, None]
    u_t = F.scaled_dot_product_attention(q, k, torch.from_numpy(c[:n_vis])[None, None], scale=sc)[0, 0].numpy()
    o, lse, u = absorbed(qn, qp, c, kp, w, sc, n_vis)
    s = sc * (np.concatenate([qn, qp], -1) @ np.concatenate([c, kp], -1)[:n_vis].T)
    return (_rel(u, u_t) <= 1e-12 and _rel(o, np.einsum("ivc,ic->iv", w, u_t)) <= 1e-12
            and np.max(np.abs(lse - torch.logsumexp(torch.from_numpy(s), 1).numpy())) <= 1e-12)


def pin_bruteforce(absorbed):
    rng = np.random.default_rng(6)
    n_h, L, dc, dr, dv = 2, 7, 5, 3, 4
    qn, qp = rng.standard_normal((n_h, dc)), rng.standard_normal((n_h, dr))
    c, kp = rng.standard_normal((L, dc)), rng.standard_normal((L, dr))
    w = rng.standard_normal((n_h, dv, dc))
    o, lse, u = absorbed(qn, qp, c, kp, w, 0.4, 6)
    o2, lse2, u2 = bf.absorbed_decode(qn.tolist(), qp.tolist(), c.tolist(), kp.tolist(), w.tolist(), 0.4, 6)
    return _rel(o, o2) <= 1e-13 and _rel(u, u2) <= 1e-13 and np.max(np.abs(lse - np.array(lse2))) <= 1e-13


def passes_all(absorbed):
    out = []
    for pin in (pin_identity, pin_sdpa, pin_bruteforce):
        try:
            out.append(bool(pin(absorbed)))
        except Exception:
            out.append(False)
    return out


# ------------------------------------------------------------------ mutants of the absorbed form

def _make(score=None, axis=1, vis=0, up=None, lse_mode="ok"):
    def absorbed(q_nope, q_pe, c, k_pe, w_uv, scale, n_vis):
        n = max(n_vis + vis, 1)
        c_, k_ = np.asarray(c, float)[:n], np.asarray(k_pe, float)[:n]
        s = score(q_nope, q_pe, c_, k_, scale) if score else scale * (q_nope @ c_.T + q_pe @ k_.T)
        m = s.max(axis=axis, keepdims=True)
        e = np.exp(s - m)
        den = e.sum(axis=axis, keepdims=True)
        u = (e / den) @ c_
        o = up(w_uv, u) if up else np.einsum("ivc,ic->iv", w_uv, u)
        lse = (m + np.log(den)).reshape(-1)[: q_nope.shape[0]] if lse_mode == "ok" else np.log(den).reshape(-1)
        return o, lse, u
    return absorbed


MUTANTS = {
    "correct": _make(),
    "drop_rope_term": _make(score=lambda qn, qp, c, k, sc: sc * (qn @ c.T)),
    "drop_content_term": _make(score=lambda qn, qp, c, k, sc: sc * (qp @ k.T)),
    "rope_term_sign": _make(score=lambda qn, qp, c, k, sc: sc * (qn @ c.T - qp @ k.T)),
    "scale_missing": _make(score=lambda qn, qp, c, k, sc: qn @ c.T + qp @ k.T),
    "scale_on_content_only": _make(score=lambda qn, qp, c, k, sc: sc * (qn @ c.T) + qp @ k.T),
    "softmax_over_heads": _make(axis=0),
    "sees_one_token_less": _make(vis=-1),
    "sees_one_token_more": _make(vis=+1),
    "w_uv_other_index": _make(up=lambda w, u: np.einsum("ivc,ic->iv", w[::-1], u)),
    "w_uv_transposed": _make(up=lambda w, u: np.einsum("icv,ic->iv", w, u)),
    "lse_without_max": _make(lse_mode="nomax"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    results = passes_all(MUTANTS[name])
    if name == "correct":
        assert all(results), results
    else:
        assert not all(results), f"mutant {name} passed every pin"


# ------------------------------------------------------------------ mutants elsewhere

def test_rope_mutants_caught(monkeypatch):
    good = ref.rope

    def sin_sign(x, pos, base=10000.0):
        return good(x, -np.asarray(pos, float), base)

    def half_split(x, pos, base=10000.0):          # the other common pairing convention
        x = np.asarray(x, float)
        d = x.shape[-1]
        perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
        inv = np.argsort(perm)
        return good(x[..., inv], pos, base)[..., perm]

    for bad in (sin_sign, half_split):
        got = bad(np.array([0.0, 0.0, 1.0, 0.0]), 3.0)
        hand_ok = np.allclose(got, [0, 0, math.cos(0.03), math.sin(0.03)], atol=1e-15, rtol=0)
        got2 = bad(np.array([1.0, 0.0]), 1.0)
        hand_ok = hand_ok and np.allclose(got2, [math.cos(1.0), math.sin(1.0)], atol=1e-15, rtol=0)
        assert not hand_ok


def test_combine_mutant_caught():
    rng = np.random.default_rng(8)
    qn, qp = rng.standard_normal((3, 8)), rng.standard_normal((3, 2))
    c, kp = rng.standard_normal((30, 8)), rng.standard_normal((30, 2))
    _, lse, u = ref.mla_absorbed(qn, qp, c, kp, np.zeros((3, 1, 8)), 0.7, 30)
    parts = [(0, 10), (10, 11), (11, 30)]
    us, ls = map(np.array, zip(*[ref.split_partial(qn, qp, c, kp, 0.7, a, b) for a, b in parts]))

    def unweighted(us, ls):                        # forgets the exp(lse_s - lse) weights
        return us.mean(0), np.log(np.exp(ls).sum(0))

    uc, lc = unweighted(us, ls)
    assert _rel(uc, u) > 1e-6


def test_split_rule_mutant_caught():
    lens = [100, 0, 4096, 70, 1]

    def share_floor(seq_lens, G, unit=64):         # floor instead of ceil for the share size
        units = [-(-L // unit) for L in seq_lens]
        total = sum(units)
        share = max(1, total // G)
        pieces = []
        start = 0
        for b, n in enumerate(units):
            for w in range(start // share, (start + n - 1) // share + 1 if n else start // share):
                u0, u1 = max(w * share, start) - start, min((w + 1) * share, start + n) - start
                pieces.append((b, w, w + b, u0 * unit, min(u1 * unit, seq_lens[b])))
            start += n
        return pieces

    _, good = bf.split_table(lens, 7)
    assert share_floor(lens, 7) != good


def test_fp8_mutant_caught():
    x = np.array([0.5625 * 2 ** -6, 17.0, 240.0, 2.0 ** -10], np.float32)     # ties and the subnormal edge
    ref_codes = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    t = fp8.e4m3_decode_table()
    finite = [c for c in range(128) if np.isfinite(t[c])]

    def half_away(v):                              # rounds ties away from zero
        d = [abs(t[c] - v) for c in finite]
        best = [c for c, dd in zip(finite, d) if dd == min(d)]
        return max(best, key=lambda c: t[c])

    assert [half_away(float(v)) for v in x] != list(ref_codes)
    assert list(fp8.e4m3_encode(x)) == list(ref_codes)


# ------------------------------------------------------------------ mutants of the per-token projections

def _project_variant(kind):
    """ref.project_tiny with one plausible slip planted in its output."""
    def project(h, w, n_h, d_h, d_r, base=10000.0):
        c, k_r, q_c, q_r = ref.project_tiny(h, w, n_h, d_h, d_r, base)
        L = h.shape[0]
        pos = np.arange(L)
        raw_k = h @ np.asarray(w["kr"]).T
        raw_q = (h @ np.asarray(w["qr"]).T).reshape(L, n_h, d_r)
        if kind == "k_rope_at_0":
            k_r = raw_k
        elif kind == "q_rope_at_0":
            q_r = raw_q
        elif kind == "q_rope_at_t_minus_1":
            q_r = ref.rope(raw_q, (pos - 1)[:, None], base)
        elif kind == "k_rope_at_j_plus_1":
            k_r = ref.rope(raw_k, pos + 1, base)
        elif kind == "c_of_next_token":
            c = np.roll(c, -1, axis=0)
        elif kind == "w_dkv_transposed":
            c = h @ np.asarray(w["dkv"])
        elif kind == "k_rope_from_first_query_head":
            k_r = ref.rope(raw_q[:, 0, :], pos, base)
        return c, k_r, q_c, q_r
    return project


PROJECTION_MUTANTS = ("k_rope_at_0", "q_rope_at_0", "q_rope_at_t_minus_1", "k_rope_at_j_plus_1",
                      "c_of_next_token", "w_dkv_transposed", "k_rope_from_first_query_head")


@pytest.mark.parametrize("kind", PROJECTION_MUTANTS)
def test_projection_mutant_is_caught(kind):
    from test_oracle_projections import TOL, projection_errors
    layer = workloads.tiny_layer(seed=1)
    err = projection_errors(_project_variant(kind), layer, positions=[0, 1, 64, 127])
    assert any(v > TOL for v in err.values()), f"projection mutant {kind} passed: {err}"
    good = projection_errors(ref.project_tiny, layer, positions=[0, 1, 64, 127])
    assert all(v <= TOL for v in good.values()), good
