"""Float64 reference for weight-absorbed MLA decode.

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by the
cpu_baseline leg of bench.py, never by the GPU library.  It shares no code with it.

Sources (web pages on Multi-head Latent Attention):
  [DC] "MLA deep compression" (operatorworld.com, ai-mla-deep-compression):
       section "Low-rank projection: cache the latent, not K/V" (the latent equation
       c_t = W^DKV h_t and the per-head up-projection equation), section
       "Absorption: an equivalent rewrite at inference" (score-side equation with
       W^QK_i, output-side equation defining u_i), section "Decoupled RoPE".
  [AA] "Attention-head anatomy: one cache, four wirings" (romaanj.github.io):
       section 3 (every wiring keeps the same scores, softmax and output projection),
       section 5 (W^UK folds into the query path, W^UV into W^O; the two dot products
       of the content and RoPE parts are added).
  [GQ] "GQLA: Group-Query Latent Attention" abstract (chatpaper.ai): decode with
       s_q = 1 and s_q = 2 query tokens per step.

Readings where the pages are silent or garbled (numbered as in the design notes):
  R1  the key up-projection that [DC] prints as W^{KR}_i is W^UK_i ([AA] section 5).
  R2  softmax scale 1/sqrt(d_h + d_r), applied to the sum of both dot products.
  R4  RoPE: interleaved pairs (x[2m], x[2m+1]) rotated by pos * base**(-2m/d_r).
  R5  k^R is cached after rotation.
  R6  a new token attends to itself: its row is appended before attention.
  R7  with s_q new tokens, query q of sequence b sits at index L_b - s_q + q and sees
      tokens 0 .. L_b - s_q + q.
  R8  the step's output is o_i = W^UV_i u_i, laid out [B, s_q, n_h, d_v].
  R14 log-sum-exp values are natural logarithms.
  R18 a cached row is [c^KV (d_c values) | k^R (d_r values)].

Pins (each function is checked by something other than itself, see tests/):
  rope               hand-computed rotations; relative-position invariance; norm.
  project_tiny       scalar-loop recomputation of c = W^DKV h, q^C = W^Q h, both rotations
                     (complex exponentials at the token's own position) and every score
                     term q^R_{t,i} . k^R_j from the unrotated projections
                     (tests/test_oracle_projections.py; planted mutants caught).
  cache_rows,
  query_rows,
  output_projection,
  fold_output_weights
                     scalar loops with complex-exponential rotations at arbitrary
                     positions; equality with project_tiny / absorb_query on the tiny
                     layer; the explicit products W^QK_i = (W^UK_i)^T W^Q_i and
                     W^O_i W^UV_i against the factored forms; the folded output path
                     against plain multi-head attention followed by W^O
                     (tests/test_oracle_adjacent.py; planted mutants caught).
  gqla_expand,
  gqla_decode        the GQLA abstract's claim that both paths are algebraically
                     equivalent: equal to the absorbed form with per-head weights
                     repeated over each group (1e-12); pure-Python brute force of the
                     non-absorbed form with those weights; n_g = n_h reduces to the
                     non-absorbed form (tests/test_oracle_gqla.py; mutants caught).
  mla_nonabsorbed    absorbed == non-absorbed identity; pure-Python brute force.
  mla_absorbed       torch SDPA in float64; brute force; closed forms.
  split_partial,
  combine            any partition == unsplit; brute force; closed forms.
  split_table        brute-force enumeration of 64-token units (integers, exact).
  gather_rows,
  paged_append       brute-force per-token copies; fp8 path via oracle.fp8 pins.
"""
import math

import numpy as np

from . import fp8 as _fp8

SPLIT_UNIT = 64  # tokens per scheduling unit of the split rule (library contract)


# ----------------------------------------------------------------------------
# Projections of one layer ([DC] low-rank projection, decoupled RoPE)
# ----------------------------------------------------------------------------

def rope(x, pos, base=10000.0):
    """Rotate x[..., d] by its position(s).

    [DC] "Decoupled RoPE": position enters only through a rotation R_t of the small
    position parts of key and query; the pages fix neither the pairing nor the
    frequencies (reading R4): pair (x[2m], x[2m+1]) turns by angle pos * theta_m,
    theta_m = base ** (-2m / d).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("RoPE needs an even dimension")
    theta = base ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    cos, sin = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, cos.shape[:-1] + (d,)))
    out[..., 0::2] = xe * cos - xo * sin
    out[..., 1::2] = xe * sin + xo * cos
    return out


def project_tiny(h, w, n_h, d_h, d_r, base=10000.0):
    """Per-token projections from hidden states h [L, d].

    [DC] latent equation: c_t = W^DKV h_t (only c_t and a position part are cached).
    [DC] "Decoupled RoPE": k^R_t = RoPE_t(W^KR h_t), one per token, shared by all
    heads; q^R_{t,i} = RoPE_t(W^QR_i h_t) per head.
    [DC] absorption section: the content query is q_i = W^Q_i h_t (full rank).

    w: dict with 'dkv' [d_c, d], 'q' [n_h*d_h, d], 'kr' [d_r, d], 'qr' [n_h*d_r, d].
    Returns c [L, d_c], k_r [L, d_r] (each rotated at its own position, R5),
    q_c [L, n_h, d_h] and q_r [L, n_h, d_r] (rotated at position t).
    """
    h = np.asarray(h, dtype=np.float64)
    L = h.shape[0]
    pos = np.arange(L)
    c = h @ np.asarray(w["dkv"], np.float64).T
    k_r = rope(h @ np.asarray(w["kr"], np.float64).T, pos, base)
    q_c = (h @ np.asarray(w["q"], np.float64).T).reshape(L, n_h, d_h)
    q_r_raw = (h @ np.asarray(w["qr"], np.float64).T).reshape(L, n_h, d_r)
    q_r = rope(q_r_raw, pos[:, None], base)
    return c, k_r, q_c, q_r


def absorb_query(q_c, w_uk):
    """Absorbed content query q~_i = (W^UK_i)^T q^C_i, shape [n_h, d_c].

    [DC] score-side equation: s_i = (W^Q_i h)^T (W^UK_i c) = ((W^UK_i)^T W^Q_i h)^T c,
    so the product W^QK_i = (W^UK_i)^T W^Q_i meets the latent directly (R1).
    w_uk: [n_h, d_h, d_c].
    """
    q_c = np.asarray(q_c, np.float64)
    w_uk = np.asarray(w_uk, np.float64)
    return np.stack([w_uk[i].T @ q_c[i] for i in range(q_c.shape[0])])


def cache_rows(h, w_dkv, w_kr, positions, base=10000.0):
    """The cache row of new tokens with hidden states h [..., d] at absolute positions [...].

    [DC] latent equation: c_t = W^DKV h_t.  [DC] "Decoupled RoPE": k^R_t = RoPE(W^KR h_t),
    rotated at the token's own position (reading R5: cached after rotation).
    w_dkv [d_c, d], w_kr [d_r, d].  Returns (c [..., d_c], k_r [..., d_r]) in float64.
    """
    h = np.asarray(h, np.float64)
    c = h @ np.asarray(w_dkv, np.float64).T
    k_r = rope(h @ np.asarray(w_kr, np.float64).T, positions, base)
    return c, k_r


def query_rows(h, w_q, w_uk, w_qr, positions, base=10000.0):
    """Absorbed and RoPE queries of new tokens with hidden states h [..., d].

    [DC] score-side equation: head i's absorbed query is W^QK_i h_t with
    W^QK_i = (W^UK_i)^T W^Q_i (reading R1: the key up-projection is W^UK_i); by
    associativity it is formed here as (W^UK_i)^T (W^Q_i h_t).  [DC] "Decoupled RoPE":
    q^R_i = RoPE(W^QR_i h_t) at the token's position.
    w_q [n_h*d_h, d] (rows of head i at i*d_h), w_uk [n_h, d_h, d_c], w_qr [n_h*d_r, d].
    Returns q_nope [..., n_h, d_c] and q_pe [..., n_h, d_r].
    """
    h = np.asarray(h, np.float64)
    w_uk = np.asarray(w_uk, np.float64)
    n_h, d_h, _ = w_uk.shape
    lead = h.shape[:-1]
    q_c = (h @ np.asarray(w_q, np.float64).T).reshape(lead + (n_h, d_h))
    q_nope = np.einsum("...ik,ikc->...ic", q_c, w_uk)
    w_qr = np.asarray(w_qr, np.float64)
    d_r = w_qr.shape[0] // n_h
    raw = (h @ w_qr.T).reshape(lead + (n_h, d_r))
    q_pe = rope(raw, np.asarray(positions, np.float64)[..., None], base)
    return q_nope, q_pe


def output_projection(o, w_o):
    """y = sum_i W^O_i o_i: the heads' outputs through the output projection.

    [AA] section 5 (the per-head outputs W^UV_i u_i feed W^O; W^UV can be folded into it).
    o [..., n_h, d_v]; w_o [d, n_h*d_v] whose column block i (columns i*d_v ..) is W^O_i.
    Returns y [..., d].
    """
    o = np.asarray(o, np.float64)
    lead = o.shape[:-2]
    return o.reshape(lead + (-1,)) @ np.asarray(w_o, np.float64).T


def fold_output_weights(w_o, w_uv):
    """W^OV with column block i = W^O_i W^UV_i, shape [d, n_h*d_c]: the output-side fold
    ([AA] section 5: W^UV folds into W^O offline), so that y = sum_i W^OV_i u_i."""
    w_o = np.asarray(w_o, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    n_h, d_v, _ = w_uv.shape
    return np.concatenate([w_o[:, i * d_v:(i + 1) * d_v] @ w_uv[i] for i in range(n_h)], axis=1)


def gqla_expand(c, w_uk_g, w_uv_g):
    """GQLA's per-group expanded cache.

    [GQ] abstract: the same weights expose an MQA-absorb path identical to MLA's and a GQA
    path with a per-group expanded cache.  Reading: heads are split into n_g equal groups
    and the heads of group g share the up-projections W^UK_g, W^UV_g; the expanded cache of
    token j holds k_{j,g} = W^UK_g c_j and v_{j,g} = W^UV_g c_j for every group (the
    position key k^R_j stays shared).  c [L, d_c]; w_uk_g [n_g, d_h, d_c];
    w_uv_g [n_g, d_v, d_c].  Returns k [L, n_g, d_h], v [L, n_g, d_v].
    """
    c = np.asarray(c, np.float64)
    k = np.einsum("gkc,jc->jgk", np.asarray(w_uk_g, np.float64), c)
    v = np.einsum("gvc,jc->jgv", np.asarray(w_uv_g, np.float64), c)
    return k, v


def gqla_decode(q_c, q_r, k_exp, v_exp, k_r, scale, n_vis):
    """GQA decode of one query position over the per-group expanded cache.

    Head i belongs to group g = i // (n_h / n_g); its key for token j is [k_{j,g} ; k^R_j]
    and its value v_{j,g}; s_ij = scale (q^C_i . k_{j,g} + q^R_i . k^R_j) and
    o_i = sum_j softmax_j(s_i)_j v_{j,g} ([AA] section 3: plain attention per head).
    q_c [n_h, d_h], q_r [n_h, d_r], k_exp [L, n_g, d_h], v_exp [L, n_g, d_v], k_r [L, d_r].
    Returns o [n_h, d_v] and lse [n_h].
    """
    q_c = np.asarray(q_c, np.float64)
    q_r = np.asarray(q_r, np.float64)
    k_exp = np.asarray(k_exp, np.float64)[:n_vis]
    v_exp = np.asarray(v_exp, np.float64)[:n_vis]
    k_r = np.asarray(k_r, np.float64)[:n_vis]
    n_h = q_c.shape[0]
    n_g = k_exp.shape[1]
    per = n_h // n_g
    o = np.zeros((n_h, v_exp.shape[2]))
    lse = np.full(n_h, -np.inf)
    if n_vis == 0:
        return o, lse
    for i in range(n_h):
        g = i // per
        s = scale * (k_exp[:, g, :] @ q_c[i] + k_r @ q_r[i])
        m = s.max()
        e = np.exp(s - m)
        o[i] = (e / e.sum()) @ v_exp[:, g, :]
        lse[i] = m + math.log(e.sum())
    return o, lse


# ----------------------------------------------------------------------------
# The two forms of one decode step
# ----------------------------------------------------------------------------

def mla_nonabsorbed(c, k_r, q_c, q_r, w_uk, w_uv, scale, n_vis):
    """Plain multi-head attention with explicit per-head keys and values.

    [DC] per-head up-projection equation: k_{j,i} = W^UK_i c_j (R1), v_{j,i} = W^UV_i c_j.
    [DC] "Decoupled RoPE": head i's key is [W^UK_i c_j ; k^R_j] and its query is
    [q^C_i ; q^R_i].  [AA] section 3: scores, softmax and weighted sum of values are
    those of standard attention.  Scale per reading R2.

    c [L, d_c], k_r [L, d_r], q_c [n_h, d_h], q_r [n_h, d_r], w_uk [n_h, d_h, d_c],
    w_uv [n_h, d_v, d_c]; only tokens 0 .. n_vis-1 are visible.
    Returns o [n_h, d_v] and lse [n_h] (natural log of the softmax denominator).
    """
    c = np.asarray(c, np.float64)[:n_vis]
    k_r = np.asarray(k_r, np.float64)[:n_vis]
    w_uk = np.asarray(w_uk, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    n_h, d_v = w_uv.shape[0], w_uv.shape[1]
    o = np.zeros((n_h, d_v))
    lse = np.full(n_h, -np.inf)
    if n_vis == 0:
        return o, lse
    for i in range(n_h):
        keys = np.concatenate([c @ w_uk[i].T, k_r], axis=1)      # [n, d_h + d_r]
        values = c @ w_uv[i].T                                    # [n, d_v]
        query = np.concatenate([np.asarray(q_c[i], np.float64), np.asarray(q_r[i], np.float64)])
        s = scale * (keys @ query)
        m = s.max()
        e = np.exp(s - m)
        den = e.sum()
        o[i] = (e / den) @ values
        lse[i] = m + math.log(den)
    return o, lse


def mla_absorbed(q_nope, q_pe, c, k_pe, w_uv, scale, n_vis):
    """Absorbed decode of one query position for all heads.

    [DC] score-side equation: each head's absorbed query q~_i (here q_nope[i]) is
    dotted with the shared latent c_j; [DC] "Decoupled RoPE" / [AA] section 5: the
    RoPE part q^R_i . k^R_j is added to it.  s_ij = scale (q~_i . c_j + q^R_i . k^R_j).
    a_i = softmax over visible j.  [DC] output-side equation: u_i = sum_j a_ij c_j,
    o_i = W^UV_i u_i.

    q_nope [n_h, d_c], q_pe [n_h, d_r], c [L, d_c], k_pe [L, d_r], w_uv [n_h, d_v, d_c].
    Returns (o [n_h, d_v], lse [n_h], u [n_h, d_c]).  No visible token: o = 0,
    u = 0, lse = -inf.
    """
    q_nope = np.asarray(q_nope, np.float64)
    q_pe = np.asarray(q_pe, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    n_h, d_c = q_nope.shape
    if n_vis == 0:
        return np.zeros((n_h, w_uv.shape[1])), np.full(n_h, -np.inf), np.zeros((n_h, d_c))
    c = np.asarray(c, np.float64)[:n_vis]
    k_pe = np.asarray(k_pe, np.float64)[:n_vis]
    s = scale * (q_nope @ c.T + q_pe @ k_pe.T)             # [n_h, n]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(axis=1, keepdims=True)
    u = (e / den) @ c                                        # [n_h, d_c]
    o = np.einsum("ivc,ic->iv", w_uv, u)
    lse = m[:, 0] + np.log(den[:, 0])
    return o, lse, u


def visible_len(seq_len, s_q, q):
    """Tokens visible to query position q (reading R7, R6): L - s_q + q + 1, floored at 0."""
    return max(0, int(seq_len) - int(s_q) + int(q) + 1)


def decode(q_nope, q_pe, rows_of, seq_lens, w_uv, scale, batches=None):
    """Absorbed decode for a batch.

    q_nope [B, s_q, n_h, d_c], q_pe [B, s_q, n_h, d_r]; rows_of(b) -> (c [L_b, d_c],
    k_pe [L_b, d_r]) in logical token order.  Returns o [B, s_q, n_h, d_v] and
    lse [B, s_q, n_h] for the sequences in `batches` (default all; others stay 0).
    """
    B, s_q, n_h, _ = q_nope.shape
    d_v = np.asarray(w_uv).shape[1]
    o = np.zeros((B, s_q, n_h, d_v))
    lse = np.full((B, s_q, n_h), -np.inf)
    for b in (range(B) if batches is None else batches):
        c, k = rows_of(b)
        for q in range(s_q):
            n = visible_len(seq_lens[b], s_q, q)
            o[b, q], lse[b, q], _ = mla_absorbed(q_nope[b, q], q_pe[b, q], c, k, w_uv, scale, n)
    return o, lse


# ----------------------------------------------------------------------------
# Cache gather and append (row layout R18; paging)
# ----------------------------------------------------------------------------

def slot_of(block_table, page_size, b, pos):
    """Pool slot of token `pos` of sequence b: page block_table[b][pos // P], offset pos % P."""
    return int(block_table[b][pos // page_size]) * page_size + pos % page_size


def gather_rows(pool_c, pool_k, block_table, page_size, b, seq_len, pool_scale=None):
    """Logical rows 0..seq_len-1 of sequence b from a paged pool, as float64.

    pool_c [slots, d_c], pool_k [slots, d_r] hold numbers (float arrays) or, with
    pool_scale given, OCP E4M3 codes (uint8) that are decoded and multiplied by the
    per-slot scale (exact in float64).
    """
    slots = np.array([slot_of(block_table, page_size, b, j) for j in range(seq_len)], dtype=np.int64)
    if pool_scale is None:
        return np.asarray(pool_c[slots], np.float64), np.asarray(pool_k[slots], np.float64)
    table = _fp8.e4m3_decode_table()
    sc = np.asarray(pool_scale, np.float64)[slots][:, None]
    return table[pool_c[slots]] * sc, table[pool_k[slots]] * sc


def paged_append(pool_c, pool_k, pool_scale, c_new, k_new, positions, block_table, page_size):
    """Write new rows [c | k^R] into the paged pool, in place.

    Without pool_scale the rows are copied bit for bit (callers pass bit patterns,
    e.g. uint16 for bf16).  With pool_scale (float32 array) the 576-value row is
    quantized per token by oracle.fp8.quantize_row and its scale stored per slot.
    positions [B, s_new] are absolute token indices.
    """
    B, s_new = positions.shape
    d_c = c_new.shape[-1]
    for b in range(B):
        for j in range(s_new):
            slot = slot_of(block_table, page_size, b, int(positions[b, j]))
            if pool_scale is None:
                pool_c[slot] = c_new[b, j]
                pool_k[slot] = k_new[b, j]
            else:
                row = np.concatenate([np.asarray(c_new[b, j], np.float32), np.asarray(k_new[b, j], np.float32)])
                codes, sc = _fp8.quantize_row(row)
                pool_c[slot] = codes[:d_c]
                pool_k[slot] = codes[d_c:]
                pool_scale[slot] = sc


# ----------------------------------------------------------------------------
# Split-KV partials and the log-sum-exp combine
# ----------------------------------------------------------------------------

def split_partial(q_nope, q_pe, c, k_pe, scale, t0, t1):
    """Softmax restricted to tokens [t0, t1) of one query position, all heads.

    Same scores as mla_absorbed.  lse_s = ln sum_{j in [t0,t1)} exp(s_j) and
    u_s = sum_j exp(s_j - lse_s) c_j.  An empty range gives lse_s = -inf, u_s = 0.
    Returns (u_s [n_h, d_c], lse_s [n_h]).
    """
    q_nope = np.asarray(q_nope, np.float64)
    n_h, d_c = q_nope.shape
    if t1 <= t0:
        return np.zeros((n_h, d_c)), np.full(n_h, -np.inf)
    cc = np.asarray(c, np.float64)[t0:t1]
    kk = np.asarray(k_pe, np.float64)[t0:t1]
    s = scale * (q_nope @ cc.T + np.asarray(q_pe, np.float64) @ kk.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(axis=1, keepdims=True)
    return (e / den) @ cc, m[:, 0] + np.log(den[:, 0])


def combine(u_parts, lse_parts):
    """Merge partials of disjoint token sets: softmax over a union of disjoint sets.

    lse = ln sum_s exp(lse_s) (shifted by the largest finite lse_s);
    u = sum_s exp(lse_s - lse) u_s.  Parts with lse_s = -inf carry no weight; if all
    are -inf the result is u = 0, lse = -inf.
    u_parts [S, n_h, d_c], lse_parts [S, n_h] -> (u [n_h, d_c], lse [n_h]).
    """
    u_parts = np.asarray(u_parts, np.float64)
    lse_parts = np.asarray(lse_parts, np.float64)
    S, n_h, d_c = u_parts.shape
    u = np.zeros((n_h, d_c))
    lse = np.full(n_h, -np.inf)
    for i in range(n_h):
        finite = np.isfinite(lse_parts[:, i])
        if not finite.any():
            continue
        m = lse_parts[finite, i].max()
        w = np.exp(lse_parts[finite, i] - m)
        tot = w.sum()
        lse[i] = m + math.log(tot)
        u[i] = (w / tot) @ u_parts[finite, i]
    return u, lse


def up_project(u, w_uv):
    """o_i = W^UV_i u_i ([DC] output-side equation). u [..., n_h, d_c] -> [..., n_h, d_v]."""
    return np.einsum("ivc,...ic->...iv", np.asarray(w_uv, np.float64), np.asarray(u, np.float64))


def split_table(seq_lens, num_splits, unit=SPLIT_UNIT):
    """The library's balanced partition of a batch into partial-attention pieces.

    Sequence b is cut into n_b = ceil(L_b / unit) units; the units of all sequences,
    in batch order, form one list of U = sum n_b units that is cut into num_splits
    equal shares of ceil(U / num_splits) units.  Share w meets sequence b in at most
    one piece; that piece is stored in slot w + b.  Returns
      table  int64 [B, 2]: (first slot, number of pieces) per sequence, (0, 0) if
             L_b = 0;
      pieces list of (b, w, slot, t0, t1): tokens [t0, t1) of sequence b.
    """
    seq_lens = [int(x) for x in seq_lens]
    B = len(seq_lens)
    n_units = [(L + unit - 1) // unit for L in seq_lens]
    total = sum(n_units)
    table = np.zeros((B, 2), dtype=np.int64)
    pieces = []
    if total == 0:
        return table, pieces
    share = (total + num_splits - 1) // num_splits
    start = 0
    for b in range(B):
        n = n_units[b]
        if n:
            w_first, w_last = start // share, (start + n - 1) // share
            table[b] = (w_first + b, w_last - w_first + 1)
            for w in range(w_first, w_last + 1):
                u0 = max(w * share, start) - start
                u1 = min((w + 1) * share, start + n) - start
                pieces.append((b, w, w + b, u0 * unit, min(u1 * unit, seq_lens[b])))
        start += n
    return table, pieces


def num_slots(batch, num_splits):
    """Capacity of the slot space used by split_table: slots are w + b < num_splits + batch."""
    return int(num_splits) + int(batch)
