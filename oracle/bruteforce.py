"""Pure-Python scalar forms of MLA decode for tiny inputs (no NumPy arithmetic).

TEST INFRASTRUCTURE ONLY (see the oracle package docstring).

These loops restate, one multiply-add at a time, the definitions that
oracle.mla_ref computes with NumPy: the absorbed score s_ij = scale (q~_i . c_j +
q^R_i . k^R_j), the softmax, the latent sum u_i and o_i = W^UV_i u_i ([DC] "MLA deep
compression", absorption section and "Decoupled RoPE"), the explicit per-head
keys/values of the non-absorbed form ([DC] low-rank projection section), and the
partition rule of oracle.mla_ref.split_table built unit by unit.
They are meant for n_h <= 2 and a handful of tokens.
"""
import math


def _dot(a, b):
    acc = 0.0
    for x, y in zip(a, b):
        acc += x * y
    return acc


def _matvec(mat, vec):
    return [_dot(row, vec) for row in mat]


def absorbed_decode(q_nope, q_pe, c, k_pe, w_uv, scale, n_vis):
    """Nested lists in, nested lists out: (o [n_h][d_v], lse [n_h], u [n_h][d_c])."""
    n_h = len(q_nope)
    d_c = len(q_nope[0])
    o, lse, u_all = [], [], []
    for i in range(n_h):
        if n_vis == 0:
            o.append([0.0] * len(w_uv[i]))
            lse.append(-math.inf)
            u_all.append([0.0] * d_c)
            continue
        s = [scale * (_dot(q_nope[i], c[j]) + _dot(q_pe[i], k_pe[j])) for j in range(n_vis)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        den = 0.0
        for x in e:
            den += x
        u = [0.0] * d_c
        for j in range(n_vis):
            a = e[j] / den
            for k in range(d_c):
                u[k] += a * c[j][k]
        o.append(_matvec(w_uv[i], u))
        lse.append(m + math.log(den))
        u_all.append(u)
    return o, lse, u_all


def nonabsorbed_decode(c, k_r, q_c, q_r, w_uk, w_uv, scale, n_vis):
    """Per-head keys [W^UK_i c_j ; k^R_j], values W^UV_i c_j, standard softmax attention."""
    n_h = len(q_c)
    o, lse = [], []
    for i in range(n_h):
        keys = [_matvec(w_uk[i], c[j]) + list(k_r[j]) for j in range(n_vis)]
        vals = [_matvec(w_uv[i], c[j]) for j in range(n_vis)]
        query = list(q_c[i]) + list(q_r[i])
        s = [scale * _dot(query, keys[j]) for j in range(n_vis)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        den = sum(e)
        out = [0.0] * len(w_uv[i])
        for j in range(n_vis):
            for k in range(len(out)):
                out[k] += e[j] / den * vals[j][k]
        o.append(out)
        lse.append(m + math.log(den))
    return o, lse


def split_table(seq_lens, num_splits, unit=64):
    """Build the partition by walking every unit of every sequence, in batch order.

    Unit g of the concatenated unit list belongs to share g // share_size; a piece is
    a maximal run of units with the same (sequence, share).  Returns (table, pieces)
    in the same format as oracle.mla_ref.split_table.
    """
    units = []  # (b, local unit index)
    for b, L in enumerate(seq_lens):
        n = -(-int(L) // unit)
        for k in range(n):
            units.append((b, k))
    B = len(seq_lens)
    table = [[0, 0] for _ in range(B)]
    pieces = []
    if not units:
        return table, pieces
    share = -(-len(units) // num_splits)
    runs = {}
    for g, (b, k) in enumerate(units):
        w = g // share
        key = (b, w)
        if key not in runs:
            runs[key] = [k, k]
        runs[key][1] = k
    for (b, w) in sorted(runs):
        k0, k1 = runs[(b, w)]
        pieces.append((b, w, w + b, k0 * unit, min((k1 + 1) * unit, int(seq_lens[b]))))
    for b in range(B):
        mine = [p for p in pieces if p[0] == b]
        if mine:
            table[b] = [min(p[2] for p in mine), len(mine)]
    return table, pieces
