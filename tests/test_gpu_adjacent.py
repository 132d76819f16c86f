"""GPU parity of the projections adjacent to the decode step, through the C ABI:

- mla_cache_write: [c | k^R] = [W^DKV h ; RoPE(W^KR h)] written into the paged pool (bf16 rows,
  float32 rows, E4M3 codes + scale), then the decode over a pool whose new rows came from it;
- mla_query_prologue: q~_i = (W^UK_i)^T W^Q_i h and q^R_i = RoPE(W^QR_i h), then the decode;
- mla_output_projection / mla_fold_output_weights / the merged-latent combine: y = sum_i W^O_i W^UV_i u_i
  unfolded (W^O applied to o) and folded (W^OV applied to u).

On the tiny float32 layer (the five-page oracle's non-absorbed form is the reference) and on
V3-shaped slices (d_model 7168, d_c 512, d_r 64, d_h = d_v = 128; 16 or 32 heads, one or eight
GPUs' share of 128).  Expected values come from oracle/ only.
"""
import math

import numpy as np
import pytest
import torch

from mla_latent_kv_03_amd import workloads
from oracle import fp8 as ofp8
from oracle import mla_ref as ref

from gpu_helpers import BF16_TOL, F32_TOL, DeviceCase, assert_close, compare_sampled, record, to_np

pytestmark = pytest.mark.gpu
V3_D = 7168


def _case(name, **kw):
    print(f"[case] {name} {kw}", flush=True)


def _bf16_ulp(x):
    """One bf16 step of x; values below 1e-3 (the rows are O(1)) get the step at 1e-3, which
    covers the float32 accumulation error of a value that cancels to near zero."""
    a = np.maximum(np.abs(np.asarray(x, np.float64)), 1e-3)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def _pool_params(binding, *, batch, s_q=1, n_h, d_c, d_r, d_v, page_size, num_pages, max_pages, stride, q, kv,
                 num_splits=0):
    return binding.make_params(batch=batch, s_q=s_q, n_h=n_h, d_c=d_c, d_r=d_r, d_v=d_v, page_size=page_size,
                               num_pages=num_pages, max_pages_per_seq=max_pages, c_kv_stride=stride, k_pe_stride=stride,
                               softmax_scale=1.0 / math.sqrt(d_v + d_r), q_dtype=q, kv_dtype=kv,
                               num_splits=num_splits)


# ------------------------------------------------------------------ cache write

def test_cache_write_tiny_layer_f32_and_decode():
    """The tiny layer (d 64, d_c 64, d_r 16, positions 0..127): all 128 rows written by
    mla_cache_write from the hidden states, compared with the oracle's cache rows; the decode
    over that pool then matches the non-absorbed form."""
    _case("cache_write tiny f32")
    from mla_latent_kv_03_amd import binding
    layer = workloads.tiny_layer(seed=1)
    L, d = layer["L"], layer["d"]
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    pool = torch.full((128, 80), float("nan"), dtype=torch.float32, device="cuda")
    table = torch.zeros(1, 1, dtype=torch.int32, device="cuda")
    pos = torch.arange(L, dtype=torch.int32, device="cuda")[None]
    p = _pool_params(binding, batch=1, n_h=8, d_c=64, d_r=16, d_v=16, page_size=128, num_pages=1, max_pages=1,
                     stride=80, q=binding.F32, kv=binding.F32)
    binding.mla_cache_write(p, f(layer["h"])[None], f(layer["dkv"]), f(layer["kr"]), pos, table, pool[:, :64],
                            pool[:, 64:])
    torch.cuda.synchronize()
    c, k_r = ref.cache_rows(layer["h"], layer["dkv"], layer["kr"], np.arange(L))
    got = pool.cpu().numpy()
    rel, mab = assert_close(got, np.concatenate([c, k_r], 1), F32_TOL, "tiny cache rows")
    record("cache_write tiny f32 rows", rel, mab, n=got.size)
    # downstream: the absorbed decode of the last token over this pool vs the non-absorbed oracle
    _, _, q_c, q_r = ref.project_tiny(layer["h"], layer, 8, 16, 16)
    q_abs = ref.absorb_query(q_c[L - 1], layer["uk"])
    out, lse, _ = binding.mla_decode_fwd(f(q_abs)[None, None], f(q_r[L - 1])[None, None], pool[:, :64], pool[:, 64:],
                                         table, torch.tensor([L], dtype=torch.int32, device="cuda"), f(layer["uv"]),
                                         softmax_scale=layer["scale"], page_size=128)
    torch.cuda.synchronize()
    o_n, lse_n = ref.mla_nonabsorbed(c, k_r, q_c[L - 1], q_r[L - 1], layer["uk"], layer["uv"], layer["scale"], L)
    rel, mab = assert_close(to_np(out)[0, 0], o_n, F32_TOL, "decode over written pool")
    assert np.max(np.abs(to_np(lse)[0, 0] - lse_n)) <= 1e-5
    record("cache_write tiny f32 -> decode", rel, mab, n=o_n.size)


def test_cache_write_tiny_layer_e4m3_bits():
    """E4M3 rows from float32 inputs: the codes and scales must be exactly the oracle's
    quantizer applied to the float32 rows the same call writes in float32 mode."""
    _case("cache_write tiny e4m3")
    from mla_latent_kv_03_amd import binding
    layer = workloads.tiny_layer(seed=1)
    L = layer["L"]
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    table = torch.tensor([[1, 0]], dtype=torch.int32, device="cuda")          # two 64-token pages, swapped
    pos = torch.arange(L, dtype=torch.int32, device="cuda")[None]
    pf = torch.zeros(128, 80, dtype=torch.float32, device="cuda")
    p32 = _pool_params(binding, batch=1, n_h=8, d_c=64, d_r=16, d_v=16, page_size=64, num_pages=2, max_pages=2,
                       stride=80, q=binding.F32, kv=binding.F32)
    binding.mla_cache_write(p32, f(layer["h"])[None], f(layer["dkv"]), f(layer["kr"]), pos, table, pf[:, :64], pf[:, 64:])
    p8 = _pool_params(binding, batch=1, n_h=8, d_c=64, d_r=16, d_v=16, page_size=64, num_pages=2, max_pages=2,
                      stride=80, q=binding.F32, kv=binding.FP8)
    codes = torch.zeros(128, 80, dtype=torch.uint8, device="cuda")
    scales = torch.zeros(128, dtype=torch.float32, device="cuda")
    binding.mla_cache_write(p8, f(layer["h"])[None], f(layer["dkv"]), f(layer["kr"]), pos, table, codes[:, :64],
                            codes[:, 64:], scales)
    torch.cuda.synchronize()
    want_codes, want_scales = ofp8.quantize_rows(pf.cpu().numpy())
    assert np.array_equal(codes.cpu().numpy(), want_codes)
    assert np.array_equal(scales.cpu().numpy().view(np.int32), want_scales.view(np.int32))
    # and the float32 rows are the oracle's (page-swapped slots)
    c, k_r = ref.cache_rows(layer["h"], layer["dkv"], layer["kr"], np.arange(L))
    rows = np.concatenate([c, k_r], 1)
    got = pf.cpu().numpy()
    slots = np.array([[64, 0][t // 64] + t % 64 for t in range(L)])
    assert_close(got[slots], rows, F32_TOL, "tiny rows, paged")


def _v3_cache_case(seed, kv, n_seq=8, s_new=2):
    """Sequences with random lengths (one near 131072 for the RoPE angle), a permuted 64-token page
    pool filled with N(0,1) rows, and the last s_new positions of each sequence as new tokens."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(70, 3000, size=n_seq)
    lens[-1] = 131071
    x = workloads.make_decode(lens.tolist(), page_size=64, kv_dtype=kv, seed=seed, **workloads.V3)
    w = workloads.layer_weights(seed + 1, d_model=V3_D, n_h=128, d_c=512, d_h=128, d_r=64, d_v=128,
                                n_tokens=n_seq * s_new, with_o=False)
    positions = np.stack([np.arange(L - s_new, L) for L in lens]).astype(np.int32)
    return x, w, positions


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_cache_write_v3_slice(kv):
    """d_model 7168: 16 new rows (two per sequence, one sequence at position ~131070) written into a
    permuted pool, every value checked against the oracle's cache rows, then the decode over the
    pool (other rows from the generator) against the oracle whose new rows are the exact ones."""
    _case("cache_write v3", kv=kv)
    from mla_latent_kv_03_amd import binding
    x, w, positions = _v3_cache_case(1201, kv)
    B, s_new = positions.shape
    case = DeviceCase(x)                                     # pool filled (bf16, or quantized by the append)
    h_bf = torch.from_numpy(w["h"]).to(torch.bfloat16)
    h = h_bf.reshape(B, s_new, V3_D).cuda()
    wd, wk = (torch.from_numpy(w[k]).to(torch.bfloat16).cuda() for k in ("dkv", "kr"))
    pos = torch.from_numpy(positions).cuda()
    params = case.params
    binding.mla_cache_write(params, h, wd, wk, pos, case.block_table, case.c_kv, case.k_pe, case.kv_scale)
    torch.cuda.synchronize()
    # oracle rows from the bf16-rounded inputs, in float64
    c, k_r = ref.cache_rows(h_bf.double().numpy(), torch.from_numpy(w["dkv"]).to(torch.bfloat16).double().numpy(),
                            torch.from_numpy(w["kr"]).to(torch.bfloat16).double().numpy(), positions.reshape(-1))
    exact = np.concatenate([c, k_r], 1)
    tab = x.block_table.numpy()
    slots = np.array([int(tab[b, p // 64]) * 64 + p % 64 for b in range(B) for p in positions[b]])
    if kv == "bf16":
        got = case.pool[torch.from_numpy(slots).cuda()].double().cpu().numpy()
        err = np.abs(got - exact) / _bf16_ulp(exact)
        assert err.max() <= 1.0, f"a stored value is more than one bf16 step from the exact row ({err.max():.3f})"
        record(f"cache_write v3 bf16 rows (max error in bf16 steps {err.max():.3f})",
               *assert_close(got, exact, BF16_TOL, "rows"), n=got.size)
    else:
        codes = case.pool[torch.from_numpy(slots).cuda()].cpu().numpy()
        sc = case.kv_scale[torch.from_numpy(slots).cuda()].cpu().numpy().astype(np.float64)
        amax = np.abs(exact).max(1)
        assert np.max(np.abs(sc - amax / 448) / (amax / 448)) <= 1e-5, "scale differs from amax / 448"
        deq = ofp8.e4m3_decode_table()[codes] * sc[:, None]
        # one E4M3 step of the value's binade (3 mantissa bits; subnormal step 2^-9), times the scale
        v = np.abs(exact) / sc[:, None]
        step = np.where(v < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(v, 2.0 ** -6))) - 3)) * sc[:, None]
        assert np.all(np.abs(deq - exact) <= step * 0.5 + 1e-6 * np.abs(exact) + 1e-12), "a code is off by a step"
        # E4M3 keeps 3 mantissa bits: the half-step bound above is the format's own error bound
        # (about 3.6% RMS relative), so the rows are not held to the bf16 tolerance.
        from gpu_helpers import errors
        record("cache_write v3 e4m3 rows (dequantized, within half an E4M3 step)", *errors(deq, exact), n=deq.size)
    # downstream decode over the written pool; the oracle's rows of the new tokens are its own
    # (exact rows, quantized by the oracle's E4M3 quantizer for an E4M3 pool)
    out, lse, _ = case.run()
    rows_of_orig = case.rows_of
    if kv == "fp8":
        q_codes, q_sc = ofp8.quantize_rows(exact.astype(np.float32))
        oracle_rows = ofp8.e4m3_decode_table()[q_codes] * q_sc.astype(np.float64)[:, None]
    else:
        oracle_rows = exact
    new = {(b, int(p)): oracle_rows[b * s_new + j] for b in range(B) for j, p in enumerate(positions[b])}

    def rows_of(b):
        cc, kk = rows_of_orig(b)
        cc, kk = cc.copy(), kk.copy()
        for (bb, p), row in new.items():
            if bb == b:
                cc[p], kk[p] = row[:512], row[512:]
        return cc, kk

    case.rows_of = rows_of
    compare_sampled(case, out, lse, range(B), BF16_TOL, lse_tol=5e-3, what=f"cache_write v3 {kv} -> decode")


@pytest.mark.parametrize("n_seq", [4, 20])
def test_cache_write_ragged_k(n_seq):
    """d_model 7200 (a multiple of 32, not of 64): the product's K chunks end inside a block of four
    k-steps, so the kernel that skips the steps past a chunk runs; 8 and 40 new rows (one and
    two 32-row tiles of A).  Every stored bf16 value against the oracle's cache rows."""
    _case("cache_write ragged K", n_seq=n_seq)
    from mla_latent_kv_03_amd import binding
    d_model, s_new = 7200, 2
    rng = np.random.default_rng(1250 + n_seq)
    lens = rng.integers(70, 3000, size=n_seq)
    x = workloads.make_decode(lens.tolist(), page_size=64, seed=1251 + n_seq, **workloads.V3)
    w = workloads.layer_weights(1252 + n_seq, d_model=d_model, n_h=128, d_c=512, d_h=128, d_r=64, d_v=128,
                                n_tokens=n_seq * s_new, with_o=False)
    positions = np.stack([np.arange(L - s_new, L) for L in lens]).astype(np.int32)
    case = DeviceCase(x)
    h_bf = torch.from_numpy(w["h"]).to(torch.bfloat16)
    wd, wk = (torch.from_numpy(w[k]).to(torch.bfloat16) for k in ("dkv", "kr"))
    binding.mla_cache_write(case.params, h_bf.reshape(n_seq, s_new, d_model).cuda(), wd.cuda(), wk.cuda(),
                            torch.from_numpy(positions).cuda(), case.block_table, case.c_kv, case.k_pe, case.kv_scale)
    torch.cuda.synchronize()
    c, k_r = ref.cache_rows(h_bf.double().numpy(), wd.double().numpy(), wk.double().numpy(), positions.reshape(-1))
    exact = np.concatenate([c, k_r], 1)
    tab = x.block_table.numpy()
    slots = np.array([int(tab[b, p // 64]) * 64 + p % 64 for b in range(n_seq) for p in positions[b]])
    got = case.pool[torch.from_numpy(slots).cuda()].double().cpu().numpy()
    err = np.abs(got - exact) / _bf16_ulp(exact)
    assert err.max() <= 1.0, f"a stored value is more than one bf16 step from the exact row ({err.max():.3f})"
    record(f"cache_write ragged K, {n_seq * s_new} rows (max error in bf16 steps {err.max():.3f})",
           *assert_close(got, exact, BF16_TOL, "rows"), n=got.size)


# ------------------------------------------------------------------ query prologue

def test_query_prologue_tiny_layer_f32():
    """The tiny layer's query (token 127): q~ and q^R from the hidden state, then the decode over
    the tiny cache against the non-absorbed form."""
    _case("query_prologue tiny f32")
    from mla_latent_kv_03_amd import binding
    layer = workloads.tiny_layer(seed=1)
    L = layer["L"]
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    p = _pool_params(binding, batch=1, n_h=8, d_c=64, d_r=16, d_v=16, page_size=128, num_pages=1, max_pages=1,
                     stride=80, q=binding.F32, kv=binding.F32)
    w_uk_t = np.ascontiguousarray(np.transpose(layer["uk"], (0, 2, 1)))
    pos = torch.tensor([[L - 1]], dtype=torch.int32, device="cuda")
    qn, qp = binding.mla_query_prologue(p, f(layer["h"][L - 1])[None, None], f(layer["q"]), f(w_uk_t), f(layer["qr"]),
                                        pos, d_h=16)
    torch.cuda.synchronize()
    want_n, want_p = ref.query_rows(layer["h"][L - 1], layer["q"], layer["uk"], layer["qr"], L - 1)
    rel, mab = assert_close(to_np(qn)[0, 0], want_n, F32_TOL, "q_nope")
    assert_close(to_np(qp)[0, 0], want_p, F32_TOL, "q_pe")
    record("query_prologue tiny f32 q_nope", rel, mab, n=want_n.size)
    c, k_r, q_c, q_r = ref.project_tiny(layer["h"], layer, 8, 16, 16)
    pool = f(np.concatenate([c, k_r], 1))
    out, lse, _ = binding.mla_decode_fwd(qn, qp, pool[:, :64], pool[:, 64:], torch.zeros(1, 1, dtype=torch.int32).cuda(),
                                         torch.tensor([L], dtype=torch.int32).cuda(), f(layer["uv"]),
                                         softmax_scale=layer["scale"], page_size=128)
    torch.cuda.synchronize()
    o_n, _ = ref.mla_nonabsorbed(c, k_r, q_c[L - 1], q_r[L - 1], layer["uk"], layer["uv"], layer["scale"], L)
    record("query_prologue tiny f32 -> decode", *assert_close(to_np(out)[0, 0], o_n, F32_TOL, "decode"), n=o_n.size)


def test_query_prologue_v3_slice():
    """d_model 7168, 32 heads (a four-GPU share), 4 sequences x 2 query tokens at positions up to
    ~131070: q_nope and q_pe against the oracle, then the decode of those queries over a paged
    bf16 cache against the oracle decode with the oracle's queries."""
    _case("query_prologue v3 slice")
    from mla_latent_kv_03_amd import binding
    n_h, B, s_q = 32, 4, 2
    w = workloads.layer_weights(1301, d_model=V3_D, n_h=n_h, d_c=512, d_h=128, d_r=64, d_v=128, n_tokens=B * s_q,
                                with_o=False)
    lens = [300, 1000, 77, 131071]
    positions = np.array([[L - 2, L - 1] for L in lens], np.int32)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16)
    h = bf(w["h"]).reshape(B, s_q, V3_D)
    wq, wqr = bf(w["q"]), bf(w["qr"])
    uk_t = bf(np.transpose(w["uk"], (0, 2, 1)))
    x = workloads.make_decode(lens, s_q=s_q, n_h=n_h, page_size=64, seed=1302, d_c=512, d_r=64, d_v=128)
    case = DeviceCase(x)
    qn, qp = binding.mla_query_prologue(case.params, h.cuda(), wq.cuda(), uk_t.cuda(), wqr.cuda(),
                                        torch.from_numpy(positions).cuda(), d_h=128)
    torch.cuda.synchronize()
    want_n, want_p = ref.query_rows(h.double().numpy(), wq.double().numpy(), bf(w["uk"]).double().numpy(),
                                    wqr.double().numpy(), positions)
    record("query_prologue v3 q_nope", *assert_close(to_np(qn), want_n, BF16_TOL, "q_nope"), n=want_n.size)
    record("query_prologue v3 q_pe", *assert_close(to_np(qp), want_p, BF16_TOL, "q_pe"), n=want_p.size)
    case.q_nope, case.q_pe = qn, qp
    out, lse, _ = case.run()
    # oracle: the decode with the exact (float64) queries
    x.q_nope, x.q_pe = torch.from_numpy(want_n), torch.from_numpy(want_p)
    compare_sampled(case, out, lse, range(B), BF16_TOL, lse_tol=5e-3, what="query_prologue v3 -> decode")


def test_query_prologue_ragged_k():
    """d_model 7200 and d_h 96 (multiples of 32, not of 64): the W^Q / W^QR products (bf16 rows of
    h) and the (W^UK_i)^T product (float32 q^C_i, K = d_h) both end their K chunks inside a block
    of four k-steps.  16 heads, 20 sequences x 2 query tokens (two 32-row tiles of A)."""
    _case("query_prologue ragged K")
    from mla_latent_kv_03_amd import binding
    n_h, B, s_q, d_model, d_h = 16, 20, 2, 7200, 96
    w = workloads.layer_weights(1351, d_model=d_model, n_h=n_h, d_c=512, d_h=d_h, d_r=64, d_v=128,
                                n_tokens=B * s_q, with_o=False)
    lens = np.random.default_rng(1352).integers(10, 5000, size=B)
    positions = np.array([[L - 2, L - 1] for L in lens], np.int32)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16)
    h = bf(w["h"]).reshape(B, s_q, d_model)
    wq, wqr = bf(w["q"]), bf(w["qr"])
    uk_t = bf(np.transpose(w["uk"], (0, 2, 1)))
    x = workloads.make_decode(lens.tolist(), s_q=s_q, n_h=n_h, page_size=64, seed=1353, d_c=512, d_r=64, d_v=128)
    case = DeviceCase(x)
    qn, qp = binding.mla_query_prologue(case.params, h.cuda(), wq.cuda(), uk_t.cuda(), wqr.cuda(),
                                        torch.from_numpy(positions).cuda(), d_h=d_h)
    torch.cuda.synchronize()
    want_n, want_p = ref.query_rows(h.double().numpy(), wq.double().numpy(), bf(w["uk"]).double().numpy(),
                                    wqr.double().numpy(), positions)
    record("query_prologue ragged K q_nope", *assert_close(to_np(qn), want_n, BF16_TOL, "q_nope"), n=want_n.size)
    record("query_prologue ragged K q_pe", *assert_close(to_np(qp), want_p, BF16_TOL, "q_pe"), n=want_p.size)


@pytest.mark.parametrize("n_h,B,d_model,d_h,d_c,d_r", [(4, 37, 512, 64, 176, 16), (2, 65, 256, 256, 528, 32)])
def test_query_prologue_token_and_column_edges(n_h, B, d_model, d_h, d_c, d_r):
    """Absorption product at widths the V3 shape does not reach: 74 and 130 query rows (two and
    three blocks of 64 tokens, the last one partial), latent widths 176 and 528 (blocks of 256
    columns ending inside a wave's 64 columns and inside a 32-column block), and d_h 256 (two
    rounds of eight k-steps).  q_nope and q_pe against the oracle."""
    _case("query_prologue edges", n_h=n_h, B=B, d_h=d_h, d_c=d_c)
    from mla_latent_kv_03_amd import binding
    s_q = 2
    w = workloads.layer_weights(1361 + d_h, d_model=d_model, n_h=n_h, d_c=d_c, d_h=d_h, d_r=d_r, d_v=16,
                                n_tokens=B * s_q, with_o=False)
    positions = np.random.default_rng(1362).integers(0, 131072, size=(B, s_q)).astype(np.int32)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16)
    h = bf(w["h"]).reshape(B, s_q, d_model)
    wq, wqr = bf(w["q"]), bf(w["qr"])
    uk_t = bf(np.transpose(w["uk"], (0, 2, 1)))
    params = binding.make_params(batch=B, s_q=s_q, n_h=n_h, d_c=d_c, d_r=d_r, d_v=16, page_size=64, num_pages=1,
                                 max_pages_per_seq=1, c_kv_stride=d_c + d_r, k_pe_stride=d_c + d_r,
                                 softmax_scale=1.0, q_dtype=binding.BF16, kv_dtype=binding.BF16)
    qn, qp = binding.mla_query_prologue(params, h.cuda(), wq.cuda(), uk_t.cuda(), wqr.cuda(),
                                        torch.from_numpy(positions).cuda(), d_h=d_h)
    torch.cuda.synchronize()
    want_n, want_p = ref.query_rows(h.double().numpy(), wq.double().numpy(), bf(w["uk"]).double().numpy(),
                                    wqr.double().numpy(), positions)
    record(f"query_prologue edges d_h={d_h} d_c={d_c} q_nope", *assert_close(to_np(qn), want_n, BF16_TOL, "q_nope"),
           n=want_n.size)
    record(f"query_prologue edges d_h={d_h} d_c={d_c} q_pe", *assert_close(to_np(qp), want_p, BF16_TOL, "q_pe"),
           n=want_p.size)


# ------------------------------------------------------------------ output projection and fold

def test_output_projection_tiny_layer_f32_both_forms():
    """y = sum_i W^O_i W^UV_i u_i of the tiny layer's last token: unfolded (W^O on the decode
    output) and folded (W^OV from mla_fold_output_weights on the merged latents), against plain
    multi-head attention followed by W^O."""
    _case("output projection tiny f32")
    from mla_latent_kv_03_amd import binding
    layer = workloads.tiny_layer(seed=1)
    L = layer["L"]
    rng = np.random.default_rng(1401)
    w_o = rng.standard_normal((64, 8 * 16)) / math.sqrt(128)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    c, k_r, q_c, q_r = ref.project_tiny(layer["h"], layer, 8, 16, 16)
    q_abs = ref.absorb_query(q_c[L - 1], layer["uk"])
    o_n, _ = ref.mla_nonabsorbed(c, k_r, q_c[L - 1], q_r[L - 1], layer["uk"], layer["uv"], layer["scale"], L)
    y_ref = ref.output_projection(o_n, w_o)
    pool = f(np.concatenate([c, k_r], 1))
    args = (f(q_abs)[None, None], f(q_r[L - 1])[None, None], pool[:, :64], pool[:, 64:],
            torch.zeros(1, 1, dtype=torch.int32).cuda(), torch.tensor([L], dtype=torch.int32).cuda(), f(layer["uv"]))
    out, _, ws = binding.mla_decode_fwd(*args, softmax_scale=layer["scale"], page_size=128, num_splits=3)
    p = binding.params_for(args[0], args[1], args[2], args[3], args[4], args[6], softmax_scale=layer["scale"],
                           page_size=128, num_splits=3)
    y = binding.mla_output_projection(p, out, f(w_o))
    w_ov = binding.mla_fold_output_weights(p, f(w_o), f(layer["uv"]))
    u = torch.empty(1, 1, 8, 64, dtype=torch.float32, device="cuda")
    binding.mla_decode_splitkv_combine(p, ws, None, u)
    y2 = binding.mla_output_projection(p, u, w_ov)
    torch.cuda.synchronize()
    assert_close(w_ov.cpu().numpy(), ref.fold_output_weights(w_o, layer["uv"]), F32_TOL, "folded weights")
    record("output projection tiny unfolded", *assert_close(to_np(y)[0, 0], y_ref, F32_TOL, "unfolded"), n=y_ref.size)
    record("output projection tiny folded", *assert_close(to_np(y2)[0, 0], y_ref, F32_TOL, "folded"), n=y_ref.size)


def test_output_projection_v3_slice_both_forms():
    """16 heads (one GPU's share of 128), d_model 7168, 4 sequences x 2 query tokens: the
    unfolded and folded forms against the oracle's sum_i W^O_i W^UV_i u_i."""
    _case("output projection v3 slice")
    from mla_latent_kv_03_amd import binding
    n_h, B, s_q = 16, 4, 2
    x = workloads.make_decode([700, 65, 2, 3000], s_q=s_q, n_h=n_h, page_size=64, seed=1501, d_c=512, d_r=64, d_v=128)
    w = workloads.layer_weights(1502, d_model=V3_D, n_h=n_h, d_c=512, d_h=128, d_r=64, d_v=128, n_tokens=1)
    w_o = torch.from_numpy(w["o"]).to(torch.bfloat16)
    case = DeviceCase(x, num_splits=9)
    out, lse, ws = case.run()
    y = binding.mla_output_projection(case.params, out, w_o.cuda())
    w_ov = binding.mla_fold_output_weights(case.params, w_o.cuda(), case.w_uv)
    u = torch.empty(B, s_q, n_h, 512, dtype=torch.float32, device="cuda")
    binding.mla_decode_splitkv_combine(case.params, ws, None, u)
    y2 = binding.mla_output_projection(case.params, u, w_ov)
    torch.cuda.synchronize()
    # oracle: u per (b, q) from the absorbed decode, then sum_i W^O_i W^UV_i u_i
    qn, qp, wuv = x.q_nope.double().numpy(), x.q_pe.double().numpy(), x.w_uv.double().numpy()
    y_ref = np.zeros((B, s_q, V3_D))
    for b in range(B):
        c, kp = case.rows_of(b)
        for q in range(s_q):
            _, _, uu = ref.mla_absorbed(qn[b, q], qp[b, q], c, kp, wuv, x.softmax_scale,
                                        ref.visible_len(int(x.seq_lens[b]), s_q, q))
            y_ref[b, q] = ref.output_projection(ref.up_project(uu, wuv), w_o.double().numpy())
    wf = ref.fold_output_weights(w_o.double().numpy(), wuv)
    record("fold v3 W^OV", *assert_close(w_ov.float().cpu().numpy(), wf, BF16_TOL, "folded weights"), n=wf.size)
    record("output projection v3 unfolded", *assert_close(to_np(y), y_ref, BF16_TOL, "unfolded"), n=y_ref.size)
    record("output projection v3 folded", *assert_close(to_np(y2), y_ref, BF16_TOL, "folded"), n=y_ref.size)
