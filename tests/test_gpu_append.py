"""GPU tests of mla_paged_cache_append: bit-exact copies and E4M3 quantization."""
import numpy as np
import pytest
import torch

from oracle import fp8 as ofp8
from oracle import mla_ref as ref

pytestmark = pytest.mark.gpu


def _params(binding, B, P, pages, max_pages, kv, d_c=512, d_r=64):
    return binding.make_params(batch=B, s_q=1, n_h=16, d_c=d_c, d_r=d_r, d_v=128, page_size=P, num_pages=pages,
                               max_pages_per_seq=max_pages, c_kv_stride=d_c + d_r, k_pe_stride=d_c + d_r,
                               softmax_scale=0.1, q_dtype=binding.BF16, kv_dtype=kv)


def _case(seed, B=3, s_new=5, P=64, pages=9, max_pages=3):
    rng = np.random.default_rng(seed)
    perm = rng.permutation(pages)[: B * max_pages].reshape(B, max_pages).astype(np.int32)
    pos = np.stack([rng.choice(P * max_pages, size=s_new, replace=False) for _ in range(B)]).astype(np.int32)
    rows = rng.standard_normal((B, s_new, 576)).astype(np.float32) * rng.choice([1e-3, 1.0, 300.0], size=(B, s_new, 1))
    rows[0, 1] = 0.0                       # amax = 0 row
    rows[1, 2, 7] = 1e4                    # one large value, the rest underflow toward subnormals
    return perm, pos, rows


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_append_copy_is_bit_exact(dtype):
    print(f"[case] append copy {dtype}", flush=True)
    from mla_latent_kv_03_amd import binding
    perm, pos, rows = _case(1)
    B, s_new, _ = rows.shape
    P, pages = 64, 9
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kv = binding.BF16 if dtype == "bf16" else binding.F32
    src = torch.from_numpy(rows).to(tdt)
    pool = torch.zeros(pages * P, 576, dtype=tdt, device="cuda")
    binding.mla_paged_cache_append(_params(binding, B, P, pages, 3, kv), src[..., :512].cuda().contiguous(),
                                   src[..., 512:].cuda().contiguous(), torch.from_numpy(pos).cuda(),
                                   torch.from_numpy(perm).cuda(), pool[:, :512], pool[:, 512:])
    torch.cuda.synchronize()
    ibits = torch.int16 if dtype == "bf16" else torch.int32
    want = torch.zeros(pages * P, 576, dtype=tdt)
    bits = src.view(ibits).numpy()
    wc = want.view(ibits).numpy()
    ref.paged_append(wc[:, :512], wc[:, 512:], None, bits[..., :512], bits[..., 512:], pos, perm, P)
    assert torch.equal(pool.cpu().view(ibits), want.view(ibits))


@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
def test_append_fp8_is_bit_exact(in_dtype):
    print(f"[case] append fp8 from {in_dtype}", flush=True)
    from mla_latent_kv_03_amd import binding
    perm, pos, rows = _case(2)
    B, s_new, _ = rows.shape
    P, pages = 64, 9
    tdt = torch.bfloat16 if in_dtype == "bf16" else torch.float32
    src = torch.from_numpy(rows).to(tdt)
    pool = torch.zeros(pages * P, 576, dtype=torch.uint8, device="cuda")
    scale = torch.full((pages * P,), -1.0, dtype=torch.float32, device="cuda")
    binding.mla_paged_cache_append(_params(binding, B, P, pages, 3, binding.FP8), src[..., :512].cuda().contiguous(),
                                   src[..., 512:].cuda().contiguous(), torch.from_numpy(pos).cuda(),
                                   torch.from_numpy(perm).cuda(), pool[:, :512], pool[:, 512:], scale)
    torch.cuda.synchronize()
    want = np.zeros((pages * P, 576), np.uint8)
    want_s = np.full(pages * P, -1.0, np.float32)
    vals = src.float().numpy()
    ref.paged_append(want[:, :512], want[:, 512:], want_s, vals[..., :512], vals[..., 512:], pos, perm, P)
    got, got_s = pool.cpu().numpy(), scale.cpu().numpy()
    bad = np.nonzero((got != want).any(axis=1))[0]
    assert bad.size == 0, f"rows differ at slots {bad[:5]}"
    assert np.array_equal(got_s.view(np.int32), want_s.view(np.int32))


def test_append_fp8_dense_value_sweep():
    """Every float32 magnitude class through the device quantizer (rows scaled so inv = 1)."""
    print("[case] append fp8 sweep", flush=True)
    from mla_latent_kv_03_amd import binding
    t = ofp8.e4m3_decode_table()
    finite = np.sort(np.unique(np.abs(t[np.isfinite(t)])))
    mids = (finite[1:] + finite[:-1]) / 2
    vals = np.concatenate([finite, mids, np.linspace(0, 448, 4000), np.linspace(0, 0.03, 2000)])
    n_rows = -(-len(vals) // 575)
    rows = np.zeros((n_rows * 575,), np.float32)
    rows[: len(vals)] = vals
    rows = rows.reshape(n_rows, 575)
    rows[::2] *= -1
    rows = np.concatenate([rows, np.full((n_rows, 1), 448.0, np.float32)], axis=1)   # amax = 448 -> inv = 1
    P = 64
    pages = -(-n_rows // P)
    pos = np.arange(n_rows, dtype=np.int32)[None]
    table = np.arange(pages, dtype=np.int32)[None]
    pool = torch.zeros(pages * P, 576, dtype=torch.uint8, device="cuda")
    scale = torch.zeros(pages * P, dtype=torch.float32, device="cuda")
    src = torch.from_numpy(rows)[None]
    binding.mla_paged_cache_append(_params(binding, 1, P, pages, pages, binding.FP8), src[..., :512].cuda().contiguous(),
                                   src[..., 512:].cuda().contiguous(), torch.from_numpy(pos).cuda(),
                                   torch.from_numpy(table).cuda(), pool[:, :512], pool[:, 512:], scale)
    torch.cuda.synchronize()
    codes, sc = ofp8.quantize_rows(rows)
    assert np.all(sc == 1.0)
    assert np.array_equal(pool.cpu().numpy()[:n_rows], codes)


def test_append_skips_out_of_range_positions():
    print("[case] append skips", flush=True)
    from mla_latent_kv_03_amd import binding
    P, pages = 64, 4
    table = torch.tensor([[0, 1], [2, 99]], dtype=torch.int32, device="cuda")      # page 99 does not exist
    pos = torch.tensor([[5, 200], [70, -1]], dtype=torch.int32, device="cuda")      # 200 >= 2 pages * 64
    src = torch.ones(2, 2, 576, dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros(pages * P, 576, dtype=torch.bfloat16, device="cuda")
    binding.mla_paged_cache_append(_params(binding, 2, P, pages, 2, binding.BF16), src[..., :512].contiguous(),
                                   src[..., 512:].contiguous(), pos, table, pool[:, :512], pool[:, 512:])
    torch.cuda.synchronize()
    written = (pool.float().abs().sum(1) > 0).nonzero().flatten().tolist()
    assert written == [5]
