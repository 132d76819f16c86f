"""GPU parity: the HIP decode path against the float64 oracle.

Small cases run every output; the five workloads run at full size in the launch
configuration the benchmark times (num_splits = auto) and compare every sequence.
Tolerances: bf16/fp8 rel-L2 <= 5e-3 and max-abs <= 2e-2; fp32 both <= 1e-5.
"""
import numpy as np
import pytest
import torch

from mla_latent_kv_03_amd import workloads
from oracle import mla_ref as ref

from gpu_helpers import BF16_TOL, F32_TOL, DeviceCase, assert_close, compare_sampled, record, to_np

pytestmark = pytest.mark.gpu


def _print_case(name, **kw):
    print(f"[case] {name} {kw}", flush=True)


# ---------------------------------------------------------------- workload 1: tiny fp32 layer

def tiny_inputs(seed=1):
    layer = workloads.tiny_layer(seed=seed)
    c, k_r, q_c, q_r = ref.project_tiny(layer["h"], layer, layer["n_h"], layer["d_h"], layer["d_r"])
    t = layer["L"] - 1
    q_abs = ref.absorb_query(q_c[t], layer["uk"])
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    x = workloads.DecodeInputs(q_nope=f(q_abs)[None, None], q_pe=f(q_r[t])[None, None],
                               pool=f(np.concatenate([c, k_r], axis=1)), block_table=torch.zeros(1, 1, dtype=torch.int32),
                               seq_lens=torch.tensor([layer["L"]], dtype=torch.int32), w_uv=f(layer["uv"]),
                               page_size=128, softmax_scale=layer["scale"], kv_dtype="f32", name="tiny_fp32")
    o_non, lse_non = ref.mla_nonabsorbed(c, k_r, q_c[t], q_r[t], layer["uk"], layer["uv"], layer["scale"], t + 1)
    return x, o_non, lse_non


@pytest.mark.parametrize("num_splits", [0, 1, 2, 3, 7])
def test_tiny_fp32_layer(num_splits):
    _print_case("tiny_fp32", num_splits=num_splits)
    x, o_non, lse_non = tiny_inputs()
    case = DeviceCase(x, num_splits=num_splits)
    out, lse, _ = case.run()
    o_ref, lse_ref = case.oracle([0])
    assert_close(to_np(out)[0, 0], o_ref[0, 0], F32_TOL, "absorbed oracle")
    rel, mab = assert_close(to_np(out)[0, 0], o_non, F32_TOL, "non-absorbed form")
    lse_err = float(np.max(np.abs(to_np(lse)[0, 0] - lse_non)))
    assert lse_err <= 1e-5
    record(f"tiny_fp32 (vs the non-absorbed form) G={num_splits}", rel, mab, lse_err, n=int(o_non.size))


@pytest.mark.parametrize("lens,s_q,n_h,num_splits", [([1, 63, 64, 65, 300], 1, 8, 4), ([130, 2, 1], 2, 4, 3),
                                                     ([0, 129], 1, 16, 2)])
def test_fp32_generic_shapes(lens, s_q, n_h, num_splits):
    _print_case("fp32_generic", lens=lens, s_q=s_q, n_h=n_h)
    x = workloads.make_decode(lens, s_q=s_q, n_h=n_h, d_c=48, d_r=8, d_v=24, page_size=64, q_dtype="f32",
                              kv_dtype="f32", seed=17)
    case = DeviceCase(x, num_splits=num_splits)
    out, lse, _ = case.run()
    o_ref, lse_ref = case.oracle(range(len(lens)))
    assert_close(to_np(out), o_ref, F32_TOL, "fp32 generic")
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(to_np(lse)))
    assert np.max(np.abs(to_np(lse)[fin] - lse_ref[fin])) <= 1e-5


# ---------------------------------------------------------------- small bf16 / fp8 cases (every output)

SMALL = [
    # lens, s_q, n_h, page_size, paged, num_splits
    ([1000, 77, 2049], 1, 128, 64, True, 0),
    ([1000, 77, 2049], 1, 128, 64, True, 1),
    ([1000, 77, 2049], 1, 128, 64, True, 5),
    ([4097, 33], 1, 128, 128, True, 16),
    ([700, 129], 2, 128, 64, True, 0),
    ([700, 129, 3], 2, 64, 64, True, 6),
    ([520, 64], 1, 16, 64, False, 3),
    ([1, 2, 63, 64, 65], 1, 128, 64, True, 0),
]


@pytest.mark.parametrize("lens,s_q,n_h,page,paged,G", SMALL)
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_small_every_output(lens, s_q, n_h, page, paged, G, kv):
    _print_case("small", lens=lens, s_q=s_q, n_h=n_h, page=page, paged=paged, G=G, kv=kv)
    x = workloads.make_decode(lens, s_q=s_q, n_h=n_h, page_size=page, paged=paged, kv_dtype=kv, seed=sum(lens) + s_q)
    case = DeviceCase(x, num_splits=G)
    out, lse, _ = case.run()
    compare_sampled(case, out, lse, list(range(len(lens))), BF16_TOL, lse_tol=5e-3,
                    what=f"small {kv} lens={lens} s_q={s_q} n_h={n_h} G={G}")


# ---------------------------------------------------------------- the four V3 workloads at full size

@pytest.fixture(scope="module")
def v3_decode_case():
    return DeviceCase(workloads.v3_decode())


def test_v3_decode_b64_l4096(v3_decode_case):
    _print_case("v3_decode_b64_l4096")
    out, lse, _ = v3_decode_case.run()
    compare_sampled(v3_decode_case, out, lse, range(64), BF16_TOL, lse_tol=5e-3, what="v3_decode_b64_l4096")


def test_v3_paged_b128():
    _print_case("v3_paged_b128")
    case = DeviceCase(workloads.v3_paged())
    out, lse, _ = case.run()
    compare_sampled(case, out, lse, range(case.x.batch), BF16_TOL, lse_tol=5e-3, what="v3_paged_b128")


def test_v3_mtp_b32_l32768():
    _print_case("v3_mtp_b32_l32768")
    case = DeviceCase(workloads.v3_mtp())
    out, lse, _ = case.run()
    compare_sampled(case, out, lse, range(32), BF16_TOL, lse_tol=5e-3, what="v3_mtp_b32_l32768")


def test_v3_long_fp8_b4_l131072():
    _print_case("v3_long_fp8_b4_l131072")
    case = DeviceCase(workloads.v3_long_fp8())
    assert case.binding.mla_decode_num_splits(case.params) == 256 or torch.cuda.get_device_properties(0).multi_processor_count != 256
    out, lse, _ = case.run()
    compare_sampled(case, out, lse, range(4), BF16_TOL, lse_tol=5e-3, what="v3_long_fp8_b4_l131072")


# ---------------------------------------------------------------- scores far above the first tile's

@pytest.mark.parametrize("G", [0, 3])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_late_dominant_token(G, kv):
    """A token deep in the sequence whose scores exceed everything before it by far
    more than 2^64 (its latent is a large multiple of the heads' mean query direction):
    softmax is dominated by it, and the kernels must still match the float64 oracle.
    With an E4M3 cache the token's row is quantized with its own scale (30 / 448)."""
    _print_case("late_dominant_token", G=G, kv=kv)
    import torch
    x = workloads.make_decode([2049, 700], n_h=128, page_size=64, kv_dtype=kv, seed=77)
    qdir = torch.sign(x.q_nope[0, 0].float().mean(dim=0))          # [d_c]
    for b, t in ((0, 1500), (1, 650)):
        slot = int(x.block_table[b, t // x.page_size]) * x.page_size + t % x.page_size
        x.pool[slot, :x.d_c] = (30.0 * qdir).to(x.pool.dtype)
    case = DeviceCase(x, num_splits=G)
    out, lse, _ = case.run()
    # The outputs here reach |o| ~ 100 (u is dominated by a latent of magnitude 30), and the
    # bf16 output alone rounds by up to |o| 2^-9: the absolute bound scales with the output
    # (a few bf16 steps of the largest value); the relative bound is the usual one.
    o_ref, _ = case.oracle([0, 1])
    tol = dict(rel_l2=BF16_TOL["rel_l2"], max_abs=max(BF16_TOL["max_abs"], 2.0 ** -7 * float(np.abs(o_ref).max())))
    compare_sampled(case, out, lse, [0, 1], tol, lse_tol=5e-3, what="late dominant token")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_late_dominant_token_long_piece(kv):
    """One piece of 94 pages (a single split): the page-id window slides forward during
    the first pass, the dominant token at position 5500 forces a second pass, and that
    pass must start again from the piece's first pages."""
    _print_case("late_dominant_token_long_piece", G=1, kv=kv)
    import torch
    x = workloads.make_decode([6000], n_h=128, page_size=64, kv_dtype=kv, seed=78)
    qdir = torch.sign(x.q_nope[0, 0].float().mean(dim=0))
    t = 5500
    slot = int(x.block_table[0, t // x.page_size]) * x.page_size + t % x.page_size
    x.pool[slot, :x.d_c] = (30.0 * qdir).to(x.pool.dtype)
    case = DeviceCase(x, num_splits=1)
    out, lse, _ = case.run()
    o_ref, _ = case.oracle([0])
    tol = dict(rel_l2=BF16_TOL["rel_l2"], max_abs=max(BF16_TOL["max_abs"], 2.0 ** -7 * float(np.abs(o_ref).max())))
    compare_sampled(case, out, lse, [0], tol, lse_tol=5e-3, what="late dominant token, long piece")
