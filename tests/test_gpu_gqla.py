"""GPU parity of GQLA's per-group path (GQLA abstract, chatpaper.ai: two algebraically
equivalent decoding paths over the same weights, MQA-absorb and GQA with a per-group expanded
cache), through the C ABI:

- mla_gqla_expand_cache against the oracle's expanded cache (every value within one bf16 step);
- mla_gqla_decode (s_q = 1 and 2, causal within the pair) against the oracle's GQA decode;
- the same weights through the absorbed path (mla_decode_fwd with q~_i = (W^UK_g)^T q^C_i and
  W^UV_i = W^UV_g) against the same oracle: the two GPU paths agree within the tolerance.
"""
import math

import numpy as np
import pytest
import torch

from mla_latent_kv_03_amd import workloads
from oracle import mla_ref as ref

from gpu_helpers import BF16_TOL, DeviceCase, assert_close, record, to_np

pytestmark = pytest.mark.gpu


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("lens,s_q,n_h,n_g,d_c,d_h,d_r,d_v", [
    ([700, 65, 3000, 2], 2, 128, 8, 512, 128, 64, 128),      # a GQLA layer of the V3 shape, MTP pair
    ([700, 65, 3000, 2], 1, 128, 8, 512, 128, 64, 128),
    ([1, 33, 96, 257, 0], 2, 8, 2, 64, 16, 16, 32),
    ([300, 31], 1, 16, 4, 64, 32, 32, 64),
])
def test_gqla_paths_agree_with_oracle(lens, s_q, n_h, n_g, d_c, d_h, d_r, d_v):
    print(f"[case] gqla lens={lens} s_q={s_q} n_h={n_h} n_g={n_g}", flush=True)
    from mla_latent_kv_03_amd import binding
    seed = 1700 + sum(lens) + s_q + n_h
    x = workloads.make_decode(lens, s_q=s_q, n_h=n_h, d_c=d_c, d_r=d_r, d_v=d_v, page_size=64, seed=seed,
                              softmax_scale=1.0 / math.sqrt(d_h + d_r))
    rng = np.random.default_rng(seed + 1)
    w_uk = _bf16(rng.standard_normal((n_g, d_h, d_c)) / math.sqrt(d_c))
    w_uv = _bf16(rng.standard_normal((n_g, d_v, d_c)) / math.sqrt(d_c))
    q_c = _bf16(rng.standard_normal((len(lens), s_q, n_h, d_h)))
    case = DeviceCase(x)
    # GQA path on the GPU
    k_exp, v_exp = binding.mla_gqla_expand_cache(case.params, w_uk.cuda(), w_uv.cuda(), case.c_kv)
    out_g, lse_g = binding.mla_gqla_decode(case.params, q_c.cuda(), case.q_pe, k_exp, v_exp, case.k_pe,
                                           case.block_table, case.seq_lens)
    torch.cuda.synchronize()
    # oracle: expanded cache and GQA decode in float64 from the same (bf16-valued) inputs
    wuk, wuv, qc, qp = w_uk.double().numpy(), w_uv.double().numpy(), q_c.double().numpy(), x.q_pe.double().numpy()
    B = len(lens)
    o_ref = np.zeros((B, s_q, n_h, d_v))
    lse_ref = np.full((B, s_q, n_h), -np.inf)
    k_err = 0.0
    k_exp_h, v_exp_h = k_exp.double().cpu().numpy(), v_exp.double().cpu().numpy()
    for b in range(B):
        c, kr = case.rows_of(b)
        k, v = ref.gqla_expand(c, wuk, wuv)
        slots = case.slots_of(b)
        if len(slots):
            for got, want in ((k_exp_h[slots], k), (v_exp_h[slots], v)):
                # one bf16 step of the exact value; values that cancel to below 1e-3 (the entries
                # are O(1)) get the step at 1e-3, which covers the float32 accumulation error
                ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(want), 1e-3))) - 7)
                k_err = max(k_err, float(np.max(np.abs(got - want) / ulp)))
        for q in range(s_q):
            n_vis = ref.visible_len(lens[b], s_q, q)
            o_ref[b, q], lse_ref[b, q] = ref.gqla_decode(qc[b, q], qp[b, q], k, v, kr, x.softmax_scale, n_vis)
    assert k_err <= 1.0, f"expanded cache value more than one bf16 step from exact ({k_err:.3f})"
    rel, mab = assert_close(to_np(out_g), o_ref, BF16_TOL, "gqa path")
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(to_np(lse_g)))
    lse_err = float(np.max(np.abs(to_np(lse_g)[fin] - lse_ref[fin])))
    assert lse_err <= 5e-3
    record(f"gqla GQA path lens={lens} s_q={s_q} n_h={n_h} n_g={n_g} (expanded cache within {k_err:.3f} bf16 steps)",
           rel, mab, lse_err, n=o_ref.size)
    if d_c != 512 or d_r != 64 or d_v != 128:
        return                      # the bf16 absorbed decode serves the V3 latent widths only
    # absorbed path with the same weights: q~_i = (W^UK_g)^T q^C_i, W^UV_i = W^UV_g
    per = n_h // n_g
    q_abs = np.stack([np.stack([ref.absorb_query(qc[b, q], np.repeat(wuk, per, axis=0)) for q in range(s_q)])
                      for b in range(B)])
    case.q_nope = _bf16(q_abs).cuda()
    case.w_uv = torch.repeat_interleave(w_uv, per, dim=0).contiguous().cuda()
    out_a, lse_a, _ = case.run()
    rel_a, mab_a = assert_close(to_np(out_a), o_ref, BF16_TOL, "absorbed path, GQLA weights")
    record(f"gqla absorbed path lens={lens} s_q={s_q} n_h={n_h} n_g={n_g}", rel_a, mab_a, n=o_ref.size)
    assert np.array_equal(np.isfinite(to_np(lse_a)), fin)
