"""Shared plumbing of the GPU tests: put seeded inputs on the device, run the library
through its C ABI, and compute the oracle on the same inputs (or a sample of them).
Expected values come only from oracle/ on the generator's inputs."""
import math
import os

import numpy as np
import torch

from oracle import fp8 as ofp8
from oracle import mla_ref as ref

BF16_TOL = dict(rel_l2=5e-3, max_abs=2e-2)
F32_TOL = dict(rel_l2=1e-5, max_abs=1e-5)


def errors(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    diff = got - want
    rel = np.linalg.norm(diff) / max(np.linalg.norm(want), 1e-300)
    return rel, float(np.max(np.abs(diff))) if diff.size else 0.0


def assert_close(got, want, tol, what=""):
    rel, mab = errors(got, want)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert rel <= tol["rel_l2"] and mab <= tol["max_abs"], f"{what}: rel_l2={rel:.3e} max_abs={mab:.3e} tol={tol}"
    return rel, mab


class DeviceCase:
    """Inputs of one decode call resident on the GPU, plus what the oracle needs."""

    def __init__(self, x, num_splits=0, device="cuda"):
        from mla_latent_kv_03_amd import binding
        self.x = x
        self.binding = binding
        d_c = x.d_c
        self.q_nope = x.q_nope.to(device)
        self.q_pe = x.q_pe.to(device)
        self.block_table = x.block_table.to(device)
        self.seq_lens = x.seq_lens.to(device)
        self.w_uv = x.w_uv.to(device)
        self.kv_scale = None
        if x.kv_dtype == "fp8":
            slots = x.pool.shape[0]
            self.pool = torch.zeros(slots, x.pool.shape[1], dtype=torch.uint8, device=device)
            self.kv_scale = torch.zeros(slots, dtype=torch.float32, device=device)
            self._quantize_on_device(device)
        else:
            self.pool = x.pool.to(device)
        self.c_kv = self.pool[:, :d_c]
        self.k_pe = self.pool[:, d_c:]
        self.params = binding.params_for(self.q_nope, self.q_pe, self.c_kv, self.k_pe, self.block_table, self.w_uv,
                                         softmax_scale=x.softmax_scale, page_size=x.page_size,
                                         num_splits=num_splits)
        if x.kv_dtype == "fp8":
            self.params.kv_dtype = binding.FP8

    def _quantize_on_device(self, device):
        """Fill the E4M3 pool with the library's append, one call per sequence."""
        x, b_ = self.x, self.binding
        d_c = x.d_c
        c_view, k_view = self.pool[:, :d_c], self.pool[:, d_c:]
        for b in range(x.batch):
            L = int(x.seq_lens[b])
            if L == 0:
                continue
            slots = self.slots_of(b)
            src = x.pool[torch.from_numpy(slots)].to(device)                 # float32 rows in logical order
            params = b_.make_params(batch=1, s_q=1, n_h=x.n_h, d_c=d_c, d_r=x.d_r, d_v=x.d_v,
                                    page_size=x.page_size, num_pages=x.num_pages,
                                    max_pages_per_seq=x.block_table.shape[1], c_kv_stride=self.pool.stride(0),
                                    k_pe_stride=self.pool.stride(0), softmax_scale=x.softmax_scale,
                                    q_dtype=b_.BF16, kv_dtype=b_.FP8)
            pos = torch.arange(L, dtype=torch.int32, device=device)[None]
            table = self.block_table_dev(device)[b:b + 1]
            b_.mla_paged_cache_append(params, src[None, :, :d_c].contiguous(), src[None, :, d_c:].contiguous(), pos,
                                      table, c_view, k_view, self.kv_scale)

    def block_table_dev(self, device):
        return self.x.block_table.to(device)

    def slots_of(self, b):
        x = self.x
        L = int(x.seq_lens[b])
        j = np.arange(L)
        tab = x.block_table.numpy()
        return tab[b, j // x.page_size].astype(np.int64) * x.page_size + j % x.page_size

    def run(self, partials_only=False, workspace=None):
        out, lse, ws = self.binding.mla_decode_fwd(self.q_nope, self.q_pe, self.c_kv, self.k_pe, self.block_table,
                                                   self.seq_lens, self.w_uv, softmax_scale=self.x.softmax_scale,
                                                   page_size=self.x.page_size, kv_scale=self.kv_scale,
                                                   params=self.params, partials_only=partials_only,
                                                   workspace=workspace)
        torch.cuda.synchronize()
        return out, lse, ws

    # ------------------------------------------------------------------ oracle side
    def rows_of(self, b):
        """float64 rows of sequence b in logical order, as the oracle sees them."""
        x = self.x
        slots = self.slots_of(b)
        rows = x.pool[torch.from_numpy(slots)].double().numpy() if len(slots) else np.zeros((0, x.d_c + x.d_r))
        if x.kv_dtype == "fp8" and len(slots):
            codes, scale = quantize_rows_chunked(rows.astype(np.float32))
            rows = ofp8.e4m3_decode_table()[codes] * scale.astype(np.float64)[:, None]
        return rows[:, :x.d_c], rows[:, x.d_c:]

    def oracle(self, batches):
        x = self.x
        qn = x.q_nope.double().numpy()
        qp = x.q_pe.double().numpy()
        w = x.w_uv.double().numpy()
        return ref.decode(qn, qp, self.rows_of, x.seq_lens.numpy(), w, x.softmax_scale, batches=batches)


def quantize_rows_chunked(rows, chunk=16384):
    codes = np.empty(rows.shape, np.uint8)
    scales = np.empty(rows.shape[0], np.float32)
    for i in range(0, rows.shape[0], chunk):
        codes[i:i + chunk], scales[i:i + chunk] = ofp8.quantize_rows(rows[i:i + chunk])
    return codes, scales


def to_np(t):
    return t.float().cpu().numpy() if t is not None else None


def record(what, rel, mab, lse_err=None, n=None):
    """Print the achieved error of one comparison and, if MLA_PARITY_LOG names a file, append
    it there (one line per comparison), so that the margins to the tolerances are visible."""
    line = f"[parity] {what}: rel_l2={rel:.3e} max_abs={mab:.3e}"
    if lse_err is not None:
        line += f" lse_max_err={lse_err:.3e}"
    if n is not None:
        line += f" outputs={n}"
    print(line, flush=True)
    path = os.environ.get("MLA_PARITY_LOG")
    if path:
        with open(path, "a") as fh:
            fh.write(line + "\n")


def compare_sampled(case, out, lse, batches, tol, lse_tol=None, what=""):
    """Every output of the sequences in `batches` against the oracle: per sequence within `tol`,
    and the whole set's rel-L2 / max-abs / lse error recorded."""
    batches = list(batches)
    o_ref, lse_ref = case.oracle(batches)
    got = to_np(out)
    got_lse = to_np(lse)
    res = []
    lse_worst = 0.0
    for b in batches:
        r = assert_close(got[b], o_ref[b], tol, f"{what} b={b}")
        fin = np.isfinite(lse_ref[b])
        assert np.array_equal(fin, np.isfinite(got_lse[b])), f"{what} b={b}: lse finiteness differs"
        if fin.any():
            lt = lse_tol if lse_tol is not None else tol["max_abs"]
            err = np.max(np.abs(got_lse[b][fin] - lse_ref[b][fin]))
            assert err <= lt, f"{what} b={b}: lse max err {err:.3e}"
            lse_worst = max(lse_worst, float(err))
        res.append(r)
    rel, mab = errors(got[batches], o_ref[batches])
    record(what, rel, mab, lse_worst, n=int(got[batches].size))
    return res
