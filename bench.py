#!/usr/bin/env python3
"""Benchmark of absorbed-MLA decode on one MI355X.

One step = the whole hot path on one batch: append the new token's cache row
(mla_paged_cache_append), partial attention over the latent cache, log-sum-exp
combine and W^UV up-projection (mla_decode_fwd + mla_decode_splitkv_combine).
Default workload: DeepSeek-V3 decode shape, batch 64, one query token, 4096-token
contiguous bf16 latent caches (576 values per token), seeded synthetic inputs.

Prints one JSON line.  value = cached tokens processed per second (sum of the
sequence lengths per step / wall time per step).  The "roofline" object reports the
dominant kernel (partial attention): algorithmic HBM bytes per launch / its average
duration measured with HIP events on the launch stream.  Inputs stay resident in
HBM; steps rotate over several copies of them so that the 256 MB Infinity Cache
cannot serve a step from the previous one.
"""
import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode latent-KV tokens/s + achieved HBM GB/s & MFMA % of peak"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6       # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_partial_traffic.json")
MI355X_SIMDS = 1024             # 256 CUs x 4 SIMDs (8 XCDs)
MI355X_XCDS = 8
CSRC = os.path.join(ROOT, "mla_latent_kv_03_amd", "csrc")


def attn_kernel(x):
    """(kernel name, source files) of the partial-attention kernel the library runs for workload x."""
    fp8 = x.kv_dtype == "fp8"
    if x.n_h % 128 == 0:
        return ("attn_partial_h128<true>" if fp8 else "attn_partial_h128<false>",
                ("mla_attn_h128.hip", "mla_device.h", "mla_split.h"))
    if fp8:
        return "attn_partial_mfma<true>", ("mla_attn_fp8_v0.hip", "mla_device.h", "mla_split.h")
    return "attn_partial_split", ("mla_attn_mfma.hip", "mla_device.h", "mla_split.h")


COMBINE_SRC = ("mla_combine.hip", "mla_device.h", "mla_kernels.h")


def source_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]

WORKLOADS = ("v3_decode_b64_l4096", "v3_paged_b128", "v3_mtp_b32_l32768", "v3_long_fp8_b4_l131072")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--min-warmup-ms", type=float, default=250.0,
                    help="keep running untimed warmup steps (after the first W) until this much wall time has "
                         "passed: the GPU's clocks settle only under sustained load")
    ap.add_argument("--workload", default=WORKLOADS[0], choices=WORKLOADS)
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate-bytes", type=float, default=1.0e9,
                    help="total bytes of rotating input copies (cold Infinity Cache per step)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="before the timed steps, run a plain streaming kernel (elementwise negation: reads and "
                         "writes this many MiB) three times, so that a counter run (rocprofv3 --pmc FETCH_SIZE / "
                         "WRITE_SIZE) sees a kernel of known traffic")
    ap.add_argument("--pmc-summary", nargs="+", metavar="RESULTS_DB",
                    help="no GPU run: read rocprofv3 counter databases of a bench run made with "
                         "--copy-calibration-mb, print the attention kernel's HBM traffic per launch and record "
                         "it in profiles/attn_partial_traffic.json")
    ap.add_argument("--pmc-command", default="", help="command line recorded with --pmc-summary")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the attainable-peak probes (HBM streaming read, bf16 MFMA chains)")
    ap.add_argument("--adjacent", action="store_true",
                    help="instead of the decode step, time the adjacent rows at the V3 shape (cache write, query "
                         "prologue, output projection unfolded and folded, GQLA per-group decode) and print one "
                         "JSON line per row")
    return ap.parse_args()


def make_workload(name):
    from mla_latent_kv_03_amd import workloads
    return {"v3_decode_b64_l4096": workloads.v3_decode, "v3_paged_b128": workloads.v3_paged,
            "v3_mtp_b32_l32768": workloads.v3_mtp, "v3_long_fp8_b4_l131072": workloads.v3_long_fp8}[name]()


class Resident:
    """One copy of a decode call's inputs in HBM, plus the tensors one step writes."""

    def __init__(self, x, binding, num_splits, dev):
        import torch
        self.x = x
        self.q_nope, self.q_pe = x.q_nope.to(dev), x.q_pe.to(dev)
        self.block_table, self.seq_lens = x.block_table.to(dev), x.seq_lens.to(dev)
        self.w_uv = x.w_uv.to(dev)
        d_c = x.d_c
        lens = x.seq_lens.numpy()
        tab = x.block_table.numpy()
        # the new token of each sequence is its last cached row: position L_b - 1
        last = [int(L) - 1 for L in lens]
        self.positions = torch.tensor(last, dtype=torch.int32, device=dev)[:, None].contiguous()
        last_slots = [int(tab[b, p // x.page_size]) * x.page_size + p % x.page_size for b, p in enumerate(last)]
        new_rows = x.pool[torch.tensor(last_slots)]
        self.kv_scale = None
        if x.kv_dtype == "fp8":
            self.pool = torch.zeros(x.pool.shape, dtype=torch.uint8, device=dev)
            self.kv_scale = torch.zeros(x.pool.shape[0], dtype=torch.float32, device=dev)
            qp = binding.make_params(batch=1, s_q=1, n_h=x.n_h, d_c=d_c, d_r=x.d_r, d_v=x.d_v, page_size=x.page_size,
                                     num_pages=x.num_pages, max_pages_per_seq=tab.shape[1], c_kv_stride=x.pool.shape[1],
                                     k_pe_stride=x.pool.shape[1], softmax_scale=x.softmax_scale, q_dtype=binding.BF16,
                                     kv_dtype=binding.FP8)
            for b in range(x.batch):
                j = torch.arange(int(lens[b]))
                slots = torch.from_numpy(tab[b])[j // x.page_size].long() * x.page_size + j % x.page_size
                src = x.pool[slots].to(dev)[None]
                binding.mla_paged_cache_append(qp, src[..., :d_c].contiguous(), src[..., d_c:].contiguous(),
                                               torch.arange(int(lens[b]), dtype=torch.int32, device=dev)[None],
                                               self.block_table[b:b + 1], self.pool[:, :d_c], self.pool[:, d_c:],
                                               self.kv_scale)
            self.new_c = new_rows[:, None, :d_c].to(dev).contiguous()             # float32 source rows
            self.new_k = new_rows[:, None, d_c:].to(dev).contiguous()
        else:
            self.pool = x.pool.to(dev)
            self.new_c = new_rows[:, None, :d_c].to(dev).contiguous()
            self.new_k = new_rows[:, None, d_c:].to(dev).contiguous()
        self.c_kv, self.k_pe = self.pool[:, :d_c], self.pool[:, d_c:]
        self.params = binding.params_for(self.q_nope, self.q_pe, self.c_kv, self.k_pe, self.block_table, self.w_uv,
                                         softmax_scale=x.softmax_scale, page_size=x.page_size, num_splits=num_splits)
        self.workspace = binding.alloc_workspace(self.params, dev)
        self.out = torch.empty(x.q_nope.shape[:3] + (x.d_v,), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(x.q_nope.shape[:3], dtype=torch.float32, device=dev)

    def prepare(self, binding):
        """Marshal each entry point's arguments once, so a step is three plain C calls."""
        import ctypes
        import torch
        P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        self.lib = binding.LIB
        # append + partial attention in one call (one launch on the 128-head bf16 path)
        self.fwd_append_args = (ctypes.byref(self.params), P(self.new_c), P(self.new_k), 1,
                                binding._DTYPE_CODE[self.new_c.dtype], P(self.positions), P(self.q_nope),
                                P(self.q_pe), P(self.c_kv), P(self.k_pe), P(self.kv_scale), P(self.block_table),
                                P(self.seq_lens), P(self.w_uv), None, None, P(self.workspace),
                                self.workspace.numel(), stream)
        self.comb_args = (ctypes.byref(self.params), P(self.workspace), self.workspace.numel(), P(self.w_uv),
                          P(self.out), P(self.lse), stream)

    def nbytes(self):
        return sum(t.numel() * t.element_size() for t in (self.pool, self.q_nope, self.q_pe, self.workspace))


def hip_runtime():
    """The HIP runtime library torch is using (for events the C library records itself)."""
    import ctypes
    import torch  # noqa: F401  (loads libamdhip64)
    hip = ctypes.CDLL("libamdhip64.so", mode=ctypes.RTLD_GLOBAL)
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return hip


def hip_event_create(hip):
    import ctypes
    ev = ctypes.c_void_p()
    if hip.hipEventCreate(ctypes.byref(ev)) != 0:
        raise RuntimeError("hipEventCreate failed")
    return ev


def hip_elapsed_ms(hip, start, stop):
    import ctypes
    ms = ctypes.c_float()
    rc = hip.hipEventElapsedTime(ctypes.byref(ms), start, stop)
    if rc != 0:
        raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
    return ms.value


def step(r, ev=None):
    """One step: append + partial attention (mla_decode_fwd_append, out = NULL), then the combine
    and up-projection (mla_decode_splitkv_combine).  ev = (stream events e0..e3 around the calls,
    kernel events k0, k1): k0/k1 are recorded by the attention kernel itself at its start and end
    (mla_set_attention_events), so its duration excludes the dispatch gap that the stream events
    around the call include."""
    rc = 0
    if ev is not None:
        ev[0].record()
        ev[1].record()
        rc |= r.lib.mla_set_attention_events(ev[6], ev[7])
    rc |= r.lib.mla_decode_fwd_append(*r.fwd_append_args)
    if ev is not None:
        ev[2].record()
    rc |= r.lib.mla_decode_splitkv_combine(*r.comb_args)
    if ev is not None:
        ev[3].record()
    if rc:
        raise RuntimeError(f"library call failed with status {rc}")


def algorithmic(x):
    """Per-call algorithmic bytes and flops (one cached token = 576 values read once)."""
    tokens = int(x.seq_lens.sum())
    per_tok_bytes = 576 * (1 if x.kv_dtype == "fp8" else 2) + (4 if x.kv_dtype == "fp8" else 0)
    q_bytes = x.batch * x.s_q * x.n_h * (x.d_c + x.d_r) * 2
    attn_bytes = tokens * per_tok_bytes + q_bytes
    # visible tokens per query row: L - s_q + q + 1
    vis = sum(max(0, int(L) - x.s_q + q + 1) for L in x.seq_lens.tolist() for q in range(x.s_q))
    attn_flops = vis * x.n_h * 2 * (x.d_c + x.d_r + x.d_c)
    up_flops = x.batch * x.s_q * x.n_h * x.d_v * x.d_c * 2
    w_bytes = x.n_h * x.d_v * x.d_c * 2
    return dict(tokens=tokens, attn_bytes=attn_bytes, attn_flops=attn_flops, total_bytes=attn_bytes + w_bytes,
                total_flops=attn_flops + up_flops)


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x, budget_s=12.0):
    """The float64 oracle on host cores over a bounded sample of the same workload: whole
    sequences in batch order (repeating the batch if it is short) until about budget_s
    seconds of oracle time."""
    import numpy as np
    from oracle import mla_ref as ref
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    qn = x.q_nope.double().numpy()
    qp = x.q_pe.double().numpy()
    w = x.w_uv.double().numpy()
    tab = x.block_table.numpy()
    done_tokens, spent, seqs, passes = 0, 0.0, 0, 0
    rows_cache = {}
    while spent < budget_s:
        for b in range(x.batch):
            L = int(x.seq_lens[b])
            if b not in rows_cache:
                j = np.arange(L)
                slots = tab[b, j // x.page_size].astype(np.int64) * x.page_size + j % x.page_size
                rows = x.pool[slots].double().numpy()
                if x.kv_dtype == "fp8":
                    from oracle import fp8
                    codes, sc = fp8.quantize_rows(rows.astype(np.float32))
                    rows = fp8.e4m3_decode_table()[codes] * sc.astype(np.float64)[:, None]
                rows_cache[b] = rows if L * 576 * 8 < 2 ** 30 else None
            else:
                rows = rows_cache[b]
            t0 = time.perf_counter()
            for q in range(x.s_q):
                ref.mla_absorbed(qn[b, q], qp[b, q], rows[:, :x.d_c], rows[:, x.d_c:], w, x.softmax_scale,
                                 ref.visible_len(L, x.s_q, q))
            spent += time.perf_counter() - t0
            done_tokens += L
            seqs += 1
            if rows_cache.get(b) is None:
                rows_cache.pop(b, None)
            if spent >= budget_s:
                break
        passes += 1
    return {"value": done_tokens / spent, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{seqs} sequences of {x.batch} in batch order ({done_tokens} cached tokens, s_q={x.s_q}, "
                      f"{passes} pass(es) over the batch), float64 NumPy absorbed-form oracle, {spent:.1f} s"}


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16")
MFMA_F8_COUNTER = "SQ_INSTS_VALU_MFMA_MOPS_F8"   # optional: the E4M3 kernel's score MFMAs


def pmc_summary(args):
    """Attention-kernel HBM traffic from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by the
    ratio the same counter shows for the plain copy kernel of known size in the same run.  If one of the
    result databases also holds SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE and
    SQ_INSTS_VALU_MFMA_MOPS_BF16 for the attention kernel, the record also gets the matrix unit's busy
    fraction (busy cycles summed over all SIMDs / (active cycles per XCD x SIMDs); the database holds
    GRBM_GUI_ACTIVE summed over the XCDs) and the counted bf16 MFMA flops (512 per MOP), medians
    over the dispatches; with SQ_INSTS_VALU_MFMA_MOPS_F8 as well, the E4M3 MFMA flops are counted the
    same way and added.  FETCH_SIZE / WRITE_SIZE of the combine kernel (same runs, same scaling) give
    the whole step's traffic per call, attention plus combine, recorded with the combine's own source
    digest.  The E4M3 step's separate append launch (a few new rows) is not counted."""
    import sqlite3
    kname, ksrc = attn_kernel(make_workload(args.workload))
    vals = {}   # (kernel kind, counter) -> per-dispatch totals
    for path in args.pmc_summary:
        db = sqlite3.connect(path)
        cols = [r[1] for r in db.execute("pragma table_info(counters_collection)")]
        ci = {c: i for i, c in enumerate(cols)}
        per = {}
        for r in db.execute("select * from counters_collection"):
            name, ctr = r[ci["kernel_name"]], r[ci["counter_name"]]
            kind = ("attn" if kname in name else "copy" if "neg_kernel" in name
                    else "comb" if "combine_upproj" in name else None)
            if kind is None or ctr not in ("FETCH_SIZE", "WRITE_SIZE", MFMA_F8_COUNTER) + MFMA_COUNTERS:
                continue
            key = (kind, ctr, path, r[ci["dispatch_id"]])
            per[key] = per.get(key, 0.0) + float(r[ci["value"]])
        for (kind, ctr, _, _), v in per.items():
            vals.setdefault((kind, ctr), []).append(v)
    need = [("attn", "FETCH_SIZE"), ("attn", "WRITE_SIZE"), ("copy", "FETCH_SIZE"), ("copy", "WRITE_SIZE")]
    missing = [k for k in need if k not in vals]
    if missing:
        raise SystemExit(f"counter data missing for {missing}")
    mean = {k: sum(v) / len(v) for k, v in vals.items()}
    copy_bytes = args.copy_calibration_mb * 2 ** 20
    f_read = mean[("copy", "FETCH_SIZE")] * 1024 / copy_bytes
    f_write = mean[("copy", "WRITE_SIZE")] * 1024 / copy_bytes
    fetch = mean[("attn", "FETCH_SIZE")] * 1024 / f_read
    write = mean[("attn", "WRITE_SIZE")] * 1024 / f_write
    rec = {"bytes_per_launch": round(fetch + write), "fetch_bytes": round(fetch), "write_bytes": round(write),
           "copy_factor_fetch": round(f_read, 4), "copy_factor_write": round(f_write, 4),
           "attn_dispatches": len(vals[("attn", "FETCH_SIZE")]), "command": args.pmc_command,
           "kernel": kname, "source_digest": source_digest(ksrc)}
    if ("comb", "FETCH_SIZE") in vals and ("comb", "WRITE_SIZE") in vals:
        c_fetch = mean[("comb", "FETCH_SIZE")] * 1024 / f_read
        c_write = mean[("comb", "WRITE_SIZE")] * 1024 / f_write
        rec.update({"combine_fetch_bytes": round(c_fetch), "combine_write_bytes": round(c_write),
                    "combine_source_digest": source_digest(COMBINE_SRC),
                    "step_bytes_per_launch": round(fetch + write + c_fetch + c_write)})
    if all(("attn", c) in vals for c in MFMA_COUNTERS):
        import statistics
        busy, active, mops = (vals[("attn", c)] for c in MFMA_COUNTERS)
        frac = [b / (a / MI355X_XCDS * MI355X_SIMDS) for b, a in zip(busy, active)]
        rec["mfma_busy_frac"] = round(statistics.median(frac), 4)
        rec["mfma_counted_flops"] = round(statistics.median(mops) * 512)
        if ("attn", MFMA_F8_COUNTER) in vals:
            rec["mfma_counted_flops_bf16"] = rec["mfma_counted_flops"]
            rec["mfma_counted_flops_f8"] = round(statistics.median(vals[("attn", MFMA_F8_COUNTER)]) * 512)
            rec["mfma_counted_flops"] += rec["mfma_counted_flops_f8"]
        print(f"workload {args.workload}: MFMA busy {rec['mfma_busy_frac']:.1%} of active SIMD cycles, "
              f"{rec['mfma_counted_flops'] / 1e9:.2f} GFLOP counted per launch")
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    data = json.load(open(TRAFFIC_FILE)) if os.path.exists(TRAFFIC_FILE) else {}
    data[args.workload] = rec
    json.dump(data, open(TRAFFIC_FILE, "w"), indent=1, sort_keys=True)
    if "step_bytes_per_launch" in rec:
        print(f"workload {args.workload}: combine kernel HBM traffic per launch "
              f"{(rec['combine_fetch_bytes'] + rec['combine_write_bytes']) / 1e6:.1f} MB; whole step "
              f"{rec['step_bytes_per_launch'] / 1e6:.1f} MB")
    print(f"workload {args.workload}: attention kernel HBM traffic per launch {rec['bytes_per_launch'] / 1e6:.1f} MB "
          f"(fetch {fetch / 1e6:.1f} MB, write {write / 1e6:.1f} MB); copy calibration: FETCH_SIZE reads "
          f"{f_read:.4f}x and WRITE_SIZE {f_write:.4f}x the {args.copy_calibration_mb} MiB copied; "
          f"{rec['attn_dispatches']} attention dispatches")


def measured_peaks(dev):
    """Attainable HBM read bandwidth (the attention kernel's buffer->LDS copy form over 4 GiB, cold)
    and bf16 MFMA throughput (32x32x16 chains on every SIMD), with HIP events; best of 3."""
    import ctypes
    import torch
    from mla_latent_kv_03_amd import build as _b
    lib = ctypes.CDLL(_b.PEAKS_LIB)
    lib.mla_peaks_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p]
    lib.mla_peaks_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    wgs = 2048
    nbytes = 4 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    src.fill_(1)
    sink = torch.empty(wgs * 256, dtype=torch.float32, device=dev)

    def timed(fn):
        best = None
        for _ in range(4):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            if fn() != 0:
                raise RuntimeError("peak probe launch failed")
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b)
            best = ms if best is None else min(best, ms)
        return best

    ms_r = timed(lambda: lib.mla_peaks_stream_read(ctypes.c_void_p(src.data_ptr()), nbytes, wgs,
                                                   ctypes.c_void_p(sink.data_ptr()), stream))
    iters = 4096
    ms_m = timed(lambda: lib.mla_peaks_mfma_bf16(ctypes.c_void_p(sink.data_ptr()), 1024, iters, stream))
    del src
    flops = 1024 * 4 * iters * 16 * 32768.0
    return {"hbm_read_gbs": round(nbytes / (ms_r * 1e-3) / 1e9, 1), "bf16_mfma_tflops": round(flops / (ms_m * 1e-3) / 1e12, 1),
            "method": "best of 4: 4 GiB streamed by 2048 workgroups of 16-byte buffer->LDS copies (streaming policy); "
                      "1024 workgroups x 4 waves x 4 chains of 32x32x16 bf16 MFMAs"}


def adjacent(args, dev):
    """Time the rows adjacent to the decode step at the V3 shape (d_model 7168, 128 heads, d_c 512,
    d_r 64, d_h = d_v = 128) on one batch of 64 new tokens, and GQLA's per-group decode; one JSON
    line each with the algorithmic bytes (weights + activations read and written once) over the
    event-timed duration against the 8 TB/s HBM peak.  Weight-streaming products are HBM-bound."""
    import numpy as np
    import torch
    from mla_latent_kv_03_amd import binding, workloads
    B, D = 64, 7168
    g = torch.Generator(device="cpu").manual_seed(6)
    rnd = lambda *shape, std=1.0: (torch.randn(*shape, generator=g) * std).to(torch.bfloat16).to(dev)

    def time_us(fn, reps=20, batches=7):
        """GPU time of one call: the call's launches are captured once in a HIP graph (on a
        side stream); after replays for at least 200 ms (clocks settle), `batches` batches of
        `reps` replays are each timed between two events and the median batch is reported,
        so that neither the host-side marshalling of each call nor a cold start is counted."""
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.2:
            for _ in range(reps):
                graph.replay()
            torch.cuda.synchronize()
        times = []
        for _ in range(batches):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                graph.replay()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b) * 1e3 / reps)
        return statistics.median(times)

    def line(row, what, us, nbytes):
        gbs = nbytes / (us * 1e-6) / 1e9
        print(json.dumps({"row": row, "workload": what, "us": round(us, 2), "algorithmic_bytes": int(nbytes),
                          "achieved_gbs": round(gbs, 1), "peak_gbs": HBM_PEAK_GBS,
                          "frac": round(gbs / HBM_PEAK_GBS, 4), "bound": "hbm", "dtype": "bf16"}), flush=True)

    h = rnd(B, 1, D)
    # cache write: [W^DKV; W^KR] h, RoPE, bf16 rows into a paged pool
    x = workloads.make_decode([4096] * B, page_size=64, seed=7, **workloads.V3)
    pool = x.pool.to(dev)
    table = x.block_table.to(dev)
    params = binding.params_for(x.q_nope, x.q_pe, pool[:, :512], pool[:, 512:], table, x.w_uv,
                                softmax_scale=x.softmax_scale, page_size=64)
    w_dkv, w_kr = rnd(512, D, std=D ** -0.5), rnd(64, D, std=D ** -0.5)
    pos = torch.full((B, 1), 4095, dtype=torch.int32, device=dev)
    ws = binding.alloc_workspace(params, dev)
    cws = torch.empty(binding.LIB.mla_cache_write_workspace_size(ctypes_ref(params), D, 1), dtype=torch.uint8, device=dev)
    us = time_us(lambda: binding.mla_cache_write(params, h, w_dkv, w_kr, pos, table, pool[:, :512], pool[:, 512:],
                                                 workspace=cws))
    line("f1 cache write", "V3: 64 tokens, d_model 7168 -> [c | RoPE k^R] bf16 rows", us,
         (576 * D + B * D) * 2 + B * 576 * 2)
    # query prologue: W^Q (16384 x 7168), W^QR (8192 x 7168), (W^UK)^T (128 x 512 x 128)
    w_q, w_qr = rnd(128 * 128, D, std=D ** -0.5), rnd(128 * 64, D, std=D ** -0.5)
    w_ukt = rnd(128, 512, 128, std=512 ** -0.5)
    qws = torch.empty(binding.LIB.mla_query_prologue_workspace_size(ctypes_ref(params), D, 128), dtype=torch.uint8,
                      device=dev)
    qn = torch.empty(B, 1, 128, 512, dtype=torch.bfloat16, device=dev)
    qp = torch.empty(B, 1, 128, 64, dtype=torch.bfloat16, device=dev)
    us = time_us(lambda: binding.mla_query_prologue(params, h, w_q, w_ukt, w_qr, pos, qn, qp, d_h=128, workspace=qws),
                 reps=10)
    line("f2 query prologue", "V3: 64 tokens, W^Q 16384x7168, W^QR 8192x7168, W^UK 128x128x512", us,
         (128 * 192 * D + 128 * 512 * 128 + B * D) * 2 + B * 128 * 576 * 2)
    del w_q, w_qr
    # output projection, unfolded (W^O 7168 x 16384 on o) and folded (W^OV 7168 x 65536 on u)
    w_o = rnd(D, 128 * 128, std=(128 * 128) ** -0.5)
    o = rnd(B, 1, 128, 128)
    y = torch.empty(B, 1, D, dtype=torch.bfloat16, device=dev)
    ows = torch.empty(binding.LIB.mla_output_projection_workspace_size(ctypes_ref(params), D, 128 * 128, binding.BF16),
                      dtype=torch.uint8, device=dev)
    us = time_us(lambda: binding.mla_output_projection(params, o, w_o, y, workspace=ows), reps=10)
    line("f3 output projection (unfolded)", "V3: 64 rows, W^O 7168x16384 on the decode output", us,
         (D * 128 * 128 + B * 128 * 128 + B * D) * 2)
    w_ov = binding.mla_fold_output_weights(params, w_o, x.w_uv.to(dev))
    u = torch.randn(B, 1, 128, 512, generator=g).to(dev)
    fws = torch.empty(binding.LIB.mla_output_projection_workspace_size(ctypes_ref(params), D, 128 * 512, binding.F32),
                      dtype=torch.uint8, device=dev)
    us = time_us(lambda: binding.mla_output_projection(params, u, w_ov, y, workspace=fws), reps=5)
    line("f3 output projection (folded)", "V3: 64 rows, W^OV 7168x65536 on float32 latents", us,
         D * 128 * 512 * 2 + B * 128 * 512 * 4 + B * D * 2)
    del w_ov, w_o
    # GQLA per-group decode: 8 groups of 16 heads, s_q = 2, 32 sequences of 4096 tokens
    xg = workloads.make_decode([4096] * 32, s_q=2, page_size=64, seed=8, **workloads.V3)
    poolg = xg.pool.to(dev)
    pg = binding.params_for(xg.q_nope, xg.q_pe, poolg[:, :512], poolg[:, 512:], xg.block_table, xg.w_uv,
                            softmax_scale=xg.softmax_scale, page_size=64)
    k_exp, v_exp = binding.mla_gqla_expand_cache(pg, rnd(8, 128, 512, std=512 ** -0.5), rnd(8, 128, 512, std=512 ** -0.5),
                                                 poolg[:, :512])
    q_c, q_pe = rnd(32, 2, 128, 128), xg.q_pe.to(dev)
    bt, sl = xg.block_table.to(dev), xg.seq_lens.to(dev)
    gws = torch.empty(binding.LIB.mla_gqla_decode_workspace_size(ctypes_ref(pg), 8, 128), dtype=torch.uint8, device=dev)
    out = torch.empty(32, 2, 128, 128, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(32, 2, 128, dtype=torch.float32, device=dev)
    us = time_us(lambda: binding.mla_gqla_decode(pg, q_c, q_pe, k_exp, v_exp, poolg[:, 512:], bt, sl, out, lse,
                                                 workspace=gws), reps=10)
    tokens = 32 * 4096
    line("f4 GQLA per-group decode", "32 sequences x 4096 tokens, s_q 2, 8 groups of 16 heads, d_h 128 + d_r 64, d_v 128",
         us, tokens * 8 * (128 + 128 + 64) * 2 + 32 * 2 * 128 * (128 + 64) * 2)


def ctypes_ref(params):
    import ctypes
    return ctypes.byref(params)


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args)
        return
    if args.adjacent:
        import torch
        torch.cuda.set_device(0)
        adjacent(args, "cuda:0")
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from mla_latent_kv_03_amd import binding
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    print(f"[bench] workload {args.workload}: generating inputs", file=sys.stderr, flush=True)
    x = make_workload(args.workload)
    first = Resident(x, binding, args.num_splits, dev)
    copies = [first]
    n_copies = max(2, min(8, math.ceil(args.rotate_bytes / max(1, first.nbytes())) + 1))
    for _ in range(n_copies - 1):
        copies.append(Resident(x, binding, args.num_splits, dev))
    for r in copies:
        r.prepare(binding)
    G = binding.mla_decode_num_splits(first.params)
    print(f"[bench] {n_copies} resident copies of {first.nbytes() / 1e6:.1f} MB, G={G}", file=sys.stderr, flush=True)

    t_w = time.perf_counter()
    i = 0
    while i < args.warmup or (time.perf_counter() - t_w) * 1e3 < args.min_warmup_ms:
        step(copies[i % n_copies])
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    n_warm = i
    if args.copy_calibration_mb:
        # a plain streaming kernel of known traffic (reads and writes n bytes): torch's negation
        n = args.copy_calibration_mb * 2 ** 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # Timed region 1 (the step rate): K steps with nothing but the three library calls.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(copies[i % n_copies])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    # Timed region 2 (per-kernel durations): the same K steps with HIP events.  The attention
    # kernel's own launch records its kernel events (mla_set_attention_events); they are created
    # and read through the HIP runtime torch has loaded, since torch did not record them.  The
    # stream events around each call also count dispatch gaps.  Events add dispatch work, which
    # is why region 1 runs without them.
    hip = hip_runtime()
    evs = []
    for _ in range(args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)] + [None, None]
        k = [hip_event_create(hip), hip_event_create(hip)]
        evs.append(e + k)
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(copies[i % n_copies], evs[i])
    torch.cuda.synchronize()
    binding.mla_set_attention_events(None, None)
    attn_ms = sum(hip_elapsed_ms(hip, e[6], e[7]) for e in evs) / args.steps
    for e in evs:
        hip.hipEventDestroy(e[6])
        hip.hipEventDestroy(e[7])
    attn_call_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps
    comb_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps
    # Distribution of the whole step (stream events around the two calls, dispatch included).
    step_us = sorted(e[0].elapsed_time(e[3]) * 1e3 for e in evs)
    pct = lambda q: step_us[min(len(step_us) - 1, int(round(q * (len(step_us) - 1))))]
    print(f"[bench] {args.steps} steps: {ms_step * 1e3:.1f} us/step; with events: attention kernel "
          f"{attn_ms * 1e3:.1f} us (append + attention call incl. dispatch {attn_call_ms * 1e3:.1f} us), "
          f"combine {comb_ms * 1e3:.1f} us", file=sys.stderr, flush=True)

    alg = algorithmic(x)
    kname, ksrc = attn_kernel(x)
    attn_gbs = alg["attn_bytes"] / (attn_ms * 1e-3) / 1e9
    attn_tflops = alg["attn_flops"] / (attn_ms * 1e-3) / 1e12
    traffic = None
    counted = {}
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE)).get(args.workload)
        # Counters taken on another kernel, or on an older source of this one, do not count.
        if rec and rec.get("kernel") == kname and rec.get("source_digest") == source_digest(ksrc):
            traffic = rec.get("bytes_per_launch")
            # The same bytes over this run's kernel time, and the matrix unit's busy fraction
            # from the counters of the profiled run.
            counted["traffic_gbs"] = round(traffic / (attn_ms * 1e-3) / 1e9, 1)
            if "mfma_busy_frac" in rec:
                counted["mfma_busy_frac_counter"] = rec["mfma_busy_frac"]
            # Whole step (attention + combine launches) against the step's algorithmic bytes
            # (cache and queries once, W^UV once), if the combine is the one the counters saw.
            if "step_bytes_per_launch" in rec and rec.get("combine_source_digest") == source_digest(COMBINE_SRC):
                counted["step_traffic"] = rec["step_bytes_per_launch"]
                counted["step_algorithmic_bytes"] = alg["total_bytes"]
                counted["step_traffic_ratio"] = round(rec["step_bytes_per_launch"] / alg["total_bytes"], 4)
    peaks = None if args.no_peaks else measured_peaks(dev)
    if peaks:
        print(f"[bench] measured peaks: HBM read {peaks['hbm_read_gbs']:.0f} GB/s, bf16 MFMA "
              f"{peaks['bf16_mfma_tflops']:.0f} TFLOP/s", file=sys.stderr, flush=True)
        counted["measured_peaks"] = peaks
        counted["frac_of_measured_hbm"] = round(attn_gbs / peaks["hbm_read_gbs"], 4)
        counted["mfma_frac_of_measured"] = round(attn_tflops / peaks["bf16_mfma_tflops"], 4)
    # The kernel's bound: HBM if its algorithmic intensity is below the machine's ridge (bf16 peak /
    # HBM peak, 314.6 flop/B), else the bf16 matrix unit (s_q = 2, or an E4M3 cache's half bytes).
    mfma_bound = alg["attn_flops"] / alg["attn_bytes"] > BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        bound = {"bound": "mfma", "achieved": round(attn_tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(attn_tflops / BF16_PEAK_TFLOPS, 4)}
    else:
        bound = {"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(attn_gbs / HBM_PEAK_GBS, 4)}
    roof = {**bound, "traffic": traffic,
            "kernel": kname, "kernel_us": round(attn_ms * 1e3, 2),
            "hbm_gbs": round(attn_gbs, 1), "hbm_frac": round(attn_gbs / HBM_PEAK_GBS, 4),
            "mfma_tflops": round(attn_tflops, 1), "mfma_frac": round(attn_tflops / BF16_PEAK_TFLOPS, 4),
            "algorithmic_bytes_per_launch": alg["attn_bytes"], "algorithmic_flops_per_launch": alg["attn_flops"],
            **counted}
    result = {
        "metric": METRIC, "value": round(alg["tokens"] / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if x.kv_dtype == "bf16" else "bf16+fp8e4m3",
        "data": "synthetic (seeded N(0,1) queries and cache, N(0,1/512) W^UV; no trained weights)",
        "config": {"workload": args.workload, "batch": x.batch, "s_q": x.s_q, "n_h": x.n_h, "d_c": x.d_c,
                   "d_r": x.d_r, "d_v": x.d_v, "context": int(x.seq_lens.max()),
                   "cached_tokens_per_step": alg["tokens"], "kv_dtype": x.kv_dtype, "page_size": x.page_size,
                   "num_splits": G, "step": "append + partial attention (one call, mla_decode_fwd_append) + "
                                            "combine/up-projection (mla_decode_splitkv_combine)",
                   "warmup_steps_run": n_warm,
                   "step_us_events": {"p10": round(pct(0.1), 2), "median": round(pct(0.5), 2),
                                      "p90": round(pct(0.9), 2), "attention_kernel_mean": round(attn_ms * 1e3, 2),
                                      "combine_call_mean": round(comb_ms * 1e3, 2)},
                   "hbm_gbs_whole_step": round(alg["total_bytes"] / (ms_step * 1e-3) / 1e9, 1)},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(x)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
