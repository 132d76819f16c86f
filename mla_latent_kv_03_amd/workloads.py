"""Seeded synthetic inputs for MLA decode (shapes of the DeepSeek-V2/V3 MLA layer).

This module only draws random numbers and lays them out (page pools, block
tables, lengths).  It holds none of the method's arithmetic: no projection,
rotation, softmax, quantization or attention.  Both the GPU tests and the CPU
oracle consume what it produces.

Recipe (fixed draw order, NumPy ``default_rng(seed)``):
  1. per-sequence lengths (if drawn), 2. page permutation (if paged),
  3. q_nope, 4. q_pe, 5. the cache pool rows [c (d_c) | k_pe (d_r)] in pool-slot order,
  6. W^UV.
Queries and cache values are N(0, 1); W^UV is N(0, 1/d_c) (fan-in rule).
bf16 tensors are the float32 draws rounded to nearest-even.
For an fp8 cache the pool holds the float32 draws; the quantized cache is made by
the append step (GPU) or its oracle.
"""
from dataclasses import dataclass, field
import math

import numpy as np
import torch

V3 = dict(n_h=128, d_c=512, d_r=64, d_v=128)     # DeepSeek-V2/V3 MLA dimensions
V3_SCALE = 1.0 / math.sqrt(128 + 64)              # 1/sqrt(d_h + d_r)


@dataclass
class DecodeInputs:
    """One decode call's inputs on the host (torch CPU tensors)."""
    q_nope: torch.Tensor          # [B, s_q, n_h, d_c]
    q_pe: torch.Tensor            # [B, s_q, n_h, d_r]
    pool: torch.Tensor            # [num_pages * page_size, d_c + d_r]  (fp32 source for fp8 caches)
    block_table: torch.Tensor     # int32 [B, max_pages_per_seq]
    seq_lens: torch.Tensor        # int32 [B]
    w_uv: torch.Tensor            # [n_h, d_v, d_c]
    page_size: int
    softmax_scale: float
    kv_dtype: str                 # "f32", "bf16" or "fp8"
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def batch(self):
        return int(self.q_nope.shape[0])

    @property
    def s_q(self):
        return int(self.q_nope.shape[1])

    @property
    def n_h(self):
        return int(self.q_nope.shape[2])

    @property
    def d_c(self):
        return int(self.q_nope.shape[3])

    @property
    def d_r(self):
        return int(self.q_pe.shape[3])

    @property
    def d_v(self):
        return int(self.w_uv.shape[1])

    @property
    def num_pages(self):
        return int(self.pool.shape[0]) // self.page_size


def _normal(rng, shape, std=1.0):
    return (rng.standard_normal(int(np.prod(shape)), dtype=np.float32) * np.float32(std)).reshape(shape)


def _to(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(dtype) if dtype != torch.float32 else t


def make_decode(seq_lens, *, s_q=1, n_h=128, d_c=512, d_r=64, d_v=128, page_size=64,
                paged=True, q_dtype="bf16", kv_dtype="bf16", w_dtype=None,
                softmax_scale=None, seed=0, poison=False, name=""):
    """Draw one decode call.

    seq_lens: per-sequence cache lengths (including the s_q new tokens), or a
    function of the generator that draws them (drawn first).
    paged=True: the pool has sum_b ceil(L_b / P) pages, dealt to the sequences in
    the order of a random permutation; paged=False: page_size is raised to the
    longest sequence (rounded up to 64) and sequence b owns page b.
    poison=True fills pool slots that no sequence reads (tails of last pages and
    one spare page) with NaN instead of normal draws.
    """
    rng = np.random.default_rng(seed)
    if callable(seq_lens):
        seq_lens = seq_lens(rng)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B = len(seq_lens)
    if not paged:
        page_size = max(64, int(-(-max(int(seq_lens.max()) if B else 1, 1) // 64) * 64))
    pages_per_seq = [max(1, -(-int(L) // page_size)) for L in seq_lens]
    spare = 1 if poison else 0
    num_pages = sum(pages_per_seq) + spare
    if paged:
        perm = rng.permutation(num_pages)
    else:
        perm = np.arange(num_pages)
    max_pages = max(pages_per_seq) if B else 1
    table = np.zeros((B, max_pages), dtype=np.int32)
    nxt = 0
    for b in range(B):
        for k in range(pages_per_seq[b]):
            table[b, k] = perm[nxt]
            nxt += 1
    qt = {"bf16": torch.bfloat16, "f32": torch.float32}[q_dtype]
    wt = {"bf16": torch.bfloat16, "f32": torch.float32}[w_dtype or q_dtype]
    q_nope = _to(_normal(rng, (B, s_q, n_h, d_c)), qt)
    q_pe = _to(_normal(rng, (B, s_q, n_h, d_r)), qt)
    pool32 = _normal(rng, (num_pages * page_size, d_c + d_r))
    w_uv = _to(_normal(rng, (n_h, d_v, d_c), 1.0 / math.sqrt(d_c)), wt)
    if poison:
        used = np.zeros(num_pages * page_size, dtype=bool)
        for b in range(B):
            for j in range(int(seq_lens[b])):
                used[int(table[b, j // page_size]) * page_size + j % page_size] = True
        pool32[~used] = np.nan
    pool_dtype = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.float32}[kv_dtype]
    pool = _to(pool32, pool_dtype)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d_v + d_r)
    return DecodeInputs(q_nope=q_nope, q_pe=q_pe, pool=pool, block_table=torch.from_numpy(table),
                        seq_lens=torch.from_numpy(seq_lens.astype(np.int32)), w_uv=w_uv,
                        page_size=page_size, softmax_scale=float(softmax_scale), kv_dtype=kv_dtype,
                        name=name, meta={"seed": seed, "paged": paged})


# ----------------------------------------------------------------------------
# The five workloads (seed = workload number)
# ----------------------------------------------------------------------------

def tiny_layer(seed=1, L=128, n_h=8, d=64, d_c=64, d_h=16, d_r=16):
    """Hidden states and the six projection matrices of one tiny MLA layer (float64).

    h ~ N(0, 1); every weight ~ N(0, 1/fan_in) with fan_in its input dimension.
    Returns a dict: h [L, d], dkv [d_c, d], q [n_h*d_h, d], uk [n_h, d_h, d_c],
    uv [n_h, d_h, d_c], kr [d_r, d], qr [n_h*d_r, d], plus the dimensions.
    """
    rng = np.random.default_rng(seed)

    def w(rows, fan_in):
        return rng.standard_normal((rows, fan_in)) / math.sqrt(fan_in)

    h = rng.standard_normal((L, d))
    out = dict(h=h, dkv=w(d_c, d), q=w(n_h * d_h, d), uk=w(n_h * d_h, d_c).reshape(n_h, d_h, d_c),
               uv=w(n_h * d_h, d_c).reshape(n_h, d_h, d_c), kr=w(d_r, d), qr=w(n_h * d_r, d))
    out.update(L=L, n_h=n_h, d=d, d_c=d_c, d_h=d_h, d_r=d_r, scale=1.0 / math.sqrt(d_h + d_r))
    return out


def v3_decode(seed=2, B=64, L=4096):
    """Batch 64, one query token, contiguous 4096-token latent caches, bf16."""
    return make_decode([L] * B, paged=False, seed=seed, softmax_scale=V3_SCALE, name="v3_decode_b64_l4096", **V3)


def v3_paged(seed=3, B=128, lo=1024, hi=16384, page_size=64, poison=False):
    """Batch 128, lengths uniform in [1024, 16384], 64-token pages dealt by a random permutation."""
    return make_decode(lambda rng: rng.integers(lo, hi, size=B, endpoint=True), page_size=page_size, seed=seed, softmax_scale=V3_SCALE,
                       poison=poison, name="v3_paged_b128", **V3)


def v3_mtp(seed=4, B=32, L=32768, page_size=64):
    """Two query tokens per sequence (causal within the pair), 32768-token paged caches."""
    return make_decode([L] * B, s_q=2, page_size=page_size, seed=seed, softmax_scale=V3_SCALE,
                       name="v3_mtp_b32_l32768", **V3)


def v3_long_fp8(seed=5, B=4, L=131072):
    """Batch 4, 131072-token caches to be stored as E4M3 + per-token scale; 64 splits each."""
    return make_decode([L] * B, paged=False, kv_dtype="fp8", seed=seed, softmax_scale=V3_SCALE,
                       name="v3_long_fp8_b4_l131072", **V3)


def layer_weights(seed, *, d_model, n_h, d_c, d_h, d_r, d_v, n_tokens, with_o=True):
    """Hidden states of n_tokens new tokens and the projection weights of one MLA layer, as
    float32 draws (fixed order: h, W^DKV, W^KR, W^Q, W^UK, W^QR, W^UV, W^O).  h ~ N(0, 1);
    every weight ~ N(0, 1/fan_in) with fan_in its input width (d_model for the projections of
    h, d_c for W^UK / W^UV, n_h * d_v for W^O).  Layouts: dkv [d_c, d_model], kr [d_r, d_model],
    q [n_h*d_h, d_model], uk [n_h, d_h, d_c], qr [n_h*d_r, d_model], uv [n_h, d_v, d_c],
    o [d_model, n_h*d_v]."""
    rng = np.random.default_rng(seed)
    out = {"h": _normal(rng, (n_tokens, d_model))}
    for name, shape, fan in (("dkv", (d_c, d_model), d_model), ("kr", (d_r, d_model), d_model),
                             ("q", (n_h * d_h, d_model), d_model), ("uk", (n_h, d_h, d_c), d_c),
                             ("qr", (n_h * d_r, d_model), d_model), ("uv", (n_h, d_v, d_c), d_c)):
        out[name] = _normal(rng, shape, 1.0 / math.sqrt(fan))
    if with_o:
        out["o"] = _normal(rng, (d_model, n_h * d_v), 1.0 / math.sqrt(n_h * d_v))
    return out
