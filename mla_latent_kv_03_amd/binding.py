"""ctypes binding of libmla_decode.so (include/mla_decode.h).

Argument marshalling only: every step of decode, combine and append runs in the
library's HIP kernels.  torch tensors supply device memory and the current HIP
stream.  Importing this module loads the library and raises if it is missing or
does not export the ABI; there is no fallback of any kind.
"""
import ctypes
import os

import torch

from . import build as _build

LIB_PATH = _build.LIB_PATH

F32, BF16, FP8 = 0, 1, 2
_DTYPE_CODE = {torch.float32: F32, torch.bfloat16: BF16, torch.float8_e4m3fn: FP8, torch.uint8: FP8}
STATUS = {0: "MLA_OK", 1: "MLA_ERR_NULL", 2: "MLA_ERR_SHAPE", 3: "MLA_ERR_DTYPE", 4: "MLA_ERR_WORKSPACE",
          5: "MLA_ERR_HIP", 6: "MLA_ERR_UNSUPPORTED", 7: "MLA_ERR_TOO_LARGE"}
EXPORTS = ("mla_decode_num_splits", "mla_decode_workspace_size", "mla_decode_fwd", "mla_decode_splitkv_combine",
           "mla_paged_cache_append", "mla_decode_fwd_append", "mla_set_attention_events", "mla_status_string",
           "mla_abi_version", "mla_decode_fwd_noalloc", "mla_decode_noalloc_capacity", "mla_cache_write",
           "mla_cache_write_workspace_size", "mla_query_prologue", "mla_query_prologue_workspace_size",
           "mla_output_projection", "mla_output_projection_workspace_size", "mla_fold_output_weights",
           "mla_fold_output_weights_workspace_size", "mla_gqla_expand_cache", "mla_gqla_decode",
           "mla_gqla_decode_workspace_size")


class DecodeParams(ctypes.Structure):
    """Mirror of mla_decode_params_t."""
    _fields_ = [("batch", ctypes.c_int32), ("s_q", ctypes.c_int32), ("n_h", ctypes.c_int32),
                ("d_c", ctypes.c_int32), ("d_r", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("num_splits", ctypes.c_int32),
                ("c_kv_stride", ctypes.c_int64), ("k_pe_stride", ctypes.c_int64),
                ("softmax_scale", ctypes.c_float),
                ("q_dtype", ctypes.c_int), ("kv_dtype", ctypes.c_int), ("w_dtype", ctypes.c_int),
                ("out_dtype", ctypes.c_int)]


class MLAError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__(f"{where}: {lib_status_string(code)} (status {code})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m mla_latent_kv_03_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name in EXPORTS:
        if not hasattr(lib, name):
            raise ImportError(f"{LIB_PATH} does not export {name}")
    P = ctypes.POINTER(DecodeParams)
    vp, i32p, f32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    lib.mla_decode_num_splits.argtypes = [P]
    lib.mla_decode_num_splits.restype = ctypes.c_int32
    lib.mla_decode_workspace_size.argtypes = [P]
    lib.mla_decode_workspace_size.restype = ctypes.c_size_t
    lib.mla_decode_fwd.argtypes = [P, vp, vp, vp, vp, f32p, i32p, i32p, vp, vp, f32p, vp, ctypes.c_size_t, vp]
    lib.mla_decode_fwd.restype = ctypes.c_int
    lib.mla_decode_splitkv_combine.argtypes = [P, vp, ctypes.c_size_t, vp, vp, f32p, vp]
    lib.mla_decode_splitkv_combine.restype = ctypes.c_int
    lib.mla_paged_cache_append.argtypes = [P, vp, vp, ctypes.c_int32, ctypes.c_int, i32p, i32p, vp, vp, f32p, vp]
    lib.mla_paged_cache_append.restype = ctypes.c_int
    lib.mla_decode_fwd_append.argtypes = [P, vp, vp, ctypes.c_int32, ctypes.c_int, i32p, vp, vp, vp, vp, f32p, i32p,
                                          i32p, vp, vp, f32p, vp, ctypes.c_size_t, vp]
    lib.mla_decode_fwd_append.restype = ctypes.c_int
    lib.mla_decode_fwd_noalloc.argtypes = [P, vp, vp, vp, vp, f32p, i32p, i32p, vp, vp, f32p, vp]
    lib.mla_decode_fwd_noalloc.restype = ctypes.c_int
    lib.mla_decode_noalloc_capacity.argtypes = []
    lib.mla_decode_noalloc_capacity.restype = ctypes.c_size_t
    i32, f32, sz = ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.mla_cache_write_workspace_size.argtypes = [P, i32, i32]
    lib.mla_cache_write_workspace_size.restype = sz
    lib.mla_cache_write.argtypes = [P, i32, i32, vp, vp, vp, i32p, f32, i32p, vp, vp, f32p, vp, sz, vp]
    lib.mla_cache_write.restype = ctypes.c_int
    lib.mla_query_prologue_workspace_size.argtypes = [P, i32, i32]
    lib.mla_query_prologue_workspace_size.restype = sz
    lib.mla_query_prologue.argtypes = [P, i32, i32, vp, vp, vp, vp, i32p, f32, vp, vp, vp, sz, vp]
    lib.mla_query_prologue.restype = ctypes.c_int
    lib.mla_output_projection_workspace_size.argtypes = [P, i32, i32, ctypes.c_int]
    lib.mla_output_projection_workspace_size.restype = sz
    lib.mla_output_projection.argtypes = [P, i32, i32, ctypes.c_int, vp, vp, vp, vp, sz, vp]
    lib.mla_output_projection.restype = ctypes.c_int
    lib.mla_fold_output_weights_workspace_size.argtypes = [P]
    lib.mla_fold_output_weights_workspace_size.restype = sz
    lib.mla_fold_output_weights.argtypes = [P, i32, vp, vp, vp, vp, sz, vp]
    lib.mla_fold_output_weights.restype = ctypes.c_int
    lib.mla_gqla_expand_cache.argtypes = [P, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.mla_gqla_expand_cache.restype = ctypes.c_int
    lib.mla_gqla_decode_workspace_size.argtypes = [P, i32, i32]
    lib.mla_gqla_decode_workspace_size.restype = sz
    lib.mla_gqla_decode.argtypes = [P, i32, i32, vp, vp, vp, vp, vp, i32p, i32p, vp, f32p, vp, sz, vp]
    lib.mla_gqla_decode.restype = ctypes.c_int
    lib.mla_set_attention_events.argtypes = [vp, vp]
    lib.mla_set_attention_events.restype = ctypes.c_int
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_abi_version.argtypes = []
    lib.mla_abi_version.restype = ctypes.c_int32
    return lib


LIB = _load()


def lib_status_string(code):
    return LIB.mla_status_string(int(code)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(code, where):
    if code != 0:
        raise MLAError(code, where)


def make_params(*, batch, s_q, n_h, d_c, d_r, d_v, page_size, num_pages, max_pages_per_seq,
                c_kv_stride, k_pe_stride, softmax_scale, q_dtype, kv_dtype, w_dtype=None, out_dtype=None,
                num_splits=0):
    w_dtype = q_dtype if w_dtype is None else w_dtype
    out_dtype = q_dtype if out_dtype is None else out_dtype
    return DecodeParams(int(batch), int(s_q), int(n_h), int(d_c), int(d_r), int(d_v), int(page_size),
                        int(num_pages), int(max_pages_per_seq), int(num_splits), int(c_kv_stride),
                        int(k_pe_stride), float(softmax_scale), int(q_dtype), int(kv_dtype), int(w_dtype),
                        int(out_dtype))


def params_for(q_nope, q_pe, c_kv, k_pe, block_table, w_uv, *, softmax_scale, page_size, num_splits=0):
    """Fill mla_decode_params_t from tensors (c_kv / k_pe are [slots, width] views of the pool)."""
    B, s_q, n_h, d_c = q_nope.shape
    d_r = q_pe.shape[-1]
    d_v = w_uv.shape[1]
    slots = c_kv.shape[0]
    return make_params(batch=B, s_q=s_q, n_h=n_h, d_c=d_c, d_r=d_r, d_v=d_v, page_size=page_size,
                       num_pages=slots // page_size, max_pages_per_seq=block_table.shape[1],
                       c_kv_stride=c_kv.stride(0), k_pe_stride=k_pe.stride(0), softmax_scale=softmax_scale,
                       q_dtype=_DTYPE_CODE[q_nope.dtype], kv_dtype=_DTYPE_CODE[c_kv.dtype],
                       w_dtype=_DTYPE_CODE[w_uv.dtype], out_dtype=_DTYPE_CODE[q_nope.dtype],
                       num_splits=num_splits)


def mla_decode_num_splits(params):
    g = LIB.mla_decode_num_splits(ctypes.byref(params))
    if g <= 0:
        raise MLAError(2, "mla_decode_num_splits")
    return g


def mla_decode_workspace_size(params):
    n = LIB.mla_decode_workspace_size(ctypes.byref(params))
    if n == 0:
        raise MLAError(2, "mla_decode_workspace_size")
    return n


def alloc_workspace(params, device=None):
    return torch.empty(mla_decode_workspace_size(params), dtype=torch.uint8, device=device or "cuda")


def mla_decode_fwd(q_nope, q_pe, c_kv, k_pe, block_table, seq_lens, w_uv, *, softmax_scale, page_size,
                   kv_scale=None, num_splits=0, out=None, lse=None, workspace=None, partials_only=False,
                   params=None):
    """Absorbed MLA decode; returns (out, lse, workspace).

    c_kv [slots, d_c] and k_pe [slots, d_r] are views of the page pool (a packed pool
    [slots, d_c + d_r] gives pool[:, :d_c] and pool[:, d_c:]).  With partials_only the
    call stops after the split partials (out is None).
    """
    if params is None:
        params = params_for(q_nope, q_pe, c_kv, k_pe, block_table, w_uv, softmax_scale=softmax_scale,
                            page_size=page_size, num_splits=num_splits)
    dev = q_nope.device
    if workspace is None:
        workspace = alloc_workspace(params, dev)
    if not partials_only:
        if out is None:
            out = torch.empty(q_nope.shape[:3] + (w_uv.shape[1],), dtype=q_nope.dtype, device=dev)
        if lse is None:
            lse = torch.empty(q_nope.shape[:3], dtype=torch.float32, device=dev)
    else:
        out, lse = None, None
    code = LIB.mla_decode_fwd(ctypes.byref(params), _ptr(q_nope), _ptr(q_pe), _ptr(c_kv), _ptr(k_pe),
                              _ptr(kv_scale), _ptr(block_table), _ptr(seq_lens), _ptr(w_uv), _ptr(out), _ptr(lse),
                              _ptr(workspace), workspace.numel(), _stream())
    _check(code, "mla_decode_fwd")
    return out, lse, workspace


def mla_decode_fwd_noalloc(q_nope, q_pe, c_kv, k_pe, block_table, seq_lens, w_uv, *, softmax_scale, page_size,
                           kv_scale=None, num_splits=0, out=None, lse=None, params=None):
    """mla_decode_fwd with the library's static workspace (no workspace argument); returns (out, lse)."""
    if params is None:
        params = params_for(q_nope, q_pe, c_kv, k_pe, block_table, w_uv, softmax_scale=softmax_scale,
                            page_size=page_size, num_splits=num_splits)
    dev = q_nope.device
    if out is None:
        out = torch.empty(q_nope.shape[:3] + (w_uv.shape[1],), dtype=q_nope.dtype, device=dev)
    if lse is None:
        lse = torch.empty(q_nope.shape[:3], dtype=torch.float32, device=dev)
    code = LIB.mla_decode_fwd_noalloc(ctypes.byref(params), _ptr(q_nope), _ptr(q_pe), _ptr(c_kv), _ptr(k_pe),
                                      _ptr(kv_scale), _ptr(block_table), _ptr(seq_lens), _ptr(w_uv), _ptr(out),
                                      _ptr(lse), _stream())
    _check(code, "mla_decode_fwd_noalloc")
    return out, lse


def mla_decode_fwd_append(c_new, k_pe_new, positions, q_nope, q_pe, c_kv, k_pe, block_table, seq_lens, w_uv, *,
                          softmax_scale, page_size, kv_scale=None, num_splits=0, out=None, lse=None, workspace=None,
                          partials_only=False, params=None):
    """mla_paged_cache_append of the new rows ([B, s_new, d]) at `positions`, then mla_decode_fwd, in
    one call (one launch on the 128-head bf16 path); returns (out, lse, workspace)."""
    if params is None:
        params = params_for(q_nope, q_pe, c_kv, k_pe, block_table, w_uv, softmax_scale=softmax_scale,
                            page_size=page_size, num_splits=num_splits)
    dev = q_nope.device
    if workspace is None:
        workspace = alloc_workspace(params, dev)
    if not partials_only:
        if out is None:
            out = torch.empty(q_nope.shape[:3] + (w_uv.shape[1],), dtype=q_nope.dtype, device=dev)
        if lse is None:
            lse = torch.empty(q_nope.shape[:3], dtype=torch.float32, device=dev)
    else:
        out, lse = None, None
    code = LIB.mla_decode_fwd_append(ctypes.byref(params), _ptr(c_new), _ptr(k_pe_new), int(c_new.shape[1]),
                                     _DTYPE_CODE[c_new.dtype], _ptr(positions), _ptr(q_nope), _ptr(q_pe), _ptr(c_kv),
                                     _ptr(k_pe), _ptr(kv_scale), _ptr(block_table), _ptr(seq_lens), _ptr(w_uv),
                                     _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream())
    _check(code, "mla_decode_fwd_append")
    return out, lse, workspace


def mla_decode_splitkv_combine(params, workspace, w_uv, out, lse=None):
    code = LIB.mla_decode_splitkv_combine(ctypes.byref(params), _ptr(workspace), workspace.numel(), _ptr(w_uv),
                                          _ptr(out), _ptr(lse), _stream())
    _check(code, "mla_decode_splitkv_combine")
    return out, lse


def mla_paged_cache_append(params, c_new, k_pe_new, positions, block_table, c_kv, k_pe, kv_scale=None):
    """Write [c | k^R] rows of the new tokens ([B, s_new, d]) into the pool views c_kv / k_pe."""
    s_new = c_new.shape[1]
    code = LIB.mla_paged_cache_append(ctypes.byref(params), _ptr(c_new), _ptr(k_pe_new), int(s_new),
                                      _DTYPE_CODE[c_new.dtype], _ptr(positions), _ptr(block_table), _ptr(c_kv),
                                      _ptr(k_pe), _ptr(kv_scale), _stream())
    _check(code, "mla_paged_cache_append")


def _workspace(nbytes, where, device):
    if nbytes == 0:
        raise MLAError(2, where)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def mla_cache_write(params, h, w_dkv, w_kr, positions, block_table, c_kv, k_pe, kv_scale=None, *, rope_base=10000.0,
                    workspace=None):
    """Cache rows of new tokens from their hidden states h [B, s_new, d_model], written into the pool views."""
    B, s_new, d_model = h.shape
    if workspace is None:
        workspace = _workspace(LIB.mla_cache_write_workspace_size(ctypes.byref(params), d_model, s_new),
                               "mla_cache_write_workspace_size", h.device)
    code = LIB.mla_cache_write(ctypes.byref(params), int(d_model), int(s_new), _ptr(h), _ptr(w_dkv), _ptr(w_kr),
                               _ptr(positions), float(rope_base), _ptr(block_table), _ptr(c_kv), _ptr(k_pe),
                               _ptr(kv_scale), _ptr(workspace), workspace.numel(), _stream())
    _check(code, "mla_cache_write")
    return workspace


def mla_query_prologue(params, h, w_q, w_uk_t, w_qr, positions, q_nope=None, q_pe=None, *, d_h, rope_base=10000.0,
                       workspace=None):
    """q_nope [B, s_q, n_h, d_c] and q_pe [B, s_q, n_h, d_r] from hidden states h [B, s_q, d_model]."""
    B, s_q, d_model = h.shape
    dt = h.dtype
    if q_nope is None:
        q_nope = torch.empty(B, s_q, params.n_h, params.d_c, dtype=dt, device=h.device)
    if q_pe is None:
        q_pe = torch.empty(B, s_q, params.n_h, params.d_r, dtype=dt, device=h.device)
    if workspace is None:
        workspace = _workspace(LIB.mla_query_prologue_workspace_size(ctypes.byref(params), d_model, int(d_h)),
                               "mla_query_prologue_workspace_size", h.device)
    code = LIB.mla_query_prologue(ctypes.byref(params), int(d_model), int(d_h), _ptr(h), _ptr(w_q), _ptr(w_uk_t),
                                  _ptr(w_qr), _ptr(positions), float(rope_base), _ptr(q_nope), _ptr(q_pe),
                                  _ptr(workspace), workspace.numel(), _stream())
    _check(code, "mla_query_prologue")
    return q_nope, q_pe


def mla_output_projection(params, x, w, y=None, *, workspace=None):
    """y [B, s_q, d_model] = W x for x [B, s_q, n_h, width_per_head] (o with W^O, or u with W^OV)."""
    B, s_q = x.shape[:2]
    width = x[0, 0].numel()
    d_model = w.shape[0]
    x_dt = _DTYPE_CODE[x.dtype]
    if y is None:
        y = torch.empty(B, s_q, d_model, dtype=torch.bfloat16 if params.out_dtype == BF16 else torch.float32,
                        device=x.device)
    if workspace is None:
        workspace = _workspace(LIB.mla_output_projection_workspace_size(ctypes.byref(params), d_model, width, x_dt),
                               "mla_output_projection_workspace_size", x.device)
    code = LIB.mla_output_projection(ctypes.byref(params), int(d_model), int(width), x_dt, _ptr(x), _ptr(w), _ptr(y),
                                     _ptr(workspace), workspace.numel(), _stream())
    _check(code, "mla_output_projection")
    return y


def mla_fold_output_weights(params, w_o, w_uv, w_ov=None):
    """W^OV [d_model, n_h * d_c] with column block i = W^O_i W^UV_i."""
    d_model = w_o.shape[0]
    if w_ov is None:
        w_ov = torch.empty(d_model, params.n_h * params.d_c, dtype=w_o.dtype, device=w_o.device)
    workspace = _workspace(LIB.mla_fold_output_weights_workspace_size(ctypes.byref(params)),
                           "mla_fold_output_weights_workspace_size", w_o.device)
    code = LIB.mla_fold_output_weights(ctypes.byref(params), int(d_model), _ptr(w_o), _ptr(w_uv), _ptr(w_ov),
                                       _ptr(workspace), workspace.numel(), _stream())
    _check(code, "mla_fold_output_weights")
    return w_ov


def mla_gqla_expand_cache(params, w_uk_g, w_uv_g, c_kv, k_exp=None, v_exp=None):
    """Per-group expanded cache of GQLA's GQA path: k_exp [slots, n_g, d_h], v_exp [slots, n_g, d_v]."""
    n_g, d_h = w_uk_g.shape[0], w_uk_g.shape[1]
    slots = params.num_pages * params.page_size
    if k_exp is None:
        k_exp = torch.empty(slots, n_g, d_h, dtype=torch.bfloat16, device=c_kv.device)
    if v_exp is None:
        v_exp = torch.empty(slots, n_g, params.d_v, dtype=torch.bfloat16, device=c_kv.device)
    code = LIB.mla_gqla_expand_cache(ctypes.byref(params), int(n_g), int(d_h), _ptr(w_uk_g), _ptr(w_uv_g), _ptr(c_kv),
                                     _ptr(k_exp), _ptr(v_exp), _stream())
    _check(code, "mla_gqla_expand_cache")
    return k_exp, v_exp


def mla_gqla_decode(params, q_c, q_pe, k_exp, v_exp, k_pe, block_table, seq_lens, out=None, lse=None,
                    workspace=None):
    """GQA decode over the per-group expanded cache; returns (out [B, s_q, n_h, d_v], lse [B, s_q, n_h])."""
    B, s_q, n_h, d_h = q_c.shape
    n_g = k_exp.shape[1]
    if out is None:
        out = torch.empty(B, s_q, n_h, params.d_v, dtype=torch.bfloat16, device=q_c.device)
    if lse is None:
        lse = torch.empty(B, s_q, n_h, dtype=torch.float32, device=q_c.device)
    if workspace is None:
        workspace = _workspace(LIB.mla_gqla_decode_workspace_size(ctypes.byref(params), int(n_g), int(d_h)),
                               "mla_gqla_decode_workspace_size", q_c.device)
    code = LIB.mla_gqla_decode(ctypes.byref(params), int(n_g), int(d_h), _ptr(q_c), _ptr(q_pe), _ptr(k_exp),
                               _ptr(v_exp), _ptr(k_pe), _ptr(block_table), _ptr(seq_lens), _ptr(out), _ptr(lse),
                               _ptr(workspace), workspace.numel(), _stream())
    _check(code, "mla_gqla_decode")
    return out, lse


def mla_set_attention_events(start=None, stop=None):
    """Record torch.cuda.Event `start` / `stop` at the beginning and end of the partial-attention
    kernel of this thread's later mla_decode_fwd calls (None, None: plain launches)."""
    h = lambda e: ctypes.c_void_p(e.cuda_event) if e is not None else None
    _check(LIB.mla_set_attention_events(h(start), h(stop)), "mla_set_attention_events")


def workspace_views(params, workspace):
    """(split_table, partial_lse, partial_u) views of a workspace, per the header's layout."""
    G = mla_decode_num_splits(params)
    B, s_q, n_h, d_c = params.batch, params.s_q, params.n_h, params.d_c
    slots = G + B
    a256 = lambda x: (x + 255) // 256 * 256
    off_lse = a256(B * 2 * 4)
    off_u = off_lse + a256(slots * s_q * n_h * 4)
    table = workspace[: B * 8].view(torch.int32).view(B, 2)
    plse = workspace[off_lse: off_lse + slots * s_q * n_h * 4].view(torch.float32).view(slots, s_q, n_h)
    u_dtype = torch.float32 if params.q_dtype == F32 else torch.bfloat16   # the header's element type E
    u_size = torch.finfo(u_dtype).bits // 8
    pu = workspace[off_u: off_u + slots * s_q * n_h * d_c * u_size].view(u_dtype).view(slots, s_q, n_h, d_c)
    return table, plse, pu
