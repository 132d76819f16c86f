// Host side of the projection entry points of include/mla_decode.h (the steps adjacent to
// the decode: cache write, query prologue, output projection and its weight fold):
// validation, K-split choice, workspace layout and launches on the caller's stream.
// Like the decode entry points: no allocation, no synchronization, no device access
// during validation.

#include <hip/hip_runtime.h>

#include <climits>

#include "mla_decode.h"
#include "mla_kernels.h"

namespace {

size_t a256(size_t x) { return (x + 255) & ~size_t(255); }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
mla_status_t status_of(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }
int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }
// The bf16 product kernel addresses an activation operand through 32-bit offsets.
bool act_fits(long long rows, long long width, int elem_bytes) { return rows * width * elem_bytes < (1LL << 31); }

// K split of C[M, N] = A[M, K] B[N, K]^T.  bf16 weights: at most four waves of the
// weight-streaming kernel per compute unit (1024 waves, each a block of 32 or 64 rows of B
// times a row tile of A, one workgroup per CU), with chunks of at least 256 (multiples of
// 64 where K is, else of 16); float32 operands use one chunk.
struct Split {
  int ksplit, kchunk;
};
Split split_of(long long M, long long N, int K, bool bf16, bool a_f32 = false) {
  if (!bf16) return {1, K};
  const int rows = 32 * mla::gemm_row_blocks(M > INT_MAX ? INT_MAX : (int)M);
  const long long waves = (long long)cdiv(N, 32 * mla::gemm_col_blocks(a_f32)) * cdiv(M, rows);
  // Rounded down: a grid of a few more workgroups than CUs puts two on some CUs, which
  // then stream twice the weights (W^O at 64 rows: K split 5, 280 workgroups, 59.7 us;
  // K split 4, 224 workgroups, 47.8 us).
  long long ks = 1024 / waves;
  const long long max_ks = K / 256 > 0 ? K / 256 : 1;
  if (ks > max_ks) ks = max_ks;
  if (ks < 1) ks = 1;
  // Chunks of whole 64-wide blocks where K allows (the product kernel's fast path).
  const int align = K % 64 == 0 ? 64 : 16;
  const int kchunk = cdiv(cdiv(K, ks), align) * align;
  return {cdiv(K, kchunk), kchunk};
}

mla::GemmArgs gemm(const void* a, int64_t lda, const void* b, int64_t ldb, void* c, int64_t ldc, int M, int N, int K,
                   const Split& sp, int64_t c_ks) {
  mla::GemmArgs g{};
  g.a = a;
  g.b = b;
  g.b2 = nullptr;
  g.c = c;
  g.lda = lda;
  g.ldb = ldb;
  g.ldc = ldc;
  g.a_bs = g.b_bs = g.c_bs = 0;
  g.c_ks = c_ks;
  g.M = M;
  g.N = N;
  g.K = K;
  g.kchunk = sp.kchunk;
  g.batch = 1;
  g.n_split = N;
  g.a_f32 = 0;
  g.out_bf16 = 0;
  return g;
}

bool is_in_dtype(mla_dtype_t t) { return t == MLA_DTYPE_BF16 || t == MLA_DTYPE_F32; }

// ---------------------------------------------------------------- cache write

struct CacheWriteLayout {
  Split sp;
  size_t bytes;         // K-split partials [ksplit][T][d_c + d_r]
};

mla_status_t check_cache_write(const mla_decode_params_t* p, int32_t d_model, int32_t s_new, CacheWriteLayout& l) {
  if (!p) return MLA_ERR_NULL;
  if (p->batch < 1 || s_new < 1 || d_model < 1 || p->d_c < 1 || p->d_r < 0) return MLA_ERR_SHAPE;
  if (p->d_c % 2 || p->d_r % 2 || p->d_c + p->d_r > 1280) return MLA_ERR_SHAPE;
  if ((long long)p->batch * s_new > INT_MAX / 2) return MLA_ERR_SHAPE;
  if (p->page_size < 64 || p->page_size % 64 || p->num_pages < 1 || p->max_pages_per_seq < 1) return MLA_ERR_SHAPE;
  if (p->c_kv_stride < p->d_c || p->k_pe_stride < p->d_r) return MLA_ERR_SHAPE;
  if (!is_in_dtype(p->q_dtype)) return MLA_ERR_DTYPE;
  const bool bf16 = p->q_dtype == MLA_DTYPE_BF16;
  if (p->kv_dtype == MLA_DTYPE_BF16 && !bf16) return MLA_ERR_DTYPE;
  if (p->kv_dtype == MLA_DTYPE_F32 && bf16) return MLA_ERR_DTYPE;
  if (bf16 && (d_model % 32 || p->d_c % 16 || p->d_r % 16)) return MLA_ERR_SHAPE;
  const long long T = (long long)p->batch * s_new;
  if (bf16 && !act_fits(T, d_model, 2)) return MLA_ERR_SHAPE;
  l.sp = split_of(T, p->d_c + p->d_r, d_model, bf16);
  l.bytes = a256((size_t)l.sp.ksplit * T * (p->d_c + p->d_r) * sizeof(float));
  return MLA_OK;
}

// ---------------------------------------------------------------- query prologue

struct QueryLayout {
  Split sc, sr;
  size_t part_c, part_r, q_c, bytes;
};

mla_status_t check_query(const mla_decode_params_t* p, int32_t d_model, int32_t d_h, QueryLayout& l) {
  if (!p) return MLA_ERR_NULL;
  if (p->batch < 1 || p->s_q < 1 || p->n_h < 1 || p->d_c < 1 || p->d_r < 0 || d_model < 1 || d_h < 1)
    return MLA_ERR_SHAPE;
  if (p->d_r % 2) return MLA_ERR_SHAPE;
  if ((long long)p->batch * p->s_q > INT_MAX / 2 || (long long)p->n_h * (d_h + p->d_r + p->d_c) > INT_MAX / 2)
    return MLA_ERR_SHAPE;
  if (!is_in_dtype(p->q_dtype)) return MLA_ERR_DTYPE;
  const bool bf16 = p->q_dtype == MLA_DTYPE_BF16;
  if (bf16 && (d_model % 32 || d_h % 32 || p->d_c % 16 || (p->n_h * p->d_r) % 16 || (p->n_h * d_h) % 16))
    return MLA_ERR_SHAPE;
  const long long T = (long long)p->batch * p->s_q;
  if (bf16 && (!act_fits(T, d_model, 2) || !act_fits(T * p->n_h, d_h, 4))) return MLA_ERR_SHAPE;
  l.sc = split_of(T, (long long)p->n_h * d_h, d_model, bf16);
  l.sr = split_of(T, (long long)p->n_h * p->d_r, d_model, bf16);
  l.part_c = 0;
  l.part_r = a256((size_t)l.sc.ksplit * T * p->n_h * d_h * sizeof(float));
  l.q_c = l.part_r + a256((size_t)l.sr.ksplit * T * p->n_h * p->d_r * sizeof(float));
  l.bytes = l.q_c + a256((size_t)T * p->n_h * d_h * sizeof(float));
  return MLA_OK;
}

// ---------------------------------------------------------------- output projection

mla_status_t check_output(const mla_decode_params_t* p, int32_t d_model, int32_t width, mla_dtype_t x_dtype,
                          Split& sp, size_t& bytes) {
  if (!p) return MLA_ERR_NULL;
  if (p->batch < 1 || p->s_q < 1 || d_model < 1 || width < 1) return MLA_ERR_SHAPE;
  if ((long long)p->batch * p->s_q > INT_MAX / 2) return MLA_ERR_SHAPE;
  if (!is_in_dtype(p->w_dtype) || !is_in_dtype(x_dtype) || !is_in_dtype(p->out_dtype)) return MLA_ERR_DTYPE;
  const bool bf16 = p->w_dtype == MLA_DTYPE_BF16;
  if (!bf16 && x_dtype != MLA_DTYPE_F32) return MLA_ERR_DTYPE;
  if (bf16 && (width % 32 || d_model % 16)) return MLA_ERR_SHAPE;
  const long long M = (long long)p->batch * p->s_q;
  if (bf16 && !act_fits(M, width, x_dtype == MLA_DTYPE_F32 ? 4 : 2)) return MLA_ERR_SHAPE;
  sp = split_of(M, d_model, width, bf16, x_dtype == MLA_DTYPE_F32);
  bytes = a256((size_t)sp.ksplit * M * d_model * sizeof(float));
  return MLA_OK;
}

}  // namespace

extern "C" {

size_t mla_cache_write_workspace_size(const mla_decode_params_t* params, int32_t d_model, int32_t s_new) {
  CacheWriteLayout l;
  return check_cache_write(params, d_model, s_new, l) == MLA_OK ? l.bytes : 0;
}

mla_status_t mla_cache_write(const mla_decode_params_t* params, int32_t d_model, int32_t s_new, const void* h,
                             const void* w_dkv, const void* w_kr, const int32_t* positions, float rope_base,
                             const int32_t* block_table, void* c_kv, void* k_pe, float* kv_scale, void* workspace,
                             size_t workspace_bytes, void* stream) {
  CacheWriteLayout l;
  mla_status_t st = check_cache_write(params, d_model, s_new, l);
  if (st != MLA_OK) return st;
  const mla_decode_params_t& p = *params;
  const bool bf16 = p.q_dtype == MLA_DTYPE_BF16;
  int mode;
  if (p.kv_dtype == MLA_DTYPE_BF16) mode = 0;
  else if (p.kv_dtype == MLA_DTYPE_F32) mode = 1;
  else if (p.kv_dtype == MLA_DTYPE_FP8_E4M3) mode = 2;
  else return MLA_ERR_DTYPE;
  if (!h || !w_dkv || !positions || !block_table || !c_kv) return MLA_ERR_NULL;
  if (p.d_r > 0 && (!w_kr || !k_pe)) return MLA_ERR_NULL;
  if ((mode == 2) != (kv_scale != nullptr)) return mode == 2 ? MLA_ERR_NULL : MLA_ERR_DTYPE;
  if (!(rope_base > 1.f) || rope_base == INFINITY) return MLA_ERR_SHAPE;
  if (bf16 && (!aligned16(h) || !aligned16(w_dkv) || (p.d_r > 0 && !aligned16(w_kr)))) return MLA_ERR_SHAPE;
  if (!workspace || workspace_bytes < l.bytes || !aligned16(workspace)) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int T = p.batch * s_new, D = p.d_c + p.d_r;
  float* part = (float*)workspace;
  const int64_t part_ks = (int64_t)T * D;
  if (bf16 && p.d_r > 0 && p.d_c % 32 == 0) {
    // One product over [W^DKV; W^KR]: the rows past d_c come from w_kr.
    mla::GemmArgs g = gemm(h, d_model, w_dkv, d_model, part, D, T, D, d_model, l.sp, part_ks);
    g.b2 = w_kr;
    g.n_split = p.d_c;
    st = status_of(mla::launch_gemm_nt(g, bf16, l.sp.ksplit, s));
    if (st != MLA_OK) return st;
  } else {
    mla::GemmArgs g = gemm(h, d_model, w_dkv, d_model, part, D, T, p.d_c, d_model, l.sp, part_ks);
    st = status_of(mla::launch_gemm_nt(g, bf16, l.sp.ksplit, s));
    if (st != MLA_OK) return st;
    if (p.d_r > 0) {
      g = gemm(h, d_model, w_kr, d_model, part + p.d_c, D, T, p.d_r, d_model, l.sp, part_ks);
      st = status_of(mla::launch_gemm_nt(g, bf16, l.sp.ksplit, s));
      if (st != MLA_OK) return st;
    }
  }
  mla::CacheWriteArgs a;
  a.part = part;
  a.part_ks = part_ks;
  a.ksplit = l.sp.ksplit;
  a.d_c = p.d_c;
  a.d_r = p.d_r;
  a.s_new = s_new;
  a.positions = positions;
  a.block_table = block_table;
  a.c_kv = c_kv;
  a.k_pe = k_pe ? k_pe : c_kv;
  a.kv_scale = kv_scale;
  a.c_stride = p.c_kv_stride;
  a.k_stride = p.k_pe_stride;
  a.page_size = p.page_size;
  a.num_pages = p.num_pages;
  a.max_pages = p.max_pages_per_seq;
  a.mode = mode;
  a.rope_base = rope_base;
  return status_of(mla::launch_cache_write_finish(a, T, s));
}

size_t mla_query_prologue_workspace_size(const mla_decode_params_t* params, int32_t d_model, int32_t d_h) {
  QueryLayout l;
  return check_query(params, d_model, d_h, l) == MLA_OK ? l.bytes : 0;
}

mla_status_t mla_query_prologue(const mla_decode_params_t* params, int32_t d_model, int32_t d_h, const void* h,
                                const void* w_q, const void* w_uk_t, const void* w_qr, const int32_t* positions,
                                float rope_base, void* q_nope, void* q_pe, void* workspace, size_t workspace_bytes,
                                void* stream) {
  QueryLayout l;
  mla_status_t st = check_query(params, d_model, d_h, l);
  if (st != MLA_OK) return st;
  const mla_decode_params_t& p = *params;
  const bool bf16 = p.q_dtype == MLA_DTYPE_BF16;
  if (!h || !w_q || !w_uk_t || !positions || !q_nope) return MLA_ERR_NULL;
  if (p.d_r > 0 && (!w_qr || !q_pe)) return MLA_ERR_NULL;
  if (!(rope_base > 1.f) || rope_base == INFINITY) return MLA_ERR_SHAPE;
  if (bf16 && (!aligned16(h) || !aligned16(w_q) || !aligned16(w_uk_t) || (p.d_r > 0 && !aligned16(w_qr))))
    return MLA_ERR_SHAPE;
  if (!workspace || workspace_bytes < l.bytes || !aligned16(workspace)) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int T = p.batch * p.s_q;
  const int nc = p.n_h * d_h, nr = p.n_h * p.d_r;
  char* ws = (char*)workspace;
  float* part_c = (float*)(ws + l.part_c);
  float* part_r = (float*)(ws + l.part_r);
  float* q_c = (float*)(ws + l.q_c);
  // q^C = W^Q h and q^R_raw = W^QR h (K-split partials).
  mla::GemmArgs g = gemm(h, d_model, w_q, d_model, part_c, nc, T, nc, d_model, l.sc, (int64_t)T * nc);
  st = status_of(mla::launch_gemm_nt(g, bf16, l.sc.ksplit, s));
  if (st != MLA_OK) return st;
  if (p.d_r > 0) {
    g = gemm(h, d_model, w_qr, d_model, part_r, nr, T, nr, d_model, l.sr, (int64_t)T * nr);
    st = status_of(mla::launch_gemm_nt(g, bf16, l.sr.ksplit, s));
    if (st != MLA_OK) return st;
  }
  // Sum the partials; q^C to float32 scratch (or, bf16 queries, straight into the absorption
  // product), q^R rotated to q_pe.
  mla::QueryArgs qa;
  qa.part_c = part_c;
  qa.part_r = part_r;
  qa.part_c_ks = (int64_t)T * nc;
  qa.part_r_ks = (int64_t)T * nr;
  qa.ksplit = l.sc.ksplit;
  qa.ksplit_r = l.sr.ksplit;
  qa.n_h = p.n_h;
  qa.d_h = d_h;
  qa.d_r = p.d_r;
  qa.positions = positions;
  qa.q_c = q_c;
  qa.q_pe = q_pe;
  qa.out_bf16 = bf16 ? 1 : 0;
  qa.rope_base = rope_base;
  qa.w_uk_t = w_uk_t;
  qa.q_nope = q_nope;
  qa.d_c = p.d_c;
  if (bf16 && d_h <= 256) {
    // q~ from the partials of q^C directly, and q^R, in one launch.
    return status_of(mla::launch_query_absorb(qa, T, s));
  }
  st = status_of(mla::launch_query_finish(qa, T, s));
  if (st != MLA_OK) return st;
  // q~_i = (W^UK_i)^T q^C_i: per head, C[T, d_c] = q^C_i[T, d_h] ((W^UK_i)^T)^T, written
  // straight to q_nope [T][n_h][d_c].
  Split one{1, d_h};
  g = gemm(q_c, nc, w_uk_t, d_h, q_nope, (int64_t)p.n_h * p.d_c, T, p.d_c, d_h, one, 0);
  g.batch = p.n_h;
  g.a_bs = d_h;
  g.b_bs = (int64_t)p.d_c * d_h;
  g.c_bs = p.d_c;
  g.a_f32 = 1;
  g.out_bf16 = bf16 ? 1 : 0;
  return status_of(mla::launch_gemm_nt(g, bf16, 1, s));
}

size_t mla_output_projection_workspace_size(const mla_decode_params_t* params, int32_t d_model, int32_t width,
                                            mla_dtype_t x_dtype) {
  Split sp;
  size_t bytes = 0;
  return check_output(params, d_model, width, x_dtype, sp, bytes) == MLA_OK ? bytes : 0;
}

mla_status_t mla_output_projection(const mla_decode_params_t* params, int32_t d_model, int32_t width,
                                   mla_dtype_t x_dtype, const void* x, const void* w, void* y, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  Split sp;
  size_t bytes = 0;
  mla_status_t st = check_output(params, d_model, width, x_dtype, sp, bytes);
  if (st != MLA_OK) return st;
  const mla_decode_params_t& p = *params;
  const bool bf16 = p.w_dtype == MLA_DTYPE_BF16;
  if (!x || !w || !y) return MLA_ERR_NULL;
  if (bf16 && (!aligned16(x) || !aligned16(w))) return MLA_ERR_SHAPE;
  if (!workspace || workspace_bytes < bytes || !aligned16(workspace)) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int M = p.batch * p.s_q;
  float* part = (float*)workspace;
  mla::GemmArgs g = gemm(x, width, w, width, part, d_model, M, d_model, width, sp, (int64_t)M * d_model);
  g.a_f32 = x_dtype == MLA_DTYPE_F32 ? 1 : 0;
  st = status_of(mla::launch_gemm_nt(g, bf16, sp.ksplit, s));
  if (st != MLA_OK) return st;
  return status_of(mla::launch_sum_partials(part, (int64_t)M * d_model, sp.ksplit, (int64_t)M * d_model, y,
                                            p.out_dtype == MLA_DTYPE_BF16, s));
}

size_t mla_fold_output_weights_workspace_size(const mla_decode_params_t* params) {
  if (!params || params->n_h < 1 || params->d_v < 1 || params->d_c < 1) return 0;
  if (!is_in_dtype(params->w_dtype)) return 0;
  const size_t elem = params->w_dtype == MLA_DTYPE_BF16 ? 2 : 4;
  return a256((size_t)params->n_h * params->d_v * params->d_c * elem);
}

mla_status_t mla_fold_output_weights(const mla_decode_params_t* params, int32_t d_model, const void* w_o,
                                     const void* w_uv, void* w_ov, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  if (!params) return MLA_ERR_NULL;
  const mla_decode_params_t& p = *params;
  if (p.n_h < 1 || p.d_v < 1 || p.d_c < 1 || d_model < 1) return MLA_ERR_SHAPE;
  if ((long long)p.n_h * (p.d_v + p.d_c) > INT_MAX / 2) return MLA_ERR_SHAPE;
  if (!is_in_dtype(p.w_dtype)) return MLA_ERR_DTYPE;
  const bool bf16 = p.w_dtype == MLA_DTYPE_BF16;
  if (bf16 && (p.d_v % 32 || p.d_c % 16)) return MLA_ERR_SHAPE;
  if (!w_o || !w_uv || !w_ov) return MLA_ERR_NULL;
  if (bf16 && (!aligned16(w_o) || !aligned16(w_uv))) return MLA_ERR_SHAPE;
  const size_t need = mla_fold_output_weights_workspace_size(params);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return MLA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  // (W^UV_i)^T per head, so that the contraction index v is contiguous in both operands.
  mla_status_t st = status_of(mla::launch_transpose_heads(w_uv, workspace, p.n_h, p.d_v, p.d_c, bf16, s));
  if (st != MLA_OK) return st;
  // Column block i of W^OV: C[d_model, d_c] = W^O_i[d_model, d_v] ((W^UV_i)^T)^T.
  Split one{1, p.d_v};
  mla::GemmArgs g = gemm(w_o, (int64_t)p.n_h * p.d_v, workspace, p.d_v, w_ov, (int64_t)p.n_h * p.d_c, d_model, p.d_c,
                         p.d_v, one, 0);
  g.batch = p.n_h;
  g.a_bs = p.d_v;
  g.b_bs = (int64_t)p.d_c * p.d_v;
  g.c_bs = p.d_c;
  g.out_bf16 = bf16 ? 1 : 0;
  return status_of(mla::launch_gemm_nt(g, bf16, 1, s));
}

}  // extern "C"

// ---------------------------------------------------------------- GQLA per-group path

namespace {

mla_status_t check_gqla(const mla_decode_params_t* p, int32_t n_g, int32_t d_h) {
  if (!p) return MLA_ERR_NULL;
  if (p->batch < 1 || p->s_q < 1 || p->n_h < 1 || n_g < 1 || d_h < 1 || p->d_r < 0 || p->d_c < 1 || p->d_v < 1)
    return MLA_ERR_SHAPE;
  if (p->n_h % n_g || (p->n_h / n_g) * p->s_q > 32) return MLA_ERR_SHAPE;
  if (p->q_dtype != MLA_DTYPE_BF16 || p->kv_dtype != MLA_DTYPE_BF16 || p->w_dtype != MLA_DTYPE_BF16 ||
      p->out_dtype != MLA_DTYPE_BF16)
    return MLA_ERR_DTYPE;
  const int kd = d_h + p->d_r;
  if (!((kd == 192 && p->d_v == 128) || (kd == 32 && p->d_v == 32) || (kd == 64 && p->d_v == 64)))
    return MLA_ERR_SHAPE;
  if (d_h % 8 || p->d_r % 8 || p->d_c % 32) return MLA_ERR_SHAPE;
  if (p->page_size < 64 || p->page_size % 64 || p->num_pages < 1 || p->max_pages_per_seq < 1) return MLA_ERR_SHAPE;
  if ((long long)p->max_pages_per_seq * p->page_size > INT_MAX) return MLA_ERR_SHAPE;
  if (p->c_kv_stride < p->d_c || p->k_pe_stride < p->d_r || p->c_kv_stride % 8 || p->k_pe_stride % 8)
    return MLA_ERR_SHAPE;
  if (!(p->softmax_scale > 0.f) || p->softmax_scale == INFINITY) return MLA_ERR_SHAPE;
  return MLA_OK;
}

// Token splits per sequence: enough (sequence, group, split) waves to fill the device
// (>= 1024), chunks of at least 256 tokens, a multiple of 32.
void gqla_splits(const mla_decode_params_t& p, int32_t n_g, int& splits, int& chunk) {
  const long long max_tokens = (long long)p.max_pages_per_seq * p.page_size;
  long long want = (1024 + (long long)p.batch * n_g - 1) / ((long long)p.batch * n_g);
  const long long most = (max_tokens + 255) / 256;
  if (want > most) want = most;
  if (want < 1) want = 1;
  chunk = (int)(((max_tokens + want - 1) / want + 31) / 32 * 32);
  splits = (int)((max_tokens + chunk - 1) / chunk);
}

}  // namespace

extern "C" {

mla_status_t mla_gqla_expand_cache(const mla_decode_params_t* params, int32_t n_g, int32_t d_h, const void* w_uk_g,
                                   const void* w_uv_g, const void* c_kv, void* k_exp, void* v_exp, void* stream) {
  mla_status_t st = check_gqla(params, n_g, d_h);
  if (st != MLA_OK) return st;
  const mla_decode_params_t& p = *params;
  if (!w_uk_g || !w_uv_g || !c_kv || !k_exp || !v_exp) return MLA_ERR_NULL;
  if (!aligned16(w_uk_g) || !aligned16(w_uv_g) || !aligned16(c_kv)) return MLA_ERR_SHAPE;
  if ((long long)p.num_pages * p.page_size > INT_MAX) return MLA_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  const int slots = p.num_pages * p.page_size;
  // k_exp[slot][g][:] = W^UK_g c_slot and v_exp[slot][g][:] = W^UV_g c_slot: C[slots, n_g * d] =
  // c[slots, d_c] W^T with W = [n_g * d, d_c] (the stacked group matrices).
  Split one{1, p.d_c};
  mla::GemmArgs g = gemm(c_kv, p.c_kv_stride, w_uk_g, p.d_c, k_exp, (int64_t)n_g * d_h, slots, n_g * d_h, p.d_c, one, 0);
  g.out_bf16 = 1;
  st = status_of(mla::launch_gemm_nt(g, true, 1, s));
  if (st != MLA_OK) return st;
  g = gemm(c_kv, p.c_kv_stride, w_uv_g, p.d_c, v_exp, (int64_t)n_g * p.d_v, slots, n_g * p.d_v, p.d_c, one, 0);
  g.out_bf16 = 1;
  return status_of(mla::launch_gemm_nt(g, true, 1, s));
}

size_t mla_gqla_decode_workspace_size(const mla_decode_params_t* params, int32_t n_g, int32_t d_h) {
  if (check_gqla(params, n_g, d_h) != MLA_OK) return 0;
  int splits, chunk;
  gqla_splits(*params, n_g, splits, chunk);
  const size_t rows = (size_t)params->batch * n_g * splits * 32;
  return a256(rows * params->d_v * sizeof(float)) + a256(rows * sizeof(float));
}

mla_status_t mla_gqla_decode(const mla_decode_params_t* params, int32_t n_g, int32_t d_h, const void* q_c,
                             const void* q_pe, const void* k_exp, const void* v_exp, const void* k_pe,
                             const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream) {
  mla_status_t st = check_gqla(params, n_g, d_h);
  if (st != MLA_OK) return st;
  const mla_decode_params_t& p = *params;
  if (!q_c || !k_exp || !v_exp || !block_table || !seq_lens || !out) return MLA_ERR_NULL;
  if (p.d_r > 0 && (!q_pe || !k_pe)) return MLA_ERR_NULL;
  if (!aligned16(q_c) || !aligned16(k_exp) || !aligned16(v_exp) || (p.d_r > 0 && (!aligned16(q_pe) || !aligned16(k_pe))))
    return MLA_ERR_SHAPE;
  const size_t need = mla_gqla_decode_workspace_size(params, n_g, d_h);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return MLA_ERR_WORKSPACE;
  mla::GqaParams g;
  gqla_splits(p, n_g, g.splits, g.chunk);
  const size_t rows = (size_t)p.batch * n_g * g.splits * 32;
  g.q_c = q_c;
  g.q_pe = q_pe ? q_pe : q_c;
  g.k_exp = k_exp;
  g.v_exp = v_exp;
  g.k_pe = k_pe ? k_pe : k_exp;
  g.block_table = block_table;
  g.seq_lens = seq_lens;
  g.part_o = (float*)workspace;
  g.part_lse = (float*)((char*)workspace + a256(rows * p.d_v * sizeof(float)));
  g.out = out;
  g.lse = lse;
  g.k_pe_stride = p.k_pe_stride;
  g.batch = p.batch;
  g.s_q = p.s_q;
  g.n_h = p.n_h;
  g.n_g = n_g;
  g.d_h = d_h;
  g.d_r = p.d_r;
  g.d_v = p.d_v;
  g.page_size = p.page_size;
  g.num_pages = p.num_pages;
  g.max_pages = p.max_pages_per_seq;
  g.max_tokens = p.max_pages_per_seq * p.page_size;
  g.scale_log2 = p.softmax_scale * 1.4426950408889634f;
  return status_of(mla::launch_gqa_decode(g, (hipStream_t)stream));
}

}  // extern "C"
