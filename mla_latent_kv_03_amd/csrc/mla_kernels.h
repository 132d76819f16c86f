// Internal interface between the host dispatch (mla_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

namespace mla {

// Arguments of the partial-attention kernels (one launch per decode call).
struct AttnParams {
  const void* q_nope;        // [B, s_q, n_h, d_c]
  const void* q_pe;          // [B, s_q, n_h, d_r]
  const void* c_kv;          // pool slot s at c_kv + s * c_stride (elements)
  const void* k_pe;          // pool slot s at k_pe + s * k_stride
  const float* kv_scale;     // per slot, fp8 caches only
  const int32_t* block_table;
  const int32_t* seq_lens;
  int64_t c_stride, k_stride;
  int32_t batch, s_q, n_h, d_c, d_r;
  int32_t page_size, num_pages, max_pages, max_tokens;
  int32_t num_splits;        // G
  int32_t rows_per_group;    // (q, head) rows per workgroup (MFMA path)
  int32_t packed_rows;       // 1: k_pe == c_kv + d_c with equal strides (one [c | k_pe] row per slot)
  float scale_log2;          // softmax_scale * log2(e)
  int32_t* split_table;      // [B][2]
  float* part_lse;           // [G + B][s_q][n_h]
  void* part_u;              // [G + B][s_q][n_h][d_c]: bf16 (bf16 / E4M3 caches) or float32 (fp32 path)
  // Fused append (128-head bf16 kernel only; new_c == null otherwise): the new rows
  // [B][s_new][d_c] / [B][s_new][d_r] (bf16) at positions [B][s_new] are written to the
  // pool by the workgroups of row group 0 (sequence b by share b % G) at the end of the
  // launch, and every tile that holds a new position gets that row from new_c / new_k.
  const void* new_c;
  const void* new_k;
  const int32_t* new_pos;
  int32_t s_new;             // 1 .. kMaxFusedNew
};
constexpr int kMaxFusedNew = 2;

// Arguments of the combine + up-projection kernels.
struct CombineParams {
  const int32_t* split_table;
  const float* part_lse;
  const void* part_u;        // bf16 for combine_upproj_bf16, float32 for the fp32 path
  const void* w_uv;          // [n_h, d_v, d_c]
  void* out;                 // [B, s_q, n_h, d_v]
  float* lse;                // [B, s_q, n_h] or null
  int32_t batch, s_q, n_h, d_c, d_v;
  int32_t num_slots;
};

struct AppendParams {
  const void* c_new;         // [B, s_new, d_c]
  const void* k_new;         // [B, s_new, d_r]
  const int32_t* positions;  // [B, s_new]
  const int32_t* block_table;
  void* c_kv;
  void* k_pe;
  float* kv_scale;
  int64_t c_stride, k_stride;
  int32_t batch, s_new, d_c, d_r;
  int32_t page_size, num_pages, max_pages;
  int32_t in_f32;            // 1: float32 input, 0: bf16 input
  int32_t mode;              // 0: copy bf16, 1: copy f32, 2: quantize to E4M3 + scale
};

// C = A B^T for the projections around the decode step (mla_proj.hip).  Element (m, k) of
// batch t of A is at a + t * a_bs + m * lda + k (B likewise); partial j of C at
// c + j * c_ks + t * c_bs + m * ldc + n.  K split into chunks of kchunk (a multiple of 32).
struct GemmArgs {
  const void* a;
  const void* b;
  const void* b2;            // bf16 product: rows n >= n_split of B are row n - n_split of b2 (or null)
  void* c;                   // float32 partials, or bf16 when out_bf16 (one chunk only)
  int64_t lda, ldb, ldc;
  int64_t a_bs, b_bs, c_bs, c_ks;
  int32_t M, N, K, kchunk, batch;
  int32_t n_split;           // with b2: a multiple of the rows of B one wave covers (32, float32 A 64)
  int32_t a_f32;             // bf16 operands: A is float32 (enters as bf16 high + remainder)
  int32_t out_bf16;
};

// Cache write finish: sums the partials [ksplit][T][d_c + d_r] of each new token's row,
// rotates its RoPE part and writes the pool slot.
struct CacheWriteArgs {
  const float* part;         // partial j of row t at part + j * part_ks + t * (d_c + d_r)
  int64_t part_ks;
  int32_t ksplit;
  int32_t d_c, d_r, s_new;
  const int32_t* positions;
  const int32_t* block_table;
  void* c_kv;
  void* k_pe;
  float* kv_scale;
  int64_t c_stride, k_stride;
  int32_t page_size, num_pages, max_pages;
  int32_t mode;              // 0: bf16 row, 1: float32 row, 2: E4M3 codes + scale
  float rope_base;
};

// Query prologue finish: q^C partials -> q_c (float32), q^R partials -> RoPE -> q_pe.
struct QueryArgs {
  const float* part_c;
  const float* part_r;
  int64_t part_c_ks, part_r_ks;
  int32_t ksplit, ksplit_r, n_h, d_h, d_r;
  const int32_t* positions;
  float* q_c;                // [T][n_h * d_h]
  void* q_pe;                // [T][n_h * d_r]
  int32_t out_bf16;
  float rope_base;
  // bf16 queries, query_absorb only: (W^UK_i)^T [n_h][d_c][d_h] and q~ out [T][n_h][d_c]
  const void* w_uk_t;
  void* q_nope;
  int32_t d_c;
};

// GQLA per-group decode (mla_gqla.hip): split partials [B][n_g][splits][32 rows][d_v] and
// lse, merged into out [B, s_q, n_h, d_v] (bf16) and lse [B, s_q, n_h].
struct GqaParams {
  const void* q_c;           // [B, s_q, n_h, d_h] bf16
  const void* q_pe;          // [B, s_q, n_h, d_r] bf16
  const void* k_exp;         // [slots, n_g, d_h] bf16
  const void* v_exp;         // [slots, n_g, d_v] bf16
  const void* k_pe;          // pool of RoPE keys, slot s at k_pe + s * k_pe_stride
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* part_o;
  float* part_lse;
  void* out;
  float* lse;
  int64_t k_pe_stride;
  int32_t batch, s_q, n_h, n_g, d_h, d_r, d_v;
  int32_t page_size, num_pages, max_pages, max_tokens, chunk, splits;
  float scale_log2;
};
hipError_t launch_gqa_decode(const GqaParams& p, hipStream_t s);

hipError_t launch_gemm_nt(const GemmArgs& g, bool bf16_operands, int ksplit, hipStream_t s);
// Geometry of the bf16 product kernel, shared with the host-side K-split choice: blocks of
// 32 rows of A per row tile (1 or 2), and of 32 rows of B per wave (float32 A: 2).
inline int gemm_row_blocks(int M) { return M > 32 ? 2 : 1; }
inline int gemm_col_blocks(bool a_f32) { return a_f32 ? 2 : 1; }
hipError_t launch_cache_write_finish(const CacheWriteArgs& a, int tokens, hipStream_t s);
hipError_t launch_query_finish(const QueryArgs& a, int tokens, hipStream_t s);
// bf16 queries: q~_i = (W^UK_i)^T q^C_i straight from the K-split partials of q^C, and the
// q^R finish, in one launch (d_h a multiple of 32, at most 256).
hipError_t launch_query_absorb(const QueryArgs& a, int tokens, hipStream_t s);
hipError_t launch_sum_partials(const float* part, int64_t part_ks, int ksplit, int64_t n, void* out, bool out_bf16,
                               hipStream_t s);
hipError_t launch_transpose_heads(const void* src, void* dst, int heads, int rows, int cols, bool bf16_elems,
                                  hipStream_t s);

// Heads of one query position handled by one workgroup of the bf16 kernel.
int attn_heads_per_group(int n_h);
// Start/stop events for the partial-attention kernel of the calling thread's next
// launches (null: a plain launch).  Set through mla_set_attention_events; used only to
// time the kernel itself, excluding the dispatch gap a stream event would include.
struct AttentionEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
AttentionEvents& attention_events();

template <class Kernel, class... Args>
hipError_t launch_attention_kernel(Kernel kernel, dim3 grid, dim3 block, hipStream_t stream, Args... args) {
  const AttentionEvents& ev = attention_events();
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, ev.start, ev.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
  return hipGetLastError();
}

hipError_t launch_attn_mfma(const AttnParams& p, bool fp8, hipStream_t stream);
hipError_t launch_attn_h128(const AttnParams& p, bool fp8, hipStream_t stream);
hipError_t launch_attn_fp8_v0(const AttnParams& p, hipStream_t stream);
hipError_t launch_attn_f32(const AttnParams& p, hipStream_t stream);
hipError_t launch_combine_bf16(const CombineParams& p, hipStream_t stream);
hipError_t launch_combine_f32(const CombineParams& p, hipStream_t stream);
hipError_t launch_append(const AppendParams& p, hipStream_t stream);

}  // namespace mla
