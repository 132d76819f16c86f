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
