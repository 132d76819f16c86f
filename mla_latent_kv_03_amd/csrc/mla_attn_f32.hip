// Partial attention of absorbed MLA decode for float32 caches and queries of any
// (small) width.  Same mathematics and split rule as the MFMA kernel:
//   s_j = softmax_scale * (q_nope . c_j + q_pe . k_pe_j),  lse = ln sum_j exp(s_j),
//   u = sum_j exp(s_j - lse) c_j   over one piece's visible tokens,
// with fp32 arithmetic throughout (products and sums in float32 FMA).
// One workgroup per (share, query row); 256 tokens per step.

#include "mla_device.h"
#include "mla_kernels.h"
#include "mla_split.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxDc = 1024;
constexpr int kMaxDr = 256;
constexpr int kColsPerThread = kMaxDc / kThreads;

struct SmemF32 {
  float q[kMaxDc + kMaxDr];
  float prob[kThreads];
  long long slot_of[kThreads];
  float red[kThreads / 64];
  SplitScratch split;
  Piece pieces[kThreads];
};

__device__ float block_reduce(float v, float* red, bool is_max) {
  v = is_max ? wave_max(v) : wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kThreads / 64; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThreads) void attn_partial_f32(const AttnParams p) {
  __shared__ SmemF32 sm;
  const int w = blockIdx.x;
  const int row = blockIdx.y;               // (q, head) row
  const int q_pos = row / p.n_h;
  const int head = row - q_pos * p.n_h;
  const int tid = threadIdx.x;
  const float* cpool = (const float*)p.c_kv;
  const float* kpool = (const float*)p.k_pe;

  for_each_piece(p.seq_lens, p.batch, p.max_tokens, p.num_splits, w, row == 0 ? p.split_table : nullptr,
                 &sm.split, sm.pieces, [&](const Piece& pc) {
    const int b = pc.b;
    const int L = clamp_len(p.seq_lens[b], p.max_tokens);
    const int end = min(pc.t1, max(0, L - p.s_q + q_pos + 1));
    const size_t qrow = ((size_t)b * p.s_q + q_pos) * p.n_h + head;
    for (int k = tid; k < p.d_c; k += kThreads) sm.q[k] = ((const float*)p.q_nope)[qrow * p.d_c + k];
    for (int k = tid; k < p.d_r; k += kThreads) sm.q[p.d_c + k] = ((const float*)p.q_pe)[qrow * p.d_r + k];
    __syncthreads();

    float m_run = -INFINITY, l_run = 0.f;
    float u[kColsPerThread];
#pragma unroll
    for (int i = 0; i < kColsPerThread; ++i) u[i] = 0.f;

    for (int t = pc.t0; t < end; t += kThreads) {
      const int j = t + tid;
      float s = -INFINITY;
      long long slot = -1;
      if (j < end) {
        const int page = p.block_table[(size_t)b * p.max_pages + j / p.page_size];
        if (page >= 0 && page < p.num_pages) {
          slot = (long long)page * p.page_size + j % p.page_size;
          const float* crow = cpool + slot * p.c_stride;
          const float* krow = kpool + slot * p.k_stride;
          float acc = 0.f;
          for (int k = 0; k < p.d_c; ++k) acc = fmaf(sm.q[k], crow[k], acc);
          for (int k = 0; k < p.d_r; ++k) acc = fmaf(sm.q[p.d_c + k], krow[k], acc);
          s = acc * p.scale_log2;
        }
      }
      const float mx = block_reduce(s, sm.red, true);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      const float pr = exp2f(s - m_use);
      sm.prob[tid] = pr;
      sm.slot_of[tid] = slot;
      const float psum = block_reduce(pr, sm.red, false);
      l_run = l_run * alpha + psum;
      m_run = m_new;
      const int n = min(kThreads, end - t);
#pragma unroll
      for (int i = 0; i < kColsPerThread; ++i) {
        const int k = tid + i * kThreads;
        if (k < p.d_c) {
          float acc = u[i] * alpha;
          for (int jj = 0; jj < n; ++jj) {
            const long long sj = sm.slot_of[jj];
            if (sj >= 0) acc = fmaf(sm.prob[jj], cpool[sj * p.c_stride + k], acc);
          }
          u[i] = acc;
        }
      }
      __syncthreads();
    }
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const size_t orow = ((size_t)pc.slot * p.s_q + q_pos) * p.n_h + head;
    if (tid == 0) p.part_lse[orow] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
#pragma unroll
    for (int i = 0; i < kColsPerThread; ++i) {
      const int k = tid + i * kThreads;
      if (k < p.d_c) ((float*)p.part_u)[orow * p.d_c + k] = u[i] * inv;
    }
    __syncthreads();
  });
}

}  // namespace

hipError_t launch_attn_f32(const AttnParams& p, hipStream_t stream) {
  dim3 grid(p.num_splits, p.s_q * p.n_h);
  return launch_attention_kernel(attn_partial_f32, grid, dim3(kThreads), stream, p);
}

}  // namespace mla
