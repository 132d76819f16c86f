// Log-sum-exp combine of split partials and the per-head up-projection.
//
// For every row (b, q) and head i, over the sequence's slots s (split table):
//   lse = ln sum_s exp(lse_s)              (largest finite lse_s subtracted first)
//   u   = sum_s exp(lse_s - lse) u_s       (softmax over a union of disjoint token sets)
//   o_i = W^UV_i u                         (page "MLA deep compression", output-side
//                                           absorption: u_i is formed in latent space,
//                                           then up-projected once)
// bf16 weights: one workgroup per (head, 64 rows); each wave forms u for 16 rows
// directly in MFMA operand layout (as a bf16 high part plus a bf16 remainder, so the
// latent enters the product with ~16 significant bits) and multiplies by W^UV_i^T
// with 16x16x32 MFMAs.  float32 weights: plain FMA loops.

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

__device__ __forceinline__ void slot_range(const CombineParams& p, int b, int& first, int& count) {
  first = p.split_table[2 * b];
  count = p.split_table[2 * b + 1];
  if (first < 0 || first >= p.num_slots || count <= 0) { first = 0; count = 0; return; }
  if (count > p.num_slots - first) count = p.num_slots - first;
}

constexpr int kDc = 512;
constexpr int kDv = 128;
constexpr int kRowsPerWg = 64;

__global__ __launch_bounds__(256) void combine_upproj_bf16(const CombineParams p) {
  const int head = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int R = p.batch * p.s_q;
  const int r = blockIdx.y * kRowsPerWg + wave * 16 + l16;   // row of this lane's A operand
  const bool valid = r < R;

  bf16x8 a_hi[kDc / 32], a_lo[kDc / 32];
  float lse_row = -INFINITY;
  {
    int first = 0, count = 0;
    const int b = valid ? r / p.s_q : 0;
    const int q = valid ? r - b * p.s_q : 0;
    if (valid) slot_range(p, b, first, count);
    float mx = -INFINITY;
    for (int s = 0; s < count; ++s)
      mx = fmaxf(mx, p.part_lse[((size_t)(first + s) * p.s_q + q) * p.n_h + head]);
    float tot = 0.f;
    for (int s = 0; s < count; ++s) {
      const float l = p.part_lse[((size_t)(first + s) * p.s_q + q) * p.n_h + head];
      if (l != -INFINITY) tot += expf(l - mx);
    }
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    if (tot > 0.f) lse_row = mx + logf(tot);
#pragma unroll
    for (int kk = 0; kk < kDc / 32; ++kk) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < count; ++s) {
        const size_t prow = ((size_t)(first + s) * p.s_q + q) * p.n_h + head;
        const float l = p.part_lse[prow];
        if (l == -INFINITY) continue;
        const float wgt = expf(l - mx) * inv;
        const f32x4* src = (const f32x4*)(p.part_u + prow * kDc + kk * 32 + 8 * g);
        const f32x4 v0 = src[0], v1 = src[1];
        acc[0] = fmaf(wgt, v0[0], acc[0]); acc[1] = fmaf(wgt, v0[1], acc[1]);
        acc[2] = fmaf(wgt, v0[2], acc[2]); acc[3] = fmaf(wgt, v0[3], acc[3]);
        acc[4] = fmaf(wgt, v1[0], acc[4]); acc[5] = fmaf(wgt, v1[1], acc[5]);
        acc[6] = fmaf(wgt, v1[2], acc[6]); acc[7] = fmaf(wgt, v1[3], acc[7]);
      }
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const bf16x2 h = pack_bf16(acc[j], acc[j + 1]);
        const bf16x2 lo = pack_bf16(acc[j] - (float)h[0], acc[j + 1] - (float)h[1]);
        a_hi[kk][j] = h[0]; a_hi[kk][j + 1] = h[1];
        a_lo[kk][j] = lo[0]; a_lo[kk][j + 1] = lo[1];
      }
    }
  }
  if (valid && g == 0 && p.lse) p.lse[(size_t)r * p.n_h + head] = lse_row;

  // O[rows, v] = U[rows, k] W^T[k, v]; lane holds O[row 4g + i][v = nb*16 + l16].
  const bf16* wh = (const bf16*)p.w_uv + (size_t)head * kDv * kDc;
  bf16* out = (bf16*)p.out;
  const int rbase = blockIdx.y * kRowsPerWg + wave * 16;
#pragma unroll 1
  for (int nb = 0; nb < kDv / 16; ++nb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const bf16* wrow = wh + (size_t)(nb * 16 + l16) * kDc + 8 * g;
#pragma unroll
    for (int kk = 0; kk < kDc / 32; ++kk) {
      const bf16x8 bw = *(const bf16x8*)(wrow + kk * 32);
      acc = mfma16x16x32(a_hi[kk], bw, acc);
      acc = mfma16x16x32(a_lo[kk], bw, acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ro = rbase + 4 * g + i;
      if (ro < R) out[((size_t)ro * p.n_h + head) * kDv + nb * 16 + l16] = (bf16)acc[i];
    }
  }
}

// float32 path: one workgroup per (head, 16 rows), any d_c <= 1024 and d_v.
constexpr int kF32Rows = 16;
constexpr int kF32MaxDc = 1024;

__global__ __launch_bounds__(256) void combine_upproj_f32(const CombineParams p) {
  __shared__ float u_s[kF32Rows][kF32MaxDc];
  const int head = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int R = p.batch * p.s_q;
  for (int rr = wave; rr < kF32Rows; rr += 4) {
    const int r = blockIdx.y * kF32Rows + rr;
    if (r >= R) continue;
    const int b = r / p.s_q, q = r - b * p.s_q;
    int first, count;
    slot_range(p, b, first, count);
    float mx = -INFINITY;
    for (int s = lane; s < count; s += 64)
      mx = fmaxf(mx, p.part_lse[((size_t)(first + s) * p.s_q + q) * p.n_h + head]);
    mx = wave_max(mx);
    float tot = 0.f;
    for (int s = lane; s < count; s += 64) {
      const float l = p.part_lse[((size_t)(first + s) * p.s_q + q) * p.n_h + head];
      if (l != -INFINITY) tot += expf(l - mx);
    }
    tot = wave_sum(tot);
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    if (lane == 0 && p.lse) p.lse[(size_t)r * p.n_h + head] = tot > 0.f ? mx + logf(tot) : -INFINITY;
    for (int k = lane; k < p.d_c; k += 64) {
      float acc = 0.f;
      for (int s = 0; s < count; ++s) {
        const size_t prow = ((size_t)(first + s) * p.s_q + q) * p.n_h + head;
        const float l = p.part_lse[prow];
        if (l != -INFINITY) acc = fmaf(expf(l - mx) * inv, p.part_u[prow * p.d_c + k], acc);
      }
      u_s[rr][k] = acc;
    }
  }
  __syncthreads();
  const float* wh = (const float*)p.w_uv + (size_t)head * p.d_v * p.d_c;
  float* out = (float*)p.out;
  for (int idx = threadIdx.x; idx < kF32Rows * p.d_v; idx += blockDim.x) {
    const int rr = idx / p.d_v, v = idx - rr * p.d_v;
    const int r = blockIdx.y * kF32Rows + rr;
    if (r >= R) continue;
    float acc = 0.f;
    for (int k = 0; k < p.d_c; ++k) acc = fmaf(wh[(size_t)v * p.d_c + k], u_s[rr][k], acc);
    out[((size_t)r * p.n_h + head) * p.d_v + v] = acc;
  }
}

}  // namespace

hipError_t launch_combine_bf16(const CombineParams& p, hipStream_t stream) {
  const int R = p.batch * p.s_q;
  dim3 grid(p.n_h, (R + kRowsPerWg - 1) / kRowsPerWg);
  hipLaunchKernelGGL(combine_upproj_bf16, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_combine_f32(const CombineParams& p, hipStream_t stream) {
  const int R = p.batch * p.s_q;
  dim3 grid(p.n_h, (R + kF32Rows - 1) / kF32Rows);
  hipLaunchKernelGGL(combine_upproj_f32, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
