// Paged cache append: writes the new tokens' rows [c (d_c) | k^R (d_r)] into the
// pool at slot block_table[b][pos / P] * P + pos % P (page "MLA deep compression":
// only the latent c_t and the rotated position key k^R_t are cached per token).
// Copy modes move the bits unchanged; the E4M3 mode quantizes each token's row with
// one float32 scale: amax = max |x|, inv = fp32(448 / amax), scale = fp32(amax / 448)
// (both 1 when amax = 0), code = E4M3_RNE_sat(fp32(x * inv)).
// One wave per new token.

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

__device__ __forceinline__ float load_in(const void* base, size_t idx, bool f32) {
  return f32 ? ((const float*)base)[idx] : (float)((const bf16*)base)[idx];
}

__global__ __launch_bounds__(64) void paged_append(const AppendParams p) {
  const int tok = blockIdx.x;                 // b * s_new + j
  const int b = tok / p.s_new;
  const int lane = threadIdx.x;
  const int pos = p.positions[tok];
  if (pos < 0) return;
  const int page_idx = pos / p.page_size;
  if (page_idx >= p.max_pages) return;
  const int page = p.block_table[(size_t)b * p.max_pages + page_idx];
  if (page < 0 || page >= p.num_pages) return;
  const long long slot = (long long)page * p.page_size + pos % p.page_size;
  const size_t cin = (size_t)tok * p.d_c, kin = (size_t)tok * p.d_r;

  if (p.mode == 0) {                          // bf16 bits
    const uint16_t* cs = (const uint16_t*)p.c_new + cin;
    const uint16_t* ks = (const uint16_t*)p.k_new + kin;
    uint16_t* cd = (uint16_t*)p.c_kv + slot * p.c_stride;
    uint16_t* kd = (uint16_t*)p.k_pe + slot * p.k_stride;
    for (int k = lane; k < p.d_c; k += 64) cd[k] = cs[k];
    for (int k = lane; k < p.d_r; k += 64) kd[k] = ks[k];
    return;
  }
  if (p.mode == 1) {                          // float32 bits
    const uint32_t* cs = (const uint32_t*)p.c_new + cin;
    const uint32_t* ks = (const uint32_t*)p.k_new + kin;
    uint32_t* cd = (uint32_t*)p.c_kv + slot * p.c_stride;
    uint32_t* kd = (uint32_t*)p.k_pe + slot * p.k_stride;
    for (int k = lane; k < p.d_c; k += 64) cd[k] = cs[k];
    for (int k = lane; k < p.d_r; k += 64) kd[k] = ks[k];
    return;
  }
  // E4M3 + per-token scale.
  const bool f32 = p.in_f32 != 0;
  float amax = 0.f;
  for (int k = lane; k < p.d_c; k += 64) amax = fmaxf(amax, fabsf(load_in(p.c_new, cin + k, f32)));
  for (int k = lane; k < p.d_r; k += 64) amax = fmaxf(amax, fabsf(load_in(p.k_new, kin + k, f32)));
  amax = wave_max(amax);
  float inv = 1.f, scale = 1.f;
  if (amax > 0.f) {
    inv = __fdiv_rn(448.f, amax);
    scale = __fdiv_rn(amax, 448.f);
  }
  uint8_t* cd = (uint8_t*)p.c_kv + slot * p.c_stride;
  uint8_t* kd = (uint8_t*)p.k_pe + slot * p.k_stride;
  for (int k = lane; k < p.d_c; k += 64) cd[k] = (uint8_t)f32_to_e4m3(__fmul_rn(load_in(p.c_new, cin + k, f32), inv));
  for (int k = lane; k < p.d_r; k += 64) kd[k] = (uint8_t)f32_to_e4m3(__fmul_rn(load_in(p.k_new, kin + k, f32), inv));
  if (lane == 0) p.kv_scale[slot] = scale;
}

}  // namespace

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(paged_append, dim3(p.batch * p.s_new), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
