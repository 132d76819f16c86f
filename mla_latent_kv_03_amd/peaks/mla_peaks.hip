// Attainable-peak probes for the roofline of the decode kernels (measurement only, not
// part of the decode library): an HBM streaming read in the attention kernel's own copy form
// (16-byte buffer -> LDS copies with the streaming policy, four waves per workgroup, two
// batches in flight), and a dense chain of 32x32x16 bf16 MFMAs on every SIMD.
// Built as libmla_peaks.so; bench.py --peaks times them with HIP events.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define PK_LDS __attribute__((address_space(3)))

// Workgroup w reads bytes [w * chunk, (w + 1) * chunk) of src, 1 KiB per wave-wide copy
// (lane l: 16 bytes at 16 l), into a 32 KiB LDS ring; every lane sums one dword of the
// ring at the end so that the reads are not dead.  chunk is a multiple of 4 KiB.
__global__ __launch_bounds__(256) void stream_read(const unsigned char* src, size_t chunk, float* sink) {
  __shared__ __attribute__((aligned(16))) unsigned char ring[32768];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned char* base = src + (size_t)blockIdx.x * chunk;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(base), 0,
                                                                       (int)chunk, 0x00020000);
  const unsigned n = (unsigned)(chunk / 1024);           // copies per workgroup
  for (unsigned i = wave; i < n; i += 4) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (PK_LDS void*)(ring + ((i / 4) % 8) * 4096 + wave * 1024), 16,
                                             i * 1024u + 16u * lane, 0, 0, 2);
    if (i >= 4 * 16) __builtin_amdgcn_s_waitcnt((15 & 15) | (7 << 4) | (15 << 8) | ((15 >> 4) << 14));   // vmcnt(15)
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  sink[blockIdx.x * 256 + threadIdx.x] = ((const float*)ring)[threadIdx.x];
}

// Four independent chains of 32x32x16 bf16 MFMAs per wave, iters x 16 MFMAs.
__global__ __launch_bounds__(256) void mfma_chain(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.0001f * (lane + j));
    b[j] = (__bf16)(0.0001f * (lane - j));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
  }
  float r = 0.f;
  for (int j = 0; j < 16; ++j) r += c0[j] + c1[j] + c2[j] + c3[j];
  out[blockIdx.x * 256 + threadIdx.x] = r;
}

}  // namespace

extern "C" {

// Stream `bytes` of src (a multiple of workgroups * 4 KiB) with `workgroups` workgroups;
// sink must hold workgroups * 256 floats.  Returns a hipError_t code.
int mla_peaks_stream_read(const void* src, size_t bytes, int workgroups, float* sink, void* stream) {
  if (!src || !sink || workgroups < 1 || bytes % ((size_t)workgroups * 4096) != 0) return (int)hipErrorInvalidValue;
  const size_t chunk = bytes / workgroups;
  if (chunk > 0x7fffffffu) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, (const unsigned char*)src,
                     chunk, sink);
  return (int)hipGetLastError();
}

// workgroups x 4 waves, each iters x 16 MFMAs of 32x32x16 (32768 flops); out holds
// workgroups * 256 floats.
int mla_peaks_mfma_bf16(float* out, int workgroups, int iters, void* stream) {
  if (!out || workgroups < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_chain, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, out, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
