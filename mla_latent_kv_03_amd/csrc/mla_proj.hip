// Projections around the decode step (page "MLA deep compression": low-rank projection,
// absorption and decoupled RoPE sections; "Attention-head anatomy" section 5: W^UV folds
// into W^O):
//   cache write       [c | k^R_raw] = [W^DKV; W^KR] h, k^R = RoPE(k^R_raw) at the token's
//                     position, then the pool row (bf16, float32, or E4M3 + scale);
//   query prologue    q^C = W^Q h, q^R = RoPE(W^QR h); q~_i = (W^UK_i)^T q^C_i;
//   output projection y = W x with x = o (W = W^O) or x = u (W = W^OV, the folded weights),
//                     and the fold itself, W^OV_i = W^O_i W^UV_i.
// Every product is C = A B^T with the contraction index contiguous in both operands.
// bf16 operands run on 16x16x32 MFMAs, split over K into float32 partials that a finishing
// kernel sums together with the row's own epilogue; float32 operands (small layers) use
// plain FMA loops with the same partial layout.

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

constexpr int kGemmWaves = 4;
constexpr int kTileN = 16 * kGemmWaves;   // columns per workgroup (16 per wave)
constexpr int kTileM = 64;                // rows per workgroup (4 MFMA row blocks)

// C[M, N] (+)= A[M, K] B[N, K]^T over K chunk blockIdx.y, for batch / row tile blockIdx.z.
// Wave w owns columns n0 .. n0 + 15 of the workgroup's tile and all 64 rows: per 32-wide
// k-step it loads one B fragment (16 rows of B, 8 consecutive k each: 16 bytes per lane)
// and four A fragments (rows clamped to M - 1; such rows are never stored), and issues four
// MFMAs.  B is read from memory exactly once per row tile; A comes from the caches.
// A_F32: A is float32 and enters as a bf16 high part plus a bf16 remainder (two MFMAs).
template <bool A_F32>
__global__ __launch_bounds__(64 * kGemmWaves) void gemm_nt_bf16(const GemmArgs g) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * kTileN + 16 * wave;
  if (n0 >= g.N) return;                         // wave-uniform; the kernel has no barrier
  const int mtiles = (g.M + kTileM - 1) / kTileM;
  const int bt = blockIdx.z / mtiles;
  const int m0 = (blockIdx.z - bt * mtiles) * kTileM;
  const int k0 = blockIdx.y * g.kchunk;
  const int k1 = min(g.K, k0 + g.kchunk);
  const bf16* brow = (const bf16*)g.b + bt * g.b_bs + (int64_t)(n0 + l16) * g.ldb + 8 * grp;
  int64_t arow[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) arow[mb] = bt * g.a_bs + (int64_t)min(m0 + 16 * mb + l16, g.M - 1) * g.lda + 8 * grp;
  f32x4 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Operands of one 32-wide k-step: the B fragment and the four A fragments (float32 A:
  // two 16-byte halves per fragment, split into bf16 high and remainder parts at use).
  struct Step {
    bf16x8 b;
    u32x4 a[4][A_F32 ? 2 : 1];
  };
  auto load = [&](int k, Step& st) {
    st.b = *(const bf16x8*)(brow + k);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if constexpr (A_F32) {
        const float* ap = (const float*)g.a + arow[mb] + k;
        st.a[mb][0] = *(const u32x4*)ap;
        st.a[mb][A_F32 ? 1 : 0] = *(const u32x4*)(ap + 4);
      } else {
        st.a[mb][0] = *(const u32x4*)((const bf16*)g.a + arow[mb] + k);
      }
    }
  };
  auto compute = [&](const Step& st) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if constexpr (A_F32) {
        const f32x4 x0 = __builtin_bit_cast(f32x4, st.a[mb][0]), x1 = __builtin_bit_cast(f32x4, st.a[mb][A_F32 ? 1 : 0]);
        bf16x8 hi, lo;
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          const bf16x2 h0 = pack_bf16(x0[j], x0[j + 1]), h1 = pack_bf16(x1[j], x1[j + 1]);
          const bf16x2 r0 = pack_bf16(x0[j] - (float)h0[0], x0[j + 1] - (float)h0[1]);
          const bf16x2 r1 = pack_bf16(x1[j] - (float)h1[0], x1[j + 1] - (float)h1[1]);
          hi[j] = h0[0]; hi[j + 1] = h0[1]; hi[4 + j] = h1[0]; hi[5 + j] = h1[1];
          lo[j] = r0[0]; lo[j + 1] = r0[1]; lo[4 + j] = r1[0]; lo[5 + j] = r1[1];
        }
        acc[mb] = mfma16x16x32(hi, st.b, acc[mb]);
        acc[mb] = mfma16x16x32(lo, st.b, acc[mb]);
      } else {
        acc[mb] = mfma16x16x32(__builtin_bit_cast(bf16x8, st.a[mb][0]), st.b, acc[mb]);
      }
    }
  };
  // Four k-steps per round, all loads issued before the MFMAs that use them.
  int k = k0;
  for (; k + 128 <= k1; k += 128) {
    Step st[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) load(k + 32 * j, st[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j) compute(st[j]);
  }
  for (; k < k1; k += 32) {
    Step st;
    load(k, st);
    compute(st);
  }
  // Lane holds C[row 16 mb + 4 grp + i][column n0 + l16].
  const int64_t cbase = (int64_t)blockIdx.y * g.c_ks + bt * g.c_bs + n0 + l16;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 16 * mb + 4 * grp + i;
      if (m >= g.M) continue;
      if (g.out_bf16)
        ((bf16*)g.c)[cbase + (int64_t)m * g.ldc] = (bf16)acc[mb][i];
      else
        ((float*)g.c)[cbase + (int64_t)m * g.ldc] = acc[mb][i];
    }
}

// float32 operands: thread (m, n) of a 4 x 64 tile sums its K chunk with FMAs.
__global__ __launch_bounds__(256) void gemm_nt_f32(const GemmArgs g) {
  const int n = blockIdx.x * 64 + (threadIdx.x & 63);
  const int mtiles = (g.M + 3) / 4;
  const int bt = blockIdx.z / mtiles;
  const int m = (blockIdx.z - bt * mtiles) * 4 + (threadIdx.x >> 6);
  if (n >= g.N || m >= g.M) return;
  const int k0 = blockIdx.y * g.kchunk;
  const int k1 = min(g.K, k0 + g.kchunk);
  const float* a = (const float*)g.a + bt * g.a_bs + (int64_t)m * g.lda;
  const float* b = (const float*)g.b + bt * g.b_bs + (int64_t)n * g.ldb;
  float acc = 0.f;
  for (int k = k0; k < k1; ++k) acc = __builtin_fmaf(a[k], b[k], acc);
  ((float*)g.c)[(int64_t)blockIdx.y * g.c_ks + bt * g.c_bs + (int64_t)m * g.ldc + n] = acc;
}

// Rotation of one interleaved pair (x, y) = (v[2m], v[2m+1]) of a d_r-wide RoPE vector at
// position pos by angle pos * base^(-2m / d_r).  The angle and its sine and cosine are taken
// in float64 (pos * theta reaches ~1.3e5 radians, where a float32 angle would be off by
// ~1e-2); the rotation itself is float32.  Lanes hold consecutive elements, so the partner
// of lane l is lane l ^ 1 (d_c and the element index of lane l have the parity of l).
__device__ __forceinline__ float rope_lane(float v, int pair, int d_r, int pos, float base, bool odd) {
  const double theta = pow((double)base, -2.0 * (double)pair / (double)d_r);
  double s, c;
  sincos((double)pos * theta, &s, &c);
  const float partner = __shfl_xor(v, 1, 64);
  const float cs = (float)c, sn = (float)s;
  // even element: x cos - y sin; odd element: x sin + y cos
  return odd ? __builtin_fmaf(partner, sn, v * cs) : __builtin_fmaf(-partner, sn, v * cs);
}

constexpr int kMaxRowPerLane = 20;   // d_c + d_r <= 1280

// One wave per new token: sums the K-split partials of its [c | k^R_raw] row, rotates the
// RoPE part at the token's position and writes the pool slot (same slot rule and skips as
// the append kernel; same E4M3 quantizer).
__global__ __launch_bounds__(64) void cache_write_finish(const CacheWriteArgs a) {
  const int tok = blockIdx.x;
  const int b = tok / a.s_new;
  const int lane = threadIdx.x;
  const int pos = a.positions[tok];
  if (pos < 0) return;
  const int page_idx = pos / a.page_size;
  if (page_idx >= a.max_pages) return;
  const int page = a.block_table[(size_t)b * a.max_pages + page_idx];
  if (page < 0 || page >= a.num_pages) return;
  const long long slot = (long long)page * a.page_size + pos % a.page_size;
  const int D = a.d_c + a.d_r;
  float v[kMaxRowPerLane];
#pragma unroll
  for (int j = 0; j < kMaxRowPerLane; ++j) {
    const int e = lane + 64 * j;
    float s = 0.f;
    if (e < D)
      for (int ks = 0; ks < a.ksplit; ++ks) s += a.part[(int64_t)ks * a.part_ks + (int64_t)tok * D + e];
    v[j] = s;
  }
#pragma unroll
  for (int j = 0; j < kMaxRowPerLane; ++j) {
    const int e = lane + 64 * j;
    if (64 * j + 63 < a.d_c || 64 * j >= D) continue;        // wave-uniform: no RoPE element in this group
    const bool rot = e >= a.d_c && e < D;
    const float r = rope_lane(v[j], (e - a.d_c) >> 1, a.d_r, pos, a.rope_base, (lane & 1) != 0);
    if (rot) v[j] = r;
  }
  if (a.mode == 0 || a.mode == 1) {
#pragma unroll
    for (int j = 0; j < kMaxRowPerLane; ++j) {
      const int e = lane + 64 * j;
      if (e >= D) continue;
      if (a.mode == 0) {
        if (e < a.d_c) ((bf16*)a.c_kv)[slot * a.c_stride + e] = (bf16)v[j];
        else ((bf16*)a.k_pe)[slot * a.k_stride + e - a.d_c] = (bf16)v[j];
      } else {
        if (e < a.d_c) ((float*)a.c_kv)[slot * a.c_stride + e] = v[j];
        else ((float*)a.k_pe)[slot * a.k_stride + e - a.d_c] = v[j];
      }
    }
    return;
  }
  // E4M3 + per-token scale (the append kernel's quantizer on the float32 row).
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxRowPerLane; ++j)
    if (lane + 64 * j < D) amax = fmaxf(amax, fabsf(v[j]));
  amax = wave_max(amax);
  float inv = 1.f, scale = 1.f;
  if (amax > 0.f) {
    inv = __fdiv_rn(448.f, amax);
    scale = __fdiv_rn(amax, 448.f);
  }
#pragma unroll
  for (int j = 0; j < kMaxRowPerLane; ++j) {
    const int e = lane + 64 * j;
    if (e >= D) continue;
    const uint8_t code = (uint8_t)f32_to_e4m3(__fmul_rn(v[j], inv));
    if (e < a.d_c) ((uint8_t*)a.c_kv)[slot * a.c_stride + e] = code;
    else ((uint8_t*)a.k_pe)[slot * a.k_stride + e - a.d_c] = code;
  }
  if (lane == 0) a.kv_scale[slot] = scale;
}

// One wave per new query token: sums the K-split partials of q^C (to float32 scratch for the
// absorption product) and of q^R_raw, and writes q^R = RoPE(q^R_raw) per head.
__global__ __launch_bounds__(64) void query_finish(const QueryArgs a) {
  const int tok = blockIdx.x;
  const int lane = threadIdx.x;
  const int pos = a.positions[tok];
  const int nc = a.n_h * a.d_h, nr = a.n_h * a.d_r;
  for (int e = lane; e < nc; e += 64) {
    float s = 0.f;
    for (int ks = 0; ks < a.ksplit; ++ks) s += a.part_c[(int64_t)ks * a.part_c_ks + (int64_t)tok * nc + e];
    a.q_c[(int64_t)tok * nc + e] = s;
  }
  for (int e0 = 0; e0 < nr; e0 += 64) {                      // wave-uniform loop
    const int e = e0 + lane;
    float s = 0.f;
    if (e < nr)
      for (int ks = 0; ks < a.ksplit_r; ++ks) s += a.part_r[(int64_t)ks * a.part_r_ks + (int64_t)tok * nr + e];
    const int within = e % a.d_r;                              // d_r even: pairs never straddle heads
    const float r = rope_lane(s, within >> 1, a.d_r, pos, a.rope_base, (lane & 1) != 0);
    if (e < nr) {
      if (a.out_bf16) ((bf16*)a.q_pe)[(int64_t)tok * nr + e] = (bf16)r;
      else ((float*)a.q_pe)[(int64_t)tok * nr + e] = r;
    }
  }
}

// Sum of K-split partials [ksplit][n] into out (float32 or bf16), n elements.
__global__ __launch_bounds__(256) void sum_partials(const float* part, int64_t part_ks, int ksplit, int64_t n,
                                                   void* out, int out_bf16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int ks = 0; ks < ksplit; ++ks) s += part[(int64_t)ks * part_ks + i];
  if (out_bf16) ((bf16*)out)[i] = (bf16)s;
  else ((float*)out)[i] = s;
}

// dst[h][c][v] = src[h][v][c] (W^UV_i transposed per head), 16-bit or 32-bit elements.
template <class T>
__global__ __launch_bounds__(256) void transpose_heads(const T* src, T* dst, int rows, int cols, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // index into dst
  if (i >= n) return;
  const int64_t per = (int64_t)rows * cols;
  const int64_t h = i / per, r = i - h * per;
  const int c = (int)(r / rows), v = (int)(r - (int64_t)c * rows);
  dst[i] = src[h * per + (int64_t)v * cols + c];
}

}  // namespace

hipError_t launch_gemm_nt(const GemmArgs& g, bool bf16_operands, int ksplit, hipStream_t s) {
  if (bf16_operands) {
    dim3 grid((g.N + kTileN - 1) / kTileN, ksplit, g.batch * ((g.M + kTileM - 1) / kTileM));
    if (g.a_f32)
      hipLaunchKernelGGL(gemm_nt_bf16<true>, grid, dim3(64 * kGemmWaves), 0, s, g);
    else
      hipLaunchKernelGGL(gemm_nt_bf16<false>, grid, dim3(64 * kGemmWaves), 0, s, g);
  } else {
    dim3 grid((g.N + 63) / 64, ksplit, g.batch * ((g.M + 3) / 4));
    hipLaunchKernelGGL(gemm_nt_f32, grid, dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

hipError_t launch_cache_write_finish(const CacheWriteArgs& a, int tokens, hipStream_t s) {
  hipLaunchKernelGGL(cache_write_finish, dim3(tokens), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_query_finish(const QueryArgs& a, int tokens, hipStream_t s) {
  hipLaunchKernelGGL(query_finish, dim3(tokens), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sum_partials(const float* part, int64_t part_ks, int ksplit, int64_t n, void* out, bool out_bf16,
                               hipStream_t s) {
  hipLaunchKernelGGL(sum_partials, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, part_ks, ksplit, n, out,
                     out_bf16 ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_transpose_heads(const void* src, void* dst, int heads, int rows, int cols, bool bf16_elems,
                                  hipStream_t s) {
  const int64_t n = (int64_t)heads * rows * cols;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (bf16_elems)
    hipLaunchKernelGGL(transpose_heads<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)src, (uint16_t*)dst, rows,
                       cols, n);
  else
    hipLaunchKernelGGL(transpose_heads<uint32_t>, grid, dim3(256), 0, s, (const uint32_t*)src, (uint32_t*)dst, rows,
                       cols, n);
  return hipGetLastError();
}

}  // namespace mla
