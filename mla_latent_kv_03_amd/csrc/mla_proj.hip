// Projections around the decode step (page "MLA deep compression": low-rank projection,
// absorption and decoupled RoPE sections; "Attention-head anatomy" section 5: W^UV folds
// into W^O):
//   cache write       [c | k^R_raw] = [W^DKV; W^KR] h, k^R = RoPE(k^R_raw) at the token's
//                     position, then the pool row (bf16, float32, or E4M3 + scale);
//   query prologue    q^C = W^Q h, q^R = RoPE(W^QR h); q~_i = (W^UK_i)^T q^C_i;
//   output projection y = W x with x = o (W = W^O) or x = u (W = W^OV, the folded weights),
//                     and the fold itself, W^OV_i = W^O_i W^UV_i.
// Every product is C = A B^T with the contraction index contiguous in both operands.
// bf16 weights run on 32x32x16 MFMAs in a weight-streaming kernel, split over K into
// float32 partials that a finishing kernel sums together with the row's own epilogue;
// float32 operands (small layers) use plain FMA loops with the same partial layout.

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGemmWaves = 4;

// C[M, N] (+)= A[M, K] B[N, K]^T for bf16 B (the weights) and bf16 or float32 A (the few
// activation rows of a decode step), built to stream B from HBM once at full rate.
//
// A workgroup of four waves covers 4 NB blocks of 32 rows of B, a K chunk (blockIdx.y)
// and a row tile of A (blockIdx.z: MB blocks of 32 rows, rows past M clamped to M - 1 and
// never stored).  Per 16-wide k-step each wave loads 16 bytes of each of its B rows into
// a register ring of D steps (loads run D steps ahead of their MFMAs) and issues NB x MB
// 32x32x16 MFMAs, with A rows as the first operand and B rows as the second, so that lane
// l ends up holding C[8(v/4) + 4(l/32) + v%4][l%32] and each 32-lane half stores 128
// contiguous bytes of a C row.
// A is read from the caches once per workgroup, not once per wave (measured: every wave
// re-reading its A fragments from the L2 held the B stream to about a third of the HBM
// rate): blocks of 4 k-steps of A are staged in LDS in MFMA fragment order (fragment
// (step, m-block) = 64 lanes x 16 bytes, float32 A: two such halves), three blocks deep;
// each wave loads its share of block b + 2 into registers while block b is computed and
// stores it after the next barrier, so one barrier per block orders everything.  Steps
// past the chunk read the chunk's last B step and zero A, so whole rounds run unguarded.
// AF32: A enters as a bf16 high part plus a bf16 remainder (two MFMAs per pair).
template <int NB, int MB, bool AF32, int D>
__global__ __launch_bounds__(64 * kGemmWaves) void gemm_stream(const GemmArgs g) {
  static_assert(D == 8, "the round is two A blocks of four steps");
  constexpr int kFrag = 1024 * (AF32 ? 2 : 1);   // bytes of one A fragment
  constexpr int kSlot = 4 * MB * kFrag;          // one A block
  __shared__ __attribute__((aligned(16))) unsigned char a_lds[3 * kSlot];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, kh = lane >> 5;
  const int n0 = (blockIdx.x * kGemmWaves + wave) * 32 * NB;   // waves past N still stage A
  constexpr int kRows = 32 * MB;
  const int mtiles = (g.M + kRows - 1) / kRows;
  const int bt = blockIdx.z / mtiles;
  const int m0 = (blockIdx.z - bt * mtiles) * kRows;
  const int k0 = blockIdx.y * g.kchunk;
  const int k1 = min(g.K, k0 + g.kchunk);
  const int nsteps = (k1 - k0) >> 4;
  if (nsteps <= 0) return;                       // workgroup-uniform
  const int nrounds = (nsteps + 7) >> 3;
  const bf16* bp[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    bp[nb] = (const bf16*)g.b + bt * g.b_bs + (int64_t)min(n0 + 32 * nb + l32, g.N - 1) * g.ldb + k0 + 8 * kh;
  // This wave's A fragments of every block: f = wave + 4 j (j < MB), step f / MB, m-block
  // f % MB; arow[j] is the start of the fragment's A row.
  int64_t arow[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const int mb = (wave + 4 * j) % MB;
    arow[j] = bt * g.a_bs + (int64_t)min(m0 + 32 * mb + l32, g.M - 1) * g.lda;
  }
  u32x4 ar[MB][AF32 ? 2 : 1];
  auto load_a = [&](int blk) {
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int f = wave + 4 * j;
      const int k = k0 + 64 * blk + 16 * (f / MB) + 8 * kh;   // 8 values; the chunk ends on a multiple of 16
      const bool in = k < k1;
      const int64_t off = arow[j] + (in ? k : k0);            // past the chunk: an in-bounds read, zeroed
      if constexpr (AF32) {
        const float* x = (const float*)g.a + off;
        ar[j][0] = *(const u32x4*)x;
        ar[j][AF32 ? 1 : 0] = *(const u32x4*)(x + 4);
        if (!in) ar[j][0] = ar[j][AF32 ? 1 : 0] = u32x4{0u, 0u, 0u, 0u};
      } else {
        ar[j][0] = *(const u32x4*)((const bf16*)g.a + off);
        if (!in) ar[j][0] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_a = [&](int slot) {
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      unsigned char* dst = a_lds + slot * kSlot + (wave + 4 * j) * kFrag + 16 * lane;
      *(u32x4*)dst = ar[j][0];
      if constexpr (AF32) *(u32x4*)(dst + 1024) = ar[j][AF32 ? 1 : 0];
    }
  };
  f32x16 acc[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[nb][mb][v] = 0.f;
  bf16x8 ring[D][NB];
  auto load_w = [&](int step, bf16x8* w) {
    const int k = 16 * min(step, nsteps - 1);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) w[nb] = *(const bf16x8*)(bp[nb] + k);
  };
  // Step j (0..3) of the block in `slot`, with B fragments w.
  auto compute = [&](int slot, int j, const bf16x8* w) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const unsigned char* src = a_lds + slot * kSlot + (j * MB + mb) * kFrag + 16 * lane;
      if constexpr (AF32) {
        const f32x4 x0 = *(const f32x4*)src, x1 = *(const f32x4*)(src + 1024);
        bf16x8 hi, lo;
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const bf16x2 h0 = pack_bf16(x0[i], x0[i + 1]), h1 = pack_bf16(x1[i], x1[i + 1]);
          const bf16x2 r0 = pack_bf16(x0[i] - (float)h0[0], x0[i + 1] - (float)h0[1]);
          const bf16x2 r1 = pack_bf16(x1[i] - (float)h1[0], x1[i + 1] - (float)h1[1]);
          hi[i] = h0[0]; hi[i + 1] = h0[1]; hi[4 + i] = h1[0]; hi[5 + i] = h1[1];
          lo[i] = r0[0]; lo[i + 1] = r0[1]; lo[4 + i] = r1[0]; lo[5 + i] = r1[1];
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, w[nb], acc[nb][mb], 0, 0, 0);
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, w[nb], acc[nb][mb], 0, 0, 0);
        }
      } else {
        const bf16x8 a = *(const bf16x8*)src;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w[nb], acc[nb][mb], 0, 0, 0);
      }
    }
  };

  load_a(0);
  store_a(0);
  load_a(1);
#pragma unroll
  for (int j = 0; j < D; ++j) load_w(j, ring[j]);
  for (int r = 0; r < nrounds; ++r) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int blk = 2 * r + h;
      __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0): this wave's A stores are done
      __builtin_amdgcn_s_barrier();                // A(blk) is in LDS; block blk - 1 is finished
      __builtin_amdgcn_sched_barrier(0);
      store_a((blk + 1) % 3);
      load_a(blk + 2);
      const int slot = blk % 3;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // Keep the program order: the scheduler would otherwise sink the loads below the
        // MFMAs and drain the ring once per round.
        __builtin_amdgcn_sched_barrier(0);
        compute(slot, j, ring[4 * h + j]);
        load_w(8 * r + 4 * h + j + D, ring[4 * h + j]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (n0 >= g.N) return;
  // Lane holds C[m0 + 32 mb + 8 (v/4) + 4 kh + v%4][n0 + 32 nb + l32].
  const int64_t cbase = (int64_t)blockIdx.y * g.c_ks + bt * g.c_bs;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = n0 + 32 * nb + l32;
    if (n >= g.N) continue;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + 32 * mb + 8 * (v >> 2) + 4 * kh + (v & 3);
        if (m >= g.M) continue;
        if (g.out_bf16)
          ((bf16*)g.c)[cbase + (int64_t)m * g.ldc + n] = (bf16)acc[nb][mb][v];
        else
          ((float*)g.c)[cbase + (int64_t)m * g.ldc + n] = acc[nb][mb][v];
      }
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

// One wave per new token: reads its summed [c | k^R_raw] row (float32; the K-split
// partials are added by sum_partials first), rotates the RoPE part at the token's position
// and writes the pool slot (same slot rule and skips as the append kernel; same E4M3
// quantizer).
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
    v[j] = e < D ? a.part[(int64_t)tok * D + e] : 0.f;
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

// Query prologue finish, one thread per element: the first ceil(T n_h d_h / 256)
// workgroups sum the K-split partials of q^C into float32 scratch (the absorption
// product's input), the others sum those of q^R_raw and rotate each interleaved pair by
// its token's position (the partner element is in the neighbouring lane: n_h d_r is even,
// so pairs never straddle a workgroup, a token or a head).
__global__ __launch_bounds__(256) void query_finish(const QueryArgs a, int tokens, int c_blocks) {
  const int64_t nc = (int64_t)tokens * a.n_h * a.d_h, nr = (int64_t)tokens * a.n_h * a.d_r;
  if ((int)blockIdx.x < c_blocks) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= nc) return;
    float v = 0.f;
    for (int ks = 0; ks < a.ksplit; ++ks) v += a.part_c[(int64_t)ks * a.part_c_ks + e];
    a.q_c[e] = v;
    return;
  }
  const int64_t e = (int64_t)(blockIdx.x - c_blocks) * 256 + threadIdx.x;
  const bool in = e < nr;
  const int64_t ec = in ? e : nr - 1;
  const int per_tok = a.n_h * a.d_r;
  const int tok = (int)(ec / per_tok);
  const int within = (int)(ec - (int64_t)tok * per_tok) % a.d_r;
  float v = 0.f;
  if (in)
    for (int ks = 0; ks < a.ksplit_r; ++ks) v += a.part_r[(int64_t)ks * a.part_r_ks + e];
  const float r = rope_lane(v, within >> 1, a.d_r, a.positions[tok], a.rope_base, (threadIdx.x & 1) != 0);
  if (!in) return;
  if (a.out_bf16) ((bf16*)a.q_pe)[e] = (bf16)r;
  else ((float*)a.q_pe)[e] = r;
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
    const int mb = gemm_row_blocks(g.M);
    const int nb = gemm_col_blocks(g.a_f32 != 0);
    dim3 grid((g.N + 32 * nb * kGemmWaves - 1) / (32 * nb * kGemmWaves), ksplit,
              g.batch * ((g.M + 32 * mb - 1) / (32 * mb)));
    dim3 block(64 * kGemmWaves);
    if (g.a_f32) {
      if (mb == 2) hipLaunchKernelGGL((gemm_stream<2, 2, true, 8>), grid, block, 0, s, g);
      else hipLaunchKernelGGL((gemm_stream<2, 1, true, 8>), grid, block, 0, s, g);
    } else {
      if (mb == 2) hipLaunchKernelGGL((gemm_stream<1, 2, false, 8>), grid, block, 0, s, g);
      else hipLaunchKernelGGL((gemm_stream<1, 1, false, 8>), grid, block, 0, s, g);
    }
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
  const int64_t nc = (int64_t)tokens * a.n_h * a.d_h, nr = (int64_t)tokens * a.n_h * a.d_r;
  const int c_blocks = (int)((nc + 255) / 256), r_blocks = (int)((nr + 255) / 256);
  hipLaunchKernelGGL(query_finish, dim3(c_blocks + r_blocks), dim3(256), 0, s, a, tokens, c_blocks);
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
