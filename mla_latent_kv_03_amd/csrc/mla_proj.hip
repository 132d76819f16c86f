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

// The buffer->LDS copy of buffer_to_lds16 with the default cache policy (the activation
// rows are read by every workgroup).
__device__ __forceinline__ void buffer_to_lds16_cached(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset, uint32_t soffset,
                                                       void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (MLA_LDS void*)(lds_wave_base), 16, voffset, soffset, 0, 0);
}

// s_waitcnt vmcnt(N) alone (lgkmcnt and expcnt left at their maxima).
template <int N>
__device__ __forceinline__ void gemm_wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
constexpr int kGemmRing = 12;      // k-steps in flight (bf16 A: 80 KiB of LDS, two workgroups per CU)
constexpr int kGemmRingF32 = 12;   // float32 A, two B blocks per wave: 160 KiB of LDS

// C[M, N] (+)= A[M, K] B[N, K]^T for bf16 B (the weights) and bf16 or float32 A (the few
// activation rows of a decode step), built to stream B from HBM once at full rate.
//
// A workgroup of four waves covers 4 NB blocks of 32 rows of B, a K chunk (blockIdx.y)
// and a row tile of A (blockIdx.z: MB blocks of 32 rows, rows past M clamped to M - 1 and
// never stored).  Per 16-wide k-step a wave issues NB MFMAs per 32-row block of A
// (32x32x16), with A rows as the first operand and B rows as the second, so that lane l
// ends up holding C[8(v/4) + 4(l/32) + v%4][l%32] and each 32-lane half stores 128
// contiguous bytes of a C row.
//
// Both operands reach the MFMAs through LDS, in blocks of four k-steps (128 bytes of a
// bf16 row, 256 of a float32 row), copied by buffer->LDS loads that read whole 128-byte
// lines: a copy covers 8 rows x 128 bytes (float32 A: 4 rows x 256), lane l taking
// 16-byte chunk (l % 8) ^ (row % 8) of its row (l % 16 for 256-byte rows), so that chunk c
// of row r sits at position c ^ (r % 8) of the row in LDS and the operand reads (16 rows,
// one chunk each) hit distinct banks.  Copies that read 32 bytes of 32 different lines
// each held the weight stream to about 3.3 TB/s; whole lines per copy are what a plain
// streaming read needs for full rate.  Copies carry no register results, so their waits
// are exact counts written here (register loads into a ring made the compiler drain the
// ring at every loop head).
//  - B: each wave streams its own rows through a private ring of RA = D / 4 blocks; block
//    b + RA is copied at the end of block b, into the slot block b has left.
//  - A: RA + 1 shared slots; block b + RA is copied at the start of block b (into the slot
//    of block b - 1, which every wave has finished at the barrier), each wave a quarter
//    of its rows; one barrier per block publishes it.
// Per wave the copies go out in a fixed order (block b: A(b + RA), then B(b + RA)), so
// the number issued after any copy is a constant.  The resources end at the operands' last
// bytes, so reads past them return zeros.  RAGGED: a chunk may end inside a block (K or
// the chunk not a multiple of 64), whose steps past the chunk are skipped; otherwise every
// block is whole and its operands are read from LDS before its MFMAs.
// AF32: A enters as a bf16 high part plus a bf16 remainder (two MFMAs per pair).
template <int NB, int MB, bool AF32, int D, bool RAGGED>
__global__ __launch_bounds__(64 * kGemmWaves) void gemm_stream(const GemmArgs g) {
  static_assert(D % 4 == 0 && D >= 8, "the ring holds whole blocks of four steps");
  constexpr int RA = D / 4;                          // blocks in flight
  constexpr int SA = RA + 1;                         // A slots
  constexpr int kAElem = AF32 ? 4 : 2;
  constexpr int kARow = 64 * kAElem;                 // bytes of an A row in one block
  constexpr int kASlot = 32 * MB * kARow;            // one A block
  constexpr int kBBlock = 32 * NB * 128;             // one block of one wave's B rows
  constexpr int kACopies = kASlot / 1024 / kGemmWaves;
  constexpr int kBCopies = kBBlock / 1024;
  constexpr int kWait = (RA - 1) * (kACopies + kBCopies);
  static_assert(kWait < 64, "vmcnt holds 6 bits");
  __shared__ __attribute__((aligned(16))) unsigned char lds[SA * kASlot + kGemmWaves * RA * kBBlock];
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
  if (nsteps <= 0) return;                           // workgroup-uniform
  const int nblocks = (nsteps + 3) >> 2;

  // B copy i of a block: rows 8 i .. 8 i + 7 of the wave's 32 NB rows, from b or, past
  // n_split, from b2 (a wave's rows lie in one of them).
  const bool second = g.b2 != nullptr && n0 >= g.n_split;
  const int b_rows = g.b2 == nullptr ? g.N : second ? g.N - g.n_split : g.n_split;
  const int nb0 = second ? n0 - g.n_split : n0;
  const int64_t b_bytes = ((int64_t)(b_rows - 1) * g.ldb + g.K) * 2;
  const __amdgpu_buffer_rsrc_t rs_b =
      buffer_rsrc((const bf16*)(second ? g.b2 : g.b) + bt * g.b_bs, (int)min(b_bytes, (int64_t)INT32_MAX));
  uint32_t vo_b[kBCopies];
#pragma unroll
  for (int i = 0; i < kBCopies; ++i) {
    const int r = 8 * i + (lane >> 3);
    vo_b[i] = (uint32_t)((int64_t)min(nb0 + r, b_rows - 1) * g.ldb * 2) + 16u * (uint32_t)((lane & 7) ^ (r & 7));
  }
  unsigned char* const bring = lds + SA * kASlot + wave * RA * kBBlock;
  auto copy_b = [&](int blk) {
    const uint32_t so = (uint32_t)(k0 + 64 * blk) * 2u;
    unsigned char* dst = bring + (blk % RA) * kBBlock;
#pragma unroll
    for (int i = 0; i < kBCopies; ++i) buffer_to_lds16_cached(rs_b, vo_b[i], so, dst + 1024 * i);
  };
  // A copy ii = wave + 4 j: rows 8 ii .. (float32: 4 ii ..) of the 32 MB rows.
  constexpr int kARowsPerCopy = 1024 / kARow;
  const int64_t a_bytes = ((int64_t)(g.M - 1) * g.lda + g.K) * kAElem;
  const __amdgpu_buffer_rsrc_t rs_a =
      buffer_rsrc((const unsigned char*)g.a + (int64_t)bt * g.a_bs * kAElem, (int)min(a_bytes, (int64_t)INT32_MAX));
  uint32_t vo_a[kACopies];
#pragma unroll
  for (int j = 0; j < kACopies; ++j) {
    const int ii = wave + kGemmWaves * j;
    const int rr = kARowsPerCopy * ii + lane / (kARow / 16);
    const int c = (lane % (kARow / 16)) ^ (rr & 7);
    vo_a[j] = (uint32_t)((int64_t)min(m0 + rr, g.M - 1) * g.lda * kAElem) + 16u * (uint32_t)c;
  }
  auto copy_a = [&](int blk) {
    const uint32_t so = (uint32_t)(k0 + 64 * blk) * (uint32_t)kAElem;
    unsigned char* slot = lds + (blk % SA) * kASlot;
#pragma unroll
    for (int j = 0; j < kACopies; ++j) buffer_to_lds16_cached(rs_a, vo_a[j], so, slot + 1024 * (wave + kGemmWaves * j));
  };

  f32x16 acc[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[nb][mb][v] = 0.f;
  // Operand rows of this lane: B row 32 nb + l32 of the wave's block, A row 32 mb + l32.
  const int sw = l32 & 7;                            // (32 x + l32) % 8
  // Operands of step j (0..3) of block blk: B fragments w, A fragments a (float32 A: the
  // two 16-byte halves of each).
  constexpr int kAF = MB * (AF32 ? 2 : 1);
  auto read_ops = [&](int blk, int j, bf16x8* w, u32x4* a) {
    const unsigned char* bsrc = bring + (blk % RA) * kBBlock + 128 * l32 + 16 * ((2 * j + kh) ^ sw);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) w[nb] = *(const bf16x8*)(bsrc + 4096 * nb);
    const unsigned char* abase = lds + (blk % SA) * kASlot + kARow * l32;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const unsigned char* arow = abase + 32 * kARow * mb;
      if constexpr (AF32) {
        a[2 * mb] = *(const u32x4*)(arow + 16 * ((4 * j + 2 * kh) ^ sw));
        a[2 * mb + 1] = *(const u32x4*)(arow + 16 * ((4 * j + 2 * kh + 1) ^ sw));
      } else {
        a[mb] = *(const u32x4*)(arow + 16 * ((2 * j + kh) ^ sw));
      }
    }
  };
  auto mfmas = [&](const bf16x8* w, const u32x4* a) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if constexpr (AF32) {
        const f32x4 x0 = (f32x4)a[2 * mb], x1 = (f32x4)a[2 * mb + 1];
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
        const bf16x8 x = (bf16x8)a[mb];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, w[nb], acc[nb][mb], 0, 0, 0);
      }
    }
  };
  auto compute = [&](int blk, int j) {
    bf16x8 w[NB];
    u32x4 a[kAF];
    read_ops(blk, j, w, a);
    mfmas(w, a);
  };

#pragma unroll
  for (int b = 0; b < RA; ++b) {
    copy_a(b);
    copy_b(b);
  }
  for (int blk = 0; blk < nblocks; ++blk) {
    gemm_wait_vmcnt<kWait>();                        // this wave's copies of A(blk) and B(blk) landed
    __builtin_amdgcn_s_barrier();                    // all of A(blk); block blk - 1 finished everywhere
    __builtin_amdgcn_sched_barrier(0);
    copy_a(blk + RA);                                // into the slot of block blk - 1
    if constexpr (RAGGED) {
      for (int j = 0; j < 4 && 4 * blk + j < nsteps; ++j) compute(blk, j);
    } else {
      // All reads of the block first (two steps at a time for float32 A), then its MFMAs.
      constexpr int kBatch = AF32 ? 2 : 4;
#pragma unroll
      for (int j0 = 0; j0 < 4; j0 += kBatch) {
        bf16x8 w[kBatch][NB];
        u32x4 a[kBatch][kAF];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) read_ops(blk, j0 + j, w[j], a[j]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kBatch; ++j) mfmas(w[j], a[j]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);              // lgkmcnt(0): B(blk) has been read
    __builtin_amdgcn_sched_barrier(0);
    copy_b(blk + RA);                                // into the slot block blk has left
  }
  gemm_wait_vmcnt<0>();                              // no copy may land after the workgroup ends
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
// ~1e-2); the rotation itself is float32.
__device__ __forceinline__ void rope_pair(float& x, float& y, int m, int d_r, int pos, float base) {
  const double theta = pow((double)base, -2.0 * (double)m / (double)d_r);
  double sd, cd;
  sincos((double)pos * theta, &sd, &cd);
  const float cs = (float)cd, sn = (float)sd;
  const float xr = __builtin_fmaf(-y, sn, x * cs), yr = __builtin_fmaf(x, sn, y * cs);
  x = xr;
  y = yr;
}

// One workgroup per new token, one thread per pair of row elements (the pair a RoPE
// rotation mixes; d_c is even): sums the pair's K-split partials in chunk order, rotates it
// if it lies in the RoPE part, and writes the pool slot (same slot rule and skips as the
// append kernel; same E4M3 quantizer on the float32 row, its amax reduced over the
// workgroup).  d_c + d_r <= 1280, so at most 640 threads.
__global__ __launch_bounds__(640) void cache_write_finish(const CacheWriteArgs a) {
  __shared__ float wave_amax[10];
  const int tok = blockIdx.x;
  const int b = tok / a.s_new;
  const int t = threadIdx.x;
  const int pos = a.positions[tok];
  if (pos < 0) return;                                       // workgroup-uniform skips
  const int page_idx = pos / a.page_size;
  if (page_idx >= a.max_pages) return;
  const int page = a.block_table[(size_t)b * a.max_pages + page_idx];
  if (page < 0 || page >= a.num_pages) return;
  const long long slot = (long long)page * a.page_size + pos % a.page_size;
  const int D = a.d_c + a.d_r;
  const int e = 2 * t;
  const bool in = e < D;
  float x = 0.f, y = 0.f;
  if (in) {
    // 16 partials in flight at a time (chunks past ksplit read chunk 0 and are not added).
    const float* src = a.part + (int64_t)tok * D + e;
    for (int j0 = 0; j0 < a.ksplit; j0 += 16) {
      f32x2 p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = j0 + i < a.ksplit ? j0 + i : 0;
        p[i] = *(const f32x2*)(src + (int64_t)j * a.part_ks);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (j0 + i < a.ksplit) {
          x += p[i][0];
          y += p[i][1];
        }
    }
    if (e >= a.d_c) rope_pair(x, y, (e - a.d_c) >> 1, a.d_r, pos, a.rope_base);
  }
  if (a.mode == 0 || a.mode == 1) {
    if (!in) return;
    const bool kpart = e >= a.d_c;
    const long long o = kpart ? slot * a.k_stride + e - a.d_c : slot * a.c_stride + e;
    if (a.mode == 0) {
      bf16* dst = (bf16*)(kpart ? a.k_pe : a.c_kv) + o;
      dst[0] = (bf16)x;
      dst[1] = (bf16)y;
    } else {
      float* dst = (float*)(kpart ? a.k_pe : a.c_kv) + o;
      dst[0] = x;
      dst[1] = y;
    }
    return;
  }
  // E4M3 + per-token scale.
  float amax = wave_max(fmaxf(fabsf(x), fabsf(y)));
  if ((t & 63) == 0) wave_amax[t >> 6] = amax;
  __syncthreads();
  amax = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) amax = fmaxf(amax, wave_amax[w]);
  float inv = 1.f, scale = 1.f;
  if (amax > 0.f) {
    inv = __fdiv_rn(448.f, amax);
    scale = __fdiv_rn(amax, 448.f);
  }
  if (in) {
    const bool kpart = e >= a.d_c;
    uint8_t* dst = (uint8_t*)(kpart ? a.k_pe : a.c_kv) + (kpart ? slot * a.k_stride + e - a.d_c : slot * a.c_stride + e);
    dst[0] = (uint8_t)f32_to_e4m3(__fmul_rn(x, inv));
    dst[1] = (uint8_t)f32_to_e4m3(__fmul_rn(y, inv));
  }
  if (t == 0) a.kv_scale[slot] = scale;
}

// Query prologue finish, four consecutive elements per thread (16-byte loads and stores
// when the widths allow; the partials of 8 K-chunks loaded together): the first
// ceil(T n_h d_h / 1024) workgroups sum the K-split partials of q^C into float32 scratch
// (the absorption product's input), the others sum those of q^R_raw and rotate each of
// their two interleaved pairs by its token's position (n_h d_r and d_r are even, so a pair
// never straddles a token or a head).
__device__ __forceinline__ f32x4 sum_partials4(const float* src, int64_t ks_stride, int ksplit, int n) {
  constexpr int kB = 8;
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (n == 4 && (reinterpret_cast<uintptr_t>(src) & 15) == 0 && (ks_stride & 3) == 0) {
    for (int j0 = 0; j0 < ksplit; j0 += kB) {
      f32x4 p[kB];
#pragma unroll
      for (int i = 0; i < kB; ++i) p[i] = *(const f32x4*)(src + (int64_t)(j0 + i < ksplit ? j0 + i : 0) * ks_stride);
#pragma unroll
      for (int i = 0; i < kB; ++i)
        if (j0 + i < ksplit) v += p[i];
    }
    return v;
  }
  for (int k = 0; k < n; ++k)
    for (int j = 0; j < ksplit; ++j) v[k] += src[(int64_t)j * ks_stride + k];
  return v;
}

// q^R finish for n elements from e0 (4 per thread): sum of the K-split partials, then each
// interleaved pair rotated by its token's position.
__device__ __forceinline__ void finish_q_rope(const QueryArgs& a, int64_t e0, int64_t nr) {
  const int n = (int)min((int64_t)4, nr - e0);
  f32x4 v = sum_partials4(a.part_r + e0, a.part_r_ks, a.ksplit_r, n);
  const int per_tok = a.n_h * a.d_r;
#pragma unroll
  for (int k = 0; k < 4; k += 2) {
    if (k >= n) break;
    const int64_t e = e0 + k;
    const int tok = (int)(e / per_tok);
    const int within = (int)(e - (int64_t)tok * per_tok) % a.d_r;
    float x = v[k], y = v[k + 1];
    rope_pair(x, y, within >> 1, a.d_r, a.positions[tok], a.rope_base);
    v[k] = x;
    v[k + 1] = y;
  }
  for (int k = 0; k < n; ++k) {
    if (a.out_bf16) ((bf16*)a.q_pe)[e0 + k] = (bf16)v[k];
    else ((float*)a.q_pe)[e0 + k] = v[k];
  }
}

__global__ __launch_bounds__(256) void query_finish(const QueryArgs a, int tokens, int c_blocks) {
  const int64_t nc = (int64_t)tokens * a.n_h * a.d_h, nr = (int64_t)tokens * a.n_h * a.d_r;
  if ((int)blockIdx.x < c_blocks) {
    const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e0 >= nc) return;
    const int n = (int)min((int64_t)4, nc - e0);
    const f32x4 v = sum_partials4(a.part_c + e0, a.part_c_ks, a.ksplit, n);
    if (n == 4 && (nc & 3) == 0) *(f32x4*)(a.q_c + e0) = v;
    else
      for (int k = 0; k < n; ++k) a.q_c[e0 + k] = v[k];
    return;
  }
  const int64_t e0 = ((int64_t)(blockIdx.x - c_blocks) * 256 + threadIdx.x) * 4;
  if (e0 < nr) finish_q_rope(a, e0, nr);
}

// The absorption product of the bf16 query prologue, fused with the partial sums:
// workgroup (head i, block of 64 tokens, block of 256 latent columns) sums the K-split
// partials of its q^C rows in float32 (every load of the workgroup in flight together),
// keeps them in LDS as a bf16 high part and remainder (the projections' float32 operand
// form: two MFMAs per k-step), and each wave multiplies them by 64 rows of (W^UK_i)^T,
// read straight from memory, on 32x32x16 MFMAs: q~_i[t][c] = sum_k q^C_i[t][k] W^UK_i[k][c].
// Chunk c (16 bytes) of LDS row r sits at c ^ (r % 8) (r % 4 when d_h is an odd multiple
// of 32: a row then holds a multiple of 4 chunks, not of 8), so the operand reads (one chunk
// of 32 rows) spread over the banks.  The workgroups past the products finish q^R.
constexpr int kQaTok = 64, kQaCols = 256, kQaMaxDh = 256;   // LDS: 64 rows x d_h x 4 bytes

__global__ __launch_bounds__(256) void query_absorb(const QueryArgs a, int tokens, int n_prod) {
  extern __shared__ __attribute__((aligned(16))) unsigned char qa_lds[];
  if ((int)blockIdx.x >= n_prod) {
    const int64_t nr = (int64_t)tokens * a.n_h * a.d_r;
    const int64_t e0 = ((int64_t)(blockIdx.x - n_prod) * 256 + threadIdx.x) * 4;
    if (e0 < nr) finish_q_rope(a, e0, nr);
    return;
  }
  const int d_h = a.d_h, d_c = a.d_c;
  const int n_tb = (tokens + kQaTok - 1) / kQaTok, n_cb = (d_c + kQaCols - 1) / kQaCols;
  const int head = (int)blockIdx.x / (n_tb * n_cb);
  const int rest = (int)blockIdx.x - head * n_tb * n_cb;
  const int t0 = (rest / n_cb) * kQaTok, c_blk = (rest % n_cb) * kQaCols;
  const int row_bytes = d_h * 2;                           // one bf16 row of A
  const int swz = d_h % 64 == 0 ? 7 : 3;
  unsigned char* a_hi = qa_lds;
  unsigned char* a_lo = qa_lds + kQaTok * row_bytes;

  // Sum of the partials, 4 elements per thread and item, 8 items' loads in flight together
  // (a loop of one item at a time would wait for each item's loads in turn); rows past the
  // tokens are zero.
  const int64_t stride_t = (int64_t)a.n_h * d_h;
  const int per_row4 = d_h / 4, items = kQaTok * per_row4;
  for (int q0 = threadIdx.x; q0 < items; q0 += 256 * 8) {
    f32x4 v[8];
    const float* src[8];
    bool ok[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int q = q0 + 256 * u;
      const int r = q / per_row4, k = (q - r * per_row4) * 4;
      ok[u] = q < items && t0 + r < tokens;
      src[u] = a.part_c + (ok[u] ? (t0 + r) * stride_t + (int64_t)head * d_h + k : 0);
      v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int j = 0; j < a.ksplit; ++j) {             // K chunks in order, as the other finishers
      f32x4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = *(const f32x4*)(src[u] + (int64_t)j * a.part_c_ks);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (ok[u]) v[u] += x[u];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int q = q0 + 256 * u;
      if (q >= items) break;
      const int r = q / per_row4, k = (q - r * per_row4) * 4;
      const bf16x4 hi = to_bf16x4(v[u]);
      const bf16x4 lo = to_bf16x4(v[u] - from_bf16x4(hi));
      const int off = r * row_bytes + 16 * ((k >> 3) ^ (r & swz)) + 2 * (k & 7);
      *(bf16x4*)(a_hi + off) = hi;
      *(bf16x4*)(a_lo + off) = lo;
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l32 = lane & 31, kh = lane >> 5;
  const int c0 = c_blk + 64 * wave;
  if (c0 >= d_c) return;
  f32x16 acc[2][2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[nb][mb][v] = 0.f;
  // B rows of this lane: columns c0 + 32 nb + l32 of q~, i.e. rows of (W^UK_i)^T.
  const bf16* wrow[2];
  bool wok[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int c = c0 + 32 * nb + l32;
    wok[nb] = c < d_c;
    wrow[nb] = (const bf16*)a.w_uk_t + ((int64_t)head * d_c + (wok[nb] ? c : 0)) * d_h + 8 * kh;
  }
  for (int k0 = 0; k0 < d_h; k0 += 128) {
    // Up to 8 k-steps of B at once (16 loads in flight per lane); steps past d_h load a
    // valid fragment of the row (its last) and are not used.
    bf16x8 w[8][2];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const bf16x8 x = *(const bf16x8*)(wrow[nb] + min(k0 + 16 * j, d_h - 16));
        w[j][nb] = wok[nb] ? x : bf16x8{};
      }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = k0 + 16 * j;
      if (k >= d_h) break;
      const int chunk = (k >> 3) + kh;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int r = 32 * mb + l32;
        const int off = r * row_bytes + 16 * (chunk ^ (r & swz));
        const bf16x8 hi = *(const bf16x8*)(a_hi + off);
        const bf16x8 lo = *(const bf16x8*)(a_lo + off);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, w[j][nb], acc[nb][mb], 0, 0, 0);
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, w[j][nb], acc[nb][mb], 0, 0, 0);
        }
      }
    }
  }
  // Lane holds q~[t0 + 32 mb + 8 (v/4) + 4 kh + v%4][c0 + 32 nb + l32].
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    if (!wok[nb]) continue;
    const int c = c0 + 32 * nb + l32;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = t0 + 32 * mb + 8 * (v >> 2) + 4 * kh + (v & 3);
        if (t < tokens) ((bf16*)a.q_nope)[((int64_t)t * a.n_h + head) * d_c + c] = (bf16)acc[nb][mb][v];
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
    // The copies address B and A through 32-bit buffer offsets: a B of 2 GiB or more runs
    // as several launches over row ranges of B (columns of C).
    const int64_t max_bytes = (int64_t)1 << 31;
    const int64_t a_bytes = ((int64_t)(g.M - 1) * g.lda + g.K) * (g.a_f32 ? 4 : 2);
    if (a_bytes >= max_bytes) return hipErrorInvalidValue;
    const int64_t b_bytes = ((int64_t)(g.N - 1) * g.ldb + g.K) * 2;
    if (g.b2 != nullptr && (b_bytes >= max_bytes || g.n_split % (32 * gemm_col_blocks(g.a_f32 != 0)) != 0))
      return hipErrorInvalidValue;
    if (b_bytes >= max_bytes) {
      const int rows = (int)((max_bytes / 2 - g.K) / g.ldb) & ~127;   // whole workgroups of B rows
      if (rows < 128) return hipErrorInvalidValue;
      for (int n = 0; n < g.N; n += rows) {
        GemmArgs part = g;
        part.b = (const bf16*)g.b + (int64_t)n * g.ldb;
        part.c = g.out_bf16 ? (void*)((bf16*)g.c + n) : (void*)((float*)g.c + n);
        part.N = min(rows, g.N - n);
        const hipError_t e = launch_gemm_nt(part, true, ksplit, s);
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    }
    const int mb = gemm_row_blocks(g.M);
    const int nb = gemm_col_blocks(g.a_f32 != 0);
    dim3 grid((g.N + 32 * nb * kGemmWaves - 1) / (32 * nb * kGemmWaves), ksplit,
              g.batch * ((g.M + 32 * mb - 1) / (32 * mb)));
    dim3 block(64 * kGemmWaves);
    const bool ragged = g.K % 64 != 0 || g.kchunk % 64 != 0;
#define MLA_GEMM(NB_, MB_, F32_, D_)                                                  \
  do {                                                                             \
    if (ragged) hipLaunchKernelGGL((gemm_stream<NB_, MB_, F32_, D_, true>), grid, block, 0, s, g);  \
    else hipLaunchKernelGGL((gemm_stream<NB_, MB_, F32_, D_, false>), grid, block, 0, s, g);        \
  } while (0)
    if (g.a_f32) {
      if (mb == 2) MLA_GEMM(2, 2, true, kGemmRingF32);
      else MLA_GEMM(2, 1, true, kGemmRingF32);
    } else {
      if (mb == 2) MLA_GEMM(1, 2, false, kGemmRing);
      else MLA_GEMM(1, 1, false, kGemmRing);
    }
#undef MLA_GEMM
  } else {
    dim3 grid((g.N + 63) / 64, ksplit, g.batch * ((g.M + 3) / 4));
    hipLaunchKernelGGL(gemm_nt_f32, grid, dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

hipError_t launch_cache_write_finish(const CacheWriteArgs& a, int tokens, hipStream_t s) {
  const int waves = (a.d_c + a.d_r + 127) / 128;   // one thread per element pair
  hipLaunchKernelGGL(cache_write_finish, dim3(tokens), dim3(64 * waves), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_query_absorb(const QueryArgs& a, int tokens, hipStream_t s) {
  if (a.d_h % 32 || a.d_h > kQaMaxDh || a.d_c < 1 || !a.out_bf16) return hipErrorInvalidValue;
  const int n_prod = a.n_h * ((tokens + kQaTok - 1) / kQaTok) * ((a.d_c + kQaCols - 1) / kQaCols);
  const int64_t nr = (int64_t)tokens * a.n_h * a.d_r;
  const int r_blocks = (int)((nr + 1023) / 1024);
  const size_t lds = (size_t)kQaTok * a.d_h * 4;          // bf16 high and low rows
  hipLaunchKernelGGL(query_absorb, dim3(n_prod + r_blocks), dim3(256), lds, s, a, tokens, n_prod);
  return hipGetLastError();
}

hipError_t launch_query_finish(const QueryArgs& a, int tokens, hipStream_t s) {
  const int64_t nc = (int64_t)tokens * a.n_h * a.d_h, nr = (int64_t)tokens * a.n_h * a.d_r;
  const int c_blocks = (int)((nc + 1023) / 1024), r_blocks = (int)((nr + 1023) / 1024);
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
