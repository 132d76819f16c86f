// Partial attention of absorbed MLA decode on gfx950 MFMA (bf16 or E4M3 cache).
//
// Computes, for every piece of the split rule and every (query position, head) row,
//   s_j = softmax_scale * (q_nope . c_j + q_pe . k_pe_j)        (page "MLA deep compression",
//   lse = ln sum_j exp(s_j),  u = sum_j exp(s_j - lse) c_j      absorption + decoupled RoPE)
// over the piece's visible tokens, streaming the shared 576-wide cache rows through LDS
// once per workgroup for all of its heads (the "absorbed MQA" shape: n_h query heads
// against one shared key/value latent).
//
// Layout of the work:
//  - grid (G, row_groups); a workgroup handles up to 128 (q, head) rows of one
//    sequence piece at a time, one wave per 16 rows (16 heads of one query position).
//  - tiles of 32 tokens x 576 values in LDS (bf16), each 16-byte chunk of a row
//    placed at chunk ^ (row & 7) so that both read patterns below are free of bank
//    conflicts; two tiles in flight (direct global->LDS copies, no register staging).
//  - scores: S^T[token, head] = K[token, :] Q^T with K from LDS (A operand) and the
//    wave's queries held in registers (B operand): 18 MFMA k-steps per 16 tokens.
//  - softmax runs on the MFMA output layout: lane l owns head l%16 and 8 tokens, so
//    the running max and sum are per lane plus two cross-lane steps.
//  - latent accumulation U^T[col, head] += V^T[col, token] P^T[token, head], with V^T
//    fetched by transposing LDS reads and P^T taken straight from the score registers
//    (same lane/token assignment, no shuffles).
//  - E4M3 caches: tiles land in a staging buffer and are widened exactly to bf16 once
//    per workgroup; the per-token scale multiplies the scores and the probabilities.

#include "mla_device.h"
#include "mla_kernels.h"
#include "mla_split.h"

namespace mla {
namespace {

constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kD = kDc + kDr;           // 576 values per cached token
constexpr int kChunks = kD / 8;         // 72 sixteen-byte bf16 chunks per token
constexpr int kT = 32;                  // tokens per tile
constexpr int kTileElems = kT * kD;     // 18432 bf16 = 36 KiB
constexpr int kFp8Chunks = kD / 16;     // 36 sixteen-byte E4M3 chunks per token
constexpr int kKc = kD / 32;            // 18 k-steps of the score MFMA
constexpr int kCb = kDc / 16;           // 32 column blocks of the latent accumulator
constexpr int kMaxThreads = 512;

template <bool FP8>
struct Smem {
  bf16 tile[FP8 ? 1 : 2][kTileElems];
  unsigned char stage[FP8 ? 2 : 1][FP8 ? kT * kD : 16];
  float kvs[2][kT];
  SplitScratch split;
  Piece pieces[kMaxThreads];
};

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <bool FP8>
__global__ __launch_bounds__(kMaxThreads) void attn_partial_mfma(const AttnParams p) {
  __shared__ __attribute__((aligned(16))) Smem<FP8> sm;

  const int w = blockIdx.x;
  const int rg = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nwaves = blockDim.x >> 6;
  const int l16 = lane & 15;
  const int g = lane >> 4;

  const int row0 = rg * p.rows_per_group + wave * 16;
  const int q_pos = row0 / p.n_h;
  const int head0 = row0 - q_pos * p.n_h;
  const int q_max = (rg * p.rows_per_group + p.rows_per_group - 1) / p.n_h;

  // Per-lane LDS offsets (bf16 elements) of the two read patterns.  The swizzle
  // chunk ^ (row & 7) only changes the low 3 bits of the chunk index, so a chunk
  // 8a + r lands at 8a + (r ^ x): a few per-lane bases plus compile-time steps of 64
  // elements (8 chunks) cover every read.  Rows r and r + 16 share the swizzle.
  // Scores: token l16 (and 16 + l16), chunk 4kc + g  (kc even: r = g, odd: r = 4 + g).
  const int qk_x = l16 & 7;
  const int qk_base0 = l16 * kD + ((g ^ qk_x) * 8);
  const int qk_base1 = l16 * kD + (((4 + g) ^ qk_x) * 8);
  // Latent accumulation: rows 4g + s (s = (lane%16)/4) and 16 + 4g + s, columns
  // cb*16 + 4*(lane%4) .. +3, i.e. chunk 2cb + (lane%4)/2 (r = 2*(cb%4) + (lane%4)/2).
  const int tr_tok = 4 * g + (l16 >> 2);
  const int tr_x = tr_tok & 7;
  const int tr_q = lane & 3;
  int tr_base[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) tr_base[r] = tr_tok * kD + (((2 * r + (tr_q >> 1)) ^ tr_x) * 8) + (tr_q & 1) * 4;

  for_each_piece(p.seq_lens, p.batch, p.max_tokens, p.num_splits, w, rg == 0 ? p.split_table : nullptr,
                 &sm.split, sm.pieces, [&](const Piece& pc_lds) {
    const int b = uniform(pc_lds.b);
    const int t0 = uniform(pc_lds.t0);
    const int t1 = uniform(pc_lds.t1);
    const int slot = uniform(pc_lds.slot);
    const int L = clamp_len(p.seq_lens[b], p.max_tokens);
    const int vis_wave = max(0, L - p.s_q + q_pos + 1);
    const int wave_end = min(t1, vis_wave);
    const int wg_end = min(t1, max(0, L - p.s_q + q_max + 1));
    const int ntiles = wg_end > t0 ? (wg_end - t0 + kT - 1) / kT : 0;
    PageWindow pw;
    pw.init(p.block_table + (size_t)b * p.max_pages, p.max_pages, p.num_pages, t0 / p.page_size);

    // Queries of this wave's 16 heads: B operand fragments, k = kc*32 + 8g + j.
    bf16x8 qf[kKc];
    {
      const size_t qrow = ((size_t)b * p.s_q + q_pos) * p.n_h + head0 + l16;
      const bf16* qn = (const bf16*)p.q_nope + qrow * kDc + 8 * g;
      const bf16* qp = (const bf16*)p.q_pe + qrow * kDr + 8 * g;
#pragma unroll
      for (int kc = 0; kc < kKc; ++kc)
        qf[kc] = kc < kDc / 32 ? *(const bf16x8*)(qn + kc * 32) : *(const bf16x8*)(qp + (kc - kDc / 32) * 32);
    }

    f32x4 U[kCb];
#pragma unroll
    for (int cb = 0; cb < kCb; ++cb) U[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    float l_run = 0.f;     // running sum of the unrounded numerators (for lse)
    float l_eff = 0.f;     // E4M3: running sum of the rounded weights over their scales (divides U)

    auto tile_page = [&](int it) -> int { return pw.get((t0 + it * kT) / p.page_size); };

    // Enqueue the copies of tile `it` into buffer `buf` (this wave's share of them).
    auto issue = [&](int it, int buf) {
      const int tt = t0 + it * kT;
      const int page = uniform(tile_page(it));
      if (page < 0) return;
      const int last = min(tt + kT, wg_end) - 1 - tt;      // last valid row of the tile
      const long long slot0 = (long long)page * p.page_size + (tt % p.page_size);
      if (!FP8) {
        char* dst = (char*)sm.tile[buf];
        for (int i = wave; i < kT * kChunks / 64; i += nwaves) {
          const int f = i * 64 + lane;
          const int j = f / kChunks;
          const int lc = (f - j * kChunks) ^ (j & 7);
          const long long s = slot0 + min(j, last);
          const bf16* src = lc < kDc / 8 ? (const bf16*)p.c_kv + s * p.c_stride + lc * 8
                                         : (const bf16*)p.k_pe + s * p.k_stride + (lc - kDc / 8) * 8;
          global_to_lds16(src, dst + i * 1024);
        }
      } else {
        char* dst = (char*)sm.stage[buf];
        for (int i = wave; i < kT * kFp8Chunks / 64; i += nwaves) {
          const int f = i * 64 + lane;
          const int j = f / kFp8Chunks;
          const int fc = f - j * kFp8Chunks;
          const long long s = slot0 + min(j, last);
          const unsigned char* src = fc < kDc / 16 ? (const unsigned char*)p.c_kv + s * p.c_stride + fc * 16
                                                   : (const unsigned char*)p.k_pe + s * p.k_stride + (fc - kDc / 16) * 16;
          global_to_lds16(src, dst + i * 1024);
        }
        if (wave == nwaves - 1 && lane < kT) {
          const long long s = slot0 + min(lane, last);
          __builtin_amdgcn_global_load_lds((const void*)(p.kv_scale + s), (MLA_LDS void*)(sm.kvs[buf]), 4, 0, 0);
        }
      }
    };

    // Widen a staged E4M3 tile into the swizzled bf16 tile (whole workgroup).
    auto widen = [&](int buf) {
      const u32x4* src = (const u32x4*)sm.stage[buf];
      for (int idx = tid; idx < kT * kFp8Chunks; idx += blockDim.x) {
        const int j = idx / kFp8Chunks;
        const int fc = idx - j * kFp8Chunks;
        const u32x4 v = src[idx];
        bf16x8 lo, hi;
        bf16x2 t;
        t = e4m3x2_to_bf16<false>(v.x); lo[0] = t[0]; lo[1] = t[1];
        t = e4m3x2_to_bf16<true>(v.x);  lo[2] = t[0]; lo[3] = t[1];
        t = e4m3x2_to_bf16<false>(v.y); lo[4] = t[0]; lo[5] = t[1];
        t = e4m3x2_to_bf16<true>(v.y);  lo[6] = t[0]; lo[7] = t[1];
        t = e4m3x2_to_bf16<false>(v.z); hi[0] = t[0]; hi[1] = t[1];
        t = e4m3x2_to_bf16<true>(v.z);  hi[2] = t[0]; hi[3] = t[1];
        t = e4m3x2_to_bf16<false>(v.w); hi[4] = t[0]; hi[5] = t[1];
        t = e4m3x2_to_bf16<true>(v.w);  hi[6] = t[0]; hi[7] = t[1];
        bf16* row = sm.tile[0] + j * kD;
        *(bf16x8*)(row + ((2 * fc) ^ (j & 7)) * 8) = lo;
        *(bf16x8*)(row + ((2 * fc + 1) ^ (j & 7)) * 8) = hi;
      }
    };

    auto compute = [&](int it, int buf) {
      const int tt = t0 + it * kT;
      if (uniform(tile_page(it)) < 0) return;
      const bf16* tile = sm.tile[FP8 ? 0 : buf];

      // Scores of 32 tokens x 16 heads: s0 tokens 0..15, s1 tokens 16..31.
      f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < kKc; ++kc) {
        const int off = ((kc & 1) ? qk_base1 : qk_base0) + (kc >> 1) * 64;
        const bf16x8 a0 = *(const bf16x8*)(tile + off);
        const bf16x8 a1 = *(const bf16x8*)(tile + off + 16 * kD);
        s0 = mfma16x16x32(a0, qf[kc], s0);
        s1 = mfma16x16x32(a1, qf[kc], s1);
      }

      // Online softmax in base 2; lane owns head l16, tokens tb*16 + 4g + i.
      float x[8];
      float mx = -INFINITY;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int j = (k >> 2) * 16 + 4 * g + (k & 3);
        float v = (k < 4 ? s0[k & 3] : s1[k & 3]) * p.scale_log2;
        if (FP8) v *= sm.kvs[buf & 1][j];
        v = (tt + j < wave_end) ? v : -INFINITY;
        x[k] = v;
        mx = fmaxf(mx, v);
      }
      mx = fmaxf(mx, shfl_xor_f(mx, 16));
      mx = fmaxf(mx, shfl_xor_f(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2_fast(m_run - m_use);
      float pr[8];
      float psum = 0.f, esum = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        pr[k] = exp2_fast(x[k] - m_use);
        psum += pr[k];
      }
      if (FP8) {
#pragma unroll
        for (int k = 0; k < 8; ++k) pr[k] *= sm.kvs[buf & 1][(k >> 2) * 16 + 4 * g + (k & 3)];
      }
      bf16x8 pf;
      {
        bf16x2 t;
        t = pack_bf16(pr[0], pr[1]); pf[0] = t[0]; pf[1] = t[1];
        t = pack_bf16(pr[2], pr[3]); pf[2] = t[0]; pf[3] = t[1];
        t = pack_bf16(pr[4], pr[5]); pf[4] = t[0]; pf[5] = t[1];
        t = pack_bf16(pr[6], pr[7]); pf[6] = t[0]; pf[7] = t[1];
      }
      if (FP8) {
        // U is divided by the sum of the weights that reach the accumulation (the bf16
        // rounding of p * scale) over the tokens' scales, so numerator and denominator
        // agree; the lse keeps the sum of the unrounded numerators.
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float r = fminf(__builtin_amdgcn_rcpf(sm.kvs[buf & 1][(k >> 2) * 16 + 4 * g + (k & 3)]), 3.0e38f);
          esum = __builtin_fmaf((float)pf[k], r, esum);
        }
      }
      l_run = l_run * alpha + psum;
      l_eff = l_eff * alpha + (FP8 ? esum : psum);
      m_run = m_new;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int cb = 0; cb < kCb; ++cb) U[cb] *= alpha;
      }

      // U^T[cols, heads] += V^T[cols, tokens] P^T[tokens, heads].
#pragma unroll
      for (int cb = 0; cb < kCb; ++cb) {
        const int off = tr_base[cb & 3] + (cb >> 2) * 64;
        const bf16x4 va = lds_read_tr16(tile + off);
        const bf16x4 vb = lds_read_tr16(tile + off + 16 * kD);
        U[cb] = mfma16x16x32(concat4(va, vb), pf, U[cb]);
      }
    };

    if (ntiles > 0) issue(0, 0);
    for (int it = 0; it < ntiles; ++it) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (FP8) {
        if (uniform(tile_page(it)) >= 0) widen(it & 1);
        __syncthreads();
      }
      if (it + 1 < ntiles) issue(it + 1, (it + 1) & 1);
      compute(it, it & 1);
    }

    // Split epilogue: normalized u and the piece's log-sum-exp (natural log).
    float l_tot = l_run + shfl_xor_f(l_run, 16);
    l_tot += shfl_xor_f(l_tot, 32);
    float l_div = l_eff + shfl_xor_f(l_eff, 16);
    l_div += shfl_xor_f(l_div, 32);
    const float inv = l_div > 0.f ? 1.f / l_div : 0.f;
    const float lse = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    const size_t orow = ((size_t)slot * p.s_q + q_pos) * p.n_h + head0 + l16;
    if (g == 0) p.part_lse[orow] = lse;
    bf16* up = (bf16*)p.part_u + orow * kDc + 4 * g;
#pragma unroll
    for (int cb = 0; cb < kCb; ++cb) *(bf16x4*)(up + cb * 16) = to_bf16x4(U[cb] * inv);
    __syncthreads();
  });
}

}  // namespace

hipError_t launch_attn_fp8_v0(const AttnParams& p, hipStream_t stream) {
  const int rows = p.s_q * p.n_h;
  const int row_groups = rows / p.rows_per_group;
  dim3 grid(p.num_splits, row_groups);
  dim3 block(64 * (p.rows_per_group / 16));
  return launch_attention_kernel(attn_partial_mfma<true>, grid, block, stream, p);
}

}  // namespace mla
