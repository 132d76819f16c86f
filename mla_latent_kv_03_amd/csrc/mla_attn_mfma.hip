// Partial attention of absorbed MLA decode on gfx950 MFMA, bf16 latent cache.
//
// For every piece of the split rule and every head of one query position:
//   s_j = softmax_scale * (q_nope . c_j + q_pe . k_pe_j)         (page "MLA deep compression":
//   lse = ln sum_j exp(s_j),   u = sum_j exp(s_j - lse) c_j       absorbed scores + decoupled RoPE,
//                                                                 latent accumulation u_i)
// All heads share one 576-wide key row and its first 512 values are also the value
// row (the "absorbed MQA" shape), so each cached row is streamed through LDS once per
// workgroup and consumed by every head of the workgroup.
//
// Work split: a workgroup covers 16*HB heads (HB head blocks of 16) of one query
// position for one piece.  Its waves have two roles that run one tile apart:
//  - S-waves (one per head block) hold the block's queries in registers, compute
//    S^T[token, head] = K Q^T on 16x16x32 MFMAs, run the online softmax on the MFMA
//    output layout (lane l owns head l%16 and 8 tokens), and publish the bf16
//    probabilities and the rescale factors of tile t in LDS;
//  - U-waves (four, 128 latent columns each) accumulate U^T[col, head] += V^T P^T for
//    ALL head blocks from tile t-1, so every transposed LDS read of V feeds HB MFMAs.
// The two roles share each SIMD (one of each), so one's softmax overlaps the other's
// MFMAs.  Tiles of 32 tokens x 576 bf16 sit in a 4-deep LDS ring filled by direct
// global->LDS copies issued by the U-waves two tiles ahead; every 16-byte chunk of a
// row is stored at chunk ^ (row & 7), which keeps both read patterns free of bank
// conflicts.  The softmax keeps a lazily updated maximum: it is raised (and the
// accumulators rescaled) only when a tile's maximum exceeds it by more than 2^8.

#include "mla_device.h"
#include "mla_kernels.h"
#include "mla_split.h"

namespace mla {
namespace {

constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kD = kDc + kDr;              // 576 values per cached token
constexpr int kChunks = kD / 8;            // 72 sixteen-byte chunks per token
constexpr int kT = 32;                     // tokens per tile
constexpr int kTileElems = kT * kD;        // 18432 bf16 = 36 KiB
constexpr int kRing = 4;                   // tiles resident in LDS
constexpr int kKc = kD / 32;               // 18 k-steps of the score MFMA
constexpr int kUWaves = 8;                 // latent-accumulation waves (64 columns each)
constexpr int kUCb = kDc / kUWaves / 16;   // 4 column blocks of 16 per U-wave
constexpr int kCopies = kT * kChunks / 64;                // 36 wave-wide 1 KiB copies per tile
constexpr float kTau = 8.f;                // lazy-maximum slack (log2 units)
constexpr int kQkAhead = 3;                // score k-steps whose K fragments are in flight

static_assert(kT * kChunks % 64 == 0, "a tile is a whole number of 1 KiB copies");

template <int HB>
struct Smem {
  bf16 tile[kRing][kTileElems];
  bf16x8 prob[2][HB][64];       // S-wave lane l's 8 probabilities, B-operand layout
  float alpha[2][16][HB];       // rescale factor of head (block hb, row i)
  float lsum[16][HB];           // final softmax denominators
};

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Workgroup barrier that orders LDS traffic only.  __syncthreads() would also drain
// every outstanding global access, including the direct-to-LDS copies of the tiles
// being prefetched; here each wave's own LDS reads/writes complete (lgkmcnt(0)) and
// the tile copies are waited for explicitly, per tile, with wait_vmcnt<>().
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt left alone
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // gfx9 s_waitcnt: vmcnt in bits [3:0] and [15:14]; expcnt (7) and lgkmcnt (15) left alone.
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// PACKED: k_pe == c_kv + 512 with one stride, i.e. one [c | k_pe] row per pool slot.
template <int HB, bool PACKED>
__global__ __launch_bounds__(64 * (HB + kUWaves)) void attn_partial_split(const AttnParams p) {
  __shared__ __attribute__((aligned(16))) Smem<HB> sm;

  const int w = blockIdx.x;
  const int rg = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const bool s_role = wave < HB;
  const int uw = wave - HB;                        // U-wave index (valid when !s_role)
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int groups_per_q = p.n_h / (16 * HB);
  const int q_pos = rg / groups_per_q;
  const int head_base = (rg - q_pos * groups_per_q) * 16 * HB;

  int32_t* table = (rg == 0 && wave == 0) ? p.split_table : nullptr;

  // Tile copies are issued by the U-waves: copy c (c = 0..35, the 1 KiB block c of the
  // tile) by U-wave c % 8, so 4 or 5 per wave and per tile; a wave stalled on a copy
  // leaves its SIMD to the other two waves.  For packed [c | k_pe] rows a copy is one
  // scalar base plus a per-lane offset fixed for the whole kernel: block c is chunk
  // f = 64c + lane, tile row j = f / 72, stored chunk f % 72 holding logical chunk
  // (f % 72) ^ (j & 7).
  constexpr int nwaves = kUWaves;
  constexpr int kMaxCopiesPerWave = (kCopies + nwaves - 1) / nwaves;   // 5
  const int cw = s_role ? 0 : uw;                                      // copy-wave index
  const int my_copies = s_role ? 0 : (kCopies - uw + nwaves - 1) / nwaves;
  uint32_t copy_off[kMaxCopiesPerWave];
#pragma unroll
  for (int k = 0; k < kMaxCopiesPerWave; ++k) {
    const int f = (cw + k * nwaves) * 64 + lane;
    const int j = f / kChunks;
    const int lc = (f - j * kChunks) ^ (j & 7);
    copy_off[k] = PACKED ? (uint32_t)((j * p.c_stride + lc * 8) * 2) : 0u;
  }

  if (s_role) {
    // ====================================================================== S-waves
    // LDS read offsets (bf16 elements).  A chunk 8a + r of a row lands at 8a + (r ^ x),
    // x = row & 7, so two per-lane bases plus compile-time steps of 64 elements cover
    // every read; rows r and r + 16 share the swizzle.  Token l16 (and 16 + l16),
    // chunk 4kc + g (kc even: r = g, odd: r = 4 + g).
    const int qk_x = l16 & 7;
    const int qk_base0 = l16 * kD + ((g ^ qk_x) * 8);
    const int qk_base1 = l16 * kD + (((4 + g) ^ qk_x) * 8);
    for_each_piece_wave(p.seq_lens, p.batch, p.max_tokens, p.num_splits, w, table, [&](const Piece& pc) {
    const int b = pc.b;
    const int t0 = pc.t0;
    const int slot = pc.slot;
    const int L = clamp_len(p.seq_lens[b], p.max_tokens);
    const int end = min(pc.t1, max(0, L - p.s_q + q_pos + 1));      // visible tokens of this piece
    const int ntiles = end > t0 ? (end - t0 + kT - 1) / kT : 0;
    PageWindow pw;
    pw.init(p.block_table + (size_t)b * p.max_pages, p.max_pages, p.num_pages, t0 / p.page_size);
    auto tile_page = [&](int it) -> int { return pw.get((t0 + it * kT) / p.page_size); };
    const size_t row_base = ((size_t)slot * p.s_q + q_pos) * p.n_h + head_base;
    // Enqueue this wave's copies of tile `it`; false if the tile's page is invalid.
    auto issue = [&](int it) {
      const int page = tile_page(it);
      if (page < 0) return false;
      if (my_copies == 0) return true;
      const int tt = t0 + it * kT;
      const int last = min(tt + kT, end) - 1 - tt;            // last row of the tile to read
      const long long slot0 = (long long)page * p.page_size + (tt % p.page_size);
      char* dst = (char*)sm.tile[it % kRing];
      if (PACKED) {
        const char* base = (const char*)p.c_kv + slot0 * p.c_stride * 2;
#pragma unroll
        for (int k = 0; k < kMaxCopiesPerWave; ++k) {
          if (k >= my_copies) break;
          const int c = cw + k * nwaves;
          uint32_t off = copy_off[k];
          if (last < kT - 1) {                                  // ragged tile: rows past `last` re-read it
            const int j = (c * 64 + lane) / kChunks;
            if (j > last) off -= (uint32_t)(j - last) * (uint32_t)p.c_stride * 2u;
          }
          global_to_lds16(base + off, dst + c * 1024);
        }
      } else {
#pragma unroll
        for (int k = 0; k < kMaxCopiesPerWave; ++k) {
          if (k >= my_copies) break;
          const int c = cw + k * nwaves;
          const int f = c * 64 + lane;
          const int j = f / kChunks;
          const int lc = (f - j * kChunks) ^ (j & 7);
          const long long sl = slot0 + min(j, last);
          const bf16* src = lc < kDc / 8 ? (const bf16*)p.c_kv + sl * p.c_stride + lc * 8
                                         : (const bf16*)p.k_pe + sl * p.k_stride + (lc - kDc / 8) * 8;
          global_to_lds16(src, dst + c * 1024);
        }
      }
      return true;
    };
    // Wait until this wave's copies of tile `it` have landed, leaving those of tile it+1
    // in flight (vector memory operations complete in order).
    auto wait_tile = [&](bool next_in_flight) {
      switch (next_in_flight ? my_copies : 0) {
        case 4: wait_vmcnt<4>(); break;
        case 5: wait_vmcnt<5>(); break;
        case 6: wait_vmcnt<6>(); break;
        case 7: wait_vmcnt<7>(); break;
        case 8: wait_vmcnt<8>(); break;
        default: wait_vmcnt<0>(); break;
      }
    };
    static_assert((kCopies + kUWaves - 1) / kUWaves <= 8, "wait_tile covers at most 8 copies per wave");
      const int head = head_base + wave * 16 + l16;
      bf16x8 qf[kKc];
      {
        const size_t qrow = ((size_t)b * p.s_q + q_pos) * p.n_h + head;
        const bf16* qn = (const bf16*)p.q_nope + qrow * kDc + 8 * g;
        const bf16* qp = (const bf16*)p.q_pe + qrow * kDr + 8 * g;
#pragma unroll
        for (int kc = 0; kc < kKc; ++kc)
          qf[kc] = kc < kDc / 32 ? *(const bf16x8*)(qn + kc * 32) : *(const bf16x8*)(qp + (kc - kDc / 32) * 32);
      }
      float m_used = -INFINITY;
      float l_part = 0.f;
      wait_vmcnt<0>();
      if (ntiles > 0) issue(0);
      bool issued_next = ntiles > 1 && issue(1);
      for (int it = 0; it <= ntiles; ++it) {
        wait_tile(issued_next);
        lds_barrier();
        issued_next = it + 2 < ntiles && issue(it + 2);
        if (it == ntiles || tile_page(it) < 0) continue;
        const int tt = t0 + it * kT;
        const bf16* tile = sm.tile[it % kRing];
        // Scores, software-pipelined: the K fragments of step kc + kQkAhead are read
        // from LDS before the two MFMAs of step kc issue.
        // Four independent accumulation chains (tokens 0-15 / 16-31 x even / odd k-steps).
        f32x4 sc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        bf16x8 ka[kQkAhead + 1][2];
#pragma unroll
        for (int kc = 0; kc < kQkAhead; ++kc) {
          const int off = ((kc & 1) ? qk_base1 : qk_base0) + (kc >> 1) * 64;
          ka[kc][0] = *(const bf16x8*)(tile + off);
          ka[kc][1] = *(const bf16x8*)(tile + off + 16 * kD);
        }
#pragma unroll
        for (int kc = 0; kc < kKc; ++kc) {
          const int nk = kc + kQkAhead;
          if (nk < kKc) {
            const int off = ((nk & 1) ? qk_base1 : qk_base0) + (nk >> 1) * 64;
            ka[nk % (kQkAhead + 1)][0] = *(const bf16x8*)(tile + off);
            ka[nk % (kQkAhead + 1)][1] = *(const bf16x8*)(tile + off + 16 * kD);
          }
          __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of this step's MFMAs
          sc[kc & 1] = mfma16x16x32(ka[kc % (kQkAhead + 1)][0], qf[kc], sc[kc & 1]);
          sc[2 + (kc & 1)] = mfma16x16x32(ka[kc % (kQkAhead + 1)][1], qf[kc], sc[2 + (kc & 1)]);
          __builtin_amdgcn_sched_barrier(0);
        }
        const f32x4 s0 = sc[0] + sc[1], s1 = sc[2] + sc[3];
        // online softmax, base 2; lane owns head l16, tokens (k/4)*16 + 4g + k%4
        float x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = (k < 4 ? s0[k & 3] : s1[k & 3]) * p.scale_log2;
        if (tt + kT > end) {                       // ragged last tile: hide tokens past the end
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (tt + (k >> 2) * 16 + 4 * g + (k & 3) >= end) x[k] = -INFINITY;
        }
        float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        mx = max_xor16(mx);
        mx = max_xor32(mx);
        const bool raise = mx > m_used + kTau;
        const float m_new = raise ? mx : m_used;
        const float alpha = raise ? exp2_fast(m_used - m_new) : 1.f;
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        float pr[8];
        float psum = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          pr[k] = exp2_fast(x[k] - m_use);
          psum += pr[k];
        }
        l_part = l_part * alpha + psum;
        m_used = m_new;
        bf16x8 pf;
#pragma unroll
        for (int k = 0; k < 8; k += 2) {
          const bf16x2 t = pack_bf16(pr[k], pr[k + 1]);
          pf[k] = t[0];
          pf[k + 1] = t[1];
        }
        sm.prob[it & 1][wave][lane] = pf;
        if (g == 0) sm.alpha[it & 1][l16][wave] = alpha;
      }
      const float l_tot = sum_xor32(sum_xor16(l_part));
      if (g == 0) {
        sm.lsum[l16][wave] = l_tot;
        p.part_lse[row_base + wave * 16 + l16] = l_tot > 0.f ? (m_used + __log2f(l_tot)) * kLn2 : -INFINITY;
      }
      __syncthreads();
      __syncthreads();
    });
  } else {
    // ====================================================================== U-waves
    // Transposed V reads: tokens 4g + (l16/4) (and +16), columns 64*uw + 16cb +
    // 4*(lane%4) .. +3, i.e. chunk 8uw + 2cb + (lane%4)/2 (r = 2*(cb%4) + (lane%4)/2).
    const int tr_tok = 4 * g + (l16 >> 2);
    const int tr_x = tr_tok & 7;
    const int tr_q = lane & 3;
    int tr_base[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      tr_base[r] = tr_tok * kD + (((2 * r + (tr_q >> 1)) ^ tr_x) * 8) + (tr_q & 1) * 4 + uw * (kDc / kUWaves);
    for_each_piece_wave(p.seq_lens, p.batch, p.max_tokens, p.num_splits, w, table, [&](const Piece& pc) {
    const int b = pc.b;
    const int t0 = pc.t0;
    const int slot = pc.slot;
    const int L = clamp_len(p.seq_lens[b], p.max_tokens);
    const int end = min(pc.t1, max(0, L - p.s_q + q_pos + 1));      // visible tokens of this piece
    const int ntiles = end > t0 ? (end - t0 + kT - 1) / kT : 0;
    PageWindow pw;
    pw.init(p.block_table + (size_t)b * p.max_pages, p.max_pages, p.num_pages, t0 / p.page_size);
    auto tile_page = [&](int it) -> int { return pw.get((t0 + it * kT) / p.page_size); };
    const size_t row_base = ((size_t)slot * p.s_q + q_pos) * p.n_h + head_base;
    // Enqueue this wave's copies of tile `it`; false if the tile's page is invalid.
    auto issue = [&](int it) {
      const int page = tile_page(it);
      if (page < 0) return false;
      if (my_copies == 0) return true;
      const int tt = t0 + it * kT;
      const int last = min(tt + kT, end) - 1 - tt;            // last row of the tile to read
      const long long slot0 = (long long)page * p.page_size + (tt % p.page_size);
      char* dst = (char*)sm.tile[it % kRing];
      if (PACKED) {
        const char* base = (const char*)p.c_kv + slot0 * p.c_stride * 2;
#pragma unroll
        for (int k = 0; k < kMaxCopiesPerWave; ++k) {
          if (k >= my_copies) break;
          const int c = cw + k * nwaves;
          uint32_t off = copy_off[k];
          if (last < kT - 1) {                                  // ragged tile: rows past `last` re-read it
            const int j = (c * 64 + lane) / kChunks;
            if (j > last) off -= (uint32_t)(j - last) * (uint32_t)p.c_stride * 2u;
          }
          global_to_lds16(base + off, dst + c * 1024);
        }
      } else {
#pragma unroll
        for (int k = 0; k < kMaxCopiesPerWave; ++k) {
          if (k >= my_copies) break;
          const int c = cw + k * nwaves;
          const int f = c * 64 + lane;
          const int j = f / kChunks;
          const int lc = (f - j * kChunks) ^ (j & 7);
          const long long sl = slot0 + min(j, last);
          const bf16* src = lc < kDc / 8 ? (const bf16*)p.c_kv + sl * p.c_stride + lc * 8
                                         : (const bf16*)p.k_pe + sl * p.k_stride + (lc - kDc / 8) * 8;
          global_to_lds16(src, dst + c * 1024);
        }
      }
      return true;
    };
    // Wait until this wave's copies of tile `it` have landed, leaving those of tile it+1
    // in flight (vector memory operations complete in order).
    auto wait_tile = [&](bool next_in_flight) {
      switch (next_in_flight ? my_copies : 0) {
        case 4: wait_vmcnt<4>(); break;
        case 5: wait_vmcnt<5>(); break;
        case 6: wait_vmcnt<6>(); break;
        case 7: wait_vmcnt<7>(); break;
        case 8: wait_vmcnt<8>(); break;
        default: wait_vmcnt<0>(); break;
      }
    };
    static_assert((kCopies + kUWaves - 1) / kUWaves <= 8, "wait_tile covers at most 8 copies per wave");
      f32x4 acc[kUCb][HB];
#pragma unroll
      for (int cb = 0; cb < kUCb; ++cb)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) acc[cb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
      wait_vmcnt<0>();
      if (ntiles > 0) issue(0);
      bool issued_next = ntiles > 1 && issue(1);
      for (int it = 0; it <= ntiles; ++it) {
        wait_tile(issued_next);
        lds_barrier();
        issued_next = it + 2 < ntiles && issue(it + 2);
        const int t = it - 1;
        if (it == 0 || tile_page(t) < 0) continue;
        const bf16* tile = sm.tile[t % kRing];
        float al[HB];
        bool any = false;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          al[hb] = sm.alpha[t & 1][l16][hb];
          any |= al[hb] != 1.f;
        }
        if (__any(any)) {
#pragma unroll
          for (int cb = 0; cb < kUCb; ++cb)
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) acc[cb][hb] *= al[hb];
        }
        bf16x8 pf[HB];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) pf[hb] = sm.prob[t & 1][hb][lane];
        // Latent accumulation: all transposed V fragments of the tile are read
        // first (they complete in order, so each group of HB MFMAs waits only for its
        // own fragment), then U^T += V^T P^T for every head block.
        bf16x8 vf[kUCb];
#pragma unroll
        for (int cb = 0; cb < kUCb; ++cb) {
          const int off = tr_base[cb & 3] + (cb >> 2) * 64;
          vf[cb] = concat4(lds_read_tr16(tile + off), lds_read_tr16(tile + off + 16 * kD));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int cb = 0; cb < kUCb; ++cb) {
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) acc[cb][hb] = mfma16x16x32(vf[cb], pf[hb], acc[cb][hb]);
        }
      }
      __syncthreads();
      float inv[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        const float ls = sm.lsum[l16][hb];
        inv[hb] = ls > 0.f ? 1.f / ls : 0.f;
      }
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        float* up = p.part_u + (row_base + hb * 16 + l16) * kDc + uw * (kDc / kUWaves) + 4 * g;
#pragma unroll
        for (int cb = 0; cb < kUCb; ++cb) *(f32x4*)(up + cb * 16) = acc[cb][hb] * inv[hb];
      }
      __syncthreads();
    });
  }
}

}  // namespace

int attn_heads_per_group(int n_h) { return n_h >= 64 ? 64 : n_h; }

hipError_t launch_attn_mfma(const AttnParams& p, bool fp8, hipStream_t stream) {
  if (fp8) return launch_attn_fp8_v0(p, stream);
  const int hg = attn_heads_per_group(p.n_h);
  const int HB = hg / 16;
  dim3 grid(p.num_splits, p.s_q * (p.n_h / hg));
  dim3 block(64 * (HB + kUWaves));
  const bool packed = p.packed_rows != 0;
#define MLA_LAUNCH(hb)                                                                          \
  if (packed)                                                                                   \
    hipLaunchKernelGGL((attn_partial_split<hb, true>), grid, block, 0, stream, p);              \
  else                                                                                          \
    hipLaunchKernelGGL((attn_partial_split<hb, false>), grid, block, 0, stream, p);
  switch (HB) {
    case 1: MLA_LAUNCH(1) break;
    case 2: MLA_LAUNCH(2) break;
    case 4: MLA_LAUNCH(4) break;
    default: return hipErrorInvalidValue;
  }
#undef MLA_LAUNCH
  return hipGetLastError();
}

}  // namespace mla
