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
// position for one piece, with two kinds of waves:
//  - S-waves (one per head block) hold the block's queries in registers and compute
//    S^T[token, head] = K Q^T on 16x16x32 MFMAs.  The online softmax runs on the MFMA
//    output layout (lane l owns head l%16 and 8 tokens) one tile behind: the softmax
//    of tile t-1 is interleaved with the score MFMAs of tile t, so its VALU and
//    transcendental work hides under the matrix pipe.  Probabilities (bf16) and
//    rescale factors go to LDS.
//  - U-waves (eight, one 64-column slice of the latent each) accumulate
//    U^T[col, head] += V^T P^T for ALL head blocks from tile t-2, so every transposed
//    LDS read of V feeds HB MFMAs.
// Each SIMD runs one S-wave and two U-waves.  Tiles of 32 tokens x 576 bf16 sit in a
// 4-deep LDS ring stored slice-major: nine 4 KiB slices (eight latent slices of 64
// values, then the RoPE part), each 32 rows of 128 bytes in which 16-byte chunk c of
// row r is stored at c ^ (r & 7) (conflict-free for both read patterns).  Slice k is
// read only by U-wave k (and by the S-waves two iterations earlier), so U-wave k
// refills its own slice with the tile two ahead as soon as its own reads of the
// slice have completed, without waiting for the other waves; the S-waves refill the
// RoPE slice.  The softmax keeps a lazily updated maximum: it is raised (and the
// accumulators rescaled) only when a tile's maximum exceeds it by more than 2^8.

#include <type_traits>

#include "mla_device.h"
#include "mla_kernels.h"
#include "mla_split.h"

namespace mla {
namespace {

constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kD = kDc + kDr;                        // 576 values per cached token
constexpr int kT = 32;                               // tokens per tile
constexpr int kSlices = kD / 64;                     // 8 latent slices + 1 RoPE slice
constexpr int kRowBytes = 128;                       // one row of one slice
constexpr int kSliceBytes = kT * kRowBytes;          // 4 KiB
constexpr int kTileBytes = kSlices * kSliceBytes;    // 36 KiB
constexpr int kCopiesPerSlice = kSliceBytes / 1024;  // wave-wide 16-byte-per-lane copies
constexpr int kRing = 4;                             // tiles resident in LDS
constexpr int kKc = kD / 32;                         // 18 k-steps of the score MFMA
constexpr int kUWaves = kDc / 64;                    // one latent slice per U-wave
constexpr int kUCb = 4;                              // 16-column blocks per U-wave
constexpr float kTau = 8.f;                          // lazy-maximum slack (log2 units)
constexpr int kQkAhead = 2;                          // score k-steps whose K fragments are in flight

static_assert(kCopiesPerSlice == 4, "a slice is four 1 KiB copies of 8 rows");

template <int HB>
struct Smem {
  unsigned char tile[kRing][kTileBytes];
  bf16x8 prob[2][HB][64];       // S-wave lane l's 8 probabilities, B-operand layout
  float alpha[2][16][HB];       // rescale factor of head (block hb, row i)
  float lsum[16][HB];           // final softmax denominators
};

// Copy c of a tile (c = 0 .. 35) fills LDS bytes [1024 c, 1024 c + 1024): rows
// 8 (c % 4) .. +7 of slice c / 4.  Lane l carries row 8 (c % 4) + l / 8 and stored
// chunk l % 8, which holds logical chunk (l % 8) ^ (l / 8) of the slice.
__device__ __forceinline__ int copy_row(int c, int lane) { return 8 * (c & 3) + (lane >> 3); }
__device__ __forceinline__ int copy_chunk(int c, int lane) {   // 16-byte chunk of the 576-wide row
  return 8 * (c >> 2) + ((lane & 7) ^ (lane >> 3));
}

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

__device__ __forceinline__ void wait_lds() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // gfx9 s_waitcnt: vmcnt in bits [3:0] and [15:14]; expcnt (7) and lgkmcnt (15) left alone.
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Wait until at most N of this wave's vector memory operations are outstanding.
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  switch (n) {
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 4: wait_vmcnt<4>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

// Enqueue the N copies cidx[] of one tile (first token tt, stored in `page`) into the
// LDS tile `dst`.  Rows at or past `end` re-read the tile's last visible row, so no
// byte past the piece is fetched.  poff[] are the per-lane byte offsets of the copies
// in a packed [c | k_pe] row layout.
template <bool PACKED, int N>
__device__ __forceinline__ void issue_copies(const AttnParams& p, const int (&cidx)[N], const uint32_t (&poff)[N],
                                             int page, int tt, int end, unsigned char* dst) {
  const int lane = threadIdx.x & 63;
  const int last = min(tt + kT, end) - 1 - tt;   // last row of the tile to read
  const long long slot0 = (long long)page * p.page_size + (tt % p.page_size);
  if (PACKED) {
    const char* base = (const char*)p.c_kv + slot0 * p.c_stride * 2;
#pragma unroll
    for (int k = 0; k < N; ++k) {
      uint32_t off = poff[k];
      if (last < kT - 1) {
        const int j = copy_row(cidx[k], lane);
        if (j > last) off -= (uint32_t)(j - last) * (uint32_t)p.c_stride * 2u;
      }
      global_to_lds16(base + off, dst + cidx[k] * 1024);
    }
  } else {
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const int c = cidx[k];
      const long long sl = slot0 + min(copy_row(c, lane), last);
      const int lc = copy_chunk(c, lane);
      const bf16* src = lc < kDc / 8 ? (const bf16*)p.c_kv + sl * p.c_stride + lc * 8
                                     : (const bf16*)p.k_pe + sl * p.k_stride + (lc - kDc / 8) * 8;
      global_to_lds16(src, dst + c * 1024);
    }
  }
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// PACKED: k_pe == c_kv + 512 with one stride, i.e. one [c | k_pe] row per pool slot.
template <int HB, bool PACKED>
__global__ __launch_bounds__(64 * (HB + kUWaves)) void attn_partial_split(const AttnParams p) {
  __shared__ __attribute__((aligned(16))) Smem<HB> sm;

  const int w = blockIdx.x;
  const int rg = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int groups_per_q = p.n_h / (16 * HB);
  const int q_pos = rg / groups_per_q;
  const int head_base = (rg - q_pos * groups_per_q) * 16 * HB;

  int32_t* table = (rg == 0 && wave == 0) ? p.split_table : nullptr;

  // Shared piece bookkeeping: visible end, tile count and the page lookups.
  struct PieceInfo {
    int t0, end, ntiles;
    size_t row_base;
  };
  auto piece_info = [&](const Piece& pc) {
    PieceInfo pi;
    const int L = clamp_len(p.seq_lens[pc.b], p.max_tokens);
    pi.t0 = pc.t0;
    pi.end = min(pc.t1, max(0, L - p.s_q + q_pos + 1));   // visible tokens of this piece
    pi.ntiles = pi.end > pc.t0 ? (pi.end - pc.t0 + kT - 1) / kT : 0;
    pi.row_base = ((size_t)pc.slot * p.s_q + q_pos) * p.n_h + head_base;
    return pi;
  };

  if (wave < HB) {
    // ====================================================================== S-waves
    // RoPE-slice copies of this wave: copies 32 + wave + k * HB.
    constexpr int kSN = kCopiesPerSlice / HB;
    int cidx[kSN];
    uint32_t poff[kSN];
#pragma unroll
    for (int k = 0; k < kSN; ++k) {
      cidx[k] = 8 * kCopiesPerSlice + wave + k * HB;
      poff[k] = PACKED ? (uint32_t)((copy_row(cidx[k], lane) * p.c_stride + copy_chunk(cidx[k], lane) * 8) * 2) : 0u;
    }
    // K fragment of k-step kc for token row r (r = l16 or l16 + 16): logical chunk
    // 4 kc + g = slice kc / 2, in-slice chunk 4 (kc % 2) + g.
    const int qk_x = l16 & 7;
    const int qk_b0 = l16 * kRowBytes + ((g ^ qk_x) << 4);
    const int qk_b1 = l16 * kRowBytes + (((4 + g) ^ qk_x) << 4);
    for_each_piece_wave(p.seq_lens, p.batch, p.max_tokens, p.num_splits, w, table, first_lens(p.seq_lens, p.batch, p.max_tokens), [&](const Piece& pc) {
      const PieceInfo pi = piece_info(pc);
      PageWindow pw;
      pw.init(p.block_table + (size_t)pc.b * p.max_pages, p.max_pages, p.num_pages, pi.t0 / p.page_size);
      auto tile_page = [&](int it) -> int { return pw.get((pi.t0 + it * kT) / p.page_size); };
      auto issue = [&](int it) {
        const int page = tile_page(it);
        if (page < 0) return false;
        issue_copies<PACKED, kSN>(p, cidx, poff, page, pi.t0 + it * kT, pi.end, sm.tile[it % kRing]);
        return true;
      };
      const int head = head_base + wave * 16 + l16;
      bf16x8 qf[kKc];
      {
        const size_t qrow = ((size_t)pc.b * p.s_q + q_pos) * p.n_h + head;
        const bf16* qn = (const bf16*)p.q_nope + qrow * kDc + 8 * g;
        const bf16* qp = (const bf16*)p.q_pe + qrow * kDr + 8 * g;
#pragma unroll
        for (int kc = 0; kc < kKc; ++kc)
          qf[kc] = kc < kDc / 32 ? *(const bf16x8*)(qn + kc * 32) : *(const bf16x8*)(qp + (kc - kDc / 32) * 32);
      }
      float m_used = -INFINITY;
      float l_part = 0.f;
      float x[8];           // base-2 scores of the tile awaiting its softmax
      bool prev = false;    // x holds a tile (it - 1)
      wait_vmcnt<0>();
      const int ntiles = pi.ntiles;
      if (ntiles > 0) issue(0);
      bool issued_next = ntiles > 1 && issue(1);

      // One iteration: score MFMAs of tile `it` (QK) interleaved with the softmax of
      // the previous tile (SM), whose probabilities go to buffer (it - 1) & 1.
      auto step = [&](auto qk_tag, auto sm_tag, int it) {
        constexpr bool QK = decltype(qk_tag)::value;
        constexpr bool SM = decltype(sm_tag)::value;
        const unsigned char* tile = sm.tile[it % kRing];
        f32x4 sc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        bf16x8 ka[kQkAhead + 1][2];
        auto kfrag = [&](int kc, int r) {
          const int off = ((kc & 1) ? qk_b1 : qk_b0) + (kc >> 1) * kSliceBytes + r * 16 * kRowBytes;
          return *(const bf16x8*)(tile + off);
        };
        if (QK) {
#pragma unroll
          for (int kc = 0; kc < kQkAhead; ++kc) {
            ka[kc][0] = kfrag(kc, 0);
            ka[kc][1] = kfrag(kc, 1);
          }
        }
        float mx = 0.f, alpha = 1.f, m_use = 0.f;
#pragma unroll
        for (int kc = 0; kc < kKc; ++kc) {
          if (QK) {
            const int nk = kc + kQkAhead;
            if (nk < kKc) {
              ka[nk % (kQkAhead + 1)][0] = kfrag(nk, 0);
              ka[nk % (kQkAhead + 1)][1] = kfrag(nk, 1);
            }
            __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of this step's MFMAs
            sc[kc & 1] = mfma16x16x32(ka[kc % (kQkAhead + 1)][0], qf[kc], sc[kc & 1]);
            sc[2 + (kc & 1)] = mfma16x16x32(ka[kc % (kQkAhead + 1)][1], qf[kc], sc[2 + (kc & 1)]);
          }
          if (SM) {
            // Softmax of the previous tile, spread over the k-steps.
            if (kc == 1) {
              mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
            } else if (kc == 2) {
              mx = max_xor16(mx);
            } else if (kc == 3) {
              mx = max_xor32(mx);
            } else if (kc == 4) {
              const bool raise = mx > m_used + kTau;
              const float m_new = raise ? mx : m_used;
              alpha = raise ? exp2_fast(m_used - m_new) : 1.f;
              m_use = m_new == -INFINITY ? 0.f : m_new;
              m_used = m_new;
            } else if (kc >= 5 && kc <= 8) {
              const int k = 2 * (kc - 5);
              x[k] = exp2_fast(x[k] - m_use);
              x[k + 1] = exp2_fast(x[k + 1] - m_use);
            } else if (kc == 9) {
              const float psum = ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
              l_part = l_part * alpha + psum;
            } else if (kc == 10) {
              bf16x8 pf;
#pragma unroll
              for (int k = 0; k < 8; k += 2) {
                const bf16x2 t = pack_bf16(x[k], x[k + 1]);
                pf[k] = t[0];
                pf[k + 1] = t[1];
              }
              sm.prob[(it - 1) & 1][wave][lane] = pf;
              if (g == 0) sm.alpha[(it - 1) & 1][l16][wave] = alpha;
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (QK) {
          const f32x4 s0 = sc[0] + sc[1], s1 = sc[2] + sc[3];
          // lane owns head l16, tokens (k / 4) * 16 + 4 g + k % 4
#pragma unroll
          for (int k = 0; k < 8; ++k) x[k] = (k < 4 ? s0[k & 3] : s1[k & 3]) * p.scale_log2;
          const int tt = pi.t0 + it * kT;
          if (tt + kT > pi.end) {                     // ragged last tile: hide tokens past the end
#pragma unroll
            for (int k = 0; k < 8; ++k)
              if (tt + (k >> 2) * 16 + 4 * g + (k & 3) >= pi.end) x[k] = -INFINITY;
          }
        }
      };

      for (int it = 0; it <= ntiles + 1; ++it) {
        wait_vmcnt_upto(issued_next ? kSN : 0);   // this wave's copies of tile `it` have landed
        lds_barrier();
        issued_next = it + 2 < ntiles && issue(it + 2);
        const bool cur = it < ntiles && tile_page(it) >= 0;
        if (cur && prev)
          step(std::true_type{}, std::true_type{}, it);
        else if (cur)
          step(std::true_type{}, std::false_type{}, it);
        else if (prev)
          step(std::false_type{}, std::true_type{}, it);
        prev = cur;
      }
      const float l_tot = sum_xor32(sum_xor16(l_part));
      if (g == 0) {
        sm.lsum[l16][wave] = l_tot;
        p.part_lse[pi.row_base + wave * 16 + l16] = l_tot > 0.f ? (m_used + __log2f(l_tot)) * kLn2 : -INFINITY;
      }
      __syncthreads();
      __syncthreads();
    });
  } else {
    // ====================================================================== U-waves
    const int uw = wave - HB;
    int cidx[kCopiesPerSlice];
    uint32_t poff[kCopiesPerSlice];
#pragma unroll
    for (int k = 0; k < kCopiesPerSlice; ++k) {
      cidx[k] = uw * kCopiesPerSlice + k;
      poff[k] = PACKED ? (uint32_t)((copy_row(cidx[k], lane) * p.c_stride + copy_chunk(cidx[k], lane) * 8) * 2) : 0u;
    }
    // Transposed V reads of slice uw: tokens 4g + (l16/4) (and +16), columns
    // 16 cb + 4 (lane % 4) .. +3 of the slice, i.e. in-slice chunk 2 cb + (lane % 4) / 2.
    const int tr_tok = 4 * g + (l16 >> 2);
    const int tr_x = tr_tok & 7;
    const int tr_q = lane & 3;
    int tr_base[kUCb];
#pragma unroll
    for (int cb = 0; cb < kUCb; ++cb)
      tr_base[cb] = uw * kSliceBytes + tr_tok * kRowBytes + (((2 * cb + (tr_q >> 1)) ^ tr_x) << 4) + (tr_q & 1) * 8;
    for_each_piece_wave(p.seq_lens, p.batch, p.max_tokens, p.num_splits, w, table, first_lens(p.seq_lens, p.batch, p.max_tokens), [&](const Piece& pc) {
      const PieceInfo pi = piece_info(pc);
      PageWindow pw;
      pw.init(p.block_table + (size_t)pc.b * p.max_pages, p.max_pages, p.num_pages, pi.t0 / p.page_size);
      auto tile_page = [&](int it) -> int { return pw.get((pi.t0 + it * kT) / p.page_size); };
      auto issue = [&](int it) {
        const int page = tile_page(it);
        if (page < 0) return false;
        issue_copies<PACKED, kCopiesPerSlice>(p, cidx, poff, page, pi.t0 + it * kT, pi.end, sm.tile[it % kRing]);
        return true;
      };
      f32x4 acc[kUCb][HB];
#pragma unroll
      for (int cb = 0; cb < kUCb; ++cb)
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) acc[cb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
      wait_vmcnt<0>();
      const int ntiles = pi.ntiles;
      if (ntiles > 0) issue(0);
      bool issued_next = ntiles > 1 && issue(1);
      for (int it = 0; it <= ntiles + 1; ++it) {
        wait_vmcnt_upto(issued_next ? kCopiesPerSlice : 0);
        lds_barrier();
        const int t = it - 2;                            // tile whose probabilities are ready
        const bool pv = t >= 0 && tile_page(t) >= 0;
        if (!pv) {
          issued_next = it + 2 < ntiles && issue(it + 2);
          continue;
        }
        const unsigned char* tile = sm.tile[t % kRing];
        float al[HB];
        bool any = false;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          al[hb] = sm.alpha[t & 1][l16][hb];
          any |= al[hb] != 1.f;
        }
        bf16x8 pf[HB];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) pf[hb] = sm.prob[t & 1][hb][lane];
        bf16x8 vf[kUCb];
#pragma unroll
        for (int cb = 0; cb < kUCb; ++cb) {
          const unsigned char* a = tile + tr_base[cb];
          vf[cb] = concat4(lds_read_tr16(a), lds_read_tr16(a + 16 * kRowBytes));
        }
        // Slice uw of this ring slot is read only by this wave: once the reads above
        // have completed, the slot can take tile t + 4 = it + 2.
        wait_lds();
        issued_next = it + 2 < ntiles && issue(it + 2);
        if (__any(any)) {
#pragma unroll
          for (int cb = 0; cb < kUCb; ++cb)
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) acc[cb][hb] *= al[hb];
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
        bf16* up = (bf16*)p.part_u + (pi.row_base + hb * 16 + l16) * kDc + uw * 64 + 4 * g;
#pragma unroll
        for (int cb = 0; cb < kUCb; ++cb) *(bf16x4*)(up + cb * 16) = to_bf16x4(acc[cb][hb] * inv[hb]);
      }
      __syncthreads();
    });
  }
}

}  // namespace

int attn_heads_per_group(int n_h) { return n_h % 128 == 0 ? 128 : (n_h >= 64 ? 64 : n_h); }

hipError_t launch_attn_mfma(const AttnParams& p, bool fp8, hipStream_t stream) {
  if (p.n_h % 128 == 0) return launch_attn_h128(p, fp8, stream);   // all heads of a query position per workgroup
  if (fp8) return launch_attn_fp8_v0(p, stream);
  const int hg = attn_heads_per_group(p.n_h);
  const int HB = hg / 16;
  dim3 grid(p.num_splits, p.s_q * (p.n_h / hg));
  dim3 block(64 * (HB + kUWaves));
  const bool packed = p.packed_rows != 0;
#define MLA_LAUNCH(hb)                                                                          \
  return packed ? launch_attention_kernel(attn_partial_split<hb, true>, grid, block, stream, p)  \
                : launch_attention_kernel(attn_partial_split<hb, false>, grid, block, stream, p);
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
