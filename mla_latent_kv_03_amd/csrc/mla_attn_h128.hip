// Partial attention of absorbed MLA decode on gfx950, bf16 or E4M3 latent cache, 128
// heads of one query position per workgroup.
//
// For every piece of the split rule and every head i of the workgroup:
//   s_j = softmax_scale * (q_nope_i . c_j + q_pe_i . k_pe_j)       (page "MLA deep compression":
//   lse = ln sum_j exp(s_j),   u_i = sum_j exp(s_j - lse) c_j        absorbed scores, decoupled
//                                                                   RoPE, latent accumulation u_i)
// Every head reads the same 576-wide cached row and its first 512 values are also the
// value row, so a workgroup that holds all 128 heads streams each cached row from HBM
// exactly once.
//
// Four waves, one per SIMD, each with the whole 512-entry register file.  The two
// contractions are split differently, because LDS read instructions, not bytes, are
// the scarce resource (about 8 clocks of the CU's LDS pipe per wave-level read, 64-bit
// or 128-bit alike):
//  - scores: wave w owns heads 32w .. 32w+31, keeps their queries in registers (144)
//    and computes S^T[token, head] = K Q^T on 32x32x16 MFMAs (36 128-bit reads of the
//    tile per wave), then their softmax on the MFMA output layout (lane l owns head l%32
//    and 16 tokens);
//  - latent accumulation: wave w owns latent columns 128w .. 128w+127 of all 128 heads,
//    U^T[col, head] += V^T P^T (4 x 4 blocks of 32 x 32, 256 accumulator registers).
//    It reads only its quarter of the value tile (16 transposed 64-bit reads) and the
//    probabilities of all heads (8 128-bit reads) from a small LDS exchange buffer that
//    every wave fills with its heads' softmax output.
// The k-order of the accumulation MFMA is chosen so that a lane's softmax output is
// already a B operand (written to the exchange buffer as is), and the transposed reads
// of V fetch the tokens in the same order.  Per 32-token tile t a wave runs the 36
// score MFMAs of t (one dependent chain) with half of the accumulation MFMAs of tile
// t-1 between them, then the softmax of t interleaved with the other half, and spreads
// its 9 tile copies of t+2 over the score steps.  One barrier per tile orders the tile
// ring and the exchange buffer.
//
// LDS: a 4-deep ring of 32 x 1024-byte latent rows (tile t-1 is still read by the
// accumulation while tile t is scored and t+1, t+2 are in flight), a 3-deep ring of
// 32 x 128-byte RoPE-key rows (read only by the scores) and two 8 KiB probability
// buffers (tile t-1 read while tile t is written).  The rings are filled by direct
// buffer->LDS copies with the streaming cache policy; each wave issues 9 of a tile's
// 36 one-KiB copies.  16-byte chunk c of latent row r is stored at c ^ sv(r),
// sv(r) = 4 (r % 4) + (r / 4) % 4 (the two halves of r's low nibble swapped): 16
// consecutive rows get 16 different positions (score reads: 16 rows, one chunk) and 4
// consecutive rows 4 different 64-byte groups (transposed reads: 4 rows, four chunks
// per 32 lanes), so neither pattern has bank conflicts.  Chunk c of RoPE row r is
// stored at c ^ ((r / 2) % 8) (128-byte rows: 16 rows, one chunk, 16 positions).
//
// Softmax reference: exp2(s - m) with any m gives the same softmax once U and the sum
// are divided by the sum, and float32 / bf16 keep their relative precision for
// probabilities up to 2^64, so each head's reference m is fixed at the maximum of its
// first visible tile and the accumulators are never rescaled.  If a later tile exceeds
// m by more than 64 (log2 units), the workgroup recomputes the piece with m = the exact
// maximum, which the first pass has seen by then.
//
// E4M3 caches (page "MLA deep compression" gives the cache bytes per token as the lever;
// one fp32 scale per token, value = code * scale): the same pipeline on tiles of 512 +
// 64 bytes per token plus the scales, at half the copies.  The scores run on the matrix
// unit's E4M3 path (scaled 32x32x64 MFMAs): two 128-bit reads give a lane 32 key values as
// stored, and the bf16 queries enter as two E4M3 parts that represent them exactly (below).
// A transposed 8-bit read gives a whole 8-token value operand, widened to bf16 exactly for
// the accumulation.  The token scales multiply the scores and the probabilities (rounded
// to bf16 afterwards), which is the dequantized attention.

#include "mla_device.h"
#include "mla_kernels.h"
#include "mla_split.h"

namespace mla {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kT = 32;                        // tokens per tile
constexpr int kHeads = 128;                   // heads per workgroup
constexpr int kWaves = 4;
constexpr int kVRow = kDc * 2;                // 1024 bytes of latent per token
constexpr int kVTile = kT * kVRow;            // 32 KiB
constexpr int kKRow = kDr * 2;                // 128 bytes of RoPE key per token
constexpr int kKTile = kT * kKRow;            // 4 KiB
constexpr int kVRing = 4;
constexpr int kKRing = 3;
constexpr int kQk = (kDc + kDr) / 16;         // 36 score k-steps of 16
constexpr int kQkV = kDc / 16;                // the first 32 read latent rows; the last 4 the RoPE part
constexpr int kPv = 32;                       // accumulation MFMAs per tile: 2 token halves x 4 x 4 blocks
// Per element type of the cache: bf16 rows (1024 + 128 bytes) or E4M3 rows (512 + 64
// bytes, plus one fp32 scale per token).  kCopies: 1 KiB copies per wave and tile (bf16:
// 8 latent rows + 1 RoPE block; E4M3: 4 two-row latent blocks + a RoPE block or the
// scales, none for wave 3).
template <bool FP8>
struct Layout {
  static constexpr int kVRow = FP8 ? kDc : kDc * 2;
  static constexpr int kVTile = kT * kVRow;
  static constexpr int kKRow = FP8 ? kDr : kDr * 2;
  static constexpr int kKTile = kT * kKRow;
  static constexpr int kCopies = FP8 ? 5 : 9;
};
constexpr int kCopies = 9;
constexpr int kPBuf = kT * kHeads * 2;        // 8 KiB of bf16 probabilities per tile
#ifndef MLA_H128_KPF
#define MLA_H128_KPF 2
#endif
constexpr int kKPf = MLA_H128_KPF;            // score operands are read this many k-steps ahead
constexpr float kHeadroom = 64.f;             // tolerated excess over the reference maximum (log2 units)

template <bool FP8>
struct Smem {
  union {
    unsigned char v[kVRing][Layout<FP8>::kVTile];
    unsigned char u_stage[kHeads][kDc * 2];   // epilogue: the piece's bf16 u, one 1 KiB row per head
  };
  unsigned char k[kKRing][Layout<FP8>::kKTile];
  unsigned char p[2][kPBuf];                  // [tile % 2][head block][token half][lane] x 16 bytes
  float sc[FP8 ? kKRing : 1][64];             // E4M3: per-token scales of the tile (32 used)
  float l[kHeads];                            // row sums, for the column-owning waves
  unsigned char stash[kMaxFusedNew][kVRow + kKRow];   // fused append: this piece's new rows
  int redo[kWaves];                           // per wave: a tile exceeded the reference maximum
};
static_assert(sizeof(Smem<false>) <= 160 * 1024 && sizeof(Smem<true>) <= 160 * 1024, "LDS budget of one workgroup");
// The bf16 score reads address the RoPE ring as the bytes right after the value ring.
static_assert(offsetof(Smem<false>, k) == kVRing * kVTile, "RoPE ring follows the value ring");

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  // C[32x32] += A[32x16] B[16x32]: lane l holds A[l%32][8(l/32) + j], B[8(l/32) + j][l%32]
  // (j = 0..7) and C[8(v/4) + 4(l/32) + v%4][l%32] (v = 0..15).
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The score chain (36 MFMAs into one 32x32 block) is written in assembly so that its
// accumulator lives in VGPRs: the latent accumulators take all 256 AGPRs, and the
// compiler gives every MFMA of a kernel the same accumulator register file.  Hazards of
// these instructions, which the compiler does not see:
//  - the first MFMA of a chain starts from the inline constant 0, so no VALU write of
//    its accumulator precedes it; the later ones read the previous result as srcC with
//    exactly the same registers, the back-to-back accumulation case the matrix unit
//    forwards;
//  - each MFMA starts with s_nop 1, covering a VALU write of its A/B registers just
//    before it (2 wait states);
//  - scores_ready() inserts 24 wait states (more than passes + 2) before any other
//    instruction reads or overwrites the accumulator.
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void score_mfma_first(f32x16& s, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0"
               : "=&v"(s)
               : "v"(__builtin_bit_cast(u32x4v, a)), "v"(__builtin_bit_cast(u32x4v, b)));
}
__device__ __forceinline__ void score_mfma(f32x16& s, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
               : "+v"(s)
               : "v"(__builtin_bit_cast(u32x4v, a)), "v"(__builtin_bit_cast(u32x4v, b)));
}
// E4M3 scores: the E4M3 key rows times an E4M3 part of the queries, 32x32x64 with E8M0
// block scales (scale_a for the keys: 1; scale_b: 1 for the queries' high part, 2^-4 for
// the remainder part), into the same VGPR accumulator and with the same hazards as above.
typedef unsigned u32x8v __attribute__((ext_vector_type(8)));
__device__ __forceinline__ void score8_first(f32x16& s, u32x8v a, u32x8v b, uint32_t sa, uint32_t sb) {
  asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel_hi:[0,0,0]"
               : "=&v"(s)
               : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
__device__ __forceinline__ void score8(f32x16& s, u32x8v a, u32x8v b, uint32_t sa, uint32_t sb) {
  asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+v"(s)
               : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
__device__ __forceinline__ void scores_ready(f32x16& s) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s));
}

// A zero the compiler cannot see through: per-lane LDS offsets derived from it are
// recomputed where they are used (one v_xor each) instead of being hoisted out of the
// tile loop as two dozen long-lived registers.
__device__ __forceinline__ uint32_t opaque_zero() {
  uint32_t z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

__device__ __forceinline__ int swz_v(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int swz_k(int r) { return (r >> 1) & 7; }
// E4M3 rows: 16-byte chunk c (of 32) of latent row r is stored at c ^ swz_v8(r), a
// permutation of r's low 4 bits (bit 0 <- r bit 2, bits 1-2 <- r bits 0-1, bit 3 <- r
// bit 3): 16 consecutive rows get 16 positions (score reads), and the 8 rows that one
// 16-lane block of a transposed read covers (4h + 0..3 and 8 + 4h + 0..3) get 8 even or
// 8 odd ones, so two adjacent chunks of them fill all 16 positions.  RoPE rows (4 chunks)
// use c ^ ((r / 4) % 4).
__device__ __forceinline__ int swz_v8(int r) { return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8); }
__device__ __forceinline__ int swz_k8(int r) { return (r >> 2) & 3; }

// 8 E4M3 values (two dwords, byte j = value j) to bf16, exactly.  (The conversion's own
// scale operand is not used for the per-token scales: MX-style conversions scale by a
// power of two.)
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2 a = e4m3x2_to_bf16<false>(w0), b = e4m3x2_to_bf16<true>(w0);
  const bf16x2 c = e4m3x2_to_bf16<false>(w1), d = e4m3x2_to_bf16<true>(w1);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt left alone
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <bool FP8>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_partial_h128(const AttnParams p) {
  __shared__ __attribute__((aligned(16))) Smem<FP8> sm;
  using LT = Layout<FP8>;

  // Every 64-byte line of the argument block is read here, in one batch: a scalar-cache
  // miss on it is a memory round trip, and the compiler would otherwise first touch the
  // later lines where they are used, one round trip after another.
  asm volatile("" ::"s"(p.q_nope), "s"(p.c_stride), "s"(p.split_table), "s"(p.s_new));

  // Consecutive shares (the pieces of one sequence) on one XCD: workgroups are dispatched
  // to the 8 XCDs round-robin, so workgroup i takes share (i % 8) * (G / 8) + i / 8.
  const int w = p.num_splits % 8 == 0 ? (int)(blockIdx.x % 8) * (p.num_splits / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const int rg = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int groups_per_q = p.n_h / kHeads;
  const int q_pos = rg / groups_per_q;
  const int head_base = (rg - q_pos * groups_per_q) * kHeads;
  int32_t* table = (rg == 0 && wave == 0) ? p.split_table : nullptr;

  // Per-lane LDS offsets (all recomputed from the lane index where they are used, so
  // that none of them stays live across the tile loop):
  //  - score reads: token l32, logical chunk 2 ks + h, stored at (2 ks + h) ^ sv(l32);
  //  - transposed latent reads: 16-lane block b1 = (lane/16)%2 gives columns 16 b1 .. +15
  //    of a 32-column block, lane 4r + q of the block the 4 columns 4q.. of token row r
  //    (rows 4h + r (+ 8 e) have sv = 4r + h + 2e);
  //  - probability buffer: 16 bytes per lane.
  //  E4M3 tiles (16-byte chunks of 16 values):
  //  - score reads: token l32, the 16 values of chunk 2 kp + h (k-steps 2 kp and 2 kp + 1
  //    take bytes 0..7 and 8..15), stored at (2 kp + h) ^ swz_v8(l32);
  //  - transposed latent reads (8-bit): 16-lane block b = lane/16, lane 2r + q of the
  //    block: token row 8 (r/4) + 4 (b/2) + r%4, bytes 8q.. of chunk 8 wave + 2 cl + b%2.
  struct LaneOffsets {
    uint32_t ln, qk_v, qk_k, tr, pb;
  };
  auto lane_offsets = [&]() {
    const uint32_t ln = lane_id_opaque();
    const int l = (int)ln, lr = l & 31, hh = l >> 5;
    LaneOffsets o;
    o.ln = ln;
    o.pb = (uint32_t)offsetof(Smem<FP8>, p) + 16 * ln;
    if constexpr (!FP8) {
      const int tr_i = l & 15, tr_r = tr_i >> 2, tr_q = tr_i & 3, tr_b1 = (l >> 4) & 1;
      const int tr_lc = (2 * tr_b1 + (tr_q >> 1)) ^ (4 * tr_r + hh);
      o.qk_v = (uint32_t)(lr * kVRow + 16 * (hh ^ swz_v(lr)));                   // ^ 32 (ks % 8), + 256 (ks / 8)
      o.qk_k = (uint32_t)(kVRing * kVTile + lr * kKRow + 16 * (hh ^ swz_k(lr)));  // ^ 32 (ks - 32)
      o.tr = (uint32_t)((4 * hh + tr_r) * kVRow + 16 * tr_lc + 8 * (tr_q & 1) + 256 * wave);
    } else {
      const int b = l >> 4, r = (l & 15) >> 1, q = l & 1;
      const int tok = 8 * (r >> 2) + 4 * (b >> 1) + (r & 3);
      const int c0 = 8 * wave + (b & 1);
      o.qk_v = (uint32_t)(lr * LT::kVRow + 16 * (hh ^ swz_v8(lr)));                                 // ^ 32 kp
      o.qk_k = (uint32_t)(offsetof(Smem<FP8>, k) + lr * LT::kKRow + 16 * (hh ^ swz_k8(lr)));        // ^ 32 (kp - 16)
      o.tr = (uint32_t)(tok * LT::kVRow + 16 * (c0 ^ swz_v8(tok)) + 8 * q);                           // ^ 32 cl, + 8192 th
    }
    return o;
  };

  const int len0 = first_lens(p.seq_lens, p.batch, p.max_tokens);

  // New row of the fused append that this wave writes to the pool at the start (below).
  const int fused_row = kWaves - 1 - wave;
  const bool fused_write = p.new_c != nullptr && rg == 0 && w < p.batch && fused_row < p.s_new;
  u32x4 new_c_row = u32x4{0u, 0u, 0u, 0u}, new_k_row = u32x4{0u, 0u, 0u, 0u};
  if (!FP8 && fused_write) {
    const uint32_t l = lane_id_opaque();
    const size_t tok = (size_t)w * p.s_new + fused_row;
    new_c_row = *(const u32x4*)((const char*)p.new_c + tok * kDc * 2 + 16 * l);
    new_k_row = *(const u32x4*)((const char*)p.new_k + tok * kDr * 2 + 16 * (l % (kKRow / 16)));
  }

  // The block-table row of the sequence this share starts in when all lengths are equal
  // is requested now, together with the lengths, instead of after the split walk (cold
  // loads take microseconds); a piece of another sequence loads its own row.
  const int b_guess = min(p.batch - 1, (int)udiv_mostly32((unsigned long long)w * (unsigned)p.batch, (unsigned)p.num_splits));
  PageWindow pw;
  pw.init(p.block_table + (size_t)b_guess * p.max_pages, p.max_pages, p.num_pages, 0);
  int pw_b = b_guess;

  // The queries of the guessed sequence are copied to LDS right away, one 1 KiB row per
  // copy, so that their transfer overlaps the split walk; the first piece reads them back
  // if its sequence is the guessed one.  (Loaded straight into the operand layout, each
  // load instruction would touch 32 rows.)  16-byte chunk c of head row r is stored at
  // c ^ (r % 16), of its RoPE row at c ^ ((r / 2) % 8), so that the operand reads (one
  // chunk of 16 consecutive rows) are free of bank conflicts.  Wave w's rows go to
  // u_stage rows 32w.. and to the probability buffers (4 KiB per wave), which nothing
  // else uses before the first piece's tile copies.
  {
    const uint32_t lz = lane_id_opaque();
    const size_t qrow0 = ((size_t)b_guess * p.s_q + q_pos) * p.n_h + head_base + 32 * wave;
    const __amdgpu_buffer_rsrc_t qn = buffer_rsrc((const char*)p.q_nope + qrow0 * (kDc * 2));
    const __amdgpu_buffer_rsrc_t qp = buffer_rsrc((const char*)p.q_pe + qrow0 * (kDr * 2));
#pragma unroll
    for (int r = 0; r < 32; ++r)
      buffer_to_lds16(qn, (uint32_t)r * (kDc * 2) + 16u * (lz ^ (uint32_t)(r & 15)), 0u, sm.u_stage[32 * wave + r]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t r = 8u * j + (lz >> 3);
      buffer_to_lds16(qp, r * (kDr * 2) + 16u * ((lz & 7u) ^ ((r >> 1) & 7u)), 0u, (unsigned char*)sm.p + wave * 4096 + j * 1024);
    }
  }
  // The guessed block-table window has to land before its first lookup; waiting for it
  // here (its load precedes the query copies, so this waits for that load alone, while the
  // split walk waits for the lengths anyway) means no later lookup waits for it, and such a
  // wait, placed by the compiler at the first lookup, also waited for the copies in flight.
  pw.settle();
  bool first_piece = true;

  // Fused append, pool write of new row i of sequence w (row group 0) by wave
  // kWaves - 1 - i, at the start (sequences w + G, w + 2G, .. are written at the end of
  // the launch).  The row is loaded before the query copies are issued, and the position
  // and page lookups go through the scalar cache, so that no wait of this write waits
  // for the query copies.  The stores' completion is never waited for: the tile loop's
  // copy waits only ever count them as outstanding, which makes those waits stricter.
  if (!FP8 && fused_write) {
    const uint32_t l = lane_id_opaque();
    const int pos = load_scalar(p.new_pos + (size_t)w * p.s_new + fused_row);
    if (pos >= 0 && pos / p.page_size < p.max_pages) {
      const int page = load_scalar(p.block_table + (size_t)w * p.max_pages + pos / p.page_size);
      if (page >= 0 && page < p.num_pages) {
        const size_t slot = (size_t)page * p.page_size + pos % p.page_size;
        *(u32x4*)((char*)const_cast<void*>(p.c_kv) + slot * ((size_t)p.c_stride * 2) + 16 * l) = new_c_row;
        if (l < kKRow / 16)
          *(u32x4*)((char*)const_cast<void*>(p.k_pe) + slot * ((size_t)p.k_stride * 2) + 16 * l) = new_k_row;
      }
    }
  }

  for_each_piece_wave(p.seq_lens, p.batch, p.max_tokens, p.num_splits, w, table, len0, [&](const Piece& pc) {
    const int L = pc.len;
    const int t0 = pc.t0;
    const int end = min(pc.t1, max(0, L - p.s_q + q_pos + 1));      // visible tokens of this piece
    const int ntiles = end > t0 ? (end - t0 + kT - 1) / kT : 0;
    const size_t row_base = ((size_t)pc.slot * p.s_q + q_pos) * p.n_h + head_base;
    if (pc.b != pw_b) {
      pw.init(p.block_table + (size_t)pc.b * p.max_pages, p.max_pages, p.num_pages, t0 / p.page_size);
      pw.settle();
      pw_b = pc.b;
    }
    // Fused append: the tile (npt) and tile row (nrow) of each new row of this sequence
    // that lies in the piece's visible tokens, else -1.  Wave-uniform; the positions come
    // through the scalar cache, so this wait does not also wait for the copies in flight.
    const bool fused = p.new_c != nullptr;
    int npt[kMaxFusedNew], nrow[kMaxFusedNew];
#pragma unroll
    for (int i = 0; i < kMaxFusedNew; ++i) {
      const int pos = fused && i < p.s_new ? load_scalar(p.new_pos + (size_t)pc.b * p.s_new + i) : -1;
      const bool in = pos >= t0 && pos < end;
      npt[i] = in ? (pos - t0) / kT : -1;
      nrow[i] = in ? (pos - t0) % kT : -1;
    }
    // Queries of head 32 wave + l32, k-steps of 16: lane holds dims 16 ks + 8 h .. +7
    // (E4M3: k-step 2 kp + s holds dims 32 kp + 16 h + 8 s .. +7, the order of the score
    // reads; a contraction may take its k index in any order both operands share).
    bf16x8 qf[kQk];
    auto load_queries = [&]() {
      const int ql = (int)lane_id_opaque(), l32 = ql & 31, h = ql >> 5;
      const size_t qrow = ((size_t)pc.b * p.s_q + q_pos) * p.n_h + head_base + 32 * wave + l32;
      if constexpr (!FP8) {
        const bf16* qn = (const bf16*)p.q_nope + qrow * kDc + 8 * h;
        const bf16* qp = (const bf16*)p.q_pe + qrow * kDr + 8 * h;
#pragma unroll
        for (int ks = 0; ks < kQkV; ++ks) qf[ks] = *(const bf16x8*)(qn + 16 * ks);
#pragma unroll
        for (int kk = 0; kk < kQk - kQkV; ++kk) qf[kQkV + kk] = *(const bf16x8*)(qp + 16 * kk);
      } else {
        const bf16* qn = (const bf16*)p.q_nope + qrow * kDc + 16 * h;
        const bf16* qp = (const bf16*)p.q_pe + qrow * kDr + 16 * h;
#pragma unroll
        for (int ks = 0; ks < kQkV; ++ks) qf[ks] = *(const bf16x8*)(qn + 32 * (ks >> 1) + 8 * (ks & 1));
#pragma unroll
        for (int kk = 0; kk < kQk - kQkV; ++kk) qf[kQkV + kk] = *(const bf16x8*)(qp + 32 * (kk >> 1) + 8 * (kk & 1));
      }
    };
    // The queries from the LDS copy made at kernel entry (same layout as load_queries).
    auto read_staged_queries = [&]() {
      const uint32_t ql = lane_id_opaque(), l32 = ql & 31u, h = ql >> 5;
      const unsigned char* qrow = sm.u_stage[32 * wave + (int)l32];
      const unsigned char* prow = (const unsigned char*)sm.p + wave * 4096 + l32 * (kDr * 2);
#pragma unroll
      for (int ks = 0; ks < kQk; ++ks) {
        // logical 16-byte chunk of the row that k-step ks reads
        const uint32_t c = !FP8 ? 2u * (uint32_t)(ks < kQkV ? ks : ks - kQkV) + h
                                : 4u * (uint32_t)((ks < kQkV ? ks : ks - kQkV) >> 1) + 2u * h + (uint32_t)(ks & 1);
        if (ks < kQkV)
          qf[ks] = *(const bf16x8*)(qrow + 16u * (c ^ (l32 & 15u)));
        else
          qf[ks] = *(const bf16x8*)(prow + 16u * (c ^ ((l32 >> 1) & 7u)));
      }
    };
    // E4M3: the queries as two E4M3 parts with one power-of-two scale 2^k per head, the B
    // operands of the scaled 32x32x64 MFMA: 2^k q = hi + lo / 16 exactly.  A bf16 value has
    // 8 significant bits; hi keeps the first 4 (nearest), and the remainder is a multiple of
    // the value's last bf16 step with at most 4 significant bits, so 16 times it is an E4M3
    // value too (k puts the head's largest element below 2^8; elements more than 15 binades
    // below it would lose bits and weigh less than 2^-15 of it).  The factor 2^-k of the
    // head's scores goes into the lane's softmax scale.  Byte j of k-block kb's operand is
    // the same dimension as byte j of the key operand: k-steps 4 kb .. 4 kb + 3 of qf in
    // order (which matches two consecutive score reads of the tile).
    u32x8v qh[kQk / 4], ql[kQk / 4];
    float qs = p.scale_log2;      // the lane's scores to base-2 logits (E4M3: times 2^-k)
    auto convert_queries = [&]() {
      float amax = 0.f;
#pragma unroll
      for (int ks = 0; ks < kQk; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf((float)qf[ks][j]));
      amax = max_xor32(amax);                        // both lane halves hold the head's row
      const int k = amax > 0.f ? 8 - __builtin_amdgcn_frexp_expf(amax) : 0;
      qs = ldexpf(p.scale_log2, -k);
#pragma unroll
      for (int kb = 0; kb < kQk / 4; ++kb)
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const bf16x8 src = qf[4 * kb + d / 2];
          float x[4], r[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = ldexpf((float)src[4 * (d % 2) + i], k);
          int hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0, false);
          hi = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], hi, true);
          const f32x2 b01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
          const f32x2 b23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
          r[0] = (x[0] - b01[0]) * 16.f;
          r[1] = (x[1] - b01[1]) * 16.f;
          r[2] = (x[2] - b23[0]) * 16.f;
          r[3] = (x[3] - b23[1]) * 16.f;
          int lo = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
          lo = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], lo, true);
          qh[kb][d] = (uint32_t)hi;
          ql[kb][d] = (uint32_t)lo;
        }
    };
    const int tiles_per_page = p.page_size / kT;
    const uint32_t c_row = (uint32_t)p.c_stride * (FP8 ? 1u : 2u), k_row = (uint32_t)p.k_stride * (FP8 ? 1u : 2u);

    // Copy cursor: the next tile to enqueue, its logical page, its tile index within
    // that page and its ring slots.
    // pg_lp / pg_id: the last logical page looked up and its id (a page holds several
    // tiles, and a lookup is a register read plus scalar checks).
    int i_tt, i_lp, i_tip, i_vs, i_ks, pg_lp, pg_id;
    auto reset_cursor = [&]() {
      pw.rewind(t0 / p.page_size);
      pg_lp = -1;
      pg_id = -1;
      i_tt = t0;
      i_lp = t0 / p.page_size;
      i_tip = (t0 - i_lp * p.page_size) / kT;
      i_vs = 0;
      i_ks = 0;
    };
    // Copies of one tile by this wave: buffer resources based at the tile's first latent
    // and RoPE rows (a tile never crosses a page, so row offsets stay far below the
    // 2 GiB record limit), its last visible row and its ring slots.  A tile with an
    // invalid page, or past the piece, gets zero-length resources: its copies read
    // nothing and fill their ring slots with zeros.
    struct TileCopy {
      __amdgpu_buffer_rsrc_t vres, kres, sres;
      int last, vs, ks;
    };
    // Describe the cursor's tile and advance the cursor (scalar work only); `ok` tells
    // whether the tile has a valid page.
    auto prepare_next = [&](bool exists, bool& ok) {
      TileCopy tc;
      if (exists && i_lp != pg_lp) {
        pg_id = pw.get(i_lp);
        pg_lp = i_lp;
      }
      const int page = exists ? pg_id : -1;
      ok = page >= 0;
      const long long slot0 = ok ? (long long)page * p.page_size + i_tip * kT : 0;
      tc.vres = buffer_rsrc((const char*)p.c_kv + slot0 * c_row, ok ? 0x7fffffff : 0);
      tc.kres = buffer_rsrc((const char*)p.k_pe + slot0 * k_row, ok ? 0x7fffffff : 0);
      if constexpr (FP8) tc.sres = buffer_rsrc(p.kv_scale + slot0, ok ? 0x7fffffff : 0);
      tc.last = min(i_tt + kT, end) - 1 - i_tt;   // rows past `last` re-read it
      tc.vs = i_vs;
      tc.ks = i_ks;
      i_tt += kT;
      if (++i_tip == tiles_per_page) {
        i_tip = 0;
        ++i_lp;
      }
      i_vs = (i_vs + 1) & (kVRing - 1);
      i_ks = i_ks == kKRing - 1 ? 0 : i_ks + 1;
      return tc;
    };
    // Copy j of this wave's 9 for tile tc: latent row 8 wave + j (j < 8; lane l: stored
    // chunk l) or the RoPE block (j = 8; lane l: row 8 wave + l/8, stored chunk l%8).
    // Per-lane offsets are recomputed from the lane index rather than kept live.
    // E4M3, copy j of this wave's 5: latent rows 2i, 2i + 1 with i = wave + 4j (j < 4;
    // lane l: row 2i + l/32, stored chunk l%32), then for waves 0 and 1 the RoPE rows
    // 16 wave .. + 15 (lane l: row 16 wave + l/4, stored chunk l%4) and for wave 2 the
    // scales (lane l: token min(l, last), 4 bytes).
    auto copy_row = [&](const TileCopy& tc, int j, uint32_t lz) {
      if constexpr (!FP8) {
        if (j < 8) {
          const int r = 8 * wave + j;
          buffer_to_lds16(tc.vres, 16u * (lz ^ (uint32_t)swz_v(r)), (uint32_t)min(r, tc.last) * c_row,
                          sm.v[tc.vs] + r * kVRow);
        } else {
          const int krow = 8 * wave + (int)(lz >> 3);
          const uint32_t kchunk = (lz & 7u) ^ (uint32_t)swz_k(krow);
          const uint32_t koff = (uint32_t)min(krow, tc.last) * k_row + 16u * kchunk;
          buffer_to_lds16(tc.kres, koff, 0u, sm.k[tc.ks] + wave * 1024);
        }
      } else {
        if (j < 4) {
          const int i = wave + 4 * j;
          const int r = 2 * i + (int)(lz >> 5);
          const uint32_t chunk = (lz & 31u) ^ (uint32_t)swz_v8(r);
          buffer_to_lds16(tc.vres, (uint32_t)min(r, tc.last) * c_row + 16u * chunk, 0u, sm.v[tc.vs] + i * 1024);
        } else if (wave < 2) {
          const int krow = 16 * wave + (int)(lz >> 2);
          const uint32_t kchunk = (lz & 3u) ^ (uint32_t)swz_k8(krow);
          buffer_to_lds16(tc.kres, (uint32_t)min(krow, tc.last) * k_row + 16u * kchunk, 0u, sm.k[tc.ks] + wave * 1024);
        } else if (wave == 2) {
          buffer_to_lds4(tc.sres, 4u * (uint32_t)min((int)lz, tc.last), 0u, sm.sc[tc.ks]);
        }
      }
    };
    // This wave's copies of all but the most recently enqueued tile have landed.
    auto wait_copies = [&]() {
      if constexpr (!FP8) {
        wait_vmcnt<kCopies>();
      } else {
        if (wave == 3)
          wait_vmcnt<4>();
        else
          wait_vmcnt<5>();
      }
    };

    f32x16 acc[16];   // U^T block (column block 4 wave + a / 4, head block a % 4)
    float m_ref = -INFINITY;       // this lane's head's reference maximum (base 2)
    float x_max = -INFINITY;       // largest log2 score above m_ref among this lane's tokens
    float l_part = 0.f;            // sum of the unrounded numerators (for lse)
    float l_eff = 0.f;             // E4M3: sum of the rounded weights over their scales (divides U)

    // One pass over the piece.  The accumulation of tile it-1 runs in every iteration;
    // before the first tile it uses zero probabilities (and reads a ring slot that holds
    // zeros or cache rows), and a tile that is not scored (invalid page, past the end)
    // yields zero probabilities, so every iteration runs the same instruction sequence.
    auto run_pass = [&](bool first_pass) {
#pragma unroll
      for (int a = 0; a < 16; ++a)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[a][v] = 0.f;
      l_part = 0.f;
      l_eff = 0.f;
      x_max = -INFINITY;
      if (first_pass && first_piece) {
        // The query copies made at kernel entry must land before the ring and the
        // probability buffers are reused; read them back if they are this piece's.
        wait_vmcnt<0>();
        if (pc.b == b_guess) read_staged_queries();
        lds_barrier();
      }
      if (first_pass) {
        // Ring slot 3 is zeroed for each piece: the accumulation step that runs before a
        // pass's first tile reads it with zero probabilities, and 0 * (stale bits) must
        // not produce NaN; before the first piece it holds queries, afterwards the
        // previous piece's staged u (not valid E4M3 codes).  Within the piece the ring
        // only holds cache rows or zeros.  (The first iteration's barrier orders these
        // writes before those reads.)
        // (Addresses and the zero vector are made here from opaque values: kept from the
        // kernel's start they were spilled to scratch and reloaded one memory round trip
        // at a time.)
        const uint32_t t = lane_id_opaque() + 64u * (uint32_t)wave;
        const uint32_t z = opaque_zero();
        unsigned char* slot3 = sm.v[kVRing - 1];
#pragma unroll
        for (int j = 0; j < LT::kVTile / (16 * 64 * kWaves); ++j)
          *(u32x4*)(slot3 + 16u * (t + 64u * kWaves * j)) = u32x4{z, z, z, z};
      }
      // Zero probabilities of "tile -1" (buffer 1), this wave's head block.
      {
        const uint32_t z = opaque_zero();
        unsigned char* pz = sm.p[1] + wave * 2 * 1024 + 16 * lane_id_opaque();
#pragma unroll
        for (int half = 0; half < 2; ++half) *(u32x4*)(pz + half * 1024) = u32x4{z, z, z, z};
      }
      // No drain of older loads here: a wave's copies land in issue order and each wave
      // writes only its own ring rows, so an earlier pass's copies cannot overwrite
      // this pass's; the query loads are covered by the first iteration's wait.
      reset_cursor();
      // Bit k of `ready`: tile it + k has a valid page.  Every iteration enqueues the 9
      // copies of tile it + 2 (no-ops past the piece), so exactly one tile's copies are
      // in flight besides tile it's at the top of an iteration.
      // The queries (first pass) are requested between tiles 0 and 1: the first
      // iteration's wait then covers exactly tile 0 and the queries, and the copies do
      // not queue behind 36 query loads.
      uint32_t ready = 0;
      const uint32_t lz0 = lane_id_opaque();
      // The first two tiles are described (page lookups, scalar work) before any copy of
      // this pass is issued: a lookup may wait for the block-table window, and such a wait
      // counts every vector-memory operation issued before it.
      bool ok0, ok1;
      const TileCopy tc0 = prepare_next(0 < ntiles, ok0);
      const TileCopy tc1 = prepare_next(1 < ntiles, ok1);
      ready |= (ok0 ? 1u : 0u) | (ok1 ? 2u : 0u);
      if (first_pass && fused) {
        // New row i goes to the stash, copied by wave i (before tile 0's copies, so the
        // first iteration's wait covers it; the first barrier makes it visible).
#pragma unroll
        for (int i = 0; i < kMaxFusedNew; ++i)
          if (npt[i] >= 0 && wave == i) {
            const size_t tok = (size_t)pc.b * p.s_new + i;
            const uint32_t l = lane_id_opaque();
            buffer_to_lds16(buffer_rsrc((const char*)p.new_c + tok * kDc * 2), 16u * l, 0u, sm.stash[i]);
            if (l < kKRow / 16)
              buffer_to_lds16(buffer_rsrc((const char*)p.new_k + tok * kDr * 2), 16u * l, 0u, sm.stash[i] + kVRow);
          }
      }
#pragma unroll
      for (int j = 0; j < LT::kCopies; ++j) copy_row(tc0, j, lz0);
      if (first_pass && !(first_piece && pc.b == b_guess)) load_queries();
#pragma unroll
      for (int j = 0; j < LT::kCopies; ++j) copy_row(tc1, j, lz0);
      if constexpr (FP8) {
        if (first_pass) convert_queries();           // waits for the query loads (and tile 0)
      }
      int vs = 0, ks3 = 0;   // ring slots of tile `it`
      for (int it = 0; it <= ntiles; ++it) {
        wait_copies();             // this wave's copies of tile `it` have landed, it+1's in flight
        lds_barrier();             // tile `it` and every wave's probabilities of it-1 are in LDS
        const bool cur = (ready & 1u) != 0;       // tile `it` is scored
        if (!FP8 && fused && cur && (npt[0] == it || npt[1] == it)) {
          // Fused append: rows of this tile whose source is a new row (its own row, and the
          // rows past the last visible one when it is the last) take the stashed row; each
          // wave patches its own rows, then a second barrier publishes them.
          const int tt = t0 + it * kT;
          const int last = min(tt + kT, end) - 1 - tt;
          const uint32_t l = lane_id_opaque();
#pragma unroll
          for (int i = 0; i < kMaxFusedNew; ++i) {
            if (npt[i] != it) continue;
#pragma unroll 1
            for (int j = 0; j < 8; ++j) {
              const int rr = 8 * wave + j;
              if (min(rr, last) != nrow[i]) continue;
              const u32x4 v = *(const u32x4*)(sm.stash[i] + 16 * l);
              *(u32x4*)(sm.v[vs] + rr * LT::kVRow + 16 * (l ^ (uint32_t)swz_v(rr))) = v;
              if (l < kKRow / 16) {
                const u32x4 k = *(const u32x4*)(sm.stash[i] + kVRow + 16 * l);
                *(u32x4*)(sm.k[ks3] + rr * LT::kKRow + 16 * (l ^ (uint32_t)swz_k(rr))) = k;
              }
            }
          }
          lds_barrier();
        }
        // Per-lane LDS offsets of this iteration: ring slot + fixed lane part; the XOR
        // swizzles only touch bits 4..7, below the slot bits.
        const unsigned char* lds = (const unsigned char*)&sm;
        const LaneOffsets lo = lane_offsets();
        const uint32_t bq = (uint32_t)(vs * LT::kVTile) + lo.qk_v;
        const uint32_t bk = (uint32_t)(ks3 * LT::kKTile) + lo.qk_k;
        const uint32_t bt = (uint32_t)(((vs + kVRing - 1) & (kVRing - 1)) * LT::kVTile) + lo.tr;
        const uint32_t bp = (uint32_t)(((it + 1) & 1) * kPBuf) + lo.pb;
        auto kfrag = [&](int ks) -> bf16x8 {
          if (ks < kQkV) return *(const bf16x8*)(lds + ((bq ^ (32u * (ks & 7))) + 256 * (ks >> 3)));
          return *(const bf16x8*)(lds + (bk ^ (32u * (ks - kQkV))));
        };
        // E4M3: the 16 values of score k-steps 2 kp and 2 kp + 1.
        auto kraw = [&](int kp) -> u32x4 {
          if (kp < kQkV / 2) return *(const u32x4*)(lds + (bq ^ (32u * kp)));
          return *(const u32x4*)(lds + (bk ^ (32u * (kp - kQkV / 2))));
        };
        // V^T fragment of this wave's column block cl (32 columns) and token half th of
        // tile it-1.
        auto vfrag = [&](int cl, int th) -> bf16x8 {
          const uint32_t o = 16384 * th;
          const bf16x4 lo = lds_read_tr16(lds + ((bt ^ (64u * cl)) + o));
          const bf16x4 hi = lds_read_tr16(lds + ((bt ^ (64u * cl ^ 32u)) + o + 8192));
          return concat4(lo, hi);
        };
        // E4M3: the 8-bit read and its widening are separate steps, a few k-steps apart, so
        // that the widening does not wait for the read right after issuing it.
        auto vraw8 = [&](int cl, int th) -> u32x2 {
          return lds_read_tr8(lds + ((bt ^ (32u * cl)) + 16 * LT::kVRow * th));
        };
        auto widen = [&](u32x2 w8) -> bf16x8 { return e4m3x8_to_bf16(w8[0], w8[1]); };
        // P^T fragment of head block hb and token half th of tile it-1.
        auto pfrag = [&](int hb, int th) -> bf16x8 { return *(const bf16x8*)(lds + bp + (hb * 2 + th) * 1024); };

        // Accumulation step a of tile it-1: token half a / 16, column block (a / 4) % 4,
        // head block a % 4.  Phase 1: the 36 score MFMAs of tile `it` (one dependent
        // chain) with steps 0..15 between every other pair of them; phase 2: the softmax
        // of tile `it` interleaved with steps 16..31.  LDS operands are read ahead: with
        // one wave per SIMD the reads' latency has to hide behind this wave's own MFMAs.
        f32x16 s;
        bf16x8 kq[kKPf + 1], va[4], pb[2][4];
        u32x8v k8[3];         // E4M3: key operand of k-block kb in k8[kb % 3], read two k-blocks ahead
        u32x2 vr[4];          // E4M3: value reads not yet widened
        f32x4 tsc[4];         // E4M3: per-token scales of tile `it` (read before the score chain ends)
        if constexpr (!FP8) {
#pragma unroll
          for (int j = 0; j < kKPf; ++j) kq[j] = kfrag(j);
          va[0] = vfrag(0, 0);
        } else {
          k8[0] = __builtin_shufflevector(kraw(0), kraw(1), 0, 1, 2, 3, 4, 5, 6, 7);
          k8[1] = __builtin_shufflevector(kraw(2), kraw(3), 0, 1, 2, 3, 4, 5, 6, 7);
          vr[0] = vraw8(0, 0);                       // widened at ks = 1, first used at ks = 3
        }
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) pb[0][hb] = pfrag(hb, 0);
        // The copy bookkeeping of tile it+2 (scalar work) runs while those first reads are
        // in flight.  Tile it+2 goes to ring slots last read in iteration it-1, which every
        // wave has finished (barrier above).
        __builtin_amdgcn_sched_barrier(0);
        bool next_ok;
        const TileCopy tn = prepare_next(it + 2 < ntiles, next_ok);
        ready |= next_ok ? 4u : 0u;
#pragma unroll
        for (int ks = 0; ks < kQk; ++ks) {
          __builtin_amdgcn_sched_barrier(0);   // keep the source order: reads ahead of use
          if constexpr (!FP8) {
            if (ks + kKPf < kQk) kq[(ks + kKPf) % (kKPf + 1)] = kfrag(ks + kKPf);
          }
          // Step a runs at ks = 2a + 3.  va[cl] holds token half 0 of column block cl
          // until its last use at ks = 8 cl + 9, then token half 1 (loaded 3 steps later).
          if constexpr (!FP8) {
            if (ks == 2) va[1] = vfrag(1, 0);
            if (ks == 10) va[2] = vfrag(2, 0);
            if (ks == 18) va[3] = vfrag(3, 0);
            if (ks == 12) va[0] = vfrag(0, 1);
            if (ks == 20) va[1] = vfrag(1, 1);
            if (ks == 28) va[2] = vfrag(2, 1);
            if (ks == 35) va[3] = vfrag(3, 1);
          } else {
            // The same loads, each widened two k-steps after its read (half 1 of column
            // block 3 at the start of phase 2).
            if (ks == 1) va[0] = widen(vr[0]);
            if (ks == 2) vr[1] = vraw8(1, 0);
            if (ks == 4) va[1] = widen(vr[1]);
            if (ks == 10) vr[2] = vraw8(2, 0);
            if (ks == 12) va[2] = widen(vr[2]);
            if (ks == 18) vr[3] = vraw8(3, 0);
            if (ks == 20) va[3] = widen(vr[3]);
            if (ks == 12) vr[0] = vraw8(0, 1);
            if (ks == 14) va[0] = widen(vr[0]);
            if (ks == 20) vr[1] = vraw8(1, 1);
            if (ks == 22) va[1] = widen(vr[1]);
            if (ks == 28) vr[2] = vraw8(2, 1);
            if (ks == 30) va[2] = widen(vr[2]);
            if (ks == 35) vr[3] = vraw8(3, 1);
            if (ks == 33) {
              const uint32_t so = (uint32_t)offsetof(Smem<FP8>, sc) + ks3 * 256 + 16 * (lane_id_opaque() >> 5);
#pragma unroll
              for (int g4 = 0; g4 < 4; ++g4) tsc[g4] = *(const f32x4*)((const unsigned char*)&sm + so + 32 * g4);
            }
          }
          if (ks >= 30 && ks < 34) pb[1][ks - 30] = pfrag(ks - 30, 1);
          if (!FP8 && ks % 4 == 1) copy_row(tn, ks / 4, lo.ln);                     // ks = 1, 5, .., 33
          if (FP8 && ks % 8 == 1) copy_row(tn, ks / 8, lo.ln);                      // ks = 1, 9, .., 33
          if constexpr (!FP8) {
            const bf16x8 ka = kq[ks % (kKPf + 1)];
            if (ks == 0)
              score_mfma_first(s, ka, qf[ks]);
            else
              score_mfma(s, ka, qf[ks]);
          } else if (ks % 2 == 0) {
            // Score MFMA j = ks / 2 (the even k-steps; the accumulation MFMAs take the odd
            // ones): k-block j / 2, the queries' high part (j even, B scale 1) or remainder
            // (j odd, B scale 2^-4).  After the high part's MFMA, k-block kb + 2 is read into
            // the slot that k-block kb - 1 left.
            const int j = ks / 2, kb = j / 2;
            const uint32_t one = 127u, sixteenth = 123u;   // E8M0 exponents of 1 and 2^-4
            if (j == 0)
              score8_first(s, k8[0], qh[0], one, one);
            else
              score8(s, k8[kb % 3], j % 2 == 0 ? qh[kb] : ql[kb], one, j % 2 == 0 ? one : sixteenth);
            if (j % 2 == 0 && kb + 2 < kQk / 4)
              k8[(kb + 2) % 3] = __builtin_shufflevector(kraw(2 * kb + 4), kraw(2 * kb + 5), 0, 1, 2, 3, 4, 5, 6, 7);
          }
          if (ks >= 3 && ks % 2 == 1 && ks < 35) {
            const int a = (ks - 3) / 2;
            acc[a] = mfma32(va[a / 4], pb[0][a % 4], acc[a]);
            // E4M3: pinned between the score MFMAs around it (the compiler otherwise sinks
            // these MFMAs, which have no side effects, below the whole score chain).
            if constexpr (FP8) asm volatile("" : "+a"(acc[a]));
          }
        }
        __builtin_amdgcn_sched_barrier(0);

        // Softmax numerators of tile `it`, base 2.  Lane owns head l32 and tokens
        // 8(v/4) + 4h + v%4; tokens at or past `rem` (all, if the tile is not scored)
        // are masked.
        scores_ready(s);
        // E4M3: the per-token scales of tile `it` for this lane's tokens 8 g + 4h + i; the
        // key rows entered the score MFMAs without them, so they multiply the scores here and
        // the probabilities below (value rows).
        if constexpr (FP8) {
#pragma unroll
          for (int v = 0; v < 16; ++v) s[v] *= tsc[v >> 2][v & 3];
        }
        const int tt = t0 + it * kT;
        const int rem = cur ? end - tt : 0;
        if (rem < kT) {
          // Last tile of the piece, or not scored: mask tokens at or past `rem`.
          const int rem_h = rem - 4 * (int)(lane_id_opaque() >> 5);   // recomputed, not kept live
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (8 * (v >> 2) + (v & 3) >= rem_h) s[v] = -INFINITY;
        }
        if (__builtin_amdgcn_readfirstlane(m_ref == -INFINITY ? 1 : 0) && cur) {
          // First scored tile: its maximum becomes the reference of this head (the same
          // tile for every head, since visibility depends only on the token).
          float mx = s[0];
#pragma unroll
          for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[v]);
          m_ref = max_xor32(mx) * qs;
        }
        __builtin_amdgcn_sched_barrier(0);
        const float nm = m_ref == -INFINITY ? 0.f : -m_ref;
        // Phase 2: the other 16 accumulation MFMAs of tile it-1, each followed by a fixed
        // share of the softmax of tile `it` (scale and shift, exponentials, running maximum,
        // bf16 packing and the exchange-buffer stores, the row-sum tree).  The groups keep
        // this order (scheduling barriers), so no run of exponentials or of dependent adds
        // holds up the next MFMA, and every operand was produced at least one group earlier.
        //
        // Token half h of this lane's probabilities is the B operand (head block `wave`,
        // token half h) of the accumulation: it is stored as is.
        // E4M3: the weight that reaches the accumulation is the bf16 rounding w~ of p * scale,
        // so U is divided by the sum of w~ / scale over the same tokens.  Numerator and
        // denominator then agree, and the rounding only perturbs each token's weight by its
        // relative rounding error, as with a bf16 cache; dividing by the sum of the unrounded
        // p instead would scale the whole row by the rounding error of one token's scale when
        // that token dominates.  The lse keeps the unrounded sum (it weights this piece
        // against the others).  A token whose scale is 0 (a tile with no valid page) has
        // w~ = 0.
        unsigned char* pout = (unsigned char*)&sm + lo.pb + (it & 1) * kPBuf + wave * 2 * 1024;
        float x[16], e[16], mx[8], ps[8], rs[FP8 ? 16 : 1];
        bf16x8 pf[2];
        float esum = 0.f;
        auto pack_half = [&](int h) {
#pragma unroll
          for (int j = 0; j < 8; j += 2) {
            const float w0 = FP8 ? e[8 * h + j] * tsc[(8 * h + j) >> 2][j & 3] : e[8 * h + j];
            const float w1 = FP8 ? e[8 * h + j + 1] * tsc[(8 * h + j + 1) >> 2][(j + 1) & 3] : e[8 * h + j + 1];
            const bf16x2 t = pack_bf16(w0, w1);
            pf[h][j] = t[0];
            pf[h][j + 1] = t[1];
          }
          *(bf16x8*)(pout + h * 1024) = pf[h];
        };
        auto eff_sum = [&](int h, int j0) {   // E4M3: w~ / scale of tokens 8h + j0 .. + 3
#pragma unroll
          for (int j = j0; j < j0 + 4; ++j) esum = __builtin_fmaf((float)pf[h][j], rs[8 * h + j], esum);
        };
#pragma unroll
        for (int g = 0; g < 16; ++g) {
          __builtin_amdgcn_sched_barrier(0);
          acc[g] = mfma32(va[g / 4], pb[1][g % 4], acc[g]);
          if (FP8 && g == 1) va[3] = widen(vr[3]);   // first use at g = 12
          if (g < 4) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              x[4 * g + j] = __builtin_fmaf(s[4 * g + j], qs, nm);
              if constexpr (FP8) rs[4 * g + j] = fminf(__builtin_amdgcn_rcpf(tsc[g][j]), 3.0e38f);
            }
          } else if (g < 12) {
            const int k = g - 4;
            e[2 * k] = exp2_fast(x[2 * k]);
            e[2 * k + 1] = exp2_fast(x[2 * k + 1]);
            if (k < 4) {
              mx[2 * k] = fmaxf(x[4 * k], x[4 * k + 1]);
              mx[2 * k + 1] = fmaxf(x[4 * k + 2], x[4 * k + 3]);
            } else if (k == 4) {
              mx[0] = fmaxf(fmaxf(mx[0], mx[1]), mx[2]);
              mx[3] = fmaxf(fmaxf(mx[3], mx[4]), mx[5]);
            } else if (k == 5) {
              x_max = fmaxf(fmaxf(x_max, mx[0]), fmaxf(mx[3], fmaxf(mx[6], mx[7])));
            } else if (k == 6) {
              pack_half(0);                  // e[0..7] exist since k = 3
            } else {
#pragma unroll
              for (int j = 0; j < 4; ++j) ps[j] = e[2 * j] + e[2 * j + 1];
            }
          } else if (g == 12) {
            pack_half(1);                    // e[14], e[15] exist since g = 11
            if constexpr (FP8) eff_sum(0, 0);
          } else if (g == 13) {
#pragma unroll
            for (int j = 4; j < 8; ++j) ps[j] = e[2 * j] + e[2 * j + 1];
            if constexpr (FP8) eff_sum(0, 4);
          } else if (g == 14) {
#pragma unroll
            for (int j = 0; j < 8; j += 2) ps[j] += ps[j + 1];
            if constexpr (FP8) eff_sum(1, 0);
          } else {
            const float psum = (ps[0] + ps[2]) + (ps[4] + ps[6]);
            if constexpr (FP8) eff_sum(1, 4);
            l_part += psum;
            l_eff += FP8 ? esum : psum;
          }
        }
        __builtin_amdgcn_sched_barrier(0);

        ready >>= 1;
        vs = (vs + 1) & (kVRing - 1);
        ks3 = ks3 == kKRing - 1 ? 0 : ks3 + 1;
      }
    };

    run_pass(true);
    // A tile above the reference by more than the headroom: every wave learns it and
    // the piece is recomputed with the exact maximum (over both lane halves of each
    // head) as the reference.
    const bool excess = __any(x_max > kHeadroom);   // vote of all 64 lanes
    if (lane == 0) sm.redo[wave] = excess ? 1 : 0;
    __syncthreads();
    const bool redo = (sm.redo[0] | sm.redo[1] | sm.redo[2] | sm.redo[3]) != 0;
    __syncthreads();
    if (redo) {
      m_ref += max_xor32(x_max);
      run_pass(false);
      wait_vmcnt<0>();
    }
    // No copy is in flight now (the vote's barrier waited for all of this wave's memory
    // operations, the redo pass ends with the same wait), so the tile ring is free.

    // Epilogue: u = U / l.  Row sums go through LDS to the column-owning waves; the
    // barriers from here on wait for LDS operations only, never for the stores.
    const int el = (int)lane_id_opaque(), l32 = el & 31, h = el >> 5;
    const float l_tot = l_part + __shfl_xor(l_part, 32, 64);
    const float l_div = FP8 ? l_eff + __shfl_xor(l_eff, 32, 64) : l_tot;
    if (h == 0) {
      sm.l[32 * wave + l32] = l_div;
      p.part_lse[row_base + 32 * wave + l32] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
    lds_barrier();
    // One head block at a time, each wave stages its columns of u for the block's 32
    // heads in the ring (16-byte chunk c of head row r at c ^ (r % 16)) and, after a
    // barrier, writes 8 whole rows of the block, one 1 KiB store each, while the next
    // block is staged; stores straight from the accumulator layout would write 16 bytes
    // of 32 different rows per instruction.
    const uint32_t el_u = lane_id_opaque();
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const float lt = sm.l[32 * hb + l32];
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const int r = 32 * hb + l32;
      unsigned char* srow = sm.u_stage[r] + 8 * h;
#pragma unroll
      for (int cl = 0; cl < 4; ++cl)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          f32x4 o;
#pragma unroll
          for (int k = 0; k < 4; ++k) o[k] = acc[4 * cl + hb][4 * g4 + k] * inv;
          const int c = 16 * wave + 4 * cl + g4;
          *(bf16x4*)(srow + 16 * (c ^ (r & 15))) = to_bf16x4(o);
        }
      lds_barrier();
      // Written through the L2: the combine launch reads these rows, and left dirty they
      // would be written back at the end of this launch, after its last workgroup.
      const __amdgpu_buffer_rsrc_t ur = buffer_rsrc((const char*)p.part_u + (row_base + 32 * hb + 8 * wave) * (kDc * 2));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int rr = 32 * hb + 8 * wave + i;
        buffer_store16<kCachePolicyWriteThrough>(*(const u32x4*)(sm.u_stage[rr] + 16 * (el_u ^ (uint32_t)(rr & 15))),
                                                 ur, 16 * el_u + (uint32_t)i * (kDc * 2));
      }
    }
    // The next piece's prologue refills ring slots 0 and 1, the row sums and the stash,
    // which other waves may still be reading for this piece.
    lds_barrier();
    first_piece = false;
  });

  // Fused append: the rest of this share's pool writes (sequences w + G, w + 2G, ..).  No
  // tile of this launch reads these rows from the pool.
  if (p.new_c && rg == 0) {
    const uint32_t l = lane_id_opaque();
    const size_t c_row_b = (size_t)p.c_stride * 2, k_row_b = (size_t)p.k_stride * 2;
    for (int b = w + p.num_splits; b < p.batch; b += p.num_splits)
      for (int i = wave; i < p.s_new; i += kWaves) {
        const int tok = b * p.s_new + i;
        const int pos = p.new_pos[tok];
        if (pos < 0) continue;
        const int pidx = pos / p.page_size;
        if (pidx >= p.max_pages) continue;
        const int page = p.block_table[(size_t)b * p.max_pages + pidx];
        if (page < 0 || page >= p.num_pages) continue;
        const size_t slot = (size_t)page * p.page_size + pos % p.page_size;
        const u32x4 c = *(const u32x4*)((const char*)p.new_c + (size_t)tok * kDc * 2 + 16 * l);
        *(u32x4*)((char*)const_cast<void*>(p.c_kv) + slot * c_row_b + 16 * l) = c;
        if (l < kKRow / 16) {
          const u32x4 k = *(const u32x4*)((const char*)p.new_k + (size_t)tok * kDr * 2 + 16 * l);
          *(u32x4*)((char*)const_cast<void*>(p.k_pe) + slot * k_row_b + 16 * l) = k;
        }
      }
  }
}

}  // namespace

hipError_t launch_attn_h128(const AttnParams& p, bool fp8, hipStream_t stream) {
  if (p.n_h % kHeads != 0 || p.d_c != kDc || p.d_r != kDr) return hipErrorInvalidValue;
  if (fp8 && (p.kv_scale == nullptr || p.new_c != nullptr)) return hipErrorInvalidValue;
  dim3 grid(p.num_splits, p.s_q * (p.n_h / kHeads));
  if (fp8) return launch_attention_kernel(attn_partial_h128<true>, grid, dim3(64 * kWaves), stream, p);
  return launch_attention_kernel(attn_partial_h128<false>, grid, dim3(64 * kWaves), stream, p);
}

}  // namespace mla
