// GQLA's per-group decode path (GQLA abstract, chatpaper.ai: the same weights expose an
// MQA-absorb path identical to MLA's and a GQA path with a per-group expanded cache).  The
// heads form n_g equal groups that share the up-projections W^UK_g and W^UV_g; the expanded
// cache holds, per pool slot j and group g, k_{j,g} = W^UK_g c_j and v_{j,g} = W^UV_g c_j
// (made by the projection GEMM), and the position key k^R_j stays in the latent pool.  Head
// i of group g then runs plain attention:
//   s_ij = softmax_scale (q^C_i . k_{j,g} + q^R_i . k^R_j),   o_i = sum_j softmax_j(s_i) v_{j,g}.
//
// One wave per (sequence, group, token split): its rows are the group's heads at every query
// position (row = q * heads_per_group + head, at most 32), 32-token tiles are staged in LDS
// through a register prefetch of the next tile (keys [k_g | k^R] and values v_g, rows
// padded by 16 bytes against bank conflicts), the
// scores S^T[token, row] run on 32x32x16 bf16 MFMAs, an online softmax (running maximum,
// rescaled accumulators) feeds U^T[col, row] += V^T P^T, where each lane's probabilities are
// already its B operand and transposed LDS reads give the V^T operand in the same token order.
// A second kernel merges the splits by log-sum-exp.

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGT = 32;            // tokens per tile
constexpr int kGMaxKD = 256;       // d_h + d_r
constexpr int kGMaxVD = 256;       // d_v

// Orders this workgroup's LDS writes before its LDS reads without waiting for the global
// loads in flight (a full __syncthreads would also wait for the prefetch of the next tile).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ f32x16 mfma32x32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int KD, int VD>
__global__ __launch_bounds__(64) void gqa_decode_partial(const GqaParams p) {
  constexpr int KS = KD / 16;                 // score k-steps
  constexpr int CB = VD / 32;                 // 32-column blocks of the values
  constexpr int KROW = KD * 2 + 16;           // LDS row strides (bytes), padded
  constexpr int VROW = VD * 2 + 16;
  __shared__ __attribute__((aligned(16))) unsigned char ks_lds[kGT * KROW];
  __shared__ __attribute__((aligned(16))) unsigned char vs_lds[kGT * VROW];
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int l32 = lane & 31, h = lane >> 5;
  const int hpg = p.n_h / p.n_g;
  const int R = hpg * p.s_q;
  int L = p.seq_lens[b];
  L = L < 0 ? 0 : (L > p.max_tokens ? p.max_tokens : L);
  const int t0 = split * p.chunk;
  const int t1 = min(L, t0 + p.chunk);

  // Queries of row l32 (masked rows past R use row R - 1 and are never stored): dims
  // 8h + 16ks .. +7 of [q^C | q^R].
  const int row = min(l32, R - 1);
  const int q_pos = row / hpg, head = g * hpg + row % hpg;
  const size_t qrow = ((size_t)b * p.s_q + q_pos) * p.n_h + head;
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int d = 16 * ks + 8 * h;
    qf[ks] = d < p.d_h ? *(const bf16x8*)((const bf16*)p.q_c + qrow * p.d_h + d)
                       : *(const bf16x8*)((const bf16*)p.q_pe + qrow * p.d_r + (d - p.d_h));
  }
  // Last visible token of each of this lane's rows is L - s_q + q_pos.
  const int vis_end = L - p.s_q + q_pos + 1;   // tokens < vis_end are visible to this lane's row

  f32x16 acc[CB];
#pragma unroll
  for (int c = 0; c < CB; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // Tile staging: a 32-token tile lies in one page (tiles start at multiples of 32 and
  // pages hold a multiple of 64 tokens), so one scalar page lookup gives the base slot.
  // Lane l holds 16-byte chunks e = l + 64 i of the tile ([k_g | k^R] rows, then v_g
  // rows); the next tile's chunks are loaded into registers while this one is computed.
  // Tokens past t1 or on an invalid page are zero-filled (and masked below).
  constexpr int KC = KD / 8, VC = VD / 8;
  constexpr int kChunks = kGT * (KC + VC);
  constexpr int kPer = (kChunks + 63) / 64;
  u32x4 pre[kPer];
  auto fetch = [&](int tt) {
    int page = -1;
    if (tt < t1) {
      page = load_scalar(p.block_table + (size_t)b * p.max_pages + tt / p.page_size);
      if (page < 0 || page >= p.num_pages) page = -1;
    }
    const size_t slot0 = page >= 0 ? (size_t)page * p.page_size + tt % p.page_size : 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane + 64 * i;
      const bool kpart = e < kGT * KC;
      const int tok = kpart ? e / KC : (e - kGT * KC) / VC;
      const int c = kpart ? e % KC : (e - kGT * KC) % VC;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (e < kChunks && page >= 0 && tt + tok < t1) {
        const size_t slot = slot0 + tok;
        if (kpart)
          v = 8 * c < p.d_h ? *(const u32x4*)((const bf16*)p.k_exp + (slot * p.n_g + g) * p.d_h + 8 * c)
                            : *(const u32x4*)((const bf16*)p.k_pe + slot * p.k_pe_stride + (8 * c - p.d_h));
        else
          v = *(const u32x4*)((const bf16*)p.v_exp + (slot * p.n_g + g) * VD + 8 * c);
      }
      pre[i] = v;
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = lane + 64 * i;
      if (e >= kChunks) continue;
      if (e < kGT * KC) *(u32x4*)(ks_lds + (e / KC) * KROW + 16 * (e % KC)) = pre[i];
      else *(u32x4*)(vs_lds + ((e - kGT * KC) / VC) * VROW + 16 * ((e - kGT * KC) % VC)) = pre[i];
    }
  };

  if (t0 < t1) fetch(t0);
  for (int tt = t0; tt < t1; tt += kGT) {
    stage();
    fetch(tt + kGT);   // the next tile's loads fly while this one is computed (none past t1)
    lds_sync();
    // S^T[token, row]: lane holds token 8(v/4) + 4h + v%4 of row l32.
    f32x16 s;
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 kf = *(const bf16x8*)(ks_lds + l32 * KROW + 2 * (16 * ks + 8 * h));
      s = mfma32x32(kf, qf[ks], s);
    }
    float x[16];
    float mx = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int t = tt + 8 * (v >> 2) + 4 * h + (v & 3);
      x[v] = (t < t1 && t < vis_end) ? s[v] * p.scale_log2 : -INFINITY;
      mx = fmaxf(mx, x[v]);
    }
    mx = max_xor32(mx);                          // both lane halves hold tokens of row l32
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_use);   // 0 while m_run = -inf
    float psum = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      x[v] = exp2_fast(x[v] - m_use);
      psum += x[v];
    }
    l_run = l_run * alpha + sum_xor32(psum);     // both lane halves' tokens of row l32
    m_run = m_new;
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[c][v] *= alpha;
    // U^T[col, row] += V^T[col, token] P^T[token, row] per token half th: the lane's
    // probabilities p[8 th .. 8 th + 7] are B[k = 8h + j] for token 16 th + 8 (j/4) + 4h + j%4,
    // and two transposed reads give V^T for the same tokens (rows 16 th + 4h' .. +3 and
    // 16 th + 8 + 4h' .. +3 of the tile, h' = lane / 32).
#pragma unroll
    for (int th = 0; th < 2; ++th) {
      bf16x8 pf;
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const bf16x2 t2 = pack_bf16(x[8 * th + j], x[8 * th + j + 1]);
        pf[j] = t2[0];
        pf[j + 1] = t2[1];
      }
      const int blk = lane >> 4, li = lane & 15, r = li >> 2, q4 = li & 3;
      const int tok_lo = 16 * th + 4 * (blk >> 1) + r;
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const int col = 32 * c + 16 * (blk & 1) + 4 * q4;
        const bf16x4 lo = lds_read_tr16(vs_lds + tok_lo * VROW + 2 * col);
        const bf16x4 hi = lds_read_tr16(vs_lds + (tok_lo + 8) * VROW + 2 * col);
        acc[c] = mfma32x32(concat4(lo, hi), pf, acc[c]);
      }
    }
    lds_sync();
  }
  // Partial of this split: u = U / l per row and its lse (natural log); an empty split gives
  // lse = -inf, o = 0.  Lane holds U^T[32c + 8(v/4) + 4h + v%4][l32].
  const size_t prow = (((size_t)b * p.n_g + g) * p.splits + split) * 32 + l32;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  if (l32 < R) {
#pragma unroll
    for (int c = 0; c < CB; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        p.part_o[prow * VD + 32 * c + 8 * (v >> 2) + 4 * h + (v & 3)] = acc[c][v] * inv;
    if (h == 0) p.part_lse[prow] = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
  }
}

// Merge the splits of every (sequence, group) row: lse = ln sum_s e^{lse_s},
// o = sum_s e^{lse_s - lse} o_s; written as [B, s_q, n_h, d_v] (bf16) and lse [B, s_q, n_h].
// Log-sum-exp merge of the splits: one thread per (row, output column), 256 / d_v rows per
// workgroup; the lse values and the partial outputs of 8 splits are loaded together (no
// load waits for another), the maximum and the sum first, then the weighted sum.
__global__ __launch_bounds__(256) void gqa_combine(const GqaParams p) {
  constexpr int kB = 8;
  const int g = blockIdx.y, b = blockIdx.z;
  const int hpg = p.n_h / p.n_g;
  const int R = hpg * p.s_q;
  const int rpw = 256 / p.d_v;
  const int row = blockIdx.x * rpw + (int)threadIdx.x / p.d_v;
  const int col = (int)threadIdx.x % p.d_v;
  if (row >= R) return;
  const size_t base = (((size_t)b * p.n_g + g) * p.splits) * 32 + row;
  float mx = -INFINITY;
  for (int s0 = 0; s0 < p.splits; s0 += kB) {
    float l[kB];
#pragma unroll
    for (int i = 0; i < kB; ++i) l[i] = s0 + i < p.splits ? p.part_lse[base + (size_t)(s0 + i) * 32] : -INFINITY;
#pragma unroll
    for (int i = 0; i < kB; ++i) mx = fmaxf(mx, l[i]);
  }
  float tot = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < p.splits; s0 += kB) {
    float l[kB], o[kB];
#pragma unroll
    for (int i = 0; i < kB; ++i) {
      const bool in = s0 + i < p.splits;
      const size_t r = base + (size_t)(in ? s0 + i : 0) * 32;
      l[i] = in ? p.part_lse[r] : -INFINITY;
      o[i] = p.part_o[r * p.d_v + col];
    }
#pragma unroll
    for (int i = 0; i < kB; ++i)
      if (l[i] != -INFINITY) {
        const float w = __expf(l[i] - mx);
        tot += w;
        acc += w * o[i];
      }
  }
  const int q_pos = row / hpg, head = g * hpg + row % hpg;
  const size_t orow = ((size_t)b * p.s_q + q_pos) * p.n_h + head;
  ((bf16*)p.out)[orow * p.d_v + col] = (bf16)(tot > 0.f ? acc / tot : 0.f);
  if (col == 0 && p.lse) p.lse[orow] = tot > 0.f ? mx + logf(tot) : -INFINITY;
}

}  // namespace

hipError_t launch_gqa_decode(const GqaParams& p, hipStream_t s) {
  dim3 grid(p.splits, p.n_g, p.batch);
  const int kd = p.d_h + p.d_r;
#define MLA_GQA(KD, VD)                                                               \
  if (kd == KD && p.d_v == VD) {                                                      \
    hipLaunchKernelGGL((gqa_decode_partial<KD, VD>), grid, dim3(64), 0, s, p);        \
  } else
  MLA_GQA(192, 128) MLA_GQA(32, 32) MLA_GQA(64, 64) { return hipErrorInvalidValue; }
#undef MLA_GQA
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 cgrid((32 + 256 / p.d_v - 1) / (256 / p.d_v), p.n_g, p.batch);
  hipLaunchKernelGGL(gqa_combine, cgrid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mla
