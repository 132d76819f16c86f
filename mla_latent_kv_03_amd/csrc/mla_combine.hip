// Log-sum-exp combine of split partials and the per-head up-projection.
//
// For every row (b, q) and head i, over the sequence's slots s (split table):
//   lse = ln sum_s exp(lse_s)              (largest finite lse_s subtracted first)
//   u   = sum_s exp(lse_s - lse) u_s       (softmax over a union of disjoint token sets)
//   o_i = W^UV_i u                         (page "MLA deep compression", output-side
//                                           absorption: u_i is formed in latent space,
//                                           then up-projected once)
// bf16 weights: one workgroup per (head, block of rows), u merged into LDS and then
// multiplied by W^UV_i^T on MFMAs (details below).  float32 weights: plain FMA loops.

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {
namespace {

__device__ __forceinline__ void slot_range(const CombineParams& p, int b, int& first, int& count) {
  first = p.split_table[2 * b];
  count = p.split_table[2 * b + 1];
  if (first < 0 || first >= p.num_slots || count <= 0) { first = 0; count = 0; return; }
  if (count > p.num_slots - first) count = p.num_slots - first;
}

constexpr int kDc = 512;
constexpr int kDv = 128;
constexpr int kCombineWaves = 8;

// LDS position (bf16 elements) of latent column k of tile row i: 16-byte chunk k/8 is
// stored at (k/8) ^ (i % 16), so an MFMA operand read (16 rows, one chunk each) hits
// 16 different bank groups.
__device__ __forceinline__ int u_pos(int i, int k) { return i * kDc + ((((k >> 3) ^ (i & 15))) << 3) + (k & 7); }

// bf16 weights: one workgroup per (head, RB rows).
//  Phase 1 merges the u of the RB rows.  A unit is (row, half row): lane l of the
//  wave that owns it holds latent columns 256 h + 4 l .. +3.  With RB >= 4 each wave
//  owns M = RB / 4 units; with RB < 4 the P = 8 / (2 RB) waves of a unit take every
//  P-th slot and their sums are added in a fixed order through LDS.  Every load of the
//  workgroup is issued before the first merge: the W^UV_i rows of phase 2 (their
//  addresses need nothing loaded), then, once the split table has come through the
//  scalar cache, the slot lse values (one slot per lane) and the first kS partial slices
//  of every unit (M kS = 32 per wave; slots past a unit's count re-read its last slot and
//  get weight 0).  So the whole working set of a workgroup is in flight at once and the
//  merge only waits for its own data.  Partial slices are read with the streaming
//  (non-temporal) policy.  u enters the product as a bf16 high part plus a bf16
//  remainder (about 16 significant bits).
//  Phase 2: O[RB x 128] = U W^UV_i^T on 16x16x32 MFMAs; wave w owns output columns
//  16 w .. 16 w + 15.
//  EARLY_W: the W^UV rows are loaded first, with everything else (one workgroup per CU);
//  otherwise after the merge, so that the merge's registers and W^UV's are not live together
//  and two workgroups fit on a CU (grids of more than one workgroup per CU).
template <int RB, bool EARLY_W>
__device__ __forceinline__ void combine_upproj_body(const CombineParams& p) {
  constexpr int kUnits = 2 * RB;
  constexpr int P = kUnits >= kCombineWaves ? 1 : kCombineWaves / kUnits;   // waves per unit
  constexpr int M = kUnits >= kCombineWaves ? kUnits / kCombineWaves : 1;   // units per wave
  constexpr int kS = 32 / M;                                                  // slices per unit in flight
  constexpr int kTileRows = RB < 16 ? 16 : RB;
  __shared__ __attribute__((aligned(16))) bf16 u_hi[kTileRows * kDc];
  __shared__ __attribute__((aligned(16))) bf16 u_lo[kTileRows * kDc];
  __shared__ __attribute__((aligned(16))) f32x4 red[P > 1 ? kCombineWaves : 1][64];
  const int head = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int R = p.batch * p.s_q;
  const int row0 = blockIdx.y * RB;
  const int nrows = min(RB, R - row0);
  const int part = wave % P;
  const size_t step = (size_t)p.s_q * p.n_h;                 // partial rows per slot
  const size_t slot_bytes = step * kDc * sizeof(bf16);

  bf16x8 bw[kDc / 32];
  auto load_w = [&]() {
    const bf16* wrow = (const bf16*)p.w_uv + ((size_t)head * kDv + 16 * wave + l16) * kDc + 8 * g;
#pragma unroll
    for (int kk = 0; kk < kDc / 32; ++kk) bw[kk] = *(const bf16x8*)(wrow + kk * 32);
  };
  if (EARLY_W && p.w_uv) load_w();

  // Units of this wave: m-th unit u = wave / P (P > 1) or wave + 8 m; row u / 2, half u % 2.
  // The split-table entries are loaded unconditionally (rows past the block clamp to the
  // last sequence) and checked afterwards, so that the scalar loads of all units are in
  // flight together.
  int u_row[M], u_half[M], u_cnt[M], u_first[M];
  size_t u_base[M];   // partial row of the unit's first slot
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int u = P > 1 ? wave / P : wave + kCombineWaves * m;
    u_row[m] = u >> 1;
    u_half[m] = u & 1;
    const int b = min((row0 + u_row[m]) / p.s_q, p.batch - 1);
    u_first[m] = load_scalar(p.split_table + 2 * b);
    u_cnt[m] = load_scalar(p.split_table + 2 * b + 1);
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
    int first = u_first[m], count = u_cnt[m];
    const bool bad = u_row[m] >= nrows || first < 0 || first >= p.num_slots || count <= 0;
    first = bad ? 0 : first;                                  // slots clipped to the pool
    count = bad ? 0 : min(count, p.num_slots - first);
    u_cnt[m] = count;
    u_base[m] = ((size_t)first * p.s_q + (row0 + u_row[m]) % p.s_q) * p.n_h + head;
  }
  // Merge layout: lane (vm, vs) = (lane / L, lane % L) holds slot vs of unit vm, so one
  // load brings the slot lse values of all the wave's units and the maximum and the sum
  // are segmented lane reductions.  A unit with more than L slots sends the wave to the
  // per-unit merge below.
  constexpr int L = 64 / M;
  const int vm = lane / L, vs = lane % L;
  int v_cnt = u_cnt[0], v_row = u_row[0], v_half = u_half[0];
  size_t v_base = u_base[0];
#pragma unroll
  for (int m = 1; m < M; ++m)
    if (vm == m) { v_cnt = u_cnt[m]; v_row = u_row[m]; v_half = u_half[m]; v_base = u_base[m]; }
  bool all_fit = true;
#pragma unroll
  for (int m = 0; m < M; ++m) all_fit = all_fit && u_cnt[m] <= L;
  const float v_l = vs < v_cnt ? p.part_lse[v_base + vs * step] : -INFINITY;
  bf16x4 u_v[M][kS];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const char* src = (const char*)((const bf16*)p.part_u + u_base[m] * kDc + 256 * u_half[m]) + 8 * lane;
    const int last = u_cnt[m] > 0 ? u_cnt[m] - 1 : 0;
#pragma unroll
    for (int k = 0; k < kS; ++k) {
      const int s = min(part + P * k, last);
      u_v[m][k] = __builtin_nontemporal_load((const bf16x4*)(src + (size_t)s * slot_bytes));
    }
  }

  // Weights w = exp(lse_s - lse) of the merge layout's slots (all units at once).
  float v_w = 0.f;
  if (all_fit) {
    float x = v_l;
#pragma unroll
    for (int o = L / 2; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    const float e = v_l == -INFINITY ? 0.f : exp2_fast((v_l - x) * kLog2e);
    float tot = e;
#pragma unroll
    for (int o = L / 2; o >= 1; o >>= 1) tot += __shfl_xor(tot, o, 64);
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    if (p.lse && vs == 0 && v_half == 0 && part == 0 && v_row < nrows)
      p.lse[(size_t)(row0 + v_row) * p.n_h + head] = tot > 0.f ? x + logf(tot) : -INFINITY;
    v_w = e * inv;
  }
  // u of unit m: its slices weighted by the merge layout's weights (lane L m + slot).
  auto accumulate = [&](int m) {
    const int cnt = u_cnt[m];
    auto weight = [&](int s) -> float { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v_w), L * m + s)); };
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kS; ++k) {
      const int s = part + P * k;
      if (s < cnt) acc += weight(s) * from_bf16x4(u_v[m][k]);
    }
    // Slots past the first kS of this wave (at most L in all): further batches of kS loads.
    const char* src = (const char*)((const bf16*)p.part_u + u_base[m] * kDc + 256 * u_half[m]) + 8 * lane;
    for (int j0 = kS; part + P * j0 < cnt; j0 += kS) {
      bf16x4 v[kS];
#pragma unroll
      for (int k = 0; k < kS; ++k) {
        const int s = min(part + P * (j0 + k), cnt - 1);
        v[k] = __builtin_nontemporal_load((const bf16x4*)(src + (size_t)s * slot_bytes));
      }
#pragma unroll
      for (int k = 0; k < kS; ++k) {
        const int s = part + P * (j0 + k);
        if (s < cnt) acc += weight(s) * from_bf16x4(v[k]);
      }
    }
    return acc;
  };
  // Per-unit merge (a unit with more than L slots): slot = lane, 64 at a time, the maximum
  // and the sum over wave-uniform values read back lane by lane.
  auto finish = [&](int m) {
    const int cnt = u_cnt[m];
    const size_t base = u_base[m];
    const float l = lane < cnt ? p.part_lse[base + lane * step] : -INFINITY;
    const int c64 = min(cnt, 64);
    float x = -INFINITY;
    for (int s = 0; s < c64; ++s) x = fmaxf(x, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), s)));
    if (cnt > 64) {
      float y = x;
      for (int s = 64 + lane; s < cnt; s += 64) y = fmaxf(y, p.part_lse[base + s * step]);
      x = wave_max(y);
    }
    const float e = l == -INFINITY ? 0.f : exp2_fast((l - x) * kLog2e);
    float tot = 0.f;
    for (int s = 0; s < c64; ++s) tot += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e), s));
    if (cnt > 64) {
      float t = 0.f;
      for (int s = 64 + lane; s < cnt; s += 64) {
        const float ls = p.part_lse[base + s * step];
        if (ls != -INFINITY) t += exp2_fast((ls - x) * kLog2e);
      }
      tot += wave_sum(t);
    }
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    if (p.lse && u_half[m] == 0 && part == 0 && lane == 0 && u_row[m] < nrows)
      p.lse[(size_t)(row0 + u_row[m]) * p.n_h + head] = tot > 0.f ? x + logf(tot) : -INFINITY;
    const float w = e * inv;
    auto weight = [&](int s) -> float {
      if (s < 64) return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), s));
      const float ls = p.part_lse[base + s * step];
      return ls == -INFINITY ? 0.f : exp2_fast((ls - x) * kLog2e) * inv;
    };
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kS; ++k) {
      const int s = part + P * k;
      if (s < cnt) acc += weight(s) * from_bf16x4(u_v[m][k]);
    }
    // Slots past the first kS of this wave: further batches of kS loads.
    const char* src = (const char*)((const bf16*)p.part_u + base * kDc + 256 * u_half[m]) + 8 * lane;
    for (int j0 = kS; part + P * j0 < cnt; j0 += kS) {
      bf16x4 v[kS];
#pragma unroll
      for (int k = 0; k < kS; ++k) {
        const int s = min(part + P * (j0 + k), cnt - 1);
        v[k] = __builtin_nontemporal_load((const bf16x4*)(src + (size_t)s * slot_bytes));
      }
#pragma unroll
      for (int k = 0; k < kS; ++k) {
        const int s = part + P * (j0 + k);
        if (s < cnt) acc += weight(s) * from_bf16x4(v[k]);
      }
    }
    return acc;
  };
  auto store_u = [&](int i, int hh, f32x4 a) {
    if (!p.w_uv) {
      // No up-projection: the merged latents go out as float32 [B, s_q, n_h, d_c].
      if (i < nrows) *(f32x4*)((float*)p.out + ((size_t)(row0 + i) * p.n_h + head) * kDc + 256 * hh + 4 * lane) = a;
      return;
    }
    bf16x4 hi, lo;
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      const bf16x2 h = pack_bf16(a[j], a[j + 1]);
      const bf16x2 rmd = pack_bf16(a[j] - (float)h[0], a[j + 1] - (float)h[1]);
      hi[j] = h[0]; hi[j + 1] = h[1];
      lo[j] = rmd[0]; lo[j + 1] = rmd[1];
    }
    const int pos = u_pos(i, 256 * hh + 4 * lane);
    *(bf16x4*)(u_hi + pos) = hi;
    *(bf16x4*)(u_lo + pos) = lo;
  };

  if (P > 1) {
    red[P > 1 ? wave : 0][lane] = all_fit ? accumulate(0) : finish(0);
    __syncthreads();
    if (part == 0) {
      f32x4 a = red[P > 1 ? wave : 0][lane];
#pragma unroll
      for (int k = 1; k < P; ++k) a += red[P > 1 ? wave + k : 0][lane];
      store_u(u_row[0], u_half[0], a);
    }
  } else {
#pragma unroll
    for (int m = 0; m < M; ++m) store_u(u_row[m], u_half[m], all_fit ? accumulate(m) : finish(m));
  }
  if (!EARLY_W && p.w_uv) load_w();
  __syncthreads();
  if (!p.w_uv) return;   // kernel-uniform

  // O[rows, v] = U[rows, k] W^T[k, v]; lane holds O[row 4g + i][v = 16 wave + l16].
  // Tile rows past the block's last row hold stale values; they only reach outputs
  // that are not stored.
  bf16* out = (bf16*)p.out;
#pragma unroll 1
  for (int rb = 0; rb < kTileRows / 16; ++rb) {
    if (16 * rb >= nrows) break;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < kDc / 32; ++kk) {
      const int pos = u_pos(16 * rb + l16, 32 * kk + 8 * g);
      o = mfma16x16x32(*(const bf16x8*)(u_hi + pos), bw[kk], o);
      o = mfma16x16x32(*(const bf16x8*)(u_lo + pos), bw[kk], o);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ri = 16 * rb + 4 * g + i;
      if (ri < nrows) out[((size_t)(row0 + ri) * p.n_h + head) * kDv + 16 * wave + l16] = (bf16)o[i];
    }
  }
}

template <int RB>
__global__ __launch_bounds__(64 * kCombineWaves) void combine_upproj_bf16(const CombineParams p) {
  combine_upproj_body<RB, true>(p);
}
template <int RB>
__global__ __launch_bounds__(64 * kCombineWaves) __attribute__((amdgpu_waves_per_eu(4, 4)))
void combine_upproj_bf16_2pc(const CombineParams p) {
  combine_upproj_body<RB, false>(p);
}

// float32 path: one workgroup per (head, 16 rows), any d_c <= 1024 and d_v.
constexpr int kF32Rows = 16;
constexpr int kF32MaxDc = 1024;

__global__ __launch_bounds__(256) void combine_upproj_f32(const CombineParams p) {
  __shared__ float u_s[kF32Rows][kF32MaxDc];
  const int head = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int R = p.batch * p.s_q;
  for (int rr = wave; rr < kF32Rows; rr += 4) {
    const int r = blockIdx.y * kF32Rows + rr;
    if (r >= R) continue;
    const int b = r / p.s_q, q = r - b * p.s_q;
    int first, count;
    slot_range(p, b, first, count);
    float mx = -INFINITY;
    for (int s = lane; s < count; s += 64)
      mx = fmaxf(mx, p.part_lse[((size_t)(first + s) * p.s_q + q) * p.n_h + head]);
    mx = wave_max(mx);
    float tot = 0.f;
    for (int s = lane; s < count; s += 64) {
      const float l = p.part_lse[((size_t)(first + s) * p.s_q + q) * p.n_h + head];
      if (l != -INFINITY) tot += expf(l - mx);
    }
    tot = wave_sum(tot);
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    if (lane == 0 && p.lse) p.lse[(size_t)r * p.n_h + head] = tot > 0.f ? mx + logf(tot) : -INFINITY;
    for (int k = lane; k < p.d_c; k += 64) {
      float acc = 0.f;
      for (int s = 0; s < count; ++s) {
        const size_t prow = ((size_t)(first + s) * p.s_q + q) * p.n_h + head;
        const float l = p.part_lse[prow];
        if (l != -INFINITY) acc = fmaf(expf(l - mx) * inv, ((const float*)p.part_u)[prow * p.d_c + k], acc);
      }
      u_s[rr][k] = acc;
      if (!p.w_uv) ((float*)p.out)[((size_t)r * p.n_h + head) * p.d_c + k] = acc;
    }
  }
  if (!p.w_uv) return;   // kernel-uniform: the merged latents were the output
  __syncthreads();
  const float* wh = (const float*)p.w_uv + (size_t)head * p.d_v * p.d_c;
  float* out = (float*)p.out;
  for (int idx = threadIdx.x; idx < kF32Rows * p.d_v; idx += blockDim.x) {
    const int rr = idx / p.d_v, v = idx - rr * p.d_v;
    const int r = blockIdx.y * kF32Rows + rr;
    if (r >= R) continue;
    float acc = 0.f;
    for (int k = 0; k < p.d_c; ++k) acc = fmaf(wh[(size_t)v * p.d_c + k], u_s[rr][k], acc);
    out[((size_t)r * p.n_h + head) * p.d_v + v] = acc;
  }
}

}  // namespace

hipError_t launch_combine_bf16(const CombineParams& p, hipStream_t stream) {
  const int R = p.batch * p.s_q;
  // Largest row block (<= 32) that still gives at least 256 workgroups.
  int rb = 32;
  while (rb > 1 && (long long)p.n_h * ((R + rb - 1) / rb) < 256) rb /= 2;
  dim3 grid(p.n_h, (R + rb - 1) / rb);
  dim3 block(64 * kCombineWaves);
  if (rb == 32 && (long long)grid.x * grid.y > 256) {
    // More workgroups than CUs: the variant that fits two per CU.
    hipLaunchKernelGGL(combine_upproj_bf16_2pc<32>, grid, block, 0, stream, p);
    return hipGetLastError();
  }
  switch (rb) {
    case 32: hipLaunchKernelGGL(combine_upproj_bf16<32>, grid, block, 0, stream, p); break;
    case 16: hipLaunchKernelGGL(combine_upproj_bf16<16>, grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL(combine_upproj_bf16<8>, grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL(combine_upproj_bf16<4>, grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL(combine_upproj_bf16<2>, grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL(combine_upproj_bf16<1>, grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_combine_f32(const CombineParams& p, hipStream_t stream) {
  const int R = p.batch * p.s_q;
  dim3 grid(p.n_h, (R + kF32Rows - 1) / kF32Rows);
  hipLaunchKernelGGL(combine_upproj_f32, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
