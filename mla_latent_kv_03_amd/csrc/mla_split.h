// Device side of the split rule: every workgroup derives, from seq_lens alone, the
// pieces of the batch that its share covers, and the owner of each sequence
// writes that sequence's (first slot, count) entry of the split table.
//
// Rule: sequence b has n_b = ceil(L_b / 64) units; the units of all sequences, in
// batch order, are cut into G shares of ceil(U / G) units (U = sum n_b).  Share w
// meets sequence b in at most one piece, stored in slot w + b.
#pragma once

#include "mla_device.h"

namespace mla {

constexpr int kSplitUnit = 64;

struct Piece {
  int b;      // sequence
  int t0;     // first token (multiple of 64)
  int t1;     // one past the last token (<= L_b)
  int slot;   // partial slot = share + b
};

struct SplitScratch {
  long long wave_sums[17];
};

__device__ __forceinline__ int clamp_len(int L, int max_tokens) {
  return L < 0 ? 0 : (L > max_tokens ? max_tokens : L);
}

// Exclusive prefix sum of v over the workgroup (blockDim.x a multiple of 64, <= 1024).
// Every thread must call it; `total` receives the workgroup sum.
__device__ inline long long block_exclusive_scan(long long v, SplitScratch* s, long long& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  long long x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    long long y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) s->wave_sums[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    long long acc = 0;
    for (int i = 0; i < nw; ++i) {
      long long t = s->wave_sums[i];
      s->wave_sums[i] = acc;
      acc += t;
    }
    s->wave_sums[16] = acc;
  }
  __syncthreads();
  long long excl = s->wave_sums[wave] + x - v;
  total = s->wave_sums[16];
  __syncthreads();
  return excl;
}

// Walks the batch in chunks of blockDim.x sequences.  For each chunk it collects the
// pieces of share w into `pieces` (LDS, blockDim.x entries) and calls process(piece)
// for each, with the whole workgroup, in sequence order.  If table != nullptr the
// workgroup also writes the split-table entries of the sequences b with b % G == w.
template <class F>
__device__ void for_each_piece(const int32_t* __restrict__ seq_lens, int B, int max_tokens, int G, int w,
                               int32_t* __restrict__ table, SplitScratch* s, Piece* pieces, F&& process) {
  const int nt = blockDim.x, tid = threadIdx.x;
  long long local = 0;
  for (int b = tid; b < B; b += nt) local += (clamp_len(seq_lens[b], max_tokens) + kSplitUnit - 1) / kSplitUnit;
  long long total;
  (void)block_exclusive_scan(local, s, total);
  if (total == 0) {
    if (table)
      for (int b = tid; b < B; b += nt)
        if (b % G == w) { table[2 * b] = 0; table[2 * b + 1] = 0; }
    return;
  }
  const long long share = (total + G - 1) / G;
  const long long lo = (long long)w * share;
  const long long hi = lo + share < total ? lo + share : total;
  long long carry = 0;
  for (int base = 0; base < B; base += nt) {
    const int b = base + tid;
    const int L = b < B ? clamp_len(seq_lens[b], max_tokens) : 0;
    const long long n = (L + kSplitUnit - 1) / kSplitUnit;
    long long chunk_total;
    const long long start = carry + block_exclusive_scan(n, s, chunk_total);
    if (table && b < B && b % G == w) {
      int first = 0, cnt = 0;
      if (n > 0) {
        const long long wf = start / share, wl = (start + n - 1) / share;
        first = (int)wf + b;
        cnt = (int)(wl - wf + 1);
      }
      table[2 * b] = first;
      table[2 * b + 1] = cnt;
    }
    const bool mine = n > 0 && start < hi && start + n > lo;
    long long np_ll;
    const int idx = (int)block_exclusive_scan(mine ? 1 : 0, s, np_ll);   // rank among this chunk's pieces
    const int np = (int)np_ll;
    if (mine) {
      const long long u0 = (lo > start ? lo : start) - start;
      const long long u1 = (hi < start + n ? hi : start + n) - start;
      Piece pc;
      pc.b = b;
      pc.t0 = (int)(u0 * kSplitUnit);
      pc.t1 = (int)(u1 * kSplitUnit < L ? u1 * kSplitUnit : L);
      pc.slot = w + b;
      pieces[idx] = pc;
    }
    __syncthreads();
    for (int i = 0; i < np; ++i) process(pieces[i]);
    carry += chunk_total;
    __syncthreads();
    if (!table && carry >= hi) break;
  }
}

}  // namespace mla
