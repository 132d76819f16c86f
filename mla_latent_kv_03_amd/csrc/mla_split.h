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

__device__ __forceinline__ long long wave_inclusive_scan(long long x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const long long y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

__device__ __forceinline__ long long wave_total(long long x) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
  return x;
}

// Same walk as for_each_piece, done by each wave on its own (64 sequences per step,
// wave-level scans, no LDS and no barriers): every wave of a workgroup derives the
// identical piece list and calls process(piece) in the same order with wave-uniform
// values.  The wave given a non-null `table` also writes the split-table entries of
// the sequences b with b % G == w.
template <class F>
__device__ void for_each_piece_wave(const int32_t* __restrict__ seq_lens, int B, int max_tokens, int G, int w,
                                    int32_t* __restrict__ table, F&& process) {
  const int lane = threadIdx.x & 63;
  long long total = 0;
  for (int base = 0; base < B; base += 64) {
    const int b = base + lane;
    total += wave_total(b < B ? (clamp_len(seq_lens[b], max_tokens) + kSplitUnit - 1) / kSplitUnit : 0);
  }
  if (total == 0) {
    if (table)
      for (int b = lane; b < B; b += 64)
        if (b % G == w) { table[2 * b] = 0; table[2 * b + 1] = 0; }
    return;
  }
  const long long share = (total + G - 1) / G;
  const long long lo = (long long)w * share;
  const long long hi = lo + share < total ? lo + share : total;
  long long carry = 0;
  for (int base = 0; base < B; base += 64) {
    const int b = base + lane;
    const int L = b < B ? clamp_len(seq_lens[b], max_tokens) : 0;
    const long long n = (L + kSplitUnit - 1) / kSplitUnit;
    const long long incl = wave_inclusive_scan(n);
    const long long start = carry + incl - n;
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
    const long long u0 = (lo > start ? lo : start) - start;
    const long long u1 = (hi < start + n ? hi : start + n) - start;
    const int t0 = (int)(u0 * kSplitUnit);
    const int t1 = (int)(u1 * kSplitUnit < L ? u1 * kSplitUnit : L);
    unsigned long long mask = __ballot(mine);
    while (mask) {
      const int src = __builtin_ctzll(mask);
      mask &= mask - 1;
      Piece pc;
      pc.b = __builtin_amdgcn_readlane(b, src);
      pc.t0 = __builtin_amdgcn_readlane(t0, src);
      pc.t1 = __builtin_amdgcn_readlane(t1, src);
      pc.slot = w + pc.b;
      process(pc);
    }
    carry += __shfl(incl, 63, 64);
    if (!table && carry >= hi) break;
  }
}

// Block-table entries of one sequence held in registers: lane j of the wave keeps the
// page id of logical page base + j (or -1 when that id is outside [0, num_pages) or
// past the table row), so looking a page up is a register read instead of a memory
// round trip.  The window slides forward (one coalesced load) when a lookup passes
// its end; lookups must not go back more than 32 pages behind the furthest one.
struct PageWindow {
  const int32_t* row;   // block_table + b * max_pages
  int max_pages, num_pages;
  int base;
  int ids;              // this lane's page id

  __device__ void load(int new_base) {
    base = new_base;
    const int lane = threadIdx.x & 63;
    const int k = base + lane;
    int id = -1;
    if (k < max_pages) {
      id = row[k];
      if (id < 0 || id >= num_pages) id = -1;
    }
    ids = id;
  }
  __device__ void init(const int32_t* row_, int max_pages_, int num_pages_, int first_page) {
    row = row_;
    max_pages = max_pages_;
    num_pages = num_pages_;
    load(first_page);
  }
  // page id of logical page `page_idx` (wave-uniform), -1 if invalid
  __device__ int get(int page_idx) {
    if (page_idx >= base + 64) load(page_idx - 32 > base ? page_idx - 32 : base + 32);
    return __builtin_amdgcn_readlane(ids, page_idx - base);
  }
};

}  // namespace mla
