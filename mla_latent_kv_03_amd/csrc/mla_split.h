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
  int len;    // L_b (clamped)
  bool last;  // the share ends within this sequence: no later piece (set by for_each_piece_wave)
};

struct SplitScratch {
  long long wave_sums[17];
};

__device__ __forceinline__ int clamp_len(int L, int max_tokens) {
  return L < 0 ? 0 : (L > max_tokens ? max_tokens : L);
}

// Units of a clamped length (at most 2^25, so a sum over 64 sequences fits 32 bits).
__device__ __forceinline__ unsigned units_of(int L) { return ((unsigned)L + (kSplitUnit - 1)) / kSplitUnit; }

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
  for (int b = tid; b < B; b += nt) local += units_of(clamp_len(seq_lens[b], max_tokens));
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
    const long long n = units_of(L);
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
      pc.len = L;
      pieces[idx] = pc;
    }
    __syncthreads();
    for (int i = 0; i < np; ++i) process(pieces[i]);
    carry += chunk_total;
    __syncthreads();
    if (!table && carry >= hi) break;
  }
}

// The lane index from an instruction the compiler cannot look through: addresses built
// from it are computed where they are used, instead of being hoisted out of loops and
// kept live (or spilled) across a kernel's main loop.
__device__ __forceinline__ uint32_t lane_id_opaque() {
  uint32_t l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Inclusive prefix sum over the 64 lanes of a wave, in 32 bits: sums within each row of
// 16 lanes by DPP row shifts of 1, 2, 4 and 8 lanes, then the totals of rows 0 and 2 are
// broadcast into rows 1 and 3, and the total of rows 0-1 into rows 2 and 3.  Lanes that a
// shift or broadcast does not reach take 0.  (Six dependent VALU steps instead of six
// rounds of cross-lane permutes through LDS.)
__device__ __forceinline__ unsigned wave_inclusive_scan_u32(unsigned x) {
  x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Lengths of sequences 0..63 as loaded (not clamped; lanes past the batch read sequence
// B - 1), which a kernel can request before other set-up work and hand to
// for_each_piece_wave.  The load is unconditional so that nothing waits for it before
// the walk uses it (a load under a lane condition is waited for where the branch joins).
__device__ __forceinline__ int first_lens(const int32_t* __restrict__ seq_lens, int B, int max_tokens) {
  (void)max_tokens;
  const int lane = threadIdx.x & 63;
  return seq_lens[lane < B ? lane : B - 1];
}

// Quotient of 64-bit values that usually fit in 32 bits (the 32-bit division is a few
// instructions, the 64-bit one a long software sequence).
__device__ __forceinline__ unsigned long long udiv_mostly32(unsigned long long a, unsigned long long d) {
  return (a | d) >> 32 ? a / d : (unsigned long long)((unsigned)a / (unsigned)d);
}

// Same rule as for_each_piece, evaluated by each wave on its own (64 sequences per
// step, wave-level scans, no LDS and no barriers): every wave of a workgroup derives
// the identical piece list and calls process(piece) in sequence order with
// wave-uniform values.  The wave given a non-null `table` also writes the split-table
// entries of the sequences b with b % G == w.  `len0` is first_lens() of the same
// arguments (sequences 0..63 are then not loaded again).
//
// The pieces are found one at a time: each search rescans the lengths and returns the
// first piece after a scalar cursor, so that no per-lane state of the scan stays live
// while process() runs (a kernel's main loop then has the vector registers to itself).
// A piece whose sequence reaches the share's end is the share's last: no search follows
// it (one piece per share is the common case).
template <class F>
__device__ void for_each_piece_wave(const int32_t* __restrict__ seq_lens, int B, int max_tokens, int G, int w,
                                    int32_t* __restrict__ table, int len0, F&& process) {
  const int lane = threadIdx.x & 63;
  // Lengths of sequences base .. base + 63.  The first search takes sequences 0..63 from
  // len0 (loaded at kernel entry), so that for batches of up to 64 it loads nothing and
  // waits for nothing (a wait for a vector load also waits for the caller's copies issued
  // before it).  Every other block, and every later search, loads its lengths where they
  // are used: len0 and what derives from it are then not live across process() (they were
  // spilled, and the reloads' waits also waited for the copies and stores in flight).
  auto len_of = [&](int base, bool from_len0) {
    const int b = base + lane;
    const int raw = from_len0 ? len0 : seq_lens[b < B ? b : B - 1];
    return b < B ? clamp_len(raw, max_tokens) : 0;
  };
  auto wave_sum = [](unsigned incl) { return (unsigned)__builtin_amdgcn_readlane((int)incl, 63); };
  unsigned long long total = wave_sum(wave_inclusive_scan_u32(units_of(len_of(0, true))));
  for (int base = 64; base < B; base += 64) total += wave_sum(wave_inclusive_scan_u32(units_of(len_of(base, false))));
  const unsigned long long share = total > 0 ? udiv_mostly32(total - 1, (unsigned)G) + 1 : 1;
  const unsigned long long lo = (unsigned long long)w * share;
  const unsigned long long hi = lo + share < total ? lo + share : total;

  if (table) {
    auto table_block = [&](int base, bool from_len0, unsigned long long& carry) {
      const int b = base + lane;
      const unsigned n = units_of(len_of(base, from_len0));
      const unsigned incl = wave_inclusive_scan_u32(n);
      const unsigned long long start = carry + (incl - n);
      if (b < B && (unsigned)b % (unsigned)G == (unsigned)w) {
        int first = 0, cnt = 0;
        if (n > 0) {
          const unsigned long long wf = udiv_mostly32(start, share), wl = udiv_mostly32(start + n - 1, share);
          first = (int)wf + b;
          cnt = (int)(wl - wf + 1);
        }
        table[2 * b] = first;
        table[2 * b + 1] = cnt;
      }
      carry += wave_sum(incl);
    };
    unsigned long long carry = 0;
    table_block(0, true, carry);
    for (int base = 64; base < B; base += 64) table_block(base, false, carry);
  }
  if (total == 0) return;

  // Looks for the share's first piece in sequences base .. base + 63 after `after`:
  // 1 = found (pc filled), 2 = the share ends before the next block, 0 = go on.
  auto try_block = [&](int base, bool from_len0, int after, unsigned long long& carry, Piece& pc) -> int {
    const int b = base + lane;
    const int L = len_of(base, from_len0);
    const unsigned n = units_of(L);
    const unsigned incl = wave_inclusive_scan_u32(n);
    const unsigned long long start = carry + (incl - n);
    const bool mine = b > after && n > 0 && start < hi && start + n > lo;
    const unsigned long long mask = __ballot(mine);
    if (mask) {
      const int src = __builtin_ctzll(mask);
      const unsigned u0 = (unsigned)((lo > start ? lo : start) - start);
      const unsigned u1 = (unsigned)((hi < start + n ? hi : start + n) - start);
      const unsigned long long e = (unsigned long long)u1 * kSplitUnit;
      pc.b = base + src;
      pc.t0 = __builtin_amdgcn_readlane((int)(u0 * kSplitUnit), src);
      pc.t1 = __builtin_amdgcn_readlane(e < (unsigned long long)L ? (int)e : L, src);
      pc.len = __builtin_amdgcn_readlane(L, src);
      pc.slot = w + pc.b;
      pc.last = __builtin_amdgcn_readlane(start + n >= hi ? 1 : 0, src) != 0;
      return 1;
    }
    carry += wave_sum(incl);
    return carry >= hi ? 2 : 0;
  };
  // First piece of share w in a sequence after `after`; false if there is none.
  auto next_piece = [&](int after, Piece& pc, bool first_search) {
    unsigned long long carry = 0;
    int r = try_block(0, first_search, after, carry, pc);
    for (int base = 64; r == 0 && base < B; base += 64) r = try_block(base, false, after, carry, pc);
    return r == 1;
  };
  Piece pc;
  if (!next_piece(-1, pc, true)) return;
  for (;;) {
    process(pc);
    if (pc.last || !next_piece(pc.b, pc, false)) break;
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

  // The loaded ids are checked only in get(), so that the load's latency can overlap
  // whatever the caller issues next.
  __device__ void load(int new_base) {
    base = new_base;
    const int lane = threadIdx.x & 63;
    const int k = base + lane;
    ids = k < max_pages ? row[k] : -1;
  }
  __device__ void init(const int32_t* row_, int max_pages_, int num_pages_, int first_page) {
    row = row_;
    max_pages = max_pages_;
    num_pages = num_pages_;
    load(first_page);
  }
  // Waits for a reload right where it is issued.  Without it the compiler, which cannot
  // tell whether the load on the rare path ran, waits at every later lookup, and that
  // wait (for all of the wave's outstanding vector-memory operations) would also wait
  // for the tile copies in flight.
  __device__ void settle() { asm volatile("v_mov_b32 %0, %0" : "+v"(ids)); }
  // Make `page_idx` (at or before the next lookups) readable: reloads the window if it
  // starts after page_idx, e.g. when a second pass over a piece goes back to its start.
  __device__ void rewind(int page_idx) {
    if (page_idx < base) {
      load(page_idx);
      settle();
    }
  }
  // page id of logical page `page_idx` (wave-uniform), -1 if invalid
  __device__ int get(int page_idx) {
    if (page_idx >= base + 64) {
      load(page_idx - 32 > base ? page_idx - 32 : base + 32);
      settle();
    }
    const int id = __builtin_amdgcn_readlane(ids, page_idx - base);
    return id >= 0 && id < num_pages ? id : -1;
  }
};

}  // namespace mla
