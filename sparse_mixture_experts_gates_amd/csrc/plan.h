// Tile plans of the grouped expert GEMMs, built on the device from the
// per-segment row ranges (segment = expert, or one shared expert).
//
// Entry order: segment-major, then column tile, then row tile, so the row
// tiles that share a weight slab are adjacent.  A plan buffer is a 128-byte
// header -- the int32 entry count, then at int32 index kPlanHeads eight
// 64-bit per-XCD queue words that the persistent GEMM claims entries with --
// followed by the 16-byte entries.  Header int32s: [0] entries, [1] entries
// in the per-XCD queues, [2] claims from the tail queue, [3] K parts of a
// tail entry (1 = no tail).  An entry's column field holds the column tile
// (bits 0-23), its K part (24-27) and, for a tail entry, its K parts (28-31).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace moe {

struct PlanEntry {
  int32_t g, m0, m1, nt;
};

constexpr int kPlanHeader = 128, kPlanHeads = 4;

// The column field's parts: the column tile in the low 24 bits, the K part
// of a split entry in bits 24-27 and, for a tail entry, its number of K parts
// in bits 28-31 (0: one).  Bit 31 is set for 8 parts, so the field is read
// as unsigned.
constexpr int kNtBits = 24;
__host__ __device__ constexpr int entry_tile(int nt) { return (int)((unsigned)nt & ((1u << kNtBits) - 1u)); }
__host__ __device__ constexpr int entry_part(int nt) { return (int)(((unsigned)nt >> 24) & 15u); }
__host__ __device__ constexpr int entry_parts(int nt) {
  return (int)((unsigned)nt >> 28) ? (int)((unsigned)nt >> 28) : 1;
}
static_assert(entry_parts((int)(5u | (7u << 24) | (8u << 28))) == 8 &&
                  entry_part((int)(5u | (7u << 24) | (8u << 28))) == 7 &&
                  entry_tile((int)(5u | (7u << 24) | (8u << 28))) == 5 && entry_parts(3) == 1,
              "plan entry column field");

// Row tile height of a segment of `rows` rows: BM, or with balanced tiles
// the rows split evenly over ceil(rows / BM) tiles and rounded up to 16.
// Equal tiles take equal time, so the workgroups that share a weight slab
// stay in step and find it in L2 (a short ragged last tile would finish
// early and desynchronise its XCD).
__device__ __forceinline__ int row_tile_height(int rows, int BM, int balanced) {
  if (!balanced || rows <= BM) return BM;
  const int m = (rows + BM - 1) / BM;
  const int h = ((rows + m - 1) / m + 15) & ~15;
  return h < BM ? h : BM;
}

// Writes the plans of ps (one or two passes over the same row tiling) for G
// segments whose rows are [start[g], start[g] + rows[g]).  Every thread of the
// (1-D) workgroup must call it (G <= 1024, G < 2 * blockDim.x); mt[G] and
// base[G + 1] are LDS scratch.
__device__ inline void build_tile_plans(const int* start, const int* rows, int G,
                                        const PlanSpec& ps, int* mt, int* base) {
  constexpr int kTab = 2048;        // row tiles the lookup table holds
  __shared__ int hs[1024];          // row tile height per segment
  __shared__ int rt_tab[kTab];      // row tile -> segment | (index in it << 10)
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int BM = ps.BM;
  for (int g = tid; g < G; g += nthr) {
    const int h = row_tile_height(rows[g], BM, ps.balanced);
    hs[g] = h;
    mt[g] = (rows[g] + h - 1) / h;
  }
  __syncthreads();   // base[g] below reads mt[g - 1], written by another thread
  // base = exclusive scan of mt (base[G] = all row tiles): an inclusive
  // Hillis-Steele scan of [0, mt[0], .., mt[G-1]], two entries per thread
  // (G < 2 * blockDim.x; a serial loop here cost microseconds at G = 128+)
  for (int g = tid; g <= G; g += nthr) base[g] = g == 0 ? 0 : mt[g - 1];
  __syncthreads();
  for (int off = 1; off <= G; off <<= 1) {
    const int g0 = tid, g1 = tid + nthr;
    const int v0 = (g0 <= G && g0 >= off) ? base[g0 - off] : 0;
    const int v1 = (g1 <= G && g1 >= off) ? base[g1 - off] : 0;
    __syncthreads();
    if (g0 <= G) base[g0] += v0;
    if (g1 <= G) base[g1] += v1;
    __syncthreads();
  }
  const int MT = base[G];   // row tiles over all segments
  // row tile -> (segment, index): each entry then costs two LDS reads
  // instead of a binary search over the segments
  const bool tab = MT <= kTab;
  if (tab)
    for (int g = tid; g < G; g += nthr)
      for (int mi = 0; mi < mt[g]; ++mi) rt_tab[base[g] + mi] = g | (mi << 10);
  __syncthreads();
  for (int pass = 0; pass < 2; ++pass) {
    // a split pass (K in S parts) lists every row tile once per part:
    // segment, column tile, part, row tile
    const int S = pass == 0 ? 1 : (ps.S2 > 1 ? ps.S2 : 1);
    const int nt_all = (pass == 0 ? ps.NT : ps.NT2) * S;
    int32_t* count = pass == 0 ? ps.plan : ps.plan2;
    if (nt_all <= 0) break;
    PlanEntry* out = reinterpret_cast<PlanEntry*>(reinterpret_cast<char*>(count) + kPlanHeader);
    const int V = MT * nt_all;
    // tail split (second pass): the first Vq entries are whole tiles, the
    // last V - Vq tiles (a partial round over tail_cus CUs) become St K parts
    // each, listed tile by tile after them
    int Vq = V, St = 1;
    if (pass == 1 && ps.tail_cus > 0 && S == 1 && tab) {
      const int ntail = V % ps.tail_cus;
      int st = ntail > 0 ? ps.tail_cus / ntail : 1;
      if (st > kTailMaxSplit) st = kTailMaxSplit;
      if (st >= 2 && ntail * st <= kTailParts) {
        St = st;
        Vq = V - ntail;
      }
    }
    if (tab) {
      // q enumerates (row tile, column entry); L is its place in the order
      // segment, column tile, part, row tile
      for (int q = tid; q < V; q += nthr) {
        const int rt = q / nt_all, c = q - rt * nt_all;
        const int v = rt_tab[rt];
        const int g = v & 1023, mi = v >> 10;
        const int L = base[g] * nt_all + c * mt[g] + mi;
        const int nt = S == 1 ? c : c / S, part = c - nt * S;
        const int h = hs[g];
        const int m0 = start[g] + mi * h;
        int m1 = m0 + h;
        if (m1 > start[g] + rows[g]) m1 = start[g] + rows[g];
        if (L < Vq) {
          out[L] = PlanEntry{g, m0, m1, nt | (part << 24)};
        } else {
          for (int p = 0; p < St; ++p)
            out[Vq + (L - Vq) * St + p] = PlanEntry{g, m0, m1, nt | (p << 24) | (St << 28)};
        }
      }
    } else
    for (int L = tid; L < V; L += nthr) {
      int lo = 0, hi = G - 1;  // last g with base[g] * nt_all <= L
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (base[mid] * nt_all <= L) lo = mid; else hi = mid - 1;
      }
      const int g = lo, rem = L - base[g] * nt_all, m = mt[g];
      const int c = rem / m, mi = rem - c * m;
      const int nt = c / S, part = c - nt * S;
      const int h = hs[g];
      const int m0 = start[g] + mi * h;
      int m1 = m0 + h;
      if (m1 > start[g] + rows[g]) m1 = start[g] + rows[g];
      out[L] = PlanEntry{g, m0, m1, nt | (part << 24)};
    }
    // header: all entries, the per-XCD queues' share, the tail queue's
    // claim counter, the tail's K parts; then the queue words
    if (tid == 0) {
      count[0] = Vq + (V - Vq) * St;
      count[1] = Vq;
      count[2] = 0;
      count[3] = St;
    }
    if (tid < 16) count[kPlanHeads + tid] = 0;   // queue words
  }
}

}  // namespace moe
