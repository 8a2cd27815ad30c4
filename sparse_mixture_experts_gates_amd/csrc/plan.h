// Tile plans of the grouped expert GEMMs, built on the device from the
// per-segment row ranges (segment = expert, or one shared expert).
//
// Entry order: segment-major, then column tile, then row tile, so the row
// tiles that share a weight slab are adjacent.  A plan buffer is a 128-byte
// header -- the int32 entry count, then at int32 index kPlanHeads eight
// 64-bit per-XCD queue words that the persistent GEMM claims entries with --
// followed by the 16-byte entries.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace moe {

struct PlanEntry {
  int32_t g, m0, m1, nt;
};

constexpr int kPlanHeader = 128, kPlanHeads = 4;

// Writes the plans of ps (one or two passes over the same row tiling) for G
// segments whose rows are [start[g], start[g] + rows[g]).  Every thread of the
// (1-D) workgroup must call it; mt[G] and base[G + 1] are LDS scratch.
__device__ inline void build_tile_plans(const int* start, const int* rows, int G,
                                        const PlanSpec& ps, int* mt, int* base) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int BM = ps.BM;
  for (int g = tid; g < G; g += nthr) mt[g] = (rows[g] + BM - 1) / BM;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int g = 0; g < G; ++g) {
      base[g] = acc;
      acc += mt[g];
    }
    base[G] = acc;
  }
  __syncthreads();
  const int MT = base[G];   // row tiles over all segments
  for (int pass = 0; pass < 2; ++pass) {
    // a split pass (K in S parts) lists every row tile once per part:
    // segment, column tile, part, row tile
    const int S = pass == 0 ? 1 : (ps.S2 > 1 ? ps.S2 : 1);
    const int nt_all = (pass == 0 ? ps.NT : ps.NT2) * S;
    int32_t* count = pass == 0 ? ps.plan : ps.plan2;
    if (nt_all <= 0) break;
    PlanEntry* out = reinterpret_cast<PlanEntry*>(reinterpret_cast<char*>(count) + kPlanHeader);
    const int V = MT * nt_all;
    for (int L = tid; L < V; L += nthr) {
      int lo = 0, hi = G - 1;  // last g with base[g] * nt_all <= L
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (base[mid] * nt_all <= L) lo = mid; else hi = mid - 1;
      }
      const int g = lo, rem = L - base[g] * nt_all, m = mt[g];
      const int c = rem / m, mi = rem - c * m;
      const int nt = c / S, part = c - nt * S;
      const int m0 = start[g] + mi * BM;
      int m1 = m0 + BM;
      if (m1 > start[g] + rows[g]) m1 = start[g] + rows[g];
      out[L] = PlanEntry{g, m0, m1, nt | (part << 24)};
    }
    if (tid == 0) count[0] = V;
    if (tid < 16) count[kPlanHeads + tid] = 0;   // queue words
  }
}

}  // namespace moe
