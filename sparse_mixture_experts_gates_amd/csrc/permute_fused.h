// The permutation of up to FUSED_MAX slots in one workgroup of 16 waves
// (1024 threads): histogram, per-expert scan with capacity, stable placement
// and, optionally, the expert GEMMs' tile plans.  Shared by the dispatch
// kernel and by the small-batch router, which runs it right after its top-k.
//
// Capacity and dropping follow "Mixture of Experts" (LLM tutorial ch. 11),
// "Expert capacity and dropped tokens": an expert keeps at most C slots, the
// first ones in priority order, and drops = sum_e max(0, c_e - C).
#pragma once

#include "common.h"
#include "launch.h"
#include "plan.h"

namespace moe {

// Slots are visited in priority order: the L-th visited slot is slot L
// (token-major: every slot of token 0, then of token 1, ...), or with
// slot-major priority (tslot = T) token L % T's choice L / T, so every
// token's first choice comes before any second choice.  Ranks, capacity and
// the row order inside each expert follow this order.
__device__ __forceinline__ int slot_of(int L, int tslot, int k) {
  return tslot ? (L % tslot) * k + L / tslot : L;
}

// All of the above in one workgroup of 16 waves, for up to FUSED_MAX slots:
// wave w owns a contiguous run of the slots; pass 1 counts its run per expert
// (ballot groups, no atomics), the per-expert prefix over waves gives each
// wave's starting ranks and the counts, capacity and offsets, and pass 2
// re-walks the run to place every slot.  Same results as the three kernels.
constexpr int FUSED_MAX = 8192;
constexpr int FUSED_WAVES = 16;
constexpr int FUSED_IT = FUSED_MAX / (FUSED_WAVES * 64);   // 64-slot groups per wave, at most

// Bits that tell expert ids 0 .. E-1 apart (E <= 256).
__host__ __device__ inline int expert_id_bits(int E) {
  int b = 0;
  while (b < 8 && (1 << b) < E) ++b;
  return b;
}

// The lanes of this wave that hold a valid slot of the same expert as this
// lane: one ballot per id bit (nbits = expert_id_bits(E); valid ids have no
// higher bits).  Each bit costs several vector instructions per wave, so
// only the bits E needs are tested.
__device__ __forceinline__ uint64_t expert_peers(int e, bool valid, int nbits) {
  uint64_t peers = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    if (b >= nbits) break;
    const bool bit = (e >> b) & 1;
    const uint64_t bb = __ballot(bit);
    peers &= bit ? bb : ~bb;
  }
  return peers;
}

__device__ inline void permute_one_workgroup(
    const int32_t* __restrict__ idx, int n, int E, int64_t cap, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src,
    int32_t* __restrict__ slot_pos, int32_t* __restrict__ num_dropped,
    int32_t* __restrict__ kept_total, PlanSpec ps, int want_plans, int tslot, int k) {
  __shared__ int run[FUSED_WAVES][256];
  __shared__ int sk[256];
  __shared__ int sdrop[256];
  __shared__ int soff[256];
  __shared__ int prows[256];
  __shared__ int pmt[256];
  __shared__ int pbase[257];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nbits = expert_id_bits(E);
  if (n <= 64) {
    // a decode batch: wave 0 alone ranks, counts, scans and places the <= 64
    // slots (lane l holds the l-th visited slot), without workgroup barriers;
    // the results are those of the general path below
    if (w == 0) {
      const uint64_t lt0 = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      const int sa = lane < n ? slot_of(lane, tslot, k) : 0;
      const int e = lane < n ? idx[sa] : -1;
      const bool valid = lane < n && e >= 0 && e < E;
      const uint64_t peers = expert_peers(e, valid, nbits);
      const int rank = __popcll(peers & lt0);
      for (int x = lane; x < 256; x += 64) sk[x] = 0;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      if (valid && rank == 0) sk[e] = __popcll(peers);          // count of expert e
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // experts 4 lane .. 4 lane + 3: counts, kept, dropped, local sums
      int c4[4], k4[4], ks = 0, ds = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int x = 4 * lane + i;
        c4[i] = x < E ? sk[x] : 0;
        k4[i] = cap < 0 ? c4[i] : (int)(c4[i] < cap ? c4[i] : cap);
        ks += k4[i];
        ds += c4[i] - k4[i];
      }
      // inclusive wave prefix of the kept sums and the total drops
      int incl = ks, dtot = ds;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
        dtot += __shfl_xor(dtot, off, 64);
      }
      const int total = __shfl(incl, 63, 64);
      int run0 = incl - ks;                                       // exclusive
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int x = 4 * lane + i;
        soff[x] = run0;
        prows[x] = k4[i];
        if (x < E) {
          if (counts) counts[x] = c4[i];
          offsets[x + 1] = run0 + k4[i];
        }
        run0 += k4[i];
      }
      if (lane == 0) {
        offsets[0] = 0;
        if (num_dropped) num_dropped[0] = dtot;
        kept_total[0] = total;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (lane < n) {
        if (valid && (cap < 0 || rank < cap)) {
          const int p = soff[e] + rank;
          slot_pos[sa] = p;
          perm_src[p] = sa;
        } else {
          slot_pos[sa] = -1;
        }
        if (lane >= total) perm_src[lane] = -1;   // rows past the kept ones
      }
    }
    if (want_plans) {
      __syncthreads();
      build_tile_plans(soff, prows, E, ps, pmt, pbase);
    }
    return;
  }
  const int per = ((n + FUSED_WAVES * 64 - 1) / (FUSED_WAVES * 64)) * 64;  // slots per wave
  const int lo = w * per;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int e = lane; e < 256; e += 64) run[w][e] = 0;
  // every expert id of this wave's run in flight at once, kept for both passes
  int ev[FUSED_IT];
#pragma unroll
  for (int i = 0; i < FUSED_IT; ++i) {
    const int a = lo + i * 64 + lane;
    ev[i] = (i * 64 < per && a < n) ? idx[slot_of(a, tslot, k)] : -1;
  }
  __syncthreads();
  // pass 1: per-wave counts; each group's peer mask is kept for pass 2
  uint64_t pk[FUSED_IT];
#pragma unroll
  for (int i = 0; i < FUSED_IT; ++i) {
    pk[i] = 0;
    if (i * 64 >= per) break;
    const int a = lo + i * 64 + lane;
    const int e = ev[i];
    const bool valid = a < n && e >= 0 && e < E;
    pk[i] = expert_peers(e, valid, nbits);
    if (valid && (pk[i] & lt) == 0) run[w][e] += __popcll(pk[i]);
  }
  __syncthreads();
  // per expert: exclusive prefix over waves, counts, capacity; then the
  // inclusive scans of kept and dropped over the experts (4 waves of 64:
  // shuffles within a wave, then the earlier waves' totals)
  __shared__ int wtot[2][4];
  int kept = 0, drop = 0;
  if (tid < 256) {
    const int e = tid;
    int tot = 0;
    for (int v = 0; v < FUSED_WAVES; ++v) {
      const int c = run[v][e];
      run[v][e] = tot;
      tot += c;
    }
    kept = e < E ? (cap < 0 ? tot : (int)(tot < cap ? tot : cap)) : 0;
    drop = e < E ? tot - kept : 0;
    if (e < E && counts) counts[e] = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(kept, off, 64), z = __shfl_up(drop, off, 64);
      if (lane >= off) {
        kept += y;
        drop += z;
      }
    }
    if (lane == 63) {
      wtot[0][w] = kept;
      wtot[1][w] = drop;
    }
  }
  __syncthreads();
  if (tid < 256) {
    for (int v = 0; v < w; ++v) {
      kept += wtot[0][v];
      drop += wtot[1][v];
    }
    sk[tid] = kept;
    sdrop[tid] = drop;
  }
  __syncthreads();
  if (tid < 256) soff[tid] = tid == 0 ? 0 : sk[tid - 1];
  if (tid < E) offsets[tid + 1] = sk[tid];
  if (tid == 0) {
    offsets[0] = 0;
    if (num_dropped) num_dropped[0] = sdrop[255];
    kept_total[0] = sk[255];
  }
  __syncthreads();
  if (want_plans) {
    // the expert FFN's tile plans from the kept counts just formed
    if (tid < E) prows[tid] = sk[tid] - soff[tid];
    __syncthreads();
    build_tile_plans(soff, prows, E, ps, pmt, pbase);
  }
  const int total = sk[255];
  // pass 2: place every slot of this wave's run
#pragma unroll
  for (int i = 0; i < FUSED_IT; ++i) {
    if (i * 64 >= per) break;
    const int a = lo + i * 64 + lane;
    const int sa = a < n ? slot_of(a, tslot, k) : 0;   // physical slot
    const int e = ev[i];
    const bool valid = a < n && e >= 0 && e < E;
    const uint64_t peers = pk[i];
    int r = 0;
    if (valid) r = run[w][e] + __popcll(peers & lt);
    __builtin_amdgcn_wave_barrier();
    if (valid && (peers & lt) == 0) run[w][e] += __popcll(peers);
    if (a < n) {
      if (valid && (cap < 0 || r < cap)) {
        const int p = soff[e] + r;
        slot_pos[sa] = p;
        perm_src[p] = sa;
      } else {
        slot_pos[sa] = -1;
      }
      if (a >= total) perm_src[a] = -1;   // rows past the kept ones
    }
  }
}

}  // namespace moe
