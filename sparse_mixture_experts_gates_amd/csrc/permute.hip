// Dispatch: per-expert histogram, scan with capacity, stable permutation and
// the row gather.
//
// Capacity and dropping follow "Mixture of Experts" (LLM tutorial ch. 11),
// "Expert capacity and dropped tokens" and Exercise 4: an expert keeps at most
// C slots, the first ones in token order, and drops = sum_e max(0, c_e - C).
// The grouping replaces the per-expert mask-and-gather loop of "Chapter 33 --
// Mixture of Experts (MoE)", "Simple MoE Layer Implementation", by one pass.
//
// Determinism without atomics on the order: the flat slot list (t*k + j) is cut
// into chunks of CH slots.  count: per-chunk histograms (LDS atomics, order
// free).  scan: per expert, an exclusive scan over chunks gives each chunk's
// starting rank; kept = min(count, C); offsets = exclusive scan of kept.
// scatter: one wave walks its chunk 64 slots at a time; lanes naming the same
// expert find each other with ballots over the bits of the expert id, so each
// slot's rank is (chunk base + earlier steps + lower lanes), exactly its rank
// in token order.  gather: one wave per kept row copies x[t] to x_perm[p].
#include "common.h"
#include "launch.h"
#include "plan.h"
#include "permute_fused.h"

namespace moe {

namespace {

constexpr int CH = 512;   // slots per chunk


__global__ __launch_bounds__(256) void permute_count_kernel(
    const int32_t* __restrict__ idx, int64_t n, int E, int32_t* __restrict__ bc, int tslot,
    int k) {
  __shared__ int hist[256];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * CH;
  for (int i = threadIdx.x; i < CH; i += 256) {
    const int64_t a = base + i;
    if (a < n) {
      const int e = idx[slot_of((int)a, tslot, k)];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) bc[(int64_t)blockIdx.x * E + e] = hist[e];
}

__global__ __launch_bounds__(256) void permute_scan_kernel(
    int32_t* __restrict__ bc, int nb, int E, int64_t cap, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ num_dropped,
    int32_t* __restrict__ kept_total) {
  __shared__ int sk[256];
  __shared__ int sdrop[256];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    // 32 chunk counts in flight per round trip (the scan is latency-bound)
    for (int b0 = 0; b0 < nb; b0 += 32) {
      int v[32];
#pragma unroll
      for (int u = 0; u < 32; ++u) v[u] = b0 + u < nb ? bc[(int64_t)(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        if (b0 + u < nb) bc[(int64_t)(b0 + u) * E + e] = run;
        run += v[u];
      }
    }
  }
  int kept = (e < E) ? (cap < 0 ? run : (int)(run < cap ? run : cap)) : 0;
  int drop = (e < E) ? run - kept : 0;
  // inclusive scans of kept and dropped over the experts: shuffles within
  // each wave of 64, then the earlier waves' totals
  __shared__ int wtot[2][4];
  const int lane = e & 63, w = e >> 6;
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
  __syncthreads();
  for (int v = 0; v < w; ++v) {
    kept += wtot[0][v];
    drop += wtot[1][v];
  }
  sk[e] = kept;
  sdrop[e] = drop;
  __syncthreads();
  if (e < E) {
    if (counts) counts[e] = run;
    offsets[e + 1] = sk[e];
  }
  if (e == 0) {
    offsets[0] = 0;
    if (num_dropped) num_dropped[0] = sdrop[255];
    kept_total[0] = sk[255];
  }
}

__global__ __launch_bounds__(64) void permute_scatter_kernel(
    const int32_t* __restrict__ idx, int64_t n, int E, int64_t cap,
    const int32_t* __restrict__ bc, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ kept_total, int32_t* __restrict__ perm_src,
    int32_t* __restrict__ slot_pos, int tslot, int k) {
  __shared__ int run[256];
  __shared__ int off_s[256];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) {
    run[e] = bc[(int64_t)blockIdx.x * E + e];
    off_s[e] = offsets[e];
  }
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * CH;
  const int64_t total = kept_total[0];
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int nbits = expert_id_bits(E);
  for (int st = 0; st < CH / 64; ++st) {
    const int64_t a = base + st * 64 + lane;
    const int sa = a < n ? slot_of((int)a, tslot, k) : 0;   // physical slot
    int e = -1;
    bool valid = a < n;
    if (valid) {
      e = idx[sa];
      valid = (e >= 0 && e < E);
    }
    const uint64_t peers = expert_peers(e, valid, nbits);
    int r = 0;
    if (valid) r = run[e] + __popcll(peers & lt);
    __syncthreads();  // every lane has read run[] before the leaders advance it
    if (valid && (peers & lt) == 0) run[e] += __popcll(peers);
    __syncthreads();
    if (a < n) {
      if (valid && (cap < 0 || r < cap)) {
        const int p = off_s[e] + r;
        slot_pos[sa] = p;
        perm_src[p] = sa;
      } else {
        slot_pos[sa] = -1;
      }
      if (a >= total) perm_src[a] = -1;   // rows past the kept ones
    }
  }
}

// The whole permutation in one workgroup (see permute_fused.h).
__global__ __launch_bounds__(1024) void permute_fused_kernel(
    const int32_t* __restrict__ idx, int n, int E, int64_t cap, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm_src,
    int32_t* __restrict__ slot_pos, int32_t* __restrict__ num_dropped,
    int32_t* __restrict__ kept_total, PlanSpec ps, int want_plans, int tslot, int k) {
  permute_one_workgroup(idx, n, E, cap, counts, offsets, perm_src, slot_pos, num_dropped,
                        kept_total, ps, want_plans, tslot, k);
}

// x_perm[p] = x[perm_src[p] / k] for p < kept_total; one wave per row.
template <typename VT, int EPV>
__global__ __launch_bounds__(256) void gather_rows_kernel(
    const VT* __restrict__ x, VT* __restrict__ xp, const int32_t* __restrict__ perm_src,
    const int32_t* __restrict__ kept_total, int64_t rows, int k, int nvec) {
  const int64_t p = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (p >= rows || p >= kept_total[0]) return;
  const int64_t t = perm_src[p] / k;
  const VT* src = x + t * nvec;
  VT* dst = xp + p * nvec;
  for (int c = threadIdx.x & 63; c < nvec; c += 64) dst[c] = src[c];
}

}  // namespace

int permute_nblocks(int64_t rows) { return (int)((rows + CH - 1) / CH); }

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s, bool* plans_built) {
  if (plans_built) *plans_built = false;
  const int64_t n = a.T * a.k;
  const int tslot = a.slot_major && a.k > 1 ? (int)a.T : 0;
  if (n == 0) return hipSuccess;
  if (n <= FUSED_MAX) {
    const int64_t prof_rec = prof_before("permute", s);
    const PlanSpec none{0, 0, 0, 1, nullptr, nullptr, 0};
    permute_fused_kernel<<<1, 1024, 0, s>>>(a.topk_idx, (int)n, a.E, a.capacity, a.counts,
                                            a.offsets, a.perm_src, a.slot_pos, a.num_dropped,
                                            a.kept_total, a.plans ? *a.plans : none,
                                            a.plans ? 1 : 0, tslot, a.k);
    if (plans_built && a.plans) *plans_built = true;
    prof_after(prof_rec, s);
  } else {
  const int nb = permute_nblocks(n);
  int64_t prof_rec = prof_before("permute_count", s);
  permute_count_kernel<<<nb, 256, 0, s>>>(a.topk_idx, n, a.E, a.block_counts, tslot, a.k);
  prof_after(prof_rec, s);
  prof_rec = prof_before("permute_scan", s);
  permute_scan_kernel<<<1, 256, 0, s>>>(a.block_counts, nb, a.E, a.capacity, a.counts,
                                        a.offsets, a.num_dropped, a.kept_total);
  prof_after(prof_rec, s);
  prof_rec = prof_before("permute_scatter", s);
  permute_scatter_kernel<<<nb, 64, 0, s>>>(a.topk_idx, n, a.E, a.capacity, a.block_counts,
                                           a.offsets, a.kept_total, a.perm_src, a.slot_pos,
                                           tslot, a.k);
  prof_after(prof_rec, s);
  }
  if (a.x_perm) {
    const unsigned grid = (unsigned)((n + 3) / 4);
    const int64_t prof_rec = prof_before("gather", s);
    if (a.dtype == MOE_BF16)
      gather_rows_kernel<uint4, 8><<<grid, 256, 0, s>>>(
          static_cast<const uint4*>(a.x), static_cast<uint4*>(a.x_perm), a.perm_src,
          a.kept_total, n, a.k, a.d / 8);
    else
      gather_rows_kernel<uint4, 4><<<grid, 256, 0, s>>>(
          static_cast<const uint4*>(a.x), static_cast<uint4*>(a.x_perm), a.perm_src,
          a.kept_total, n, a.k, a.d / 4);
    prof_after(prof_rec, s);
  }
  return hipGetLastError();
}

}  // namespace moe
