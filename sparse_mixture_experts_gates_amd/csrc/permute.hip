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

namespace moe {

namespace {

constexpr int CH = 1024;  // slots per chunk

// Slots are visited in priority order: the L-th visited slot is slot L
// (token-major: every slot of token 0, then of token 1, ...), or with
// slot-major priority (tslot = T) token L % T's choice L / T, so every
// token's first choice comes before any second choice.  Ranks, capacity and
// the row order inside each expert follow this order.
__device__ __forceinline__ int slot_of(int L, int tslot, int k) {
  return tslot ? (L % tslot) * k + L / tslot : L;
}

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
    int b = 0;
    for (; b + 4 <= nb; b += 4) {
      const int v0 = bc[(int64_t)(b + 0) * E + e];
      const int v1 = bc[(int64_t)(b + 1) * E + e];
      const int v2 = bc[(int64_t)(b + 2) * E + e];
      const int v3 = bc[(int64_t)(b + 3) * E + e];
      bc[(int64_t)(b + 0) * E + e] = run; run += v0;
      bc[(int64_t)(b + 1) * E + e] = run; run += v1;
      bc[(int64_t)(b + 2) * E + e] = run; run += v2;
      bc[(int64_t)(b + 3) * E + e] = run; run += v3;
    }
    for (; b < nb; ++b) {
      const int v = bc[(int64_t)b * E + e];
      bc[(int64_t)b * E + e] = run;
      run += v;
    }
  }
  const int kept = (e < E) ? (cap < 0 ? run : (int)(run < cap ? run : cap)) : 0;
  sk[e] = kept;
  sdrop[e] = (e < E) ? run - kept : 0;
  __syncthreads();
  // inclusive scans (Hillis-Steele) of kept and a sum of drops
  for (int off = 1; off < 256; off <<= 1) {
    const int v = e >= off ? sk[e - off] : 0;
    const int w = e >= off ? sdrop[e - off] : 0;
    __syncthreads();
    sk[e] += v;
    sdrop[e] += w;
    __syncthreads();
  }
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
  for (int st = 0; st < CH / 64; ++st) {
    const int64_t a = base + st * 64 + lane;
    const int sa = a < n ? slot_of((int)a, tslot, k) : 0;   // physical slot
    int e = -1;
    bool valid = a < n;
    if (valid) {
      e = idx[sa];
      valid = (e >= 0 && e < E);
    }
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      peers &= bit ? bb : ~bb;
    }
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

// All of the above in one workgroup of 16 waves, for up to FUSED_MAX slots:
// wave w owns a contiguous run of the slots; pass 1 counts its run per expert
// (ballot groups, no atomics), the per-expert prefix over waves gives each
// wave's starting ranks and the counts, capacity and offsets, and pass 2
// re-walks the run to place every slot.  Same results as the three kernels.
constexpr int FUSED_MAX = 8192;
constexpr int FUSED_WAVES = 16;
constexpr int FUSED_IT = FUSED_MAX / (FUSED_WAVES * 64);   // 64-slot groups per wave, at most

__device__ __forceinline__ uint64_t expert_peers(int e, bool valid) {
  uint64_t peers = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bb = __ballot(bit);
    peers &= bit ? bb : ~bb;
  }
  return peers;
}

__global__ __launch_bounds__(1024) void permute_fused_kernel(
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
  // pass 1: per-wave counts
#pragma unroll
  for (int i = 0; i < FUSED_IT; ++i) {
    if (i * 64 >= per) break;
    const int a = lo + i * 64 + lane;
    const int e = ev[i];
    const bool valid = a < n && e >= 0 && e < E;
    const uint64_t peers = expert_peers(e, valid);
    if (valid && (peers & lt) == 0) run[w][e] += __popcll(peers);
  }
  __syncthreads();
  // per expert: exclusive prefix over waves, counts, capacity
  if (tid < 256) {
    const int e = tid;
    int tot = 0;
    for (int v = 0; v < FUSED_WAVES; ++v) {
      const int c = run[v][e];
      run[v][e] = tot;
      tot += c;
    }
    const int kept = e < E ? (cap < 0 ? tot : (int)(tot < cap ? tot : cap)) : 0;
    sk[e] = kept;
    sdrop[e] = e < E ? tot - kept : 0;
    if (e < E && counts) counts[e] = tot;
  }
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    int v = 0, u = 0;
    if (tid < 256 && tid >= off) {
      v = sk[tid - off];
      u = sdrop[tid - off];
    }
    __syncthreads();
    if (tid < 256) {
      sk[tid] += v;
      sdrop[tid] += u;
    }
    __syncthreads();
  }
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
    const uint64_t peers = expert_peers(e, valid);
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
    prof_before("permute", s);
    const PlanSpec none{0, 0, 0, 1, nullptr, nullptr};
    permute_fused_kernel<<<1, 1024, 0, s>>>(a.topk_idx, (int)n, a.E, a.capacity, a.counts,
                                            a.offsets, a.perm_src, a.slot_pos, a.num_dropped,
                                            a.kept_total, a.plans ? *a.plans : none,
                                            a.plans ? 1 : 0, tslot, a.k);
    if (plans_built && a.plans) *plans_built = true;
    prof_after(s);
  } else {
  const int nb = permute_nblocks(n);
  prof_before("permute_count", s);
  permute_count_kernel<<<nb, 256, 0, s>>>(a.topk_idx, n, a.E, a.block_counts, tslot, a.k);
  prof_after(s);
  prof_before("permute_scan", s);
  permute_scan_kernel<<<1, 256, 0, s>>>(a.block_counts, nb, a.E, a.capacity, a.counts,
                                        a.offsets, a.num_dropped, a.kept_total);
  prof_after(s);
  prof_before("permute_scatter", s);
  permute_scatter_kernel<<<nb, 64, 0, s>>>(a.topk_idx, n, a.E, a.capacity, a.block_counts,
                                           a.offsets, a.kept_total, a.perm_src, a.slot_pos,
                                           tslot, a.k);
  prof_after(s);
  }
  if (a.x_perm) {
    const unsigned grid = (unsigned)((n + 3) / 4);
    prof_before("gather", s);
    if (a.dtype == MOE_BF16)
      gather_rows_kernel<uint4, 8><<<grid, 256, 0, s>>>(
          static_cast<const uint4*>(a.x), static_cast<uint4*>(a.x_perm), a.perm_src,
          a.kept_total, n, a.k, a.d / 8);
    else
      gather_rows_kernel<uint4, 4><<<grid, 256, 0, s>>>(
          static_cast<const uint4*>(a.x), static_cast<uint4*>(a.x_perm), a.perm_src,
          a.kept_total, n, a.k, a.d / 4);
    prof_after(s);
  }
  return hipGetLastError();
}

}  // namespace moe
