// Expert FFN: ragged grouped GEMMs over per-expert row segments.
//
// Each selected expert runs on the rows routed to it and nowhere else
// ("Mixture of experts", Inside the Model ch. 14, "The computation": only the
// selected experts run; LLM tutorial ch. 11, "The mathematics": FLOPs scale
// with k).  An expert is W2 . act(W1 . x) or the SwiGLU gated MLP
// W2 . (silu(W1 . x) * (W3 . x)) (LLM tutorial ch. 11, "Modern MoE variants",
// gate W1 / up W3 / down W2), computed as two passes:
//   pass 1: H = act(X_e . W1_e^T)  or  silu(X_e . W1_e^T) * (X_e . W3_e^T)
//   pass 2: Y = H_e . W2_e^T
//
// A pass is a device-built tile plan plus one GEMM launch.  The plan kernel
// turns the segment offsets into (segment, row range, column tile) entries,
// expert-major, then column tile, then row tile, so the tiles that share a
// weight slab are adjacent, and splits them into 8 contiguous queues, one
// per XCD (blocks are dealt round-robin over the 8 XCDs), which keeps each
// shared slab in one L2.  The prefill GEMMs are persistent: one block per CU
// drains its XCD's queue, then helps the others, so XCDs whose tiles are
// cheaper (ragged segment ends) do not finish early and idle.  No host
// synchronisation: the queue words live in the plan and the plan kernel
// resets them.
//
// bf16 GEMM: K in 64-wide slabs brought into XOR-swizzled LDS rings by
// direct-to-LDS loads and software-pipelined across slabs;
// v_mfma_f32_16x16x32_bf16 with weights on the MFMA row side, so each lane
// ends with 4 adjacent output columns of one row (8-byte stores).  SwiGLU
// interleaves W1 and W3 rows inside every wave's slab so the gate and up
// accumulators of a column sit in the same lane and the epilogue is
// elementwise.  Row sub-tiles past the end of a segment skip their MFMAs.
// The fp32 variant is a plain LDS-tiled FMA GEMM.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "plan.h"

namespace moe {

namespace {

constexpr int MODE_PLAIN = 0, MODE_RELU = 1, MODE_GELU = 2, MODE_SWIGLU = 3;
constexpr int BK = 64;

struct KArgs {
  const uint16_t* A;   // or float*
  const uint16_t* W;
  const uint16_t* Wu;
  uint16_t* C;
  const PlanEntry* plan;
  const int32_t* count;
  unsigned long long* queues;   // 8 per-XCD queue words (persistent launches)
  int32_t* tail;                // claims from the tail queue (header int 2)
  const int32_t* a_rows;  // optional row indirection for A (row gather folded in)
  int a_div;
  int K, N;
  int64_t a_seg_rows, c_seg_rows;  // extra row offset per segment (shared experts)
  float* part;                     // split: fp32 partial tiles [kTailParts][256][256]
  uint16_t* save1;                 // SAVE: pre-activations (W1 x), laid out like C
  uint16_t* save2;                 // SAVE, SwiGLU: W3 x
};


// Plan: one workgroup; G <= 1024 segments (offsets seg[G+1], or G dense
// segments of dense_rows rows).
__global__ __launch_bounds__(1024) void ffn_plan_kernel(const int32_t* __restrict__ seg, int G,
                                                        int64_t dense_rows, PlanSpec ps) {
  __shared__ int mt[1024];
  __shared__ int start[1024];
  __shared__ int rows_s[1024];
  __shared__ int base[1025];
  for (int g = threadIdx.x; g < G; g += 1024) {
    const int r0 = seg ? seg[g] : 0;
    const int r1 = seg ? seg[g + 1] : (int)dense_rows;
    start[g] = r0;
    rows_s[g] = r1 - r0;
  }
  __syncthreads();
  build_tile_plans(start, rows_s, G, ps, mt, base);
}

// XCD-aware order: physical block P runs on XCD P % 8; give each XCD a
// contiguous run of the V valid plan entries.
__device__ __forceinline__ int xcd_remap(int P, int V) {
  const int x = P & 7, i = P >> 3, q = V >> 3, r = V & 7;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

// Start of XCD x's share of the V entries (the split xcd_remap uses).
__device__ __forceinline__ int xcd_start(int x, int V) {
  const int q = V >> 3, r = V & 7;
  return x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
}

// Persistent launches: a block on XCD x takes the next entry of XCD x's
// queue, and once that is drained, the next entry of the tail queue (when
// the plan has one), then steals from the other XCDs' queues.  A
// queue word holds the entries taken from its front (low 32 bits, by its own
// XCD) and from its back (high 32 bits, by thieves): one atomic add claims
// an entry from either end, and the entry exists while front + back < len.
// Thieves take the last entries, whose weight slabs the owner XCD has not
// fetched yet, so a slab is not pulled into two L2s.  Returns -1 when every
// queue is drained.  Called by one lane.
__device__ int next_tile(unsigned long long* queues, int V, int x, int32_t* tail, int ntail) {
  // the tail queue (K parts of the partial last round) before stealing
  if (ntail > 0 && __hip_atomic_load(tail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < ntail) {
    const int t = atomicAdd(tail, 1);
    if (t < ntail) return V + t;
  }
#pragma unroll 1
  for (int s = 0; s < 8; ++s) {
    const int y = (x + s) & 7;
    const unsigned len = (unsigned)(xcd_start(y + 1, V) - xcd_start(y, V));
    const unsigned long long q0 = __hip_atomic_load(queues + y, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((unsigned)q0 + (unsigned)(q0 >> 32) >= len) continue;
    const bool back = s > 0;
    const unsigned long long q = atomicAdd(queues + y, back ? (1ull << 32) : 1ull);
    const unsigned f = (unsigned)q, b = (unsigned)(q >> 32);
    if (f + b < len) return xcd_start(y, V) + (int)(back ? len - 1 - b : f);
  }
  return -1;
}

__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}
__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

template <int MODE>
__device__ __forceinline__ float act1(float v) {
  if (MODE == MODE_RELU) return v > 0.f ? v : 0.f;
  if (MODE == MODE_GELU) return gelu_erf(v);
  return v;
}

// Grouped GEMM tile: BM rows of A (tokens) x BN rows of W (weights), K in
// slabs of 64 through an NSTAGE-deep LDS ring filled by direct-to-LDS loads
// (global_load_lds_dwordx4).  A slab row is 128 bytes (8 chunks of 16 B) and
// chunk c of row r sits at chunk c ^ (r & 7), so the MFMA operand reads
// (16 rows at one chunk) hit distinct banks.  One load instruction fills 8
// whole rows (1 KB): lane l writes LDS bytes 16*l, i.e. row l/8, chunk l%8,
// so it fetches logical chunk (l%8) ^ (l/8) of its row -- full 128-byte lines
// per 8 lanes.  Slab kt+NSTAGE-1 is requested while slab kt is multiplied;
// one barrier per slab.
template <int BM, int BN, int WM, int WN, int NSTAGE, int NSB, int MODE, bool PERSIST,
          bool SPLIT = false, bool SAVE = false>
__global__ __launch_bounds__(64 * WM * WN)
void ffn_bf16_kernel(KArgs a) {
  static_assert(!SPLIT || (MODE == MODE_PLAIN && NSTAGE == 2), "split: plain-mode 256 x 256 only");
  constexpr int NW = WM * WN;
  constexpr int BMW = BM / WM, BNW = BN / WN;   // wave tile (tokens, weight rows)
  constexpr int TM = BMW / 16, TN = BNW / 16;
  constexpr int HALF = BNW / 2;                  // SwiGLU: gate rows per wave
  constexpr int BNOUT = MODE == MODE_SWIGLU ? BN / 2 : BN;
  constexpr int NG = (BM + BN) / 8;              // 8-row load groups per slab
  constexpr int DPW = NG / NW;                   // load instructions per wave per slab
  static_assert(NG % NW == 0, "load groups must divide evenly over the waves");
  constexpr int SEL = (BM + BN) * BK;            // bf16 elements per slab
  static_assert(MODE != MODE_SWIGLU || TN % 2 == 0, "SwiGLU needs paired tiles");

  // NSTAGE == 2: token ring [2][BM*BK] then weight ring [NSB][BN*BK];
  // otherwise NSTAGE stages of [BM*BK tokens | BN*BK weights]
  constexpr int LDS_ELEMS = NSTAGE == 2 ? 2 * BM * BK + NSB * BN * BK : NSTAGE * SEL;
  // One LDS object only (a second one makes the compiler assume the operand
  // reads may alias the in-flight direct-to-LDS writes and wait for them);
  // two int slots pass the next tile id to every wave: after the ring, or,
  // when the ring fills the 160 KB, at its start (the ring is idle between
  // tiles; every wave reads the slot before the next slabs are requested).
  constexpr bool SLOT_IN_RING = (LDS_ELEMS + 4) * 2 > 160 * 1024;
  __shared__ __attribute__((aligned(1024))) uint16_t ring[LDS_ELEMS + (SLOT_IN_RING ? 0 : 4)];
  int* const tile_slot = reinterpret_cast<int*>(ring + (SLOT_IN_RING ? 0 : LDS_ELEMS));

  const int V = a.count[0];
  // persistent launches: entries [0, Vq) in the per-XCD queues, the rest
  // (K parts of tail tiles) in the tail queue
  const int Vq = PERSIST ? a.count[1] : V;
  const int P = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int wm = wave / WN, wn = wave % WN;
  const int K = a.K, N = a.N;
  // persistent: lane 0 claims the next entry of its own queue just before
  // each epilogue, so the atomic's round trip hides behind the stores (a
  // claim made earlier would hold an entry that an idle block could take)
  const int xq = P & 7;
  const int own0 = xcd_start(xq, Vq), own_len = xcd_start(xq + 1, Vq) - own0;
  unsigned long long claimed = ~0ull;
  for (int it = 0;; ++it) {
  int e;
  if constexpr (PERSIST) {
    if (tid == 0) {
      int nxt = -1;
      if (claimed != ~0ull) {
        const unsigned f = (unsigned)claimed, b = (unsigned)(claimed >> 32);
        if (f + b < (unsigned)own_len) nxt = own0 + (int)f;
      }
      tile_slot[it & 1] = nxt >= 0 ? nxt : next_tile(a.queues, Vq, xq, a.tail, V - Vq);
    }
    // also: every wave is done with the previous tile's LDS (its loads have
    // landed before the epilogue; its stores need not wait: outstanding
    // stores only make the next prologue's vmcnt wait longer)
    wait_lgkm0();
    ring_barrier();
    e = __builtin_amdgcn_readfirstlane(tile_slot[it & 1]);
    if constexpr (SLOT_IN_RING) ring_barrier();   // read before the ring is refilled
    if (e < 0) break;
  } else {
    if (it > 0 || P >= V) break;
    e = xcd_remap(P, V);
  }
  // lane id, opaque to the optimiser so that nothing derived from it is
  // hoisted out of the tile loop (it would stay live across every slab)
  int lane = tid & 63;
  asm volatile("" : "+v"(lane));
  const PlanEntry pe = a.plan[e];
  const int ks = SPLIT ? entry_part(pe.nt) : 0;
  const int nks = SPLIT ? entry_parts(pe.nt) : 1;
  const int n0 = entry_tile(pe.nt) * BNOUT;
  const int64_t arow0 = (int64_t)pe.g * a.a_seg_rows;
  const int64_t wbase = (int64_t)pe.g * N * K;

  // K slabs of this entry: all of them, or part ks of nks (a tail entry)
  const int nk_all = K / BK;
  const int kb0 = SPLIT ? (int)((int64_t)nk_all * ks / nks) : 0;
  const int nk = SPLIT ? (int)((int64_t)nk_all * (ks + 1) / nks) - kb0 : nk_all;
  // this lane's source (row, logical chunk) for each 8-row group the wave
  // loads: token groups first (rows past the segment end clamped to its last
  // row), then weight groups
  constexpr int DPA0 = BM / 8 / NW;
  static_assert((BM / 8) % NW == 0, "token load groups must divide over the waves");
  const uint16_t* src[DPW];
  {
    int rr[DPA0];
#pragma unroll
    for (int i = 0; i < DPA0; ++i) {
      const int r = pe.m0 + (wave + i * NW) * 8 + dma_row(lane);
      rr[i] = r > pe.m1 - 1 ? pe.m1 - 1 : r;
    }
    int64_t sr[DPA0];
    if (a.a_rows) {
      // gathered rows: every index load in flight before the first use
      int v[DPA0];
#pragma unroll
      for (int i = 0; i < DPA0; ++i) v[i] = a.a_rows[rr[i]];
#pragma unroll
      for (int i = 0; i < DPA0; ++i) sr[i] = v[i] / a.a_div;
    } else {
#pragma unroll
      for (int i = 0; i < DPA0; ++i) sr[i] = arow0 + rr[i];
    }
#pragma unroll
    for (int i = 0; i < DPA0; ++i) src[i] = a.A + sr[i] * K + dma_chunk(lane) * 8 + kb0 * BK;
  }
#pragma unroll
  for (int i = DPA0; i < DPW; ++i) {
    const int rho = (wave + i * NW) * 8 + dma_row(lane) - BM;
    int n;
    const uint16_t* Wm = a.W;
    if (MODE == MODE_SWIGLU) {
      const int wq = rho / BNW, wi = rho - wq * BNW;
      n = n0 + wq * HALF + (wi < HALF ? wi : wi - HALF);
      if (wi >= HALF) Wm = a.Wu;
    } else {
      n = n0 + rho;
    }
    if (n > N - 1) n = N - 1;
    src[i] = Wm + wbase + (int64_t)n * K + dma_chunk(lane) * 8 + kb0 * BK;
  }

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if constexpr (NSTAGE == 2) {
    // Software pipeline across slabs: the token slabs sit in a 2-stage ring,
    // the weight slabs in an NSB-stage ring (weights mostly come from HBM,
    // so they are requested NSB-1 slabs ahead).  Each slab is used in two
    // halves of 32 k.  Step kt: (A) MFMAs of half 0 of slab kt, with the
    // reads of half 1 spread between them; (B) wait for slab kt+1, barrier,
    // request token slab kt+2 and weight slab kt+NSB into the stages slab kt
    // occupied; (C) MFMAs of half 1 of slab kt, with the reads of half 0 of
    // slab kt+1 spread between them.  LDS reads never wait at a slab start.
    constexpr int SA = BM * BK, SB = BN * BK;
    constexpr int DPA = BM / 8 / NW, DPB = DPW - DPA;
    static_assert((BM / 8) % NW == 0, "token load groups must divide over the waves");
    uint16_t* const ring_a = ring;
    uint16_t* const ring_b = ring + 2 * SA;
    auto issue = [&](int kta, int stage_a, int ktb, int stage_b) {
      const int ka = kta < nk ? kta : nk - 1;   // past the end: a harmless reload
      const int kb = ktb < nk ? ktb : nk - 1;
#pragma unroll
      for (int i = 0; i < DPA; ++i)
        dma_rows(src[i] + ka * BK, ring_a + stage_a * SA + (wave + i * NW) * 512);
#pragma unroll
      for (int i = DPA; i < DPW; ++i)
        dma_rows(src[i] + kb * BK, ring_b + stage_b * SB + (wave + i * NW - BM / 8) * 512);
    };
    // Rows of this wave's tile that hold tokens: a tile at the ragged end of
    // a segment multiplies only its live 16-row sub-tiles.
    const int rows_left = pe.m1 - pe.m0 - wm * BMW;
    const int nlive = rows_left >= BMW ? TM : (rows_left <= 0 ? 0 : (rows_left + 15) >> 4);
    // KIND 2: every sub-tile live; 1: some; 0: none (loads and barriers only)
    auto pipeline = [&](auto kind_tag) {
      constexpr int KIND = decltype(kind_tag)::value;
      constexpr bool FULL = KIND == 2;
      constexpr int NR = TN + TM, NM = TM * TN, PER = NM / NR > 0 ? NM / NR : 1;
      auto read_half = [&](const uint16_t* sa, const uint16_t* sb, int half, bf16x8_t* fw,
                           bf16x8_t* fx) {
        const int ch = half * 4 + (lane >> 4);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          fw[j] = *reinterpret_cast<const bf16x8_t*>(sb + swz(wn * BNW + j * 16 + (lane & 15), ch));
#pragma unroll
        for (int i = 0; i < TM; ++i)
          fx[i] = *reinterpret_cast<const bf16x8_t*>(sa + swz(wm * BMW + i * 16 + (lane & 15), ch));
      };
      auto mfma_half = [&](const bf16x8_t* fw, const bf16x8_t* fx) {
        if constexpr (KIND == 0) return;
#pragma unroll
        for (int i = 0; i < TM; ++i)
          if (FULL || i < nlive)
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[j], fx[i], acc[i][j], 0, 0, 0);
      };
      issue(0, 0, 0, 0);
      issue(1, 1, 1, 1);
#pragma unroll
      for (int st = 2; st < NSB; ++st) {
        const int kb = st < nk ? st : nk - 1;
#pragma unroll
        for (int i = DPA; i < DPW; ++i)
          dma_rows(src[i] + kb * BK, ring_b + st * SB + (wave + i * NW - BM / 8) * 512);
      }
      wait_vm_lgkm0<DPW + (NSB - 2) * DPB>();
      ring_barrier();
      bf16x8_t w0[TN], x0[TM], w1[TN], x1[TM];
      read_half(ring_a, ring_b, 0, w0, x0);
      int sb_cur = 0, sb_nxt = 1;   // weight ring stages of slabs kt and kt+1
      for (int kt = 0; kt < nk; ++kt) {
        const uint16_t* cur_a = ring_a + (kt & 1) * SA;
        const uint16_t* nxt_a = ring_a + ((kt + 1) & 1) * SA;
        const uint16_t* cur_b = ring_b + sb_cur * SB;
        const uint16_t* nxt_b = ring_b + sb_nxt * SB;
        // (A)
        read_half(cur_a, cur_b, 1, w1, x1);
        mfma_half(w0, x0);
        if constexpr (FULL) {
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, NM - NR * PER, 0);
        }
        // (B) slab kt+1 has landed once only weight slabs kt+2.. remain
        wait_vm_lgkm0<(NSB - 2) * DPB>();
        ring_barrier();
        issue(kt + 2, kt & 1, kt + NSB, sb_cur);
        // (C)
        read_half(nxt_a, nxt_b, 0, w0, x0);
        mfma_half(w1, x1);
        if constexpr (FULL) {
          // spread the slab loads over the MFMAs so the address path never
          // backs up into the instruction stream
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            if (r < DPW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          if (DPW > NR) __builtin_amdgcn_sched_group_barrier(0x020, DPW > NR ? DPW - NR : 0, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, NM - NR * PER, 0);
        }
        sb_cur = sb_nxt;
        sb_nxt = sb_nxt + 1 == NSB ? 0 : sb_nxt + 1;
      }
    };
    if (nlive == TM) pipeline(std::integral_constant<int, 2>{});
    else if (nlive == 0) pipeline(std::integral_constant<int, 0>{});
    else pipeline(std::integral_constant<int, 1>{});
  } else {
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s) {
    const int kk = s < nk ? s : nk - 1;
#pragma unroll
    for (int i = 0; i < DPW; ++i)
      dma_rows(src[i] + kk * BK, ring + s * SEL + (wave + i * NW) * 512);
  }
  int cur_s = 0;                          // ring stage of slab kt
  int nxt_s = NSTAGE - 1;                 // ring stage of slab kt + NSTAGE - 1
  for (int kt = 0; kt < nk; ++kt) {
    // slab kt has landed for this wave once at most NSTAGE-2 younger slabs remain
    wait_vm_lgkm0<(NSTAGE - 2) * DPW>();
    ring_barrier();
    // refill the stage consumed in step kt-1 (past the end: a harmless reload
    // of the last slab, so every step has the same shape)
    const int kn = kt + NSTAGE - 1 < nk ? kt + NSTAGE - 1 : nk - 1;
    uint16_t* nxt = ring + nxt_s * SEL;
#pragma unroll
    for (int i = 0; i < DPW; ++i)
      dma_rows(src[i] + kn * BK, nxt + (wave + i * NW) * 512);
    const uint16_t* sa = ring + cur_s * SEL;
    const uint16_t* sb = sa + BM * BK;
    // operand reads of the first 32 k, then its MFMAs with the reads of the
    // second 32 k spread between them, then the second half's MFMAs
    bf16x8_t fw[2][TN], fx[2][TM];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ch = kk * 4 + (lane >> 4);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fw[kk][j] = *reinterpret_cast<const bf16x8_t*>(sb + swz(wn * BNW + j * 16 + (lane & 15), ch));
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fx[kk][i] = *reinterpret_cast<const bf16x8_t*>(sa + swz(wm * BMW + i * 16 + (lane & 15), ch));
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[kk][j], fx[kk][i], acc[i][j], 0, 0, 0);
    {
      constexpr int NR = TN + TM, NM = TM * TN, PER = NM / NR > 0 ? NM / NR : 1;
      __builtin_amdgcn_sched_group_barrier(0x020, DPW, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * NM - NR * PER, 0);
    }
    cur_s = cur_s + 1 == NSTAGE ? 0 : cur_s + 1;
    nxt_s = nxt_s + 1 == NSTAGE ? 0 : nxt_s + 1;
  }
  }
  wait_vm_lgkm0<0>();   // the trailing reloads must land before the LDS is released
  if (PERSIST && tid == 0) claimed = atomicAdd(a.queues + xq, 1ull);

  // epilogue: lane holds columns 4*(lane/16)+q of tile j, row lane%16 of
  // tile i.  N is a multiple of 64, so a 4-column group is either wholly in
  // range or wholly out.
  const int64_t crow0 = (int64_t)pe.g * a.c_seg_rows;
  constexpr int JOUT = MODE == MODE_SWIGLU ? TN / 2 : TN;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int r = pe.m0 + wm * BMW + i * 16 + (lane & 15);
    const bool row_ok = r < pe.m1;
    uint16_t* crow = a.C + (crow0 + r) * (int64_t)N;
#pragma unroll
    for (int j = 0; j < JOUT; ++j) {
      float v[4];
      int col;
      // training forward: keep the pre-activations for the backward pass
      auto save = [&](uint16_t* dst, const f32x4_t& z) {
        uint2 pz;
        pz.x = pack_bf16x2(z[0], z[1]);
        pz.y = pack_bf16x2(z[2], z[3]);
        if (row_ok && col < N) *reinterpret_cast<uint2*>(dst + (crow0 + r) * (int64_t)N + col) = pz;
      };
      if (MODE == MODE_SWIGLU) {
        col = n0 + wn * HALF + j * 16 + 4 * (lane >> 4);
        if constexpr (SAVE) {
          save(a.save1, acc[i][j]);
          save(a.save2, acc[i][j + TN / 2]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = silu_f(acc[i][j][q]) * acc[i][j + TN / 2][q];
      } else {
        col = n0 + wn * BNW + j * 16 + 4 * (lane >> 4);
        if constexpr (SAVE) save(a.save1, acc[i][j]);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = act1<MODE>(acc[i][j][q]);
      }
      if constexpr (SPLIT) {
        if (nks > 1) {
          // a tail entry: the fp32 partial of part ks in its tile's slot
          // (added in order and rounded by the tail reduce)
          // tail entries are listed tile by tile, part by part: e - Vq is
          // the entry's partial-tile slot
          float* prow = a.part + ((int64_t)(e - Vq) * 256 + (r - pe.m0)) * 256;
          if (row_ok && col < N)
            *reinterpret_cast<f32x4_t*>(prow + (col - n0)) = f32x4_t{v[0], v[1], v[2], v[3]};
          continue;
        }
      }
      uint2 pk;
      pk.x = pack_bf16x2(v[0], v[1]);
      pk.y = pack_bf16x2(v[2], v[3]);
      if (row_ok && col < N) *reinterpret_cast<uint2*>(crow + col) = pk;
    }
  }
  }  // tiles
}

// fp32: 64 x 64 output tile, 16-deep K slabs, 4 x 4 outputs per thread
// (x 2 accumulators for SwiGLU).
template <int MODE>
__global__ __launch_bounds__(256) void ffn_f32_kernel(KArgs a) {
  constexpr int TB = 64, KS = 16, LDT = TB + 4;
  __shared__ float As[KS][LDT];
  __shared__ float Ws[KS][LDT];
  __shared__ float Us[KS][LDT];
  const int V = a.count[0];
  const int P = blockIdx.x;
  if (P >= V) return;
  const PlanEntry pe = a.plan[P];
  const float* A = reinterpret_cast<const float*>(a.A);
  const float* W = reinterpret_cast<const float*>(a.W);
  const float* Wu = reinterpret_cast<const float*>(a.Wu);
  float* C = reinterpret_cast<float*>(a.C);
  const int K = a.K, N = a.N;
  const int n0 = entry_tile(pe.nt) * TB;
  const int64_t arow0 = (int64_t)pe.g * a.a_seg_rows;
  const int64_t wbase = (int64_t)pe.g * N * K;
  const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
  float acc[4][4], accu[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = accu[i][j] = 0.f;
  for (int k0 = 0; k0 < K; k0 += KS) {
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      const int idx = tid + l * 256, row = idx >> 4, kk = idx & 15;
      const bool kin = k0 + kk < K;
      int r = pe.m0 + row;
      if (r > pe.m1 - 1) r = pe.m1 - 1;
      const int64_t sr = a.a_rows ? (int64_t)(a.a_rows[r] / a.a_div) : arow0 + r;
      As[kk][row] = kin ? A[sr * K + k0 + kk] : 0.f;
      int n = n0 + row;
      if (n > N - 1) n = N - 1;
      Ws[kk][row] = kin ? W[wbase + (int64_t)n * K + k0 + kk] : 0.f;
      if (MODE == MODE_SWIGLU) Us[kk][row] = kin ? Wu[wbase + (int64_t)n * K + k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      float av[4], wv[4], uv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][tr * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) wv[j] = Ws[kk][tc * 4 + j];
      if (MODE == MODE_SWIGLU) {
#pragma unroll
        for (int j = 0; j < 4; ++j) uv[j] = Us[kk][tc * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(av[i], wv[j], acc[i][j]);
          if (MODE == MODE_SWIGLU) accu[i][j] = fmaf(av[i], uv[j], accu[i][j]);
        }
    }
    __syncthreads();
  }
  const int64_t crow0 = (int64_t)pe.g * a.c_seg_rows;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = pe.m0 + tr * 4 + i;
    if (r >= pe.m1) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tc * 4 + j;
      if (col >= N) continue;
      float v;
      if (MODE == MODE_SWIGLU) {
        const float z = acc[i][j];
        v = z / (1.0f + expf(-z)) * accu[i][j];
      } else {
        v = act1<MODE>(acc[i][j]);
      }
      C[(crow0 + r) * N + col] = v;
    }
  }
}

struct Shape {
  int BM, BNOUT, id;   // id: 0 fp32, 1 small batch SwiGLU 32x128, 2 256x256, 3 256x128,
                       //     4 small batch plain 32x64
};

constexpr int kCUs = 256;

// Tile shape of one pass.  Prefill passes use 256 x 256 tiles unless that
// leaves fewer than two rounds of tiles over the CUs (a short pass), where
// 256 x 128 tiles trim the last, partial round.
Shape pick_shape(int dtype, bool small, int mode, int64_t max_rows, int N) {
  if (dtype == MOE_F32) return {64, 64, 0};
  const bool glu = mode == MODE_SWIGLU;
  // small batches stream each active expert's weights once; narrower
  // 64-row weight tiles (3 blocks per CU) shorten the last round
  if (small) return glu ? Shape{32, 64, 1} : Shape{32, 64, 4};
  const int64_t big_tiles = ((max_rows + 255) / 256) * ((N + (glu ? 127 : 255)) / (glu ? 128 : 256));
  if (big_tiles < 2 * kCUs) return {256, glu ? 64 : 128, 3};
  return {256, glu ? 128 : 256, 2};
}

// Upper bound of the plan entries: a row tile holds at least one row, and
// each segment adds at most one partial tile.
int64_t max_entries(int64_t max_rows, int G, int N, Shape sh) {
  const int64_t nt = (N + sh.BNOUT - 1) / sh.BNOUT;
  int64_t mt = (max_rows + sh.BM - 1) / sh.BM + G;
  if (mt > max_rows) mt = max_rows;
  return mt * nt;
}

template <int BM, int BN, int WM, int WN, int NS, int NSB, bool PERSIST>
void launch_bf16(int mode, unsigned grid, const KArgs& k, hipStream_t s) {
  constexpr int T = 64 * WM * WN;
  if (k.save1) {   // training forward: the activation passes keep their pre-activations
    switch (mode) {
      case MODE_RELU: ffn_bf16_kernel<BM, BN, WM, WN, NS, NSB, MODE_RELU, PERSIST, false, true><<<grid, T, 0, s>>>(k); break;
      case MODE_GELU: ffn_bf16_kernel<BM, BN, WM, WN, NS, NSB, MODE_GELU, PERSIST, false, true><<<grid, T, 0, s>>>(k); break;
      default: ffn_bf16_kernel<BM, BN, WM, WN, NS, NSB, MODE_SWIGLU, PERSIST, false, true><<<grid, T, 0, s>>>(k); break;
    }
    return;
  }
  switch (mode) {
    case MODE_PLAIN: ffn_bf16_kernel<BM, BN, WM, WN, NS, NSB, MODE_PLAIN, PERSIST><<<grid, T, 0, s>>>(k); break;
    case MODE_RELU: ffn_bf16_kernel<BM, BN, WM, WN, NS, NSB, MODE_RELU, PERSIST><<<grid, T, 0, s>>>(k); break;
    case MODE_GELU: ffn_bf16_kernel<BM, BN, WM, WN, NS, NSB, MODE_GELU, PERSIST><<<grid, T, 0, s>>>(k); break;
    default: ffn_bf16_kernel<BM, BN, WM, WN, NS, NSB, MODE_SWIGLU, PERSIST><<<grid, T, 0, s>>>(k); break;
  }
}


}  // namespace

size_t ffn_plan_bytes(int64_t max_rows, int G, int N, bool small, int dtype, int split) {
  size_t best = 0;
  for (int mode = 0; mode < 4; ++mode) {
    // a tail split adds at most kTailParts entries (the tail tiles' parts)
    const size_t b = kPlanHeader + 16 * ((size_t)max_entries(max_rows, G, N,
                                                             pick_shape(dtype, small, mode,
                                                                        max_rows, N)) +
                                         (split > 1 ? (size_t)kTailParts : 0));
    if (b > best) best = b;
  }
  return (best + 255) / 256 * 256;
}

// Tail split for a routed second expert GEMM (plain mode) on 256 x 256
// tiles with a long K and only a few rounds of tiles: the tiles of its
// partial last round run in K parts, so that round keeps every CU busy (the
// plan kernel picks the parts from the real tile count).
int ffn_split(int64_t max_rows, int G, int N, int K, bool small, int dtype) {
  if (dtype != MOE_BF16 || small) return 1;
  const Shape sh = pick_shape(dtype, false, MODE_PLAIN, max_rows, N);
  if (sh.id != 2 || K / BK < 64) return 1;
  return max_entries(max_rows, G, N, sh) < 8 * kCUs ? 2 : 1;
}

namespace {
int pass_nt(const FfnPassArgs& p) {
  const Shape sh = pick_shape(p.dtype, p.small, p.mode, p.max_rows, p.N);
  return (p.N + sh.BNOUT - 1) / sh.BNOUT;
}
}  // namespace

bool ffn_plan_spec(const FfnPassArgs& p1, const FfnPassArgs& p2, PlanSpec* ps) {
  const Shape sh1 = pick_shape(p1.dtype, p1.small, p1.mode, p1.max_rows, p1.N);
  const Shape sh2 = pick_shape(p2.dtype, p2.small, p2.mode, p2.max_rows, p2.N);
  if (sh1.BM != sh2.BM || p1.seg_offsets != p2.seg_offsets) return false;
  if (max_entries(p1.max_rows, p1.G, p1.N, sh1) == 0) return false;
  ps->BM = sh1.BM;
  ps->NT = pass_nt(p1);
  ps->NT2 = pass_nt(p2);
  ps->S2 = 1;
  ps->tail_cus = 0;
  if (p2.split > 1) {
    const int cus = cu_count();
    ps->tail_cus = cus < kTailParts ? cus : kTailParts;
  }
  ps->plan = static_cast<int32_t*>(p1.plan);
  ps->plan2 = static_cast<int32_t*>(p2.plan);
  ps->balanced = 1;
  return true;
}

hipError_t launch_plan_kernel(const int32_t* seg, int G, int64_t dense_rows, const PlanSpec& ps,
                              hipStream_t s) {
  if (G > 1024) return hipErrorInvalidValue;
  const int64_t prof_rec = prof_before("plan", s);
  ffn_plan_kernel<<<1, 1024, 0, s>>>(seg, G, dense_rows, ps);
  prof_after(prof_rec, s);
  return hipGetLastError();
}

hipError_t launch_ffn_plans(const FfnPassArgs& p1, const FfnPassArgs& p2, hipStream_t s) {
  PlanSpec ps{};
  if (!ffn_plan_spec(p1, p2, &ps)) {
    const Shape sh1 = pick_shape(p1.dtype, p1.small, p1.mode, p1.max_rows, p1.N);
    return max_entries(p1.max_rows, p1.G, p1.N, sh1) == 0 ? hipSuccess : hipErrorInvalidValue;
  }
  const int64_t prof_rec = prof_before(p1.seg_offsets ? "ffn_plan" : "ffn_plan_shared", s);
  ffn_plan_kernel<<<1, 1024, 0, s>>>(p1.seg_offsets, p1.G, p1.dense_rows, ps);
  prof_after(prof_rec, s);
  return hipGetLastError();
}

hipError_t launch_ffn_pass(const FfnPassArgs& p, hipStream_t s) {
  const Shape sh = pick_shape(p.dtype, p.small, p.mode, p.max_rows, p.N);
  const int split = p.split > 1 ? p.split : 1;
  if (split > 1 && (sh.id != 2 || p.mode != MODE_PLAIN || !p.part)) return hipErrorInvalidValue;
  const int64_t grid = max_entries(p.max_rows, p.G, p.N, sh) + (split > 1 ? kTailParts : 0);
  if (grid == 0) return hipSuccess;
  int32_t* count = static_cast<int32_t*>(p.plan);
  PlanEntry* plan = reinterpret_cast<PlanEntry*>(static_cast<char*>(p.plan) + kPlanHeader);
  KArgs k;
  k.A = static_cast<const uint16_t*>(p.A);
  k.W = static_cast<const uint16_t*>(p.w);
  k.Wu = static_cast<const uint16_t*>(p.w_up ? p.w_up : p.w);
  k.C = static_cast<uint16_t*>(p.C);
  k.plan = plan;
  k.count = count;
  k.queues = reinterpret_cast<unsigned long long*>(count + kPlanHeads);
  k.a_rows = p.a_rows;
  k.a_div = p.a_div > 0 ? p.a_div : 1;
  k.K = p.K;
  k.N = p.N;
  k.a_seg_rows = p.a_seg_rows;
  k.c_seg_rows = p.c_seg_rows;
  k.tail = count + 2;
  k.part = p.part;
  k.save1 = static_cast<uint16_t*>(p.save1);
  k.save2 = static_cast<uint16_t*>(p.save2);
  if (k.save1 && (p.dtype != MOE_BF16 || p.mode == MODE_PLAIN || split > 1 ||
                  (p.mode == MODE_SWIGLU && !k.save2)))
    return hipErrorInvalidValue;
  const char* nm = p.seg_offsets ? (p.mode == MODE_PLAIN ? "ffn2" : "ffn1")
                                 : (p.mode == MODE_PLAIN ? "ffn2_shared" : "ffn1_shared");
  const int64_t prof_rec = prof_before(nm, s);
  if (p.dtype == MOE_F32) {
    switch (p.mode) {
      case MODE_PLAIN: ffn_f32_kernel<MODE_PLAIN><<<(unsigned)grid, 256, 0, s>>>(k); break;
      case MODE_RELU: ffn_f32_kernel<MODE_RELU><<<(unsigned)grid, 256, 0, s>>>(k); break;
      case MODE_GELU: ffn_f32_kernel<MODE_GELU><<<(unsigned)grid, 256, 0, s>>>(k); break;
      default: ffn_f32_kernel<MODE_SWIGLU><<<(unsigned)grid, 256, 0, s>>>(k); break;
    }
  } else if (sh.id == 1) {
    launch_bf16<32, 128, 1, 4, 4, 4, false>(p.mode, (unsigned)grid, k, s);
  } else if (sh.id == 4) {
    // plain / ReLU / GeLU only (a SwiGLU wave needs a pair of column tiles)
    constexpr int T4 = 64 * 4;
    if (k.save1) {
      if (p.mode == MODE_RELU) ffn_bf16_kernel<32, 64, 1, 4, 4, 4, MODE_RELU, false, false, true><<<(unsigned)grid, T4, 0, s>>>(k);
      else if (p.mode == MODE_GELU) ffn_bf16_kernel<32, 64, 1, 4, 4, 4, MODE_GELU, false, false, true><<<(unsigned)grid, T4, 0, s>>>(k);
      else return hipErrorInvalidValue;
      prof_after(prof_rec, s);
      return hipGetLastError();
    }
    switch (p.mode) {
      case MODE_PLAIN: ffn_bf16_kernel<32, 64, 1, 4, 4, 4, MODE_PLAIN, false><<<(unsigned)grid, T4, 0, s>>>(k); break;
      case MODE_RELU: ffn_bf16_kernel<32, 64, 1, 4, 4, 4, MODE_RELU, false><<<(unsigned)grid, T4, 0, s>>>(k); break;
      case MODE_GELU: ffn_bf16_kernel<32, 64, 1, 4, 4, 4, MODE_GELU, false><<<(unsigned)grid, T4, 0, s>>>(k); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    // With at least two rounds of tiles: one persistent block per CU (the
    // LDS ring fills a CU).  Fewer, short tiles do not repay the queue.
    const int cus = cu_count();
    if (split > 1) {   // the tail queue needs the persistent launch
      ffn_bf16_kernel<256, 256, 2, 4, 2, 3, MODE_PLAIN, true, true><<<(unsigned)cus, 512, 0, s>>>(k);
    } else if (grid >= 2 * (int64_t)cus) {
      if (sh.id == 3) launch_bf16<256, 128, 4, 2, 3, 3, true>(p.mode, (unsigned)cus, k, s);
      else launch_bf16<256, 256, 2, 4, 2, 3, true>(p.mode, (unsigned)cus, k, s);
    } else {
      if (sh.id == 3) launch_bf16<256, 128, 4, 2, 3, 3, false>(p.mode, (unsigned)grid, k, s);
      else launch_bf16<256, 256, 2, 4, 2, 2, false>(p.mode, (unsigned)grid, k, s);
    }
  }
  prof_after(prof_rec, s);
  return hipGetLastError();
}

namespace {
// The tail tiles of a split pass: C = bf16(part 0 + part 1 + ...) in part
// order, from the fp32 partial tiles.  Workgroup (tile, 16-row strip): each
// thread sums two 8-column chunks of its strip with all their parts' loads
// in flight at once (the sums are latency-bound otherwise).
constexpr int kReduceStrips = 16;   // 16-row strips of a 256-row tile

__global__ __launch_bounds__(256) void tail_reduce_kernel(const int32_t* __restrict__ count,
                                                          const PlanEntry* __restrict__ plan,
                                                          const float* __restrict__ part,
                                                          uint16_t* __restrict__ C, int N,
                                                          int64_t c_seg_rows) {
  const int V = count[0], Vq = count[1], St = count[3];
  const int ntiles = St > 1 ? (V - Vq) / St : 0;
  const int tt = blockIdx.x / kReduceStrips, strip = blockIdx.x % kReduceStrips;
  if (tt >= ntiles) return;
  const PlanEntry pe = plan[Vq + tt * St];
  const int n0 = entry_tile(pe.nt) * 256;
  const int rows = pe.m1 - pe.m0;
  const float* base = part + (int64_t)tt * St * 65536;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = threadIdx.x + h * 256;               // 16 rows x 32 chunks
    const int r = strip * 16 + (i >> 5), c = (i & 31) * 8;
    if (r >= rows || n0 + c >= N) continue;
    f32x4_t q[kTailMaxSplit][2];
#pragma unroll
    for (int p = 0; p < kTailMaxSplit; ++p) {
      if (p < St) {
        const f32x4_t* src = reinterpret_cast<const f32x4_t*>(base + ((int64_t)p * 256 + r) * 256 + c);
        q[p][0] = src[0];
        q[p][1] = src[1];
      }
    }
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < kTailMaxSplit; ++p) {
      if (p < St) {
        s0 += q[p][0];
        s1 += q[p][1];
      }
    }
    u32x4_t o;
    o[0] = pack_bf16x2(s0[0], s0[1]);
    o[1] = pack_bf16x2(s0[2], s0[3]);
    o[2] = pack_bf16x2(s1[0], s1[1]);
    o[3] = pack_bf16x2(s1[2], s1[3]);
    *reinterpret_cast<u32x4_t*>(C + ((int64_t)pe.g * c_seg_rows + pe.m0 + r) * N + n0 + c) = o;
  }
}
}  // namespace

hipError_t launch_tail_reduce(const void* plan_buf, const float* part, void* C, int N,
                              int64_t c_seg_rows, const char* name, hipStream_t s) {
  const int32_t* count = static_cast<const int32_t*>(plan_buf);
  const PlanEntry* plan =
      reinterpret_cast<const PlanEntry*>(static_cast<const char*>(plan_buf) + kPlanHeader);
  const int64_t prof_rec = prof_before(name, s);
  // at most kTailParts / 2 tail tiles (each has at least two parts)
  tail_reduce_kernel<<<kTailParts / 2 * kReduceStrips, 256, 0, s>>>(
      count, plan, part, static_cast<uint16_t*>(C), N, c_seg_rows);
  prof_after(prof_rec, s);
  return hipGetLastError();
}

hipError_t launch_ffn_tail_reduce(const FfnPassArgs& p, hipStream_t s) {
  if (p.split <= 1) return hipSuccess;
  return launch_tail_reduce(p.plan, p.part, p.C, p.N, p.c_seg_rows, "ffn2_tail_reduce", s);
}

}  // namespace moe
