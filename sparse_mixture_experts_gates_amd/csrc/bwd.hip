// Backward pass of the sparse MoE layer, bf16 operands, fp32 accumulation.
//
// The routing is held fixed: the gradient reaches the router only through the
// soft gate values and, with the balance loss, through the mean router
// probabilities ("Mixture of Experts", LLM tutorial ch. 11, "The routing
// decision" and "Training instability"; "Mixture of experts", Inside the
// Model ch. 14, "Auxiliary loss" and "Check yourself").  Steps:
//
//   gate kernel   per token: dg_j = <dy, O_j> for each kept slot, the expert
//                 output gradient dO_j = g_j dy (bf16, on the permuted row),
//                 and the score gradient ds = J^T dg (+ balance loss), fp32
//   dH GEMM       dH = dO . W2_e over each expert's rows; the epilogue applies
//                 the activation's derivative with the saved pre-activations
//                 (SwiGLU: dG = dH u silu'(g), dU = dH silu(g))
//   dX GEMM       dX = dG . W1_e (+ dU . W3_e) over each expert's rows; with
//                 only a few rounds of tiles, the partial last round's tiles
//                 in K parts (fp32 partials, added by the tail reduce)
//   dW GEMMs      dW2_e = dO_e^T H_e, dW1_e = dG_e^T X_e, dW3_e = dU_e^T X_e:
//                 the contraction runs over the expert's rows (ragged K)
//   dx kernel     dx_t = sum over kept slots of dX rows + shared experts'
//                 dX + ds_t . W_r, one rounding
//   router        dW_r = ds^T x, fp32, fixed-order partial sums
//
// GEMM layout.  Every backward GEMM has its output's contiguous dimension on
// the MFMA row side (P) and its other dimension on the column side (Q), as
// the forward does.  For dH and dX, P is a weight stored with that dimension
// contiguous (W2_e for dH, W1_e / W3_e for dX), so its K index is strided: P
// tiles are staged in LDS as k-rows of 64-element lines and read with
// ds_read_b64_tr_b16, which hands each lane 4 consecutive k of one column
// (two reads make one 8-k MFMA operand); Q holds activation rows
// (K-contiguous), read like the forward's operands.  The weight gradients
// contract over rows, so both operands are k-strided and both are read
// transposed from LDS (rows past a segment's end read as zeros).  (Copying
// the routed operands into K-contiguous transposes first made the GEMMs
// faster per slab, but the five transposes cost more than that.)
//
// Loads.  Slabs go straight from global memory to LDS (global_load_lds) in
// rings, issued from asm so that the compiler does not wait for the newest
// slab before every ds_read_b64_tr_b16 (it cannot tell the two apart).
//
// Scheduling.  Row tiles of dH / dX follow the device-built plans, dealt
// round-robin over the XCDs.  Weight-gradient tiles run persistent: one
// workgroup per CU claims tiles one ahead from its XCD's queue (stealing from
// the next queues once it is empty), experts with the most rows first; the
// next tile's first two slabs are requested before the current tile's
// output block is stored, and the block goes out through LDS as whole
// 128-byte row segments.
#include <atomic>
#include <string.h>

#include "common.h"
#include "launch.h"
#include "plan.h"

namespace moe {

namespace {

constexpr int BK = 64;
constexpr int GB_BM = 256, GB_BN = 256;     // output tile: Q extent x P extent
constexpr int GB_WM = 2, GB_WN = 4;         // waves along Q, along P
constexpr int GB_NW = GB_WM * GB_WN;
constexpr int GB_MAX_SEGS = 1024;           // segments a weight-gradient launch may hold
constexpr int GB_QUEUES = 8;                // tile queues of a persistent launch (one per XCD)

typedef short i16x4_t __attribute__((ext_vector_type(4)));

// P-side / MN-major LDS tile: BK k-rows, each split into 64-element lines of
// 128 bytes.  Line (k, nb) sits at index k * NL + nb; within a line, 16-byte
// chunk c sits at chunk c ^ ((k & 3) << 1), so the four k-rows one transposed
// read touches (same columns) land on distinct bank groups.
template <int NL>
__device__ __forceinline__ int mn_off(int k, int col) {   // bf16 element offset
  const int nb = col >> 6, c = (col >> 3) & 7, h = col & 7;
  return (k * NL + nb) * 64 + ((c ^ ((k & 3) << 1)) << 3) + h;
}

// One MFMA operand (16 columns x 32 k) from an MN-major tile: lane l covers
// column l%16, k 8*(l/16) .. +7.  Each transposed read gathers 4 k-rows x 16
// columns over a 16-lane group: lanes 4q..4q+3 address row q, 4 columns each.
template <int NL>
__device__ __forceinline__ bf16x8_t read_mn(const uint16_t* tile, int col0, int k0, int lane) {
  const int q = (lane & 15) >> 2;
  const int col = col0 + 4 * (lane & 3);
  const int kr = k0 + 8 * (lane >> 4) + q;
  auto p0 = (__attribute__((address_space(3))) i16x4_t*)MOE_LDS_PTR(tile + mn_off<NL>(kr, col));
  auto p1 = (__attribute__((address_space(3))) i16x4_t*)MOE_LDS_PTR(tile + mn_off<NL>(kr + 4, col));
  const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p0);
  const i16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p1);
  const i16x4_t v[2] = {a, b};
  return __builtin_bit_cast(bf16x8_t, v);
}

// dma_rows issued from an asm block with no register outputs, so that the
// compiler does not know of the direct-to-LDS write.  It cannot tell such a
// write apart from the LDS reads of ds_read_b64_tr_b16 and would otherwise
// wait for every load in flight (the slab requested for two steps later
// included) before the first transposed read of each step; the kernel's own
// s_waitcnt calls order the slabs instead.
__device__ __forceinline__ void dma_rows_untracked(const uint16_t* src, uint16_t* lds_group) {
  const uint32_t lds = (uint32_t)(uintptr_t)MOE_LDS_PTR(lds_group);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds) : "memory", "m0");
}

// Direct-to-LDS load of 8 lines of an MN-major tile (1 KB): lane l fills line
// l/8, stored chunk l%8, so it fetches logical chunk (l%8) ^ ((k & 3) << 1).
__device__ __forceinline__ int mn_chunk(int lane, int k) { return (lane & 7) ^ ((k & 3) << 1); }

struct GemmArgs {
  int kind;                   // BG_DH, BG_DX, BG_DW
  const uint16_t* P;          // MN-major operand (see launch.h)
  const uint16_t* P2;
  int64_t ldp, p_seg;         // row pitch; per-segment element offset (dH/dX weights)
  int64_t p_row_seg;          // dW: per-segment row offset of P
  const uint16_t* Q;
  const uint16_t* Q2;
  int64_t ldq;
  int64_t q_row_seg;          // row offset of segment g in Q (dense segments)
  uint16_t* C;
  uint16_t* C2;
  int64_t ldc, c_seg;         // dW: per-segment element offset of C
  int64_t c_row_seg;          // dH/dX: row offset of segment g in C (dense segments)
  const uint16_t* S1;         // dH: saved pre-activations (G or Z) and U
  const uint16_t* S2;
  const PlanEntry* plan;      // dH/dX row tiles
  const int32_t* count;
  const int32_t* seg;         // dW: [G+1] row offsets, or null (dense)
  const int32_t* order;       // dW: segments by descending row count (or null: natural)
  int* counter;               // dW: GB_QUEUES tile counters of a persistent launch (or null)
  int64_t dense_rows;
  const uint16_t* zero;       // >= 256 zero elements
  int K, N, M;                // dH/dX: K per operand pair; N output cols; dW: M output rows
  int nk1;                    // dX: slabs of the first operand pair
  int G, MT, NT;              // dW tile grid
  float* part;                // dX tail entries: fp32 partial tiles [kTailParts][256][256]
};

__device__ __forceinline__ float sigm(float z) { return 1.0f / (1.0f + __expf(-z)); }

// d/dz of the erf GeLU: Phi(z) + z phi(z)
__device__ __forceinline__ float gelu_grad(float z) {
  return 0.5f * (1.0f + erff(z * 0.70710678118654752f)) +
         z * 0.39894228040143268f * __expf(-0.5f * z * z);
}

template <int KIND, int EPI>
__global__ __launch_bounds__(64 * GB_NW) void bwd_gemm_kernel(GemmArgs a) {
  constexpr int BM = GB_BM, BN = GB_BN, WN = GB_WN, NW = GB_NW;
  constexpr int BMW = BM / GB_WM, BNW = BN / WN;
  constexpr int TM = BMW / 16, TN = BNW / 16;
  constexpr int NLP = BN / 64, NLQ = BM / 64;
  constexpr int SP = BK * BN, SQ = BK * BM;
  constexpr bool QMN = KIND == BG_DW;       // Q stored k-strided (read transposed)
  constexpr bool WGRAD = KIND == BG_DW;
  constexpr int DP = BK * NLP / 8 / NW;     // P load instructions per wave per slab
  constexpr int DQ = (QMN ? BK * NLQ : BM) / 8 / NW;
  static_assert(DP * NW * 8 == BK * NLP && DQ * NW * 8 == (QMN ? BK * NLQ : BM), "load split");
  // the ring, then two int slots that pass a claimed tile to every wave, then
  // (weight gradients) the segment order and row offsets.  One LDS object: a
  // second one makes the compiler wait for in-flight direct-to-LDS writes
  // before every operand read.
  constexpr int TAB = WGRAD ? 2 * GB_MAX_SEGS + 1 : 0;   // ints
  // P stages: three for dH, whose P is a weight streamed from HBM (its slabs
  // are requested two ahead; the rings then fill the 160 KB), two otherwise
  // (a third made dX slower)
  constexpr int NSP = KIND == BG_DH ? 3 : 2;
  constexpr int RING = NSP * SP + 2 * SQ;
  __shared__ __attribute__((aligned(1024))) uint16_t ring[RING + (WGRAD ? 4 + 2 * TAB : 0)];
  // stages: dX and the weight gradients keep each stage's P and Q side by
  // side; dH, with its third P stage, has the P stages, then the Q stages
  constexpr bool ILV = KIND == BG_DX || KIND == BG_DW;
  static_assert(!ILV || NSP == 2, "interleaved stages hold one P and one Q slab each");
  constexpr int P_STRIDE = ILV ? SP + SQ : SP, Q_STRIDE = ILV ? SP + SQ : SQ;
  uint16_t* const ring_p = ring;
  uint16_t* const ring_q = ring + (ILV ? SP : NSP * SP);
  int* const tile_slot = reinterpret_cast<int*>(ring + RING);   // weight gradients only
  int* const tab_order = tile_slot + 2;
  int* const tab_off = tab_order + GB_MAX_SEGS;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // Weight gradients with a tile counter run persistent: one workgroup per CU
  // claims tiles in order until none is left, one tile ahead, so that the
  // next tile's first two slabs are requested before this tile's stores.
  // Otherwise one tile per block.
  const bool persist = WGRAD && a.counter != nullptr;
  // One tile queue per XCD: workgroups are dispatched round-robin over the
  // 8 XCDs, so block b runs on XCD b % 8 and takes tiles q, q + 8, q + 16, ...
  // of queue q = b % 8; the tiles one XCD runs at a time then share their Q
  // row blocks (and, within a column block, their P block) in its L2.  A
  // claim is one plain atomic whose result is waited for only where it is
  // used: the counter's address goes in as a per-lane value, which keeps the
  // compiler from turning it into a wave-combined atomic that waits for its
  // own result (and so for every load in flight) at once.
  // A block whose queue runs dry takes tiles from the next queues.
  const int nq = gridDim.x < GB_QUEUES ? gridDim.x : GB_QUEUES;
  int cq = blockIdx.x % nq, hops = 0;
  int zl = 0;
  asm volatile("" : "+v"(zl));
  // the tile of the claim in tile_slot[slot]; every wave calls it after a
  // barrier that made the claim visible
  auto claimed_tile = [&](int slot) -> int {
    const int V = a.G * a.MT * a.NT;
    int e = cq + nq * __builtin_amdgcn_readfirstlane(tile_slot[slot]);
    while (e >= V && hops + 1 < nq) {
      ++hops;
      cq = cq + 1 == nq ? 0 : cq + 1;
      ring_barrier();    // every wave has read the slot
      if (tid == 0) tile_slot[slot] = atomicAdd(a.counter + cq + zl, 1);
      wait_lgkm0();
      ring_barrier();
      e = cq + nq * __builtin_amdgcn_readfirstlane(tile_slot[slot]);
    }
    return e;
  };
  int e0;
  if (persist) {
    for (int i = tid; i < a.G; i += 64 * NW) tab_order[i] = a.order[i];
    for (int i = tid; i <= a.G; i += 64 * NW) tab_off[i] = a.seg[i];
    if (tid == 0) tile_slot[0] = atomicAdd(a.counter + cq + zl, 1);
    wait_lgkm0();
    ring_barrier();
    e0 = claimed_tile(0);
  } else {
    e0 = blockIdx.x;
  }
  const int N = a.N;
  const int64_t ldp = a.ldp, ldq = a.ldq;
  const uint16_t* const zp = a.zero;   // every lane may read the same zeros

  // Per-tile state, set by setup().  Load sources: P in DP instructions of 8
  // lines, Q in DQ instructions (8 rows of 64 k, or 8 lines of an MN-major
  // tile).  Instruction i of a wave fills lines L = (wave + i NW) 8 + lane/8,
  // i.e. k-row k0 + i KSTEP and line lane/8 % NL of it: the column and the
  // chunk swizzle (k & 3) are the same for every i.  Each lane's sources are
  // a base pointer (its k-row k0 and column folded in) plus a wave-uniform
  // offset per slab and instruction.
  static_assert(8 % NLP == 0 && 8 % NLQ == 0, "lines per k-row");
  constexpr int KSP = NW * 8 / NLP, KSQ = NW * 8 / NLQ;
  static_assert(KSP % 4 == 0 && KSQ % 4 == 0, "swizzle must repeat across instructions");
  int lane = 0;
  int g = 0, m0 = 0, m1 = 0, n0 = 0, nk = 0, ks = 0, kb0 = 0, klen32 = 0, pk0 = 0, qk0 = 0;
  int tail = -1;                 // dX tail entry: its partial-tile slot
  int64_t q_off[QMN ? 1 : DQ];   // K-major Q: element offset of this lane's row and chunk
  const uint16_t* pb = nullptr;  // P at k-row pk0 of slab 0
  const uint16_t* pb2 = nullptr;
  const uint16_t* qb = nullptr;
  auto setup = [&](int e) -> bool {
    // lane id, opaque to the optimiser so that nothing derived from it is
    // hoisted out of the tile loop (it would stay live across every slab)
    lane = tid & 63;
    asm volatile("" : "+v"(lane));
    int64_t prow0 = 0, qrow0 = 0, klen = 0;
    ks = 0;
    kb0 = 0;
    if constexpr (WGRAD) {
      // Segments with rows longest first, so the costliest tiles start first
      // and the short ones fill in at the end, with the segments without rows
      // (blocks of zeros: stores only) spread between them; within a segment, row blocks vary
      // fastest, so an XCD's queue holds every eighth row block (its own
      // slice of the Q operand) while the column blocks stream past.
      const int V = a.G * a.MT * a.NT;
      if (e >= V) return false;
      const int rank = e / (a.MT * a.NT);
      const int rem = e - rank * a.MT * a.NT;
      const int nt = rem / a.MT, mt = rem - nt * a.MT;
      m0 = mt * BM;
      m1 = m0 + BM < a.M ? m0 + BM : a.M;
      n0 = nt * BN;
      if (persist) {
        g = __builtin_amdgcn_readfirstlane(tab_order[rank]);
        const int o0 = __builtin_amdgcn_readfirstlane(tab_off[g]);
        klen = __builtin_amdgcn_readfirstlane(tab_off[g + 1]) - o0;
        prow0 = (int64_t)g * a.p_row_seg + o0;
        qrow0 = (int64_t)g * a.q_row_seg + o0;
      } else {
        g = rank;
        const int64_t r0 = a.seg ? a.seg[g] : 0;
        klen = a.seg ? a.seg[g + 1] - r0 : a.dense_rows;
        prow0 = (int64_t)g * a.p_row_seg + r0;
        qrow0 = (int64_t)g * a.q_row_seg + r0;
      }
      nk = (int)((klen + BK - 1) / BK);
    } else {
      const int V = a.count[0];
      if (e >= V) return false;
      // plan order, dealt round-robin over the XCDs: each XCD takes every
      // eighth row tile of a column tile, so a skewed segment's tiles spread
      // over the whole chip and each L2 keeps its own slice of the rows
      const PlanEntry pe = a.plan[e];
      g = pe.g;
      m0 = pe.m0;
      m1 = pe.m1;
      n0 = entry_tile(pe.nt) * BN;
      ks = entry_part(pe.nt);
      // a tail entry: part ks of nks, its partial tile in slot e - Vq
      const int nks = entry_parts(pe.nt);
      tail = nks > 1 ? e - a.count[1] : -1;
      qrow0 = (int64_t)g * a.q_row_seg;
      // the slabs of this entry: all of them, or part ks of a tail entry
      const int nk_all = KIND == BG_DX && EPI == 1 ? 2 * a.nk1 : a.K / BK;
      kb0 = (int)((int64_t)nk_all * ks / nks);
      nk = (int)((int64_t)nk_all * (ks + 1) / nks) - kb0;
    }
    klen32 = (int)klen;
    pk0 = wave * (8 / NLP) + (lane >> 3) / NLP;
    int pcol = n0 + ((lane >> 3) % NLP) * 64;
    if (pcol > N - 64) pcol = N - 64;            // past the last column: any valid line
    pcol += mn_chunk(lane, pk0) * 8;
    int qcol = 0;
    if constexpr (QMN) {
      qk0 = wave * (8 / NLQ) + (lane >> 3) / NLQ;
      qcol = m0 + ((lane >> 3) % NLQ) * 64;
      if (qcol > a.M - 64) qcol = a.M - 64;
      qcol += mn_chunk(lane, qk0) * 8;
      q_off[0] = 0;
    } else {
#pragma unroll
      for (int i = 0; i < DQ; ++i) {
        int r = m0 + (wave + i * NW) * 8 + dma_row(lane);
        if (r > m1 - 1) r = m1 - 1;
        q_off[i] = (qrow0 + r) * ldq + dma_chunk(lane) * 8;
      }
    }
    if constexpr (KIND == BG_DW) {
      pb = a.P + (prow0 + pk0) * ldp + pcol;
    } else {
      pb = a.P + (int64_t)g * a.p_seg + pk0 * ldp + pcol;
      if constexpr (KIND == BG_DX) pb2 = (a.P2 ? a.P2 : a.P) + (int64_t)g * a.p_seg + pk0 * ldp + pcol;
    }
    qb = QMN ? a.Q + (qrow0 + qk0) * ldq + qcol : a.Q;
    return true;
  };

  // requests for slab ktr (relative to the tile's first slab) of P, of Q
  auto issue_p = [&](int ktr, int stage) {
    uint16_t* sp = ring_p + stage * P_STRIDE;
    const int kt = ktr + kb0;                              // slab index within K
    const bool second = KIND == BG_DX && kt >= a.nk1;
    const int kb = (second ? kt - a.nk1 : kt) * BK;      // first k-row of the slab
#pragma unroll
    for (int i = 0; i < DP; ++i) {
      const int kr = kb + i * KSP;                         // uniform
      const uint16_t* src = (second ? pb2 : pb) + (int64_t)kr * ldp;
      if constexpr (KIND == BG_DW) src = pk0 + kr < klen32 ? src : zp;
      dma_rows_untracked(src, sp + (wave + i * NW) * 512);
    }
  };
  auto issue_q = [&](int ktr, int stage) {
    uint16_t* sq = ring_q + stage * Q_STRIDE;
    const int kt = ktr + kb0;
    const bool second = KIND == BG_DX && kt >= a.nk1;
    const int kb = (second ? kt - a.nk1 : kt) * BK;
#pragma unroll
    for (int i = 0; i < DQ; ++i) {
      const uint16_t* src;
      if constexpr (QMN) {
        const int kr = kb + i * KSQ;
        src = qk0 + kr < klen32 ? qb + (int64_t)kr * ldq : zp;
      } else {
        src = (second ? a.Q2 : a.Q) + q_off[i] + kb;
      }
      dma_rows_untracked(src, sq + (wave + i * NW) * 512);
    }
  };
  // the tile's first slabs: P and Q of slabs 0 and 1, then (three P stages)
  // P of slab 2; past the last slab the requests reload it (harmless)
  auto prologue = [&]() {
    issue_p(0, 0);
    issue_q(0, 0);
    issue_p(1 < nk ? 1 : 0, 1);
    issue_q(1 < nk ? 1 : 0, 1);
    if constexpr (NSP == 3) issue_p(2 < nk ? 2 : nk - 1, 2);
  };

  // Software pipeline over 64-k slabs in LDS rings (Q: 2 stages, P: NSP),
  // each slab used in two halves of 32 k.  Step kt: (A) MFMAs of half 0 of
  // slab kt with the reads of half 1 spread between them; (B) wait for slab
  // kt+1, barrier, request Q of slab kt+2 and P of slab kt+NSP into the
  // stages slab kt held; (C) MFMAs of half 1 with the reads of half 0 of
  // slab kt+1 (and the new requests) spread between them.  Past the last
  // slab the requests reload it (harmless).
  constexpr int NRD = 2 * TN + (QMN ? 2 : 1) * TM;   // LDS read instructions per half
  constexpr int NM = TM * TN, PER = NM / NRD > 0 ? NM / NRD : 1;
  constexpr int DPW = DP + DQ;
  auto read_half = [&](const uint16_t* sp, const uint16_t* sq, int kk, bf16x8_t* fp, bf16x8_t* fq) {
#pragma unroll
    for (int j = 0; j < TN; ++j) fp[j] = read_mn<NLP>(sp, wn * BNW + j * 16, kk * 32, lane);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if constexpr (QMN) {
        fq[i] = read_mn<NLQ>(sq, wm * BMW + i * 16, kk * 32, lane);
      } else {
        const int ch = kk * 4 + (lane >> 4);
        fq[i] = *reinterpret_cast<const bf16x8_t*>(sq + swz(wm * BMW + i * 16 + (lane & 15), ch));
      }
    }
  };

  if (!setup(e0)) return;
  if (nk > 0) prologue();
  int claim = 0;   // thread 0: the tile after the current one
  if (persist && tid == 0) claim = atomicAdd(a.counter + cq + zl, 1);
  // The previous tile's epilogue issued exactly NSTORE stores per wave after
  // this tile's first two slabs (it was a whole tile), so the wait for slab 0
  // may leave them in flight: vector memory operations complete in order.
  constexpr int NSTORE = WGRAD ? 2 * TM : TM * TN;   // stores per wave of a whole tile
  bool exact = false;
  for (int it = 0;; ++it) {
    f32x4_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto mfma_half = [&](const bf16x8_t* fp, const bf16x8_t* fq) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp[j], fq[i], acc[i][j], 0, 0, 0);
    };
    if (nk > 0) {
      // slab 0 has landed (slab 1, P of slab 2, the claim and the stores may
      // be in flight)
      if (exact) wait_vm_lgkm0<DPW + (NSP - 2) * DP + NSTORE>();
      else wait_vm_lgkm0<DPW + (NSP - 2) * DP>();
      ring_barrier();
      bf16x8_t p0[TN], q0[TM], p1[TN], q1[TM];
      read_half(ring_p, ring_q, 0, p0, q0);
      int sp_cur = 0, sp_nxt = 1;   // P stages of slabs kt and kt+1
      for (int kt = 0; kt < nk; ++kt) {
        // (A)
        read_half(ring_p + sp_cur * P_STRIDE, ring_q + (kt & 1) * Q_STRIDE, 1, p1, q1);
        mfma_half(p0, q0);
#pragma unroll
        for (int r = 0; r < NRD; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if (NM > NRD * PER) __builtin_amdgcn_sched_group_barrier(0x008, NM - NRD * PER, 0);
        // (B) slab kt+1 has landed once only P of slab kt+2 may remain
        wait_vm_lgkm0<(NSP - 2) * DP>();
        ring_barrier();
        issue_q(kt + 2 < nk ? kt + 2 : nk - 1, kt & 1);
        issue_p(kt + NSP < nk ? kt + NSP : nk - 1, sp_cur);
        // (C)
        read_half(ring_p + sp_nxt * P_STRIDE, ring_q + ((kt + 1) & 1) * Q_STRIDE, 0, p0, q0);
        mfma_half(p1, q1);
#pragma unroll
        for (int r = 0; r < NRD; ++r) {
          if (r < DPW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if (NM > NRD * PER) __builtin_amdgcn_sched_group_barrier(0x008, NM - NRD * PER, 0);
        sp_cur = sp_nxt;
        sp_nxt = sp_nxt + 1 == NSP ? 0 : sp_nxt + 1;
      }
    }
    wait_vm_lgkm0<0>();

    // this tile's output block; then (persistent) the next tile's slabs are
    // requested before the stores
    const int cg = g, cm0 = m0, cm1 = m1, cn0 = n0, ctail = tail;
    bool more = false;
    // Weight gradients: the block leaves through LDS.  In registers lane
    // (r, c) = (lane % 16, lane / 16) holds columns 16 j + 4 c .. +3 of row r;
    // each wave parks its 128 x 64 block in the idle ring (rows of 128 bytes,
    // 16-byte chunks XOR-swizzled by the row) and reads it back as 16-byte
    // pieces, 8 lanes to a row, so that each store writes whole 128-byte row
    // segments with consecutive lanes on consecutive bytes.
    u32x4_t stv[WGRAD ? 2 * TM : 1];
    if constexpr (WGRAD) {
      if (persist && tid == 0) tile_slot[(it + 1) & 1] = claim;
      wait_lgkm0();
      ring_barrier();    // every wave is done with the ring; the claim is visible
      uint16_t* const st = ring + wave * (BMW * BNW);
      static_assert(BNW == 64 && NW * BMW * BNW <= 2 * (SP + SQ), "staging fits the ring");
      const int r = lane & 15, c = lane >> 4;
      if (nk == 0) {   // a segment without rows: its block is zero
#pragma unroll
        for (int t = 0; t < 2 * TM; ++t) stv[t] = u32x4_t{0u, 0u, 0u, 0u};
      } else {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          uint2 pk;
          pk.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
          pk.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
          const int row = i * 16 + r;
          *reinterpret_cast<uint2*>(st + row * 64 + (((2 * j + (c >> 1)) ^ (row & 7)) << 3) + (c & 1) * 4) = pk;
        }
#pragma unroll
      for (int t = 0; t < 2 * TM; ++t) {
        const int row = t * 8 + (lane >> 3);
        stv[t] = *reinterpret_cast<const u32x4_t*>(st + row * 64 + (((lane & 7) ^ (row & 7)) << 3));
      }
      wait_lgkm0();
      ring_barrier();    // every wave has its rows back
      }
    }
    if (persist) {
      more = setup(claimed_tile((it + 1) & 1));
      if (more) {
        if (nk > 0) prologue();
        if (tid == 0) claim = atomicAdd(a.counter + cq + zl, 1);
      }
    }

    // epilogue: lane holds output columns 4*(lane/16)+q of tile j, row lane%16
    // of tile i.  dH: the saved pre-activations of row block i+1 are requested
    // before block i is finished, so their latency overlaps the stores.
    const int64_t crow0 = WGRAD ? 0 : (int64_t)cg * a.c_row_seg;
    uint16_t* const cbase = a.C + (WGRAD ? (int64_t)cg * a.c_seg : 0);
    constexpr bool LOADS = KIND == BG_DH && EPI != 0;
    uint2 s1v[2][TN], s2v[2][TN];
    auto load_saved = [&](int i, int buf) {
      const int m = cm0 + wm * BMW + i * 16 + (lane & 15);
      const int64_t row = (crow0 + m) * a.ldc;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = cn0 + wn * BNW + j * 16 + 4 * (lane >> 4);
        const bool ok = m < cm1 && col < N;
        s1v[buf][j] = ok ? *reinterpret_cast<const uint2*>(a.S1 + row + col) : uint2{0u, 0u};
        if constexpr (EPI == 3)
          s2v[buf][j] = ok ? *reinterpret_cast<const uint2*>(a.S2 + row + col) : uint2{0u, 0u};
      }
    };
    if constexpr (WGRAD) {
#pragma unroll
      for (int t = 0; t < 2 * TM; ++t) {
        const int m = cm0 + wm * BMW + t * 8 + (lane >> 3);
        const int col = cn0 + wn * BNW + 8 * (lane & 7);
        if (m < cm1 && col < N) *reinterpret_cast<u32x4_t*>(cbase + (int64_t)m * a.ldc + col) = stv[t];
      }
    } else {
    if constexpr (LOADS) load_saved(0, 0);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if constexpr (LOADS) {
        if (i + 1 < TM) load_saved(i + 1, (i + 1) & 1);
      }
      const int m = cm0 + wm * BMW + i * 16 + (lane & 15);
      if (m >= cm1) continue;
      const int64_t row = (crow0 + m) * a.ldc;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = cn0 + wn * BNW + j * 16 + 4 * (lane >> 4);
        if (col >= N) continue;
        float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
        if constexpr (KIND == BG_DX) {
          if (ctail >= 0) {   // a tail entry: its fp32 partial, added in order by the tail reduce
            *reinterpret_cast<f32x4_t*>(a.part + ((int64_t)ctail * 256 + (m - cm0)) * 256 +
                                        (col - cn0)) = f32x4_t{v[0], v[1], v[2], v[3]};
            continue;
          }
        }
        if constexpr (LOADS) {
          // activation backward with the saved pre-activations
          const uint2 s1 = s1v[i & 1][j];
          const uint32_t z32[4] = {s1.x & 0xffffu, s1.x >> 16, s1.y & 0xffffu, s1.y >> 16};
          if constexpr (EPI == 3) {
            const uint2 s2 = s2v[i & 1][j];
            const uint32_t u32[4] = {s2.x & 0xffffu, s2.x >> 16, s2.y & 0xffffu, s2.y >> 16};
            float dg[4], du[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float z = bf16_to_f32(z32[q]), u = bf16_to_f32(u32[q]);
              const float sg = sigm(z);
              du[q] = v[q] * z * sg;
              dg[q] = v[q] * u * sg * (1.0f + z * (1.0f - sg));
            }
            uint2 pg, pu;
            pg.x = pack_bf16x2(dg[0], dg[1]);
            pg.y = pack_bf16x2(dg[2], dg[3]);
            pu.x = pack_bf16x2(du[0], du[1]);
            pu.y = pack_bf16x2(du[2], du[3]);
            *reinterpret_cast<uint2*>(cbase + row + col) = pg;
            *reinterpret_cast<uint2*>(a.C2 + row + col) = pu;
            continue;
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float z = bf16_to_f32(z32[q]);
            v[q] = EPI == 1 ? (z > 0.f ? v[q] : 0.f) : v[q] * gelu_grad(z);
          }
        }
        uint2 pk;
        pk.x = pack_bf16x2(v[0], v[1]);
        pk.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(cbase + row + col) = pk;
      }
    }
    }
    exact = cm1 - cm0 == BM && cn0 + BN <= N;
    if (!more) break;
  }  // tiles
}

// ---------------------------------------------------------------- gate step
// One wave per token.  dg_j = <dy_t, O_j> over the kept slots (O the bf16
// expert outputs the forward combined), dO_j = bf16(g_j dy_t) on the
// slot's permuted row, then the score gradient of the token (dense [E]).
__global__ __launch_bounds__(256) void gate_bwd_kernel(GateBwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int d = a.d, k = a.k, E = a.E;
  const int nch = d >> 3;                      // 8-element chunks per row
  const uint16_t* dyr = a.dy + t * d;
  // slot-indexed values stay in registers: every loop over the k <= 16 slots
  // is unrolled with a guard
  float dgv[16], gv[16];
  int ev[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    dgv[j] = 0.f;
    gv[j] = 0.f;
    ev[j] = -1;
    if (j >= k) continue;
    const int r = a.slot_pos[t * k + j];
    const float g = a.gate[t * k + j];
    ev[j] = a.topk_idx[t * k + j];
    gv[j] = g;
    if (r < 0) continue;                       // dropped: no output, dg = 0
    float s = 0.f;
    for (int c = lane; c < nch; c += 64) {
      const u32x4_t y8 = *reinterpret_cast<const u32x4_t*>(dyr + c * 8);
      float yf[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        yf[2 * q] = bf16_to_f32(y8[q] & 0xffffu);
        yf[2 * q + 1] = bf16_to_f32(y8[q] >> 16);
      }
      float of[8];
      const u32x4_t o8 = *reinterpret_cast<const u32x4_t*>(a.eout + (int64_t)r * d + c * 8);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        of[2 * q] = bf16_to_f32(o8[q] & 0xffffu);
        of[2 * q + 1] = bf16_to_f32(o8[q] >> 16);
      }
      u32x4_t w;
#pragma unroll
      for (int q = 0; q < 8; ++q) s += yf[q] * of[q];
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = pack_bf16x2(g * yf[2 * q], g * yf[2 * q + 1]);
      *reinterpret_cast<u32x4_t*>(a.d_out + (int64_t)r * d + c * 8) = w;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    dgv[j] = s;
  }
  float A = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j < k) A += gv[j] * dgv[j];
  if (a.d_gate && lane < k) {
    float v = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j == lane) v = dgv[j];
    a.d_gate[t * k + lane] = v;
  }
  const float* s_t = a.logits + t * E;
  // full softmax p (needed by the full-softmax gates and by the balance loss)
  const bool need_p = a.gating == MOE_GATE_SOFTMAX_FULL || a.aux_scale != 0.f;
  float sv[4], pv[4];
  float mx = -INFINITY;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = lane + 64 * u;
    sv[u] = e < E ? s_t[e] : -INFINITY;
    mx = fmaxf(mx, sv[u]);
  }
  float fp = 0.f;
  if (need_p) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    float z = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      pv[u] = lane + 64 * u < E ? __expf(sv[u] - mx) : 0.f;
      z += pv[u];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off, 64);
    const float inv = 1.0f / z;
#pragma unroll
    for (int u = 0; u < 4; ++u) pv[u] *= inv;
    if (a.aux_scale != 0.f) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = lane + 64 * u;
        if (e < E) fp += pv[u] * (float)a.counts[e];
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) fp += __shfl_xor(fp, off, 64);
    }
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) pv[u] = 0.f;
  }
  // sigmoid gates: Z = sum of the selected sigmoids
  float Zs = 0.f;
  if (a.gating == MOE_GATE_SIGMOID_TOPK) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < k) Zs += sigm(s_t[ev[j]]);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = lane + 64 * u;
    if (e >= E) continue;
    // this expert's slot, if selected
    int js = -1;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j < k && ev[j] == e) js = j;
    float dgs = 0.f, gs = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (j == js) {
        dgs = dgv[j];
        gs = gv[j];
      }
    float ds = 0.f;
    if (a.gating == MOE_GATE_SOFTMAX_TOPK) {
      if (js >= 0) ds = gs * (dgs - A);
    } else if (a.gating == MOE_GATE_SIGMOID_TOPK) {
      if (js >= 0) {
        const float sg = sigm(sv[u]);
        ds = sg * (1.0f - sg) * (dgs - A) / Zs;
      }
    } else {
      ds = pv[u] * ((js >= 0 ? dgs : 0.f) - A);
    }
    if (a.aux_scale != 0.f) ds += a.aux_scale * pv[u] * ((float)a.counts[e] - fp);
    a.d_logits[t * E + e] = ds;
  }
}

// ------------------------------------------------------------------ dx step
// One wave per (token, 512 columns), 8 columns per lane: the kept slots' dX
// rows in slot order, then the shared experts', then the router term
// sum_e ds_e W_r[e] (only the selected experts' when the score gradient is
// zero elsewhere).
__global__ __launch_bounds__(256) void dx_kernel(DxArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int d = a.d, k = a.k, E = a.E;
  const float* ds = a.d_logits + t * E;
  {
    const int c = blockIdx.y * 64 + lane;
    if (c >= (d >> 3)) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int r = a.slot_pos[t * k + j];
      if (r < 0) continue;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(a.dxp + (int64_t)r * d + c * 8);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16_to_f32(v[q] & 0xffffu);
        acc[2 * q + 1] += bf16_to_f32(v[q] >> 16);
      }
    }
    for (int s = 0; s < a.S; ++s) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(a.dxs + ((int64_t)s * a.T + t) * d + c * 8);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16_to_f32(v[q] & 0xffffu);
        acc[2 * q + 1] += bf16_to_f32(v[q] >> 16);
      }
    }
    const int n_r = a.sparse_ds ? k : E;
    for (int j = 0; j < n_r; ++j) {
      const int e = a.sparse_ds ? a.topk_idx[t * k + j] : j;
      const float w = ds[e];
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(a.w_router + (int64_t)e * d + c * 8);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += w * bf16_to_f32(v[q] & 0xffffu);
        acc[2 * q + 1] += w * bf16_to_f32(v[q] >> 16);
      }
    }
    u32x4_t o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    *reinterpret_cast<u32x4_t*>(a.dx + t * d + c * 8) = o;
  }
}

// -------------------------------------------------------------- router dW_r
// dW_r[e, i] = sum_t ds[t, e] x[t, i].  Workgroup (1024 columns, 32 experts,
// a chunk of tokens): thread c sums columns 4c..4c+3 over the chunk's tokens
// for the 32 experts, reading each token's 32 score gradients from LDS four
// at a time; the chunks are then added in order.
constexpr int WR_EB = 32;
constexpr int WR_COLS = 1024;
__global__ __launch_bounds__(256) void wr_partial_kernel(WrArgs a) {
  __shared__ __attribute__((aligned(16))) float dsl[64][WR_EB];
  const int i = blockIdx.x * WR_COLS + threadIdx.x * 4;
  const bool col_ok = i < a.d;                 // d is a multiple of 64: 4 columns in or out
  const int e0 = blockIdx.y * WR_EB;
  const int64_t t0 = (int64_t)blockIdx.z * a.chunk;
  const int64_t t1 = t0 + a.chunk < a.T ? t0 + a.chunk : a.T;
  const int ne = a.E - e0 < WR_EB ? a.E - e0 : WR_EB;
  float acc[WR_EB][4];
#pragma unroll
  for (int e = 0; e < WR_EB; ++e)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[e][c] = 0.f;
  for (int64_t tb = t0; tb < t1; tb += 64) {
    __syncthreads();
    for (int q = threadIdx.x; q < 64 * WR_EB; q += 256) {
      const int tt = q / WR_EB, e = q % WR_EB;
      dsl[tt][e] = (tb + tt < t1 && e < ne) ? a.d_logits[(tb + tt) * a.E + e0 + e] : 0.f;
    }
    __syncthreads();
    const int nt = t1 - tb < 64 ? (int)(t1 - tb) : 64;
    // x of 8 tokens in flight before the first is used (tokens past nt read
    // the chunk's last token and add zero: their ds rows are zero in LDS)
    for (int tt = 0; tt < nt && col_ok; tt += 8) {
      uint2 xv[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const int t = tt + v < nt ? tt + v : nt - 1;
        xv[v] = *reinterpret_cast<const uint2*>(a.x + (tb + t) * a.d + i);
      }
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        const float x4[4] = {bf16_to_f32(xv[v].x & 0xffffu), bf16_to_f32(xv[v].x >> 16),
                             bf16_to_f32(xv[v].y & 0xffffu), bf16_to_f32(xv[v].y >> 16)};
#pragma unroll
        for (int e4 = 0; e4 < WR_EB; e4 += 4) {
          const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(&dsl[tt + v][e4]);
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[e4 + u][c] += d4[u] * x4[c];
        }
      }
    }
  }
  if (!col_ok) return;
  float* out = a.partial + ((int64_t)blockIdx.z * a.E + e0) * a.d + i;
#pragma unroll
  for (int e = 0; e < WR_EB; ++e)
    if (e < ne)
      *reinterpret_cast<f32x4_t*>(out + (int64_t)e * a.d) = f32x4_t{acc[e][0], acc[e][1], acc[e][2], acc[e][3]};
}

__global__ __launch_bounds__(256) void wr_reduce_kernel(WrArgs a, int nchunks) {
  const int64_t n = (int64_t)a.E * a.d;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n) return;
  float s = 0.f;
  for (int c = 0; c < nchunks; ++c) s += a.partial[(int64_t)c * n + idx];
  a.dw_router[idx] = s;
}

// order[] lists the segments with rows by decreasing row count (ties: lower
// index) and spreads the empty ones evenly between them: segment r of the nz
// non-empty ones and empty segment j of the z others are merged by the keys
// (2r + 1) z and (2j + 1) nz (a non-empty one first on equal keys), so the
// blocks that are only zeros are written while other blocks compute instead
// of all at the end.  Also clears the tile counters of the launch that follows.
__global__ __launch_bounds__(256) void seg_order_kernel(const int32_t* seg, int G, int32_t* order,
                                                        int* counter) {
  __shared__ int len[1024];
  __shared__ int nz_count;
  if (threadIdx.x < GB_QUEUES) counter[threadIdx.x] = 0;
  if (threadIdx.x == 0) nz_count = 0;
  for (int g = threadIdx.x; g < G; g += 256) len[g] = seg[g + 1] - seg[g];
  __syncthreads();
  for (int g = threadIdx.x; g < G; g += 256)
    if (len[g] > 0) atomicAdd(&nz_count, 1);
  __syncthreads();
  const int64_t nz = nz_count, z = G - nz_count;
  for (int g = threadIdx.x; g < G; g += 256) {
    int r = 0, pos;
    if (len[g] > 0) {
      for (int h = 0; h < G; ++h) r += len[h] > len[g] || (len[h] == len[g] && h < g);
      // empty segments j with (2j + 1) nz < (2r + 1) z go before it
      const int64_t key = (2 * (int64_t)r + 1) * z;
      int before = 0;
      for (int j = 0; j < z; ++j) before += (2 * (int64_t)j + 1) * nz < key;
      pos = r + before;
    } else {
      for (int h = 0; h < g; ++h) r += len[h] == 0;
      // non-empty segments q with (2q + 1) z <= (2r + 1) nz go before it
      const int64_t key = (2 * (int64_t)r + 1) * nz;
      int before = 0;
      for (int q = 0; q < nz; ++q) before += (2 * (int64_t)q + 1) * z <= key;
      pos = r + before;
    }
    order[pos] = g;
  }
}

__global__ __launch_bounds__(256) void zero_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

int wr_chunk(int64_t T, int E, int d) {
  // enough workgroups to cover the chip about four times over
  const int64_t per = (int64_t)((d + WR_COLS - 1) / WR_COLS) * ((E + WR_EB - 1) / WR_EB);
  int64_t chunks = (4 * 256 + per - 1) / per;
  if (chunks > (T + 63) / 64) chunks = (T + 63) / 64;
  if (chunks < 1) chunks = 1;
  int64_t c = (T + chunks - 1) / chunks;
  c = (c + 63) / 64 * 64;
  return (int)c;
}

}  // namespace

size_t wr_ws_bytes(int64_t T, int E, int d) {
  const int c = wr_chunk(T, E, d);
  const int64_t nch = (T + c - 1) / c;
  return (size_t)nch * E * d * 4;
}

int64_t bwd_dw_blocks(int G, int M, int N) {
  return (int64_t)G * ((M + GB_BM - 1) / GB_BM) * ((N + GB_BN - 1) / GB_BN);
}

// Tail split of a routed dX pass: the plan has about (ceil(rows / BM) + G / 2)
// row tiles per column tile; with fewer than 8 rounds of tiles over the CUs,
// the tiles of the partial last round run in K parts (the plan kernel picks
// the parts from the real tile count: as many as fill the idle CUs, at most
// 8), written as fp32 partials that the tail reduce adds in order; the other
// tiles write bf16 rows.  K must hold at least 32 slabs.
int bwd_dx_split(int64_t rows, int G, int N, int K_all) {
  const int64_t NT = (N + GB_BN - 1) / GB_BN;
  const int64_t V = ((rows + GB_BM - 1) / GB_BM + G / 2) * NT;
  return V > 0 && V < 8 * 256 && K_all / BK >= 32 ? 2 : 1;   // MI355X: 256 CUs
}


int bwd_tile_rows() { return GB_BM; }
int bwd_tile_cols() { return GB_BN; }

hipError_t launch_bwd_gemm(const BwdGemm& b, hipStream_t s) {
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.kind = b.kind;
  a.P = static_cast<const uint16_t*>(b.P);
  a.P2 = static_cast<const uint16_t*>(b.P2);
  a.ldp = b.ldp;
  a.p_seg = b.p_seg;
  a.p_row_seg = b.p_row_seg;
  a.Q = static_cast<const uint16_t*>(b.Q);
  a.Q2 = static_cast<const uint16_t*>(b.Q2 ? b.Q2 : b.Q);
  a.ldq = b.ldq;
  a.q_row_seg = b.q_row_seg;
  a.C = static_cast<uint16_t*>(b.C);
  a.C2 = static_cast<uint16_t*>(b.C2);
  a.ldc = b.ldc;
  a.c_seg = b.c_seg;
  a.c_row_seg = b.c_row_seg;
  a.S1 = static_cast<const uint16_t*>(b.S1);
  a.S2 = static_cast<const uint16_t*>(b.S2);
  a.count = static_cast<const int32_t*>(b.plan);
  a.plan = b.plan ? reinterpret_cast<const PlanEntry*>(static_cast<const char*>(b.plan) + kPlanHeader)
                  : nullptr;
  a.seg = b.seg;
  a.order = b.seg ? b.order : nullptr;
  a.counter = b.seg && b.order ? b.order + b.G : nullptr;   // the ints after the order
  if (a.order) {
    if (b.G > GB_MAX_SEGS) return hipErrorInvalidValue;
    seg_order_kernel<<<1, 256, 0, s>>>(b.seg, b.G, b.order, a.counter);
  }
  a.dense_rows = b.dense_rows;
  a.zero = static_cast<const uint16_t*>(b.zero);
  a.K = b.K;
  a.N = b.N;
  a.M = b.M;
  a.nk1 = b.K / BK;
  a.part = b.part;
  if (b.part && b.kind != BG_DX) return hipErrorInvalidValue;
  a.G = b.G;
  a.MT = (b.M + GB_BM - 1) / GB_BM;
  a.NT = (b.N + GB_BN - 1) / GB_BN;
  constexpr int TH = 64 * GB_NW;
  unsigned grid;
  int64_t prof_rec;
  if (b.kind == BG_DW) {
    const int64_t V = (int64_t)a.G * a.MT * a.NT;
    if (V == 0) return hipSuccess;
    grid = (unsigned)(a.counter && V > cu_count() ? cu_count() : V);
    prof_rec = prof_before(b.name, s);
    bwd_gemm_kernel<BG_DW, 0><<<grid, TH, 0, s>>>(a);
  } else {
    if (b.max_entries == 0) return hipSuccess;
    grid = (unsigned)b.max_entries;
    prof_rec = prof_before(b.name, s);
    if (b.kind == BG_DX) {
      if (b.epi == 1) bwd_gemm_kernel<BG_DX, 1><<<grid, TH, 0, s>>>(a);
      else bwd_gemm_kernel<BG_DX, 0><<<grid, TH, 0, s>>>(a);
    } else {
      switch (b.epi) {
        case 1: bwd_gemm_kernel<BG_DH, 1><<<grid, TH, 0, s>>>(a); break;
        case 2: bwd_gemm_kernel<BG_DH, 2><<<grid, TH, 0, s>>>(a); break;
        case 3: bwd_gemm_kernel<BG_DH, 3><<<grid, TH, 0, s>>>(a); break;
        default: bwd_gemm_kernel<BG_DH, 0><<<grid, TH, 0, s>>>(a); break;
      }
    }
  }
  prof_after(prof_rec, s);
  return hipGetLastError();
}

hipError_t launch_gate_bwd(const GateBwdArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int64_t prof_rec = prof_before("bwd_gate", s);
  gate_bwd_kernel<<<(unsigned)((a.T + 3) / 4), 256, 0, s>>>(a);
  prof_after(prof_rec, s);
  return hipGetLastError();
}

hipError_t launch_dx(const DxArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int64_t prof_rec = prof_before("bwd_dx_sum", s);
  dx_kernel<<<dim3((unsigned)((a.T + 3) / 4), (unsigned)((a.d / 8 + 63) / 64)), 256, 0, s>>>(a);
  prof_after(prof_rec, s);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const WrArgs& in, hipStream_t s) {
  if (in.T == 0) return hipSuccess;
  WrArgs a = in;
  a.chunk = wr_chunk(a.T, a.E, a.d);
  const int nch = (int)((a.T + a.chunk - 1) / a.chunk);
  const int64_t prof_rec = prof_before("bwd_router", s);
  dim3 grid((a.d + WR_COLS - 1) / WR_COLS, (a.E + WR_EB - 1) / WR_EB, nch);
  wr_partial_kernel<<<grid, 256, 0, s>>>(a);
  const int64_t n = (int64_t)a.E * a.d;
  wr_reduce_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a, nch);
  prof_after(prof_rec, s);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 4);
  if (n == 0) return hipSuccess;
  zero_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

}  // namespace moe
