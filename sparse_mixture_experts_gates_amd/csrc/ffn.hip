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
// weight slab are adjacent; the GEMM remaps block ids so that adjacent plan
// entries land on the same XCD (blocks are dealt round-robin over the 8 XCDs),
// which keeps each shared slab in one L2.  No host synchronisation: the grid
// is sized for the worst case and surplus blocks return at once.
//
// bf16 GEMM: XOR-swizzled LDS tiles of 64-wide K slabs, double-buffered
// through registers; v_mfma_f32_16x16x32_bf16 with weights on the MFMA row
// side, so each lane ends with 4 adjacent output columns of one row (8-byte
// stores).  SwiGLU interleaves W1 and W3 rows inside every wave's slab so the
// gate and up accumulators of a column sit in the same lane and the epilogue
// is elementwise.  The fp32 variant is a plain LDS-tiled FMA GEMM.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int MODE_PLAIN = 0, MODE_RELU = 1, MODE_GELU = 2, MODE_SWIGLU = 3;
constexpr int BK = 64;

struct PlanEntry {
  int32_t g, m0, m1, nt;
};

struct KArgs {
  const uint16_t* A;   // or float*
  const uint16_t* W;
  const uint16_t* Wu;
  uint16_t* C;
  const PlanEntry* plan;
  const int32_t* count;
  const int32_t* a_rows;  // optional row indirection for A (row gather folded in)
  int a_div;
  int K, N;
  int64_t a_seg_rows, c_seg_rows;  // extra row offset per segment (shared experts)
};

// Plan: one workgroup; G <= 1024 segments.  Writes the entries of one pass
// (NT column tiles) and, when NT2 > 0, of a second pass over the same row
// tiles with NT2 column tiles (the two expert GEMMs share their row tiling).
__global__ __launch_bounds__(1024) void ffn_plan_kernel(
    const int32_t* __restrict__ seg, int G, int64_t dense_rows, int BM, int NT,
    PlanEntry* __restrict__ plan, int32_t* __restrict__ count, int NT2,
    PlanEntry* __restrict__ plan2, int32_t* __restrict__ count2) {
  __shared__ int mt[1024];
  __shared__ int start[1024];
  __shared__ int rows_s[1024];
  __shared__ int base[1025];
  const int tid = threadIdx.x;
  for (int g = tid; g < G; g += 1024) {
    const int r0 = seg ? seg[g] : 0;
    const int r1 = seg ? seg[g + 1] : (int)dense_rows;
    start[g] = r0;
    rows_s[g] = r1 - r0;
    mt[g] = (r1 - r0 + BM - 1) / BM;
  }
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
    const int nt_all = pass == 0 ? NT : NT2;
    PlanEntry* out = pass == 0 ? plan : plan2;
    if (nt_all <= 0) break;
    const int V = MT * nt_all;
    for (int L = tid; L < V; L += 1024) {
      // entry L: segment-major, then column tile, then row tile
      int lo = 0, hi = G - 1;  // last g with base[g] * nt_all <= L
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (base[mid] * nt_all <= L) lo = mid; else hi = mid - 1;
      }
      const int g = lo, rem = L - base[g] * nt_all, m = mt[g];
      const int nt = rem / m, mi = rem - nt * m;
      const int m0 = start[g] + mi * BM;
      int m1 = m0 + BM;
      if (m1 > start[g] + rows_s[g]) m1 = start[g] + rows_s[g];
      out[L] = PlanEntry{g, m0, m1, nt};
    }
    if (tid == 0) (pass == 0 ? count : count2)[0] = V;
  }
}

// XCD-aware order: physical block P runs on XCD P % 8; give each XCD a
// contiguous run of the V valid plan entries.
__device__ __forceinline__ int xcd_remap(int P, int V) {
  const int x = P & 7, i = P >> 3, q = V >> 3, r = V & 7;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
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
template <int BM, int BN, int WM, int WN, int NSTAGE, int MODE>
__global__ __launch_bounds__(64 * WM * WN)
void ffn_bf16_kernel(KArgs a) {
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

  __shared__ __attribute__((aligned(1024))) uint16_t ring[NSTAGE * SEL];

  const int V = a.count[0];
  const int P = blockIdx.x;
  if (P >= V) return;
  const PlanEntry pe = a.plan[xcd_remap(P, V)];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int wm = wave / WN, wn = wave % WN;
  const int K = a.K, N = a.N;
  const int n0 = pe.nt * BNOUT;
  const int64_t arow0 = (int64_t)pe.g * a.a_seg_rows;
  const int64_t wbase = (int64_t)pe.g * N * K;

  // slab row `row` (tokens first, then weight rows) -> its global row start
  auto row_ptr = [&](int row) -> const uint16_t* {
    if (row < BM) {
      int r = pe.m0 + row;
      if (r > pe.m1 - 1) r = pe.m1 - 1;
      const int64_t sr = a.a_rows ? (int64_t)(a.a_rows[r] / a.a_div) : arow0 + r;
      return a.A + sr * K;
    }
    const int rho = row - BM;
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
    return Wm + wbase + (int64_t)n * K;
  };
  // this lane's source (row, logical chunk) for each 8-row group the wave loads
  const uint16_t* src[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i)
    src[i] = row_ptr((wave + i * NW) * 8 + dma_row(lane)) + dma_chunk(lane) * 8;

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = K / BK;
  if constexpr (NSTAGE == 2) {
    // Two-stage ring, software-pipelined across slabs.  Each slab is used in
    // two halves of 32 k.  Step kt: (A) MFMAs of half 0 of slab kt, with the
    // reads of half 1 spread between them; (B) wait for slab kt+1, barrier,
    // request slab kt+2 into the stage slab kt occupied; (C) MFMAs of half 1
    // of slab kt, with the reads of half 0 of slab kt+1 spread between them.
    // LDS reads never wait at the start of a slab.
    constexpr int NR = TN + TM, NM = TM * TN, PER = NM / NR > 0 ? NM / NR : 1;
    auto read_half = [&](const uint16_t* st, int half, bf16x8_t* fw, bf16x8_t* fx) {
      const uint16_t* sb = st + BM * BK;
      const int ch = half * 4 + (lane >> 4);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fw[j] = *reinterpret_cast<const bf16x8_t*>(sb + swz(wn * BNW + j * 16 + (lane & 15), ch));
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fx[i] = *reinterpret_cast<const bf16x8_t*>(st + swz(wm * BMW + i * 16 + (lane & 15), ch));
    };
#pragma unroll
    for (int i = 0; i < DPW; ++i) dma_rows(src[i], ring + (wave + i * NW) * 512);
    {
      const int k1 = nk > 1 ? 1 : 0;
#pragma unroll
      for (int i = 0; i < DPW; ++i) dma_rows(src[i] + k1 * BK, ring + SEL + (wave + i * NW) * 512);
    }
    wait_vm_lgkm0<DPW>();
    ring_barrier();
    bf16x8_t w0[TN], x0[TM], w1[TN], x1[TM];
    read_half(ring, 0, w0, x0);
    for (int kt = 0; kt < nk; ++kt) {
      const uint16_t* cur = ring + (kt & 1) * SEL;
      const uint16_t* nxt = ring + ((kt + 1) & 1) * SEL;
      // (A)
      read_half(cur, 1, w1, x1);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0[j], x0[i], acc[i][j], 0, 0, 0);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NM - NR * PER, 0);
      // (B)
      wait_vm_lgkm0<0>();
      ring_barrier();
      const int kn = kt + 2 < nk ? kt + 2 : nk - 1;
#pragma unroll
      for (int i = 0; i < DPW; ++i)
        dma_rows(src[i] + kn * BK, const_cast<uint16_t*>(cur) + (wave + i * NW) * 512);
      // (C)
      read_half(nxt, 0, w0, x0);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1[j], x1[i], acc[i][j], 0, 0, 0);
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
      if (MODE == MODE_SWIGLU) {
        col = n0 + wn * HALF + j * 16 + 4 * (lane >> 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = silu_f(acc[i][j][q]) * acc[i][j + TN / 2][q];
      } else {
        col = n0 + wn * BNW + j * 16 + 4 * (lane >> 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = act1<MODE>(acc[i][j][q]);
      }
      uint2 pk;
      pk.x = pack_bf16x2(v[0], v[1]);
      pk.y = pack_bf16x2(v[2], v[3]);
      if (row_ok && col < N) *reinterpret_cast<uint2*>(crow + col) = pk;
    }
  }
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
  const int n0 = pe.nt * TB;
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
  int BM, BNOUT, id;   // id: 0 fp32, 1 small batch, 2 big 256x256, 3 256x128
};

constexpr int kCUs = 256;

// Tile shape of one pass.  Prefill passes use 256 x 256 tiles unless that
// leaves fewer than four rounds of tiles over the CUs (e.g. the second expert
// GEMM with a short N), where 256 x 128 tiles trim the last, partial round.
Shape pick_shape(int dtype, bool small, int mode, int64_t max_rows, int N) {
  if (dtype == MOE_F32) return {64, 64, 0};
  const bool glu = mode == MODE_SWIGLU;
  if (small) return {32, glu ? 64 : 128, 1};
  const int64_t big_tiles = ((max_rows + 255) / 256) * ((N + (glu ? 127 : 255)) / (glu ? 128 : 256));
  if (big_tiles < 4 * kCUs) return {256, glu ? 64 : 128, 3};
  return {256, glu ? 128 : 256, 2};
}

int64_t max_entries(int64_t max_rows, int G, int N, Shape sh) {
  const int64_t nt = (N + sh.BNOUT - 1) / sh.BNOUT;
  return ((max_rows + sh.BM - 1) / sh.BM + G) * nt;
}

template <int BM, int BN, int WM, int WN, int NS>
void launch_bf16(int mode, unsigned grid, const KArgs& k, hipStream_t s) {
  switch (mode) {
    case MODE_PLAIN: ffn_bf16_kernel<BM, BN, WM, WN, NS, MODE_PLAIN><<<grid, 64 * WM * WN, 0, s>>>(k); break;
    case MODE_RELU: ffn_bf16_kernel<BM, BN, WM, WN, NS, MODE_RELU><<<grid, 64 * WM * WN, 0, s>>>(k); break;
    case MODE_GELU: ffn_bf16_kernel<BM, BN, WM, WN, NS, MODE_GELU><<<grid, 64 * WM * WN, 0, s>>>(k); break;
    default: ffn_bf16_kernel<BM, BN, WM, WN, NS, MODE_SWIGLU><<<grid, 64 * WM * WN, 0, s>>>(k); break;
  }
}

}  // namespace

size_t ffn_plan_bytes(int64_t max_rows, int G, int N, bool small, int dtype) {
  size_t best = 0;
  for (int mode = 0; mode < 4; ++mode) {
    const size_t b = 16 + 16 * (size_t)max_entries(max_rows, G, N, pick_shape(dtype, small, mode, max_rows, N));
    if (b > best) best = b;
  }
  return (best + 255) / 256 * 256;
}

namespace {
int pass_nt(const FfnPassArgs& p) {
  const Shape sh = pick_shape(p.dtype, p.small, p.mode, p.max_rows, p.N);
  return (p.N + sh.BNOUT - 1) / sh.BNOUT;
}
}  // namespace

hipError_t launch_ffn_plans(const FfnPassArgs& p1, const FfnPassArgs& p2, hipStream_t s) {
  const Shape sh1 = pick_shape(p1.dtype, p1.small, p1.mode, p1.max_rows, p1.N);
  const Shape sh2 = pick_shape(p2.dtype, p2.small, p2.mode, p2.max_rows, p2.N);
  if (sh1.BM != sh2.BM || p1.seg_offsets != p2.seg_offsets) return hipErrorInvalidValue;
  if (max_entries(p1.max_rows, p1.G, p1.N, sh1) == 0) return hipSuccess;
  int32_t* c1 = static_cast<int32_t*>(p1.plan);
  int32_t* c2 = static_cast<int32_t*>(p2.plan);
  PlanEntry* e1 = reinterpret_cast<PlanEntry*>(static_cast<char*>(p1.plan) + 16);
  PlanEntry* e2 = reinterpret_cast<PlanEntry*>(static_cast<char*>(p2.plan) + 16);
  prof_before(p1.seg_offsets ? "ffn_plan" : "ffn_plan_shared", s);
  ffn_plan_kernel<<<1, 1024, 0, s>>>(p1.seg_offsets, p1.G, p1.dense_rows, sh1.BM, pass_nt(p1), e1, c1,
                                     pass_nt(p2), e2, c2);
  prof_after(s);
  return hipGetLastError();
}

hipError_t launch_ffn_pass(const FfnPassArgs& p, hipStream_t s) {
  const Shape sh = pick_shape(p.dtype, p.small, p.mode, p.max_rows, p.N);
  const int64_t grid = max_entries(p.max_rows, p.G, p.N, sh);
  if (grid == 0) return hipSuccess;
  int32_t* count = static_cast<int32_t*>(p.plan);
  PlanEntry* plan = reinterpret_cast<PlanEntry*>(static_cast<char*>(p.plan) + 16);
  KArgs k;
  k.A = static_cast<const uint16_t*>(p.A);
  k.W = static_cast<const uint16_t*>(p.w);
  k.Wu = static_cast<const uint16_t*>(p.w_up ? p.w_up : p.w);
  k.C = static_cast<uint16_t*>(p.C);
  k.plan = plan;
  k.count = count;
  k.a_rows = p.a_rows;
  k.a_div = p.a_div > 0 ? p.a_div : 1;
  k.K = p.K;
  k.N = p.N;
  k.a_seg_rows = p.a_seg_rows;
  k.c_seg_rows = p.c_seg_rows;
  const char* nm = p.seg_offsets ? (p.mode == MODE_PLAIN ? "ffn2" : "ffn1")
                                 : (p.mode == MODE_PLAIN ? "ffn2_shared" : "ffn1_shared");
  prof_before(nm, s);
  if (p.dtype == MOE_F32) {
    switch (p.mode) {
      case MODE_PLAIN: ffn_f32_kernel<MODE_PLAIN><<<(unsigned)grid, 256, 0, s>>>(k); break;
      case MODE_RELU: ffn_f32_kernel<MODE_RELU><<<(unsigned)grid, 256, 0, s>>>(k); break;
      case MODE_GELU: ffn_f32_kernel<MODE_GELU><<<(unsigned)grid, 256, 0, s>>>(k); break;
      default: ffn_f32_kernel<MODE_SWIGLU><<<(unsigned)grid, 256, 0, s>>>(k); break;
    }
  } else if (sh.id == 1) {
    launch_bf16<32, 128, 1, 4, 4>(p.mode, (unsigned)grid, k, s);
  } else if (sh.id == 3) {
    launch_bf16<256, 128, 4, 2, 3>(p.mode, (unsigned)grid, k, s);
  } else {
    launch_bf16<256, 256, 2, 4, 2>(p.mode, (unsigned)grid, k, s);
  }
  prof_after(s);
  return hipGetLastError();
}

}  // namespace moe
