// Router: score GEMM fused with per-token top-k and gates.
//
// s = W_r x (+ o) ["Mixture of experts", Inside the Model ch. 14, "The
// computation"], top-k of the selection key and the gates over the kept
// experts ["Mixture of Experts", LLM tutorial ch. 11, "The routing decision";
// Inside the Model ch. 14, "Auxiliary-loss-free balancing"], all in FP32 as
// the LLM tutorial's "Training instability" section requires of the router.
//
// One workgroup (4 waves) owns BT tokens (16..64, fewer for small E so the
// grid covers the chip) and all E (<= 256) experts.  The K loop streams
// 64-wide slabs of x and W_r into an LDS ring with direct-to-LDS loads (whole
// 128-byte lines, XOR-swizzled chunks, several slabs in flight) and runs
// v_mfma_f32_16x16x32_bf16 with experts on the MFMA row side and tokens on the
// column side.  The fp32 scores of the tile then go to LDS, and each wave
// selects the top-k of its tokens with 64-bit (key, ~index) maxima reduced by
// cross-lane shuffles, so ties resolve to the lower expert index.  For E > 64
// (with T > 16) the workgroups of a token block split the experts and write
// the scores, and a second kernel selects from them.
#include "common.h"
#include "launch.h"
#include "permute_fused.h"

namespace moe {

namespace {

constexpr int RT_BT = 64;       // tokens per workgroup (fp32 path)
// From 128 padded experts up (E > 64), T > 16 and a place for the scores, the
// scores are computed in expert slices of 64 (E <= 128) or 128, two per token
// block, and a second kernel runs the top-k: one workgroup per token block
// with every expert streams the whole router matrix through each CU, with
// half the CUs busy at E = 256 (DeepSeek-V3 shape: 0.195 -> 0.086 ms;
// gpt-oss, E = 128: 0.082 -> 0.050 ms, with the four-token selection below).
constexpr int RT_SPLIT_MIN = 128;
constexpr int RT_THREADS = 256;

// Top-k and gates for the BT tokens whose scores sit in lg[BT][ld]; each of
// the 4 waves handles BT/4 tokens, TPW_ of them at a time (0: as many as
// keep one key per lane, at least one).
template <int EP, int BT, int TPW_ = 0>
__device__ void topk_from_lds(const float* lg, int ld, const RouteArgs& a,
                              int64_t t0) {
  constexpr int TPW = TPW_ ? TPW_ : (EP <= 16 ? 4 : (EP <= 32 ? 2 : 1));  // tokens per pass
  constexpr int LPT = 64 / TPW;                            // lanes per token
  constexpr int KPL = EP > LPT ? EP / LPT : 1;             // keys per lane
  static_assert(LPT >= 16, "a token's k <= 16 winners are written by its first k lanes");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sl = lane % LPT;
  const int E = a.E, k = a.k;
  static_assert((BT / 4) % TPW == 0, "tokens per wave");
  for (int tg = 0; tg < (BT / 4) / TPW; ++tg) {
    const int tl = wave * (BT / 4) + tg * TPW + lane / LPT;
    const int64_t t = t0 + tl;
    const float* row = lg + tl * ld;
    uint64_t key[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int e = sl + i * LPT;
      key[i] = 0;
      if (e < E) {
        const float sv = row[e];
        float q = (a.gating == MOE_GATE_SIGMOID_TOPK) ? sigmoidf_(sv) : sv;
        if (a.bias) q = q + a.bias[e];
        key[i] = ((uint64_t)sortable_key(q) << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
      }
    }
    int sel_e[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (r >= k) break;
      uint64_t best = key[0];
#pragma unroll
      for (int i = 1; i < KPL; ++i) best = key[i] > best ? key[i] : best;
#pragma unroll
      for (int off = 1; off < LPT; off <<= 1) {
        const uint64_t o = shfl_xor_u64(best, off);
        best = o > best ? o : best;
      }
      const int e = (int)(0xffffffffu - (uint32_t)best);
      sel_e[r] = e;
#pragma unroll
      for (int i = 0; i < KPL; ++i)
        if (sl + i * LPT == e) key[i] = 0;
    }
    // gates from the raw scores of the kept experts
    float gsum = 0.f, m = -INFINITY;
    float gval[16];
    if (a.gating == MOE_GATE_SOFTMAX_FULL) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        const int e = sl + i * LPT;
        if (e < E) mx = fmaxf(mx, row[e]);
      }
#pragma unroll
      for (int off = 1; off < LPT; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
      float z = 0.f;
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        const int e = sl + i * LPT;
        if (e < E) z += expf(row[e] - mx);
      }
#pragma unroll
      for (int off = 1; off < LPT; off <<= 1) z += __shfl_xor(z, off, 64);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (r >= k) break;
        gval[r] = expf(row[sel_e[r]] - mx) / z;
      }
    } else if (a.gating == MOE_GATE_SIGMOID_TOPK) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (r >= k) break;
        gval[r] = sigmoidf_(row[sel_e[r]]);
        gsum += gval[r];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (r >= k) break;
        gval[r] = gval[r] / gsum;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (r >= k) break;
        m = fmaxf(m, row[sel_e[r]]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (r >= k) break;
        gval[r] = expf(row[sel_e[r]] - m);
        gsum += gval[r];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (r >= k) break;
        gval[r] = gval[r] / gsum;
      }
    }
    if (t < a.T) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (r >= k) break;
        if (sl == r) {
          a.topk_idx[t * k + r] = sel_e[r];
          a.topk_gate[t * k + r] = gval[r];
        }
      }
    }
  }
}

// SCORES: the workgroup takes experts blockIdx.y * EP .. + EP - 1 of the
// tokens' scores and writes them (offset added) to a.logits [T, E] instead of
// running the top-k, which a second kernel then does for all E.
template <int EP, int BT, int NSTAGE, bool SCORES = false>
__global__ __launch_bounds__(RT_THREADS) void route_bf16_kernel(RouteArgs a) {
  constexpr int ROWS = BT + EP;                  // x rows then W_r rows per slab
  constexpr int NG = ROWS / 8, DPW = NG / 4;     // 8-row load groups; per wave
  static_assert(NG % 4 == 0, "load groups must divide over the 4 waves");
  constexpr int SEL = ROWS * 64;                 // bf16 elements per slab
  constexpr int LD = EP + 4;
  constexpr int RING_BYTES = NSTAGE * SEL * 2;
  constexpr int LOGIT_BYTES = BT * LD * 4;
  __shared__ __attribute__((aligned(1024)))
  unsigned char smem[RING_BYTES > LOGIT_BYTES ? RING_BYTES : LOGIT_BYTES];
  uint16_t* ring = reinterpret_cast<uint16_t*>(smem);
  float* lg = reinterpret_cast<float*>(smem);    // aliased after the K loop

  constexpr int ET = EP / 16, TT = BT / 16;
  constexpr int WE = ET < 4 ? ET : 4, WT = 4 / WE;
  constexpr int NE = ET / WE, NT = (TT + WT - 1) / WT;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int we = wave % WE, wt = wave / WE;
  const int64_t t0 = (int64_t)blockIdx.x * BT;
  const int d = a.d, E = a.E;
  const int eb = SCORES ? (int)blockIdx.y * EP : 0;   // first expert of the tile
  const uint16_t* X = static_cast<const uint16_t*>(a.x);
  const uint16_t* W = static_cast<const uint16_t*>(a.w);

  const uint16_t* src[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int row = (wave + i * 4) * 8 + dma_row(lane);
    const int ch = dma_chunk(lane);
    if (row < BT) {
      int64_t t = t0 + row;
      if (t > a.T - 1) t = a.T - 1;
      src[i] = X + t * d + ch * 8;
    } else {
      int e = eb + row - BT;
      if (e > E - 1) e = E - 1;
      src[i] = W + (int64_t)e * d + ch * 8;
    }
  }

  f32x4_t acc[NE][NT];
#pragma unroll
  for (int i = 0; i < NE; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = d / 64;
#pragma unroll
  for (int s = 0; s < NSTAGE - 1; ++s) {
    const int kk = s < nk ? s : nk - 1;
#pragma unroll
    for (int i = 0; i < DPW; ++i) dma_rows(src[i] + kk * 64, ring + s * SEL + (wave + i * 4) * 512);
  }
  int cur_s = 0, nxt_s = NSTAGE - 1;
  for (int kt = 0; kt < nk; ++kt) {
    wait_vm_lgkm0<(NSTAGE - 2) * DPW>();
    ring_barrier();
    const int kn = kt + NSTAGE - 1 < nk ? kt + NSTAGE - 1 : nk - 1;
#pragma unroll
    for (int i = 0; i < DPW; ++i) dma_rows(src[i] + kn * 64, ring + nxt_s * SEL + (wave + i * 4) * 512);
    const uint16_t* bx = ring + cur_s * SEL;
    const uint16_t* bw = bx + BT * 64;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ch = kk * 4 + (lane >> 4);
      bf16x8_t fx[NT], fw[NE];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int tt = wt + j * WT;
        fx[j] = *reinterpret_cast<const bf16x8_t*>(bx + swz((tt < TT ? tt : 0) * 16 + (lane & 15), ch));
      }
#pragma unroll
      for (int i = 0; i < NE; ++i)
        fw[i] = *reinterpret_cast<const bf16x8_t*>(bw + swz((we + i * WE) * 16 + (lane & 15), ch));
#pragma unroll
      for (int i = 0; i < NE; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[i], fx[j], acc[i][j], 0, 0, 0);
    }
    cur_s = cur_s + 1 == NSTAGE ? 0 : cur_s + 1;
    nxt_s = nxt_s + 1 == NSTAGE ? 0 : nxt_s + 1;
  }
  wait_vm_lgkm0<0>();
  ring_barrier();   // every wave is done with the ring before it becomes the score tile
  // scores -> LDS: lane holds experts 4*(lane/16)+r of tile i, token lane%16 of tile j
#pragma unroll
  for (int i = 0; i < NE; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int tt = wt + j * WT;
      if (tt >= TT) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = (we + i * WE) * 16 + 4 * (lane >> 4) + r;
        const int tl = tt * 16 + (lane & 15);
        float v = acc[i][j][r];
        if (a.offset && eb + e < E) v += a.offset[eb + e];
        lg[tl * LD + e] = v;
      }
    }
  __syncthreads();
  if constexpr (SCORES) {
    for (int idx = tid; idx < BT * EP; idx += RT_THREADS) {
      const int tl = idx / EP, e = idx - tl * EP;
      if (t0 + tl < a.T && eb + e < E) a.logits[(t0 + tl) * E + eb + e] = lg[tl * LD + e];
    }
    return;
  }
  if (a.logits) {
    for (int idx = tid; idx < BT * E; idx += RT_THREADS) {
      const int tl = idx / E, e = idx - tl * E;
      if (t0 + tl < a.T) a.logits[(t0 + tl) * E + e] = lg[tl * LD + e];
    }
  }
  topk_from_lds<EP, BT>(lg, LD, a, t0);
}

// Top-k and gates of BT tokens from scores [T, E] in global memory (written
// by the SCORES passes).
template <int EP, int BT>
__global__ __launch_bounds__(RT_THREADS) void route_topk_kernel(RouteArgs a, const float* sc) {
  constexpr int LD = EP + 4;
  __shared__ float lg[BT * LD];
  const int64_t t0 = (int64_t)blockIdx.x * BT;
  const int E = a.E;
  // every load of the tile in flight before the first LDS store
  constexpr int PER = BT * EP / RT_THREADS;
  static_assert(BT * EP % RT_THREADS == 0, "tile divides over the threads");
  float v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int idx = u * RT_THREADS + threadIdx.x;
    const int tl = idx / EP, e = idx - tl * EP;
    const int64_t t = t0 + tl < a.T ? t0 + tl : a.T - 1;
    v[u] = e < E ? sc[t * E + e] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int idx = u * RT_THREADS + threadIdx.x;
    lg[(idx / EP) * LD + idx % EP] = v[u];
  }
  __syncthreads();
  // four tokens per wave pass: 16 lanes per token, so each selection round is
  // four shuffle steps and four tokens advance together.  Full-softmax gates
  // sum exp over every expert across the lanes, so they keep the fused
  // kernel's lane layout (and its summation order: the same bits).
  if (a.gating == MOE_GATE_SOFTMAX_FULL)
    topk_from_lds<EP, BT>(lg, LD, a, t0);
  else
    topk_from_lds<EP, BT, 4>(lg, LD, a, t0);
}

// Small batches (T <= 16, bf16): one workgroup of 8 waves splits the K
// dimension instead of the tokens.  Wave w takes the 32-wide k steps
// s = w, w+8, ...; its operands come straight from global memory into the
// MFMA operand registers (16 bytes per lane: token or expert row l%16, k
// chunk l/16), two steps in flight.  The 8 partial score tiles are summed in
// LDS in wave order (deterministic), then the usual top-k runs.
constexpr int RS_WAVES = 8;
constexpr int RS_THREADS = 64 * RS_WAVES;

template <int EP>
__global__ __launch_bounds__(RS_THREADS) void route_small_kernel(RouteArgs a) {
  constexpr int ET = EP / 16, LD = EP + 4;
  __shared__ float lg[16 * LD];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d = a.d, E = a.E;
  const uint16_t* X = static_cast<const uint16_t*>(a.x);
  const uint16_t* W = static_cast<const uint16_t*>(a.w);
  int t = lane & 15;
  if (t > a.T - 1) t = (int)a.T - 1;
  const uint16_t* xrow = X + (int64_t)t * d + 8 * (lane >> 4);
  const uint16_t* wrow[ET];
#pragma unroll
  for (int i = 0; i < ET; ++i) {
    int e = i * 16 + (lane & 15);
    if (e > E - 1) e = E - 1;
    wrow[i] = W + (int64_t)e * d + 8 * (lane >> 4);
  }
  f32x4_t acc[ET];
#pragma unroll
  for (int i = 0; i < ET; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int ns = d / 32;
  constexpr int STEP = EP <= 128 ? 2 : 1;   // k steps in flight per wave
  for (int st = wave; st < ns; st += STEP * RS_WAVES) {
    const int st2 = st + RS_WAVES;
    const bool two = STEP == 2 && st2 < ns;
    const bf16x8_t x0 = *reinterpret_cast<const bf16x8_t*>(xrow + st * 32);
    bf16x8_t w0[ET], w1[ET], x1 = x0;
#pragma unroll
    for (int i = 0; i < ET; ++i) w0[i] = *reinterpret_cast<const bf16x8_t*>(wrow[i] + st * 32);
    if (two) {
      x1 = *reinterpret_cast<const bf16x8_t*>(xrow + st2 * 32);
#pragma unroll
      for (int i = 0; i < ET; ++i) w1[i] = *reinterpret_cast<const bf16x8_t*>(wrow[i] + st2 * 32);
    }
#pragma unroll
    for (int i = 0; i < ET; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0[i], x0, acc[i], 0, 0, 0);
    if (two) {
#pragma unroll
      for (int i = 0; i < ET; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1[i], x1, acc[i], 0, 0, 0);
    }
  }
  // sum the partial tiles in wave order
  for (int w = 0; w < RS_WAVES; ++w) {
    if (wave == w) {
#pragma unroll
      for (int i = 0; i < ET; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = i * 16 + 4 * (lane >> 4) + r;
          float* dst = &lg[(lane & 15) * LD + e];
          *dst = (w == 0 ? 0.f : *dst) + acc[i][r];
        }
    }
    __syncthreads();
  }
  if (a.offset) {
    for (int idx = tid; idx < 16 * E; idx += RS_THREADS) {
      const int tl = idx / E, e = idx - tl * E;
      lg[tl * LD + e] += a.offset[e];
    }
    __syncthreads();
  }
  if (a.logits) {
    for (int idx = tid; idx < (int)a.T * E; idx += RS_THREADS) {
      const int tl = idx / E, e = idx - tl * E;
      a.logits[tl * E + e] = lg[tl * LD + e];
    }
  }
  if (wave < 4) topk_from_lds<EP, 16>(lg, LD, a, 0);
}

// Small batches with a workspace: the same scores from many workgroups.
// Workgroup (e, s) computes the 16-expert x 16-token tile e over the s-th
// part of K (4 waves, operands straight from global memory), sums its waves
// in LDS in wave order and stores the partial tile; one more workgroup adds
// the parts in order and runs the top-k.  Deterministic, and the weights are
// read by the whole chip instead of one CU.
constexpr int RP_MAX_SPLIT = 64;

template <int EP>
__global__ __launch_bounds__(256) void route_partial_kernel(RouteArgs a, int nsplit,
                                                            int* done = nullptr) {
  __shared__ float red[16 * 17];
  if (done && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *done = 0;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int et = blockIdx.x, ks = blockIdx.y;
  const int d = a.d, E = a.E;
  const uint16_t* X = static_cast<const uint16_t*>(a.x);
  const uint16_t* W = static_cast<const uint16_t*>(a.w);
  int t = lane & 15;
  if (t > a.T - 1) t = (int)a.T - 1;
  int e = et * 16 + (lane & 15);
  if (e > E - 1) e = E - 1;
  const uint16_t* xrow = X + (int64_t)t * d + 8 * (lane >> 4);
  const uint16_t* wrow = W + (int64_t)e * d + 8 * (lane >> 4);
  const int ns = d / 32;
  const int per = (ns + nsplit - 1) / nsplit;
  const int s0 = ks * per, s1 = s0 + per < ns ? s0 + per : ns;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int st = s0 + wave; st < s1; st += 4) {
    const bf16x8_t xv = *reinterpret_cast<const bf16x8_t*>(xrow + st * 32);
    const bf16x8_t wv = *reinterpret_cast<const bf16x8_t*>(wrow + st * 32);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv, xv, acc, 0, 0, 0);
  }
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float* dst = &red[(lane & 15) * 17 + 4 * (lane >> 4) + r];
        *dst = (w == 0 ? 0.f : *dst) + acc[r];
      }
    }
    __syncthreads();
  }
  // partial[ks][token][EP]
  float* out = a.partial + (int64_t)ks * 16 * EP;
  const int tl = tid >> 4, ei = tid & 15;
  out[tl * EP + et * 16 + ei] = red[tl * 17 + ei];
}

// One workgroup per token: a single CU keeps only so many misses in flight,
// so the parts (written by other XCDs, hence read from beyond L2) are spread
// over T workgroups.  Block b adds the parts of token b in order and runs
// the top-k for it alone (the other rows of the score tile are masked by
// passing T = b + 1).
// Every thread of the workgroup calls it (it holds a barrier); the first 256
// do the work.
template <int EP>
__device__ void route_reduce_topk_body(const RouteArgs& a, int nsplit, int b) {
  constexpr int TPW = EP <= 16 ? 4 : (EP <= 32 ? 2 : 1);   // as in topk_from_lds
  constexpr int BT = 4 * TPW, LD = EP + 4;
  __shared__ float lg[BT * LD];
  const int tid = threadIdx.x, E = a.E;
  for (int e = tid; e < EP && tid < 256; e += 256) {
    float p[16];
    float v = 0.f;
    for (int ks0 = 0; ks0 < nsplit; ks0 += 16) {
#pragma unroll
      for (int u = 0; u < 16; ++u)
        p[u] = ks0 + u < nsplit ? a.partial[((int64_t)(ks0 + u) * 16 + b) * EP + e] : 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u) v += p[u];
    }
    lg[e] = v + ((a.offset && e < E) ? a.offset[e] : 0.f);
  }
  __syncthreads();
  if (tid >= 256) return;
  if (a.logits)
    for (int e = tid; e < E; e += 256) a.logits[(int64_t)b * E + e] = lg[e];
  RouteArgs one = a;
  one.T = b + 1;
  topk_from_lds<EP, BT>(lg, LD, one, b);
}

template <int EP>
__global__ __launch_bounds__(256) void route_reduce_topk_kernel(RouteArgs a, int nsplit) {
  route_reduce_topk_body<EP>(a, nsplit, blockIdx.x);
}

// Small batches in moe_forward: route_reduce_topk_kernel's per-token
// workgroups (1024 threads, the first 256 of them as there), and the last
// of them to finish runs the whole permutation (with the GEMM plans), which
// saves the permutation's own launch on a decode step.  A workgroup counts
// itself done with an agent-scope acquire-release increment after its
// indices are written; route_partial_kernel zeroes the counter before.
// Scores, indices and gates are those of the two-kernel route.
struct RoutePermuteArgs {
  RouteArgs r;
  int nsplit;
  int* done;               // workspace counter, zeroed by the score kernel
  int64_t capacity;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm_src;
  int32_t* slot_pos;
  int32_t* num_dropped;
  int32_t* kept_total;
  PlanSpec ps{};
  int want_plans, tslot;
};

template <int EP>
__global__ __launch_bounds__(1024) void route_reduce_permute_kernel(RoutePermuteArgs p) {
  __shared__ int last;
  const int tid = threadIdx.x;
  route_reduce_topk_body<EP>(p.r, p.nsplit, blockIdx.x);   // all threads: it has a barrier
  __syncthreads();   // this token's indices are written (and acknowledged)
  if (tid == 0)
    last = __hip_atomic_fetch_add(p.done, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
           (int)p.r.T - 1;
  __syncthreads();
  if (!last) return;
  const RouteArgs& a = p.r;
  permute_one_workgroup(a.topk_idx, (int)a.T * a.k, a.E, p.capacity, p.counts, p.offsets,
                        p.perm_src, p.slot_pos, p.num_dropped, p.kept_total, p.ps, p.want_plans,
                        p.tslot, a.k);
}

template <int EP>
void launch_rp(const RoutePermuteArgs& p, hipStream_t s) {
  route_partial_kernel<EP><<<dim3(EP / 16, p.nsplit), 256, 0, s>>>(p.r, p.nsplit, p.done);
  route_reduce_permute_kernel<EP><<<(unsigned)p.r.T, 1024, 0, s>>>(p);
}

int route_split(int d, int E) {
  const int et = (E + 15) / 16;
  int ns = d / 32;
  int sp = 128 / et;
  if (sp > ns / 2) sp = ns / 2;
  if (sp > RP_MAX_SPLIT) sp = RP_MAX_SPLIT;
  return sp < 1 ? 1 : sp;
}

// fp32 inputs: the same tile and top-k, scores by fp32 FMA from LDS slabs.
template <int EP>
__global__ __launch_bounds__(RT_THREADS) void route_f32_kernel(RouteArgs a) {
  constexpr int KS = 32;                       // K slab (floats)
  constexpr int XLD = KS + 1;
  constexpr int LD = EP + 4;
  constexpr int SLAB = (RT_BT + EP) * XLD * 4;
  constexpr int LOGIT = RT_BT * LD * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SLAB > LOGIT ? SLAB : LOGIT];
  float* xs = reinterpret_cast<float*>(smem);   // [64][XLD]
  float* ws = xs + RT_BT * XLD;                 // [EP][XLD]
  float* lg = reinterpret_cast<float*>(smem);

  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * RT_BT;
  const int d = a.d, E = a.E;
  const float* X = static_cast<const float*>(a.x);
  const float* W = static_cast<const float*>(a.w);
  const int tl = tid & 63, eg = tid >> 6;
  constexpr int NPT = EP / 4;
  float acc[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) acc[i] = 0.f;
  for (int k0 = 0; k0 < d; k0 += KS) {
    const int kw = d - k0 < KS ? d - k0 : KS;
    for (int idx = tid; idx < (RT_BT + EP) * KS; idx += RT_THREADS) {
      const int row = idx / KS, kk = idx - row * KS;
      float v = 0.f;
      if (kk < kw) {
        if (row < RT_BT) {
          int64_t t = t0 + row;
          if (t > a.T - 1) t = a.T - 1;
          v = X[t * d + k0 + kk];
        } else {
          int e = row - RT_BT;
          if (e > E - 1) e = E - 1;
          v = W[(int64_t)e * d + k0 + kk];
        }
      }
      xs[row * XLD + kk] = v;   // ws follows xs contiguously with the same stride
    }
    __syncthreads();
    for (int kk = 0; kk < kw; ++kk) {
      const float xv = xs[tl * XLD + kk];
#pragma unroll
      for (int i = 0; i < NPT; ++i) acc[i] = fmaf(xv, ws[(eg + 4 * i) * XLD + kk], acc[i]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int e = eg + 4 * i;
    float v = acc[i];
    if (a.offset && e < E) v += a.offset[e];
    lg[tl * LD + e] = v;
  }
  __syncthreads();
  if (a.logits) {
    for (int idx = tid; idx < RT_BT * E; idx += RT_THREADS) {
      const int t = idx / E, e = idx - t * E;
      if (t0 + t < a.T) a.logits[(t0 + t) * E + e] = lg[t * LD + e];
    }
  }
  topk_from_lds<EP, RT_BT>(lg, LD, a, t0);
}

template <int EP, int BT, int NS>
hipError_t launch_ep(const RouteArgs& a, hipStream_t s) {
  const int64_t prof_rec = prof_before("route", s);
  if (a.dtype == MOE_BF16 && a.T <= 16 && a.partial) {
    const int sp = route_split(a.d, a.E);
    route_partial_kernel<EP><<<dim3(EP / 16, sp), 256, 0, s>>>(a, sp);
    route_reduce_topk_kernel<EP><<<(unsigned)a.T, 256, 0, s>>>(a, sp);
  } else if (a.dtype == MOE_BF16 && a.T <= 16) {
    route_small_kernel<EP><<<1, RS_THREADS, 0, s>>>(a);
  } else if (EP >= RT_SPLIT_MIN && a.dtype == MOE_BF16 && (a.logits || a.partial)) {
    if constexpr (EP >= RT_SPLIT_MIN) {
      constexpr int EPW = EP > 128 ? 128 : 64;   // experts per workgroup
      RouteArgs b = a;
      b.logits = a.logits ? a.logits : a.partial;
      route_bf16_kernel<EPW, 64, 4, true>
          <<<dim3((unsigned)((a.T + 63) / 64), EP / EPW), RT_THREADS, 0, s>>>(b);
      route_topk_kernel<EP, 16><<<(unsigned)((a.T + 15) / 16), RT_THREADS, 0, s>>>(a, b.logits);
    }
  } else if (a.dtype == MOE_BF16)
    route_bf16_kernel<EP, BT, NS><<<(unsigned)((a.T + BT - 1) / BT), RT_THREADS, 0, s>>>(a);
  else
    route_f32_kernel<EP><<<(unsigned)((a.T + RT_BT - 1) / RT_BT), RT_THREADS, 0, s>>>(a);
  prof_after(prof_rec, s);
  return hipGetLastError();
}

}  // namespace

static int padded_experts(int E) {
  return E <= 16 ? 16 : E <= 32 ? 32 : E <= 64 ? 64 : E <= 128 ? 128 : 256;
}

size_t route_ws_bytes(int64_t T, int E, int dtype) {
  if (dtype != MOE_BF16) return 0;
  if (T > 16) return E > RT_SPLIT_MIN / 2 ? (size_t)T * E * 4 : 0;   // scores of the split pass
  // the score parts, then the done-counter of the fused small-batch path
  return (size_t)RP_MAX_SPLIT * 16 * padded_experts(E) * 4 + 256;
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  // (padded E, tokens per workgroup, ring depth): fewer tokens per workgroup
  // for small E so that the grid covers the chip
  // E <= 16: 4 KB slabs, so a long K keeps 11 of them in flight (Mixtral
  // shape, d = 4096: 19 -> 15 us); a short one (Switch, d = 768) is faster
  // with 4 stages and more workgroups per CU
  if (a.E <= 16) return a.d >= 2048 ? launch_ep<16, 16, 12>(a, s) : launch_ep<16, 16, 4>(a, s);
  if (a.E <= 32) return launch_ep<32, 32, 4>(a, s);
  if (a.E <= 64) return launch_ep<64, 32, 4>(a, s);
  if (a.E <= 128) return launch_ep<128, 64, 4>(a, s);
  return launch_ep<256, 64, 3>(a, s);
}

bool route_permute_small_ok(const RouteArgs& ra, const PermuteArgs& pa) {
  return ra.dtype == MOE_BF16 && ra.T >= 1 && ra.T <= 16 && ra.partial && pa.x_perm == nullptr &&
         ra.T * ra.k <= FUSED_MAX;
}

hipError_t launch_route_permute_small(const RouteArgs& ra, const PermuteArgs& pa, hipStream_t s,
                                      bool* plans_built) {
  if (plans_built) *plans_built = false;
  if (!route_permute_small_ok(ra, pa)) return hipErrorInvalidValue;
  RoutePermuteArgs p;
  p.r = ra;
  p.nsplit = route_split(ra.d, ra.E);
  p.done = reinterpret_cast<int*>(ra.partial + (size_t)RP_MAX_SPLIT * 16 * padded_experts(ra.E));
  p.capacity = pa.capacity;
  p.counts = pa.counts;
  p.offsets = pa.offsets;
  p.perm_src = pa.perm_src;
  p.slot_pos = pa.slot_pos;
  p.num_dropped = pa.num_dropped;
  p.kept_total = pa.kept_total;
  p.ps = pa.plans ? *pa.plans : PlanSpec{0, 0, 0, 1, nullptr, nullptr, 0};
  p.want_plans = pa.plans ? 1 : 0;
  p.tslot = pa.slot_major && pa.k > 1 ? (int)pa.T : 0;
  const int64_t prof_rec = prof_before("route_permute", s);
  if (ra.E <= 16) launch_rp<16>(p, s);
  else if (ra.E <= 32) launch_rp<32>(p, s);
  else if (ra.E <= 64) launch_rp<64>(p, s);
  else if (ra.E <= 128) launch_rp<128>(p, s);
  else launch_rp<256>(p, s);
  prof_after(prof_rec, s);
  if (plans_built && pa.plans) *plans_built = true;
  return hipGetLastError();
}

}  // namespace moe
