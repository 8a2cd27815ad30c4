// Router: score GEMM fused with per-token top-k and gates.
//
// s = W_r x (+ o) ["Mixture of experts", Inside the Model ch. 14, "The
// computation"], top-k of the selection key and the gates over the kept
// experts ["Mixture of Experts", LLM tutorial ch. 11, "The routing decision";
// Inside the Model ch. 14, "Auxiliary-loss-free balancing"], all in FP32 as
// the LLM tutorial's "Training instability" section requires of the router.
//
// One workgroup (4 waves) owns 64 tokens and all E (<= 256) experts.  The
// K loop stages 64-wide slabs of x and W_r in LDS (XOR-swizzled 16-byte
// chunks, double-buffered through registers) and runs v_mfma_f32_16x16x32_bf16
// with experts on the MFMA row side and tokens on the column side.  The fp32
// scores of the tile then go to LDS, and each wave selects the top-k of its
// tokens with 64-bit (key, ~index) maxima reduced by cross-lane shuffles, so
// ties resolve to the lower expert index.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int RT_BT = 64;       // tokens per workgroup
constexpr int RT_BK = 64;       // K slab (elements)
constexpr int RT_THREADS = 256;

__device__ __forceinline__ int swz(int row, int chunk) {  // bf16 element offset
  return row * RT_BK + ((chunk ^ (row & 7)) << 3);
}

// Top-k and gates for the 64 tokens whose scores sit in lg[64][ld].
template <int EP>
__device__ void topk_from_lds(const float* lg, int ld, const RouteArgs& a,
                              int64_t t0) {
  constexpr int TPW = EP <= 16 ? 4 : (EP <= 32 ? 2 : 1);  // tokens per wave pass
  constexpr int LPT = 64 / TPW;                            // lanes per token
  constexpr int KPL = EP > 64 ? EP / 64 : 1;               // keys per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sl = lane % LPT;
  const int E = a.E, k = a.k;
  for (int tg = 0; tg < 16 / TPW; ++tg) {
    const int tl = wave * 16 + tg * TPW + lane / LPT;
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

template <int EP>
struct RouteLds {
  static constexpr int SX = RT_BT * RT_BK;   // bf16 elements per x stage
  static constexpr int SW = EP * RT_BK;      // bf16 elements per w stage
  static constexpr int STAGE_BYTES = 2 * (SX + SW) * 2;
  static constexpr int LD = EP + 4;
  static constexpr int LOGIT_BYTES = RT_BT * LD * 4;
  static constexpr int BYTES = STAGE_BYTES > LOGIT_BYTES ? STAGE_BYTES : LOGIT_BYTES;
};

template <int EP>
__global__ __launch_bounds__(RT_THREADS) void route_bf16_kernel(RouteArgs a) {
  using L = RouteLds<EP>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::BYTES];
  uint16_t* sx = reinterpret_cast<uint16_t*>(smem);        // [2][SX]
  uint16_t* sw = sx + 2 * L::SX;                           // [2][SW]
  float* lg = reinterpret_cast<float*>(smem);              // aliased after the K loop

  constexpr int ET = EP / 16, TT = RT_BT / 16;
  constexpr int WE = ET < 4 ? ET : 4, WT = 4 / WE;
  constexpr int NE = ET / WE, NT = TT / WT;
  constexpr int CHUNKS = (RT_BT + EP) * 8;
  constexpr int CPT = (CHUNKS + RT_THREADS - 1) / RT_THREADS;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int we = wave % WE, wt = wave / WE;
  const int64_t t0 = (int64_t)blockIdx.x * RT_BT;
  const int d = a.d, E = a.E;
  const uint16_t* X = static_cast<const uint16_t*>(a.x);
  const uint16_t* W = static_cast<const uint16_t*>(a.w);

  const uint16_t* src[CPT];
  int dst[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + i * RT_THREADS;
    src[i] = nullptr;
    dst[i] = -1;
    if (c < CHUNKS) {
      const int row = c >> 3, ch = c & 7;
      if (row < RT_BT) {
        int64_t t = t0 + row;
        if (t > a.T - 1) t = a.T - 1;
        src[i] = X + t * d + ch * 8;
        dst[i] = swz(row, ch);
      } else {
        int e = row - RT_BT;
        if (e > E - 1) e = E - 1;
        src[i] = W + (int64_t)e * d + ch * 8;
        dst[i] = L::SX * 2 + swz(row - RT_BT, ch);   // offset into sw region of stage 0
      }
    }
  }
  u32x4_t stage[CPT];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      if (dst[i] >= 0) stage[i] = *reinterpret_cast<const u32x4_t*>(src[i] + k0);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      if (dst[i] < 0) continue;
      int off = dst[i];
      // x chunks live in sx[buf], w chunks in sw[buf]
      uint16_t* base = off >= L::SX * 2 ? sw + buf * L::SW + (off - L::SX * 2)
                                        : sx + buf * L::SX + off;
      *reinterpret_cast<u32x4_t*>(base) = stage[i];
    }
  };

  f32x4_t acc[NE][NT];
#pragma unroll
  for (int i = 0; i < NE; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = d / RT_BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * RT_BK);
    const uint16_t* bx = sx + buf * L::SX;
    const uint16_t* bw = sw + buf * L::SW;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ch = kk * 4 + (lane >> 4);
      bf16x8_t fx[NT], fw[NE];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int row = (wt + j * WT) * 16 + (lane & 15);
        fx[j] = *reinterpret_cast<const bf16x8_t*>(bx + swz(row, ch));
      }
#pragma unroll
      for (int i = 0; i < NE; ++i) {
        const int row = (we + i * WE) * 16 + (lane & 15);
        fw[i] = *reinterpret_cast<const bf16x8_t*>(bw + swz(row, ch));
      }
#pragma unroll
      for (int i = 0; i < NE; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[i], fx[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }
  // scores -> LDS: lane holds experts 4*(lane/16)+r of tile i, token lane%16 of tile j
#pragma unroll
  for (int i = 0; i < NE; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = (we + i * WE) * 16 + 4 * (lane >> 4) + r;
        const int tl = (wt + j * WT) * 16 + (lane & 15);
        float v = acc[i][j][r];
        if (a.offset && e < E) v += a.offset[e];
        lg[tl * L::LD + e] = v;
      }
  __syncthreads();
  if (a.logits) {
    for (int idx = tid; idx < RT_BT * E; idx += RT_THREADS) {
      const int tl = idx / E, e = idx - tl * E;
      if (t0 + tl < a.T) a.logits[(t0 + tl) * E + e] = lg[tl * L::LD + e];
    }
  }
  topk_from_lds<EP>(lg, L::LD, a, t0);
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
  topk_from_lds<EP>(lg, LD, a, t0);
}

template <int EP>
hipError_t launch_ep(const RouteArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)((a.T + RT_BT - 1) / RT_BT);
  prof_before("route", s);
  if (a.dtype == MOE_BF16)
    route_bf16_kernel<EP><<<grid, RT_THREADS, 0, s>>>(a);
  else
    route_f32_kernel<EP><<<grid, RT_THREADS, 0, s>>>(a);
  prof_after(s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.E <= 16) return launch_ep<16>(a, s);
  if (a.E <= 32) return launch_ep<32>(a, s);
  if (a.E <= 64) return launch_ep<64>(a, s);
  if (a.E <= 128) return launch_ep<128>(a, s);
  return launch_ep<256>(a, s);
}

}  // namespace moe
