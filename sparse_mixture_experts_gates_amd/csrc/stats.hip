// Routing statistics of one batch: the balance signals a routing pass yields.
//
//   f_i  = count_i / T                 fraction of the tokens sent to expert i
//   P_i  = (1/T) sum_t softmax(s_t)_i  average router probability of expert i
//   loss = alpha * E * sum_i f_i P_i   the Switch balance loss
// ("Mixture of experts", Inside the Model ch. 14, "Auxiliary loss", balance
// loss equation; "Mixture of Experts", LLM tutorial ch. 11, "The auxiliary
// loss"), the drop rate dropped / (T k) (LLM tutorial ch. 11, Exercise 4),
// and the loss-free bias update: b_i moves down by gamma for an expert above
// the mean load T k / E and up by gamma below it (Inside the Model ch. 14,
// "Auxiliary-loss-free balancing").
//
// Two kernels, no atomics, every sum in a fixed order: each workgroup sums
// the softmax probabilities of 128 tokens per expert (per lane over its
// tokens, then the token groups and waves in order), then one workgroup adds
// the workgroups' sums (in chunks, then the chunks in order) and forms the
// rest.  The scores are read once.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int ST_TOKENS = 128;   // tokens per workgroup (32 per wave)
constexpr int ST_FINAL = 1024;   // threads of the finishing workgroup

// Wave layout for E <= EP: TPW tokens side by side, LPT lanes per token, KPL
// experts per lane.  A wave walks its 32 tokens in passes of TPW; eight
// passes of loads are in flight before the first sum.
template <int EP>
__global__ __launch_bounds__(256) void stats_probs_kernel(StatsArgs a) {
  constexpr int TPW = EP >= 64 ? 1 : 64 / EP;
  constexpr int LPT = 64 / TPW;
  constexpr int KPL = EP > 64 ? EP / 64 : 1;
  constexpr int PASSES = 32 / TPW;
  constexpr int BATCH = PASSES < 8 ? PASSES : 8;
  __shared__ float red[4][TPW][EP];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = lane / LPT, sl = lane % LPT;
  const int E = a.E;
  const int64_t t0 = (int64_t)blockIdx.x * ST_TOKENS + wave * 32;
  float acc[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) acc[j] = 0.f;
  for (int pb = 0; pb < PASSES; pb += BATCH) {
    float v[BATCH][KPL];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int64_t t = t0 + (int64_t)(pb + u) * TPW + grp;
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const int e = sl + LPT * j;
        v[u][j] = (t < a.T && e < E) ? a.logits[t * E + e] : -INFINITY;
      }
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int64_t t = t0 + (int64_t)(pb + u) * TPW + grp;
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < KPL; ++j) mx = fmaxf(mx, v[u][j]);
#pragma unroll
      for (int off = LPT / 2; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
      float ex[KPL];
      float z = 0.f;
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        ex[j] = sl + LPT * j < E ? expf(v[u][j] - mx) : 0.f;
        z += ex[j];
      }
#pragma unroll
      for (int off = LPT / 2; off >= 1; off >>= 1) z += __shfl_xor(z, off, 64);
      if (t < a.T) {
#pragma unroll
        for (int j = 0; j < KPL; ++j) acc[j] += ex[j] / z;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < KPL; ++j)
    if (sl + LPT * j < EP) red[wave][grp][sl + LPT * j] = acc[j];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int g = 0; g < TPW; ++g) s += red[w][g][e];
    a.partial[(int64_t)blockIdx.x * E + e] = s;
  }
}

// Thread (chunk c, expert e) adds its chunk of the workgroups' sums in
// order; expert e then adds its chunks in order.
__global__ __launch_bounds__(ST_FINAL) void stats_final_kernel(StatsArgs a, int nblk) {
  __shared__ float part[ST_FINAL];
  __shared__ float fp[256];
  const int E = a.E;
  const int nch = ST_FINAL / E;                       // chunks per expert
  const int per = (nblk + nch - 1) / nch;
  const int tid = threadIdx.x;
  if (tid < nch * E) {
    const int c = tid / E, e = tid - c * E;
    const int b0 = c * per;
    const int b1 = b0 + per < nblk ? b0 + per : nblk;
    float s = 0.f;
    for (int b = b0; b < b1; b += 16) {
      float p[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) p[u] = b + u < b1 ? a.partial[(int64_t)(b + u) * E + e] : 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u) s += p[u];
    }
    part[tid] = s;
  }
  __syncthreads();
  const float T = (float)a.T;
  if (tid < E) {
    const int e = tid;
    float s = 0.f;
    for (int c = 0; c < nch; ++c) s += part[c * E + e];
    const int cnt = a.counts[e];
    const float P = s / T;
    const float f = (float)cnt / T;
    a.P[e] = P;
    a.f[e] = f;
    fp[e] = f * P;
    if (a.bias_out) {
      const int64_t load = (int64_t)cnt * E, mean = a.T * a.k;   // exact comparison
      const float b = a.bias[e];
      a.bias_out[e] = load > mean ? b - a.gamma : (load < mean ? b + a.gamma : b);
    }
  }
  __syncthreads();
  if (tid == 0) {
    float sum = 0.f;
    for (int e = 0; e < E; ++e) sum += fp[e];
    a.loss[0] = a.alpha * (float)E * sum;
    if (a.drop_rate) a.drop_rate[0] = (float)a.dropped[0] / (T * (float)a.k);
  }
}

}  // namespace

int stats_nblocks(int64_t T) { return (int)((T + ST_TOKENS - 1) / ST_TOKENS); }

size_t stats_ws_bytes(int64_t T, int E) { return (size_t)stats_nblocks(T) * E * 4; }

hipError_t launch_stats(const StatsArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int nblk = stats_nblocks(a.T);
  const int64_t prof_rec = prof_before("routing_stats", s);
  if (a.E <= 8) stats_probs_kernel<8><<<nblk, 256, 0, s>>>(a);
  else if (a.E <= 16) stats_probs_kernel<16><<<nblk, 256, 0, s>>>(a);
  else if (a.E <= 32) stats_probs_kernel<32><<<nblk, 256, 0, s>>>(a);
  else if (a.E <= 64) stats_probs_kernel<64><<<nblk, 256, 0, s>>>(a);
  else if (a.E <= 128) stats_probs_kernel<128><<<nblk, 256, 0, s>>>(a);
  else stats_probs_kernel<256><<<nblk, 256, 0, s>>>(a);
  stats_final_kernel<<<1, ST_FINAL, 0, s>>>(a, nblk);
  prof_after(prof_rec, s);
  return hipGetLastError();
}

}  // namespace moe
