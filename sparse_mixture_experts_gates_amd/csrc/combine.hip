// Gate-weighted combine: y_t = sum_{kept j} g_tj * out[slot_pos_tj] + shared.
//
// The weighted sum of "Mixture of experts" (Inside the Model ch. 14, "The
// computation"); unselected and dropped experts add exactly zero
// ("Mixture-of-Experts", Neural Networks Visually ch. 15, "Show the math";
// LLM tutorial ch. 11, "Expert capacity and dropped tokens").  One wave per
// token gathers its k expert rows with 16-byte loads, accumulates in fp32 in
// the fixed order j = 0..k-1 then shared experts, and rounds once.  No
// atomics, so the result does not depend on scheduling.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

// One wave per (token, 512 NC-column group): every lane owns NC chunks of 8
// columns, 512 columns apart (one 16-byte load per chunk and source row);
// the loads of all k rows are issued before the sums so that each wave waits
// for memory once.  NC is chosen so that about CB_LOADS loads per lane are in
// flight whatever k is.
constexpr int CB_LOADS = 8;

template <int KMAX, int NC>
__global__ __launch_bounds__(256) void combine_bf16_kernel(CombineArgs a) {
  constexpr int CB_NC = NC, CB_COLS = 512 * NC;
  const int ncg = (a.d + CB_COLS - 1) / CB_COLS;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t t = wid / ncg;
  if (t >= a.T) return;
  const int cg = (int)(wid - t * ncg);
  const int lane = threadIdx.x & 63, k = a.k, d = a.d;
  const int c0 = cg * CB_COLS + lane * 8;
  if (c0 >= d) return;
  const uint16_t* eo = static_cast<const uint16_t*>(a.expert_out);
  const uint16_t* so = static_cast<const uint16_t*>(a.shared_out);
  int sp[KMAX];
  float g[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    sp[j] = j < k ? a.slot_pos[t * k + j] : -1;
    g[j] = sp[j] >= 0 ? a.gate[t * k + j] : 0.f;
  }
  u32x4_t v[KMAX][CB_NC];
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
#pragma unroll
    for (int u = 0; u < CB_NC; ++u) {
      const int c = c0 + u * 512;
      v[j][u] = sp[j] >= 0 && c < d ? *reinterpret_cast<const u32x4_t*>(eo + (int64_t)sp[j] * d + c)
                                    : u32x4_t{0u, 0u, 0u, 0u};
    }
  uint16_t* y = static_cast<uint16_t*>(a.y);
#pragma unroll
  for (int u = 0; u < CB_NC; ++u) {
    const int c = c0 + u * 512;
    if (c >= d) break;
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (sp[j] < 0) continue;   // dropped or absent slots add nothing
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(g[j], bf16_to_f32(v[j][u][q] & 0xffffu), acc[2 * q]);
        acc[2 * q + 1] = fmaf(g[j], bf16_to_f32(v[j][u][q] >> 16), acc[2 * q + 1]);
      }
    }
    for (int s = 0; s < a.S; ++s) {
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(so + ((int64_t)s * a.T + t) * d + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16_to_f32(w[q] & 0xffffu);
        acc[2 * q + 1] += bf16_to_f32(w[q] >> 16);
      }
    }
    u32x4_t o;
    o[0] = pack_bf16x2(acc[0], acc[1]);
    o[1] = pack_bf16x2(acc[2], acc[3]);
    o[2] = pack_bf16x2(acc[4], acc[5]);
    o[3] = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<u32x4_t*>(y + t * d + c) = o;
  }
}

// fp32: 4 columns per lane, 256 per wave.
__global__ __launch_bounds__(256) void combine_f32_kernel(CombineArgs a) {
  const int ncg = (a.d + 255) / 256;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t t = wid / ncg;
  if (t >= a.T) return;
  const int cg = (int)(wid - t * ncg);
  const int lane = threadIdx.x & 63, k = a.k, d = a.d;
  const int c = cg * 256 + lane * 4;
  if (c >= d) return;
  const float* eo = static_cast<const float*>(a.expert_out);
  const float* so = static_cast<const float*>(a.shared_out);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j >= k) break;
    const int sp = a.slot_pos[t * k + j];
    if (sp < 0) continue;
    const float g = a.gate[t * k + j];
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(eo + (int64_t)sp * d + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = fmaf(g, v[q], acc[q]);
  }
  for (int s = 0; s < a.S; ++s) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(so + ((int64_t)s * a.T + t) * d + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] += v[q];
  }
  *reinterpret_cast<f32x4_t*>(static_cast<float*>(a.y) + t * d + c) = acc;
}

}  // namespace

namespace {
constexpr int cb_nc(int kmax) {
  return CB_LOADS / kmax < 1 ? 1 : (CB_LOADS / kmax > 4 ? 4 : CB_LOADS / kmax);
}
template <int KMAX>
void launch_combine_bf16(const CombineArgs& a, hipStream_t s) {
  constexpr int NC = cb_nc(KMAX);
  const int64_t ncg = (a.d + 512 * NC - 1) / (512 * NC);
  combine_bf16_kernel<KMAX, NC><<<(unsigned)((a.T * ncg + 3) / 4), 256, 0, s>>>(a);
}
}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int64_t prof_rec = prof_before("combine", s);
  if (a.dtype == MOE_BF16) {
    if (a.k <= 2) launch_combine_bf16<2>(a, s);
    else if (a.k <= 4) launch_combine_bf16<4>(a, s);
    else if (a.k <= 8) launch_combine_bf16<8>(a, s);
    else launch_combine_bf16<16>(a, s);
  } else {
    const int64_t ncg = (a.d + 255) / 256;
    combine_f32_kernel<<<(unsigned)((a.T * ncg + 3) / 4), 256, 0, s>>>(a);
  }
  prof_after(prof_rec, s);
  return hipGetLastError();
}

}  // namespace moe
