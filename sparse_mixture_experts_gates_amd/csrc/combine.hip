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

// One wave per (token, 512-column group): every lane owns 8 columns (one
// 16-byte load per source row); the loads of all k rows are issued before
// the sums so that each wave waits for memory once.
constexpr int CB_COLS = 512;

template <int KMAX>
__global__ __launch_bounds__(256) void combine_bf16_kernel(CombineArgs a) {
  const int ncg = (a.d + CB_COLS - 1) / CB_COLS;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t t = wid / ncg;
  if (t >= a.T) return;
  const int cg = (int)(wid - t * ncg);
  const int lane = threadIdx.x & 63, k = a.k, d = a.d;
  const int c = cg * CB_COLS + lane * 8;
  if (c >= d) return;
  const uint16_t* eo = static_cast<const uint16_t*>(a.expert_out);
  const uint16_t* so = static_cast<const uint16_t*>(a.shared_out);
  u32x4_t v[KMAX];
  float g[KMAX];
  bool on[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int sp = j < k ? a.slot_pos[t * k + j] : -1;
    on[j] = sp >= 0;
    g[j] = on[j] ? a.gate[t * k + j] : 0.f;
    v[j] = on[j] ? *reinterpret_cast<const u32x4_t*>(eo + (int64_t)sp * d + c)
                 : u32x4_t{0u, 0u, 0u, 0u};
  }
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (!on[j]) continue;   // dropped or absent slots add nothing
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[2 * q] = fmaf(g[j], bf16_to_f32(v[j][q] & 0xffffu), acc[2 * q]);
      acc[2 * q + 1] = fmaf(g[j], bf16_to_f32(v[j][q] >> 16), acc[2 * q + 1]);
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
  uint16_t* y = static_cast<uint16_t*>(a.y);
  u32x4_t o;
  o[0] = pack_bf16x2(acc[0], acc[1]);
  o[1] = pack_bf16x2(acc[2], acc[3]);
  o[2] = pack_bf16x2(acc[4], acc[5]);
  o[3] = pack_bf16x2(acc[6], acc[7]);
  *reinterpret_cast<u32x4_t*>(y + t * d + c) = o;
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

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const int64_t ncg = a.dtype == MOE_BF16 ? (a.d + CB_COLS - 1) / CB_COLS : (a.d + 255) / 256;
  const unsigned grid = (unsigned)((a.T * ncg + 3) / 4);
  const int64_t prof_rec = prof_before("combine", s);
  if (a.dtype == MOE_BF16) {
    if (a.k <= 2) combine_bf16_kernel<2><<<grid, 256, 0, s>>>(a);
    else if (a.k <= 4) combine_bf16_kernel<4><<<grid, 256, 0, s>>>(a);
    else if (a.k <= 8) combine_bf16_kernel<8><<<grid, 256, 0, s>>>(a);
    else combine_bf16_kernel<16><<<grid, 256, 0, s>>>(a);
  }
  else
    combine_f32_kernel<<<grid, 256, 0, s>>>(a);
  prof_after(prof_rec, s);
  return hipGetLastError();
}

}  // namespace moe
