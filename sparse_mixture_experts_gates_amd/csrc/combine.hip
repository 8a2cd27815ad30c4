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

__global__ __launch_bounds__(256) void combine_bf16_kernel(CombineArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int lane = threadIdx.x & 63, k = a.k, d = a.d;
  int sp[16];
  float g[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j >= k) break;
    sp[j] = a.slot_pos[t * k + j];
    g[j] = a.gate[t * k + j];
  }
  const uint16_t* eo = static_cast<const uint16_t*>(a.expert_out);
  const uint16_t* so = static_cast<const uint16_t*>(a.shared_out);
  uint16_t* y = static_cast<uint16_t*>(a.y);
  for (int c = lane; c < d / 8; c += 64) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j >= k) break;
      if (sp[j] < 0) continue;
      const uint4 v = *reinterpret_cast<const uint4*>(eo + (int64_t)sp[j] * d + c * 8);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(g[j], bf16_to_f32(w[q] & 0xffffu), acc[2 * q]);
        acc[2 * q + 1] = fmaf(g[j], bf16_to_f32(w[q] >> 16), acc[2 * q + 1]);
      }
    }
    for (int s = 0; s < a.S; ++s) {
      const uint4 v = *reinterpret_cast<const uint4*>(so + ((int64_t)s * a.T + t) * d + c * 8);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16_to_f32(w[q] & 0xffffu);
        acc[2 * q + 1] += bf16_to_f32(w[q] >> 16);
      }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(y + t * d + c * 8) = o;
  }
}

__global__ __launch_bounds__(256) void combine_f32_kernel(CombineArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int lane = threadIdx.x & 63, k = a.k, d = a.d;
  int sp[16];
  float g[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j >= k) break;
    sp[j] = a.slot_pos[t * k + j];
    g[j] = a.gate[t * k + j];
  }
  const float* eo = static_cast<const float*>(a.expert_out);
  const float* so = static_cast<const float*>(a.shared_out);
  float* y = static_cast<float*>(a.y);
  for (int c = lane; c < d / 4; c += 64) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j >= k) break;
      if (sp[j] < 0) continue;
      const float4 v = *reinterpret_cast<const float4*>(eo + (int64_t)sp[j] * d + c * 4);
      acc.x = fmaf(g[j], v.x, acc.x);
      acc.y = fmaf(g[j], v.y, acc.y);
      acc.z = fmaf(g[j], v.z, acc.z);
      acc.w = fmaf(g[j], v.w, acc.w);
    }
    for (int s = 0; s < a.S; ++s) {
      const float4 v = *reinterpret_cast<const float4*>(so + ((int64_t)s * a.T + t) * d + c * 4);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    *reinterpret_cast<float4*>(y + t * d + c * 4) = acc;
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const unsigned grid = (unsigned)((a.T + 3) / 4);
  prof_before("combine", s);
  if (a.dtype == MOE_BF16)
    combine_bf16_kernel<<<grid, 256, 0, s>>>(a);
  else
    combine_f32_kernel<<<grid, 256, 0, s>>>(a);
  prof_after(s);
  return hipGetLastError();
}

}  // namespace moe
