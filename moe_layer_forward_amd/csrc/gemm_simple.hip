// Grouped SwiGLU experts in fp32 (plain kernels for fp32 layers; one wave per output element: the
// lanes split the dot product, then a fixed-order butterfly adds the 64 partial sums).
// Same computation as the bf16 kernels ("Kimi K2.5 模型架构深度拆解" §4.3 / §10.2 Steps 5-6) without
// MFMA: h = SiLU(a Wg^T) * (a Wu^T) in fp32, then y = h Wd^T.
#include "kernels.h"

namespace moe {
namespace {

struct SimpleArgs {
  int32_t n_groups;
  const int32_t* group_offsets;
  int64_t max_rows;
  const int32_t* row_index;
  Weights w;
  const float* a;
  float* out;
  const float* row_scale;
  int H, I;
};

// Group of row r: the g with off[g] <= r < off[g+1] (offsets clamped to max_rows), or -1.
__device__ int find_group(const int32_t* off, int G, int64_t max_rows, int64_t r) {
  int64_t end = off[G] < max_rows ? off[G] : max_rows;
  if (r >= end) return -1;
  int lo = 0, hi = G;  // invariant: off[lo] <= r < off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= r)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

// Sum over the wave's 64 lanes, the same order on every call; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__global__ __launch_bounds__(256) void gateup_f32_kernel(SimpleArgs p) {
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // this wave's output element
  const int lane = threadIdx.x & 63;
  if (i >= p.max_rows * p.I) return;
  const int64_t r = i / p.I;
  const int n = (int)(i - r * p.I);
  const int g = find_group(p.group_offsets, p.n_groups, p.max_rows, r);
  if (g < 0) return;
  const bool sh = g == p.w.shared_group;
  const float* wg = (sh ? (const float*)p.w.s_gate : (const float*)p.w.gate + (int64_t)g * p.I * p.H) + (int64_t)n * p.H;
  const float* wu = (sh ? (const float*)p.w.s_up : (const float*)p.w.up + (int64_t)g * p.I * p.H) + (int64_t)n * p.H;
  const float* a = p.a + (p.row_index ? (int64_t)p.row_index[r] : r) * p.H;
  float gs = 0.f, us = 0.f;
  for (int k = lane; k < p.H; k += 64) {
    gs = fmaf(a[k], wg[k], gs);
    us = fmaf(a[k], wu[k], us);
  }
  gs = wave_sum(gs);
  us = wave_sum(us);
  if (lane == 0) p.out[r * p.I + n] = swiglu_f32(gs, us);
}

__global__ __launch_bounds__(256) void down_f32_kernel(SimpleArgs p) {
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= p.max_rows * p.H) return;
  const int64_t r = i / p.H;
  const int n = (int)(i - r * p.H);
  const int g = find_group(p.group_offsets, p.n_groups, p.max_rows, r);
  if (g < 0) return;
  const bool sh = g == p.w.shared_group;
  const float* wd = (sh ? (const float*)p.w.s_down : (const float*)p.w.down + (int64_t)g * p.H * p.I) + (int64_t)n * p.I;
  const float* h = p.a + r * p.I;
  float acc = 0.f;
  for (int k = lane; k < p.I; k += 64) acc = fmaf(h[k], wd[k], acc);
  acc = wave_sum(acc);
  if (lane == 0) p.out[r * p.H + n] = acc * (p.row_scale ? p.row_scale[r] : 1.f);
}

}  // namespace

hipError_t launch_gateup_f32(const Groups& g, const Weights& w, const float* x, float* h, int H, int I,
                             hipStream_t s) {
  SimpleArgs p{g.n_groups, g.group_offsets, g.max_rows, g.row_index, w, x, h, nullptr, H, I};
  const int64_t n = g.max_rows * I;  // one wave per output, 4 per work-group
  gateup_f32_kernel<<<(unsigned)((n + 3) / 4), 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_down_f32(const Groups& g, const Weights& w, const float* h, float* y_rows, const float* row_scale,
                           int H, int I, hipStream_t s) {
  SimpleArgs p{g.n_groups, g.group_offsets, g.max_rows, nullptr, w, h, y_rows, row_scale, H, I};
  const int64_t n = g.max_rows * H;
  down_f32_kernel<<<(unsigned)((n + 3) / 4), 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
