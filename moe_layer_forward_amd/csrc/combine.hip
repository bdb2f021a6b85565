// Weighted combine: "Kimi K2.5 模型架构深度拆解" §10.2 Steps 6-7 and "Kimi K2.5 架构 QA" Q8.3 add each
// routed expert's output, times its routing weight, into the token's row (index_add_) and add the
// shared expert's output.  Here every token gathers its K rows instead, so no atomics are needed and
// the result is bitwise reproducible:
//     y[t] = sum_k w[t,k] * y_rows[pair_row[t,k]]  (k ascending)  + y_shared[t],
// accumulated in fp32 and rounded once.  One thread per (token, 8 columns), 16-byte loads.
#include "kernels.h"

namespace moe {
namespace {

template <bool ROWS_BF16>
__device__ __forceinline__ void load8(const void* base, int64_t idx, float (&v)[8]) {
  if (ROWS_BF16) {
    const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <bool ROWS_BF16, bool Y_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y_rows,
                                                      const int32_t* __restrict__ pair_row,
                                                      const float* __restrict__ weights,
                                                      const void* __restrict__ y_shared, void* __restrict__ y,
                                                      int64_t T, int K, int H) {
  // one thread per (token, 8 columns); the row loads of up to 8 k (and the shared row) are issued
  // before any of them is added, and the sum keeps k order, then adds the shared row
  const int cpr = H / 8;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * cpr) return;
  const int64_t t = i / cpr;
  const int c = (int)(i % cpr) * 8;
  const int32_t* pr = pair_row + t * K;
  const float* wt = weights + t * K;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float sh[8];
  if (y_shared) load8<ROWS_BF16>(y_shared, t * H + c, sh);
  int k = 0;
  for (; k + 8 <= K; k += 8) {
    float v[8][8], w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      w[u] = wt[k + u];
      load8<ROWS_BF16>(y_rows, (int64_t)pr[k + u] * H + c, v[u]);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(w[u], v[u][e], acc[e]);
  }
  for (; k + 4 <= K; k += 4) {
    float v[4][8], w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      w[u] = wt[k + u];
      load8<ROWS_BF16>(y_rows, (int64_t)pr[k + u] * H + c, v[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(w[u], v[u][e], acc[e]);
  }
  for (; k < K; ++k) {
    float v[8];
    const float w = wt[k];
    load8<ROWS_BF16>(y_rows, (int64_t)pr[k] * H + c, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, v[e], acc[e]);
  }
  if (y_shared) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += sh[e];
  }
  if (Y_BF16) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)f32_to_bf16(acc[2 * e]) | ((uint32_t)f32_to_bf16(acc[2 * e + 1]) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + t * H + c) = uint4{w[0], w[1], w[2], w[3]};
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(y) + t * H + c);
    p[0] = float4{acc[0], acc[1], acc[2], acc[3]};
    p[1] = float4{acc[4], acc[5], acc[6], acc[7]};
  }
}

}  // namespace

hipError_t launch_combine(const void* y_rows, bool rows_bf16, const int32_t* pair_row, const float* weights,
                          const void* y_shared, void* y, bool y_bf16, int64_t T, int K, int H, hipStream_t s) {
  const int64_t threads = T * (H / 8);
  const unsigned grid = (unsigned)((threads + 255) / 256);
  if (rows_bf16 && y_bf16)
    combine_kernel<true, true><<<grid, 256, 0, s>>>(y_rows, pair_row, weights, y_shared, y, T, K, H);
  else if (rows_bf16)
    combine_kernel<true, false><<<grid, 256, 0, s>>>(y_rows, pair_row, weights, y_shared, y, T, K, H);
  else if (y_bf16)
    combine_kernel<false, true><<<grid, 256, 0, s>>>(y_rows, pair_row, weights, y_shared, y, T, K, H);
  else
    combine_kernel<false, false><<<grid, 256, 0, s>>>(y_rows, pair_row, weights, y_shared, y, T, K, H);
  return hipGetLastError();
}

}  // namespace moe
