// Router of the K2 MoE layer ("Kimi K2.5 模型架构深度拆解" §10.2 Steps 1-4, §4.2; no expert groups per
// the Zhihu K2-inference answer §2.4; scale 2.827 per the K2-pretraining answer and "Kimi K2.5 架构 QA"
// Q2.3).
//
//   logits  : x[T, H] . W_router[E, H]^T on bf16 MFMA with fp32 accumulation, split over K into S
//             partial sums [S, T, E] so that small T still spreads over the whole chip.
//   top-K   : one wave per token.  Each lane holds experts lane, lane+64, ... as 64-bit keys
//             (order-preserving fp32 bits of sigmoid(l)+bias in the high word, inverted id in the low
//             word, so a larger key wins and equal keys go to the smaller id).  K rounds of a
//             register-only wave max (xor butterfly) pick the winners; the winning lane retires its
//             entry.  Weights = rsf * s / sum(s) over the winners, with the unbiased scores s.
#include "tile_core.h"

namespace moe {
namespace {

using RS = TileShape<128, 128, 64, 2>;

// Number of K splits for the router GEMM: enough work-groups to cover the chip, partial sums no
// larger than the router weight itself, and each split a whole number of 64-wide K steps.
int router_splits(int64_t T, int H, int E) {
  const int64_t tiles = ((T + RS::BM - 1) / RS::BM) * ((E + RS::BN - 1) / RS::BN);
  const int ksteps = H / RS::BK;
  // partials [S, T, E] fp32: no more than the router weight or two copies of the logits
  const int64_t cap = H / (2 * T) > 2 ? H / (2 * T) : 2;
  int best = 1;
  for (int s = 1; s <= ksteps; ++s) {
    if (ksteps % s) continue;
    if (s > cap || H / s < 256) break;
    best = s;
    if (tiles * s >= 256) break;
  }
  return best;
}

__global__ __launch_bounds__(512) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wr, float* __restrict__ part,
                                                            int64_t T, int H, int E, int ksplit) {
  __shared__ __align__(16) char smem[RS::kSmemBytes];
  const int tid = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.x * RS::BM;
  const int n0 = blockIdx.y * RS::BN;
  const int split = blockIdx.z;
  const int k0 = split * ksplit;
  Operands<RS> o;
  const int w = tid >> 6, lane = tid & 63;
  o.a_base = reinterpret_cast<const char*>(x + k0);
  o.b_base = reinterpret_cast<const char*>(wr + k0);
#pragma unroll
  for (int j = 0; j < RS::kALoads; ++j) {
    const int rl = RS::load_row(w, j, lane, RS::kALoads);
    const int64_t t = m0 + rl;
    o.a_off[j] = (uint32_t)(((t < T ? t : 0) * H + 8 * RS::load_chunk(rl, lane)) * 2);
  }
#pragma unroll
  for (int j = 0; j < RS::kBLoads; ++j) {
    const int rl = RS::load_row(w, j, lane, RS::kBLoads);
    const int e = n0 + rl;  // experts past E read row 0, never stored
    o.b_off[j] = (uint32_t)(((int64_t)(e < E ? e : 0) * H + 8 * RS::load_chunk(rl, lane)) * 2);
  }
  f32x16 acc[RS::kMSub][RS::kNSub];
  tile_mainloop<RS>(o, T - m0 < RS::BM ? (int)(T - m0) : RS::BM, ksplit, smem, acc);

  const int wm = w >> 2, wn = w & 3;
  float* out = part + (int64_t)split * T * E;
#pragma unroll
  for (int i = 0; i < RS::kMSub; ++i)
#pragma unroll
    for (int u = 0; u < RS::kNSub; ++u) {
      const int e = n0 + wn * RS::kWaveN + 32 * u + (lane & 31);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t t = m0 + RS::sub_row(wm, i) + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        if (t < T && e < E) out[t * E + e] = acc[i][u][q];
      }
    }
}

// One wave per logit: the lanes split the dot product, a fixed-order butterfly adds the partial sums.
__global__ __launch_bounds__(256) void router_logits_f32_kernel(const float* __restrict__ x,
                                                                const float* __restrict__ w,
                                                                float* __restrict__ logits, int64_t T, int H,
                                                                int E) {
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= T * E) return;
  const int64_t t = i / E;
  const int e = (int)(i - t * E);
  const float* xr = x + t * H;
  const float* wr = w + (int64_t)e * H;
  float acc = 0.f;
  for (int k = lane; k < H; k += 64) acc = fmaf(xr[k], wr[k], acc);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (lane == 0) logits[i] = acc;
}

__device__ __forceinline__ uint32_t order_bits(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;  // -0 sorts with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// J = experts per lane (E <= 64 * J <= 512).
template <int J>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ part, int nsplit,
                                                   const float* __restrict__ logit_offset,
                                                   const float* __restrict__ score_bias, int64_t T, int E, int K,
                                                   float rsf, int32_t* __restrict__ ids,
                                                   float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave leaves together

  // logits: the K-split partial sums added in split order (4 splits' loads in flight per round)
  float lg[J];
#pragma unroll
  for (int j = 0; j < J; ++j) lg[j] = 0.f;
  const float* pt = part + t * E;
  const int64_t sstride = T * E;
  int sp = 0;
  for (; sp + 4 <= nsplit; sp += 4) {
    float v[4][J];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int e = lane + 64 * j;
        v[u][j] = e < E ? pt[(sp + u) * sstride + e] : 0.f;
      }
#pragma unroll
    for (int j = 0; j < J; ++j) lg[j] = (((lg[j] + v[0][j]) + v[1][j]) + v[2][j]) + v[3][j];
  }
  for (; sp < nsplit; ++sp)
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = lane + 64 * j;
      if (e < E) lg[j] += pt[sp * sstride + e];
    }

  uint64_t key[J];
  float sc[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + 64 * j;
    key[j] = 0;
    sc[j] = 0.f;
    if (e < E) {
      float l = lg[j];
      if (logit_offset) l += logit_offset[e];
      const float score = sigmoid_f32(l);
      const float kv = score_bias ? score + score_bias[e] : score;
      sc[j] = score;
      key[j] = ((uint64_t)order_bits(kv) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
    }
  }

  int my_e = 0;
  float my_s = 0.f;
#pragma unroll 1
  for (int k = 0; k < K; ++k) {
    uint64_t best = 0;
    float best_s = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (key[j] > best) {
        best = key[j];
        best_s = sc[j];
      }
    const uint64_t wmax = wave_max_u64(best);
    const bool win = best == wmax;  // keys are distinct (they carry the id), so one lane wins
    const uint64_t wins = __ballot(win);
    const int wl = __ffsll((unsigned long long)wins) - 1;
    const float s_k = __shfl(best_s, wl, 64);
    if (win) {
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (key[j] == wmax) key[j] = 0;
    }
    if (lane == k) {
      my_e = (int)(0xffffffffu - (uint32_t)(wmax & 0xffffffffu));
      my_s = s_k;
    }
  }
  const float sum = wave_sum_f32(lane < K ? my_s : 0.f);
  if (lane < K) {
    ids[t * K + lane] = my_e;
    weights[t * K + lane] = my_s / sum * rsf;
  }
}

}  // namespace

int router_nsplit(int64_t T, int H, int E, bool bf16) { return bf16 ? router_splits(T, H, E) : 1; }

hipError_t launch_router_logits_bf16(const uint16_t* x, const uint16_t* w_router, float* part, int64_t T, int H,
                                     int E, hipStream_t s) {
  const int S = router_splits(T, H, E);
  dim3 grid((unsigned)((T + RS::BM - 1) / RS::BM), (unsigned)((E + RS::BN - 1) / RS::BN), (unsigned)S);
  router_logits_kernel<<<grid, RS::kThreads, 0, s>>>(x, w_router, part, T, H, E, H / S);
  return hipGetLastError();
}

hipError_t launch_router_logits_f32(const float* x, const float* w_router, float* logits, int64_t T, int H, int E,
                                    hipStream_t s) {
  const int64_t n = T * E;  // one wave per logit, 4 per work-group
  router_logits_f32_kernel<<<(unsigned)((n + 3) / 4), 256, 0, s>>>(x, w_router, logits, T, H, E);
  return hipGetLastError();
}

hipError_t launch_topk(const float* part, int nsplit, const float* logit_offset, const float* score_bias, int64_t T,
                       int E, int K, float rsf, int32_t* ids, float* weights, hipStream_t s) {
  const unsigned grid = (unsigned)((T + 3) / 4);
  const int need = (E + 63) / 64;
  if (need <= 1)
    topk_kernel<1><<<grid, 256, 0, s>>>(part, nsplit, logit_offset, score_bias, T, E, K, rsf, ids, weights);
  else if (need <= 2)
    topk_kernel<2><<<grid, 256, 0, s>>>(part, nsplit, logit_offset, score_bias, T, E, K, rsf, ids, weights);
  else if (need <= 4)
    topk_kernel<4><<<grid, 256, 0, s>>>(part, nsplit, logit_offset, score_bias, T, E, K, rsf, ids, weights);
  else if (need <= 6)
    topk_kernel<6><<<grid, 256, 0, s>>>(part, nsplit, logit_offset, score_bias, T, E, K, rsf, ids, weights);
  else
    topk_kernel<8><<<grid, 256, 0, s>>>(part, nsplit, logit_offset, score_bias, T, E, K, rsf, ids, weights);
  return hipGetLastError();
}

}  // namespace moe
