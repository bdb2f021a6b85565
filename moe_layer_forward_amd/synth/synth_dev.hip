// Seeded synthetic inputs for the MoE layer workloads, device side.
//
// Independent twin of synth_host.c: the same element definition, written
// again for the GPU so that multi-gigabyte weight stacks are produced in HBM
// in milliseconds while the host can regenerate any single expert, row or
// element bit-for-bit.  No arithmetic of the MoE layer lives here.
//
// Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11), ten rounds
// with multipliers 0xD2511F53 / 0xCD9E8D57 and key increments
// 0x9E3779B9 / 0xBB67AE85.  Element e of tensor (seed, stream, index):
//   counter = (e lo32, e hi32, index, 0), key = (seed, stream)
//   d = sum of the eight 16-bit halves of the four output words
//   value = fl32((float)(2*d - 524280) * scale), bf16 by round-to-nearest-even.
//
// 4-bit weight storage (synth_dev_quantize_q4), input preparation like an offline checkpoint
// conversion, the same fp32 operations as the host twin: per group of 32 consecutive inputs,
//   s = f16_rne(max|w| / 7), q = clamp(rint(w / s), -8, 7) (0 when s == 0),
// codes 8 per 32-bit word (input k at bits 4*(k % 8), two's complement), scales as f16 bits.
//
// 8-bit weight storage (synth_dev_quantize_fp8), the same fp32 operations as the host twin: per
// 128 x 128 block of a matrix, s = max|w| / 448, c = e4m3_rne(w / s) saturating at +-448 (0 when
// s == 0); codes one byte per weight (OCP E4M3), scales fp32 [rows/128, cols/128].
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ void philox_round(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3,
                                             uint32_t k0, uint32_t k1) {
  const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
  const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
  const uint32_t n1 = (uint32_t)p1;
  const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
  const uint32_t n3 = (uint32_t)p0;
  c0 = n0; c1 = n1; c2 = n2; c3 = n3;
}

__device__ __forceinline__ float element_value(uint32_t seed, uint32_t stream, uint32_t index,
                                               uint64_t e, float scale) {
  uint32_t c0 = (uint32_t)e, c1 = (uint32_t)(e >> 32), c2 = index, c3 = 0u;
  uint32_t k0 = seed, k1 = stream;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    philox_round(c0, c1, c2, c3, k0, k1);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  const int32_t d = (int32_t)((c0 & 0xffffu) + (c0 >> 16) + (c1 & 0xffffu) + (c1 >> 16) +
                              (c2 & 0xffffu) + (c2 >> 16) + (c3 & 0xffffu) + (c3 >> 16));
  const int32_t c = 2 * d - 524280;
  return __fmul_rn((float)c, scale);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// out is a stack of n_index tensors of per_index elements each, tensor j
// being (seed, stream, index0 + j).
template <bool BF16>
__global__ void synth_fill_kernel(void* __restrict__ out, uint32_t seed, uint32_t stream,
                                  uint32_t index0, int64_t per_index, int64_t total, float scale) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total; g += stride) {
    const int64_t j = g / per_index;
    const int64_t e = g - j * per_index;
    const float v = element_value(seed, stream, index0 + (uint32_t)j, (uint64_t)e, scale);
    if (BF16)
      static_cast<uint16_t*>(out)[g] = bf16_rne(v);
    else
      static_cast<float*>(out)[g] = v;
  }
}

// One group of 32 bf16 weights per thread; groups are consecutive in memory.
__global__ void synth_quantize_q4_kernel(const uint16_t* __restrict__ w, int64_t n_groups,
                                         uint32_t* __restrict__ codes, uint16_t* __restrict__ scales) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gi < n_groups; gi += stride) {
    float v[32], amax = 0.f;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      v[k] = __uint_as_float((uint32_t)w[gi * 32 + k] << 16);
      amax = fmaxf(amax, fabsf(v[k]));
    }
    const _Float16 s16 = (_Float16)__fdiv_rn(amax, 7.0f);
    const float s = (float)s16;
    scales[gi] = __builtin_bit_cast(uint16_t, s16);
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int q = 0;
        if (s > 0.f) {
          const float t = __builtin_rintf(__fdiv_rn(v[8 * wd + i], s));
          q = t > 7.f ? 7 : (t < -8.f ? -8 : (int)t);
        }
        word |= ((uint32_t)q & 0xfu) << (4 * i);
      }
      codes[gi * 4 + wd] = word;
    }
  }
}

// OCP E4M3 code of an fp32 value, round to nearest even, saturating at +-448 (as on the host).
__device__ __forceinline__ uint8_t f32_to_e4m3_rne(float t) {
  uint32_t u = __float_as_uint(t);
  const uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
  u &= 0x7fffffffu;
  const float a = __uint_as_float(u);
  if (!(a < 448.0f)) return sign | 0x7e;
  if (a < 0.015625f) return sign | (uint8_t)__builtin_rintf(a * 512.0f);
  int e = (int)(u >> 23) - 127;
  float q = __builtin_rintf(a * __uint_as_float((uint32_t)(127 + 3 - e) << 23));
  if (q == 16.0f) {
    q = 8.0f;
    ++e;
  }
  return sign | (uint8_t)(((e + 7) << 3) | ((int)q - 8));
}

// One 128 x 128 block per work-group of 256 threads: thread t covers row t/2, columns 64*(t%2) ..
// +63 of the block, read as 8 x 16 bytes and written as 4 x 16 bytes of codes.
__global__ __launch_bounds__(256) void synth_quantize_fp8_kernel(const uint16_t* __restrict__ w, int64_t rows,
                                                                 int64_t cols, uint8_t* __restrict__ codes,
                                                                 float* __restrict__ scales) {
  __shared__ float wmax[4];
  const int64_t br = rows / 128, bc = cols / 128, bi = blockIdx.x;
  const int64_t m = bi / (br * bc), r0 = (bi / bc) % br * 128, c0 = bi % bc * 128;
  const int64_t at = m * rows * cols + (r0 + threadIdx.x / 2) * cols + c0 + 64 * (threadIdx.x % 2);
  uint4 v[8];
  const uint4* src = reinterpret_cast<const uint4*>(w + at);
  for (int j = 0; j < 8; ++j) v[j] = src[j];
  const uint32_t* h = reinterpret_cast<const uint32_t*>(v);  // 32 words of 2 bf16 each
  float amax = 0.f;
  for (int i = 0; i < 32; ++i)
    amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(h[i] << 16)), fabsf(__uint_as_float(h[i] & 0xffff0000u))));
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s = __fdiv_rn(amax, 448.0f);
  if (threadIdx.x == 0) scales[bi] = s;
  uint4* dst = reinterpret_cast<uint4*>(codes + at);
  for (int j = 0; j < 4; ++j) {
    uint32_t out[4];
    for (int k = 0; k < 4; ++k) {
      uint32_t word = 0;
      for (int b = 0; b < 4; ++b) {
        const int e = 16 * j + 4 * k + b;  // element of the thread's 64
        const uint32_t bits = (e & 1) ? (h[e >> 1] & 0xffff0000u) : (h[e >> 1] << 16);
        const uint8_t c = s > 0.f ? f32_to_e4m3_rne(__fdiv_rn(__uint_as_float(bits), s)) : 0;
        word |= (uint32_t)c << (8 * b);
      }
      out[k] = word;
    }
    dst[j] = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

}  // namespace

extern "C" int synth_dev_quantize_q4(const void* w, int64_t n_groups, void* codes, void* scales,
                                     void* hip_stream) {
  if (!w || !codes || !scales || n_groups < 0) return 1;
  if (n_groups == 0) return 0;
  int64_t blocks = (n_groups + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  synth_quantize_q4_kernel<<<(unsigned)blocks, 256, 0, static_cast<hipStream_t>(hip_stream)>>>(
      static_cast<const uint16_t*>(w), n_groups, static_cast<uint32_t*>(codes), static_cast<uint16_t*>(scales));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int synth_dev_fill(void* out, int32_t is_bf16, uint32_t seed, uint32_t stream,
                              uint32_t index0, int64_t n_index, int64_t per_index, float scale,
                              void* hip_stream) {
  if (out == nullptr || n_index < 0 || per_index < 0) return 1;
  const int64_t total = n_index * per_index;
  if (total == 0) return 0;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (is_bf16)
    synth_fill_kernel<true><<<(unsigned)blocks, threads, 0, s>>>(out, seed, stream, index0, per_index,
                                                                 total, scale);
  else
    synth_fill_kernel<false><<<(unsigned)blocks, threads, 0, s>>>(out, seed, stream, index0, per_index,
                                                                  total, scale);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// n_mats matrices [rows, cols] of bf16 (rows, cols multiples of 128) -> codes [n_mats, rows, cols]
// bytes and scales [n_mats, rows/128, cols/128] fp32.  Returns 0, 1 (bad arguments) or 4 (launch).
extern "C" int synth_dev_quantize_fp8(const void* w, int64_t n_mats, int64_t rows, int64_t cols, void* codes,
                                      void* scales, void* hip_stream) {
  if (!w || !codes || !scales || n_mats < 0 || rows < 0 || cols < 0 || rows % 128 || cols % 128) return 1;
  const int64_t blocks = n_mats * (rows / 128) * (cols / 128);
  if (blocks == 0) return 0;
  if (blocks > 0x7fffffffLL) return 1;
  synth_quantize_fp8_kernel<<<(unsigned)blocks, 256, 0, static_cast<hipStream_t>(hip_stream)>>>(
      static_cast<const uint16_t*>(w), rows, cols, static_cast<uint8_t*>(codes), static_cast<float*>(scales));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
