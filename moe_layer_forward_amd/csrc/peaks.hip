// Measured machine peaks that the benchmark reports beside the published ones: a streaming HBM
// read, a streaming copy, and a loop of independent bf16 MFMAs.  Measurement support only; the
// layer does not use this library.
//
//   peaks_read : every wave streams its own contiguous span with gfx950's direct global -> LDS loads
//                (global_load_lds_dwordx4, non-temporal: 1 KiB of whole cache lines per instruction,
//                the load form of the layer's weight-stream kernels), kInFlight loads in flight
//   peaks_read_vgpr : the same span reads into registers (16 bytes per lane, 8 loads in flight)
//   peaks_copy : the same, storing each chunk to dst
//   peaks_mfma : each wave runs `iters` rounds of 4 independent v_mfma_f32_32x32x16_bf16
//                (32,768 FLOP each); 4 waves per work-group
// Results are folded into a sink that is written only on an impossible value, so nothing is
// optimised away.  Every entry point returns a hipError_t (0 = success).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// A work-group reads 8 x 256 consecutive chunks (32 KiB) per round, 8 loads in flight per thread.
constexpr int kUnroll = 8;

__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, int64_t n, uint32_t* sink) {
  uint32_t acc = 0;
  const int64_t round = (int64_t)gridDim.x * 256 * kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * 256 * kUnroll + threadIdx.x; base < n; base += round) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t i = base + (int64_t)j * 256;
      v[j] = i < n ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) acc ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
  if (acc == 0x9e3779b9u) sink[threadIdx.x] = acc;
}

// Direct-to-LDS streaming read: the buffer is n_pieces pieces of 1 KiB; wave w of the W waves of the
// grid reads pieces w, w + W, w + 2W, ... (so the waves in flight together cover neighbouring
// pieces, spread over the HBM channels) into a private 8 KiB LDS ring it never reads back (the loads
// are the measurement).  An explicit wait every kInFlight/2 loads bounds the loads in flight; the
// wave drains before it exits.
constexpr int kInFlight = 16;

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

__global__ __launch_bounds__(256) void read_lds_kernel(const char* __restrict__ src, int64_t n_pieces) {
  __shared__ __align__(16) char ring[4][8 * 1024];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t W = (int64_t)gridDim.x * 4, gw = (int64_t)blockIdx.x * 4 + wave;
  const int64_t n = gw < n_pieces ? (n_pieces - gw + W - 1) / W : 0;  // pieces of this wave
  const char* p = src + gw * 1024 + lane * 16;
  char* dst = ring[wave];
  int64_t i = 0;
  for (; i + kInFlight / 2 <= n; i += kInFlight / 2) {
#pragma unroll
    for (int j = 0; j < kInFlight / 2; ++j)
      __builtin_amdgcn_global_load_lds(p + (i + j) * W * 1024, dst + j * 1024, 16, 0, 2);
    wait_vm<kInFlight / 2>();
  }
  for (; i < n; ++i) __builtin_amdgcn_global_load_lds(p + i * W * 1024, dst, 16, 0, 2);
  wait_vm<0>();
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(float)((lane + j) & 7);
    b[j] = (__bf16)(float)((lane * 3 + j) & 7);
  }
  f32x16 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    acc[c] = f32x16{};
    acc[c][0] = (float)(c + lane);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  if (s == -1.2345f) sink[threadIdx.x] = s;
}

unsigned stream_grid(int64_t chunks, int per_thread) {
  int64_t g = (chunks + 256 * per_thread - 1) / (256 * per_thread);
  const int64_t cap = 256 * 8;  // 8 work-groups per CU, each looping
  return (unsigned)(g < cap ? (g > 0 ? g : 1) : cap);
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 1 KiB) from src with direct-to-LDS loads: `blocks` work-groups of 4
// waves.
int peaks_read(const void* src, int64_t bytes, int32_t blocks, void* stream) {
  if (!src || blocks <= 0 || bytes <= 0 || bytes % 1024) return (int)hipErrorInvalidValue;
  read_lds_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const char*>(src),
                                                                         bytes / 1024);
  return (int)hipGetLastError();
}

// Reads `bytes` (a multiple of 16) from src into registers.  sink: 256 uint32 of device scratch.
int peaks_read_vgpr(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16) return (int)hipErrorInvalidValue;
  const int64_t n = bytes / 16;
  read_kernel<<<stream_grid(n, kUnroll), 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const u32x4*>(src), n, sink);
  return (int)hipGetLastError();
}

// Copies `bytes` (a multiple of 16) from src to dst (the two must not overlap).
int peaks_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (!src || !dst || bytes <= 0 || bytes % 16) return (int)hipErrorInvalidValue;
  const int64_t n = bytes / 16;
  copy_kernel<<<stream_grid(n, 1), 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const u32x4*>(src),
                                                                            static_cast<u32x4*>(dst), n);
  return (int)hipGetLastError();
}

// `blocks` work-groups of 4 waves, each wave 4 * iters MFMAs of 32,768 FLOP.  sink: 256 floats.
int peaks_mfma(int32_t blocks, int32_t iters, float* sink, void* stream) {
  if (!sink || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  mfma_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
