// LDS-tiled bf16 MFMA main loop shared by the tile GEMMs (router logits, grouped gate/up, grouped down).
//
// C[BM, BN] (fp32) = A[BM, K] . B[BN, K]^T with both operands K-contiguous ("NT"), as the nn.Linear
// [out, in] weights and the token rows are.  256 threads = 4 waves in a 2 x 2 grid, each wave owning a
// (BM/2) x (BN/2) block of v_mfma_f32_16x16x32_bf16 tiles.  Global -> registers -> LDS staging with
// two LDS buffers: the loads of step k+1 are in flight while step k's MFMAs run, one barrier a step.
// Operand rows are handed in as per-thread pointers plus a validity mask, so the gather of token rows
// and the choice of expert happen in the caller, not here.
#pragma once
#include "kernels.h"

namespace moe {

template <int BM_, int BN_, int BK_>
struct TileShape {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int kThreads = 256;
  static constexpr int kLd = BK + 8;               // LDS row pitch in bf16: +16 B breaks bank aliasing
  static constexpr int kChunksPerRow = BK / 8;     // 16-byte chunks per operand row and step
  static constexpr int kALoads = BM * kChunksPerRow / kThreads;
  static constexpr int kBLoads = BN * kChunksPerRow / kThreads;
  static constexpr int kStageElems = (BM + BN) * kLd;
  static constexpr int kSmemBytes = 2 * kStageElems * 2;
  static constexpr int kWaveM = BM / 2, kWaveN = BN / 2;
  static constexpr int kMI = kWaveM / 16, kNI = kWaveN / 16;
  static_assert(BM * kChunksPerRow % kThreads == 0 && BN * kChunksPerRow % kThreads == 0, "staging");
  static_assert(BK % 32 == 0, "BK");

  // Row and column (bf16 elements) of the j-th 16-byte chunk this thread stages.
  __device__ static __forceinline__ int stage_row(int tid, int j) { return (tid + j * kThreads) / kChunksPerRow; }
  __device__ static __forceinline__ int stage_col(int tid, int j) {
    return ((tid + j * kThreads) % kChunksPerRow) * 8;
  }
};

// acc[mi][ni] holds, in lane l, C[wm*kWaveM + mi*16 + 4*(l/16) + i][wn*kWaveN + ni*16 + l%16], i = 0..3.
// aptr[j] / bptr[j]: start (row, stage_col) of the j-th staged chunk's row at k = 0, or null.
template <class S>
__device__ __forceinline__ void tile_gload(const uint16_t* const (&aptr)[S::kALoads],
                                           const uint16_t* const (&bptr)[S::kBLoads], uint32_t amask, uint32_t bmask,
                                           int kt, uint4 (&ra)[S::kALoads], uint4 (&rb)[S::kBLoads]) {
#pragma unroll
  for (int j = 0; j < S::kALoads; ++j) {
    const uint4 v = *reinterpret_cast<const uint4*>(aptr[j] + (int64_t)kt * S::BK);
    const uint32_t keep = (amask >> j) & 1u ? 0xffffffffu : 0u;
    ra[j] = uint4{v.x & keep, v.y & keep, v.z & keep, v.w & keep};
  }
#pragma unroll
  for (int j = 0; j < S::kBLoads; ++j) {
    const uint4 v = *reinterpret_cast<const uint4*>(bptr[j] + (int64_t)kt * S::BK);
    const uint32_t keep = (bmask >> j) & 1u ? 0xffffffffu : 0u;
    rb[j] = uint4{v.x & keep, v.y & keep, v.z & keep, v.w & keep};
  }
}

template <class S>
__device__ __forceinline__ void tile_sstore(uint16_t* stage, const uint4 (&ra)[S::kALoads],
                                            const uint4 (&rb)[S::kBLoads]) {
  const int tid = threadIdx.x;
  uint16_t* Bs = stage + S::BM * S::kLd;
#pragma unroll
  for (int j = 0; j < S::kALoads; ++j)
    *reinterpret_cast<uint4*>(stage + S::stage_row(tid, j) * S::kLd + S::stage_col(tid, j)) = ra[j];
#pragma unroll
  for (int j = 0; j < S::kBLoads; ++j)
    *reinterpret_cast<uint4*>(Bs + S::stage_row(tid, j) * S::kLd + S::stage_col(tid, j)) = rb[j];
}

template <class S>
__device__ __forceinline__ void tile_compute(const uint16_t* stage, f32x4 (&acc)[S::kMI][S::kNI]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  const uint16_t* Bs = stage + S::BM * S::kLd;
#pragma unroll
  for (int ks = 0; ks < S::BK / 32; ++ks) {
    bf16x8 a[S::kMI], b[S::kNI];
#pragma unroll
    for (int mi = 0; mi < S::kMI; ++mi)
      a[mi] = *reinterpret_cast<const bf16x8*>(stage + (wm * S::kWaveM + mi * 16 + (lane & 15)) * S::kLd + ks * 32 +
                                               (lane >> 4) * 8);
#pragma unroll
    for (int ni = 0; ni < S::kNI; ++ni)
      b[ni] = *reinterpret_cast<const bf16x8*>(Bs + (wn * S::kWaveN + ni * 16 + (lane & 15)) * S::kLd + ks * 32 +
                                               (lane >> 4) * 8);
#pragma unroll
    for (int mi = 0; mi < S::kMI; ++mi)
#pragma unroll
      for (int ni = 0; ni < S::kNI; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mi], b[ni], acc[mi][ni], 0, 0, 0);
  }
}

// acc[mi][ni] holds, in lane l, C[wm*kWaveM + mi*16 + 4*(l/16) + i][wn*kWaveN + ni*16 + l%16], i = 0..3.
// aptr[j] / bptr[j]: start (row, stage_col) of the j-th staged chunk's row at k = 0.  Every pointer
// must be readable; bit j of amask / bmask clear makes that chunk a zero row (rows past the end of a
// group point at a valid row and are masked, so the loads never branch).
template <class S>
__device__ __forceinline__ void tile_mainloop(const uint16_t* const (&aptr)[S::kALoads],
                                              const uint16_t* const (&bptr)[S::kBLoads], uint32_t amask,
                                              uint32_t bmask, int K, uint16_t* smem, f32x4 (&acc)[S::kMI][S::kNI]) {
  uint4 ra[S::kALoads], rb[S::kBLoads];
#pragma unroll
  for (int mi = 0; mi < S::kMI; ++mi)
#pragma unroll
    for (int ni = 0; ni < S::kNI; ++ni) acc[mi][ni] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / S::BK;
  tile_gload<S>(aptr, bptr, amask, bmask, 0, ra, rb);
  tile_sstore<S>(smem, ra, rb);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    uint16_t* cur = smem + (kt & 1) * S::kStageElems;
    uint16_t* nxt = smem + ((kt + 1) & 1) * S::kStageElems;
    if (kt + 1 < nk) tile_gload<S>(aptr, bptr, amask, bmask, kt + 1, ra, rb);
    tile_compute<S>(cur, acc);
    if (kt + 1 < nk) tile_sstore<S>(nxt, ra, rb);
    __syncthreads();
  }
}

// Work item L of n_work, dealt so that consecutive L run on the same XCD: the hardware hands
// blockIdx b to XCD b % 8, so XCD x takes the contiguous range [x*per, (x+1)*per).
// Returns false for padding work-groups.
__device__ __forceinline__ bool xcd_work_item(int64_t n_work, int64_t& L) {
  const int64_t b = blockIdx.x;
  const int64_t xcd = b % kXcds, local = b / kXcds;
  const int64_t per = (n_work + kXcds - 1) / kXcds;
  if (local >= per) return false;
  L = xcd * per + local;
  return L < n_work;
}

}  // namespace moe
