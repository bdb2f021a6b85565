// LDS-tiled bf16 MFMA main loop shared by the tile GEMMs (router logits, grouped gate/up, grouped down).
//
// C[BM, BN] (fp32) = A[BM, K] . B[BN, K]^T with both operands K-contiguous ("NT"), as the nn.Linear
// [out, in] weights and the token rows are.  512 threads = 8 waves in a 2 (M) x 4 (N) grid; a wave
// owns BN/4 columns and BM/2 rows, the rows as 32-row sub-tiles dealt alternately to the two wave
// rows (sub-tile s goes to wave row s % 2).  v_mfma_f32_32x32x16_bf16 throughout.
//
// Operand staging uses gfx950's direct global -> LDS loads (global_load_lds_dwordx4): each load
// instruction moves 64 lanes x 16 bytes straight into 1 KiB of LDS, lane-contiguous, with no
// register round trip.  The LDS holds a ring of STAGES K-steps; the loads of steps k+1 .. k+STAGES-1
// are in flight while step k's MFMAs run, and one barrier per step both publishes step k and
// frees the slot step k+STAGES-1 is loaded into.
//
// LDS rows are BK*2 bytes, unpadded; the 16-byte chunk c of row r sits at position c ^ swz(r), which
// puts the 16 rows read by one 16-lane group of a fragment load in 16 different bank groups.  A
// load lane picks the global chunk that belongs in its LDS slot, so every load still reads whole
// contiguous row segments.
#pragma once
#include <type_traits>

#include "kernels.h"

namespace moe {

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int BM_, int BN_, int BK_, int STAGES_>
struct TileShape {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_;
  static constexpr int kThreads = 512, kWaves = 8;
  static constexpr int kRowBytes = BK * 2;
  static constexpr int kCpr = BK / 8;                      // 16-byte chunks per row
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;    // rows one wave-wide load fills
  static constexpr int kALoads = BM / kRowsPerLoad / kWaves;  // per wave per step
  static constexpr int kBLoads = BN / kRowsPerLoad / kWaves;
  static constexpr int kLoads = kALoads + kBLoads;
  static constexpr int kStageBytes = (BM + BN) * kRowBytes;
  static constexpr int kSmemBytes = STAGES * kStageBytes;
  static constexpr int kMSub = BM / 64;          // 32-row sub-tiles per wave row
  static constexpr int kNSub = BN / 128;         // 32-column sub-tiles per wave
  static constexpr int kWaveN = BN / 4;
  static_assert(BM % 64 == 0 && BN % 128 == 0 && (BK == 32 || BK == 64), "shape");
  static_assert(kALoads >= 1 && kBLoads >= 1 && BM % (kRowsPerLoad * kWaves) == 0 &&
                    BN % (kRowsPerLoad * kWaves) == 0, "staging");
  static_assert(kSmemBytes <= 160 * 1024, "LDS");
  static_assert(kLoads * (STAGES - 2) <= 63, "vmcnt");

  __device__ static __forceinline__ int swz(int r) { return (r / (16 / kCpr)) % kCpr; }
  // Operand row of lane `lane` in the j-th A (or B) load of wave w (nloads loads per wave).
  __device__ static __forceinline__ int load_row(int w, int j, int lane, int nloads) {
    return (w * nloads + j) * kRowsPerLoad + lane / kCpr;
  }
  // Logical chunk (k offset in units of 8 elements) that lane's LDS slot must receive.
  __device__ static __forceinline__ int load_chunk(int row, int lane) { return (lane % kCpr) ^ swz(row); }
  // First row of the i-th sub-tile of wave row wm.
  __device__ static __forceinline__ int sub_row(int wm, int i) { return (2 * i + wm) * 32; }
};

// Compile-time loop: f(integral_constant<int, I>) for I = 0 .. N-1.
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(const F& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Work-group barrier that waits only for this wave's LDS traffic, not for its global loads in flight
// (a full __syncthreads() also drains the vector-memory counter, which would stall the prefetch).
__device__ __forceinline__ void block_sync_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// Per-lane operand addresses: a uniform base plus a 32-bit byte offset per load (the operand
// matrices stay under 4 GiB); the offset already includes the lane's chunk.
template <class S>
struct Operands {
  const char* a_base;
  const char* b_base;
  uint32_t a_off[S::kALoads];
  uint32_t b_off[S::kBLoads];
};

// Issue the direct-to-LDS loads of K step kt into ring slot `stage`.  Weights are streamed with the
// non-temporal cache policy (read once); token rows with the default one (shared across tiles).
template <class S>
__device__ __forceinline__ void tile_issue(const Operands<S>& o, int kt, char* stage) {
  const int w = threadIdx.x >> 6;
  const uint32_t kb = (uint32_t)kt * S::kRowBytes;
#pragma unroll
  for (int j = 0; j < S::kALoads; ++j)
    __builtin_amdgcn_global_load_lds(o.a_base + (o.a_off[j] + kb), stage + (w * S::kALoads + j) * 1024, 16, 0, 0);
  char* bst = stage + S::BM * S::kRowBytes;
#pragma unroll
  for (int j = 0; j < S::kBLoads; ++j)
    __builtin_amdgcn_global_load_lds(o.b_base + (o.b_off[j] + kb), bst + (w * S::kBLoads + j) * 1024, 16, 0, 2);
}

// Wait for the loads of the step computed next, allowing `ahead` later steps to stay in flight.
template <class S>
__device__ __forceinline__ void tile_wait(int ahead) {
  static_assert(S::STAGES <= 5, "tile_wait cases");
  switch (ahead) {
    case 3: wait_vmcnt<3 * S::kLoads>(); break;
    case 2: wait_vmcnt<2 * S::kLoads>(); break;
    case 1: wait_vmcnt<1 * S::kLoads>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

// One K step of MFMAs from a ring slot over the first NS sub-tiles of this wave's rows (rows past
// the group end cost no MFMA).
// acc[i][t]: sub-tile i of this wave's rows x sub-tile t of its columns.  Lane l, register q holds
// C[sub_row(wm, i) + 8*(q/4) + 4*(l/32) + q%4][wn*kWaveN + 32*t + l%32].
template <class S, int NS>
__device__ __forceinline__ void tile_compute(const char* stage, f32x16 (&acc)[S::kMSub][S::kNSub]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 2, wn = wave & 3;
  const char* Bs = stage + S::BM * S::kRowBytes;
#pragma unroll
  for (int kk = 0; kk < S::BK / 16; ++kk) {
    const int c = kk * 2 + (lane >> 5);  // logical chunk of this lane's 8 k values
    bf16x8 b[S::kNSub];
#pragma unroll
    for (int t = 0; t < S::kNSub; ++t) {
      const int r = wn * S::kWaveN + 32 * t + (lane & 31);
      b[t] = *reinterpret_cast<const bf16x8*>(Bs + r * S::kRowBytes + ((c ^ S::swz(r)) << 4));
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int r = S::sub_row(wm, i) + (lane & 31);
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(stage + r * S::kRowBytes + ((c ^ S::swz(r)) << 4));
#pragma unroll
      for (int t = 0; t < S::kNSub; ++t)
        acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[t], acc[i][t], 0, 0, 0);
    }
  }
}

template <class S, int NS>
__device__ __forceinline__ void tile_kloop(const Operands<S>& o, int nk, char* smem,
                                           f32x16 (&acc)[S::kMSub][S::kNSub]) {
#pragma unroll
  for (int s = 0; s < S::STAGES - 1; ++s)
    if (s < nk) tile_issue<S>(o, s, smem + s * S::kStageBytes);
  int slot = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const int issued_after = nk - 1 - kt < S::STAGES - 2 ? nk - 1 - kt : S::STAGES - 2;
    tile_wait<S>(issued_after);  // this wave's loads of step kt have landed
    block_sync_lds();            // ... everyone's have; everyone is done with step kt-1's slot
    if (kt + S::STAGES - 1 < nk) {
      int nslot = slot + S::STAGES - 1;
      if (nslot >= S::STAGES) nslot -= S::STAGES;
      tile_issue<S>(o, kt + S::STAGES - 1, smem + nslot * S::kStageBytes);
    }
    tile_compute<S, NS>(smem + slot * S::kStageBytes, acc);
    if (++slot == S::STAGES) slot = 0;
  }
}

// Full K loop over K (a multiple of BK).  m_valid = rows of this tile that exist; each wave spends
// MFMAs only on its non-empty 32-row sub-tiles (all waves issue the same loads and pass the same
// barriers).
template <class S>
__device__ __forceinline__ void tile_mainloop(const Operands<S>& o, int m_valid, int K, char* smem,
                                              f32x16 (&acc)[S::kMSub][S::kNSub]) {
#pragma unroll
  for (int i = 0; i < S::kMSub; ++i)
#pragma unroll
    for (int t = 0; t < S::kNSub; ++t) acc[i][t] = f32x16{};
  const int nk = K / S::BK;
  const int wm = __builtin_amdgcn_readfirstlane(threadIdx.x >> 8);  // wave row (waves 0-3: 0, 4-7: 1)
  const int nsub = (m_valid + 31) / 32;
  int ns = (nsub - wm + 1) / 2;
  ns = ns < 0 ? 0 : (ns > S::kMSub ? S::kMSub : ns);
  static_assert(S::kMSub == 2 || S::kMSub == 4, "dispatch");
  // One K-loop instance per sub-tile count (a branch inside the loop would make the accumulators
  // live across diverging code and spill).  Device pass only: these instances are device code.
#if defined(__HIP_DEVICE_COMPILE__)
  if constexpr (S::kMSub == 4) {
    switch (ns) {
      case 4: tile_kloop<S, 4>(o, nk, smem, acc); break;
      case 3: tile_kloop<S, 3>(o, nk, smem, acc); break;
      case 2: tile_kloop<S, 2>(o, nk, smem, acc); break;
      case 1: tile_kloop<S, 1>(o, nk, smem, acc); break;
      default: tile_kloop<S, 0>(o, nk, smem, acc); break;
    }
  } else {
    switch (ns) {
      case 2: tile_kloop<S, 2>(o, nk, smem, acc); break;
      case 1: tile_kloop<S, 1>(o, nk, smem, acc); break;
      default: tile_kloop<S, 0>(o, nk, smem, acc); break;
    }
  }
#else
  (void)ns;
  (void)nk;
#endif
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
