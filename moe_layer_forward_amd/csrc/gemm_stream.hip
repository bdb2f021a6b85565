// Grouped SwiGLU expert GEMMs for few rows per expert (decode-like shapes): weight streaming.
//
// Experts as in "Kimi K2.5 模型架构深度拆解" §4.3 / §10.2 Steps 5-6, batched over the experts present
// (the grouped GEMM of "Kimi K2.5 架构 QA" Q8.3).  With ~1-2 tokens per expert every weight byte is
// used once or twice, so the kernel is a weight stream: each weight byte crosses HBM once per pass
// over the group's rows (one pass covers up to 32 rows).
//
// A wave streams two 16-row sets of weight rows of one group: the 16 gate rows and the 16 matching
// up rows of 16 h columns (gate/up), or 32 rows of W_down, i.e. 32 output columns (down), so both
// kernels issue the same mix of weight and token-row loads.  Its weight rows stream through a wave-private LDS ring with gfx950's direct
// global -> LDS loads: one load instruction moves 4 rows x 256 contiguous bytes (whole cache lines)
// with the streaming (non-temporal) policy -- measured on MI355X at ~7.0 TB/s, against ~6.2 TB/s for
// 16-row x 64-byte register loads -- and kDepth K steps are in flight.  The 16 x 256-byte rows of a
// step sit in LDS with 16-byte chunk c of row r at position c ^ r, so the v_mfma_f32_16x16x32_bf16
// B-operand reads (16 rows, one chunk each per 16-lane group) hit 16 different bank groups.  The
// token rows (A operand, from L2) are loaded into registers in the same step as their weights, so the
// wave's in-order load counter never makes a weight load wait for a younger token-row load.
// The ring is private to the wave: no barriers.  Each ring stage is its own __shared__ array and the
// K loop is unrolled by the stage count, so the compiler can tell which LDS reads depend on which
// direct loads.
// Work-groups = 4 waves (64 h columns, or 128 output columns of down) of one group; groups come from
// the plan's active list, largest first, so the long-running many-row groups start early.  Besides
// decode-like calls (every group here), the kernels take the groups of at most kStreamRows rows of
// calls with many groups whose larger groups go to the tile kernels (small_only: the plan's active
// list from counters[2] on).
#include <type_traits>

#include "kernels.h"
#include "tile_core.h"

namespace moe {
namespace {

struct StreamArgs {
  const int32_t* group_offsets;
  const int32_t* row_index;
  const int32_t* active;
  const int32_t* counters;
  int64_t max_rows;
  Weights w;
  const uint16_t* a;
  void* out;
  int out_bf16;
  const float* row_scale;
  int H, I, n_nblk;
  int small_only;  // only the groups active[counters[2] ..) (the tile kernels take the others)
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kStepK = 128;                 // k per step: 256 bytes of each weight row
constexpr int kSetBytes = 16 * 256;         // one 16-row set of one step
constexpr int kMaxPasses = 2;               // 16-row passes per stream of the weights

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// R weight-row sets per wave (2: gate + up, 1: down), D ring stages, NP 16-row passes.
template <int R, int D>
struct Ring {
  static constexpr int kWaveBytes = R * kSetBytes;           // one wave's part of one stage
  static constexpr int kStageBytes = kWaves * kWaveBytes;
  char* st[D];
};

// Token-row fragments of one step for NP passes: 4 x 16 bytes per lane per pass.
template <int NP>
struct AFrag {
  u32x4 v[NP][4];
};

template <int R, int D, int NP>
struct Stream {
  static constexpr int kLoads = 4 * R + 4 * NP;  // vector-memory ops per step per wave
  static_assert((D - 1) * kLoads <= 63, "vmcnt");

  const char* wb[R];        // weight-row sets: first row of this wave's 16 (uniform)
  uint32_t w_off[4];        // lane offsets of the 4 direct loads of a set (row, swizzled chunk)
  const uint16_t* arow[NP]; // token row of each pass for this lane (row lane % 16), at k = 8*(lane/16)
  int wave_off;             // this wave's part of a stage
  int skew, nsteps;         // the K steps are visited from step skew on, wrapping at nsteps

  __device__ __forceinline__ void issue(const Ring<R, D>& ring, int d, int st, AFrag<NP>& a) const {
    char* dst = ring.st[d] + wave_off;
    int ks = st + skew;  // the K step loaded as step st (st < nsteps, skew < nsteps)
    if (ks >= nsteps) ks -= nsteps;
    const uint32_t kb = (uint32_t)ks * (kStepK * 2);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds(wb[r] + (w_off[i] + kb), dst + r * kSetBytes + i * 1024, 16, 0, 2);
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int j = 0; j < 4; ++j) a.v[p][j] = *reinterpret_cast<const u32x4*>(arow[p] + ks * kStepK + 32 * j);
  }

  // MFMAs of one step: B fragments from this wave's ring part, A fragments from registers.
  __device__ __forceinline__ void compute(const Ring<R, D>& ring, int d, const AFrag<NP>& a,
                                          f32x4 (&acc)[NP][R]) const {
    const int lane = threadIdx.x & 63, c = lane & 15, q = lane >> 4;
    const char* src = ring.st[d] + wave_off + c * 256;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(src + r * kSetBytes + (((4 * j + q) ^ c) << 4));
#pragma unroll
        for (int p = 0; p < NP; ++p)
          acc[p][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a.v[p][j]), b, acc[p][r], 0, 0, 0);
      }
    }
  }

  // One step (st % D == DS): wait for its loads, refill its stage and A slot with step st + D - 1
  // (issued first: the loads of a step are its weights then its token rows, and step st's are the
  // oldest D-1 steps back), multiply.
  template <int DS, bool kTail>
  __device__ __forceinline__ void step(const Ring<R, D>& ring, int st, int nsteps, AFrag<NP> (&a)[D],
                                       f32x4 (&acc)[NP][R]) const {
    const int ahead = kTail ? nsteps - 1 - st : D - 1;  // later steps already issued
    if constexpr (D == 2) {
      if (ahead >= 1) wait_vmcnt<kLoads>(); else wait_vmcnt<0>();
    } else {
      static_assert(D == 4, "waits below");
      if (ahead >= 3) wait_vmcnt<3 * kLoads>();
      else if (ahead == 2) wait_vmcnt<2 * kLoads>();
      else if (ahead == 1) wait_vmcnt<kLoads>();
      else wait_vmcnt<0>();
    }
    // nothing of this step moves above the wait (the compiler would then wait for every load itself)
    __builtin_amdgcn_sched_barrier(0);
    compute(ring, DS, a[DS], acc);
    // every LDS read of this stage is done before it is refilled
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (!kTail || st + D < nsteps) issue(ring, DS, st + D, a[DS]);
  }

  // The whole K stream (nsteps steps) into acc.
  __device__ __forceinline__ void run(const Ring<R, D>& ring, int nsteps, f32x4 (&acc)[NP][R]) const {
    AFrag<NP> a[D];
    int st = 0;
    if (nsteps >= 2 * D) {
      // unconditional prologue and steady state: every refill of an unrolled block exists
#pragma unroll
      for (int s = 0; s < D; ++s) issue(ring, s, s, a[s]);
      for (; st + 2 * D <= nsteps; st += D) unrolled<false>(ring, st, nsteps, a, acc);
    } else {
#pragma unroll
      for (int s = 0; s < D; ++s)
        if (s < nsteps) issue(ring, s, s, a[s]);
    }
    // the last D .. 2D-1 steps (or all of a short stream), refills checked
    for (; st + D <= nsteps; st += D) unrolled<true>(ring, st, nsteps, a, acc);
    tail_steps(ring, st, nsteps, a, acc);
  }

  template <bool kTail>
  __device__ __forceinline__ void unrolled(const Ring<R, D>& ring, int st, int nsteps, AFrag<NP> (&a)[D],
                                           f32x4 (&acc)[NP][R]) const {
    step<0, kTail>(ring, st, nsteps, a, acc);
    step<1, kTail>(ring, st + 1, nsteps, a, acc);
    if constexpr (D == 4) {
      step<2, kTail>(ring, st + 2, nsteps, a, acc);
      step<3, kTail>(ring, st + 3, nsteps, a, acc);
    }
  }

  __device__ __forceinline__ void tail_steps(const Ring<R, D>& ring, int st, int nsteps, AFrag<NP> (&a)[D],
                                             f32x4 (&acc)[NP][R]) const {
    if (st < nsteps) step<0, true>(ring, st, nsteps, a, acc);
    if constexpr (D == 4) {
      if (st + 1 < nsteps) step<1, true>(ring, st + 1, nsteps, a, acc);
      if (st + 2 < nsteps) step<2, true>(ring, st + 2, nsteps, a, acc);
    }
  }
};

// One pass over the weights for rows [mb, mb + 16*NP) of the group (rows past r1 are computed from a
// copy of row mb and never stored), then the epilogue.
template <bool SWIGLU, int D, int NP>
__device__ __forceinline__ void stream_pass(const StreamArgs& p, const Ring<2, D>& ring, const char* const (&wb)[2],
                                            int n0, int skew, int64_t mb, int64_t r1) {
  constexpr int R = 2;
  const int H = p.H, I = p.I, K = SWIGLU ? H : I;
  const int lane = threadIdx.x & 63;
  // wave-uniform, so the LDS destinations of the direct loads stay visibly inside their stage array
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Stream<R, D, NP> s;
#pragma unroll
  for (int r = 0; r < R; ++r) s.wb[r] = wb[r];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * i + (lane >> 4);  // lane's row in the 16-row set, its slot = chunk position
    s.w_off[i] = (uint32_t)(row * K * 2 + (((lane & 15) ^ row) << 4));
  }
#pragma unroll
  for (int q = 0; q < NP; ++q) {
    const int64_t r = mb + 16 * q + (lane & 15);
    const int64_t rr = r < r1 ? r : mb;
    const int64_t src = SWIGLU ? (p.row_index ? (int64_t)p.row_index[rr] : rr) : rr;
    s.arow[q] = p.a + src * K + (lane >> 4) * 8;
  }
  s.wave_off = wave * Ring<R, D>::kWaveBytes;
  s.skew = skew;
  s.nsteps = K / kStepK;

  f32x4 acc[NP][R];
#pragma unroll
  for (int q = 0; q < NP; ++q)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[q][r] = f32x4{0.f, 0.f, 0.f, 0.f};
  s.run(ring, K / kStepK, acc);

  // lane holds rows mb + 16q + 4*(lane/16) + e, column n0 + lane%16
  const int col = n0 + (lane & 15);
#pragma unroll
  for (int q = 0; q < NP; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t row = mb + 16 * q + 4 * (lane >> 4) + e;
      if (row >= r1) continue;
      if (SWIGLU) {
        static_cast<uint16_t*>(p.out)[row * I + col] = f32_to_bf16(swiglu_f32(acc[q][0][e], acc[q][1][e]));
      } else {
        const float sc = p.row_scale ? p.row_scale[row] : 1.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {  // set r covers output columns n0 + 16r ..
          const float v = acc[q][r][e] * sc;
          if (p.out_bf16)
            static_cast<uint16_t*>(p.out)[row * H + col + 16 * r] = f32_to_bf16(v);
          else
            static_cast<float*>(p.out)[row * H + col + 16 * r] = v;
        }
      }
    }
}

template <bool SWIGLU, int D>
__global__ __launch_bounds__(256) void stream_kernel(StreamArgs p) {
  constexpr int R = 2;
  constexpr int kStage = Ring<R, D>::kStageBytes;
  __shared__ __align__(16) char s0[kStage], s1[kStage], s2[D == 4 ? kStage : 16], s3[D == 4 ? kStage : 16];
  Ring<R, D> ring;
  ring.st[0] = s0;
  ring.st[1] = s1;
  if constexpr (D == 4) {
    ring.st[2] = s2;
    ring.st[3] = s3;
  } else {
    (void)s2;
    (void)s3;
  }

  const int slot = (p.small_only ? p.counters[2] : 0) + (int)blockIdx.x / p.n_nblk, nb = blockIdx.x % p.n_nblk;
  if (slot >= p.counters[0]) return;
  const int g = p.active[slot];
  int64_t r0 = p.group_offsets[g], r1 = p.group_offsets[g + 1];
  if (r0 > p.max_rows) r0 = p.max_rows;
  if (r1 > p.max_rows) r1 = p.max_rows;
  const int H = p.H, I = p.I;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = nb * (SWIGLU ? 64 : 128) + wave * (SWIGLU ? 16 : 32);  // first output column of this wave
  const bool sh = g == p.w.shared_group;

  const char* wb[R];
  if constexpr (SWIGLU) {
    const uint16_t* wg = sh ? (const uint16_t*)p.w.s_gate : (const uint16_t*)p.w.gate + (int64_t)g * I * H;
    const uint16_t* wu = sh ? (const uint16_t*)p.w.s_up : (const uint16_t*)p.w.up + (int64_t)g * I * H;
    wb[0] = reinterpret_cast<const char*>(wg + (int64_t)n0 * H);
    wb[1] = reinterpret_cast<const char*>(wu + (int64_t)n0 * H);
  } else {
    const uint16_t* wd = sh ? (const uint16_t*)p.w.s_down : (const uint16_t*)p.w.down + (int64_t)g * H * I;
    wb[0] = reinterpret_cast<const char*>(wd + (int64_t)n0 * I);
    wb[1] = reinterpret_cast<const char*>(wd + (int64_t)(n0 + 16) * I);
  }
  // Passes of 32 rows (two 16-row MFMA row blocks).  A single-block variant for groups of at most
  // 16 rows would save the second block's token-row loads and MFMAs, but its K loop gets a full
  // drain of the load counter at every loop head from the compiler, which costs far more than the
  // redundant row loads (they hit L1/L2: the rows past the group's end repeat its first row).
  // Device pass only: the pass is device code.
#if defined(__HIP_DEVICE_COMPILE__)
  // Weight rows a multiple of 4 KiB apart put the same K step of every row on few HBM channels
  // (measured: 6.7 TB/s for 4 KiB rows against 7.2 when the waves start at different K steps), so
  // then each wave starts its K loop at its own step and wraps around.
  const int nst = (SWIGLU ? H : I) / kStepK;
  const int skew = ((SWIGLU ? H : I) * 2) % 4096 == 0 ? (nb * 4 + wave) * 5 % nst : 0;
  for (int64_t mb = r0; mb < r1; mb += 16 * kMaxPasses)
    stream_pass<SWIGLU, D, kMaxPasses>(p, ring, wb, n0, skew, mb, r1);
#else
  (void)wb;
  (void)n0;
#endif
}

// 2 x 32 KiB of LDS: two work-groups per CU, so one's ring fills while the other's drains (4 stages
// and one work-group per CU measured 1.5% slower on decode, 3.5% on the short down streams)
constexpr int kDepthGateUp = 2;
constexpr int kDepthDown = 2;

}  // namespace

hipError_t launch_gateup_stream_bf16(const Groups& g, const Weights& w, const uint16_t* x, uint16_t* h, int H, int I,
                                     bool small_only, hipStream_t s) {
  StreamArgs p{g.group_offsets, g.row_index, g.active, g.counters, g.max_rows, w, x, h, 1, nullptr, H, I, I / 64,
               small_only ? 1 : 0};
  const int64_t blocks = (int64_t)g.n_groups * p.n_nblk;
  stream_kernel<true, kDepthGateUp><<<(unsigned)blocks, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_down_stream_bf16(const Groups& g, const Weights& w, const uint16_t* h, void* y_rows, bool y_bf16,
                                   const float* row_scale, int H, int I, bool small_only, hipStream_t s) {
  StreamArgs p{g.group_offsets, nullptr, g.active, g.counters, g.max_rows, w, h, y_rows, y_bf16 ? 1 : 0, row_scale,
               H, I, H / 128, small_only ? 1 : 0};
  const int64_t blocks = (int64_t)g.n_groups * p.n_nblk;
  stream_kernel<false, kDepthDown><<<(unsigned)blocks, 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
