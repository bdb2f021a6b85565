// Grouped SwiGLU expert GEMMs for at most 64 rows in all, more than the weight-stream kernels take per
// group (the dense first-layer FFN of a decode step, a handful of busy experts): bf16, weight streaming.
//
// The experts are the SwiGLU FFNs of "Kimi K2.5 模型架构深度拆解" §4.3 / §10.2 Steps 5-6 (the dense
// layer of §4.1 has the same form with its own intermediate size), batched over the groups present
// as the grouped GEMM of "Kimi K2.5 架构 QA" Q8.3.
//
// With at most 64 token rows every weight byte feeds at most 64 rows, so the launch is bound by
// streaming the weights once from HBM; the 64 rows ride along.  The shape that reaches the HBM roof:
//   * One work-group per CU (the LDS ring takes the CU), and the work cut so that the grid is a whole
//     number of rounds over the 256 CUs: the work-group is nw waves (4..9), each owning one
//     "granule" of 16 weight rows -- gate/up: the gate rows and the up rows of 8 h columns; down: 16
//     output columns of one K range.  The host picks nw (and for down the number of K ranges, whose
//     fp32 partial sums a reduction adds in K order) from the shape: the dense 7168 -> 18432 FFN
//     runs 256 work-groups of 9 waves for gate/up and 4 K ranges x 64 work-groups of 7 waves for down.
//   * K in steps of 64 (128-byte row segments, whole cache lines), each step one stage of an LDS ring
//     of D stages (7 for up to 7 waves, else 6): the step's 64 token rows (8 KiB, shared by the
//     waves) and each wave's 16 weight rows (2 KiB), all loaded with gfx950's direct global -> LDS loads (one instruction =
//     8 rows x 128 bytes), weights with the streaming policy.  D-1 steps are in flight; one barrier
//     per step publishes a stage and frees the one refilled next.  Each stage is its own __shared__
//     array and the K loop is unrolled by D, so the compiler can tell which LDS reads depend on which
//     direct loads.
//   * 16-byte chunk c of LDS row r sits at c ^ ((r >> 1) & 7): the 16 rows read by one 16-lane group
//     of a v_mfma_f32_16x16x32_bf16 operand fall in 16 different bank groups; token and weight rows
//     share the layout, so one address pattern serves both operands.
//   * Gate/up: a granule's MFMA block has the 8 gate rows as columns 0..7 and the 8 up rows as
//     columns 8..15, so the lane holding gate column c takes its up value from lane c + 8 (a lane
//     exchange) for SiLU(g) * u.
//   * Rows past a group's end are loaded as copies of its first row and never stored; the MFMA row
//     blocks stop at the group's last 16-row block.
// Weight rows a multiple of 4 KiB apart (W_down of the dense FFN: 36 KiB) would put every
// work-group's step on the same HBM channels, so then each work-group starts its K range at its
// own step and wraps around.
#include <type_traits>

#include "kernels.h"
#include "tile_core.h"

namespace moe {
namespace {

constexpr int kSkRows = 64;  // token rows at most (4 MFMA row blocks)
constexpr int kSkLds = 160 * 1024;
constexpr int kSkMinWaves = 4, kSkMaxWaves = 9;

// K step of the gate/up and the down kernels (64 or 128 k: 128- or 256-byte row segments).
// (measured on the dense 7168 -> 18432 FFN at 64 rows: 128 is 2-3% faster than 64 for both)
#ifndef MOE_SKINNY_BK_GATEUP
#define MOE_SKINNY_BK_GATEUP 128
#endif
#ifndef MOE_SKINNY_BK_DOWN
#define MOE_SKINNY_BK_DOWN 128
#endif

// Ring shape for K step BK: D stages, each the step's 64 token rows plus up to kSkMaxWaves waves'
// 16 weight rows, in the whole LDS; NA token-row pieces per wave per step for nw waves.
template <int BK>
struct SkGeom {
  static constexpr int kRowB = 2 * BK;                  // bytes of one row of one step
  static constexpr int kCpr = kRowB / 16;               // 16-byte chunks per row
  static constexpr int kRpl = 1024 / kRowB;             // rows one direct load fills
  static constexpr int kPieces = 16 / kRpl;             // direct loads of one wave's 16 weight rows
  static constexpr int kAPieces = kSkRows / kRpl;       // direct loads of the 64 token rows
  static constexpr int kABytes = kSkRows * kRowB;
  static constexpr int kSetBytes = 16 * kRowB;
  static constexpr int kKSub = BK / 32;                 // MFMA k blocks per step
  // stages: as many as hold kSkMaxWaves waves (7 for up to 7 waves at BK = 64)
  static constexpr int depth(int nw) {
    return BK == 64 ? (nw <= 7 ? 7 : 6) : (nw <= 6 ? 4 : 3);
  }
  template <int D>
  static constexpr int stage_bytes() {
    return kSkLds / D / kSetBytes * kSetBytes;
  }
  static constexpr int apieces(int nw) { return (kAPieces + nw - 1) / nw; }
  static constexpr int max_waves(int D) {  // the most waves a ring of depth D holds
    return BK == 64 ? (D == 7 ? 7 : kSkMaxWaves) : (D == 4 ? 6 : kSkMaxWaves);
  }
  // the 16-byte chunk c of LDS row r sits at c ^ swz(r): the 16 rows one 16-lane group reads fall in
  // 16 different bank groups
  __device__ static __forceinline__ int swz(int r) { return kRowB == 128 ? (r >> 1) & 7 : r & 15; }
};
static_assert(SkGeom<64>::stage_bytes<7>() >= SkGeom<64>::kABytes + 7 * SkGeom<64>::kSetBytes &&
                  SkGeom<64>::stage_bytes<6>() >= SkGeom<64>::kABytes + kSkMaxWaves * SkGeom<64>::kSetBytes &&
                  SkGeom<128>::stage_bytes<4>() >= SkGeom<128>::kABytes + 6 * SkGeom<128>::kSetBytes &&
                  SkGeom<128>::stage_bytes<3>() >= SkGeom<128>::kABytes + kSkMaxWaves * SkGeom<128>::kSetBytes,
              "ring depth per wave count");

struct SkinnyArgs {
  const int32_t* group_offsets;
  const int32_t* row_index;  // gate/up: token row of row r (null: r)
  int64_t max_rows;
  Weights w;
  const uint16_t* a;         // gate/up: x [*, H]; down: h [max_rows, I]
  void* out;                 // gate/up: h (bf16); down: y_rows (bf16 or fp32)
  int out_bf16;
  const float* row_scale;
  float* part;               // down with n_ks > 1: [n_ks, max_rows, H] fp32 partial sums
  int H, I;
  int nw;                    // waves per work-group
  int n_nblk;                // work-groups per group and K range
  int n_ks;                  // K ranges (1 for gate/up)
};

// The ring of one work-group: D stage arrays.
template <int D>
struct SkRing {
  char* st[D];
};

// Loads and MFMAs of one work-group's K range.  NA token-row pieces per wave per step, the pieces
// dealt round-robin: when nw does not divide them, some waves load a piece another wave loads too
// (same bytes to the same place), so every wave issues the same loads and one wait count fits all.
template <int BK, int D, int NA>
struct SkStream {
  using G = SkGeom<BK>;
  static constexpr int kLoads = G::kPieces + NA;  // vector-memory operations per step per wave
  static_assert((D - 2) * kLoads <= 63, "vmcnt");

  const char* wsrc[G::kPieces];  // the wave's weight pieces at the first k of the range (uniform)
  uint32_t w_off[G::kPieces];    // lane offset in each piece: its row, swizzled chunk
  const char* asrc[NA];          // lane's token row + swizzled chunk at the first k of the range
  int a_dst[NA];                 // LDS offsets of the token-row pieces (uniform)
  int w_dst;                     // LDS offset of this wave's weight rows (uniform)
  int nsteps, skew;

  __device__ __forceinline__ void issue(const SkRing<D>& ring, int d, int st) const {
    int ks = st + skew;
    if (ks >= nsteps) ks -= nsteps;
    const uint32_t kb = (uint32_t)ks * G::kRowB;
    char* stage = ring.st[d];
#pragma unroll
    for (int pc = 0; pc < G::kPieces; ++pc)
      __builtin_amdgcn_global_load_lds(wsrc[pc] + (w_off[pc] + kb), stage + w_dst + pc * 1024, 16, 0, 2);
#pragma unroll
    for (int j = 0; j < NA; ++j) __builtin_amdgcn_global_load_lds(asrc[j] + kb, stage + a_dst[j], 16, 0, 0);
  }

  // MFMAs of one step over NP 16-row blocks: B from this wave's weight rows, A from the shared rows.
  template <int NP>
  __device__ __forceinline__ void compute(const SkRing<D>& ring, int d, f32x4 (&acc)[NP]) const {
    const int lane = threadIdx.x & 63, c = lane & 15, q = lane >> 4;
    const char* stage = ring.st[d];
    const int sw = G::swz(c);
#pragma unroll
    for (int j = 0; j < G::kKSub; ++j) {
      const int pos = ((4 * j + q) ^ sw) << 4;
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(stage + w_dst + c * G::kRowB + pos);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(stage + (16 * i + c) * G::kRowB + pos);
        acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
      }
    }
  }

  // Wait for this wave's loads of a step, `ahead` later steps' loads still in flight.
  __device__ __forceinline__ static void wait(int ahead) {
    static_assert(D <= 7, "wait cases");
    switch (ahead) {
      case 5: wait_vmcnt<5 * kLoads>(); break;
      case 4: wait_vmcnt<4 * kLoads>(); break;
      case 3: wait_vmcnt<3 * kLoads>(); break;
      case 2: wait_vmcnt<2 * kLoads>(); break;
      case 1: wait_vmcnt<1 * kLoads>(); break;
      default: wait_vmcnt<0>(); break;
    }
  }

  // Step st (stage DS = st % D): its loads landed everywhere (wait + barrier, which also tells that
  // every wave is done with step st - 1), refill step st - 1's stage with step st + D - 1, multiply.
  template <int DS, bool kTail, int NP>
  __device__ __forceinline__ void step(const SkRing<D>& ring, int st, f32x4 (&acc)[NP]) const {
    if (kTail) {
      const int later = nsteps - 1 - st;
      wait(later < D - 2 ? later : D - 2);
    } else {
      wait_vmcnt<(D - 2) * kLoads>();
    }
    block_sync_lds();
    if (!kTail || st + D - 1 < nsteps) issue(ring, (DS + D - 1) % D, st + D - 1);
    compute<NP>(ring, DS, acc);
  }

  template <bool kTail, int NP>
  __device__ __forceinline__ void unrolled(const SkRing<D>& ring, int st, f32x4 (&acc)[NP]) const {
    static_for<D>([&](auto i) {
      constexpr int s = decltype(i)::value;
      if (!kTail || st + s < nsteps) step<s, kTail, NP>(ring, st + s, acc);
    });
  }

  template <int NP>
  __device__ __forceinline__ void run(const SkRing<D>& ring, f32x4 (&acc)[NP]) const {
#pragma unroll
    for (int i = 0; i < NP; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    int st = 0;
    if (nsteps >= 2 * D - 1) {
      // unconditional prologue and steady state: every refill of these steps exists and every wait
      // leaves D - 2 steps in flight
      static_for<D - 1>([&](auto i) { issue(ring, decltype(i)::value, decltype(i)::value); });
      for (; st + 2 * D - 1 <= nsteps; st += D) unrolled<false, NP>(ring, st, acc);
    } else {
      static_for<D - 1>([&](auto i) {
        constexpr int s = decltype(i)::value;
        if (s < nsteps) issue(ring, s, s);
      });
    }
    for (; st < nsteps; st += D) unrolled<true, NP>(ring, st, acc);
  }
};

template <bool GU, int BK, int D, int NA>
__device__ __forceinline__ void skinny_body(const SkinnyArgs& p, const SkRing<D>& ring);

// Exactly D stage arrays (no placeholder arrays: the ring takes the whole LDS).
template <bool GU, int BK, int D, int NA>
__global__ __launch_bounds__(64 * SkGeom<BK>::max_waves(D)) void skinny_kernel(SkinnyArgs p) {
  constexpr int S = SkGeom<BK>::template stage_bytes<D>();
  if constexpr (D == 3) {
    __shared__ __align__(1024) char s0[S], s1[S], s2[S];
    skinny_body<GU, BK, D, NA>(p, SkRing<D>{{s0, s1, s2}});
  } else if constexpr (D == 4) {
    __shared__ __align__(1024) char s0[S], s1[S], s2[S], s3[S];
    skinny_body<GU, BK, D, NA>(p, SkRing<D>{{s0, s1, s2, s3}});
  } else if constexpr (D == 6) {
    __shared__ __align__(1024) char s0[S], s1[S], s2[S], s3[S], s4[S], s5[S];
    skinny_body<GU, BK, D, NA>(p, SkRing<D>{{s0, s1, s2, s3, s4, s5}});
  } else {
    static_assert(D == 7, "ring depths 3, 4, 6, 7");
    __shared__ __align__(1024) char s0[S], s1[S], s2[S], s3[S], s4[S], s5[S], s6[S];
    skinny_body<GU, BK, D, NA>(p, SkRing<D>{{s0, s1, s2, s3, s4, s5, s6}});
  }
}

template <bool GU, int BK, int D, int NA>
__device__ __forceinline__ void skinny_body(const SkinnyArgs& p, const SkRing<D>& ring) {
  // device pass only (the host pass does not resolve the device members the body calls)
#if defined(__HIP_DEVICE_COMPILE__)
  using G = SkGeom<BK>;
  const int per_group = p.n_nblk * p.n_ks;
  const int g = (int)blockIdx.x / per_group, rem = (int)blockIdx.x % per_group;
  const int nb = rem / p.n_ks, kr = rem % p.n_ks;
  int64_t r0 = p.group_offsets[g], r1 = p.group_offsets[g + 1];
  if (r0 > p.max_rows) r0 = p.max_rows;
  if (r1 > p.max_rows) r1 = p.max_rows;
  if (r1 - r0 > kSkRows) r1 = r0 + kSkRows;  // never: the host takes this path for at most 64 rows
  if (r1 <= r0) return;
  const int nrows = (int)(r1 - r0);

  const int H = p.H, I = p.I, K = GU ? H : I;
  const int kc = K / p.n_ks, k0 = kr * kc;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gran = nb * p.nw + wave;  // this wave's granule
  const bool sh = g == p.w.shared_group;

  SkStream<BK, D, NA> s;
  s.nsteps = kc / BK;
  s.skew = (K * 2) % 4096 == 0 ? (nb * 5 + kr * 3) % s.nsteps : 0;
  s.w_dst = G::kABytes + wave * G::kSetBytes;
  int n0;  // first output column of this wave (gate/up: h column)
  constexpr int kHalf = G::kPieces / 2;
  if constexpr (GU) {
    // set rows 0..7: the gate rows of h columns n0 .., rows 8..15: the up rows
    n0 = gran * 8;
    const uint16_t* wg = sh ? (const uint16_t*)p.w.s_gate : (const uint16_t*)p.w.gate + (int64_t)g * I * H;
    const uint16_t* wu = sh ? (const uint16_t*)p.w.s_up : (const uint16_t*)p.w.up + (int64_t)g * I * H;
#pragma unroll
    for (int pc = 0; pc < G::kPieces; ++pc) {
      const uint16_t* base = pc < kHalf ? wg : wu;
      s.wsrc[pc] = reinterpret_cast<const char*>(base + (int64_t)(n0 + G::kRpl * (pc % kHalf)) * H + k0);
    }
  } else {
    n0 = gran * 16;
    const uint16_t* wd = sh ? (const uint16_t*)p.w.s_down : (const uint16_t*)p.w.down + (int64_t)g * H * I;
#pragma unroll
    for (int pc = 0; pc < G::kPieces; ++pc)
      s.wsrc[pc] = reinterpret_cast<const char*>(wd + (int64_t)(n0 + G::kRpl * pc) * I + k0);
  }
#pragma unroll
  for (int pc = 0; pc < G::kPieces; ++pc) {
    const int r = lane / G::kCpr;  // row in the piece; set row kRpl * pc + r
    s.w_off[pc] = (uint32_t)(r * K * 2 + (((lane % G::kCpr) ^ G::swz(G::kRpl * pc + r)) << 4));
  }
  const int nw = p.nw;
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int piece = (wave + j * nw) % G::kAPieces;
    const int row = G::kRpl * piece + lane / G::kCpr;
    const int64_t rr = r0 + (row < nrows ? row : 0);
    const int64_t src = GU ? (p.row_index ? (int64_t)p.row_index[rr] : rr) : rr;
    s.asrc[j] = reinterpret_cast<const char*>(p.a + src * K + k0 + (((lane % G::kCpr) ^ G::swz(row)) << 3));
    s.a_dst[j] = piece * 1024;
  }
  const int c = lane & 15, q = lane >> 4;
  const auto finish = [&](auto np_c) {
    constexpr int NP = decltype(np_c)::value;
    f32x4 acc[NP];
    s.template run<NP>(ring, acc);
#pragma unroll
    for (int i = 0; i < NP; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * i + 4 * q + e;
        if constexpr (GU) {
          const float u = __shfl_xor(acc[i][e], 8);
          if (c < 8 && row < nrows)
            static_cast<uint16_t*>(p.out)[(r0 + row) * I + n0 + c] = f32_to_bf16(swiglu_f32(acc[i][e], u));
        } else {
          if (row >= nrows) continue;
          const float v = acc[i][e] * (p.row_scale ? p.row_scale[r0 + row] : 1.f);
          const int64_t o = (r0 + row) * H + n0 + c;
          if (p.n_ks > 1)
            p.part[(int64_t)kr * p.max_rows * H + o] = v;
          else if (p.out_bf16)
            static_cast<uint16_t*>(p.out)[o] = f32_to_bf16(v);
          else
            static_cast<float*>(p.out)[o] = v;
        }
      }
  };
  switch ((nrows + 15) >> 4) {
    case 1: finish(std::integral_constant<int, 1>{}); break;
    case 2: finish(std::integral_constant<int, 2>{}); break;
    case 3: finish(std::integral_constant<int, 3>{}); break;
    default: finish(std::integral_constant<int, 4>{}); break;
  }
#else
  (void)p;
  (void)ring;
#endif
}

constexpr int kSkCUs = 256;  // MI355X compute units; one work-group per CU

// Fraction of a full round of work-groups over the CUs that `wgs` work-groups fill.
double sk_fill(int64_t wgs) {
  const int64_t rounds = (wgs + kSkCUs - 1) / kSkCUs;
  return (double)wgs / (double)(rounds * kSkCUs);
}

template <bool GU, int BK, int D, int NA>
void launch_skinny_as(const SkinnyArgs& a, int64_t blocks, hipStream_t s) {
  static_assert(SkGeom<BK>::template stage_bytes<D>() * D <= kSkLds, "LDS");
  skinny_kernel<GU, BK, D, NA><<<(unsigned)blocks, dim3(64 * a.nw), 0, s>>>(a);
}

// The instantiation for nw waves: ring depth and token-row pieces per wave follow from nw.
template <bool GU, int BK>
hipError_t launch_skinny(const SkinnyArgs& a, int G, hipStream_t s) {
  using Gm = SkGeom<BK>;
  const int64_t blocks = (int64_t)G * a.n_nblk * a.n_ks;
  const int nw = a.nw;
  if (nw < kSkMinWaves || nw > kSkMaxWaves) return hipErrorInvalidValue;
  const int D = Gm::depth(nw), NA = Gm::apieces(nw);
  if constexpr (BK == 64) {
    if (D == 7 && NA == 2) launch_skinny_as<GU, BK, 7, 2>(a, blocks, s);
    else if (D == 6 && NA == 1) launch_skinny_as<GU, BK, 6, 1>(a, blocks, s);
    else return hipErrorInvalidValue;
  } else {
    static_assert(BK == 128, "K step 64 or 128");
    if (D == 4 && NA == 4) launch_skinny_as<GU, BK, 4, 4>(a, blocks, s);
    else if (D == 4 && NA == 3) launch_skinny_as<GU, BK, 4, 3>(a, blocks, s);
    else if (D == 3 && NA == 3) launch_skinny_as<GU, BK, 3, 3>(a, blocks, s);
    else if (D == 3 && NA == 2) launch_skinny_as<GU, BK, 3, 2>(a, blocks, s);
    else return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool skinny_ok(int64_t max_rows, int H, int I) {
  constexpr int bg = MOE_SKINNY_BK_GATEUP, bd = MOE_SKINNY_BK_DOWN;
  return max_rows >= 1 && max_rows <= kSkRows && H % 64 == 0 && I % 64 == 0 && H >= bg && H % bg == 0 && I >= bd &&
         I % bd == 0;
}

SkinnyPlan skinny_gateup_plan(int G, int H, int I) {
  (void)H;
  SkinnyPlan best{8, I / 64, 1};  // I % 64 == 0: 8 waves always divide the I / 8 granules
  double best_fill = -1.0;
  for (int nw = kSkMinWaves; nw <= kSkMaxWaves; ++nw) {
    if ((I / 8) % nw) continue;
    const double f = sk_fill((int64_t)G * (I / 8 / nw));
    if (f > best_fill - 1e-9) {  // ties: the larger work-group (fewer rounds, more loads in flight per CU)
      best_fill = f;
      best = SkinnyPlan{nw, I / 8 / nw, 1};
    }
  }
  return best;
}

SkinnyPlan skinny_down_plan(int G, int64_t max_rows, int H, int I) {
  // cost in bytes moved: the weights scaled by the CU rounds they take, plus each K range's fp32
  // partial sums written and read back
  const double wbytes = 2.0 * G * H * I;
  SkinnyPlan best{4, H / 64, 1};
  double best_cost = 1e300;
  const int nk = I / MOE_SKINNY_BK_DOWN;
  for (int nw = kSkMinWaves; nw <= kSkMaxWaves; ++nw) {
    if ((H / 16) % nw) continue;
    for (int ks = 1; ks <= 16; ++ks) {
      if (nk % ks) continue;
      const int64_t wgs = (int64_t)G * (H / 16 / nw) * ks;
      const double cost = wbytes / sk_fill(wgs) + (ks > 1 ? 8.0 * ks * max_rows * H : 0.0);
      if (cost < best_cost * (1 + 1e-9)) {  // ties: the larger work-group
        best_cost = cost;
        best = SkinnyPlan{nw, H / 16 / nw, ks};
      }
    }
  }
  return best;
}

hipError_t launch_gateup_skinny_bf16(const Groups& g, const Weights& w, const uint16_t* x, uint16_t* h, int H,
                                     int I, hipStream_t s) {
  if (!skinny_ok(g.max_rows, H, I)) return hipErrorInvalidValue;
  const SkinnyPlan pl = skinny_gateup_plan(g.n_groups, H, I);
  SkinnyArgs a{g.group_offsets, g.row_index, g.max_rows, w, x, h, 1, nullptr, nullptr, H, I, pl.nw, pl.nblk, 1};
  return launch_skinny<true, MOE_SKINNY_BK_GATEUP>(a, g.n_groups, s);
}

hipError_t launch_down_skinny_bf16(const Groups& g, const Weights& w, const uint16_t* h, void* y_rows, bool y_bf16,
                                   const float* row_scale, float* part, int H, int I, hipStream_t s) {
  if (!skinny_ok(g.max_rows, H, I)) return hipErrorInvalidValue;
  const SkinnyPlan pl = skinny_down_plan(g.n_groups, g.max_rows, H, I);
  if (pl.ks > 1 && !part) return hipErrorInvalidValue;
  SkinnyArgs a{g.group_offsets, nullptr, g.max_rows, w, h, y_rows, y_bf16 ? 1 : 0, row_scale,
               pl.ks > 1 ? part : nullptr, H, I, pl.nw, pl.nblk, pl.ks};
  hipError_t e = launch_skinny<false, MOE_SKINNY_BK_DOWN>(a, g.n_groups, s);
  if (e != hipSuccess || pl.ks == 1) return e;
  return launch_ksplit_reduce(part, pl.ks, g, 0, H, y_rows, y_bf16, s);
}

}  // namespace moe
