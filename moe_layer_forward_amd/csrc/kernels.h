// Internal interface between the C-ABI host layer (moe_api.cpp) and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ----------------------------------------------------------------------------- element helpers
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Logistic function in fp32 with IEEE division.
__device__ __forceinline__ float sigmoid_f32(float z) { return 1.0f / (1.0f + expf(-z)); }

// SwiGLU activation of one (gate, up) pair: SiLU(g) * u.
__device__ __forceinline__ float swiglu_f32(float g, float u) { return g * sigmoid_f32(g) * u; }

// One group of 8 bf16 values -> binary16 (exact widening, then round to nearest even), stored in the
// order 0,4,1,5,2,6,3,7: the operand order of the 4-bit kernels (a code word decodes in that order).
__device__ __forceinline__ void f16_group_pairs(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst) {
  typedef uint32_t u32x4_ __attribute__((ext_vector_type(4)));
  typedef _Float16 f16x8_ __attribute__((ext_vector_type(8)));
  const u32x4_ v = *reinterpret_cast<const u32x4_*>(src);
  _Float16 h[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t bits = (v[t >> 1] >> (16 * (t & 1))) & 0xffffu;
    h[(t & 3) * 2 + (t >> 2)] = (_Float16)__uint_as_float(bits << 16);
  }
  *reinterpret_cast<f16x8_*>(dst) = f16x8_{h[0], h[1], h[2], h[3], h[4], h[5], h[6], h[7]};
}

constexpr int kXcds = 8;  // MI355X: 8 XCDs, work-groups dealt round-robin by blockIdx

// ----------------------------------------------------------------------------- launch descriptors
// Row groups of a grouped GEMM.  Rows of group g are [group_offsets[g], group_offsets[g+1]),
// clamped to max_rows; the A row of row r is row_index ? row_index[r] : r.
struct Groups {
  int32_t n_groups = 0;
  const int32_t* group_offsets = nullptr;  // [G+1] device
  int64_t max_rows = 0;
  const int32_t* row_index = nullptr;      // [max_rows] device or null
  // Plan (workspace), written by launch_plan.
  int32_t* active = nullptr;               // [G] ids of groups with rows
  int32_t* counters = nullptr;             // [0] n_active, [1] n_tiles, [2] n_large
  int32_t* tiles = nullptr;                // [2 * max_tiles] (group, first row in group)
  int32_t max_tiles = 0;
  int32_t tile_m = 0;                      // rows per tile in the tile list
  int32_t stream_rows = 0;                 // 0, or kStreamRows: groups of at most this many rows stay
                                           // out of the tile list (see below)
};
// With many groups, groups of at most kStreamRows rows (one pass of the weight-stream kernels) stay
// out of the tile list and go to the stream kernels: active[0 .. n_large) are the larger groups,
// active[n_large .. n_active) the small ones.  Calls with fewer than kStreamMinGroups groups keep
// every group in the tile list (two more launches would cost more than the few small groups gain).
constexpr int kStreamRows = 32;
constexpr int kStreamMinGroups = 16;

// Expert weights by group: group g < shared_group uses the stacked tensors at index g; the group
// equal to shared_group uses the s_* tensors.
struct Weights {
  const void* gate = nullptr;  // [*, I, H]
  const void* up = nullptr;    // [*, I, H]
  const void* down = nullptr;  // [*, H, I]
  const void* s_gate = nullptr;
  const void* s_up = nullptr;
  const void* s_down = nullptr;
  int32_t shared_group = -1;
};

// Quantized routed-expert weights, by storage format:
//   kInt4: w = q * s, one binary16 scale per 32 consecutive inputs: codes [E, N, K/8] uint32 (q of
//          input k in bits 4*(k % 8) of word k/8, two's complement), scales [E, N, K/32] binary16
//   kFp8:  w = e4m3(c) * s, one fp32 scale per 128 x 128 block: codes [E, N, K] bytes (OCP E4M3),
//          scales [E, N/128, K/128] fp32
enum class QFormat { kInt4, kFp8 };
struct QWeights {
  QFormat format = QFormat::kInt4;
  const void* gate_codes = nullptr;   // [E, I, H] inputs per row
  const void* gate_scales = nullptr;
  const void* up_codes = nullptr;
  const void* up_scales = nullptr;
  const void* down_codes = nullptr;   // [E, H, I] inputs per row
  const void* down_scales = nullptr;
};

// ----------------------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error.

// routing ---------------------------------------------------------------------
// K splits of the router GEMM (its partial sums are [nsplit, T, E] fp32); 1 for fp32 inputs.
int router_nsplit(int64_t T, int H, int E, bool bf16);
// part[s, T, E] (fp32) = x[T, H] . w_router[E, H]^T restricted to the s-th K range
hipError_t launch_router_logits_bf16(const uint16_t* x, const uint16_t* w_router, float* part, int64_t T,
                                     int H, int E, hipStream_t s);
hipError_t launch_router_logits_f32(const float* x, const float* w_router, float* logits, int64_t T, int H,
                                    int E, hipStream_t s);
// sum of the partials, sigmoid, bias, top-K, normalise, scale: one wave per token.
hipError_t launch_topk(const float* part, int nsplit, const float* logit_offset, const float* score_bias,
                       int64_t T, int E, int K, float rsf, int32_t* ids, float* weights, hipStream_t s);

// permutation -----------------------------------------------------------------
int64_t permute_blocks(int64_t pairs);
// Scratch ints the permutation needs (block counts).
int64_t permute_scratch_ints(int64_t pairs, int E);
// group_offsets gets E+1 entries, plus a final T*K + T entry when shared_rows (the shared
// expert's rows follow the routed rows; row_token of those rows is filled with t).
hipError_t launch_permute(const int32_t* ids, int64_t T, int K, int E, int32_t* group_offsets,
                          int32_t* row_token, int32_t* pair_row, int32_t* scratch, bool shared_rows,
                          hipStream_t s);
// Few pairs (permute_plan_fused): the permutation above and, when plan.n_groups > 0,
// launch_plan(plan) in one launch, plus x16[T, H] = the binary16 token rows (f16_group_pairs order)
// when x16 is given.
bool permute_plan_fused(int64_t pairs, int E, int G);
hipError_t launch_permute_plan(const int32_t* ids, int64_t T, int K, int E, int32_t* group_offsets,
                               int32_t* row_token, int32_t* pair_row, bool shared_rows, const Groups& plan,
                               const uint16_t* x, uint16_t* x16, int H, hipStream_t s);
hipError_t launch_gather_rows(const void* x, const int32_t* row_token, void* x_perm, int64_t rows, int H,
                              int elem_bytes, hipStream_t s);

// plan --------------------------------------------------------------------------
hipError_t launch_plan(const Groups& g, hipStream_t s);

// grouped SwiGLU, bf16 ------------------------------------------------------------
// h[r, I] (bf16) = SiLU(a Wg^T) * (a Wu^T) for every row of every active group (the stream kernels:
// of the small groups only, active[n_large ..), when small_only; the tile kernels: of the groups in
// the tile list).
hipError_t launch_gateup_stream_bf16(const Groups& g, const Weights& w, const uint16_t* x, uint16_t* h, int H,
                                     int I, bool small_only, hipStream_t s);
hipError_t launch_gateup_tile_bf16(const Groups& g, const Weights& w, const uint16_t* x, uint16_t* h, int H,
                                   int I, hipStream_t s);
// y_rows[r, H] = row_scale[r] * h[r] Wd^T   (y fp32 when y_bf16 == false)
hipError_t launch_down_stream_bf16(const Groups& g, const Weights& w, const uint16_t* h, void* y_rows,
                                   bool y_bf16, const float* row_scale, int H, int I, bool small_only,
                                   hipStream_t s);
// With few row tiles the K dimension is split (down_tile_ksplit ranges, partial sums in part,
// [split, max_rows, H] fp32, then a reduction into y_rows).
hipError_t launch_down_tile_bf16(const Groups& g, const Weights& w, const uint16_t* h, void* y_rows,
                                 bool y_bf16, const float* row_scale, float* part, int H, int I, hipStream_t s);
int down_tile_ksplit(int64_t max_rows, int G, int H, int I);
// y_rows[r, :] = sum over ks of part[ks, r, :] (K-range order) for the rows of the groups (those of more
// than stream_rows rows when stream_rows > 0), bf16 or fp32.
hipError_t launch_ksplit_reduce(const float* part, int split, const Groups& g, int stream_rows, int H, void* y_rows,
                                bool y_bf16, hipStream_t s);
// Groups of at most 64 rows in all (skinny kernels: weight streaming with the token rows shared in
// LDS, one work-group of nw waves per CU).  H, I multiples of 64.
bool skinny_ok(int64_t max_rows, int H, int I);
struct SkinnyPlan {
  int nw;    // waves per work-group, one 16-weight-row granule each
  int nblk;  // work-groups per group and K range
  int ks;    // K ranges (down; their fp32 partial sums go to part, [ks, max_rows, H])
};
SkinnyPlan skinny_gateup_plan(int G, int H, int I);
SkinnyPlan skinny_down_plan(int G, int64_t max_rows, int H, int I);
hipError_t launch_gateup_skinny_bf16(const Groups& g, const Weights& w, const uint16_t* x, uint16_t* h, int H,
                                     int I, hipStream_t s);
// With more than one K range the partial sums go to part, then launch_ksplit_reduce adds them.
hipError_t launch_down_skinny_bf16(const Groups& g, const Weights& w, const uint16_t* h, void* y_rows, bool y_bf16,
                                   const float* row_scale, float* part, int H, int I, hipStream_t s);
// Rows per tile used by the tile kernels' plan.
constexpr int kTileM = 256;     // rows per tile of the tile GEMMs
constexpr int kTileMFp8 = 224;  // rows per tile of the FP8 tile GEMMs (their plan's tile_m)
constexpr int kTileMQ4 = 192;  // rows per tile of the 4-bit tile GEMMs

// grouped SwiGLU, 4-bit routed experts (weight streaming) ----------------------------
// The shared expert (bf16), computed by the first work-groups of the 4-bit launches: its rows are
// [offsets[0], offsets[1]) of the row space (token row_index[r] for gate/up), its h rows bf16.
struct SharedBf16 {
  const int32_t* offsets = nullptr;    // 2 entries, device
  const int32_t* row_index = nullptr;  // [rows] device
  const uint16_t* gate = nullptr;      // [I, H]
  const uint16_t* up = nullptr;        // [I, H]
  const uint16_t* down = nullptr;      // [H, I]
  const uint16_t* x = nullptr;         // bf16 token rows [x_rows, H]
  int64_t x_rows = 0;
  const uint16_t* h = nullptr;         // the h buffer [h_rows, I] (its shared rows bf16)
  int64_t h_rows = 0;
};
// y16[r, c] (f16) = x[r, c] with every group of 8 columns in the order 0,4,1,5,2,6,3,7.
hipError_t launch_f16_rows(const uint16_t* x, uint16_t* y16, int64_t rows, int cols, hipStream_t s);
// Whether the quantized stream kernels take these sizes (4-bit: H, I multiples of 256; FP8:
// multiples of 128, at most 8192).
bool qshape_ok(QFormat f, int H, int I);
// h16[r, I] (f16, same column order) = SiLU(a Wg^T) * (a Wu^T), a = x16 rows (x_rows of them) through
// row_index; plus the shared expert's h rows (bf16) when sh is given.  Groups g < n_routed of the plan
// are routed experts (a plan that also lists the shared expert's rows as group n_routed leaves that
// group to sh).  small_only: only the plan's small groups (active[n_large ..)), and the shared expert
// only if it has at most g.stream_rows rows; the tile kernels take the rest.
hipError_t launch_gateup_q_stream(const Groups& g, const QWeights& w, const uint16_t* x16, int64_t x_rows,
                                  uint16_t* h16, const SharedBf16* sh, int H, int I, int n_routed, bool small_only,
                                  hipStream_t s);
// y_rows[r, H] (bf16) = h16[r] Wd^T, plus the shared expert's rows when sh is given (as above).
hipError_t launch_down_q_stream(const Groups& g, const QWeights& w, const uint16_t* h16, uint16_t* y_rows,
                                const SharedBf16* sh, int H, int I, int n_routed, bool small_only, hipStream_t s);

// grouped SwiGLU, quantized routed experts, many rows per group (tile kernels) -------------
// The groups of the tile list: routed groups from their codes and scales (FP8: E4M3 codes with one
// fp32 scale per 128 x 128 block; 4-bit: the stream kernels' codes and binary16 scales per 32
// inputs), A rows binary16 in the order of launch_f16_rows (h likewise); the shared group
// (g == w.shared_group) in bf16 from w.s_* (A: x or h rows in bf16).
// FP8: H, I multiples of 128, at most 8192.  4-bit: H, I multiples of 256.
bool tile_quant_shape_ok(QFormat f, int H, int I);
// h[r, I] = SiLU(a Wg^T) * (a Wu^T): routed rows binary16 from x16 rows, shared rows bf16 from x rows
// (both through row_index).
hipError_t launch_gateup_tile_quant(const Groups& g, const Weights& w, const QWeights& q, const uint16_t* x,
                                    const uint16_t* x16, uint16_t* h, int H, int I, hipStream_t s);
// y_rows[r, H] (bf16) = h[r] Wd^T (h binary16 for routed rows, bf16 for the shared group's rows).
hipError_t launch_down_tile_quant(const Groups& g, const Weights& w, const QWeights& q, const uint16_t* h,
                                  uint16_t* y_rows, int H, int I, hipStream_t s);
// The 4-bit forms of the two (gemm_tile_q4.hip), which the two above call for QFormat::kInt4.
hipError_t launch_gateup_tile_q4(const Groups& g, const Weights& w, const QWeights& q, const uint16_t* x,
                                 const uint16_t* x16, uint16_t* h, int H, int I, hipStream_t s);
hipError_t launch_down_tile_q4(const Groups& g, const Weights& w, const QWeights& q, const uint16_t* h,
                               uint16_t* y_rows, int H, int I, hipStream_t s);

// grouped SwiGLU, fp32 (plain kernels) ---------------------------------------------
hipError_t launch_gateup_f32(const Groups& g, const Weights& w, const float* x, float* h, int H, int I,
                             hipStream_t s);
hipError_t launch_down_f32(const Groups& g, const Weights& w, const float* h, float* y_rows,
                           const float* row_scale, int H, int I, hipStream_t s);

// combine -------------------------------------------------------------------------
hipError_t launch_combine(const void* y_rows, bool rows_bf16, const int32_t* pair_row, const float* weights,
                          const void* y_shared, void* y, bool y_bf16, int64_t T, int K, int H, hipStream_t s);

}  // namespace moe
