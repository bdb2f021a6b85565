// Quantized routed experts, weight streaming (decode-like shapes, few rows per expert).
//
// Two storage formats of the routed-expert weights W [G, N, K], one kernel design:
//  * 4-bit, as "Kimi K2.5 模型架构深度拆解" §7.2 configures them: signed 4-bit integers, one scale
//    per 32 consecutive inputs, symmetric (w = q * s).  In memory:
//      codes  [G, N, K/8]  uint32: q of input k in bits 4*(k % 8) of word k/8, two's complement
//      scales [G, N, K/32] binary16
//  * 8-bit floating point, the FP8 quantization of the Baidu developer article on K2-Instruct
//    (developer.baidu.com article 8800668, §3.2 item 1), which fixes neither format nor scaling;
//    read here as OCP E4M3 codes with one fp32 scale per 128 x 128 block of each matrix:
//      codes  [G, N, K] bytes (sign, 4 exponent bits with bias 7, 3 mantissa bits)
//      scales [G, N/128, K/128] fp32;  w = e4m3(code) * s
// Only the storage is quantized ("Kimi K2.5 架构 QA" Q7.1): the matmuls run on
// v_mfma_f32_16x16x32_f16 with every code entering exactly, the token rows converted once from bf16
// to binary16 (f16_rows_kernel) and h kept in binary16, and the scales are applied in fp32 to
// partial sums.
//
// 4-bit decoding: after xor with 0x88888888 a code is offset binary u = q + 8; a field in bits 0..3
// of a 16-bit half ORed into 0x6400 reads 1024 + u, a field in bits 4..7 ORed into 0x5400 reads
// 64 + u, and since the OR constant is disjoint from the field, xor + mask + OR is one
// v_bitop3_b32.  A word's 8 codes come out in the order 0,4,1,5,2,6,3,7, so every operand keeps
// each group of 8 inputs in that order (x16 and h are written that way; the dot product is
// unchanged).  Per group of 32 inputs one MFMA against the constant -(1032 | 72) seeds the
// accumulator of the two weight sets' MFMAs, which leaves c = sum x*q exactly in fp32; then
// acc += s * c.
// FP8 decoding: a byte permute puts the codes of inputs (0,4,1,5) and (2,6,3,7) of a group of 8 into
// one word each (the same operand order), and v_cvt_scalef32_pk_f16_fp8 with scale 1 turns two
// codes into two binary16 values (every E4M3 value is a normal binary16 value, so exactly).  The 4
// MFMAs of a step (128 inputs, one scale block) sum into a partial that is scaled into acc in fp32.
//
// The stream: a wave streams two 16-row sets of weight rows (gate + up of 16 h columns, or 32 rows
// of W_down) through a 4-stage LDS ring of direct buffer->LDS loads, one instruction = 8 rows x 128
// contiguous bytes (whole lines) with the streaming policy; the 16-byte chunk c of a 128-byte row r
// sits at c ^ ((r >> 1) & 7) so the 16 rows of one B-operand read hit different banks.  A step
// covers 128 bytes of codes per row (256 inputs of 4-bit codes, 128 of FP8).  The token rows of a
// pass (4 rows of 256 inputs, or 16 rows of 128) are shared by the work-group's 4 waves through the
// same ring (a barrier per step); the 4-bit scales come a 4-step block at a time through LDS, the
// FP8 scales of a wave's whole rows sit one per lane in a register.
// Work-groups = 4 waves; groups from the plan's active list, largest first; the first work-groups
// of a launch stream the bf16 shared expert instead.
#include <type_traits>

#include "kernels.h"
#include "tile_core.h"

namespace moe {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 4;
constexpr int kCodeRowB = 128;          // bytes of codes per row per step
constexpr int kSetCodeB = 16 * kCodeRowB;
constexpr int kWaveB = 2 * kSetCodeB;   // one wave's part of the codes of one ring stage
constexpr int kCodesB = kWaves * kWaveB;
constexpr int kD = 4;                   // ring stages = steps in flight = steps per 4-bit scale block
constexpr int kScaleRowB = kD * 16;     // a row's binary16 scales for the kD steps of a block
constexpr int kScaleSetB = 16 * kScaleRowB;  // = one 64-lane 16-byte store
constexpr int kScaleWaveB = 2 * kScaleSetB;  // one wave's part of one scale buffer

// Per-format geometry: inputs per step, token rows per pass (MFMA rows past them are padding).
template <QFormat F>
struct Fmt;
template <>
struct Fmt<QFormat::kInt4> {
  static constexpr int kStepK = 256;
  static constexpr int kPassRows = 4;
};
template <>
struct Fmt<QFormat::kFp8> {
  static constexpr int kStepK = 128;
  static constexpr int kPassRows = 16;
  static constexpr int kBlock = 128;   // scale block edge
  static constexpr int kMaxSteps = 64; // a wave's row of scales fits one register of 64 lanes
};
// bytes of f16 token row per step, and bytes of codes per weight row of K inputs
template <QFormat F>
constexpr int a_row_bytes() {
  return 2 * Fmt<F>::kStepK;
}
template <QFormat F>
constexpr int64_t code_row_bytes(int64_t K) {
  return K * kCodeRowB / Fmt<F>::kStepK;
}
// a pass's token rows of one step (in the ring stage, shared by the waves), and the whole stage
template <QFormat F>
constexpr int a_stage_bytes() {
  return Fmt<F>::kPassRows * a_row_bytes<F>();
}
template <QFormat F>
constexpr int stage_bytes() {
  return kCodesB + a_stage_bytes<F>();
}
static_assert(a_stage_bytes<QFormat::kInt4>() == 2048 && a_stage_bytes<QFormat::kFp8>() == 4096, "token rows");
// two work-groups per CU: 4 stages each, plus the 4-bit scale buffer, within the 160 KiB of LDS
static_assert(2 * (4 * stage_bytes<QFormat::kFp8>()) <= 160 * 1024, "LDS");
static_assert(2 * (4 * stage_bytes<QFormat::kInt4>() + kWaves * kScaleWaveB) <= 160 * 1024, "LDS");

struct QArgs {
  const int32_t* group_offsets;
  const int32_t* row_index;  // gate/up: token row of each routed row
  const int32_t* active;
  const int32_t* counters;
  int64_t max_rows;
  const void* codes0;        // gate (gate/up) or down codes
  const void* scales0;
  const void* codes1;        // up codes (gate/up)
  const void* scales1;
  const uint16_t* a;         // f16 rows, groups of 8 inputs in the order 0,4,1,5,2,6,3,7
  uint32_t a_bytes;          // bytes of a the kernel may read (< 4 GiB)
  void* out;
  int out_bf16;
  const float* row_scale;
  int H, I, n_wg;
  // The shared expert (bf16 weights and rows) in the same launch: work-groups [0, sh_blocks).
  int sh_blocks;
  const int32_t* sh_offsets;    // its rows: [sh_offsets[0], sh_offsets[1])
  const int32_t* sh_row_index;  // gate/up: token row of each of its rows
  const uint16_t* sh_w0;        // gate (gate/up) or down weight
  const uint16_t* sh_w1;        // up weight (gate/up)
  const uint16_t* sh_a;         // bf16 x (gate/up) or h (down) rows
  uint32_t sh_a_bytes;
  // Calls whose larger groups go to the tile kernels: only the groups active[counters[2] ..) of at
  // most stream_rows rows, and the shared expert only if it has at most stream_rows rows.
  int small_only;
  int stream_rows;
  int n_routed;  // groups >= n_routed (the shared expert's, when the plan lists it) are not streamed
};

__device__ __forceinline__ int code_swz(int r) { return (r >> 1) & 7; }

// Position of input t (0..7) of a group of 8 in the f16 operand order 0,4,1,5,2,6,3,7.
__device__ __forceinline__ int pair_pos(int t) { return ((t & 3) << 1) | (t >> 2); }

// The binary16 scale of group J of a step as fp32: the low half of scale word J/2 for even J, the
// high half for odd J.
template <int J>
__device__ __forceinline__ float scale_f32(uint32_t sw) {
  const uint16_t h = (J & 1) ? (uint16_t)(sw >> 16) : (uint16_t)(sw & 0xffffu);
  return (float)__builtin_bit_cast(_Float16, h);
}

// The 8 codes of one word as exact binary16 integers, in the operand order 0,4,1,5,2,6,3,7:
// code k in bits 4k..4k+3 (two's complement q) -> offset binary u = q + 8; a field in bits 0..3 of a
// 16-bit half ORed into 0x6400 reads 1024 + u, a field in bits 4..7 ORed into 0x5400 reads 64 + u.
// The constant parts (1032 and 72 per input position, kBias) are removed by the bias matmul.  Since
// the OR constant is disjoint from the field, ((w ^ 0x88888888) & M) | C == (w & M) ^ K with
// K = (0x88888888 & M) | C: one three-input bit operation per pair of codes.
__device__ __forceinline__ f16x8 decode(uint32_t w) {
  const uint32_t w8 = w >> 8;
  u32x4 r;
  r[0] = (w & 0x000F000Fu) ^ 0x64086408u;   // codes 0, 4: 1024 + u
  r[1] = (w & 0x00F000F0u) ^ 0x54805480u;   // codes 1, 5: 64 + u
  r[2] = (w8 & 0x000F000Fu) ^ 0x64086408u;  // codes 2, 6
  r[3] = (w8 & 0x00F000F0u) ^ 0x54805480u;  // codes 3, 7
  return __builtin_bit_cast(f16x8, r);
}

// Minus the constant part of each decoded position (B operand of the bias matmul).
__device__ __forceinline__ f16x8 bias_operand() {
  const _Float16 a = (_Float16)-1032.f, b = (_Float16)-72.f;
  return f16x8{a, a, b, b, a, a, b, b};
}

// The 8 E4M3 codes of inputs 0..7 (bytes of w.x then w.y) as binary16 values in the operand order
// 0,4,1,5,2,6,3,7: v_perm_b32 gathers bytes (0,4,1,5) and (2,6,3,7), and each conversion takes the
// low or the high byte pair of a word.
__device__ __forceinline__ f16x8 decode_fp8(u32x2 w) {
  const uint32_t p0 = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);  // bytes: codes 0, 4, 1, 5
  const uint32_t p1 = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);  // codes 2, 6, 3, 7
  const f16x2 h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(p0, 1.0f, false);
  const f16x2 h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(p0, 1.0f, true);
  const f16x2 h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(p1, 1.0f, false);
  const f16x2 h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(p1, 1.0f, true);
  return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

typedef __amdgpu_buffer_rsrc_t Rsrc;

// Buffer descriptor of `bytes` bytes at base: a load at an offset past the end returns zeros and
// reads no memory (how the ring's padded steps stay uniform).
// base and bytes must be wave-uniform (a descriptor in VGPRs makes the compiler wrap each load in a
// loop over the wave's distinct descriptors).
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void* LdsPtr;

// Token rows in a ring stage: row r of the pass at r * a_row_bytes, its 16-byte piece g at a
// position xor-ed with the row (4-bit: 4 rows of 32 pieces, g ^ 4r; FP8: 16 rows of 16 pieces,
// g ^ r), so the rows one A-operand read touches fall in different banks.
template <QFormat F>
__device__ __forceinline__ int a_pos(int r, int g) {
  return F == QFormat::kInt4 ? g ^ (4 * r) : g ^ r;
}

template <QFormat F>
struct QStream {
  static constexpr bool kQ4 = F == QFormat::kInt4;
  static constexpr int kPassRows = Fmt<F>::kPassRows;
  static constexpr int kARowB = a_row_bytes<F>();
  // per step: codes (2 sets x 2 direct loads), and this wave's part of the pass's token rows (FP8: a
  // quarter, one per wave; 4-bit: a half, loaded by waves w and w + 2 alike)
  static constexpr int kLoads = 2 * 2 + 1;
  static constexpr int kScaleLoads = kQ4 ? 2 : 0;  // per block of kD steps: 4-bit scales (into registers)
  static_assert(2 * kLoads + kScaleLoads <= 63, "vmcnt");

  const void* cb[2];        // codes of each set's 16 rows (uniform)
  const void* sb[2];        // scales of each set's rows (uniform; FP8: the wave's block row)
  const void* abase;        // token rows (f16)
  uint32_t c_bytes, s_bytes, a_bytes;  // bytes the descriptors of codes, scales, token rows span
  uint32_t c_off[2];        // lane offsets of the two direct loads of a set (row, swizzled chunk)
  uint32_t s_off;           // 4-bit: lane offset of the scale load (row lane/4, piece lane%4 of a block)
  uint32_t a_off;           // lane offset of this wave's token-row load (row, swizzled piece)
  uint32_t blk_cb, blk_sb;  // bytes between consecutive column blocks of the codes / the scales
  int wave_off, sc_wave_off, a_dst;  // this wave's codes, scale buffer, and its part of the token rows

  // Position (b, k) + off steps, where a column block has ksteps steps: one carry is enough to
  // tell live steps (b < the chain length) from the padded ones past the end.
  __device__ __forceinline__ static void adv(int b, int k, int off, int ksteps, int& b2, int& k2) {
    k2 = k + off;
    b2 = b;
    if (k2 >= ksteps) {
      k2 -= ksteps;
      ++b2;
    }
  }

  // The codes of step k of column block b into ring stage d; past the last block (nblk) they read
  // nothing and fill zeros.
  __device__ __forceinline__ void issue_codes(char* const (&ring)[kD], int d, int b, int k, int nblk) const {
    // b, k through readfirstlane: scalar, and opaque to the optimiser, which would otherwise
    // precompute addresses per (step, load) of the prologue, keep them live across the whole pass
    // and spill them
    b = __builtin_amdgcn_readfirstlane(b);
    k = __builtin_amdgcn_readfirstlane(k);
    const uint32_t cn = __builtin_amdgcn_readfirstlane(b < nblk ? c_bytes : 0u);
    const uint32_t base = (uint32_t)b * blk_cb + (uint32_t)k * kCodeRowB;
    char* dst = ring[d] + wave_off;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const Rsrc rc = make_rsrc(cb[r], cn);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (LdsPtr)(dst + r * kSetCodeB + i * 1024), 16, c_off[i] + base,
                                                 0, 0, 2);
    }
  }

  // This wave's 1 KiB part of the pass's token rows of step k into ring stage d (the same rows for
  // every column block): a quarter for FP8; a half for 4-bit, which waves w and w + 2 both load
  // (identical bytes to the same place), so that every wave issues the same loads.
  __device__ __forceinline__ void issue_rows(char* const (&ring)[kD], int d, int b, int k, int nblk) const {
    b = __builtin_amdgcn_readfirstlane(b);
    k = __builtin_amdgcn_readfirstlane(k);
    const uint32_t an = __builtin_amdgcn_readfirstlane(b < nblk ? a_bytes : 0u);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(abase, an), (LdsPtr)(ring[d] + kCodesB + a_dst), 16,
                                             a_off + (uint32_t)k * kARowB, 0, 0, 0);
  }

  // 4-bit: the scales of steps k .. k + kD - 1 of column block b (k a multiple of kD) into
  // registers: lane l holds the 16 bytes of step k + l%4 of row l/4 (each scale line in two
  // requests, not eight).  Past the last block they read nothing.
  __device__ __forceinline__ void issue_scales(int b, int k, int nblk, u32x4 (&sr)[2]) const {
    b = __builtin_amdgcn_readfirstlane(b);
    k = __builtin_amdgcn_readfirstlane(k);
    const uint32_t sn = __builtin_amdgcn_readfirstlane(b < nblk ? s_bytes : 0u);
    const uint32_t base = (uint32_t)b * blk_sb + (uint32_t)k * 16;
#pragma unroll
    for (int r = 0; r < 2; ++r)
      sr[r] = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(sb[r], sn), s_off + base, 0, 0);
  }

  // ... and from registers into the wave's scale buffer: [set][row][kD steps x 8 scales].  (Plain
  // LDS stores: direct loads into more LDS arrays would make the compiler wait for them before
  // every ring read.)
  __device__ __forceinline__ void store_scales(char* sc, const u32x4 (&sr)[2]) const {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int r = 0; r < 2; ++r) *reinterpret_cast<u32x4*>(sc + sc_wave_off + r * kScaleSetB + lane * 16) = sr[r];
  }

  // One 4-bit step: for each group j of 32 inputs, c = A_j . (-bias) + A_j . (1024|64 + u) = A_j . q
  // (exact integer weights, fp32 sums), then acc += s_j * c with the group's scale in fp32.
  // Software pipelined by hand: code words and token-row fragments are read one group ahead, and
  // group j's products are scaled into acc while group j+1's matmuls run (scheduling barriers keep
  // the compiler from hoisting more).  d: ring stage; sc: the scale buffer holding the step's block.
  __device__ __forceinline__ void compute_q4(char* const (&ring)[kD], int d, const char* sc, f32x4 (&acc)[2]) const {
    const int lane = threadIdx.x & 63, c = lane & 15, q = lane >> 4;
    const char* src = ring[d] + wave_off + c * kCodeRowB + 4 * q;
    const int ar = c & (kPassRows - 1);  // FP8 passes fill all 16 MFMA rows: no padding rows
    const char* arow = ring[d] + kCodesB + ar * kARowB;
    u32x4 sv[2];  // the step's 8 scales of row c of each set
#pragma unroll
    for (int r = 0; r < 2; ++r)
      sv[r] = *reinterpret_cast<const u32x4*>(sc + sc_wave_off + r * kScaleSetB + c * kScaleRowB + d * 16);
    const f16x8 nb = bias_operand();
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    auto read = [&](auto jc, uint32_t (&wd)[2], u32x4& af) {
      constexpr int j = decltype(jc)::value;
#pragma unroll
      for (int r = 0; r < 2; ++r)
        wd[r] = *reinterpret_cast<const uint32_t*>(src + r * kSetCodeB + ((j ^ code_swz(c)) << 4));
      af = *reinterpret_cast<const u32x4*>(arow + (a_pos<F>(ar, 4 * j + q) << 4));
    };
    uint32_t wd[2][2];
    u32x4 af[2];
    f32x4 pend[2];
    float pend_s[2];
    read(std::integral_constant<int, 0>{}, wd[0], af[0]);
    static_for<8>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      if constexpr (j + 1 < 8) read(std::integral_constant<int, j + 1>{}, wd[(j + 1) & 1], af[(j + 1) & 1]);
      const f16x8 a = __builtin_bit_cast(f16x8, af[j & 1]);
      const f32x4 cb = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, nb, zero, 0, 0, 0);
      f32x4 cur[2];
#pragma unroll
      for (int r = 0; r < 2; ++r) cur[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, decode(wd[j & 1][r]), cb, 0, 0, 0);
      if constexpr (j > 0) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[r][e] = __builtin_fmaf(pend_s[r], pend[r][e], acc[r][e]);
      }
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        pend[r] = cur[r];
        pend_s[r] = scale_f32<j>(sv[r][j >> 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[r][e] = __builtin_fmaf(pend_s[r], pend[r][e], acc[r][e]);
  }

  // One FP8 step (128 inputs = one scale block along K): 4 groups of 32 inputs, lane (column c,
  // quarter q) holding inputs 32j + 8q .. +7 of group j; the 4 products of a set sum into a partial
  // in fp32, and acc += s * partial with the block's scale, read from lane `si` of fsc (each set's
  // scale of column block b, step k in lane b * ksteps + k).
  __device__ __forceinline__ void compute_fp8(char* const (&ring)[kD], int d, int si, const uint32_t (&fsc)[2],
                                              f32x4 (&acc)[2]) const {
    const int lane = threadIdx.x & 63, c = lane & 15, q = lane >> 4;
    const char* src = ring[d] + wave_off + c * kCodeRowB + 8 * (q & 1);
    const int ar = c & (kPassRows - 1);  // FP8 passes fill all 16 MFMA rows: no padding rows
    const char* arow = ring[d] + kCodesB + ar * kARowB;
    u32x2 wd[4][2];
    u32x4 af[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
        wd[j][r] = *reinterpret_cast<const u32x2*>(src + r * kSetCodeB + (((2 * j + (q >> 1)) ^ code_swz(c)) << 4));
      af[j] = *reinterpret_cast<const u32x4*>(arow + (a_pos<F>(ar, 4 * j + q) << 4));
    }
    f32x4 part[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 2; ++r)
        part[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, af[j]), decode_fp8(wd[j][r]),
                                                        part[r], 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const float s = __builtin_bit_cast(float, __builtin_amdgcn_readlane(fsc[r], si));
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[r][e] = __builtin_fmaf(s, part[r][e], acc[r][e]);
    }
  }

  // The K loop of one pass over CHAIN consecutive column blocks of ksteps steps each (one pipeline:
  // the loads of block b + 1's first steps are issued during block b's last steps; CHAIN > 1 needs
  // ksteps % kD == 0).  The token rows of a step are shared by the work-group's waves, so every
  // step starts with a barrier: after it, every wave's rows of this step have arrived and every
  // wave is done with the previous step's stage, whose rows are then refilled with those of the
  // step kD - 1 later (the stage's codes were refilled at the end of the previous step).  Loads past
  // the end read nothing, so the waits are fixed; steps past a block's end (CHAIN == 1 only) skip
  // the multiply.  Loads in issue order: ... rows(v), codes(v+1), rows(v+1), codes(v+2), ..., with
  // (4-bit) a scale block's scales just before the codes of its first step.
  // FP8: the pass's scales go to one register per set (lane b * ksteps + k), loaded first.
  template <int CHAIN>
  __device__ __forceinline__ void run(char* const (&ring)[kD], char* sc, int ksteps, f32x4 (&acc)[CHAIN][2]) const {
    u32x4 sr[2];
    uint32_t fsc[2];
    __builtin_amdgcn_s_barrier();  // the previous pass is done with the shared rows
    // the prologue in issue order, fenced against reordering (the waits below count on it)
    if constexpr (kQ4) {
      issue_scales(0, 0, CHAIN, sr);
    } else {
      const int lane = threadIdx.x & 63;
#pragma unroll
      for (int r = 0; r < 2; ++r)
        fsc[r] = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(sb[r], s_bytes), lane * 4, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    static_for<kD>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      int b2, k2;
      adv(0, 0, i, ksteps, b2, k2);
      issue_codes(ring, i, b2, k2, CHAIN);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (i + 1 < kD) issue_rows(ring, i, b2, k2, CHAIN);
      __builtin_amdgcn_sched_barrier(0);
    });
    // FP8: have the compiler wait for the scales here, where it can count the loads issued after
    // them (they arrive before the first codes anyway); left to the K loop, it loses count across
    // the column blocks and drains every load in flight at the first scale read
    if constexpr (!kQ4) asm volatile("" : "+v"(fsc[0]), "+v"(fsc[1]));
    static_for<CHAIN>([&](auto bc) {
      constexpr int b = decltype(bc)::value;
      for (int g = 0; g < ksteps; g += kD) {
        static_for<kD>([&](auto ic) {
          constexpr int i = decltype(ic)::value;
          const int k = g + i;
          // after rows(v): codes and rows of the next kD - 2 steps, the codes of the one after,
          // and (4-bit) a scale block's scales among them unless this step starts one
          wait_vmcnt<(kD - 1) * 4 + (kD - 2) * 1 + (i == 0 ? 0 : kScaleLoads)>();
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
          int b2, k2;
          adv(b, k, kD - 1, ksteps, b2, k2);
          issue_rows(ring, (i + kD - 1) % kD, b2, k2, CHAIN);
          if constexpr (kQ4 && i == 0) store_scales(sc, sr);  // this scale block, loaded a block ago
          if (k < ksteps) {
            if constexpr (kQ4)
              compute_q4(ring, i, sc, acc[b]);
            else
              compute_fp8(ring, i, __builtin_amdgcn_readfirstlane(b * ksteps + k), fsc, acc[b]);
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this stage's LDS reads are done
          if constexpr (kQ4 && i == 0) {
            adv(b, g, kD, ksteps, b2, k2);
            issue_scales(b2, k2, CHAIN, sr);
          }
          adv(b, k, kD, ksteps, b2, k2);
          issue_codes(ring, i, b2, k2, CHAIN);
        });
      }
    });
    wait_vmcnt<0>();  // the last loads past the end still write (zeros) into the ring
  }
};

// Column blocks per work-group of the down launch (a pipeline over 2 x 128 W_down rows): W_down's
// rows are short (I/256 4-bit steps, I/128 FP8 steps), so one block alone would mostly fill and
// drain the ring.
constexpr int kDownChain = 2;

template <QFormat F, bool SWIGLU, int CHAIN>
__device__ __forceinline__ void q_pass(const QArgs& p, char* const (&ring)[kD], char* sc, const QStream<F>& base,
                                       int n0, int64_t mb, int64_t r1) {
  constexpr int kPassRows = Fmt<F>::kPassRows;
  constexpr int kARowB = a_row_bytes<F>();
  constexpr int kRowLanes = kARowB / 16;  // lanes per token row of a wave's load
  constexpr int kParts = a_stage_bytes<F>() / 1024;  // 1 KiB parts of a step's rows (2 or 4 waves' loads)
  constexpr int kPartRows = kPassRows / kParts;
  const int H = p.H, I = p.I, K = SWIGLU ? H : I;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int part = wave % kParts;  // with 2 parts, waves w and w + 2 load the same one
  QStream<F> s = base;
  {  // this wave's row kPartRows * part + lane/kRowLanes, piece position lane % kRowLanes
    const int rl = kPartRows * part + lane / kRowLanes;
    const int64_t r = mb + rl;
    const int64_t rr = r < r1 ? r : mb;  // rows past the group end repeat its first row, never stored
    const int64_t src = SWIGLU ? (p.row_index ? (int64_t)p.row_index[rr] : rr) : rr;
    s.a_off = (uint32_t)(src * K * 2 + (a_pos<F>(rl, lane % kRowLanes) << 4));
  }
  s.a_dst = part * 1024;
  f32x4 acc[CHAIN][2];
#pragma unroll
  for (int b = 0; b < CHAIN; ++b) acc[b][0] = acc[b][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  s.template run<CHAIN>(ring, sc, K / Fmt<F>::kStepK, acc);

  // lane holds MFMA rows 4*(lane/16) + e, column n0 + lane%16 (+16 for set 1 of down, +128 per
  // further column block); the pass's rows are MFMA rows 0 .. kPassRows-1
  const int col = n0 + (lane & 15);
  const int64_t rend = mb + kPassRows < r1 ? mb + kPassRows : r1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t row = mb + 4 * (lane >> 4) + e;
    if ((lane >> 4) >= kPassRows / 4 || row >= rend) continue;
    if constexpr (SWIGLU) {
      // h in f16, each group of 8 columns in the operand order of the down matmul
      const _Float16 v = (_Float16)swiglu_f32(acc[0][0][e], acc[0][1][e]);
      static_cast<_Float16*>(p.out)[row * I + (col & ~7) + pair_pos(col & 7)] = v;
    } else {
      const float sc = p.row_scale ? p.row_scale[row] : 1.f;
#pragma unroll
      for (int b = 0; b < CHAIN; ++b)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const float v = acc[b][r][e] * sc;
          const int64_t at = row * H + col + 128 * b + 16 * r;
          if (p.out_bf16)
            static_cast<uint16_t*>(p.out)[at] = f32_to_bf16(v);
          else
            static_cast<float*>(p.out)[at] = v;
        }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// The shared expert (bf16 weights, bf16 token rows), streamed through the same ring by the first
// work-groups of the launch so that it overlaps the routed experts: a step covers 64 inputs (128
// bytes of each of a wave's 2 x 16 weight rows, swizzled as the codes are), passes of 32 rows.
constexpr int kShStepK = 64;
constexpr int kShNP = 2;  // 16-row MFMA blocks per pass

struct ShSlot {
  u32x4 a[kShNP][2];
};

struct ShStream {
  static constexpr int kLoads = 2 * 2 + 2 * kShNP;
  static_assert((kD - 1) * kLoads <= 63, "vmcnt");

  const void* wb[2];        // each set's 16 weight rows (uniform)
  const void* abase;
  uint32_t w_bytes, a_bytes;
  uint32_t c_off[2];        // lane offsets of the two direct loads of a set (row, swizzled chunk)
  uint32_t a_off[kShNP];    // lane offsets of its token-row fragments
  int wave_off;

  __device__ __forceinline__ void issue(char* const (&ring)[kD], int d, int st, int nsteps, ShSlot& sl) const {
    asm volatile("" : "+s"(st));
    const bool live = st < nsteps;
    const uint32_t wn = __builtin_amdgcn_readfirstlane(live ? w_bytes : 0u);
    const uint32_t an = __builtin_amdgcn_readfirstlane(live ? a_bytes : 0u);
    char* dst = ring[d] + wave_off;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const Rsrc rw = make_rsrc(wb[r], wn);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (LdsPtr)(dst + r * kSetCodeB + i * 1024), 16,
                                                 c_off[i] + (uint32_t)st * (2 * kShStepK), 0, 0, 2);
    }
    const Rsrc ra = make_rsrc(abase, an);
#pragma unroll
    for (int p = 0; p < kShNP; ++p)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        sl.a[p][j] = __builtin_amdgcn_raw_buffer_load_b128(ra, a_off[p] + (uint32_t)st * (2 * kShStepK) + 64 * j, 0, 0);
  }

  __device__ __forceinline__ void compute(char* const (&ring)[kD], int d, const ShSlot& sl,
                                          f32x4 (&acc)[kShNP][2]) const {
    const int lane = threadIdx.x & 63, c = lane & 15, q = lane >> 4;
    const char* src = ring[d] + wave_off + c * kCodeRowB;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(src + r * kSetCodeB + (((4 * j + q) ^ code_swz(c)) << 4));
#pragma unroll
        for (int p = 0; p < kShNP; ++p)
          acc[p][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, sl.a[p][j]), b, acc[p][r],
                                                             0, 0, 0);
      }
  }

  // As QStream::run, without scales.
  __device__ __forceinline__ void run(char* const (&ring)[kD], int nsteps, f32x4 (&acc)[kShNP][2]) const {
    ShSlot sl[kD];
    static_for<kD>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      issue(ring, i, i, nsteps, sl[i]);
    });
    for (int g = 0; g < nsteps; g += kD) {
      static_for<kD>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        wait_vmcnt<(kD - 1) * kLoads>();
        __builtin_amdgcn_sched_barrier(0);
        if (g + i < nsteps) compute(ring, i, sl[i], acc);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue(ring, i, g + i + kD, nsteps, sl[i]);
      });
    }
    wait_vmcnt<0>();
  }
};

// Work-group blk of the shared expert: output columns of 4 waves, every row of the expert.
template <bool SWIGLU>
__device__ __forceinline__ void shared_part(const QArgs& p, char* const (&ring)[kD], int blk) {
  const int H = p.H, I = p.I, K = SWIGLU ? H : I;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blk * (SWIGLU ? 64 : 128) + wave * (SWIGLU ? 16 : 32);
  const int64_t r0 = p.sh_offsets[0], r1 = p.sh_offsets[1];
  ShStream s;
  s.wb[0] = p.sh_w0 + (int64_t)n0 * K;
  s.wb[1] = SWIGLU ? p.sh_w1 + (int64_t)n0 * K : p.sh_w0 + (int64_t)(n0 + 16) * K;
  s.abase = p.sh_a;
  s.w_bytes = (uint32_t)(16 * K * 2);
  s.a_bytes = p.sh_a_bytes;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 8 * i + (lane >> 3);
    s.c_off[i] = (uint32_t)(row * K * 2 + (((lane & 7) ^ code_swz(row)) << 4));
  }
  s.wave_off = wave * kWaveB;
  const int col = n0 + (lane & 15);
  for (int64_t mb = r0; mb < r1; mb += 16 * kShNP) {
#pragma unroll
    for (int q = 0; q < kShNP; ++q) {
      const int64_t r = mb + 16 * q + (lane & 15);
      const int64_t rr = r < r1 ? r : mb;  // rows past the end repeat row mb, never stored
      const int64_t src = SWIGLU ? (int64_t)p.sh_row_index[rr] : rr;
      s.a_off[q] = (uint32_t)(src * K * 2 + (lane >> 4) * 16);
    }
    f32x4 acc[kShNP][2];
#pragma unroll
    for (int q = 0; q < kShNP; ++q) acc[q][0] = acc[q][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    s.run(ring, K / kShStepK, acc);
#pragma unroll
    for (int q = 0; q < kShNP; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = mb + 16 * q + 4 * (lane >> 4) + e;
        if (row >= r1) continue;
        if (SWIGLU) {
          static_cast<uint16_t*>(p.out)[row * I + col] = f32_to_bf16(swiglu_f32(acc[q][0][e], acc[q][1][e]));
        } else {
#pragma unroll
          for (int r = 0; r < 2; ++r) static_cast<uint16_t*>(p.out)[row * H + col + 16 * r] = f32_to_bf16(acc[q][r][e]);
        }
      }
  }
}

// The 4-bit scale buffer (LDS); FP8 has none, so that two FP8 work-groups fit a CU's LDS.
template <QFormat F>
struct ScaleBuf {
  __device__ static char* get() {
    __shared__ __align__(16) char sc[kWaves * kScaleWaveB];
    return sc;
  }
};
template <>
struct ScaleBuf<QFormat::kFp8> {
  __device__ static char* get() { return nullptr; }
};

template <QFormat F, bool SWIGLU, int CHAIN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void q_stream_kernel(QArgs p) {
  // one array per stage: the compiler then tells the stages' direct loads and LDS reads apart
  constexpr int kStageB = stage_bytes<F>();
  __shared__ __align__(16) char s0[kStageB], s1[kStageB], s2[kStageB], s3[kStageB];
  char* const sc = ScaleBuf<F>::get();
  static_assert(kD == 4, "one LDS array per ring stage");
  char* const ring[kD] = {s0, s1, s2, s3};

  if ((int)blockIdx.x < p.sh_blocks) {
    if (p.small_only && p.sh_offsets[1] - p.sh_offsets[0] > p.stream_rows) return;  // a tile-list group
#if defined(__HIP_DEVICE_COMPILE__)
    shared_part<SWIGLU>(p, ring, blockIdx.x);
#endif
    return;
  }
  static_assert(SWIGLU ? CHAIN == 1 : CHAIN >= 1, "column-block chains are for the down launch");
  const int bid = (int)blockIdx.x - p.sh_blocks;
  const int slot = (p.small_only ? p.counters[2] : 0) + bid / p.n_wg, nb = bid % p.n_wg;
  if (slot >= p.counters[0]) return;
  const int g = p.active[slot];
  if (g >= p.n_routed) return;
  int64_t r0 = p.group_offsets[g], r1 = p.group_offsets[g + 1];
  if (r0 > p.max_rows) r0 = p.max_rows;
  if (r1 > p.max_rows) r1 = p.max_rows;
  const int H = p.H, I = p.I, K = SWIGLU ? H : I, N = SWIGLU ? I : H;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // first output column of this wave (down: in the first of the work-group's CHAIN column blocks)
  const int n0 = nb * CHAIN * (SWIGLU ? 64 : 128) + wave * (SWIGLU ? 16 : 32);

  // rows of the two 16-row sets: gate and up rows n0.. (gate/up), or W_down rows n0.. and n0+16..
  const int64_t row0[2] = {n0, SWIGLU ? n0 : n0 + 16};
  const int64_t rowb = code_row_bytes<F>(K);  // bytes of codes per weight row
  const char* cm[2] = {static_cast<const char*>(p.codes0) + (int64_t)g * N * rowb,
                       static_cast<const char*>(SWIGLU ? p.codes1 : p.codes0) + (int64_t)g * N * rowb};
  const void* sm[2] = {p.scales0, SWIGLU ? p.scales1 : p.scales0};
  QStream<F> s;
#pragma unroll
  for (int r = 0; r < 2; ++r) s.cb[r] = cm[r] + row0[r] * rowb;
  s.abase = p.a;
  s.a_bytes = p.a_bytes;
  // column block b of this wave's rows starts 128 rows (down) further on; the descriptors span all
  s.blk_cb = (uint32_t)(128 * rowb);
  s.c_bytes = (uint32_t)((CHAIN - 1) * s.blk_cb + 16 * rowb);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 8 * i + (lane >> 3);  // lane's row in the 16-row set; its slot = chunk position
    s.c_off[i] = (uint32_t)(row * rowb + (((lane & 7) ^ code_swz(row)) << 4));
  }
  if constexpr (F == QFormat::kInt4) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
      s.sb[r] = static_cast<const uint16_t*>(sm[r]) + (int64_t)g * N * (K / 32) + row0[r] * (K / 32);
    s.blk_sb = (uint32_t)(128 * (K / 16));
    s.s_bytes = (uint32_t)((CHAIN - 1) * s.blk_sb + 16 * (K / 16));
    s.s_off = (uint32_t)((lane >> 2) * (K / 16) + (lane & 3) * 16);
  } else {
    // the scales of the wave's rows: block row n0/128 (+ b for column block b) of [N/128, K/128],
    // consecutive in memory, so lane b*ksteps + k reads element (n0/128) * ksteps + lane
    const int ksteps = K / Fmt<F>::kBlock;
#pragma unroll
    for (int r = 0; r < 2; ++r)
      s.sb[r] = static_cast<const float*>(sm[r]) + ((int64_t)g * (N / 128) + n0 / 128) * ksteps;
    s.s_bytes = (uint32_t)(CHAIN * ksteps * 4);
  }
  s.wave_off = wave * kWaveB;
  s.sc_wave_off = wave * kScaleWaveB;
#if defined(__HIP_DEVICE_COMPILE__)
  for (int64_t mb = r0; mb < r1; mb += Fmt<F>::kPassRows) q_pass<F, SWIGLU, CHAIN>(p, ring, sc, s, n0, mb, r1);
#else
  (void)s;
  (void)n0;
  (void)r0;
#endif
}

// bf16 rows -> f16 rows with each group of 8 inputs in the order 0,4,1,5,2,6,3,7 (one group per thread).
__global__ __launch_bounds__(256) void f16_rows_kernel(const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
                                                       int64_t n_groups) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_groups; i += stride)
    f16_group_pairs(x + 8 * i, y + 8 * i);
}

}  // namespace

hipError_t launch_f16_rows(const uint16_t* x, uint16_t* y, int64_t rows, int cols, hipStream_t s) {
  const int64_t n = rows * cols / 8;
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  f16_rows_kernel<<<(unsigned)blocks, 256, 0, s>>>(x, y, n);
  return hipGetLastError();
}

// Bytes of a [rows, cols] f16 operand, as a buffer record count (callers keep operands below 4 GiB).
static uint32_t operand_bytes(int64_t rows, int cols) {
  const int64_t b = rows * cols * 2;
  return b >= 0xffffffffLL ? 0xffffffffu : (uint32_t)b;
}

// Shared-expert fields of the launch arguments.
static void set_shared(QArgs& p, const SharedBf16* sh, bool swiglu, int H, int I) {
  p.sh_blocks = 0;
  if (!sh) return;
  p.sh_blocks = swiglu ? I / 64 : H / 128;
  p.sh_offsets = sh->offsets;
  p.sh_row_index = sh->row_index;
  p.sh_w0 = swiglu ? sh->gate : sh->down;
  p.sh_w1 = swiglu ? sh->up : nullptr;
  p.sh_a = swiglu ? sh->x : sh->h;
  p.sh_a_bytes = swiglu ? operand_bytes(sh->x_rows, H) : operand_bytes(sh->h_rows, I);
}

bool qshape_ok(QFormat f, int H, int I) {
  if (f == QFormat::kInt4) return H > 0 && I > 0 && H % 256 == 0 && I % 256 == 0;
  constexpr int kMax = Fmt<QFormat::kFp8>::kBlock * Fmt<QFormat::kFp8>::kMaxSteps;
  return H > 0 && I > 0 && H % 128 == 0 && I % 128 == 0 && H <= kMax && I <= kMax;
}

// Fields of a call that streams only the small groups (the tile kernels take the others).
static void set_small(QArgs& p, const Groups& g, int n_routed, bool small_only) {
  p.small_only = small_only ? 1 : 0;
  p.stream_rows = g.stream_rows;
  p.n_routed = n_routed;
}

hipError_t launch_gateup_q_stream(const Groups& g, const QWeights& w, const uint16_t* x16, int64_t x_rows,
                                  uint16_t* h16, const SharedBf16* sh, int H, int I, int n_routed, bool small_only,
                                  hipStream_t s) {
  if (!qshape_ok(w.format, H, I) || (small_only && g.stream_rows <= 0)) return hipErrorInvalidValue;
  QArgs p{g.group_offsets, g.row_index, g.active, g.counters, g.max_rows, w.gate_codes, w.gate_scales,
          w.up_codes, w.up_scales, x16, operand_bytes(x_rows, H), h16, 0, nullptr, H, I, I / 64};
  set_shared(p, sh, true, H, I);
  set_small(p, g, n_routed, small_only);
  const unsigned grid = (unsigned)(p.sh_blocks + (int64_t)g.n_groups * p.n_wg);  // one slot per listed group
  if (w.format == QFormat::kInt4)
    q_stream_kernel<QFormat::kInt4, true, 1><<<grid, 256, 0, s>>>(p);
  else
    q_stream_kernel<QFormat::kFp8, true, 1><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_down_q_stream(const Groups& g, const QWeights& w, const uint16_t* h16, uint16_t* y_rows,
                                const SharedBf16* sh, int H, int I, int n_routed, bool small_only, hipStream_t s) {
  if (!qshape_ok(w.format, H, I) || (small_only && g.stream_rows <= 0)) return hipErrorInvalidValue;
  const bool q4 = w.format == QFormat::kInt4;
  // chained column blocks when they divide the columns and the K steps fill whole 4-bit scale
  // blocks (FP8: while the chain's scales fit one register)
  const int ksteps = I / (q4 ? Fmt<QFormat::kInt4>::kStepK : Fmt<QFormat::kFp8>::kStepK);
  const bool chain = (H / 128) % kDownChain == 0 && ksteps % kD == 0 &&
                     (q4 || kDownChain * ksteps <= Fmt<QFormat::kFp8>::kMaxSteps);
  QArgs p{g.group_offsets, nullptr, g.active, g.counters, g.max_rows, w.down_codes, w.down_scales, nullptr,
          nullptr, h16, operand_bytes(g.max_rows, I), y_rows, 1, nullptr, H, I, H / 128 / (chain ? kDownChain : 1)};
  set_shared(p, sh, false, H, I);
  set_small(p, g, n_routed, small_only);
  const unsigned grid = (unsigned)(p.sh_blocks + (int64_t)g.n_groups * p.n_wg);  // one slot per listed group
  if (q4) {
    if (chain)
      q_stream_kernel<QFormat::kInt4, false, kDownChain><<<grid, 256, 0, s>>>(p);
    else
      q_stream_kernel<QFormat::kInt4, false, 1><<<grid, 256, 0, s>>>(p);
  } else {
    if (chain)
      q_stream_kernel<QFormat::kFp8, false, kDownChain><<<grid, 256, 0, s>>>(p);
    else
      q_stream_kernel<QFormat::kFp8, false, 1><<<grid, 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace moe
