// Shared machinery of the tile GEMMs (gemm_tile.hip: bf16 and FP8 weights; gemm_tile_q4.hip: 4-bit
// weights): work-item dealing, LDS rings, direct loads, the bf16 K loop and work items (also used for
// the shared expert's tiles beside quantized routed experts), and the K-step schedule of the
// quantized tiles, generic over the weight format.
//
// Grouped SwiGLU expert GEMMs for many rows per expert (prefill-like shapes), bf16 MFMA.
//
// The experts are the SwiGLU FFNs of "Kimi K2.5 模型架构深度拆解" §4.3 / §10.2 Steps 5-6
// (gate + up -> SiLU -> multiply -> down), batched over experts as the grouped GEMM that
// "Kimi K2.5 架构 QA" Q8.3 names in place of the per-expert loop.
//
// Work item = (row tile of one group, column slab; for down with few row tiles also a K range,
// whose fp32 partial sums a second kernel adds in K order).  Row tiles come from the device-side plan
// (largest groups first, kTileM = 256 rows each, so a K2 expert's ~170 prefill rows are one tile
// and every weight byte is read from HBM once).  A tile is up to 256 token rows x 256 weight rows
// (gate/up: the gate and up rows of 128 h columns; down: 256 output columns), K in steps of 64.
//
// Both operands reach the matrix cores through LDS, loaded with gfx950's direct global -> LDS
// loads (buffer_load_dwordx4 ... lds): one instruction moves 8 rows x 128 contiguous bytes (whole
// cache lines).  On MI355X that form moves ~54 B/clk per CU from L2, against ~16 B/clk for loads
// straight into MFMA operand registers (16 rows x 64 bytes per instruction, the operand layout),
// which would spend as long on a step's 32 KiB of weights as the step's MFMAs take.
//   * LDS: two stages of token rows (A) and three of weight rows (B), 5 x 32 KiB = 160 KiB, each
//     stage its own __shared__ array, the K loop unrolled by 6 so every access names its stage
//     statically (the compiler can then tell which LDS reads depend on which direct loads).  A is
//     loaded one step ahead (it comes from L2), B two steps ahead (it streams from HBM).
//   * 8 waves in a 2 (rows) x 4 (columns) grid; a wave owns 64 weight rows and every other 16-row
//     block of the token rows (blocks wr, wr+2, ...), so the two wave rows split any row count
//     evenly.  Each A fragment read from LDS feeds 4 v_mfma_f32_16x16x32_bf16 and each B fragment
//     up to 8; accumulators stay in VGPRs (at most 128), two waves per SIMD.
//   * LDS rows are 128 bytes, unpadded; 16-byte chunk c of row r sits at c ^ ((r >> 1) & 7), so the
//     16 rows one 16-lane group reads fall in 16 different bank groups.  A load lane picks the
//     global chunk that belongs in its LDS slot, so every load still reads whole row segments.
//   * The K loop is instantiated per (16-row blocks of this wave, A loads per wave), chosen outside
//     the loop: padding rows cost no MFMA and A rows past the group's last 16-row block are not
//     loaded.  One barrier per K step (LDS traffic only; the loads in flight stay in flight).
//   * Outputs leave through LDS (the free rings), as whole 16-byte chunks of contiguous rows.
// Row tiles are dealt round-robin to the XCDs; the column slabs of one row tile run on the same XCD at
// the same time and share its rows of A in that XCD's L2.
#pragma once

#include <type_traits>

#include "tile_core.h"

namespace moe {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512, kWaves = 8;
constexpr int kBK = 64;                              // k per step
constexpr int kRowBytes = kBK * 2;                   // one row of one step in LDS
constexpr int kTileN = 256;                          // weight rows per tile
constexpr int kStageBytes = 256 * kRowBytes;         // 32 KiB: 256 rows of one step
constexpr int kBLoads = kTileN * kRowBytes / 1024 / kWaves;  // B pieces (8 rows) per wave per step: 4
constexpr int kMaxBlk = kTileM / 32;                 // 16-row blocks per wave row: 8
static_assert(kTileM == 256 && kRowBytes == 128 && kBLoads == 4, "tile shape");

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

struct TileArgs {
  const int32_t* group_offsets;
  const int32_t* row_index;
  const int32_t* tiles;
  const int32_t* counters;
  int64_t max_rows;
  Weights w;
  const uint16_t* a;
  void* out;
  int out_bf16;
  const float* row_scale;
  int H, I, n_ntiles;
  int n_ksplit;  // down: K ranges per output tile (partial sums go to part, then a reduction kernel)
  float* part;   // [n_ksplit, max_rows, H] fp32 when n_ksplit > 1
  int tile_m;    // rows per row tile of the plan (kTileM; kTileMFp8 or kTileMQ4 for the quantized tiles)
};

struct TileRows {
  int g;
  int64_t rbeg, rend;
};

// Work-group -> (row tile, column slab nt, K range ks).  The hardware hands work-group b to XCD b % 8;
// the plan's tile list (largest groups first, a group's tiles consecutive) is cut into blocks of
// kGroupTiles consecutive tiles, dealt to the XCDs round-robin (block c to XCD c % 8, so every XCD gets
// the same mix of large and small groups, and the tiles of a group of many rows share blocks; with
// fewer than 8 blocks, single tiles are dealt round-robin and an XCD's blocks are every 8th tile).  A block of tiles of one group (a group of many rows) runs
// slab by slab, its tiles side by side, so the work-groups reading a weight slab run together and share
// it in the XCD's L2 (instead of the slab being streamed again for every row tile); any other block
// runs tile by tile, a tile's slabs side by side, sharing the tile's token rows in L2.  With fewer
// tiles than XCDs the tiles' items are spread over all XCDs instead.
constexpr int kGroupTiles = 4;

__device__ __forceinline__ bool tile_of(const TileArgs& p, int& nt, int& ks, TileRows& t) {
  const int per_tile = p.n_ntiles * p.n_ksplit;
  const int64_t b = blockIdx.x, local = b / kXcds, x = b % kXcds;
  const int64_t n_tiles = p.counters[1];
  int64_t tile64;
  int rem;
  if (n_tiles < kXcds) {
    // fewer row tiles than XCDs: each tile's items are cut into c chunks dealt round-robin, so that
    // every XCD has work (unit u = chunk u % c of tile u / c goes to XCD u % 8)
    if (n_tiles <= 0) return false;
    const int c = (int)((kXcds + n_tiles - 1) / n_tiles) < per_tile ? (int)((kXcds + n_tiles - 1) / n_tiles) : per_tile;
    const int cs = (per_tile + c - 1) / c;
    const int64_t u = (local / cs) * kXcds + x;
    rem = (int)((u % c) * cs + local % cs);
    tile64 = u / c;
    if (tile64 >= n_tiles || rem >= per_tile) return false;
  } else {
    const int64_t blk = local / ((int64_t)kGroupTiles * per_tile);  // block of this XCD's tiles
    const int q = (int)(local % ((int64_t)kGroupTiles * per_tile));
    // tile i of the block: kGroupTiles consecutive tiles of the list once every XCD gets a whole
    // block; with fewer tiles single tiles go round-robin (XCD-local tile j is tile j * 8 + x)
    const bool chunked = n_tiles >= (int64_t)kXcds * kGroupTiles;
    const auto tile_at = [&](int i) -> int64_t {
      return chunked ? (blk * kXcds + x) * kGroupTiles + i : (blk * kGroupTiles + i) * kXcds + x;
    };
    int in_blk = 0;  // tiles of the block
    bool one_group = true;
    for (int i = 0; i < kGroupTiles; ++i) {
      const int64_t ti = tile_at(i);
      if (ti >= n_tiles) break;
      ++in_blk;
      if (p.tiles[2 * ti] != p.tiles[2 * tile_at(0)]) one_group = false;
    }
    int j;
    if (one_group && in_blk == kGroupTiles) {
      j = q % kGroupTiles;
      rem = q / kGroupTiles;
    } else {
      j = q / per_tile;
      rem = q % per_tile;
    }
    if (j >= in_blk) return false;
    tile64 = tile_at(j);
  }
  const int tile = (int)tile64;
  nt = rem / p.n_ksplit;
  ks = rem % p.n_ksplit;
  t.g = p.tiles[2 * tile];
  const int m0 = p.tiles[2 * tile + 1];
  int64_t r0 = p.group_offsets[t.g], r1 = p.group_offsets[t.g + 1];
  if (r0 > p.max_rows) r0 = p.max_rows;
  if (r1 > p.max_rows) r1 = p.max_rows;
  if (r1 < r0) r1 = r0;
  t.rbeg = r0 + m0;
  t.rend = t.rbeg + p.tile_m < r1 ? t.rbeg + p.tile_m : r1;
  return t.rbeg < t.rend;
}

// The two LDS rings.
struct Rings {
  char* a[2];
  char* b[3];
};

// Direct-load addressing: uniform bases plus 32-bit per-lane byte offsets (operands stay below 4 GiB);
// a lane offset already names the row and the chunk that belongs in the lane's LDS slot.
struct Loads {
  const char* a_base;
  uint32_t a_off[4];         // A pieces w, w + 8, ... (the first NAL of them are loaded)
  const char* b_base[kBLoads];  // B piece w + 8j: its weight tensor (uniform)
  uint32_t b_off[kBLoads];
  int skew, nk;              // step kt loads K step (kt + skew) mod nk (uniform over the work-group)
  int wave;                  // w, uniform: the LDS destinations derive from it, not from threadIdx
};

typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef __attribute__((address_space(3))) void* LdsPtr;

// Buffer descriptor over an operand (a uniform base; the byte offsets stay below 4 GiB).  The direct
// loads go through buffer descriptors rather than global addresses: the compiler counts a
// global -> LDS load as possibly touching LDS through the flat path as well, and then waits for every
// LDS read in flight (lgkmcnt(0)) wherever it needs one of them.
__device__ __forceinline__ Rsrc operand_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)0xffffffffu, 0x00020000);
}

__device__ __forceinline__ uint32_t kbytes(const Loads& o, int kt) {
  int k = kt + o.skew;
  if (k >= o.nk) k -= o.nk;
  return (uint32_t)k * kRowBytes;
}

template <int NAL>
__device__ __forceinline__ void issue_a(const Loads& o, int kt, char* stage) {
  const int w = o.wave;
  const uint32_t kb = kbytes(o, kt);
  const Rsrc rs = operand_rsrc(o.a_base);
#pragma unroll
  for (int j = 0; j < NAL; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LdsPtr)(stage + (w + kWaves * j) * 1024), 16, o.a_off[j] + kb, 0, 0,
                                             0);
}

__device__ __forceinline__ void issue_b(const Loads& o, int kt, char* stage) {
  const int w = o.wave;
  const uint32_t kb = kbytes(o, kt);
#pragma unroll
  for (int j = 0; j < kBLoads; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(operand_rsrc(o.b_base[j]), (LdsPtr)(stage + (w + kWaves * j) * 1024), 16,
                                             o.b_off[j] + kb, 0, 0, 0);
}

// Per-wave LDS read geometry: lane l reads row (l & 15) of a 16-row block at logical chunk
// 4 kk + (l >> 4); the chunk's position is the same in every 16-row block.
struct Frag {
  uint32_t off[2];      // byte offset inside a block for k-substep kk = 0, 1
  uint32_t a_row0;      // byte offset of this wave's first A block (blocks wr, wr + 2, ...)
  uint32_t b_row0[4];   // byte offset of B column block s of this wave
};

// MFMAs of one K step: NBW 16-row blocks x 4 column blocks x 2 k-substeps, as one sequence of 2 NBW
// fragments (fragment fi: k-substep fi / NBW, row block fi % NBW).  The weight fragment is the MFMA's
// first operand, so acc[i][s] holds the block transposed: lane l, element e = token row
// 16 (wr + 2i) + (l & 15), column 4 (l >> 4) + e of column block s (4 consecutive columns per lane,
// which the epilogues write as one 8-byte piece).  Each A fragment is read from LDS
// two fragments ahead of its MFMAs and the second k-substep's 4 B fragments two fragments before
// that substep starts, in a fixed order (a scheduling barrier after each fragment's MFMAs), so each
// LDS read has 8 MFMAs to land behind.
template <int NBW>
__device__ __forceinline__ void compute_step(const char* As, const char* Bs, const Frag& f, f32x4 (&acc)[NBW > 0 ? NBW : 1][4]) {
  if constexpr (NBW > 0) {
    constexpr int NF = 2 * NBW;
    constexpr int kB1 = NBW >= 2 ? NBW - 2 : 0;  // fragment before whose MFMAs the second B set is read
    auto read_a = [&](int fi) {
      return *reinterpret_cast<const bf16x8*>(As + f.a_row0 + f.off[fi / NBW] + (fi % NBW) * 2 * 16 * kRowBytes);
    };
    bf16x8 b[2][4];
    bf16x8 a[NF];
#pragma unroll
    for (int s = 0; s < 4; ++s) b[0][s] = *reinterpret_cast<const bf16x8*>(Bs + f.b_row0[s] + f.off[0]);
    a[0] = read_a(0);
    a[1] = read_a(1);
#pragma unroll
    for (int fi = 0; fi < NF; ++fi) {
      if (fi + 2 < NF) a[fi + 2] = read_a(fi + 2);
      if (fi == kB1) {
#pragma unroll
        for (int s = 0; s < 4; ++s) b[1][s] = *reinterpret_cast<const bf16x8*>(Bs + f.b_row0[s] + f.off[1]);
      }
      const int kk = fi / NBW, i = fi % NBW;
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[i][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[kk][s], a[fi], acc[i][s], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    (void)As;
    (void)Bs;
    (void)f;
    (void)acc;
  }
}

// One K step kt (kt % 6 == D): wait for this wave's loads of A(kt) and B(kt), barrier (everyone's
// have landed; everyone is done with step kt-1's stages), load A(kt+1) into the A stage step kt-1
// used and B(kt+2) into the B stage step kt-1 used, multiply.  Per wave the vector-memory order is
// B(0) A(0) B(1) | A(1) B(2) | A(2) B(3) | ...: when step kt starts, only B(kt+1) (kBLoads ops, when it
// exists) may still be in flight.
template <int NBW, int NAL, int D, bool kTail>
__device__ __forceinline__ void kstep(const Loads& o, int kt, int nk, const Rings& r, const Frag& f,
                                      f32x4 (&acc)[NBW > 0 ? NBW : 1][4]) {
  if (!kTail || kt + 1 < nk)
    wait_vmcnt<kBLoads>();
  else
    wait_vmcnt<0>();
  block_sync_lds();
  if (!kTail || kt + 1 < nk) issue_a<NAL>(o, kt + 1, r.a[(D + 1) % 2]);
  if (!kTail || kt + 2 < nk) issue_b(o, kt + 2, r.b[(D + 2) % 3]);
  __builtin_amdgcn_sched_barrier(0);
  compute_step<NBW>(r.a[D % 2], r.b[D % 3], f, acc);
  __builtin_amdgcn_sched_barrier(0);
}

template <int NBW, int NAL>
__device__ __forceinline__ void kloop(const Loads& o, int nk, const Rings& r, const Frag& f,
                                      f32x4 (&acc)[NBW > 0 ? NBW : 1][4]) {
  // prologue in the steady state's issue order (the loads into b0, a0, b1 in that order, as the two
  // steps before the loop head issue them), fenced against reordering: with another order the
  // compiler's wait before the loop head's first LDS read drains every load in flight
  issue_b(o, 0, r.b[0]);
  __builtin_amdgcn_sched_barrier(0);
  issue_a<NAL>(o, 0, r.a[0]);
  __builtin_amdgcn_sched_barrier(0);
  if (nk > 1) issue_b(o, 1, r.b[1]);
  __builtin_amdgcn_sched_barrier(0);
  // step 0 is peeled off: with the loop head at a step that the prologue does not lead into, the
  // compiler's wait before the head's first LDS read no longer drains every load in flight
  kstep<NBW, NAL, 0, true>(o, 0, nk, r, f, acc);
  int kt = 1;
  // steady state: every load these six steps issue exists (kt + 7 < nk)
  for (; kt + 8 <= nk; kt += 6) {
    kstep<NBW, NAL, 1, false>(o, kt, nk, r, f, acc);
    kstep<NBW, NAL, 2, false>(o, kt + 1, nk, r, f, acc);
    kstep<NBW, NAL, 3, false>(o, kt + 2, nk, r, f, acc);
    kstep<NBW, NAL, 4, false>(o, kt + 3, nk, r, f, acc);
    kstep<NBW, NAL, 5, false>(o, kt + 4, nk, r, f, acc);
    kstep<NBW, NAL, 0, false>(o, kt + 5, nk, r, f, acc);
  }
  // the last 0 .. 6 steps (or all of a short loop); kt % 6 == 1 here
  while (kt < nk) {
    kstep<NBW, NAL, 1, true>(o, kt, nk, r, f, acc);
    if (++kt == nk) break;
    kstep<NBW, NAL, 2, true>(o, kt, nk, r, f, acc);
    if (++kt == nk) break;
    kstep<NBW, NAL, 3, true>(o, kt, nk, r, f, acc);
    if (++kt == nk) break;
    kstep<NBW, NAL, 4, true>(o, kt, nk, r, f, acc);
    if (++kt == nk) break;
    kstep<NBW, NAL, 5, true>(o, kt, nk, r, f, acc);
    if (++kt == nk) break;
    kstep<NBW, NAL, 0, true>(o, kt, nk, r, f, acc);
    ++kt;
  }
}

template <int NBW, int NAL, class Epilogue>
__device__ __forceinline__ void tile_body(const Loads& o, const Rings& r, const Frag& f, const Epilogue& epilogue) {
  f32x4 acc[NBW > 0 ? NBW : 1][4];
#pragma unroll
  for (int i = 0; i < (NBW > 0 ? NBW : 1); ++i)
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[i][s] = f32x4{0.f, 0.f, 0.f, 0.f};
  kloop<NBW, NAL>(o, o.nk, r, f, acc);
  epilogue(std::integral_constant<int, NBW>{}, acc);
}

// body(NBW, NAL) for the (16-row blocks of this wave, A loads per wave) pair of a tile of nblk 16-row
// blocks: wave row wr takes ceil((nblk - wr) / 2) of them, and the 2 nblk A pieces of 8 rows are spread
// over the 8 waves, ceil(nblk / 4) each.  One instance per pair that a row count of 1 .. 32 kMaxNbw
// produces (only those: the kernel's registers are the largest instance's); device pass only (these
// instances are device code).
template <int kMaxNbw = 8, class Body>
__device__ __forceinline__ void run_tile(int nblk, int wr, const Body& body) {
  const int nbw = (nblk - wr + 1) / 2;
  const int nal = (nblk + 3) / 4;
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int kMaxNal = (2 * kMaxNbw + 3) / 4;
#define MOE_TILE_CASE(B, A)                                                                                    \
  if constexpr (B <= kMaxNbw && A <= kMaxNal) {                                                                \
    if (nbw == B && nal == A) return body(std::integral_constant<int, B>{}, std::integral_constant<int, A>{}); \
  }
  MOE_TILE_CASE(8, 4)
  MOE_TILE_CASE(7, 4)
  MOE_TILE_CASE(6, 4)
  MOE_TILE_CASE(6, 3)
  MOE_TILE_CASE(5, 3)
  MOE_TILE_CASE(4, 3)
  MOE_TILE_CASE(4, 2)
  MOE_TILE_CASE(3, 2)
  MOE_TILE_CASE(2, 2)
  MOE_TILE_CASE(2, 1)
  MOE_TILE_CASE(1, 1)
  MOE_TILE_CASE(0, 1)
#undef MOE_TILE_CASE
#else
  (void)body;
  (void)nbw;
  (void)nal;
#endif
}

// Output tiles leave through LDS so that global stores are whole 16-byte chunks of contiguous rows.
// A bf16 tile of kCols columns is staged over the free ring arrays in order (a0, a1, b0, b1, b2),
// kRowsPer rows each; 16-byte chunk c of row r at position c ^ out_swz(r).  A row is 256 or 512 bytes,
// so position p of any row lies in bank group p mod 16: the 16 consecutive rows of an 8-byte staging
// write (transposed accumulators), the 4 rows 4 apart of a 2-byte write (plain order) and the chunks
// of one row that a store reads all fall in distinct bank groups.
__device__ __forceinline__ int out_swz(int r) { return r & 15; }

template <int kCols>
struct OutTile {
  static constexpr int kRowB = kCols * 2;
  static constexpr int kRowsPer = kStageBytes / kRowB;
  static constexpr int kChunks = kRowB / 16;
  static_assert(kRowsPer % 16 == 0 && kRowsPer * 5 >= kTileM, "staging");

  __device__ static __forceinline__ char* stage(const Rings& r, int i) {
    return i == 0 ? r.a[0] : i == 1 ? r.a[1] : i == 2 ? r.b[0] : i == 3 ? r.b[1] : r.b[2];
  }
  __device__ static __forceinline__ void put(const Rings& r, int row, int col, float v) {
    char* st = stage(r, row / kRowsPer);
    *reinterpret_cast<uint16_t*>(st + (row % kRowsPer) * kRowB + (((col >> 3) ^ out_swz(row)) << 4) + (col & 7) * 2) =
        f32_to_bf16(v);
  }
  // columns col .. col + 3 (col a multiple of 4) of a row: one 8-byte write
  __device__ static __forceinline__ void put4(const Rings& r, int row, int col, const float (&v)[4]) {
    char* st = stage(r, row / kRowsPer);
    const uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    *reinterpret_cast<u32x2*>(st + (row % kRowsPer) * kRowB + (((col >> 3) ^ out_swz(row)) << 4) + (col & 7) * 2) =
        u32x2{lo, hi};
  }
  // binary16, column c at position (c & ~7) | pair_pos(c & 7) (the operand order of the quantized tiles)
  __device__ static __forceinline__ void put_f16_pairs(const Rings& r, int row, int col, float v) {
    char* st = stage(r, row / kRowsPer);
    const int c = (col & ~7) | (((col & 3) << 1) | ((col >> 2) & 1));
    *reinterpret_cast<_Float16*>(st + (row % kRowsPer) * kRowB + (((c >> 3) ^ out_swz(row)) << 4) + (c & 7) * 2) =
        (_Float16)v;
  }
  // rows [0, m_valid) of the staged tile -> out[(rbeg + r) * ld + col0 + ...], columns below col_end
  __device__ static __forceinline__ void store(const Rings& r, int m_valid, uint16_t* out, int64_t ld, int64_t rbeg,
                                               int col0, int col_end) {
    const int n = m_valid * kChunks;
    for (int ch = threadIdx.x; ch < n; ch += kThreads) {
      const int row = ch / kChunks, c = ch % kChunks;
      if (col0 + 8 * c >= col_end) continue;
      const char* st = stage(r, row / kRowsPer);
      const u32x4 v = *reinterpret_cast<const u32x4*>(st + (row % kRowsPer) * kRowB + ((c ^ out_swz(row)) << 4));
      *reinterpret_cast<u32x4*>(out + (rbeg + row) * ld + col0 + 8 * c) = v;
    }
  }
};

// Lane offsets of this wave's A pieces: piece p = w + 8 j holds tile rows 8p .. 8p + 7; row rl of the
// tile is source row src(rl) of a [*, K] matrix.
template <class RowOf>
__device__ __forceinline__ void a_offsets(Loads& o, int K, RowOf row_of) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int rl = (w + kWaves * j) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(rl);  // the chunk that belongs in this lane's LDS slot
    o.a_off[j] = (uint32_t)((row_of(rl) * K + 8 * chunk) * 2);
  }
}

// Lane offset of B piece j (tile rows 8p .. 8p + 7, p = w + 8 j) inside its weight tensor, whose row
// rl sits at weight row wrow(rl) (rows K elements long).
__device__ __forceinline__ uint32_t b_offset(int j, int64_t wrow, int K) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rl = (w + kWaves * j) * 8 + (lane >> 3);
  const int chunk = (lane & 7) ^ swz(rl);
  return (uint32_t)((wrow * K + 8 * chunk) * 2);
}

__device__ __forceinline__ Frag make_frag(int wr, const int (&b_rows)[4]) {
  const int lane = threadIdx.x & 63, x = lane & 15, g = lane >> 4;
  Frag f;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) f.off[kk] = (uint32_t)(x * kRowBytes + (((4 * kk + g) ^ swz(x)) << 4));
  f.a_row0 = (uint32_t)(wr * 16 * kRowBytes);
#pragma unroll
  for (int s = 0; s < 4; ++s) f.b_row0[s] = (uint32_t)(b_rows[s] * kRowBytes);
  return f;
}

#define MOE_TILE_SMEM                                                                                          \
  __shared__ __align__(16) char a0_[kStageBytes], a1_[kStageBytes], b0_[kStageBytes], b1_[kStageBytes], \
      b2_[kStageBytes];                                                                                        \
  const Rings rings{{a0_, a1_}, {b0_, b1_, b2_}};

// Gate/up work item (row tile t, h columns nt*128 ..): h rows in bf16.
__device__ __forceinline__ void gateup_bf16_item(const TileArgs& p, const Rings& rings, int nt, const TileRows& t) {
  const int H = p.H, I = p.I;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = w >> 2, wc = w & 3;  // wave row (token-row blocks wr, wr + 2, ...), wave column
  const bool sh = t.g == p.w.shared_group;
  const uint16_t* wg = sh ? (const uint16_t*)p.w.s_gate : (const uint16_t*)p.w.gate + (int64_t)t.g * I * H;
  const uint16_t* wu = sh ? (const uint16_t*)p.w.s_up : (const uint16_t*)p.w.up + (int64_t)t.g * I * H;
  const int h0 = nt * 128;  // first h column of the tile; B tile rows 0-127 gate, 128-255 up

  Loads o;
  o.wave = w;
  o.a_base = reinterpret_cast<const char*>(p.a);
  a_offsets(o, H, [&](int rl) -> int64_t {
    const int64_t r = t.rbeg + rl;
    const int64_t rr = r < t.rend ? r : t.rbeg;  // rows past the group end re-read its first row
    return p.row_index ? (int64_t)p.row_index[rr] : rr;
  });
#pragma unroll
  for (int j = 0; j < kBLoads; ++j) {  // pieces w, w + 8 are gate rows, w + 16, w + 24 up rows
    const int rl = (w + kWaves * j) * 8 + (lane >> 3);
    o.b_base[j] = reinterpret_cast<const char*>(j < 2 ? wg : wu);
    o.b_off[j] = b_offset(j, h0 + (rl & 127), H);
  }
  o.nk = H / kBK;
  o.skew = 0;  // 14,336-byte rows (K2) spread over the channels on their own

  // wave column wc: gate rows 32 wc .. +32 (blocks 0, 1) and the up rows of the same h columns
  const int b_rows[4] = {32 * wc, 32 * wc + 16, 128 + 32 * wc, 128 + 32 * wc + 16};
  const Frag f = make_frag(wr, b_rows);
  uint16_t* h = static_cast<uint16_t*>(p.out);
  const int64_t rbeg = t.rbeg;
  const int m_valid = (int)(t.rend - t.rbeg);
  const auto epilogue = [&](auto nbw_c, const auto& acc) {
    constexpr int NBW = decltype(nbw_c)::value;
    using Out = OutTile<128>;
    block_sync_lds();  // every wave is done reading the rings
    static_for<NBW>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int row = 16 * (wr + 2 * i) + (lane & 15);
#pragma unroll
      for (int s = 0; s < 2; ++s) {  // gate block s and up block s + 2 hold the same h columns
        float hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] = swiglu_f32(acc[i][s][e], acc[i][s + 2][e]);
        Out::put4(rings, row, 32 * wc + 16 * s + 4 * (lane >> 4), hv);
      }
    });
    block_sync_lds();
    Out::store(rings, m_valid, h, I, rbeg, h0, I);
  };
  run_tile((m_valid + 15) / 16, wr, [&](auto b, auto a) {
    tile_body<decltype(b)::value, decltype(a)::value>(o, rings, f, epilogue);
  });
}

// Down work item (row tile t, output columns nt*256 .., K range ks).
__device__ __forceinline__ void down_bf16_item(const TileArgs& p, const Rings& rings, int nt, int ks,
                                               const TileRows& t) {
  const int H = p.H, I = p.I;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = w >> 2, wc = w & 3;
  const uint16_t* wd = t.g == p.w.shared_group ? (const uint16_t*)p.w.s_down
                                                : (const uint16_t*)p.w.down + (int64_t)t.g * H * I;
  const int n0 = nt * 256;  // first output column of the tile

  // this item's K range [k0, k0 + kc) of the h rows and of W_down's rows
  const int kc = I / p.n_ksplit, k0 = ks * kc;
  Loads o;
  o.wave = w;
  o.a_base = reinterpret_cast<const char*>(p.a + k0);
  a_offsets(o, I, [&](int rl) -> int64_t {
    const int64_t r = t.rbeg + rl;
    return r < t.rend ? r : t.rbeg;
  });
#pragma unroll
  for (int j = 0; j < kBLoads; ++j) {  // output columns past H (the last slab of an H that is not a
    const int rl = (w + kWaves * j) * 8 + (lane >> 3);  // multiple of 256) re-read row n0, never stored
    o.b_base[j] = reinterpret_cast<const char*>(wd + k0);
    o.b_off[j] = b_offset(j, n0 + rl < H ? n0 + rl : n0, I);
  }
  // W_down rows a multiple of 4 KiB apart put the same K step of all 256 rows on few HBM channels:
  // the column slabs then start their K loops at different steps (and wrap around).  Only while the
  // tile's block of h for this K range is small (kc <= 4096: at most 2 MiB): the slabs of a tile
  // share it through L2 only while they walk K together.
  o.nk = kc / kBK;
  o.skew = (I * 2) % 4096 == 0 && kc <= 4096 ? nt * 5 % o.nk : 0;

  const int b_rows[4] = {64 * wc, 64 * wc + 16, 64 * wc + 32, 64 * wc + 48};
  const Frag f = make_frag(wr, b_rows);
  const int64_t rbeg = t.rbeg, rend = t.rend;
  const int m_valid = (int)(rend - rbeg);
  const float* row_scale = p.row_scale;
  const bool split = p.n_ksplit > 1;
  void* out = split ? static_cast<void*>(p.part + (int64_t)ks * p.max_rows * H) : p.out;
  const auto epilogue = [&](auto nbw_c, const auto& acc) {
    constexpr int NBW = decltype(nbw_c)::value;
    if (p.out_bf16 && !split) {
      using Out = OutTile<256>;
      block_sync_lds();  // every wave is done reading the rings
      static_for<NBW>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const int row = 16 * (wr + 2 * i) + (lane & 15);
        const float sc = row_scale && row < m_valid ? row_scale[rbeg + row] : 1.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float v[4] = {acc[i][s][0] * sc, acc[i][s][1] * sc, acc[i][s][2] * sc, acc[i][s][3] * sc};
          Out::put4(rings, row, 64 * wc + 16 * s + 4 * (lane >> 4), v);
        }
      });
      block_sync_lds();
      Out::store(rings, m_valid, static_cast<uint16_t*>(out), H, rbeg, n0, H);
      return;
    }
    // fp32 rows (a caller's choice in moe_grouped_swiglu, or a K range's partial sums): direct stores
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      const int64_t r = rbeg + 16 * (wr + 2 * i) + (lane & 15);
      if (r >= rend) continue;
      const float sc = row_scale ? row_scale[r] : 1.f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {  // 4 consecutive columns: all below H or none (H is a multiple of 128)
        const int col = n0 + 64 * wc + 16 * s + 4 * (lane >> 4);
        if (col < H)
          *reinterpret_cast<f32x4*>(static_cast<float*>(out) + r * H + col) =
              f32x4{acc[i][s][0] * sc, acc[i][s][1] * sc, acc[i][s][2] * sc, acc[i][s][3] * sc};
      }
    }
  };
  run_tile((m_valid + 15) / 16, wr, [&](auto b, auto a) {
    tile_body<decltype(b)::value, decltype(a)::value>(o, rings, f, epilogue);
  });
}

// ----------------------------------------------------------------------------- quantized weights
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

struct QTileArgs {
  TileArgs p;             // plan, bf16 operands of the shared expert (a: bf16 rows), output
  const uint16_t* a16;    // routed rows' binary16 A rows (gate/up: x16 through row_index; down: h)
  const uint8_t* codes0;  // gate (gate/up) or down codes [E, N, K]
  const uint8_t* codes1;  // up codes
  const void* scales0;    // FP8: fp32 [E, N / 128, K / 128]; 4-bit: binary16 [E, N, K / 32]
  const void* scales1;
};

// LDS rings of the quantized tiles: three stages of token rows, two of codes (each a K block of two
// K steps), over the same five 32 KiB arrays as Rings.
struct QRings {
  char* a[3];
  char* b[2];
};

// Fragment of the substep (0 .. NBW-1) in which column block s is decoded: spread over the first
// min(NBW, 4) fragments, so each fragment's MFMAs cover about one column block's decoding.
template <int NBW>
constexpr int decode_frag(int s) {
  return s * (NBW < 4 ? NBW : 4) / 4;
}

// One K step kt (kt % 12 == D) of the quantized tiles (format P).  A K step reads a step's share of
// the codes of every one of the 256 weight rows, so a K block (two steps) is loaded whole: block b at
// step 2 b - 3.  Per wave the vector-memory order is Q(0) A(0) A(1) Q(1) | A(2) | A(3) Q(2) | A(4) |
// A(5) Q(3) | ... (Q(b): the P::kLoads loads of block b): step kt issues A(kt + 2) and, when kt is
// odd, Q((kt + 3) / 2).  When step kt starts, only the loads of step kt - 1 may still be in flight
// (A(kt + 1), and Q((kt + 2) / 2) when kt is even), so A(kt) and the block of step kt + 1 have
// landed: after the barrier they are visible to every wave, and the step reads the next step's codes
// during its own MFMAs.  A(kt + 2) overwrites the rows of step kt - 1; Q(b) the block two earlier,
// whose codes were last read in step 2 b - 4.
template <class P, int NBW, int NAL, int D, bool kTail, bool kFirst = false>
__device__ __forceinline__ void q_kstep(const Loads& o, int kt, int nk, const QRings& r, const typename P::Ctx& x,
                                        typename P::Carry& c, f32x4 (&acc)[NBW > 0 ? NBW : 1][4]) {
  if constexpr (D % 2 == 0) {
    if (!kTail || kt + 2 < nk)
      wait_vmcnt<NAL + P::kLoads>();
    else if (kt + 1 < nk)
      wait_vmcnt<NAL>();
    else
      wait_vmcnt<0>();
  } else {
    if (!kTail || kt + 1 < nk)
      wait_vmcnt<NAL>();
    else
      wait_vmcnt<0>();
  }
  block_sync_lds();
  if (!kTail || kt + 2 < nk) issue_a<NAL>(o, kt + 2, r.a[(D + 2) % 3]);
  if constexpr (D % 2 == 1) {
    if (!kTail || kt + 3 < nk) P::issue_block(o, (kt + 3) / 2, r.b[((D + 3) / 2) % 2]);
  }
  const bool has_next = !kTail || kt + 1 < nk;
  P::template step<NBW, D % 2, (D + 1) % 2, kFirst>(r.a[D % 3], r.b[(D / 2) % 2], r.b[((D + 1) / 2) % 2], has_next,
                                                    kt, x, c, acc);
  __builtin_amdgcn_sched_barrier(0);
}

template <class P, int NBW, int NAL>
__device__ __forceinline__ void q_kloop(const Loads& o, int nk, const QRings& r, const typename P::Ctx& x,
                                        f32x4 (&acc)[NBW > 0 ? NBW : 1][4]) {
  // prologue in the steady state's issue order (nk is even: whole K blocks), fenced
  P::issue_block(o, 0, r.b[0]);
  __builtin_amdgcn_sched_barrier(0);
  issue_a<NAL>(o, 0, r.a[0]);
  __builtin_amdgcn_sched_barrier(0);
  issue_a<NAL>(o, 1, r.a[1]);
  __builtin_amdgcn_sched_barrier(0);
  if (nk > 2) P::issue_block(o, 1, r.b[1]);
  __builtin_amdgcn_sched_barrier(0);
  typename P::Carry c;
  q_kstep<P, NBW, NAL, 0, true, true>(o, 0, nk, r, x, c, acc);
  int kt = 1;
  // steady state: every load these twelve steps issue exists (kt + 14 < nk)
  for (; kt + 15 <= nk; kt += 12) {
    static_for<12>([&](auto ic) {
      constexpr int j = decltype(ic)::value;
      q_kstep<P, NBW, NAL, (j + 1) % 12, false>(o, kt + j, nk, r, x, c, acc);
    });
  }
  // the last 3 .. 14 steps, or all of a short loop (kt % 12 == 1 here)
  while (kt < nk) {
    bool done = false;
    static_for<12>([&](auto ic) {
      constexpr int j = decltype(ic)::value;
      if (!done) {
        q_kstep<P, NBW, NAL, (j + 1) % 12, true>(o, kt, nk, r, x, c, acc);
        if (++kt == nk) done = true;
      }
    });
  }
}

template <class P, int NBW, int NAL, class Epilogue>
__device__ __forceinline__ void q_tile_body(const Loads& o, const QRings& r, const typename P::Ctx& x,
                                            const Epilogue& epilogue) {
  f32x4 acc[NBW > 0 ? NBW : 1][4];
#pragma unroll
  for (int i = 0; i < (NBW > 0 ? NBW : 1); ++i)
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[i][s] = f32x4{0.f, 0.f, 0.f, 0.f};
  q_kloop<P, NBW, NAL>(o, o.nk, r, x, acc);
  epilogue(std::integral_constant<int, NBW>{}, acc);
}

// Work-groups for up to max_tiles row tiles dealt to the XCDs in blocks of kGroupTiles: at most
// ceil(max_tiles / (8 kGroupTiles)) blocks per XCD either way, each tile n_ntiles * n_ksplit work-groups
// (with fewer than 8 tiles, an XCD gets at most two chunks of at most per_tile / 2 work-groups each,
// which this covers).
inline unsigned grid_for(int64_t max_tiles, int n_ntiles, int n_ksplit = 1) {
  const int64_t per_xcd = (max_tiles + kXcds - 1) / kXcds;
  const int64_t blocks = (per_xcd + kGroupTiles - 1) / kGroupTiles;
  return (unsigned)(blocks * kGroupTiles * n_ntiles * n_ksplit * kXcds);
}


}  // namespace
}  // namespace moe
