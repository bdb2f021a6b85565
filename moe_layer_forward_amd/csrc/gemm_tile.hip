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
#include <type_traits>

#include "tile_core.h"

namespace moe {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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
  int tile_m;    // rows per row tile of the plan (kTileM, or kTileMFp8 for the FP8 tiles)
};

struct TileRows {
  int g;
  int64_t rbeg, rend;
};

// Work-group -> (row tile, column slab nt, K range ks).  The hardware hands work-group b to XCD b % 8;
// row tiles are dealt to the XCDs round-robin (tile t to XCD t % 8, from the plan's largest-first
// list, so every XCD gets the same mix of large and small groups).  An XCD takes its tiles in blocks
// of kGroupTiles: a block of tiles of one group (a group of many rows) runs slab by slab, its tiles
// side by side, so the work-groups reading a weight slab run together and share it in the XCD's L2
// (instead of the slab being streamed again for every row tile); any other block runs tile by tile,
// a tile's slabs side by side, sharing the tile's token rows in L2.  With fewer tiles than XCDs the
// tiles' items are spread over all XCDs instead.
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
    const int64_t j0 = blk * kGroupTiles;                            // first tile of the block, XCD-local
    int in_blk = 0;                                                  // tiles of this XCD in the block
    bool one_group = true;
    for (int i = 0; i < kGroupTiles; ++i) {
      const int64_t ti = (j0 + i) * kXcds + x;
      if (ti >= n_tiles) break;
      ++in_blk;
      if (p.tiles[2 * ti] != p.tiles[2 * (j0 * kXcds + x)]) one_group = false;
    }
    int j;
    if (one_group && in_blk == kGroupTiles) {
      j = q % kGroupTiles;
      rem = q / kGroupTiles;
    } else {
      j = q / per_tile;
      rem = q % per_tile;
    }
    tile64 = (j0 + j) * kXcds + x;
    if (j >= in_blk || tile64 >= n_tiles) return false;
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
// fragments (fragment fi: k-substep fi / NBW, row block fi % NBW).  acc[i][s]: lane l, element e =
// row 16 (wr + 2i) + 4 (l >> 4) + e, column block s, column l & 15.  Each A fragment is read from LDS
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
      for (int s = 0; s < 4; ++s) acc[i][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[fi], b[kk][s], acc[i][s], 0, 0, 0);
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
// over the 8 waves, ceil(nblk / 4) each.  One instance per pair that a row count of 1 .. 256 produces;
// device pass only (these instances are device code).
template <int kMaxNbw = 8, class Body>
__device__ __forceinline__ void run_tile(int nblk, int wr, const Body& body) {
  const int nbw = (nblk - wr + 1) / 2;
  const int nal = (nblk + 3) / 4;
#if defined(__HIP_DEVICE_COMPILE__)
#define MOE_TILE_CASE(B, A) \
  if (nbw == B && nal == A) return body(std::integral_constant<int, B>{}, std::integral_constant<int, A>{});
  if constexpr (kMaxNbw >= 8) {
    MOE_TILE_CASE(8, 4)
  }
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
// kRowsPer rows each; 16-byte chunk c of row r at position c ^ out_swz(r).
__device__ __forceinline__ int out_swz(int r) { return ((r >> 2) & 3) << 1; }

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
  // binary16, column c at position (c & ~7) | pair_pos(c & 7) (the operand order of the FP8 tiles)
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
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * (wr + 2 * i) + 4 * (lane >> 4) + e;
#pragma unroll
        for (int s = 0; s < 2; ++s)
          Out::put(rings, row, 32 * wc + 16 * s + (lane & 15), swiglu_f32(acc[i][s][e], acc[i][s + 2][e]));
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
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * (wr + 2 * i) + 4 * (lane >> 4) + e;
          const float sc = row_scale && row < m_valid ? row_scale[rbeg + row] : 1.f;
#pragma unroll
          for (int s = 0; s < 4; ++s) Out::put(rings, row, 64 * wc + 16 * s + (lane & 15), acc[i][s][e] * sc);
        }
      });
      block_sync_lds();
      Out::store(rings, m_valid, static_cast<uint16_t*>(out), H, rbeg, n0, H);
      return;
    }
    // fp32 rows (a caller's choice in moe_grouped_swiglu, or a K range's partial sums): direct stores
#pragma unroll
    for (int i = 0; i < NBW; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t r = rbeg + 16 * (wr + 2 * i) + 4 * (lane >> 4) + e;
        if (r >= rend) continue;
        const float sc = row_scale ? row_scale[r] : 1.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int col = n0 + 64 * wc + 16 * s + (lane & 15);
          if (col < H) static_cast<float*>(out)[r * H + col] = acc[i][s][e] * sc;
        }
      }
  };
  run_tile((m_valid + 15) / 16, wr, [&](auto b, auto a) {
    tile_body<decltype(b)::value, decltype(a)::value>(o, rings, f, epilogue);
  });
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gateup_tile_kernel(TileArgs p) {
  MOE_TILE_SMEM
  int nt, ks;
  TileRows t;
  if (tile_of(p, nt, ks, t)) gateup_bf16_item(p, rings, nt, t);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void down_tile_kernel(TileArgs p) {
  MOE_TILE_SMEM
  int nt, ks;
  TileRows t;
  if (tile_of(p, nt, ks, t)) down_bf16_item(p, rings, nt, ks, t);
}

// ----------------------------------------------------------------------------- FP8 routed experts
// The routed experts' weights as E4M3 codes with one fp32 scale per 128 x 128 block (the storage the
// weight-stream kernels read; see QWeights).  Same tiles, waves, LDS rings and dealing; what changes:
//   * A B stage holds 256 weight rows x 128 codes: 128 inputs (one scale block along K, whole cache
//     lines) for two K steps of 64.  LDS holds three stages of token rows and two of codes (the same
//     5 x 32 KiB), so token rows are loaded two steps ahead and each K block two steps before the
//     step that first reads it.
//   * The token rows (A) are binary16 with each group of 8 inputs in the order 0,4,1,5,2,6,3,7, and
//     v_mfma_f32_16x16x32_f16 runs the products.  Per step a lane reads 16 codes of each of its 4
//     weight rows in one 16-byte LDS read (inputs 16 g .. 16 g + 15 of the step, g = lane / 16) and
//     feeds the first 8 to the step's first MFMA k-substep and the next 8 to the second, so A's
//     fragment of substep kk is chunk 2 g + kk of the step's 128-byte row.
//   * Decoding: a byte permute puts codes (0,4,1,5) and (2,6,3,7) of 8 inputs into one word each, and
//     v_cvt_scalef32_pk_f16_fp8 makes two binary16 values of a word's low or high code pair.  That
//     conversion multiplies by 2^floor(log2 s) of its scale operand s (only the exponent counts), so
//     passing the block scale applies its power of two exactly; the mantissa part m = s / 2^floor(log2 s)
//     (in [1, 2), exact in binary16 to 11 bits) follows as one packed binary16 multiply.  A weight is
//     thus f16(f16(e4m3(c) 2^e) f16(m)), within 2^-10 of e4m3(c) s relative (binary16 subnormals
//     below 2^-14 absolute).  A wave's 64 weight rows lie in one 128-row scale block, so its scales
//     are one per K block: lane j holds K block j's (at most 64 blocks, K <= 8192).
//   * The shared expert (bf16 weights) is a group of the same tile list: its tiles run the bf16 body.
//   * Row tiles are 224 rows (kTileMFp8): at most 7 16-row blocks per wave, 112 accumulator VGPRs,
//     so that the decode's registers fit beside them without spills (a spill reload inside the K
//     loop waits for every load in flight).  A K2 prefill expert (~170 rows) is still one tile.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct QTileArgs {
  TileArgs p;             // plan, bf16 operands of the shared expert (a: bf16 rows), output
  const uint16_t* a16;    // routed rows' binary16 A rows (gate/up: x16 through row_index; down: h)
  const uint8_t* codes0;  // gate (gate/up) or down codes [E, N, K]
  const uint8_t* codes1;  // up codes
  const float* scales0;   // [E, N / 128, K / 128]
  const float* scales1;
};

// Lane j's block scale s (K block j of the wave's 128-row block); 1.0 past the last block.
struct LaneScale {
  float s;
};

__device__ __forceinline__ LaneScale lane_scale(const float* blocks, int nkb) {
  const int lane = threadIdx.x & 63;
  return LaneScale{lane < nkb ? blocks[lane] : 1.f};
}

// f16(m) twice, m = s with its exponent field replaced by that of 1.0 (the sign stays with m), from
// the bits of s: the 23 mantissa bits rounded to nearest even into 10 (a carry gives 2.0 exactly).
// Integer operations on a uniform value (scalar unit).
__device__ __forceinline__ uint32_t mantissa_f16x2(uint32_t sb) {
  const uint32_t mant = sb & 0x7fffffu;
  const uint32_t h = (0x3c00u + ((mant + 0xfffu + ((mant >> 13) & 1u)) >> 13)) | ((sb >> 16) & 0x8000u);
  return h | (h << 16);
}

// The scales of one K block, uniform over the wave: NS sets (gate/up: [0] gate rows, [1] up rows; down:
// one).  s goes to the conversion, which applies its power of two; m is the rest.
template <int NS>
struct StepScale {
  float s[NS];
  f16x2 m[NS];
};

template <int NS>
__device__ __forceinline__ StepScale<NS> step_scale(const LaneScale (&ls)[NS], int j) {
  StepScale<NS> r;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const uint32_t sb = (uint32_t)__builtin_amdgcn_readlane(__float_as_int(ls[i].s), j);
    r.s[i] = __uint_as_float(sb);
    r.m[i] = __builtin_bit_cast(f16x2, mantissa_f16x2(sb));
  }
  return r;
}

// 8 codes (inputs 0..7: the bytes of lo, then of hi) -> binary16 weights in the order 0,4,1,5,2,6,3,7.
__device__ __forceinline__ f16x8 dequant8(uint32_t lo, uint32_t hi, float s, f16x2 m) {
  const uint32_t p0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // bytes: codes 0, 4, 1, 5
  const uint32_t p1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // codes 2, 6, 3, 7
  const f16x2 h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(p0, s, false) * m;
  const f16x2 h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(p0, s, true) * m;
  const f16x2 h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(p1, s, false) * m;
  const f16x2 h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(p1, s, true) * m;
  return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// LDS read geometry of the FP8 tiles (16-row blocks as in Frag).
struct QFrag {
  uint32_t a_off[2];  // A, k-substep kk: logical chunk 2 g + kk of row x
  uint32_t b_off[2];  // B, step half hf (the step's 64 codes of the stage's 128): chunk 4 hf + g
  uint32_t a_row0;
  uint32_t b_row0[4];
};

__device__ __forceinline__ QFrag make_qfrag(int wr, const int (&b_rows)[4]) {
  const int lane = threadIdx.x & 63, x = lane & 15, g = lane >> 4;
  QFrag f;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    f.a_off[kk] = (uint32_t)(x * kRowBytes + (((2 * g + kk) ^ swz(x)) << 4));
    f.b_off[kk] = (uint32_t)(x * kRowBytes + (((4 * kk + g) ^ swz(x)) << 4));
  }
  f.a_row0 = (uint32_t)(wr * 16 * kRowBytes);
#pragma unroll
  for (int s = 0; s < 4; ++s) f.b_row0[s] = (uint32_t)(b_rows[s] * kRowBytes);
  return f;
}

// Lane offset of B piece j inside a code tensor whose rows are K bytes (row rl of the tile at weight
// row wrow); K block b adds 128 b.
__device__ __forceinline__ uint32_t qb_offset(int j, int64_t wrow, int K) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rl = (w + kWaves * j) * 8 + (lane >> 3);
  const int chunk = (lane & 7) ^ swz(rl);
  return (uint32_t)(wrow * K + 16 * chunk);
}

// K block b of the codes (128 inputs) of all 256 weight rows of the tile: B pieces 0 .. 3.
__device__ __forceinline__ void issue_qblock(const Loads& o, int b, char* stage) {
  const int w = o.wave;
  const uint32_t kb = (uint32_t)b * kRowBytes;
#pragma unroll
  for (int j = 0; j < kBLoads; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(operand_rsrc(o.b_base[j]), (LdsPtr)(stage + (w + kWaves * j) * 1024), 16,
                                             o.b_off[j] + kb, 0, 0, 0);
}

// Weights carried from one K step to the next: the first k-substep's decoded fragments of the 4 column
// blocks, and the raw codes of the second's.
struct QCarry {
  f16x8 b0[4];
  u32x2 zw[4];
};

// Fragment of the substep (0 .. NBW-1) in which column block s is decoded: spread over the first
// min(NBW, 4) fragments, so each fragment's MFMAs cover about one column block's decoding.
template <int NBW>
constexpr int decode_frag(int s) {
  return s * (NBW < 4 ? NBW : 4) / 4;
}

// Reads the 16 codes per column block of step half HF of a B stage.
template <int HF>
__device__ __forceinline__ void read_codes(const char* Bs, const QFrag& f, u32x4 (&q)[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) q[s] = *reinterpret_cast<const u32x4*>(Bs + f.b_row0[s] + f.b_off[HF]);
}

// MFMAs of one K step, in compute_step's fragment order, software-pipelined with the decoding: the
// step's second-substep weights are decoded from the carried codes during its first substep, the next
// step's codes are read from LDS (their stage is complete and visible since this step's barrier, and
// no load of this step writes it) and its first-substep weights decoded during the second substep.
// Each fragment's MFMAs are independent of the decoding placed beside them.  Column block s uses scale
// set GU && s >= 2 (the up rows).  kFirst: the step decodes its own first substep first (the tile's
// first step).  HF, HFN: this and the next step's half of their B stages.
template <int NBW, int HF, int HFN, bool GU, bool kFirst, int NS = GU ? 2 : 1>
__device__ __forceinline__ void q_compute_step(const char* As, const char* Bs, const char* Bn, bool has_next,
                                               const QFrag& f, const StepScale<NS>& sc, const StepScale<NS>& scn,
                                               QCarry& c, f32x4 (&acc)[NBW > 0 ? NBW : 1][4]) {
  if constexpr (NBW > 0) {
    constexpr int NF = 2 * NBW;
    constexpr int kReadNext = NBW < 5 ? NBW - 1 : 4;  // fragment that reads the next step's codes
    auto set = [](int s) { return GU && s >= 2 ? 1 : 0; };
    if constexpr (kFirst) {
      u32x4 q[4];
      read_codes<HF>(Bs, f, q);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        c.b0[s] = dequant8(q[s][0], q[s][1], sc.s[set(s)], sc.m[set(s)]);
        c.zw[s] = u32x2{q[s][2], q[s][3]};
      }
    } else {
      (void)Bs;
    }
    auto read_a = [&](int fi) {
      return *reinterpret_cast<const f16x8*>(As + f.a_row0 + f.a_off[fi / NBW] + (fi % NBW) * 2 * 16 * kRowBytes);
    };
    f16x8 b1[4];
    u32x4 qn[4];
    f16x8 a[NF];
    a[0] = read_a(0);
    a[1] = read_a(1);
#pragma unroll
    for (int fi = 0; fi < NF; ++fi) {
      if (fi + 2 < NF) a[fi + 2] = read_a(fi + 2);
      if (fi < NBW) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          if (decode_frag<NBW>(s) == fi) b1[s] = dequant8(c.zw[s][0], c.zw[s][1], sc.s[set(s)], sc.m[set(s)]);
        if (fi == kReadNext && has_next) read_codes<HFN>(Bn, f, qn);
      } else if (has_next) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          if (decode_frag<NBW>(s) == fi - NBW) {
            c.b0[s] = dequant8(qn[s][0], qn[s][1], scn.s[set(s)], scn.m[set(s)]);
            c.zw[s] = u32x2{qn[s][2], qn[s][3]};
          }
      }
      const int kk = fi / NBW, i = fi % NBW;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc[i][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[fi], kk == 0 ? c.b0[s] : b1[s], acc[i][s], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    (void)As;
    (void)Bs;
    (void)Bn;
    (void)has_next;
    (void)f;
    (void)sc;
    (void)scn;
    (void)c;
    (void)acc;
  }
}

// LDS rings of the FP8 tiles: three stages of token rows, two of codes (each two K steps), over the
// same five 32 KiB arrays as Rings.
struct QRings {
  char* a[3];
  char* b[2];
};

// One K step kt (kt % 12 == D) of the FP8 tiles.  A K step reads 64 codes of every one of the 256
// weight rows, so a K block (two steps) is loaded whole: block b at step 2 b - 3.  Per wave the
// vector-memory order is Q(0) A(0) A(1) Q(1) | A(2) | A(3) Q(2) | A(4) | A(5) Q(3) | ... (Q(b): the 4
// loads of block b): step kt issues A(kt + 2) and, when kt is odd, Q((kt + 3) / 2).  When step kt
// starts, only the loads of step kt - 1 may still be in flight (A(kt + 1), and Q((kt + 2) / 2) when kt
// is even), so A(kt) and the block of step kt + 1 have landed: after the barrier they are visible to
// every wave, and the step reads the next step's codes during its own MFMAs.  A(kt + 2) overwrites the
// rows of step kt - 1; Q(b) the block two earlier, whose codes were last read in step 2 b - 4.
template <int NBW, int NAL, int D, bool kTail, bool GU, bool kFirst = false, int NS = GU ? 2 : 1>
__device__ __forceinline__ void q_kstep(const Loads& o, int kt, int nk, const QRings& r, const QFrag& f,
                                        const LaneScale (&ls)[NS], QCarry& c, f32x4 (&acc)[NBW > 0 ? NBW : 1][4]) {
  if constexpr (D % 2 == 0) {
    if (!kTail || kt + 2 < nk)
      wait_vmcnt<NAL + kBLoads>();
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
    if (!kTail || kt + 3 < nk) issue_qblock(o, (kt + 3) / 2, r.b[((D + 3) / 2) % 2]);
  }
  const bool has_next = !kTail || kt + 1 < nk;
  const StepScale<NS> sc = step_scale(ls, kt >> 1);
  const StepScale<NS> scn = step_scale(ls, has_next ? (kt + 1) >> 1 : kt >> 1);
  __builtin_amdgcn_sched_barrier(0);
  q_compute_step<NBW, D % 2, (D + 1) % 2, GU, kFirst>(r.a[D % 3], r.b[(D / 2) % 2], r.b[((D + 1) / 2) % 2], has_next,
                                                      f, sc, scn, c, acc);
  __builtin_amdgcn_sched_barrier(0);
}

template <int NBW, int NAL, bool GU, int NS = GU ? 2 : 1>
__device__ __forceinline__ void q_kloop(const Loads& o, int nk, const QRings& r, const QFrag& f,
                                        const LaneScale (&ls)[NS], f32x4 (&acc)[NBW > 0 ? NBW : 1][4]) {
  // prologue in the steady state's issue order (nk is even: whole K blocks), fenced
  issue_qblock(o, 0, r.b[0]);
  __builtin_amdgcn_sched_barrier(0);
  issue_a<NAL>(o, 0, r.a[0]);
  __builtin_amdgcn_sched_barrier(0);
  issue_a<NAL>(o, 1, r.a[1]);
  __builtin_amdgcn_sched_barrier(0);
  if (nk > 2) issue_qblock(o, 1, r.b[1]);
  __builtin_amdgcn_sched_barrier(0);
  QCarry c;
  q_kstep<NBW, NAL, 0, true, GU, true>(o, 0, nk, r, f, ls, c, acc);
  int kt = 1;
  // steady state: every load these twelve steps issue exists (kt + 14 < nk)
  for (; kt + 15 <= nk; kt += 12) {
    static_for<12>([&](auto ic) {
      constexpr int j = decltype(ic)::value;
      q_kstep<NBW, NAL, (j + 1) % 12, false, GU>(o, kt + j, nk, r, f, ls, c, acc);
    });
  }
  // the last 3 .. 14 steps, or all of a short loop (kt % 12 == 1 here)
  while (kt < nk) {
    bool done = false;
    static_for<12>([&](auto ic) {
      constexpr int j = decltype(ic)::value;
      if (!done) {
        q_kstep<NBW, NAL, (j + 1) % 12, true, GU>(o, kt, nk, r, f, ls, c, acc);
        if (++kt == nk) done = true;
      }
    });
  }
}

template <int NBW, int NAL, bool GU, class Epilogue, int NS = GU ? 2 : 1>
__device__ __forceinline__ void q_tile_body(const Loads& o, const QRings& r, const QFrag& f, const LaneScale (&ls)[NS],
                                            const Epilogue& epilogue) {
  f32x4 acc[NBW > 0 ? NBW : 1][4];
#pragma unroll
  for (int i = 0; i < (NBW > 0 ? NBW : 1); ++i)
#pragma unroll
    for (int s = 0; s < 4; ++s) acc[i][s] = f32x4{0.f, 0.f, 0.f, 0.f};
  q_kloop<NBW, NAL, GU>(o, o.nk, r, f, ls, acc);
  epilogue(std::integral_constant<int, NBW>{}, acc);
}

// Gate/up work item of a routed group: h rows in binary16 (operand order), as the bf16 item.
__device__ __forceinline__ void gateup_fp8_item(const QTileArgs& q, const Rings& rings, int nt, const TileRows& t) {
  const TileArgs& p = q.p;
  const int H = p.H, I = p.I;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = w >> 2, wc = w & 3;
  const int64_t gsz = (int64_t)I * H;
  const uint8_t* cg = q.codes0 + t.g * gsz;
  const uint8_t* cu = q.codes1 + t.g * gsz;
  const int h0 = nt * 128;

  Loads o;
  o.wave = w;
  o.a_base = reinterpret_cast<const char*>(q.a16);
  a_offsets(o, H, [&](int rl) -> int64_t {
    const int64_t r = t.rbeg + rl;
    const int64_t rr = r < t.rend ? r : t.rbeg;
    return p.row_index ? (int64_t)p.row_index[rr] : rr;
  });
  // pieces w, w + 8: gate rows h0 + 8 w .. and h0 + 64 + 8 w ..; w + 16, w + 24: the same up rows.  The
  // piece's first row goes into its (uniform) base, so one lane offset serves all four (a lane's
  // swizzled chunk is the same in each piece: the pieces are 64 rows apart).
  const uint32_t b_lane = qb_offset(0, 8 * w + (lane >> 3), H);
#pragma unroll
  for (int j = 0; j < kBLoads; ++j) {
    o.b_base[j] = reinterpret_cast<const char*>(j < 2 ? cg : cu) + (int64_t)(h0 + 64 * (j & 1)) * H;
    o.b_off[j] = b_lane;
  }
  o.nk = H / kBK;
  o.skew = 0;
  // every h column of the tile lies in scale block row nt of W_gate and of W_up
  const int nkb = H / 128;
  const LaneScale ls[2] = {lane_scale(q.scales0 + ((int64_t)t.g * (I / 128) + nt) * nkb, nkb),
                           lane_scale(q.scales1 + ((int64_t)t.g * (I / 128) + nt) * nkb, nkb)};

  const int b_rows[4] = {32 * wc, 32 * wc + 16, 128 + 32 * wc, 128 + 32 * wc + 16};
  const QFrag f = make_qfrag(wr, b_rows);
  uint16_t* h = static_cast<uint16_t*>(p.out);
  const int64_t rbeg = t.rbeg;
  const int m_valid = (int)(t.rend - t.rbeg);
  const auto epilogue = [&](auto nbw_c, const auto& acc) {
    constexpr int NBW = decltype(nbw_c)::value;
    using Out = OutTile<128>;
    block_sync_lds();  // every wave is done reading the rings
    static_for<NBW>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * (wr + 2 * i) + 4 * (lane >> 4) + e;
#pragma unroll
        for (int s = 0; s < 2; ++s)
          Out::put_f16_pairs(rings, row, 32 * wc + 16 * s + (lane & 15), swiglu_f32(acc[i][s][e], acc[i][s + 2][e]));
      }
    });
    block_sync_lds();
    Out::store(rings, m_valid, h, I, rbeg, h0, I);
  };
  const QRings qr{{rings.a[0], rings.a[1], rings.b[0]}, {rings.b[1], rings.b[2]}};
  run_tile<kTileMFp8 / 32>((m_valid + 15) / 16, wr, [&](auto b, auto a) {
    q_tile_body<decltype(b)::value, decltype(a)::value, true>(o, qr, f, ls, epilogue);
  });
}

// Down work item of a routed group: y rows in bf16.
__device__ __forceinline__ void down_fp8_item(const QTileArgs& q, const Rings& rings, int nt, const TileRows& t) {
  const TileArgs& p = q.p;
  const int H = p.H, I = p.I;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = w >> 2, wc = w & 3;
  const uint8_t* cd = q.codes0 + t.g * ((int64_t)H * I);
  const int n0 = nt * 256;

  Loads o;
  o.wave = w;
  o.a_base = reinterpret_cast<const char*>(q.a16);
  a_offsets(o, I, [&](int rl) -> int64_t {
    const int64_t r = t.rbeg + rl;
    return r < t.rend ? r : t.rbeg;
  });
  // piece w + 8 j: W_down rows n0 + 64 j + 8 w .. (first row in the uniform base, one lane offset for
  // all four).  With H a multiple of 128 a piece lies wholly inside or past H; a piece past H (the
  // last slab's pieces 2 and 3) re-reads the rows of piece j - 2, whose columns are never stored.
  const uint32_t b_lane = qb_offset(0, 8 * w + (lane >> 3), I);
#pragma unroll
  for (int j = 0; j < kBLoads; ++j) {
    const int r0 = n0 + 64 * j < H ? n0 + 64 * j : n0 + 64 * (j - 2);
    o.b_base[j] = reinterpret_cast<const char*>(cd) + (int64_t)r0 * I;
    o.b_off[j] = b_lane;
  }
  o.nk = I / kBK;
  o.skew = 0;
  // the wave's 64 output columns lie in scale block row (n0 + 64 wc) / 128 (past H: the last one)
  const int nkb = I / 128;
  int rb = (n0 + 64 * wc) / 128;
  if (rb > H / 128 - 1) rb = H / 128 - 1;
  const LaneScale ls[1] = {lane_scale(q.scales0 + ((int64_t)t.g * (H / 128) + rb) * nkb, nkb)};

  const int b_rows[4] = {64 * wc, 64 * wc + 16, 64 * wc + 32, 64 * wc + 48};
  const QFrag f = make_qfrag(wr, b_rows);
  const int64_t rbeg = t.rbeg;
  const int m_valid = (int)(t.rend - t.rbeg);
  uint16_t* y = static_cast<uint16_t*>(p.out);
  const auto epilogue = [&](auto nbw_c, const auto& acc) {
    constexpr int NBW = decltype(nbw_c)::value;
    using Out = OutTile<256>;
    block_sync_lds();
    static_for<NBW>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * (wr + 2 * i) + 4 * (lane >> 4) + e;
#pragma unroll
        for (int s = 0; s < 4; ++s) Out::put(rings, row, 64 * wc + 16 * s + (lane & 15), acc[i][s][e]);
      }
    });
    block_sync_lds();
    Out::store(rings, m_valid, y, H, rbeg, n0, H);
  };
  const QRings qr{{rings.a[0], rings.a[1], rings.b[0]}, {rings.b[1], rings.b[2]}};
  run_tile<kTileMFp8 / 32>((m_valid + 15) / 16, wr, [&](auto b, auto a) {
    q_tile_body<decltype(b)::value, decltype(a)::value, false>(o, qr, f, ls, epilogue);
  });
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gateup_tile_fp8_kernel(
    QTileArgs q) {
  MOE_TILE_SMEM
  int nt, ks;
  TileRows t;
  if (!tile_of(q.p, nt, ks, t)) return;
  if (t.g == q.p.w.shared_group)
    gateup_bf16_item(q.p, rings, nt, t);
  else
    gateup_fp8_item(q, rings, nt, t);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void down_tile_fp8_kernel(
    QTileArgs q) {
  MOE_TILE_SMEM
  int nt, ks;
  TileRows t;
  if (!tile_of(q.p, nt, ks, t)) return;
  if (t.g == q.p.w.shared_group)
    down_bf16_item(q.p, rings, nt, 0, t);
  else
    down_fp8_item(q, rings, nt, t);
}

// Work-groups for up to max_tiles row tiles dealt round-robin to the XCDs: ceil(max_tiles / 8) tiles
// per XCD in blocks of kGroupTiles, each tile n_ntiles * n_ksplit work-groups (with fewer than 8 tiles,
// an XCD gets at most two chunks of at most per_tile / 2 work-groups each, which this covers).
unsigned grid_for(int64_t max_tiles, int n_ntiles, int n_ksplit = 1) {
  const int64_t per_xcd = (max_tiles + kXcds - 1) / kXcds;
  const int64_t blocks = (per_xcd + kGroupTiles - 1) / kGroupTiles;
  return (unsigned)(blocks * kGroupTiles * n_ntiles * n_ksplit * kXcds);
}

// Whether row r belongs to a group of the tile list, i.e. of more than stream_rows rows counted as
// the plan counts them (clamped to max_rows); the smaller groups' rows come from the weight-stream
// kernels, and rows before offsets[0] belong to no group.  Binary search over offsets[0 .. G].
__device__ __forceinline__ bool row_in_tile_list(const int32_t* __restrict__ offsets, int G, int64_t max_rows,
                                                 int stream_rows, int64_t r) {
  if (r < offsets[0]) return false;
  if (stream_rows == 0) return true;
  int lo = 0, hi = G;  // offsets[lo] <= r < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (offsets[mid] <= r) lo = mid; else hi = mid;
  }
  const int64_t a = offsets[lo] < max_rows ? offsets[lo] : max_rows;
  const int64_t b = offsets[lo + 1] < max_rows ? offsets[lo + 1] : max_rows;
  return b - a > stream_rows;
}

// y[r, :] = sum over the K ranges of part[ks, r, :] (in ks order), rows [0, offsets[G]) clamped to
// max_rows that belong to groups of the tile list; 8 columns per thread.
__global__ __launch_bounds__(256) void ksplit_reduce_kernel(const float* __restrict__ part, int n_ksplit,
                                                            const int32_t* __restrict__ offsets, int G,
                                                            int64_t max_rows, int stream_rows, int H,
                                                            void* __restrict__ out, int out_bf16) {
  int64_t rows = offsets[G];
  if (rows > max_rows) rows = max_rows;
  const int64_t n = rows * (H / 8);
  const int64_t plane = max_rows * H;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = 8 * i;  // row e / H, columns e % H .. +7
    if (!row_in_tile_list(offsets, G, max_rows, stream_rows, e / H)) continue;
    f32x4 lo = *reinterpret_cast<const f32x4*>(part + e), hi = *reinterpret_cast<const f32x4*>(part + e + 4);
    for (int ks = 1; ks < n_ksplit; ++ks) {
      lo += *reinterpret_cast<const f32x4*>(part + ks * plane + e);
      hi += *reinterpret_cast<const f32x4*>(part + ks * plane + e + 4);
    }
    if (out_bf16) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        w[j] = (uint32_t)f32_to_bf16(lo[2 * j]) | ((uint32_t)f32_to_bf16(lo[2 * j + 1]) << 16);
        w[2 + j] = (uint32_t)f32_to_bf16(hi[2 * j]) | ((uint32_t)f32_to_bf16(hi[2 * j + 1]) << 16);
      }
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + e) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(out) + e) = lo;
      *reinterpret_cast<f32x4*>(static_cast<float*>(out) + e + 4) = hi;
    }
  }
}

constexpr int kCUs = 256;  // MI355X compute units; one tile work-group per CU

// K ranges per work item for a launch of `items` items over nk K steps: with fewer items than CUs,
// the divisor s of nk (s <= 16, at least 4 steps per range) with the smallest ceil(items * s / CUs) / s,
// i.e. the fewest rounds of work per range, each range's partial sums (part_frac of an item's weight
// bytes, written and read back once) counted against it.
int tile_ksplit(int64_t items, int nk, double part_frac) {
  if (items <= 0 || items >= kCUs) return 1;
  int best = 1;
  double best_cost = 1.0;
  for (int sp = 2; sp <= 16; ++sp) {
    if (nk % sp || nk / sp < 4) continue;
    const int64_t rounds = (items * sp + kCUs - 1) / kCUs;
    const double cost = (double)rounds / sp * (1.0 + sp * part_frac);
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = sp;
    }
  }
  return best;
}

int64_t rows_per_tile_est(int64_t max_rows) { return max_rows < kTileM ? max_rows : kTileM; }

}  // namespace

int down_tile_ksplit(int64_t max_rows, int G, int H, int I) {
  (void)G;
  // items if the rows formed full tiles; an item's partial sums: rows x 256 columns fp32
  const int64_t items = ((max_rows + kTileM - 1) / kTileM) * ((H + 255) / 256);
  const double part_frac = (double)rows_per_tile_est(max_rows) * 256 * 4 * 2 / (256.0 * I * 2);
  return tile_ksplit(items, I / kBK, part_frac);
}

hipError_t launch_gateup_tile_bf16(const Groups& g, const Weights& w, const uint16_t* x, uint16_t* h, int H, int I,
                                   hipStream_t s) {
  if (g.tile_m != kTileM) return hipErrorInvalidValue;
  TileArgs p{g.group_offsets, g.row_index, g.tiles, g.counters, g.max_rows, w, x, h, 1, nullptr, H, I, I / 128,
             1, nullptr, kTileM};
  gateup_tile_kernel<<<grid_for(g.max_tiles, p.n_ntiles), kThreads, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_down_tile_bf16(const Groups& g, const Weights& w, const uint16_t* h, void* y_rows, bool y_bf16,
                                 const float* row_scale, float* part, int H, int I, hipStream_t s) {
  const int split = down_tile_ksplit(g.max_rows, g.n_groups, H, I);
  if ((split > 1 && !part) || g.tile_m != kTileM) return hipErrorInvalidValue;
  TileArgs p{g.group_offsets, nullptr, g.tiles, g.counters, g.max_rows, w, h, y_rows, y_bf16 ? 1 : 0, row_scale,
             H, I, (H + 255) / 256, split, part, kTileM};
  down_tile_kernel<<<grid_for(g.max_tiles, p.n_ntiles, split), kThreads, 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || split == 1) return e;
  return launch_ksplit_reduce(part, split, g, g.stream_rows, H, y_rows, y_bf16, s);
}

hipError_t launch_ksplit_reduce(const float* part, int split, const Groups& g, int stream_rows, int H, void* y_rows,
                                bool y_bf16, hipStream_t s) {
  const int64_t n = g.max_rows * (H / 8);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  ksplit_reduce_kernel<<<(unsigned)blocks, 256, 0, s>>>(part, split, g.group_offsets, g.n_groups, g.max_rows,
                                                        stream_rows, H, y_rows, y_bf16 ? 1 : 0);
  return hipGetLastError();
}

bool tile_fp8_shape_ok(int H, int I) {
  return H > 0 && I > 0 && H % 128 == 0 && I % 128 == 0 && H <= 128 * 64 && I <= 128 * 64;
}

hipError_t launch_gateup_tile_fp8(const Groups& g, const Weights& w, const QWeights& q, const uint16_t* x,
                                  const uint16_t* x16, uint16_t* h, int H, int I, hipStream_t s) {
  if (q.format != QFormat::kFp8 || !tile_fp8_shape_ok(H, I) || g.tile_m != kTileMFp8) return hipErrorInvalidValue;
  QTileArgs a{{g.group_offsets, g.row_index, g.tiles, g.counters, g.max_rows, w, x, h, 1, nullptr, H, I, I / 128, 1,
               nullptr, kTileMFp8},
              x16,
              static_cast<const uint8_t*>(q.gate_codes),
              static_cast<const uint8_t*>(q.up_codes),
              static_cast<const float*>(q.gate_scales),
              static_cast<const float*>(q.up_scales)};
  gateup_tile_fp8_kernel<<<grid_for(g.max_tiles, a.p.n_ntiles), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_down_tile_fp8(const Groups& g, const Weights& w, const QWeights& q, const uint16_t* h,
                                uint16_t* y_rows, int H, int I, hipStream_t s) {
  if (q.format != QFormat::kFp8 || !tile_fp8_shape_ok(H, I) || g.tile_m != kTileMFp8) return hipErrorInvalidValue;
  QTileArgs a{{g.group_offsets, nullptr, g.tiles, g.counters, g.max_rows, w, h, y_rows, 1, nullptr, H, I,
               (H + 255) / 256, 1, nullptr, kTileMFp8},
              h,
              static_cast<const uint8_t*>(q.down_codes),
              nullptr,
              static_cast<const float*>(q.down_scales),
              nullptr};
  down_tile_fp8_kernel<<<grid_for(g.max_tiles, a.p.n_ntiles), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
