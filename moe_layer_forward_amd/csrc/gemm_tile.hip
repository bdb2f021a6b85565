// Grouped SwiGLU expert GEMMs for many rows per expert (prefill-like shapes), bf16 MFMA.
//
// The experts are the SwiGLU FFNs of "Kimi K2.5 模型架构深度拆解" §4.3 / §10.2 Steps 5-6
// (gate + up -> SiLU -> multiply -> down), batched over experts as the grouped GEMM that
// "Kimi K2.5 架构 QA" Q8.3 names in place of the per-expert loop.
//
// Work item = (row tile of one group, column slab; for down with few row tiles also a K range,
// whose fp32 partial sums a second kernel adds in K order).  Row tiles come from the device-side plan
// (largest groups first, kTileM = 256 rows each, so a K2 expert's ~170 prefill rows are one tile
// and every weight byte is read from HBM once).  With ~170 rows per expert the layer moves ~170
// FLOP per weight byte, below the MI355X ridge (~310), so these kernels are weight streams first
// and matrix-core loops second:
//
//   * B (weights) never touches LDS.  Each wave owns 32 weight rows (output columns) and loads them
//     straight into v_mfma_f32_16x16x32_bf16 B-operand registers: one load instruction covers 64
//     contiguous bytes of each of 16 rows, and kDepth K steps of it are in flight per wave (a
//     register ring).  8 waves, two per SIMD (up to 128 accumulators
//     and the 64-register ring fit a wave's 256 registers), so one wave's MFMAs cover the other's
//     waits.
//   * A (token rows) is shared by the 8 waves and staged through a kStages-deep LDS ring with
//     gfx950's direct global -> LDS loads (no register round trip).  Each stage is its own
//     __shared__ array and every access names its stage statically (the K loop is unrolled by
//     kStages), so the compiler can tell which LDS reads depend on which direct loads; with a
//     single array it would make every LDS read wait for the newest direct load, i.e. for all
//     loads in flight, weights included.  Rows are gathered straight
//     from x through row_index, so no permuted copy of x is written.  LDS rows are unpadded;
//     16-byte chunk c of row r sits at c ^ swz(r), so the 16 rows one 16-lane group reads land in
//     16 different bank groups.
//   * Every wave multiplies all rows of the tile, in 32-row steps up to the group's end: the K loop
//     is instantiated per row count (chosen outside the loop), so padding rows cost no MFMA and
//     the A rows past the last 32-row step are not even loaded.
//   * One barrier per K step (LDS traffic only; the loads in flight stay in flight).
//
//   gate/up: wave w owns h columns n0 + 16w .. +16 of the tile's 128: column sub-tile 0 is their
//            gate rows, sub-tile 1 their up rows, so h = SiLU(g) * u is formed in registers.
//   down:    wave w owns 32 rows of W_down; y_rows (fp32 or bf16), times row_scale if given.
// Work items are dealt XCD-major, so the column slabs of one row tile run on the same XCD at the
// same time and share its rows of A in that XCD's L2.
#include <type_traits>

#include "tile_core.h"

namespace moe {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512, kWaves = 8;
constexpr int kBK = 64;                                // k per step
constexpr int kRowBytes = kBK * 2;                     // one A row of one step in LDS
constexpr int kStages = 4;                             // LDS ring of A (one __shared__ array per stage)
constexpr int kDepth = kStages;                        // K steps of weights in flight per wave
constexpr int kADist = kStages - 1;                    // A is loaded this many steps ahead
constexpr int kStageBytes = kTileM * kRowBytes;        // 32 KiB
constexpr int kSmemBytes = kStages * kStageBytes;      // 128 KiB
constexpr int kALoads = kStageBytes / 1024 / kWaves;   // direct-to-LDS loads per wave per step (at most)
constexpr int kNSub = 2;                               // 16-column sub-tiles per wave
constexpr int kBLoads = 2 * kNSub;                     // 2 k-substeps x 2 column sub-tiles
constexpr int kLoads = kALoads + kBLoads;              // vector-memory ops per wave per step
constexpr int kSub = kTileM / 16;                      // 16-row sub-tiles of a tile
static_assert(kALoads * kWaves * 1024 == kStageBytes && kRowBytes == 128 && kTileM % 32 == 0, "A staging");
static_assert(kSmemBytes <= 160 * 1024, "LDS");
static_assert(3 * kBLoads + 2 * kALoads <= 63, "vmcnt");

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
};

struct TileRows {
  int g;
  int64_t rbeg, rend;
};

// Work item -> (row tile, column slab nt, K range ks); consecutive items (one XCD's share) walk the
// slabs and K ranges of one row tile.
__device__ __forceinline__ bool tile_of(const TileArgs& p, int& nt, int& ks, TileRows& t) {
  int64_t L;
  const int per_tile = p.n_ntiles * p.n_ksplit;
  if (!xcd_work_item((int64_t)p.counters[1] * per_tile, L)) return false;
  const int tile = (int)(L / per_tile);
  const int rem = (int)(L % per_tile);
  nt = rem / p.n_ksplit;
  ks = rem % p.n_ksplit;
  t.g = p.tiles[2 * tile];
  const int m0 = p.tiles[2 * tile + 1];
  int64_t r0 = p.group_offsets[t.g], r1 = p.group_offsets[t.g + 1];
  if (r0 > p.max_rows) r0 = p.max_rows;
  if (r1 > p.max_rows) r1 = p.max_rows;
  if (r1 < r0) r1 = r0;
  t.rbeg = r0 + m0;
  t.rend = t.rbeg + kTileM < r1 ? t.rbeg + kTileM : r1;
  return t.rbeg < t.rend;
}

// Operand addressing: uniform bases plus 32-bit per-lane byte offsets (operands stay below 4 GiB).
struct Operands {
  const char* a_base;          // A rows; lane offsets a_off[j] include the row and the LDS chunk
  uint32_t a_off[kALoads];
  const char* b[kNSub];        // first weight row of each 16-column sub-tile of this wave
  uint32_t b_off;              // row (lane % 16) and 16-byte quarter (lane / 16) of a 64-byte piece
  int skew, nk;                // step kt loads K step (kt + skew) mod nk (uniform over the work-group)
};

// Byte offset along K of the step loaded as step kt (kt < nk).
__device__ __forceinline__ uint32_t kbytes(const Operands& o, int kt) {
  int ks = kt + o.skew;
  if (ks >= o.nk) ks -= o.nk;
  return (uint32_t)ks * kRowBytes;
}

// B fragments of one K step: [k-substep][column sub-tile].
struct BFrag {
  u32x4 v[2][kNSub];
};

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ void load_b(BFrag& f, const Operands& o, uint32_t kb) {
  const uint32_t off = o.b_off + kb;
#pragma unroll
  for (int s = 0; s < kNSub; ++s) {
    f.v[0][s] = *reinterpret_cast<const u32x4*>(o.b[s] + off);
    f.v[1][s] = *reinterpret_cast<const u32x4*>(o.b[s] + off + 64);
  }
}

// A loads per wave per step when only the first 32*NP rows are multiplied.
template <int NP>
constexpr int a_loads() { return (4 * NP + kWaves - 1) / kWaves; }

// Direct global -> LDS loads of step kt's A block: 1 KiB piece g (rows 8g .. 8g+7) is loaded by
// wave g % kWaves; only the pieces under the first 32*NP rows are loaded.
template <int NP>
__device__ __forceinline__ void issue_a(const Operands& o, uint32_t kb, char* stage) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int j = 0; j < a_loads<NP>(); ++j)
    __builtin_amdgcn_global_load_lds(o.a_base + (o.a_off[j] + kb), stage + (j * kWaves + w) * 1024, 16, 0, 0);
}

// MFMAs of one K step over the first 2*NP 16-row sub-tiles.  acc[i][s]: rows 16i.., column
// sub-tile s; lane l, element e holds row 16i + 4*(l/16) + e, column 16s + l%16 of this wave.
// The A fragments of the step (2 k-substeps x 2*NP sub-tiles) are read from LDS two ahead of the
// MFMAs that use them, in a fixed order (a scheduling barrier after each fragment's MFMAs), so
// only three are live at a time and each read has 8 MFMAs to land behind.
template <int NP>
__device__ __forceinline__ void compute_step(const char* stage, const BFrag& b, f32x4 (&acc)[2 * NP][kNSub]) {
  constexpr int kFrags = 2 * (2 * NP);
  const int lane = threadIdx.x & 63, r16 = lane & 15, q = lane >> 4;
  // swz(16i + r16) == swz(r16): the lane's chunk position is the same in every sub-tile
  const char* ap0 = stage + r16 * kRowBytes + ((q ^ swz(r16)) << 4);
  const char* ap1 = stage + r16 * kRowBytes + (((4 + q) ^ swz(r16)) << 4);
  auto read = [&](int f) {
    const int kk = f / (2 * NP), i = f % (2 * NP);
    return *reinterpret_cast<const bf16x8*>((kk ? ap1 : ap0) + i * 16 * kRowBytes);
  };
  bf16x8 a[kFrags];
  a[0] = read(0);
  a[1] = read(1);
#pragma unroll
  for (int f = 0; f < kFrags; ++f) {
    if (f + 2 < kFrags) a[f + 2] = read(f + 2);
    const int kk = f / (2 * NP), i = f % (2 * NP);
#pragma unroll
    for (int s = 0; s < kNSub; ++s)
      acc[i][s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[f], as_bf16x8(b.v[kk][s]), acc[i][s], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The A ring: stage d of step kt is array kt % kStages.
struct Ring {
  char* st[kStages];
};

// One K step (kt % kStages == D): wait for this wave's A block of step kt, then for every wave's
// (barrier, which also frees the stage of step kt-1), refill that stage with step kt+kADist,
// multiply, and refill this step's register slot with the weights of step kt+kDepth.
// Vector-memory order per wave: ..., A(j), B(j+1), A(j+1), B(j+2), ...  so when step kt starts,
// the operations issued after A(kt) are B(kt+1), A(kt+1), B(kt+2), A(kt+2), B(kt+3) (those that
// exist), kBLoads or a_loads<NP>() each.
template <int NP, int D, bool kTail>
__device__ __forceinline__ void kstep(const Operands& o, int kt, int nk, const Ring& ring, BFrag (&b)[kDepth],
                                      f32x4 (&acc)[2 * NP][kNSub]) {
  constexpr int kA = a_loads<NP>();
  const int ahead = kTail ? nk - 1 - kt : 3;
  if (ahead >= 3)
    wait_vmcnt<3 * kBLoads + 2 * kA>();
  else if (ahead == 2)
    wait_vmcnt<2 * kBLoads + 2 * kA>();
  else if (ahead == 1)
    wait_vmcnt<kBLoads + kA>();
  else
    wait_vmcnt<0>();
  block_sync_lds();
  if (!kTail || kt + kADist < nk) issue_a<NP>(o, kbytes(o, kt + kADist), ring.st[(D + kADist) % kStages]);
  compute_step<NP>(ring.st[D], b[D], acc);
  if (!kTail || kt + kDepth < nk) load_b(b[D], o, kbytes(o, kt + kDepth));
}

template <int NP>
__device__ __forceinline__ void kloop(const Operands& o, int nk, const Ring& ring, f32x4 (&acc)[2 * NP][kNSub]) {
  static_assert(kStages == 4 && kDepth == 4 && kADist == 3, "the unrolling below");
  BFrag b[kDepth];
  int kt = 0;
  if (nk >= 8) {
    // prologue in the steady-state order B(0), A(0), B(1), A(1), B(2), A(2), B(3); unconditional,
    // and fenced against reordering, so the compiler's own wait for B(kt) at the loop head sees the
    // full count of later loads (a reordered prologue makes it drain every load once per 4 steps)
#pragma unroll
    for (int s = 0; s < kDepth; ++s) {
      load_b(b[s], o, kbytes(o, s));
      __builtin_amdgcn_sched_barrier(0);
      if (s < kADist) issue_a<NP>(o, kbytes(o, s), ring.st[s]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // steady state: every refill of these four steps exists (kt + 7 < nk), no conditions
    for (; kt + 8 <= nk; kt += 4) {
      kstep<NP, 0, false>(o, kt, nk, ring, b, acc);
      kstep<NP, 1, false>(o, kt + 1, nk, ring, b, acc);
      kstep<NP, 2, false>(o, kt + 2, nk, ring, b, acc);
      kstep<NP, 3, false>(o, kt + 3, nk, ring, b, acc);
    }
  } else {
#pragma unroll
    for (int s = 0; s < kDepth; ++s) {
      if (s < nk) load_b(b[s], o, kbytes(o, s));
      if (s < kADist && s < nk) issue_a<NP>(o, kbytes(o, s), ring.st[s]);
    }
  }
  // the last 2 to 6 steps (K is a multiple of 128, so nk is even)
  if (kt + 4 <= nk) {
    kstep<NP, 0, true>(o, kt, nk, ring, b, acc);
    kstep<NP, 1, true>(o, kt + 1, nk, ring, b, acc);
    kstep<NP, 2, true>(o, kt + 2, nk, ring, b, acc);
    kstep<NP, 3, true>(o, kt + 3, nk, ring, b, acc);
    kt += 4;
  }
  if (kt < nk) kstep<NP, 0, true>(o, kt, nk, ring, b, acc);
  if (kt + 1 < nk) kstep<NP, 1, true>(o, kt + 1, nk, ring, b, acc);
}

// The tile's product over the full K (a multiple of kBK) for its first 2*NP 16-row sub-tiles,
// then the epilogue on the accumulators.
template <int NP, class Epilogue>
__device__ __forceinline__ void tile_body(const Operands& o, int K, const Ring& smem, const Epilogue& epilogue) {
  f32x4 acc[2 * NP][kNSub];
#pragma unroll
  for (int i = 0; i < 2 * NP; ++i)
#pragma unroll
    for (int s = 0; s < kNSub; ++s) acc[i][s] = f32x4{0.f, 0.f, 0.f, 0.f};
  kloop<NP>(o, K / kBK, smem, acc);
  epilogue(acc);
}

// One instance of the whole tile body per 32-row count of the tile (1..8): the accumulators of
// each instance are sized to its rows, and nothing is merged across instances.  Device pass
// only: these instances are device code.
template <class Epilogue>
__device__ __forceinline__ void run_tile(const Operands& o, int m_valid, int K, const Ring& smem, const Epilogue& epilogue) {
  static_assert(kSub == 16, "dispatch below covers 1..8 row pairs");
  const int np = (m_valid + 31) / 32;
#if defined(__HIP_DEVICE_COMPILE__)
  switch (np) {
    case 8: tile_body<8>(o, K, smem, epilogue); break;
    case 7: tile_body<7>(o, K, smem, epilogue); break;
    case 6: tile_body<6>(o, K, smem, epilogue); break;
    case 5: tile_body<5>(o, K, smem, epilogue); break;
    case 4: tile_body<4>(o, K, smem, epilogue); break;
    case 3: tile_body<3>(o, K, smem, epilogue); break;
    case 2: tile_body<2>(o, K, smem, epilogue); break;
    default: tile_body<1>(o, K, smem, epilogue); break;
  }
#else
  (void)np;
  (void)o;
  (void)K;
  (void)smem;
  (void)epilogue;
#endif
}

// Output tiles leave through LDS so that global stores are whole 16-byte chunks of contiguous rows
// (the MFMA layout would give 2-byte stores, 32 bytes per row per instruction).  After the K loop
// the A ring is free; a bf16 tile of kCols columns is staged there, row r in stage r / kRowsPerStage,
// and 16-byte chunk c of row r at position c ^ out_swz(r) (the four row groups one MFMA result
// register spans land in different banks).
__device__ __forceinline__ int out_swz(int r) { return ((r >> 2) & 3) << 1; }

template <int kCols>
struct OutTile {
  static constexpr int kRowB = kCols * 2;                 // bytes per staged row
  static constexpr int kRowsPerStage = kStageBytes / kRowB;
  static constexpr int kChunks = kRowB / 16;              // 16-byte chunks per row
  static_assert(kRowsPerStage % 16 == 0 && kRowsPerStage * kStages >= kTileM, "staging");

  // Write one bf16 value of row r (tile-relative), column col (tile-relative).  i is the 16-row
  // sub-tile of r, so the stage index is a compile-time constant.
  template <int I>
  __device__ static __forceinline__ void put(const Ring& ring, int r, int col, float v) {
    char* st = ring.st[(16 * I) / kRowsPerStage];
    *reinterpret_cast<uint16_t*>(st + (r % kRowsPerStage) * kRowB + (((col >> 3) ^ out_swz(r)) << 4) +
                                 (col & 7) * 2) = f32_to_bf16(v);
  }

  // Store rows [0, m_valid) of the staged tile to out[(rbeg + r) * ld + col0 + c], columns below
  // col_end only; every thread of the work-group takes part.
  __device__ static __forceinline__ void store(const Ring& ring, int m_valid, uint16_t* out, int64_t ld,
                                               int64_t rbeg, int col0, int col_end) {
    constexpr int kPerThread = kRowsPerStage * kChunks / kThreads;
    static_assert(kPerThread * kThreads == kRowsPerStage * kChunks, "chunks per thread");
#pragma unroll
    for (int st = 0; st < kStages; ++st) {
      if (st * kRowsPerStage >= m_valid) break;
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) {
        const int ch = j * kThreads + threadIdx.x;
        const int rl = ch / kChunks, c = ch % kChunks;
        const int r = st * kRowsPerStage + rl;
        if (r < m_valid && col0 + 8 * c < col_end) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(ring.st[st] + rl * kRowB + ((c ^ out_swz(r)) << 4));
          *reinterpret_cast<u32x4*>(out + (rbeg + r) * ld + col0 + 8 * c) = v;
        }
      }
    }
  }
};

// Compile-time loop helper: f(integral_constant<int, I>) for I = 0 .. N-1.
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(const F& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Lane offsets of the A loads: row rl of the tile is source row src(rl) of a [*, K] matrix.
template <class RowOf>
__device__ __forceinline__ void a_offsets(Operands& o, int K, RowOf row_of) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < kALoads; ++j) {
    const int rl = (j * kWaves + w) * 8 + (lane >> 3);  // 8 rows of 128 bytes per 1 KiB load
    const int chunk = (lane & 7) ^ swz(rl);              // the chunk that belongs in this lane's slot
    o.a_off[j] = (uint32_t)((row_of(rl) * K + 8 * chunk) * 2);
  }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gateup_tile_kernel(TileArgs p) {
  __shared__ __align__(16) char a0[kStageBytes], a1[kStageBytes], a2[kStageBytes], a3[kStageBytes];
  const Ring smem{{a0, a1, a2, a3}};
  int nt, ks;
  TileRows t;
  if (!tile_of(p, nt, ks, t)) return;
  const int H = p.H, I = p.I;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool sh = t.g == p.w.shared_group;
  const uint16_t* wg = sh ? (const uint16_t*)p.w.s_gate : (const uint16_t*)p.w.gate + (int64_t)t.g * I * H;
  const uint16_t* wu = sh ? (const uint16_t*)p.w.s_up : (const uint16_t*)p.w.up + (int64_t)t.g * I * H;
  const int c0 = nt * 128 + 16 * w;  // first h column of this wave

  Operands o;
  o.a_base = reinterpret_cast<const char*>(p.a);
  a_offsets(o, H, [&](int rl) -> int64_t {
    const int64_t r = t.rbeg + rl;
    const int64_t rr = r < t.rend ? r : t.rbeg;  // rows past the group end re-read its first row
    return p.row_index ? (int64_t)p.row_index[rr] : rr;
  });
  o.b[0] = reinterpret_cast<const char*>(wg + (int64_t)c0 * H);  // gate rows of the wave's 16 columns
  o.b[1] = reinterpret_cast<const char*>(wu + (int64_t)c0 * H);  // their up rows
  o.b_off = (uint32_t)((lane & 15) * H * 2 + 16 * (lane >> 4));
  o.nk = H / kBK;
  o.skew = 0;  // 14,336-byte rows (K2) spread over the channels on their own

  uint16_t* h = static_cast<uint16_t*>(p.out);
  const int64_t rbeg = t.rbeg;
  const int m_valid = (int)(t.rend - t.rbeg);
  run_tile(o, m_valid, H, smem, [&](const auto& acc) {
    constexpr int n16 = sizeof(acc) / sizeof(acc[0]);
    using Out = OutTile<128>;
    block_sync_lds();  // every wave is done reading the A ring
    static_for<n16>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        Out::put<i>(smem, 16 * i + 4 * (lane >> 4) + e, 16 * w + (lane & 15),
                    swiglu_f32(acc[i][0][e], acc[i][1][e]));
    });
    block_sync_lds();
    Out::store(smem, m_valid, h, I, rbeg, nt * 128, I);
  });
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void down_tile_kernel(TileArgs p) {
  __shared__ __align__(16) char a0[kStageBytes], a1[kStageBytes], a2[kStageBytes], a3[kStageBytes];
  const Ring smem{{a0, a1, a2, a3}};
  int nt, ks;
  TileRows t;
  if (!tile_of(p, nt, ks, t)) return;
  const int H = p.H, I = p.I;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint16_t* wd = t.g == p.w.shared_group ? (const uint16_t*)p.w.s_down
                                                : (const uint16_t*)p.w.down + (int64_t)t.g * H * I;
  const int c0 = nt * 256 + 32 * w;  // first output column of this wave (H is a multiple of 32)
  const bool cols_ok = c0 < H;       // the last slab of an H that is not a multiple of 256

  // this item's K range [k0, k0 + kc) of the h rows and of W_down's rows
  const int kc = I / p.n_ksplit, k0 = ks * kc;
  Operands o;
  o.a_base = reinterpret_cast<const char*>(p.a + k0);
  a_offsets(o, I, [&](int rl) -> int64_t {
    const int64_t r = t.rbeg + rl;
    return r < t.rend ? r : t.rbeg;
  });
#pragma unroll
  for (int s = 0; s < kNSub; ++s)  // idle waves re-read the first rows
    o.b[s] = reinterpret_cast<const char*>(wd + (int64_t)((cols_ok ? c0 : 0) + 16 * s) * I + k0);
  o.b_off = (uint32_t)((lane & 15) * I * 2 + 16 * (lane >> 4));
  // W_down rows a multiple of 4 KiB apart put the same K step of all 256 rows on few HBM channels:
  // the column slabs then start their K loops at different steps (and wrap around).  Only while the
  // tile's h block is small (I <= 4096: at most 2 MiB): the slabs of a tile share it through L2 only
  // while they walk K together (the dense layer's I = 18432 measured 7% slower with the skew).
  o.nk = kc / kBK;
  o.skew = (I * 2) % 4096 == 0 && I <= 4096 ? nt * 5 % o.nk : 0;

  const int64_t rbeg = t.rbeg, rend = t.rend;
  const int m_valid = (int)(rend - rbeg);
  const float* row_scale = p.row_scale;
  const bool split = p.n_ksplit > 1;
  void* out = split ? static_cast<void*>(p.part + (int64_t)ks * p.max_rows * H) : p.out;
  run_tile(o, m_valid, kc, smem, [&](const auto& acc) {
    constexpr int n16 = sizeof(acc) / sizeof(acc[0]);
    if (p.out_bf16 && !split) {
      using Out = OutTile<256>;
      block_sync_lds();  // every wave is done reading the A ring
      static_for<n16>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * i + 4 * (lane >> 4) + e;
          const float sc = row_scale && r < m_valid ? row_scale[rbeg + r] : 1.f;
#pragma unroll
          for (int s = 0; s < kNSub; ++s) Out::put<i>(smem, r, 32 * w + 16 * s + (lane & 15), acc[i][s][e] * sc);
        }
      });
      block_sync_lds();
      Out::store(smem, m_valid, static_cast<uint16_t*>(out), H, rbeg, nt * 256, H);
      return;
    }
    // fp32 rows (a caller's choice in moe_grouped_swiglu, or a K range's partial sums): direct stores
    if (!cols_ok) return;
#pragma unroll
    for (int i = 0; i < n16; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t r = rbeg + 16 * i + 4 * (lane >> 4) + e;
        if (r >= rend) continue;
        const float sc = row_scale ? row_scale[r] : 1.f;
#pragma unroll
        for (int s = 0; s < kNSub; ++s)
          static_cast<float*>(out)[r * H + c0 + 16 * s + (lane & 15)] = acc[i][s][e] * sc;
      }
  });
}

unsigned grid_for(int64_t max_tiles, int n_ntiles, int n_ksplit = 1) {
  int64_t n = max_tiles * n_ntiles * n_ksplit;
  n = (n + kXcds - 1) / kXcds * kXcds;
  return (unsigned)n;
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
// the divisor s of nk (s <= 16, an even number of at least 4 steps per range, as the K loop's tail
// expects) with the smallest ceil(items * s / CUs) / s, i.e. the fewest rounds of work per range,
// each range's partial sums (part_frac of an item's weight bytes, written and read back once)
// counted against it.
int tile_ksplit(int64_t items, int nk, double part_frac) {
  if (items <= 0 || items >= kCUs) return 1;
  int best = 1;
  double best_cost = 1.0;
  for (int sp = 2; sp <= 16; ++sp) {
    if (nk % sp || nk / sp < 4 || (nk / sp) % 2) continue;
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
  TileArgs p{g.group_offsets, g.row_index, g.tiles, g.counters, g.max_rows, w, x, h, 1, nullptr, H, I, I / 128,
             1, nullptr};
  gateup_tile_kernel<<<grid_for(g.max_tiles, p.n_ntiles), kThreads, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_down_tile_bf16(const Groups& g, const Weights& w, const uint16_t* h, void* y_rows, bool y_bf16,
                                 const float* row_scale, float* part, int H, int I, hipStream_t s) {
  const int split = down_tile_ksplit(g.max_rows, g.n_groups, H, I);
  if (split > 1 && !part) return hipErrorInvalidValue;
  TileArgs p{g.group_offsets, nullptr, g.tiles, g.counters, g.max_rows, w, h, y_rows, y_bf16 ? 1 : 0, row_scale,
             H, I, (H + 255) / 256, split, part};
  down_tile_kernel<<<grid_for(g.max_tiles, p.n_ntiles, split), kThreads, 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || split == 1) return e;
  const int64_t n = g.max_rows * (H / 8);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  ksplit_reduce_kernel<<<(unsigned)blocks, 256, 0, s>>>(part, split, g.group_offsets, g.n_groups, g.max_rows,
                                                        g.stream_rows, H, y_rows, y_bf16 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace moe
