// Grouped SwiGLU tile GEMMs with bf16 or FP8 routed-expert weights (the tiles, rings and dealing are
// described in tile_gemm.h), the K-range reduction, and the launchers of the tile kernels.
#include "tile_gemm.h"

namespace moe {
namespace {

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

// Reads the 16 codes per column block of step half HF of a B stage.
template <int HF>
__device__ __forceinline__ void read_codes(const char* Bs, const QFrag& f, u32x4 (&q)[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) q[s] = *reinterpret_cast<const u32x4*>(Bs + f.b_row0[s] + f.b_off[HF]);
}

// MFMAs of one K step, in compute_step's fragment order, software-pipelined with the decoding (the down
// GEMM with the weights as the MFMA's first operand, its accumulators transposed as in compute_step;
// the gate/up GEMM in the plain order, which its registers need): the
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
        acc[i][s] = GU ? __builtin_amdgcn_mfma_f32_16x16x32_f16(a[fi], kk == 0 ? c.b0[s] : b1[s], acc[i][s], 0, 0, 0)
                       : __builtin_amdgcn_mfma_f32_16x16x32_f16(kk == 0 ? c.b0[s] : b1[s], a[fi], acc[i][s], 0, 0, 0);
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

// The FP8 format of the quantized tiles (the code above): a K block is 128 codes of each weight row,
// 4 loads per wave; block scales one per lane, picked per step with v_readlane.
template <bool GU>
struct Fp8Tiles {
  static constexpr int kLoads = kBLoads;
  static constexpr int NS = GU ? 2 : 1;
  struct Ctx {
    QFrag f;
    LaneScale ls[NS];
  };
  typedef QCarry Carry;
  __device__ static __forceinline__ void issue_block(const Loads& o, int b, char* stage) { issue_qblock(o, b, stage); }
  template <int NBW, int HF, int HFN, bool kFirst>
  __device__ static __forceinline__ void step(const char* As, const char* Bs, const char* Bn, bool has_next, int kt,
                                              const Ctx& x, Carry& c, f32x4 (&acc)[NBW > 0 ? NBW : 1][4]) {
    const StepScale<NS> sc = step_scale(x.ls, kt >> 1);
    const StepScale<NS> scn = step_scale(x.ls, has_next ? (kt + 1) >> 1 : kt >> 1);
    __builtin_amdgcn_sched_barrier(0);
    q_compute_step<NBW, HF, HFN, GU, kFirst>(As, Bs, Bn, has_next, x.f, sc, scn, c, acc);
  }
};

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
  const float* sg = static_cast<const float*>(q.scales0);
  const float* su = static_cast<const float*>(q.scales1);
  const int b_rows[4] = {32 * wc, 32 * wc + 16, 128 + 32 * wc, 128 + 32 * wc + 16};
  const Fp8Tiles<true>::Ctx x{make_qfrag(wr, b_rows),
                              {lane_scale(sg + ((int64_t)t.g * (I / 128) + nt) * nkb, nkb),
                               lane_scale(su + ((int64_t)t.g * (I / 128) + nt) * nkb, nkb)}};
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
    q_tile_body<Fp8Tiles<true>, decltype(b)::value, decltype(a)::value>(o, qr, x, epilogue);
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
  const int b_rows[4] = {64 * wc, 64 * wc + 16, 64 * wc + 32, 64 * wc + 48};
  const Fp8Tiles<false>::Ctx x{make_qfrag(wr, b_rows),
                               {lane_scale(static_cast<const float*>(q.scales0) + ((int64_t)t.g * (H / 128) + rb) * nkb,
                                           nkb)}};
  const int64_t rbeg = t.rbeg;
  const int m_valid = (int)(t.rend - t.rbeg);
  uint16_t* y = static_cast<uint16_t*>(p.out);
  const auto epilogue = [&](auto nbw_c, const auto& acc) {
    constexpr int NBW = decltype(nbw_c)::value;
    using Out = OutTile<256>;
    block_sync_lds();
    static_for<NBW>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int row = 16 * (wr + 2 * i) + (lane & 15);  // accumulators transposed (q_compute_step, !GU)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const float v[4] = {acc[i][s][0], acc[i][s][1], acc[i][s][2], acc[i][s][3]};
        Out::put4(rings, row, 64 * wc + 16 * s + 4 * (lane >> 4), v);
      }
    });
    block_sync_lds();
    Out::store(rings, m_valid, y, H, rbeg, n0, H);
  };
  const QRings qr{{rings.a[0], rings.a[1], rings.b[0]}, {rings.b[1], rings.b[2]}};
  run_tile<kTileMFp8 / 32>((m_valid + 15) / 16, wr, [&](auto b, auto a) {
    q_tile_body<Fp8Tiles<false>, decltype(b)::value, decltype(a)::value>(o, qr, x, epilogue);
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

bool tile_quant_shape_ok(QFormat f, int H, int I) {
  if (f == QFormat::kInt4) return H > 0 && I > 0 && H % 256 == 0 && I % 256 == 0;
  return H > 0 && I > 0 && H % 128 == 0 && I % 128 == 0 && H <= 128 * 64 && I <= 128 * 64;
}

hipError_t launch_gateup_tile_quant(const Groups& g, const Weights& w, const QWeights& q, const uint16_t* x,
                                    const uint16_t* x16, uint16_t* h, int H, int I, hipStream_t s) {
  if (q.format == QFormat::kInt4) return launch_gateup_tile_q4(g, w, q, x, x16, h, H, I, s);
  if (!tile_quant_shape_ok(q.format, H, I) || g.tile_m != kTileMFp8) return hipErrorInvalidValue;
  QTileArgs a{{g.group_offsets, g.row_index, g.tiles, g.counters, g.max_rows, w, x, h, 1, nullptr, H, I, I / 128, 1,
               nullptr, kTileMFp8},
              x16,
              static_cast<const uint8_t*>(q.gate_codes),
              static_cast<const uint8_t*>(q.up_codes),
              q.gate_scales,
              q.up_scales};
  gateup_tile_fp8_kernel<<<grid_for(g.max_tiles, a.p.n_ntiles), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_down_tile_quant(const Groups& g, const Weights& w, const QWeights& q, const uint16_t* h,
                                  uint16_t* y_rows, int H, int I, hipStream_t s) {
  if (q.format == QFormat::kInt4) return launch_down_tile_q4(g, w, q, h, y_rows, H, I, s);
  if (!tile_quant_shape_ok(q.format, H, I) || g.tile_m != kTileMFp8) return hipErrorInvalidValue;
  QTileArgs a{{g.group_offsets, nullptr, g.tiles, g.counters, g.max_rows, w, h, y_rows, 1, nullptr, H, I,
               (H + 255) / 256, 1, nullptr, kTileMFp8},
              h,
              static_cast<const uint8_t*>(q.down_codes),
              nullptr,
              q.down_scales,
              nullptr};
  down_tile_fp8_kernel<<<grid_for(g.max_tiles, a.p.n_ntiles), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
