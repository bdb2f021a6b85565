// Grouped SwiGLU tile GEMMs with 4-bit routed-expert weights: the FP8 tiles' schedule (tile_gemm.h)
// over 4-bit codes and binary16 scales per 32 inputs, decoded in registers.
#include "tile_gemm.h"

namespace moe {
namespace {

// ----------------------------------------------------------------------------- 4-bit routed experts
// The routed experts' weights as the 4-bit stream kernels read them: codes [E, N, K / 8] 32-bit words
// (input k's two's-complement code q in bits 4 (k mod 8) .. + 3 of word k / 8), binary16 scales
// [E, N, K / 32], w = q s ("Kimi K2.5 模型架构深度拆解" §7.2: symmetric 4-bit integers, one scale per
// group of 32 inputs).  The FP8 tiles' tiles, waves, token-row rings, load schedule and software
// pipelining; what changes:
//   * A K block is 128 inputs (two K steps): 64 bytes of codes and 4 scales (8 bytes) per weight row.
//     A B stage holds the codes of the 256 weight rows (16 KiB) and their scales (2 KiB) in the first
//     18 KiB of an FP8 code stage.  Per wave and block: 2 code pieces of 16 rows x 64 bytes (16-byte
//     lanes) and one scale piece of 32 rows x 8 bytes (4-byte lanes), 3 loads.
//   * LDS: 16-byte chunk c (0 .. 3) of a 64-byte code row r sits at c ^ ((r >> 2) & 3), so the 8-byte
//     reads of two 16-lane groups (the 16 rows of a column block, both halves of one chunk) fall in
//     all 64 banks.
//   * A lane of group g (lane / 16) takes inputs 16 g .. 16 g + 15 of a step, as in the FP8 tiles:
//     two words of codes (k-substeps 0 and 1) and one scale (group (64 (kt mod 2) + 16 g) / 32 of the
//     block) per column block and step.
//   * Decoding: the stream kernels' bit trick turns a word into 1024 + u and 64 + u (u = q + 8) as
//     binary16 in the operand order 0,4,1,5,2,6,3,7; a packed subtraction of 1032 / 72 leaves q
//     exactly, and a packed multiply by the scale gives the weight f16(q s) (one rounding: within 2^-11
//     of q s relative, binary16 subnormals below 2^-14 absolute).  13 operations per 8 weights.
constexpr int kQ4Loads = 3;                // loads per wave per K block
constexpr int kQ4ScaleOff = 256 * 64;      // the scale rows' place in a B stage
constexpr int kQ4RowBytes = 64;            // code bytes per weight row per K block

__device__ __forceinline__ int swz4(int r) { return (r >> 2) & 3; }

// Per-wave LDS read geometry of the 4-bit tiles, as per-lane offsets that include the wave's first A
// block and first weight row b0 (a multiple of 16): A as QFrag; the codes of step half hf (bytes
// 32 hf + 8 g .. of a row's 64) and the scale of group 2 hf + g / 2, of row b0 + x.  Column block s
// starts kQ4Col<GU>(s) rows further, a constant folded into the reads' offsets.
struct Q4Frag {
  uint32_t a_off[2];
  uint32_t c_off[2];
  uint32_t s_off[2];
};

// Weight rows of column block s past the wave's first: gate/up {gate rows, gate rows + 16, up rows,
// up rows + 16} of the wave's 32 h columns; down 4 consecutive 16-row blocks.
template <bool GU>
constexpr int kQ4Col(int s) {
  return GU ? (s & 1) * 16 + (s >> 1) * 128 : 16 * s;
}

__device__ __forceinline__ Q4Frag make_q4frag(int wr, int b0) {
  const int lane = threadIdx.x & 63, x = lane & 15, g = lane >> 4;
  Q4Frag f;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    f.a_off[kk] = (uint32_t)(wr * 16 * kRowBytes + x * kRowBytes + (((2 * g + kk) ^ swz(x)) << 4));
    // column blocks start at multiples of 16 rows, so row b0 + kQ4Col(s) + x swizzles as x does
    f.c_off[kk] = (uint32_t)((b0 + x) * kQ4RowBytes + (((2 * kk + (g >> 1)) ^ swz4(x)) << 4) + 8 * (g & 1));
    f.s_off[kk] = (uint32_t)(kQ4ScaleOff + (b0 + x) * 8 + 2 * (2 * kk + (g >> 1)));
  }
  return f;
}

// K block b of the 256 weight rows: code pieces w and w + 8 (tile rows 16 p .. 16 p + 15) through
// b_base/b_off[0, 1], scale piece w (tile rows 32 w .. 32 w + 31) through b_base/b_off[2].
__device__ __forceinline__ void issue_q4block(const Loads& o, int b, char* stage) {
  const int w = o.wave;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(operand_rsrc(o.b_base[j]), (LdsPtr)(stage + (w + kWaves * j) * 1024), 16,
                                             o.b_off[j] + (uint32_t)b * kQ4RowBytes, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(operand_rsrc(o.b_base[2]), (LdsPtr)(stage + kQ4ScaleOff + w * 256), 4,
                                           o.b_off[2] + (uint32_t)b * 8, 0, 0, 0);
}

// Lane offset of this lane's slot in a code piece (16 rows of rb code bytes): row lane / 4, the chunk
// that belongs in slot lane % 4.
__device__ __forceinline__ uint32_t q4_code_lane(int64_t rb) {
  const int lane = threadIdx.x & 63;
  return (uint32_t)((lane >> 2) * rb + 16 * ((lane & 3) ^ swz4(lane >> 2)));
}

// Lane offset in a scale piece (32 rows of rb scale bytes): row lane / 2, 4-byte half lane % 2.
__device__ __forceinline__ uint32_t q4_scale_lane(int64_t rb) {
  const int lane = threadIdx.x & 63;
  return (uint32_t)((lane >> 1) * rb + 4 * (lane & 1));
}

// One word of 8 codes -> f16(q s) in the order 0,4,1,5,2,6,3,7 (s in both halves of sc).
__device__ __forceinline__ f16x8 dequant4(uint32_t w, f16x2 sc) {
  const uint32_t w8 = w >> 8;
  const f16x2 lo = {(_Float16)-1032.f, (_Float16)-1032.f}, hi = {(_Float16)-72.f, (_Float16)-72.f};
  const f16x2 h0 = (__builtin_bit_cast(f16x2, (w & 0x000F000Fu) ^ 0x64086408u) + lo) * sc;   // codes 0, 4
  const f16x2 h1 = (__builtin_bit_cast(f16x2, (w & 0x00F000F0u) ^ 0x54805480u) + hi) * sc;   // codes 1, 5
  const f16x2 h2 = (__builtin_bit_cast(f16x2, (w8 & 0x000F000Fu) ^ 0x64086408u) + lo) * sc;  // codes 2, 6
  const f16x2 h3 = (__builtin_bit_cast(f16x2, (w8 & 0x00F000F0u) ^ 0x54805480u) + hi) * sc;  // codes 3, 7
  return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// Weights carried from one K step to the next: the first k-substep's decoded fragments of the 4 column
// blocks, the second's codes and the step's scales.
struct Q4Carry {
  f16x8 b0[4];
  uint32_t zw[4];
  f16x2 sc[4];
};

template <bool GU, int HF>
__device__ __forceinline__ void read_codes4(const char* Bs, const Q4Frag& f, u32x2 (&q)[4], f16x2 (&sc)[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    q[s] = *reinterpret_cast<const u32x2*>(Bs + f.c_off[HF] + kQ4Col<GU>(s) * kQ4RowBytes);
    const uint32_t h = *reinterpret_cast<const uint16_t*>(Bs + f.s_off[HF] + kQ4Col<GU>(s) * 8);
    sc[s] = __builtin_bit_cast(f16x2, h | (h << 16));
  }
}

// MFMAs of one K step of the 4-bit tiles, pipelined with the decoding exactly as q_compute_step, with
// the weights as the MFMA's first operand: the accumulators hold their blocks transposed, as in
// compute_step (the FP8 tiles keep the other order, which their registers need).
template <int NBW, int HF, int HFN, bool GU, bool kFirst>
__device__ __forceinline__ void q4_compute_step(const char* As, const char* Bs, const char* Bn, bool has_next,
                                                const Q4Frag& f, Q4Carry& c, f32x4 (&acc)[NBW > 0 ? NBW : 1][4]) {
  if constexpr (NBW > 0) {
    constexpr int NF = 2 * NBW;
    constexpr int kReadNext = NBW < 5 ? NBW - 1 : 4;  // fragment that reads the next step's codes
    if constexpr (kFirst) {
      u32x2 q[4];
      read_codes4<GU, HF>(Bs, f, q, c.sc);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        c.b0[s] = dequant4(q[s][0], c.sc[s]);
        c.zw[s] = q[s][1];
      }
    } else {
      (void)Bs;
    }
    auto read_a = [&](int fi) {
      return *reinterpret_cast<const f16x8*>(As + f.a_off[fi / NBW] + (fi % NBW) * 2 * 16 * kRowBytes);
    };
    f16x8 b1[4];
    u32x2 qn[4];
    f16x2 sn[4];
    f16x8 a[NF];
    a[0] = read_a(0);
    a[1] = read_a(1);
#pragma unroll
    for (int fi = 0; fi < NF; ++fi) {
      if (fi + 2 < NF) a[fi + 2] = read_a(fi + 2);
      if (fi < NBW) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          if (decode_frag<NBW>(s) == fi) b1[s] = dequant4(c.zw[s], c.sc[s]);
        if (fi == kReadNext && has_next) read_codes4<GU, HFN>(Bn, f, qn, sn);
      } else if (has_next) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          if (decode_frag<NBW>(s) == fi - NBW) {
            c.b0[s] = dequant4(qn[s][0], sn[s]);
            c.zw[s] = qn[s][1];
            c.sc[s] = sn[s];
          }
      }
      const int kk = fi / NBW, i = fi % NBW;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc[i][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kk == 0 ? c.b0[s] : b1[s], a[fi], acc[i][s], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    (void)As;
    (void)Bs;
    (void)Bn;
    (void)has_next;
    (void)f;
    (void)c;
    (void)acc;
  }
}

template <bool GU>
struct Q4Tiles {
  static constexpr int kLoads = kQ4Loads;
  typedef Q4Frag Ctx;
  typedef Q4Carry Carry;
  __device__ static __forceinline__ void issue_block(const Loads& o, int b, char* stage) { issue_q4block(o, b, stage); }
  template <int NBW, int HF, int HFN, bool kFirst>
  __device__ static __forceinline__ void step(const char* As, const char* Bs, const char* Bn, bool has_next, int kt,
                                              const Ctx& f, Carry& c, f32x4 (&acc)[NBW > 0 ? NBW : 1][4]) {
    (void)kt;
    __builtin_amdgcn_sched_barrier(0);
    q4_compute_step<NBW, HF, HFN, GU, kFirst>(As, Bs, Bn, has_next, f, c, acc);
  }
};

// Gate/up work item of a routed group with 4-bit weights: h rows in binary16 (operand order).
__device__ __forceinline__ void gateup_q4_item(const QTileArgs& q, const Rings& rings, int nt, const TileRows& t) {
  const TileArgs& p = q.p;
  const int H = p.H, I = p.I;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = w >> 2, wc = w & 3;
  const int64_t crow = H / 2, srow = H / 16;  // code and scale bytes per weight row
  const char* cg = reinterpret_cast<const char*>(q.codes0) + t.g * (int64_t)I * crow;
  const char* cu = reinterpret_cast<const char*>(q.codes1) + t.g * (int64_t)I * crow;
  const char* sg = static_cast<const char*>(q.scales0) + t.g * (int64_t)I * srow;
  const char* su = static_cast<const char*>(q.scales1) + t.g * (int64_t)I * srow;
  const int h0 = nt * 128;

  Loads o;
  o.wave = w;
  o.a_base = reinterpret_cast<const char*>(q.a16);
  a_offsets(o, H, [&](int rl) -> int64_t {
    const int64_t r = t.rbeg + rl;
    const int64_t rr = r < t.rend ? r : t.rbeg;
    return p.row_index ? (int64_t)p.row_index[rr] : rr;
  });
  // code pieces w (tile rows 16 w ..: gate rows h0 + 16 w ..) and w + 8 (tile rows 128 + 16 w ..: the
  // same up rows); scale piece w: tile rows 32 w .., gate rows for w < 4, up rows after
  o.b_base[0] = cg + (int64_t)(h0 + 16 * w) * crow;
  o.b_base[1] = cu + (int64_t)(h0 + 16 * w) * crow;
  o.b_base[2] = (w < 4 ? sg : su) + (int64_t)(h0 + 32 * (w & 3)) * srow;
  o.b_base[3] = o.b_base[2];
  o.b_off[0] = o.b_off[1] = q4_code_lane(crow);
  o.b_off[2] = q4_scale_lane(srow);
  o.b_off[3] = 0;
  o.nk = H / kBK;
  o.skew = 0;

  const Q4Frag f = make_q4frag(wr, 32 * wc);
  uint16_t* h = static_cast<uint16_t*>(p.out);
  const int64_t rbeg = t.rbeg;
  const int m_valid = (int)(t.rend - t.rbeg);
  const auto epilogue = [&](auto nbw_c, const auto& acc) {
    constexpr int NBW = decltype(nbw_c)::value;
    using Out = OutTile<128>;
    block_sync_lds();  // every wave is done reading the rings
    static_for<NBW>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int row = 16 * (wr + 2 * i) + (lane & 15);  // accumulators transposed, as in compute_step
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Out::put_f16_pairs(rings, row, 32 * wc + 16 * s + 4 * (lane >> 4) + e,
                             swiglu_f32(acc[i][s][e], acc[i][s + 2][e]));
    });
    block_sync_lds();
    Out::store(rings, m_valid, h, I, rbeg, h0, I);
  };
  const QRings qr{{rings.a[0], rings.a[1], rings.b[0]}, {rings.b[1], rings.b[2]}};
  run_tile<kTileMQ4 / 32>((m_valid + 15) / 16, wr, [&](auto b, auto a) {
    q_tile_body<Q4Tiles<true>, decltype(b)::value, decltype(a)::value>(o, qr, f, epilogue);
  });
}

// Down work item of a routed group with 4-bit weights: y rows in bf16.  H is a multiple of 256, so
// every column slab is whole.
__device__ __forceinline__ void down_q4_item(const QTileArgs& q, const Rings& rings, int nt, const TileRows& t) {
  const TileArgs& p = q.p;
  const int H = p.H, I = p.I;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wr = w >> 2, wc = w & 3;
  const int64_t crow = I / 2, srow = I / 16;
  const char* cd = reinterpret_cast<const char*>(q.codes0) + t.g * (int64_t)H * crow;
  const char* sd = static_cast<const char*>(q.scales0) + t.g * (int64_t)H * srow;
  const int n0 = nt * 256;

  Loads o;
  o.wave = w;
  o.a_base = reinterpret_cast<const char*>(q.a16);
  a_offsets(o, I, [&](int rl) -> int64_t {
    const int64_t r = t.rbeg + rl;
    return r < t.rend ? r : t.rbeg;
  });
  // code pieces w, w + 8: W_down rows n0 + 16 w .., n0 + 128 + 16 w ..; scale piece w: rows n0 + 32 w ..
  o.b_base[0] = cd + (int64_t)(n0 + 16 * w) * crow;
  o.b_base[1] = cd + (int64_t)(n0 + 128 + 16 * w) * crow;
  o.b_base[2] = sd + (int64_t)(n0 + 32 * w) * srow;
  o.b_base[3] = o.b_base[2];
  o.b_off[0] = o.b_off[1] = q4_code_lane(crow);
  o.b_off[2] = q4_scale_lane(srow);
  o.b_off[3] = 0;
  o.nk = I / kBK;
  o.skew = 0;

  const Q4Frag f = make_q4frag(wr, 64 * wc);
  const int64_t rbeg = t.rbeg;
  const int m_valid = (int)(t.rend - t.rbeg);
  uint16_t* y = static_cast<uint16_t*>(p.out);
  const auto epilogue = [&](auto nbw_c, const auto& acc) {
    constexpr int NBW = decltype(nbw_c)::value;
    using Out = OutTile<256>;
    block_sync_lds();
    static_for<NBW>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int row = 16 * (wr + 2 * i) + (lane & 15);  // accumulators transposed, as in compute_step
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
  run_tile<kTileMQ4 / 32>((m_valid + 15) / 16, wr, [&](auto b, auto a) {
    q_tile_body<Q4Tiles<false>, decltype(b)::value, decltype(a)::value>(o, qr, f, epilogue);
  });
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gateup_tile_q4_kernel(
    QTileArgs q) {
  MOE_TILE_SMEM
  int nt, ks;
  TileRows t;
  if (!tile_of(q.p, nt, ks, t)) return;
  if (t.g == q.p.w.shared_group)
    gateup_bf16_item(q.p, rings, nt, t);
  else
    gateup_q4_item(q, rings, nt, t);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void down_tile_q4_kernel(
    QTileArgs q) {
  MOE_TILE_SMEM
  int nt, ks;
  TileRows t;
  if (!tile_of(q.p, nt, ks, t)) return;
  if (t.g == q.p.w.shared_group)
    down_bf16_item(q.p, rings, nt, 0, t);
  else
    down_q4_item(q, rings, nt, t);
}

}  // namespace

hipError_t launch_gateup_tile_q4(const Groups& g, const Weights& w, const QWeights& q, const uint16_t* x,
                                 const uint16_t* x16, uint16_t* h, int H, int I, hipStream_t s) {
  if (q.format != QFormat::kInt4 || !tile_quant_shape_ok(q.format, H, I) || g.tile_m != kTileMQ4)
    return hipErrorInvalidValue;
  QTileArgs a{{g.group_offsets, g.row_index, g.tiles, g.counters, g.max_rows, w, x, h, 1, nullptr, H, I, I / 128, 1,
               nullptr, kTileMQ4},
              x16,
              static_cast<const uint8_t*>(q.gate_codes),
              static_cast<const uint8_t*>(q.up_codes),
              q.gate_scales,
              q.up_scales};
  gateup_tile_q4_kernel<<<grid_for(g.max_tiles, a.p.n_ntiles), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_down_tile_q4(const Groups& g, const Weights& w, const QWeights& q, const uint16_t* h,
                               uint16_t* y_rows, int H, int I, hipStream_t s) {
  if (q.format != QFormat::kInt4 || !tile_quant_shape_ok(q.format, H, I) || g.tile_m != kTileMQ4)
    return hipErrorInvalidValue;
  QTileArgs a{{g.group_offsets, nullptr, g.tiles, g.counters, g.max_rows, w, h, y_rows, 1, nullptr, H, I,
               (H + 255) / 256, 1, nullptr, kTileMQ4},
              h,
              static_cast<const uint8_t*>(q.down_codes),
              nullptr,
              q.down_scales,
              nullptr};
  down_tile_q4_kernel<<<grid_for(g.max_tiles, a.p.n_ntiles), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe
