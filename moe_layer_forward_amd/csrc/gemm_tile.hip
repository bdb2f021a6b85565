// Grouped SwiGLU expert GEMMs for many rows per expert (prefill-like shapes), bf16 MFMA.
//
// The experts are the SwiGLU FFNs of "Kimi K2.5 模型架构深度拆解" §4.3 / §10.2 Steps 5-6
// (gate + up -> SiLU -> multiply -> down), batched over experts as the grouped GEMM that
// "Kimi K2.5 架构 QA" Q8.3 names in place of the per-expert loop.
//
// Work item = (row tile of one group, column tile).  The row tiles come from the device-side plan
// (largest groups first, 256 rows each, so a K2 expert's ~170 prefill rows are one tile and every
// weight byte is read once); a work-group stages the tile's rows -- gathered straight from the token
// rows through row_index, so no permuted copy of x is ever written -- and a 256-row slice of the
// weights through LDS, and runs the MFMA main loop of tile_core.h, which skips the 32-row
// sub-tiles past the group's end.
//   gate/up: the 256 weight rows are 128 gate rows and the 128 matching up rows, interleaved in
//            32-row blocks, so column sub-tiles 2p and 2p+1 of a wave are the gate and up columns of
//            the same 32 h columns, in the same lanes; the epilogue writes h = SiLU(g) * u as bf16.
//   down:    256 rows of W_down; the epilogue writes y_rows (fp32 or bf16), times row_scale if given.
// Work items are dealt XCD-major (tile_core.h) so the column tiles of one row tile run on the same
// XCD at the same time and share its rows of A in that XCD's L2 while each weight byte is read once.
#include "tile_core.h"

namespace moe {
namespace {

using S = TileShape<kTileM, 256, 64, 2>;
static_assert(S::kRowsPerLoad * S::kBLoads == 32, "wave w loads B rows [32w, 32w+32): one gate or up block");

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
};

struct TileRows {
  int g;
  int64_t rbeg, rend;
};

__device__ __forceinline__ bool tile_of(const TileArgs& p, int& nt, TileRows& t) {
  int64_t L;
  if (!xcd_work_item((int64_t)p.counters[1] * p.n_ntiles, L)) return false;
  const int tile = (int)(L / p.n_ntiles);
  nt = (int)(L % p.n_ntiles);
  t.g = p.tiles[2 * tile];
  const int m0 = p.tiles[2 * tile + 1];
  int64_t r0 = p.group_offsets[t.g], r1 = p.group_offsets[t.g + 1];
  if (r0 > p.max_rows) r0 = p.max_rows;
  if (r1 > p.max_rows) r1 = p.max_rows;
  if (r1 < r0) r1 = r0;
  t.rbeg = r0 + m0;
  t.rend = t.rbeg + S::BM < r1 ? t.rbeg + S::BM : r1;
  return t.rbeg < t.rend;
}

__global__ __launch_bounds__(512) void gateup_tile_kernel(TileArgs p) {
  __shared__ __align__(16) char smem[S::kSmemBytes];
  int nt;
  TileRows t;
  if (!tile_of(p, nt, t)) return;
  const int H = p.H, I = p.I;
  const bool sh = t.g == p.w.shared_group;
  const uint16_t* wg = sh ? (const uint16_t*)p.w.s_gate : (const uint16_t*)p.w.gate + (int64_t)t.g * I * H;
  const uint16_t* wu = sh ? (const uint16_t*)p.w.s_up : (const uint16_t*)p.w.up + (int64_t)t.g * I * H;
  const int n0 = nt * (S::BN / 2);  // first h column of this tile (128 per tile)

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  Operands<S> o;
  o.a_base = reinterpret_cast<const char*>(p.a);
  // B rows (virtual columns) are 32-row blocks alternating gate / up; wave w loads block w, so its
  // rows are gate rows when w is even and up rows when w is odd.  With the 2x4 wave grid every
  // wave's two 32-column sub-tiles are then a gate block and the matching up block.  Virtual column
  // vc holds h column n0 + 32*(vc/64) + vc%32.
  const bool up_rows = __builtin_amdgcn_readfirstlane(w & 1) != 0;
  o.b_base = reinterpret_cast<const char*>((up_rows ? wu : wg) + (int64_t)n0 * H);
#pragma unroll
  for (int j = 0; j < S::kALoads; ++j) {
    const int rl = S::load_row(w, j, lane, S::kALoads);
    const int64_t r = t.rbeg + rl;
    const int64_t rr = r < t.rend ? r : t.rbeg;  // rows past the group end re-read its first row
    const int64_t src = p.row_index ? (int64_t)p.row_index[rr] : rr;
    o.a_off[j] = (uint32_t)((src * H + 8 * S::load_chunk(rl, lane)) * 2);
  }
#pragma unroll
  for (int j = 0; j < S::kBLoads; ++j) {
    const int vc = S::load_row(w, j, lane, S::kBLoads);
    const int n = (vc >> 6) * 32 + (vc & 31);
    o.b_off[j] = (uint32_t)(((int64_t)n * H + 8 * S::load_chunk(vc, lane)) * 2);
  }
  f32x16 acc[S::kMSub][S::kNSub];
  const int m_valid = (int)(t.rend - t.rbeg);
  tile_mainloop<S>(o, m_valid, H, smem, acc);

  const int wave = w, wm = wave >> 2, wn = wave & 3;
  uint16_t* h = static_cast<uint16_t*>(p.out);
  const int nsv = (m_valid + 31) / 32;
#pragma unroll
  for (int i = 0; i < S::kMSub; ++i) {
    if (2 * i + wm >= nsv) continue;
#pragma unroll
    for (int pr = 0; pr < S::kNSub / 2; ++pr) {
      const int col = n0 + wn * (S::kWaveN / 2) + pr * 32 + (lane & 31);  // kWaveN/2 = 32 h columns
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t r = t.rbeg + S::sub_row(wm, i) + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        if (r < t.rend) h[r * I + col] = f32_to_bf16(swiglu_f32(acc[i][2 * pr][q], acc[i][2 * pr + 1][q]));
      }
    }
  }
}

__global__ __launch_bounds__(512) void down_tile_kernel(TileArgs p) {
  __shared__ __align__(16) char smem[S::kSmemBytes];
  int nt;
  TileRows t;
  if (!tile_of(p, nt, t)) return;
  const int H = p.H, I = p.I;
  const uint16_t* wd = t.g == p.w.shared_group ? (const uint16_t*)p.w.s_down
                                                : (const uint16_t*)p.w.down + (int64_t)t.g * H * I;
  const int n0 = nt * S::BN;

  const int tid = threadIdx.x, w = tid >> 6;
  Operands<S> o;
  o.a_base = reinterpret_cast<const char*>(p.a);
  o.b_base = reinterpret_cast<const char*>(wd);
#pragma unroll
  for (int j = 0; j < S::kALoads; ++j) {
    const int rl = S::load_row(w, j, tid & 63, S::kALoads);
    const int64_t r = t.rbeg + rl;
    o.a_off[j] = (uint32_t)(((r < t.rend ? r : t.rbeg) * I + 8 * S::load_chunk(rl, tid & 63)) * 2);
  }
#pragma unroll
  for (int j = 0; j < S::kBLoads; ++j) {
    const int vc = S::load_row(w, j, tid & 63, S::kBLoads);
    const int n = n0 + vc;  // columns past H (last tile) read row 0, never stored
    o.b_off[j] = (uint32_t)(((int64_t)(n < H ? n : 0) * I + 8 * S::load_chunk(vc, tid & 63)) * 2);
  }
  f32x16 acc[S::kMSub][S::kNSub];
  const int m_valid = (int)(t.rend - t.rbeg);
  tile_mainloop<S>(o, m_valid, I, smem, acc);

  const int lane = tid & 63, wave = w, wm = wave >> 2, wn = wave & 3;
#pragma unroll
  for (int i = 0; i < S::kMSub; ++i) {
    if (2 * i + wm >= (m_valid + 31) / 32) continue;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int64_t r = t.rbeg + S::sub_row(wm, i) + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
      if (r >= t.rend) continue;
      const float sc = p.row_scale ? p.row_scale[r] : 1.f;
#pragma unroll
      for (int u = 0; u < S::kNSub; ++u) {
        const int col = n0 + wn * S::kWaveN + 32 * u + (lane & 31);
        if (col >= H) continue;
        const float v = acc[i][u][q] * sc;
        if (p.out_bf16)
          static_cast<uint16_t*>(p.out)[r * H + col] = f32_to_bf16(v);
        else
          static_cast<float*>(p.out)[r * H + col] = v;
      }
    }
  }
}

unsigned grid_for(int64_t max_tiles, int n_ntiles) {
  int64_t n = max_tiles * n_ntiles;
  n = (n + kXcds - 1) / kXcds * kXcds;
  return (unsigned)n;
}

}  // namespace

hipError_t launch_gateup_tile_bf16(const Groups& g, const Weights& w, const uint16_t* x, uint16_t* h, int H, int I,
                                   hipStream_t s) {
  TileArgs p{g.group_offsets, g.row_index, g.tiles, g.counters, g.max_rows, w, x, h, 1, nullptr, H, I,
             I / (S::BN / 2)};
  gateup_tile_kernel<<<grid_for(g.max_tiles, p.n_ntiles), S::kThreads, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_down_tile_bf16(const Groups& g, const Weights& w, const uint16_t* h, void* y_rows, bool y_bf16,
                                 const float* row_scale, int H, int I, hipStream_t s) {
  TileArgs p{g.group_offsets, nullptr, g.tiles, g.counters, g.max_rows, w, h, y_rows, y_bf16 ? 1 : 0, row_scale,
             H, I, (H + S::BN - 1) / S::BN};
  down_tile_kernel<<<grid_for(g.max_tiles, p.n_ntiles), S::kThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
