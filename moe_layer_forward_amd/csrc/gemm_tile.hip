// Grouped SwiGLU expert GEMMs for many rows per expert (prefill-like shapes), bf16 MFMA.
//
// The experts are the SwiGLU FFNs of "Kimi K2.5 模型架构深度拆解" §4.3 / §10.2 Steps 5-6
// (gate + up -> SiLU -> multiply -> down), batched over experts as the grouped GEMM that
// "Kimi K2.5 架构 QA" Q8.3 names in place of the per-expert loop.
//
// Work item = (row tile of one group, column tile).  The row tiles come from the device-side plan
// (largest groups first); a work-group stages 128 rows of its group -- gathered straight from the
// token rows through row_index, so no permuted copy of x is ever written -- and a 128-row slice of
// the weights through LDS, and runs the MFMA main loop of tile_core.h.
//   gate/up: the 128 weight rows are 64 gate rows and the 64 matching up rows, interleaved in
//            16-row blocks so each wave ends with gate and up accumulators of the same h columns in
//            the same lanes; the epilogue writes h = SiLU(g) * u as bf16.
//   down:    128 rows of W_down; the epilogue writes y_rows (fp32 or bf16), times row_scale if given.
// Work items are dealt XCD-major (tile_core.h) so the column tiles of one row tile run on the same
// XCD at the same time and share its rows of A in that XCD's L2 while each weight byte is read once.
#include "tile_core.h"

namespace moe {
namespace {

using S = TileShape<kTileM, 128, 64>;

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

__device__ __forceinline__ void group_rows(const int32_t* off, int64_t max_rows, int g, int64_t& r0, int64_t& r1) {
  r0 = off[g];
  r1 = off[g + 1];
  if (r0 > max_rows) r0 = max_rows;
  if (r1 > max_rows) r1 = max_rows;
  if (r1 < r0) r1 = r0;
}

__global__ __launch_bounds__(256) void gateup_tile_kernel(TileArgs p) {
  __shared__ __align__(16) uint16_t smem[S::kSmemBytes / 2];
  int64_t L;
  if (!xcd_work_item((int64_t)p.counters[1] * p.n_ntiles, L)) return;
  const int tile = (int)(L / p.n_ntiles), nt = (int)(L % p.n_ntiles);
  const int g = p.tiles[2 * tile], m0 = p.tiles[2 * tile + 1];
  int64_t r0, r1;
  group_rows(p.group_offsets, p.max_rows, g, r0, r1);
  const int64_t rbeg = r0 + m0;
  const int64_t rend = rbeg + S::BM < r1 ? rbeg + S::BM : r1;
  const int H = p.H, I = p.I;
  const bool sh = g == p.w.shared_group;
  const uint16_t* wg = sh ? (const uint16_t*)p.w.s_gate : (const uint16_t*)p.w.gate + (int64_t)g * I * H;
  const uint16_t* wu = sh ? (const uint16_t*)p.w.s_up : (const uint16_t*)p.w.up + (int64_t)g * I * H;
  const int n0 = nt * 64;  // first h column of this tile

  const int tid = threadIdx.x;
  const uint16_t* aptr[S::kALoads];
  const uint16_t* bptr[S::kBLoads];
  uint32_t amask = 0;
#pragma unroll
  for (int j = 0; j < S::kALoads; ++j) {
    const int64_t r = rbeg + S::stage_row(tid, j);
    const bool ok = r < rend;
    const int64_t src = ok ? (p.row_index ? (int64_t)p.row_index[r] : r) : 0;
    amask |= (ok ? 1u : 0u) << j;
    aptr[j] = p.a + src * H + S::stage_col(tid, j);
  }
#pragma unroll
  for (int j = 0; j < S::kBLoads; ++j) {
    const int vc = S::stage_row(tid, j);  // virtual column: 16 gate rows, 16 up rows, ...
    const int n = n0 + (vc >> 5) * 16 + (vc & 15);
    bptr[j] = ((vc >> 4) & 1 ? wu : wg) + (int64_t)n * H + S::stage_col(tid, j);
  }
  f32x4 acc[S::kMI][S::kNI];
  tile_mainloop<S>(aptr, bptr, amask, 0xffffffffu, H, smem, acc);

  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  uint16_t* h = static_cast<uint16_t*>(p.out);
#pragma unroll
  for (int mi = 0; mi < S::kMI; ++mi)
#pragma unroll
    for (int pr = 0; pr < S::kNI / 2; ++pr) {
      const int col = n0 + (2 * wn + pr) * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = rbeg + wm * S::kWaveM + mi * 16 + 4 * (lane >> 4) + i;
        if (r < rend) h[r * I + col] = f32_to_bf16(swiglu_f32(acc[mi][2 * pr][i], acc[mi][2 * pr + 1][i]));
      }
    }
}

__global__ __launch_bounds__(256) void down_tile_kernel(TileArgs p) {
  __shared__ __align__(16) uint16_t smem[S::kSmemBytes / 2];
  int64_t L;
  if (!xcd_work_item((int64_t)p.counters[1] * p.n_ntiles, L)) return;
  const int tile = (int)(L / p.n_ntiles), nt = (int)(L % p.n_ntiles);
  const int g = p.tiles[2 * tile], m0 = p.tiles[2 * tile + 1];
  int64_t r0, r1;
  group_rows(p.group_offsets, p.max_rows, g, r0, r1);
  const int64_t rbeg = r0 + m0;
  const int64_t rend = rbeg + S::BM < r1 ? rbeg + S::BM : r1;
  const int H = p.H, I = p.I;
  const uint16_t* wd = g == p.w.shared_group ? (const uint16_t*)p.w.s_down
                                              : (const uint16_t*)p.w.down + (int64_t)g * H * I;
  const int n0 = nt * S::BN;

  const int tid = threadIdx.x;
  const uint16_t* aptr[S::kALoads];
  const uint16_t* bptr[S::kBLoads];
  uint32_t amask = 0;
#pragma unroll
  for (int j = 0; j < S::kALoads; ++j) {
    const int64_t r = rbeg + S::stage_row(tid, j);
    const bool ok = r < rend;
    amask |= (ok ? 1u : 0u) << j;
    aptr[j] = p.a + (ok ? r : rbeg) * I + S::stage_col(tid, j);
  }
#pragma unroll
  for (int j = 0; j < S::kBLoads; ++j)
    bptr[j] = wd + (int64_t)(n0 + S::stage_row(tid, j)) * I + S::stage_col(tid, j);
  f32x4 acc[S::kMI][S::kNI];
  tile_mainloop<S>(aptr, bptr, amask, 0xffffffffu, I, smem, acc);

  const int lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int mi = 0; mi < S::kMI; ++mi)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = rbeg + wm * S::kWaveM + mi * 16 + 4 * (lane >> 4) + i;
      if (r >= rend) continue;
      const float sc = p.row_scale ? p.row_scale[r] : 1.f;
#pragma unroll
      for (int ni = 0; ni < S::kNI; ++ni) {
        const int col = n0 + wn * S::kWaveN + ni * 16 + (lane & 15);
        const float v = acc[mi][ni][i] * sc;
        if (p.out_bf16)
          static_cast<uint16_t*>(p.out)[r * H + col] = f32_to_bf16(v);
        else
          static_cast<float*>(p.out)[r * H + col] = v;
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
  TileArgs p{g.group_offsets, g.row_index, g.tiles, g.counters, g.max_rows, w, x, h, 1, nullptr, H, I, I / 64};
  gateup_tile_kernel<<<grid_for(g.max_tiles, p.n_ntiles), S::kThreads, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_down_tile_bf16(const Groups& g, const Weights& w, const uint16_t* h, void* y_rows, bool y_bf16,
                                 const float* row_scale, int H, int I, hipStream_t s) {
  TileArgs p{g.group_offsets, nullptr, g.tiles, g.counters, g.max_rows, w, h, y_rows, y_bf16 ? 1 : 0, row_scale,
             H, I, H / S::BN};
  down_tile_kernel<<<grid_for(g.max_tiles, p.n_ntiles), S::kThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
