// Grouped SwiGLU expert GEMMs for few rows per expert (decode-like shapes): weight streaming.
//
// Experts as in "Kimi K2.5 模型架构深度拆解" §4.3 / §10.2 Steps 5-6, batched over the experts present
// (the grouped GEMM of "Kimi K2.5 架构 QA" Q8.3).  With ~1-2 tokens per expert every weight byte is
// used once or twice, so the kernel is a weight stream: each weight row is read exactly once per
// 16-row pass, straight from HBM into the MFMA B operand (no LDS), and the handful of token rows ride
// along as the A operand from L2.
//
// A wave owns 16 output columns of one group: 16 gate rows + the 16 matching up rows (gate/up) or 16
// rows of W_down (down).  A 128-wide K step of a weight row is 256 bytes; load j (j = 0..3) of lane l
// takes bytes 64*j + 16*(l/16) .. +16 of row l%16, so each load covers 64 contiguous bytes of each of
// 16 rows, and load j is the B operand of the j-th 16x16x32 MFMA.  Because the K sum is order-free,
// the token rows (A operand) are read with the same K permutation, so no shuffle is needed.  The next
// step's loads are issued before the current step's MFMAs (register double buffer).  Plain loads:
// measured on MI355X, this row-strided shape streams at ~6.2 TB/s with ordinary loads and far
// slower with non-temporal ones.
// Work-groups = 4 waves = 64 columns of one group; groups come from the plan's active list, largest
// first, so the long-running many-row groups start early.
#include "kernels.h"

namespace moe {
namespace {

struct StreamArgs {
  const int32_t* group_offsets;
  const int32_t* row_index;
  const int32_t* active;
  const int32_t* counters;
  int64_t max_rows;
  Weights w;
  const uint16_t* a;
  void* out;
  int out_bf16;
  const float* row_scale;
  int H, I, n_nblk;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Frag {
  u32x4 v[4];
};

// Four 16-byte loads at p, p + 32, p + 64, p + 96 elements (64-byte stride): one K step of one row.
__device__ __forceinline__ void load_frag(Frag& f, const uint16_t* p) {
#pragma unroll
  for (int j = 0; j < 4; ++j) f.v[j] = *reinterpret_cast<const u32x4*>(p + 32 * j);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

template <bool SWIGLU>
__global__ __launch_bounds__(256) void stream_kernel(StreamArgs p) {
  const int slot = blockIdx.x / p.n_nblk, nb = blockIdx.x % p.n_nblk;
  if (slot >= p.counters[0]) return;
  const int g = p.active[slot];
  int64_t r0 = p.group_offsets[g], r1 = p.group_offsets[g + 1];
  if (r0 > p.max_rows) r0 = p.max_rows;
  if (r1 > p.max_rows) r1 = p.max_rows;
  const int H = p.H, I = p.I;
  const int K = SWIGLU ? H : I;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = nb * 64 + wave * 16;       // first output column of this wave
  const int kq = (lane >> 4) * 8;           // this lane's 16-byte slot inside each 64-byte quarter
  const bool sh = g == p.w.shared_group;

  const uint16_t* w0;
  const uint16_t* w1 = nullptr;
  if (SWIGLU) {
    const uint16_t* wg = sh ? (const uint16_t*)p.w.s_gate : (const uint16_t*)p.w.gate + (int64_t)g * I * H;
    const uint16_t* wu = sh ? (const uint16_t*)p.w.s_up : (const uint16_t*)p.w.up + (int64_t)g * I * H;
    w0 = wg + (int64_t)(n0 + (lane & 15)) * H + kq;
    w1 = wu + (int64_t)(n0 + (lane & 15)) * H + kq;
  } else {
    const uint16_t* wd = sh ? (const uint16_t*)p.w.s_down : (const uint16_t*)p.w.down + (int64_t)g * H * I;
    w0 = wd + (int64_t)(n0 + (lane & 15)) * I + kq;
  }
  const int nsteps = K / 128;

  for (int64_t mb = r0; mb < r1; mb += 16) {
    // Rows past the group end read the group's first row and are zeroed (no branch around loads).
    const int64_t r = mb + (lane & 15);
    const bool rok = r < r1;
    const int64_t rr = rok ? r : mb;
    const int64_t src = SWIGLU ? (p.row_index ? (int64_t)p.row_index[rr] : rr) : rr;
    const uint16_t* arow = p.a + src * K + kq;
    const uint32_t keep = rok ? 0xffffffffu : 0u;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    Frag a[2], b0[2], b1[2];
    auto load = [&](int buf, int st) {
      const int64_t off = (int64_t)st * 128;
      load_frag(a[buf], arow + off);
#pragma unroll
      for (int j = 0; j < 4; ++j) a[buf].v[j] &= keep;
      load_frag(b0[buf], w0 + off);
      if (SWIGLU) load_frag(b1[buf], w1 + off);
    };
    auto mma = [&](int buf) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 av = as_bf16x8(a[buf].v[j]);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, as_bf16x8(b0[buf].v[j]), acc0, 0, 0, 0);
        if (SWIGLU) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, as_bf16x8(b1[buf].v[j]), acc1, 0, 0, 0);
      }
    };
    load(0, 0);
    int st = 0;
    for (; st + 2 <= nsteps; st += 2) {
      load(1, st + 1);
      mma(0);
      if (st + 2 < nsteps) load(0, st + 2);
      mma(1);
    }
    if (st < nsteps) mma(0);  // odd step count: the last step sits in buffer 0

    // lane holds rows mb + 4*(lane/16) + i, column n0 + lane%16
    const int col = n0 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = mb + 4 * (lane >> 4) + i;
      if (row >= r1) continue;
      if (SWIGLU) {
        static_cast<uint16_t*>(p.out)[row * I + col] = f32_to_bf16(swiglu_f32(acc0[i], acc1[i]));
      } else {
        const float v = acc0[i] * (p.row_scale ? p.row_scale[row] : 1.f);
        if (p.out_bf16)
          static_cast<uint16_t*>(p.out)[row * H + col] = f32_to_bf16(v);
        else
          static_cast<float*>(p.out)[row * H + col] = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_gateup_stream_bf16(const Groups& g, const Weights& w, const uint16_t* x, uint16_t* h, int H, int I,
                                     hipStream_t s) {
  StreamArgs p{g.group_offsets, g.row_index, g.active, g.counters, g.max_rows, w, x, h, 1, nullptr, H, I, I / 64};
  const int64_t blocks = (int64_t)g.n_groups * p.n_nblk;
  stream_kernel<true><<<(unsigned)blocks, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_down_stream_bf16(const Groups& g, const Weights& w, const uint16_t* h, void* y_rows, bool y_bf16,
                                   const float* row_scale, int H, int I, hipStream_t s) {
  StreamArgs p{g.group_offsets, nullptr, g.active, g.counters, g.max_rows, w, h, y_rows, y_bf16 ? 1 : 0, row_scale,
               H, I, H / 64};
  const int64_t blocks = (int64_t)g.n_groups * p.n_nblk;
  stream_kernel<false><<<(unsigned)blocks, 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
