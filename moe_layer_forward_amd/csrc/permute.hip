// Dispatch permutation and grouped-GEMM plan.
//
// "Kimi K2.5 模型架构深度拆解" §10.2 Step 6 gathers, for each expert present, the tokens routed to it.
// Here that becomes a counting sort of the T*K (token, slot) pairs by expert into contiguous
// segments, stable in (t, k) order:
//   hist    : per chunk of 4096 pairs, an LDS histogram of expert ids -> counts[chunk][E]
//   scan    : one work-group turns the counts into segment offsets and per-chunk bases
//   scatter : per chunk, each wave ranks its pairs in 64-pair rounds: lanes holding the same expert
//             find each other with one ballot per id bit, rank = popcount of lower peers, and the
//             last peer advances the wave's running cursor for that expert (LDS), so the order
//             inside a segment is exactly (t, k) order without atomics on the output.
// The plan kernel turns group offsets into (a) the list of groups with rows, largest first, for
// the weight-streaming kernels and (b) the list of kTileM-row tiles for the tile kernels.  Group
// sizes never leave the device.
#include "kernels.h"

namespace moe {
namespace {

constexpr int kChunk = 4096;        // pairs per hist/scatter work-group
constexpr int kMaxExperts = 1024;

// Ids outside [0, E) are a caller error; they are clamped so that no access leaves its buffer.
__device__ __forceinline__ int clamp_id(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ ids, int64_t P, int E,
                                                   int32_t* __restrict__ counts) {
  __shared__ int32_t h[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  for (int i = threadIdx.x; i < kChunk; i += 256) {
    const int64_t p = base + i;
    if (p < P) atomicAdd(&h[clamp_id(ids[p], E)], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) counts[(int64_t)blockIdx.x * E + e] = h[e];
}

// counts[b][e] -> base[b][e] (in place): first row of chunk b's pairs of expert e.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ counts, int nblk, int E,
                                                    int32_t* __restrict__ offsets, int64_t P, int64_t tail_rows) {
  __shared__ int32_t tot[kMaxExperts];
  __shared__ int32_t excl[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += 1024) {
    int32_t s = 0;
    for (int b = 0; b < nblk; ++b) s += counts[(int64_t)b * E + e];
    tot[e] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t run = 0;
    for (int e = 0; e < E; ++e) {
      excl[e] = run;
      run += tot[e];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 1024) {
    int32_t run = excl[e];
    for (int b = 0; b < nblk; ++b) {
      const int32_t c = counts[(int64_t)b * E + e];
      counts[(int64_t)b * E + e] = run;
      run += c;
    }
    offsets[e] = excl[e];
  }
  if (threadIdx.x == 0) {
    offsets[E] = (int32_t)P;
    if (tail_rows > 0) offsets[E + 1] = (int32_t)(P + tail_rows);
  }
}

__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ ids, int64_t P, int K, int E,
                                                      int nbits, const int32_t* __restrict__ base,
                                                      int32_t* __restrict__ row_token, int32_t* __restrict__ pair_row,
                                                      int64_t T, int shared_rows) {
  __shared__ int32_t cur[4][kMaxExperts];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t cbeg = (int64_t)blockIdx.x * kChunk;
  const int64_t wbeg = cbeg + wave * (kChunk / 4);
  int64_t wend = wbeg + kChunk / 4;
  if (wend > P) wend = P;

  for (int e = threadIdx.x; e < 4 * kMaxExperts; e += 256) (&cur[0][0])[e] = 0;
  __syncthreads();
  for (int64_t p = wbeg + lane; p < wend; p += 64) atomicAdd(&cur[wave][clamp_id(ids[p], E)], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    int32_t run = base[(int64_t)blockIdx.x * E + e];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int32_t c = cur[w][e];
      cur[w][e] = run;
      run += c;
    }
  }
  __syncthreads();

  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t p0 = wbeg; p0 < wend; p0 += 64) {
    const int64_t p = p0 + lane;
    const bool valid = p < wend;
    const int e = valid ? clamp_id(ids[p], E) : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t bal = __ballot((e >> b) & 1);
      peers &= ((e >> b) & 1) ? bal : ~bal;
    }
    if (valid) {
      const int rank = __popcll(peers & lower);
      const int32_t row = cur[wave][e] + rank;
      row_token[row] = (int32_t)(p / K);
      pair_row[p] = row;
      const int n = __popcll(peers);
      if (rank == n - 1) cur[wave][e] = row + 1;
    }
  }
  if (shared_rows) {
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < T; t += (int64_t)gridDim.x * 256)
      row_token[P + t] = (int32_t)t;
  }
}

// Exclusive scan of v over the 1024 threads of the block; returns the block total in *total.
__device__ int32_t block_excl_scan(int32_t v, int32_t* sh, int32_t* total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t add = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  const int32_t incl = sh[tid];
  *total = sh[1023];
  __syncthreads();
  return incl - v;
}

constexpr int kBuckets = 64;     // size classes for largest-first ordering (16-row passes, capped)
constexpr int kPlanPerThread = 4;  // groups per thread -> at most 4096 groups

// The plan of G groups (one 1024-thread work-group): active groups largest first, and the tiles of
// those with more than stream_rows rows (0 or kStreamRows; the smaller ones, a suffix of the active
// list since the size classes are 16 rows wide, go to the weight-stream kernels).
__device__ void plan_block(const int32_t* __restrict__ off, int G, int64_t max_rows, int tile_m, int max_tiles,
                           int stream_rows, int32_t* __restrict__ active, int32_t* __restrict__ counters,
                           int32_t* __restrict__ tiles) {
  __shared__ int32_t bucket_cnt[kBuckets];
  __shared__ int32_t bucket_cur[kBuckets];
  __shared__ int32_t scan_buf[1024];
  __shared__ int32_t pos_of[kPlanPerThread * 1024];
  __shared__ int32_t g_of[kPlanPerThread * 1024];
  __shared__ int32_t n_active_sh;
  const int tid = threadIdx.x;
  if (tid < kBuckets) bucket_cnt[tid] = 0;
  __syncthreads();

  int32_t rows[kPlanPerThread];
  int32_t bucket[kPlanPerThread];
#pragma unroll
  for (int j = 0; j < kPlanPerThread; ++j) {
    const int g = tid * kPlanPerThread + j;
    rows[j] = 0;
    bucket[j] = -1;
    if (g < G) {
      int64_t a = off[g], b = off[g + 1];
      if (a > max_rows) a = max_rows;
      if (b > max_rows) b = max_rows;
      rows[j] = b > a ? (int32_t)(b - a) : 0;
      if (rows[j] > 0) {
        int c = (rows[j] + 15) / 16;
        bucket[j] = kBuckets - (c < kBuckets ? c : kBuckets);  // bigger groups -> lower bucket index
        atomicAdd(&bucket_cnt[bucket[j]], 1);
      }
    }
  }
  __syncthreads();
  static_assert(kStreamRows % 16 == 0, "small groups fill whole size classes");
  if (tid == 0) {
    const int small_b = kBuckets - stream_rows / 16;  // the size classes of the small groups start here
    int32_t run = 0, n_large = 0;
    for (int b = 0; b < kBuckets; ++b) {
      if (b == small_b) n_large = run;
      bucket_cur[b] = run;
      run += bucket_cnt[b];
    }
    counters[0] = run;
    counters[2] = stream_rows > 0 ? n_large : run;
    n_active_sh = run;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPlanPerThread; ++j) {
    const int g = tid * kPlanPerThread + j;
    if (bucket[j] >= 0) {
      const int pos = atomicAdd(&bucket_cur[bucket[j]], 1);
      active[pos] = g;
      g_of[pos] = g;
      pos_of[pos] = rows[j];
    }
  }
  __syncthreads();
  const int n_active = n_active_sh;
  // tiles, in active order: thread tid owns active positions [tid*4, tid*4+4)
  int32_t ntl[kPlanPerThread];
  int32_t mine = 0;
#pragma unroll
  for (int j = 0; j < kPlanPerThread; ++j) {
    const int pos = tid * kPlanPerThread + j;
    ntl[j] = pos < n_active && pos_of[pos] > stream_rows ? (pos_of[pos] + tile_m - 1) / tile_m : 0;
    mine += ntl[j];
  }
  int32_t total;
  int32_t t0 = block_excl_scan(mine, scan_buf, &total);
#pragma unroll
  for (int j = 0; j < kPlanPerThread; ++j) {
    const int pos = tid * kPlanPerThread + j;
    if (pos < n_active) {
      const int g = g_of[pos];
      for (int q = 0; q < ntl[j]; ++q, ++t0)
        if (t0 < max_tiles) {
          tiles[2 * t0] = g;
          tiles[2 * t0 + 1] = q * tile_m;
        }
    }
  }
  if (tid == 0) counters[1] = total < max_tiles ? total : max_tiles;
}

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ off, int G, int64_t max_rows,
                                                    int tile_m, int max_tiles, int stream_rows,
                                                    int32_t* __restrict__ active, int32_t* __restrict__ counters,
                                                    int32_t* __restrict__ tiles) {
  plan_block(off, G, max_rows, tile_m, max_tiles, stream_rows, active, counters, tiles);
}

// Few pairs (P <= kChunk): histogram, scan, stable scatter and (when plan.n_groups > 0) the plan in
// one 1024-thread work-group (16 waves, each ranking P/16 consecutive pairs as scatter_kernel does,
// so the rows come out in the same order); the other work-groups of the launch convert the token
// rows to binary16 when x16 is given.
constexpr int kSmallWaves = 16;
constexpr int kSmallExperts = 512;

__global__ __launch_bounds__(1024) void permute_plan_small_kernel(
    const int32_t* __restrict__ ids, int64_t T, int K, int E, int nbits, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_token, int32_t* __restrict__ pair_row, int shared_rows, Groups plan,
    const uint16_t* __restrict__ x, uint16_t* __restrict__ x16, int64_t x_groups) {
  if (blockIdx.x > 0) {
    const int64_t stride = (int64_t)(gridDim.x - 1) * 1024;
    for (int64_t i = (int64_t)(blockIdx.x - 1) * 1024 + threadIdx.x; i < x_groups; i += stride)
      f16_group_pairs(x + 8 * i, x16 + 8 * i);
    return;
  }
  __shared__ int32_t cur[kSmallWaves][kSmallExperts];
  __shared__ int32_t scan_buf[1024];
  const int64_t P = T * K;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x;
  const int64_t per = (P + kSmallWaves - 1) / kSmallWaves;
  const int64_t wbeg = wave * per;
  const int64_t wend = wbeg + per < P ? wbeg + per : P;
  for (int e = tid; e < kSmallWaves * kSmallExperts; e += 1024) (&cur[0][0])[e] = 0;
  __syncthreads();
  for (int64_t q = wbeg + lane; q < wend; q += 64) atomicAdd(&cur[wave][clamp_id(ids[q], E)], 1);
  __syncthreads();
  // segment offsets: expert e's total, exclusive scan over the experts (one per thread)
  int32_t tot = 0;
  if (tid < E)
    for (int w = 0; w < kSmallWaves; ++w) tot += cur[w][tid];
  int32_t all;
  int32_t run = block_excl_scan(tot, scan_buf, &all);
  if (tid < E) {
    offsets[tid] = run;
    for (int w = 0; w < kSmallWaves; ++w) {  // each wave's first row of expert e
      const int32_t c = cur[w][tid];
      cur[w][tid] = run;
      run += c;
    }
  }
  if (tid == 0) {
    offsets[E] = (int32_t)P;
    if (shared_rows) offsets[E + 1] = (int32_t)(P + T);
  }
  __syncthreads();
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t p0 = wbeg; p0 < wend; p0 += 64) {
    const int64_t q = p0 + lane;
    const bool valid = q < wend;
    const int e = valid ? clamp_id(ids[q], E) : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t bal = __ballot((e >> b) & 1);
      peers &= ((e >> b) & 1) ? bal : ~bal;
    }
    if (valid) {
      const int rank = __popcll(peers & lower);
      const int32_t row = cur[wave][e] + rank;
      row_token[row] = (int32_t)(q / K);
      pair_row[q] = row;
      const int n = __popcll(peers);
      if (rank == n - 1) cur[wave][e] = row + 1;
    }
  }
  if (shared_rows)
    for (int64_t t = tid; t < T; t += 1024) row_token[P + t] = (int32_t)t;
  if (plan.n_groups == 0) return;  // permutation only
  __threadfence_block();
  __syncthreads();  // offsets written above are read back by the plan
  plan_block(offsets, plan.n_groups, plan.max_rows, plan.tile_m, plan.max_tiles, plan.stream_rows, plan.active,
             plan.counters, plan.tiles);
}

__global__ __launch_bounds__(256) void gather_kernel(const uint4* __restrict__ x, const int32_t* __restrict__ row_token,
                                                     uint4* __restrict__ x_perm, int64_t rows, int chunks_per_row) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * chunks_per_row) return;
  const int64_t r = i / chunks_per_row;
  const int c = (int)(i - r * chunks_per_row);
  x_perm[i] = x[(int64_t)row_token[r] * chunks_per_row + c];
}

}  // namespace

int64_t permute_blocks(int64_t pairs) { return (pairs + kChunk - 1) / kChunk; }

int64_t permute_scratch_ints(int64_t pairs, int E) { return permute_blocks(pairs) * E; }

hipError_t launch_permute(const int32_t* ids, int64_t T, int K, int E, int32_t* group_offsets, int32_t* row_token,
                          int32_t* pair_row, int32_t* scratch, bool shared_rows, hipStream_t s) {
  const int64_t P = T * K;
  const int nblk = (int)permute_blocks(P);
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  hist_kernel<<<nblk, 256, 0, s>>>(ids, P, E, scratch);
  scan_kernel<<<1, 1024, 0, s>>>(scratch, nblk, E, group_offsets, P, shared_rows ? T : 0);
  scatter_kernel<<<nblk, 256, 0, s>>>(ids, P, K, E, nbits, scratch, row_token, pair_row, T, shared_rows ? 1 : 0);
  return hipGetLastError();
}

bool permute_plan_fused(int64_t pairs, int E, int G) {
  return pairs <= kChunk && E <= kSmallExperts && G <= kPlanPerThread * 1024;
}

hipError_t launch_permute_plan(const int32_t* ids, int64_t T, int K, int E, int32_t* group_offsets,
                               int32_t* row_token, int32_t* pair_row, bool shared_rows, const Groups& plan,
                               const uint16_t* x, uint16_t* x16, int H, hipStream_t s) {
  if (!permute_plan_fused(T * K, E, plan.n_groups)) return hipErrorInvalidValue;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int64_t x_groups = x16 ? T * H / 8 : 0;
  int64_t conv = (x_groups + 1023) / 1024;
  if (conv > 256) conv = 256;
  permute_plan_small_kernel<<<(unsigned)(1 + conv), 1024, 0, s>>>(ids, T, K, E, nbits, group_offsets, row_token,
                                                                  pair_row, shared_rows ? 1 : 0, plan, x, x16,
                                                                  x_groups);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* row_token, void* x_perm, int64_t rows, int H,
                              int elem_bytes, hipStream_t s) {
  const int cpr = H * elem_bytes / 16;
  const int64_t n = rows * cpr;
  gather_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(static_cast<const uint4*>(x), row_token,
                                                             static_cast<uint4*>(x_perm), rows, cpr);
  return hipGetLastError();
}

hipError_t launch_plan(const Groups& g, hipStream_t s) {
  plan_kernel<<<1, 1024, 0, s>>>(g.group_offsets, g.n_groups, g.max_rows, g.tile_m, g.max_tiles, g.stream_rows,
                                 g.active, g.counters, g.tiles);
  return hipGetLastError();
}

}  // namespace moe
