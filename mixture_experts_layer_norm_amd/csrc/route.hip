// Top-k routing and the device-side schedule (histogram + scan + stable placement).
//
// Routing follows the Cursor blog "Mixture-of-Kittens: our open-source MoE megakernel for
// NVL72s", section "Overlapping computation and communication in MoE": each token picks its
// top-k routed experts and weights them with g_i = s_i / sum_{j in E} s_j (s = softmax of the
// router logits, which cancels to exp(l_i - l_max) / sum over the chosen experts).
//
// The schedule is the one-source-rank case of the pull schedule of the blog's "Scheduling"
// section: per-expert counts, region offsets by exclusive scan, then every route written to
// offsets[e] + (number of earlier routes to e), which is the sort key (local expert,
// per-source ordinal, source rank) of the sparsenotes page "Mixture-of-Kittens: MoE Megakernel
// for NVL72s", section "Pull dispatch, push combine", with one source rank. Positions come from
// route order, never from the order in which atomics return, so the table is bit-exact.
#include "common.h"

namespace moe {

// Total order on fp32 as uint32: larger value -> larger key; -0.0 == +0.0; NaN lowest.
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t m = u & 0x7fffffffu;
  if (m > 0x7f800000u) return 0u;
  if (m == 0u) return 0x80000000u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = __shfl_xor((unsigned)(v & 0xffffffffu), off, 64);
    uint32_t hi = __shfl_xor((unsigned)(v >> 32), off, 64);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

// Top-K of one token from its keys (key = (value order << 32) | ~e: the max picks the larger
// value, then the lower index), then g_k = exp(v_k - v_0) / sum_j exp(v_j - v_0). One wavefront.
template <int NV>
__device__ __forceinline__ void topk_from_keys(uint64_t (&key)[NV], int K, int lane, int32_t* __restrict__ idx_row,
                                               float* __restrict__ w_row) {
  int my_e = 0;
  float my_v = 0.f;
  float vmax = 0.f;
  for (int k = 0; k < K; ++k) {
    uint64_t best = key[0];
#pragma unroll
    for (int j = 1; j < NV; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_u64(best);
    const int e = (int)(0xffffffffu - (uint32_t)(best & 0xffffffffu));
    const float v = key_value((uint32_t)(best >> 32));
#pragma unroll
    for (int j = 0; j < NV; ++j)
      if (lane + 64 * j == e) key[j] = 0ull;
    if (k == 0) vmax = v;
    if (lane == k) { my_e = e; my_v = v; }
  }
  // lane k holds choice k (K <= 64)
  float z = (lane < K) ? expf(my_v - vmax) : 0.f;
  float s = z;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane < K) {
    idx_row[lane] = my_e;
    w_row[lane] = z / s;
  }
}

__device__ __forceinline__ uint64_t route_key(float v, int e) {
  return ((uint64_t)order_key(v) << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
}

// One wavefront per token. NV = logits per lane (E <= 64 * NV).
template <int NV>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                         int32_t* __restrict__ idx,
                                                         float* __restrict__ wout, int T, int E,
                                                         int K) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  uint64_t key[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int e = lane + 64 * j;
    key[j] = (e < E) ? route_key(row[e], e) : 0ull;
  }
  topk_from_keys<NV>(key, K, lane, idx + (size_t)t * K, wout + (size_t)t * K);
}

// The same from S split-K partial products of the router GEMM: logit = sum over s of part[s]
// (s ascending, fp32), also stored to logits when it is not null.
template <int NV>
__global__ __launch_bounds__(256) void route_topk_partials_kernel(const float* __restrict__ part, int S,
                                                                  int64_t part_stride, float* __restrict__ logits,
                                                                  int32_t* __restrict__ idx, float* __restrict__ wout,
                                                                  int T, int E, int K) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  uint64_t key[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int e = lane + 64 * j;
    key[j] = 0ull;
    if (e < E) {
      const float* p = part + (size_t)t * E + e;
      float v = p[0];
      for (int q = 1; q < S; ++q) v += p[q * part_stride];
      if (logits) logits[(size_t)t * E + e] = v;
      key[j] = route_key(v, e);
    }
  }
  topk_from_keys<NV>(key, K, lane, idx + (size_t)t * K, wout + (size_t)t * K);
}

int launch_route_topk_partials(const float* part, int S, int64_t part_stride, float* logits, int32_t* idx, float* w,
                               int T, int E, int K, hipStream_t s) {
  dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    hipLaunchKernelGGL(route_topk_partials_kernel<1>, grid, block, 0, s, part, S, part_stride, logits, idx, w, T, E, K);
  else if (E <= 128)
    hipLaunchKernelGGL(route_topk_partials_kernel<2>, grid, block, 0, s, part, S, part_stride, logits, idx, w, T, E, K);
  else if (E <= 256)
    hipLaunchKernelGGL(route_topk_partials_kernel<4>, grid, block, 0, s, part, S, part_stride, logits, idx, w, T, E, K);
  else if (E <= 512)
    hipLaunchKernelGGL(route_topk_partials_kernel<8>, grid, block, 0, s, part, S, part_stride, logits, idx, w, T, E, K);
  else
    hipLaunchKernelGGL(route_topk_partials_kernel<16>, grid, block, 0, s, part, S, part_stride, logits, idx, w, T, E, K);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

int launch_route_topk(const float* logits, int32_t* idx, float* w, int T, int E, int K, hipStream_t s) {
  dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    hipLaunchKernelGGL(route_topk_kernel<1>, grid, block, 0, s, logits, idx, w, T, E, K);
  else if (E <= 128)
    hipLaunchKernelGGL(route_topk_kernel<2>, grid, block, 0, s, logits, idx, w, T, E, K);
  else if (E <= 256)
    hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, 0, s, logits, idx, w, T, E, K);
  else if (E <= 512)
    hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, s, logits, idx, w, T, E, K);
  else
    hipLaunchKernelGGL(route_topk_kernel<16>, grid, block, 0, s, logits, idx, w, T, E, K);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

// ---------------------------------------------------------------------------------------------
// schedule
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ int checked_expert(int e, int E, int32_t* err) {
  if ((unsigned)e >= (unsigned)E) {
    atomicOr(err, 1);   // sticky: expert id out of range (clamped to 0)
    return 0;
  }
  return e;
}

// pass 1: per-block histogram of kRouteRowsPerBlock consecutive routes
__global__ __launch_bounds__(256) void sched_hist_kernel(const int32_t* __restrict__ idx, int n, int E,
                                                         int32_t* __restrict__ blk_hist,
                                                         int32_t* err) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * kRouteRowsPerBlock;
  const int end = min(n, base + kRouteRowsPerBlock);
  for (int r = base + threadIdx.x; r < end; r += 256) atomicAdd(&hist[checked_expert(idx[r], E, err)], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) blk_hist[(size_t)blockIdx.x * E + e] = hist[e];
}

// block-wide exclusive scan of v over 1024 threads (in LDS), returns the exclusive prefix
__device__ int block_exclusive_scan_1024(int v, int* sbuf, int* total) {
  const int tid = threadIdx.x;
  sbuf[tid] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int add = tid >= off ? sbuf[tid - off] : 0;
    __syncthreads();
    sbuf[tid] += add;
    __syncthreads();
  }
  int incl = sbuf[tid];
  *total = sbuf[1023];
  __syncthreads();
  return incl - v;
}

// pass 2 (one block of 1024 threads): per-expert totals over blocks, exclusive scan over
// experts, m-tile prefix for the grouped GEMMs, and each block's starting position per expert.
__global__ __launch_bounds__(1024) void sched_scan_kernel(int32_t* __restrict__ blk_hist, int nblk, int E,
                                                          int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ tile_off) {
  __shared__ int sbuf[1024];
  const int e = threadIdx.x;
  // the per-block counts are read kScanBatch at a time, so that their loads are in flight
  // together instead of one after another
  constexpr int kScanBatch = 16;
  int running = 0;
  if (e < E) {
    for (int b0 = 0; b0 < nblk; b0 += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) v[j] = b0 + j < nblk ? blk_hist[(size_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) {
        if (b0 + j < nblk) blk_hist[(size_t)(b0 + j) * E + e] = running;
        running += v[j];
      }
    }
  }
  int total;
  const int off = block_exclusive_scan_1024(e < E ? running : 0, sbuf, &total);
  const int tiles = e < E ? (running + kGemmBM - 1) / kGemmBM : 0;
  int ttotal;
  const int toff = block_exclusive_scan_1024(tiles, sbuf, &ttotal);
  if (e < E) {
    counts[e] = running;
    offsets[e] = off;
    tile_off[e] = toff;
    for (int b0 = 0; b0 < nblk; b0 += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) v[j] = b0 + j < nblk ? blk_hist[(size_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j)
        if (b0 + j < nblk) blk_hist[(size_t)(b0 + j) * E + e] = v[j] + off;
    }
  }
  if (e == 0) {
    offsets[E] = total;
    tile_off[E] = ttotal;
  }
}

// pass 3: stable placement. Each block walks its routes in order, 256 at a time; inside a
// wave the rank among equal experts comes from comparing all 64 lanes' experts, across waves
// from per-wave counts.
__global__ __launch_bounds__(256) void sched_place_kernel(const int32_t* __restrict__ idx, int n, int E,
                                                          const int32_t* __restrict__ blk_start,
                                                          int32_t* __restrict__ perm,
                                                          int32_t* __restrict__ inv_perm,
                                                          int32_t* err) {
  extern __shared__ int32_t sm[];
  int32_t* cnt = sm;          // [E]  next position per expert for this block
  int32_t* wcnt = sm + E;     // [4][E] routes per expert in each wave of the current round
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int e = tid; e < E; e += 256) cnt[e] = blk_start[(size_t)blockIdx.x * E + e];
  const int base = blockIdx.x * kRouteRowsPerBlock;
  const int end = min(n, base + kRouteRowsPerBlock);
  for (int rb = base; rb < end; rb += 256) {
    for (int i = tid; i < 4 * E; i += 256) wcnt[i] = 0;
    __syncthreads();
    const int r = rb + tid;
    const bool valid = r < end;
    const int e = valid ? checked_expert(idx[r], E, err) : -1;
    // rank = earlier lanes of this wave with the same expert; the last such lane also records
    // the wave's count for that expert. Every lane reads every other lane's expert (readlane
    // with a constant lane index), so the cost is fixed whatever the mix of experts.
    int rank = 0, later = 0;
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      const int ej = __builtin_amdgcn_readlane(e, j);
      const int same = ej == e ? 1 : 0;
      rank += j < lane ? same : 0;
      later += j > lane ? same : 0;
    }
    if (valid && later == 0) wcnt[w * E + e] = rank + 1;
    __syncthreads();
    if (valid) {
      int pos = cnt[e] + rank;
      for (int q = 0; q < w; ++q) pos += wcnt[q * E + e];
      perm[pos] = r;
      inv_perm[r] = pos;
    }
    __syncthreads();
    for (int x = tid; x < E; x += 256) cnt[x] += wcnt[x] + wcnt[E + x] + wcnt[2 * E + x] + wcnt[3 * E + x];
    __syncthreads();
  }
}

int launch_schedule(const int32_t* idx, int T, int K, int E, int32_t* counts, int32_t* offsets,
                    int32_t* perm, int32_t* inv_perm, int32_t* blk_hist, int32_t* tile_off,
                    int32_t* err, hipStream_t s) {
  const int n = T * K;
  const int nblk = (n + kRouteRowsPerBlock - 1) / kRouteRowsPerBlock;
  hipLaunchKernelGGL(sched_hist_kernel, dim3(nblk), dim3(256), E * sizeof(int32_t), s, idx, n, E, blk_hist, err);
  MOE_LAUNCH_CHECK();
  hipLaunchKernelGGL(sched_scan_kernel, dim3(1), dim3(1024), 0, s, blk_hist, nblk, E, counts, offsets, tile_off);
  MOE_LAUNCH_CHECK();
  hipLaunchKernelGGL(sched_place_kernel, dim3(nblk), dim3(256), 5 * E * sizeof(int32_t), s, idx, n, E,
                     blk_hist, perm, inv_perm, err);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
