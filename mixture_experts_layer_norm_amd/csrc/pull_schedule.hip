// Pull-dispatch schedule of one rank among R source ranks (Blog, "Scheduling"; the order inside
// each region is the sort key of the Notes, "Pull dispatch, push combine").
//
// Every rank holds the routing of all R source ranks (after an all-gather of topk_idx): route
// (r, i, k) of source rank r goes to global expert routing[r][i][k]; rank c owns the L experts
// [c L, (c + 1) L). For each of its local experts l the rank pulls the routes addressed to it into
// one contiguous region, ordered by (l, o, r) where the ordinal o of a route is the number of
// earlier routes (in (i, k) order) of the same source rank to the same expert. With
// M[l][r] = routes from r to l, the position of route (r, o) in region l is
//     S[l] + sum_r' min(M[l][r'], o) + #{ r' < r : M[l][r'] > o },
// i.e. first all routes of lower ordinal, then those of the same ordinal from lower ranks:
// consecutive slots alternate over the source ranks, so that a pull from peers keeps every link
// busy.
//
// Three passes, all deterministic (no order-dependent atomics):
//   1. per block of routes, a histogram over the R L (source rank, local expert) keys;
//   2. one block: per-key prefix over blocks (each block's first ordinal per key), M, the region
//      sizes T[l] and their exclusive scan S;
//   3. per block, the stable rank of each route among equal keys (a comparison with every lane's
//      key inside a wavefront, per-wavefront counts across), hence its ordinal and its position
//      by the formula above.
#include "common.h"

namespace moe {

namespace {

constexpr int kPullBlock = 2048;   // routes per histogram / placement block

// key of route j (r-major over [R][N][K]): r * L + local expert, or -1 when another rank owns it
__device__ __forceinline__ int pull_key(const int32_t* __restrict__ routing, int64_t j, int NK, int L, int RL,
                                        int rank, int32_t* err) {
  int e = routing[j];
  if ((unsigned)e >= (unsigned)RL) {
    atomicOr(err, 1);   // sticky: expert id out of range (taken as expert 0)
    e = 0;
  }
  const int owner = e / L;
  if (owner != rank) return -1;
  const int r = (int)(j / NK);
  return r * L + (e - owner * L);
}

__global__ __launch_bounds__(256) void pull_hist_kernel(const int32_t* __restrict__ routing, int64_t n, int NK,
                                                        int L, int RL, int rank, int32_t* __restrict__ blk_hist,
                                                        int32_t* err) {
  extern __shared__ int32_t hist[];
  for (int q = threadIdx.x; q < RL; q += 256) hist[q] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kPullBlock;
  const int64_t end = min(n, base + kPullBlock);
  for (int64_t j = base + threadIdx.x; j < end; j += 256) {
    const int q = pull_key(routing, j, NK, L, RL, rank, err);
    if (q >= 0) atomicAdd(&hist[q], 1);
  }
  __syncthreads();
  for (int q = threadIdx.x; q < RL; q += 256) blk_hist[(size_t)blockIdx.x * RL + q] = hist[q];
}

// block-wide exclusive scan over 1024 threads
__device__ int scan_1024(int v, int* sbuf, int* total) {
  const int tid = threadIdx.x;
  sbuf[tid] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = tid >= off ? sbuf[tid - off] : 0;
    __syncthreads();
    sbuf[tid] += add;
    __syncthreads();
  }
  const int incl = sbuf[tid];
  *total = sbuf[1023];
  __syncthreads();
  return incl - v;
}

// one block of 1024 threads; RL <= 1024
__global__ __launch_bounds__(1024) void pull_scan_kernel(int32_t* __restrict__ blk_hist, int nblk, int R, int L,
                                                         int32_t* __restrict__ counts, int32_t* __restrict__ src_counts,
                                                         int32_t* __restrict__ offsets) {
  __shared__ int sbuf[1024];
  __shared__ int mtot[1024];
  const int q = threadIdx.x, RL = R * L;
  int running = 0;
  if (q < RL) {
    for (int b = 0; b < nblk; ++b) {
      const int v = blk_hist[(size_t)b * RL + q];
      blk_hist[(size_t)b * RL + q] = running;    // first ordinal of key q in block b
      running += v;
    }
    mtot[q] = running;
  }
  __syncthreads();
  int tl = 0;
  if (q < L) {
    for (int r = 0; r < R; ++r) {
      const int m = mtot[r * L + q];
      src_counts[(size_t)q * R + r] = m;
      tl += m;
    }
  }
  int total;
  const int s = scan_1024(q < L ? tl : 0, sbuf, &total);
  if (q < L) {
    counts[q] = tl;
    offsets[q] = s;
  }
  if (q == 0) offsets[L] = total;
}

// LDS: cnt [RL] next ordinal per key for this block, wcnt [4][RL] per-wavefront counts of the
// current round, m [RL] = M as [l][r], s [L] = region starts
__global__ __launch_bounds__(256) void pull_place_kernel(const int32_t* __restrict__ routing, int64_t n, int NK, int R,
                                                         int L, int rank, const int32_t* __restrict__ blk_start,
                                                         const int32_t* __restrict__ src_counts,
                                                         const int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ phi_src, int32_t* __restrict__ phi_idx,
                                                         int32_t* __restrict__ route_pos, int32_t* err) {
  extern __shared__ int32_t sm[];
  const int RL = R * L;
  int32_t* cnt = sm;
  int32_t* wcnt = sm + RL;
  int32_t* m = sm + 5 * RL;
  int32_t* s = sm + 6 * RL;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int q = tid; q < RL; q += 256) {
    cnt[q] = blk_start[(size_t)blockIdx.x * RL + q];
    m[q] = src_counts[q];
  }
  for (int l = tid; l < L; l += 256) s[l] = offsets[l];
  const int64_t base = (int64_t)blockIdx.x * kPullBlock;
  const int64_t end = min(n, base + kPullBlock);
  for (int64_t rb = base; rb < end; rb += 256) {
    for (int i = tid; i < 4 * RL; i += 256) wcnt[i] = 0;
    __syncthreads();
    const int64_t j = rb + tid;
    const bool valid = j < end;
    const int key = valid ? pull_key(routing, j, NK, L, RL, rank, err) : -1;
    // rank among earlier lanes of this wave with the same key, read lane by lane with readlane
    // (a fixed 64 steps); the last lane of a key records the wave's count for it
    int rank_in_wave = 0, later = 0;
#pragma unroll
    for (int q = 0; q < 64; ++q) {
      const int kq = __builtin_amdgcn_readlane(key, q);
      const int same = kq == key ? 1 : 0;
      rank_in_wave += q < lane ? same : 0;
      later += q > lane ? same : 0;
    }
    if (key >= 0 && later == 0) wcnt[w * RL + key] = rank_in_wave + 1;
    __syncthreads();
    if (key >= 0) {
      int o = cnt[key] + rank_in_wave;
      for (int q = 0; q < w; ++q) o += wcnt[q * RL + key];
      const int r = key / L, l = key - r * L;
      const int32_t* ml = m + l * R;
      int p = s[l];
      for (int r2 = 0; r2 < R; ++r2) {
        const int mm = ml[r2];
        p += min(mm, o) + ((r2 < r && mm > o) ? 1 : 0);
      }
      phi_src[p] = r;
      phi_idx[p] = (int32_t)(j - (int64_t)r * NK);
      if (route_pos) route_pos[j] = p;
    } else if (valid && route_pos) {
      route_pos[j] = -1;
    }
    __syncthreads();
    for (int q = tid; q < RL; q += 256) cnt[q] += wcnt[q] + wcnt[RL + q] + wcnt[2 * RL + q] + wcnt[3 * RL + q];
    __syncthreads();
  }
}

struct PullWs {
  size_t err, blk_hist, total;
};

PullWs pull_ws(int64_t n, int RL) {
  PullWs w{};
  const int64_t nblk = (n + kPullBlock - 1) / kPullBlock;
  w.err = 0;
  w.blk_hist = 256;
  w.total = w.blk_hist + (((size_t)nblk * RL * 4 + 255) / 256) * 256;
  return w;
}

int validate_pull(int R, int N, int K, int L, int rank) {
  if (R < 1 || N < 1 || K < 1 || L < 1 || rank < 0 || rank >= R) return MOE_ERR_INVALID_ARG;
  if ((int64_t)R * L > 1024) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)R * N * K >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace

}  // namespace moe

using namespace moe;

extern "C" {

int moe_pull_schedule_workspace_size(int32_t R, int32_t N, int32_t K, int32_t L, size_t* bytes) {
  int st = validate_pull(R, N, K, L, 0);
  if (st) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = pull_ws((int64_t)R * N * K, R * L).total;
  return MOE_OK;
}

int moe_pull_schedule(int32_t R, int32_t N, int32_t K, int32_t L, int32_t rank, const int32_t* routing,
                      int32_t* counts, int32_t* src_counts, int32_t* offsets, int32_t* phi_src, int32_t* phi_idx,
                      int32_t* route_pos, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = validate_pull(R, N, K, L, rank);
  if (st) return st;
  if (!routing || !counts || !src_counts || !offsets || !phi_src || !phi_idx) return MOE_ERR_INVALID_ARG;
  const int64_t n = (int64_t)R * N * K;
  const int RL = R * L, NK = N * K;
  const PullWs W = pull_ws(n, RL);
  if (!ws || ws_bytes < W.total) return MOE_ERR_WORKSPACE;
  char* wsb = (char*)ws;
  int32_t* err = (int32_t*)(wsb + W.err);
  int32_t* blk = (int32_t*)(wsb + W.blk_hist);
  const int nblk = (int)((n + kPullBlock - 1) / kPullBlock);
  hipLaunchKernelGGL(pull_hist_kernel, dim3(nblk), dim3(256), RL * sizeof(int32_t), stream, routing, n, NK, L, RL,
                     rank, blk, err);
  MOE_LAUNCH_CHECK();
  hipLaunchKernelGGL(pull_scan_kernel, dim3(1), dim3(1024), 0, stream, blk, nblk, R, L, counts, src_counts, offsets);
  MOE_LAUNCH_CHECK();
  hipLaunchKernelGGL(pull_place_kernel, dim3(nblk), dim3(256), (6 * RL + L) * sizeof(int32_t), stream, routing, n,
                     NK, R, L, rank, blk, src_counts, offsets, phi_src, phi_idx, route_pos, err);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // extern "C"
