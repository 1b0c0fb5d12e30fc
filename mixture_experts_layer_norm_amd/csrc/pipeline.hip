// Chunked forward pipeline in one persistent kernel with a macrobatch ring buffer.
//
// Follows the sparsenotes page "Mixture-of-Kittens: MoE Megakernel for NVL72s":
//  * "Granularity as a tunable": the routed slots are cut into chunks of b rows (b at run time);
//    a chunk is carried through the whole expert FFN (up/gate + SwiGLU, then down) before the
//    compute side takes the next one, while dispatch runs ahead over later chunks;
//  * "A ring buffer instead of a host round-trip": dispatched rows and the gated activation live
//    in a device ring of S chunk stages; chunk c uses stage c % S and may only be written once
//    chunk c - S has been consumed; nothing is sized from host-side counts;
//  * "The production details": the shared expert is placed first, into the window before the
//    first chunk is dispatched.
// Work is a fixed sequence of items taken from one atomic ticket counter:
//   [shared up/gate tiles] [dispatch(0) .. dispatch(S-1)]
//   then for each chunk c: [up/gate(c)] [dispatch(c+S)] [down(c)], and the shared down tiles
//   after down(0).
// An item waits only for items earlier in the sequence (through per-chunk counters with
// agent-scope release/acquire), so the kernel cannot deadlock even when fewer workgroups are
// resident than launched; every wait is bounded, sets the sticky error word (bit 4) on expiry,
// and once that bit is set every other wait returns at once, so the kernel always drains.
// Each output tile is computed by one workgroup with a fixed summation order, so results are
// bitwise identical for every chunk size, ring depth and workgroup count.
#include "gemm_tile.h"
#include "pipeline.h"

namespace moe {



__device__ __forceinline__ int nd_of(const PipeArgs& p, int c) {
  const int rows = min(p.b, p.n - c * p.b);
  return (rows + kGemmBM - 1) / kGemmBM;
}

// Wait until *ctr >= target. Thread 0 polls with relaxed agent-scope loads (an acquire load
// would invalidate the L2 on every poll and starve the workgroups doing the work), then one
// acquire fence publishes the producers' data to the whole workgroup. The poll is bounded
// (about a second); on expiry, or when another wait already expired (bit 4 of the error word),
// it gives up so that the kernel always drains.
__device__ __forceinline__ void wait_geq(int32_t* ctr, int target, int32_t* err) {
  if (threadIdx.x == 0) {
    int spins = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(8);
      if ((++spins & 255) == 0) {
        if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 4) break;
        if (spins > (1 << 20)) {
          atomicOr(err, 4);
          break;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

__device__ __forceinline__ void signal_done(int32_t* ctr) {
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// m-tile t of chunk c -> expert, first slot, rows
__device__ __forceinline__ void chunk_tile(const PipeArgs& p, int c, int t, TileCoord& tc) {
  const int32_t* ct = p.ctile + (int64_t)c * (p.E + 1);
  int lo = 0, hi = p.E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ct[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int c0 = c * p.b, c1 = min(p.n, c0 + p.b);
  const int s0 = max(p.offsets[lo], c0), s1 = min(p.offsets[lo + 1], c1);
  tc.grp = lo;
  tc.r0 = s0 + (t - ct[lo]) * kGemmBM;
  tc.rows = min(kGemmBM, s1 - tc.r0);
}

__global__ __launch_bounds__(512, 1) void pipeline_kernel(PipeArgs p) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[kGemmSmemElems];
  __shared__ int s_item;
  int32_t* ticket = p.ctr;
  int32_t* sh1cnt = p.ctr + 1;
  int32_t* dcnt = p.ctr + 2;
  int32_t* g1cnt = dcnt + p.C;
  int32_t* g2cnt = g1cnt + p.C;
  const int total = p.chunk_base[p.C];
  while (true) {
    if (threadIdx.x == 0) s_item = atomicAdd(ticket, 1);
    __syncthreads();
    const int item = s_item;
    __syncthreads();
    if (item >= total) break;

    int kind, c = 0, local;
    if (item < p.n_sh1) {
      kind = 0; local = item;                                   // shared up/gate tile
    } else if (item < p.n_sh1 + p.d_pre) {
      kind = 2; local = item - p.n_sh1;                         // dispatch of the first S chunks
      while (local >= nd_of(p, c)) { local -= nd_of(p, c); ++c; }
    } else {
      int lo = 0, hi = p.C - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.chunk_base[mid] <= item) lo = mid; else hi = mid - 1;
      }
      c = lo;
      local = item - p.chunk_base[c];
      const int tc_n = p.ctile[(int64_t)c * (p.E + 1) + p.E];
      const int a1 = tc_n * p.ntn1;
      const int ad = (c + p.S < p.C) ? nd_of(p, c + p.S) : 0;
      const int a2 = tc_n * p.ntn2;
      if (local < a1) kind = 3;
      else if (local < a1 + ad) { kind = 2; local -= a1; c += p.S; }
      else if (local < a1 + ad + a2) { kind = 4; local -= a1 + ad; }
      else { kind = 1; local -= a1 + ad + a2; }
    }

    if (kind == 0 || kind == 1) {
      // shared expert tile over all T tokens (one group)
      TileCoord tc;
      tc.grp = 0;
      const int ntn = kind == 0 ? p.ntn_s1 : p.ntn_s2;
      tc.nt = local % ntn;
      tc.r0 = (local / ntn) * kGemmBM;
      tc.rows = min(kGemmBM, p.T - tc.r0);
      GemmArgs a;
      if (kind == 0) {
        a.A = p.x; a.lda = p.D; a.B = p.sg; a.B2 = p.su; a.ldb = p.D; a.N = p.Is; a.K = p.D;
        a.C = p.sh_h; a.ldc = p.Is;
        gemm_tile<EPI_SWIGLU, false, 64, 4, 32>(a, tc, 0, p.D / BK, ntn, smem);
        signal_done(sh1cnt);
      } else {
        wait_geq(sh1cnt, p.n_sh1, p.err);
        a.A = p.sh_h; a.lda = p.Is; a.B = p.sd; a.ldb = p.Is; a.N = p.D; a.K = p.Is; a.C = p.sh_out;
        a.ldc = p.D;
        gemm_tile<EPI_STORE, false, 64, 4, 32>(a, tc, 0, p.Is / BK, ntn, smem);
        __syncthreads();
      }
    } else if (kind == 2) {
      // dispatch rows [c*b + 256*local, ...) of chunk c into ring stage c % S
      if (c >= p.S) {
        const int prev = c - p.S;
        wait_geq(g1cnt + prev, p.ctile[(int64_t)prev * (p.E + 1) + p.E] * p.ntn1, p.err);
      }
      const int j0 = c * p.b + local * kGemmBM;
      const int j1 = min(min(j0 + kGemmBM, (c + 1) * p.b), p.n);
      const int64_t ring0 = (int64_t)(c % p.S) * p.b - (int64_t)c * p.b;   // slot -> ring row shift
      const int cpr = p.D / 8;                                              // 16-byte chunks per row
      const int total_chunks = (j1 - j0) * cpr;
      for (int q = threadIdx.x; q < total_chunks; q += 512) {
        const int j = j0 + q / cpr, cc = q % cpr;
        const int64_t src = p.perm[j] / p.K;
        const u32x4 v = reinterpret_cast<const u32x4*>(p.x + src * p.D)[cc];
        reinterpret_cast<u32x4*>(p.x_ring + (j + ring0) * p.D)[cc] = v;
      }
      signal_done(dcnt + c);
    } else if (kind == 3) {
      // up/gate + SwiGLU tile of chunk c
      wait_geq(dcnt + c, nd_of(p, c), p.err);
      if (c >= p.S) {
        const int prev = c - p.S;
        wait_geq(g2cnt + prev, p.ctile[(int64_t)prev * (p.E + 1) + p.E] * p.ntn2, p.err);
      }
      TileCoord tc;
      tc.nt = local % p.ntn1;
      chunk_tile(p, c, local / p.ntn1, tc);
      const int64_t ring0 = (int64_t)(c % p.S) * p.b - (int64_t)c * p.b;
      GemmArgs a;
      a.A = p.x_ring + ring0 * p.D; a.lda = p.D; a.B = p.wg; a.B2 = p.wu; a.ldb = p.D;
      a.b_group_stride = (int64_t)p.I * p.D; a.N = p.I; a.K = p.D; a.C = p.h_ring + ring0 * p.I; a.ldc = p.I;
      gemm_tile<EPI_SWIGLU, false, 64, 4, 32>(a, tc, 0, p.D / BK, p.ntn1, smem);
      signal_done(g1cnt + c);
    } else {
      // down tile of chunk c, rows scattered to their route ids
      wait_geq(g1cnt + c, p.ctile[(int64_t)c * (p.E + 1) + p.E] * p.ntn1, p.err);
      TileCoord tc;
      tc.nt = local % p.ntn2;
      chunk_tile(p, c, local / p.ntn2, tc);
      const int64_t ring0 = (int64_t)(c % p.S) * p.b - (int64_t)c * p.b;
      GemmArgs a;
      a.A = p.h_ring + ring0 * p.I; a.lda = p.I; a.B = p.wd; a.ldb = p.I; a.b_group_stride = (int64_t)p.D * p.I;
      a.N = p.D; a.K = p.I; a.C = p.y; a.ldc = p.D; a.c_scatter = p.perm;
      gemm_tile<EPI_STORE, false, 64, 4, 32>(a, tc, 0, p.I / BK, p.ntn2, smem);
      signal_done(g2cnt + c);
    }
  }
}

// per chunk: m-tiles of every expert's part of the chunk, prefix over experts (one block per chunk)
__global__ __launch_bounds__(1024) void chunk_tiles_kernel(const int32_t* __restrict__ offsets, int E, int n, int b,
                                                           int32_t* __restrict__ ctile, int32_t* __restrict__ crow) {
  __shared__ int sb[1024];
  const int c = blockIdx.x, e = threadIdx.x;
  const int c0 = c * b, c1 = min(n, c0 + b);
  int t = 0;
  if (e < E) {
    const int len = min(offsets[e + 1], c1) - max(offsets[e], c0);
    t = len > 0 ? (len + kGemmBM - 1) / kGemmBM : 0;
  }
  sb[e] = t;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = e >= off ? sb[e - off] : 0;
    __syncthreads();
    sb[e] += v;
    __syncthreads();
  }
  int32_t* row = ctile + (int64_t)c * (E + 1);
  if (e < E) row[e + 1] = sb[e];
  if (e == 0) row[0] = 0;
  if (crow) {   // each expert's row range clamped to the chunk (row offsets of the chunk's groups)
    int32_t* ro = crow + (int64_t)c * (E + 1);
    if (e < E) ro[e + 1] = min(max(offsets[e + 1], c0), c1);
    if (e == 0) ro[0] = c0;
  }
}

// item blocks of the chunks (prefix over chunks) and zeroed counters (one block)
__global__ __launch_bounds__(1024) void chunk_base_kernel(PipeArgs p, int32_t* __restrict__ chunk_base) {
  __shared__ int sb[1024];
  const int c = threadIdx.x;
  int v = 0;
  if (c < p.C) {
    const int tcn = p.ctile[(int64_t)c * (p.E + 1) + p.E];
    v = tcn * (p.ntn1 + p.ntn2) + ((c + p.S < p.C) ? nd_of(p, c + p.S) : 0) + (c == 0 ? p.n_sh2 : 0);
  }
  sb[c] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int u = c >= off ? sb[c - off] : 0;
    __syncthreads();
    sb[c] += u;
    __syncthreads();
  }
  const int base = p.n_sh1 + p.d_pre;
  if (c < p.C) chunk_base[c + 1] = base + sb[c];
  if (c == 0) chunk_base[0] = base;
  for (int i = c; i < 2 + 3 * p.C; i += 1024) p.ctr[i] = 0;
}

int launch_pipeline(const PipeArgs& host, int32_t* chunk_base_dev, int ncu, hipStream_t s) {
  hipLaunchKernelGGL(chunk_tiles_kernel, dim3(host.C), dim3(1024), 0, s, host.offsets, host.E, host.n, host.b,
                     (int32_t*)host.ctile, nullptr);
  MOE_LAUNCH_CHECK();
  hipLaunchKernelGGL(chunk_base_kernel, dim3(1), dim3(1024), 0, s, host, chunk_base_dev);
  MOE_LAUNCH_CHECK();
  hipLaunchKernelGGL(pipeline_kernel, dim3(ncu), dim3(512), 0, s, host);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

// Chunk tables for the multi-launch chunked path: per chunk, the m-tile prefix over experts
// (ctile [C][E+1]) and the experts' row ranges clamped to the chunk (crow [C][E+1]).
int launch_chunk_tables(const int32_t* offsets, int E, int n, int b, int C, int32_t* ctile, int32_t* crow,
                        hipStream_t s) {
  hipLaunchKernelGGL(chunk_tiles_kernel, dim3(C), dim3(1024), 0, s, offsets, E, n, b, ctile, crow);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
