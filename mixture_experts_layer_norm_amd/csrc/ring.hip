// Device tables of the chunked ring (the sparsenotes page "Mixture-of-Kittens: MoE Megakernel for
// NVL72s", sections "Granularity as a tunable" and "A ring buffer instead of a host round-trip").
//
// The routed slots are cut into chunks of b rows (b chosen at run time). Chunk c holds slots
// [c b, min(n, (c + 1) b)), which, the slots being expert-contiguous, are a run of whole experts
// plus at most one split expert at each end. For every chunk this kernel writes the experts' row
// ranges clamped to the chunk and the prefix of their m-tile counts, so that the grouped GEMM
// launches of a chunk find their tiles on the device: the host never reads the routing back.
#include "common.h"

namespace moe {

// One block per chunk, one thread per expert (E <= 1024):
//   ctile[c][e + 1] = sum over e' <= e of ceil(rows of e' inside chunk c / 256), ctile[c][0] = 0
//   crow[c][e + 1]  = offsets[e + 1] clamped to [c b, min(n, (c + 1) b)], crow[c][0] = c b
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
  int32_t* ro = crow + (int64_t)c * (E + 1);
  if (e < E) ro[e + 1] = min(max(offsets[e + 1], c0), c1);
  if (e == 0) ro[0] = c0;
}

int launch_chunk_tables(const int32_t* offsets, int E, int n, int b, int C, int32_t* ctile, int32_t* crow,
                        hipStream_t s) {
  if (C <= 0) return MOE_OK;
  hipLaunchKernelGGL(chunk_tiles_kernel, dim3(C), dim3(1024), 0, s, offsets, E, n, b, ctile, crow);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
