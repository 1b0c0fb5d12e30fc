// Backward of the router projection logits = x W_r^T (the router of the Cursor blog
// "Mixture-of-Kittens: our open-source MoE megakernel for NVL72s", section "Overlapping
// computation and communication in MoE", whose logits moe_route_gemm computes):
//   dW_r [E][D] = d_logits^T x        (contraction over the T tokens)
//   dx   [T][D] += d_logits W_r       (contraction over the E experts, added to the experts' dx)
// d_logits is fp32 (nonzero only on each token's K chosen experts, as moe_backward writes it),
// x and W_r are bf16. Both products are formed exactly in fp32 (a bf16 times an fp32 value has
// at most 8 + 24 significant bits, so only the fp32 accumulation rounds) by one strided FMA
// GEMM: 64 x 64 outputs per workgroup, 4 x 4 per thread, K slices of 32 staged through LDS
// with coalesced loads whichever operand axis is contiguous. Each output is one thread's sum in
// ascending k, so the results are deterministic and independent of the launch shape.
#include "common.h"

namespace moe {

constexpr int kRB = 64;   // outputs per workgroup tile side
constexpr int kRK = 32;   // K slice

// C[m][n] = sum_k A(m, k) B(n, k) with A(m, k) = A[m sam + k sak] (fp32) and
// B(n, k) = B[n sbn + k sbk] (bf16). accumulate_bf16: C is bf16 and receives bf16(C + sum);
// otherwise C is fp32 and is overwritten.
__global__ __launch_bounds__(256) void router_gemm_f32_kernel(const float* __restrict__ A, int64_t sam, int64_t sak,
                                                              const uint16_t* __restrict__ B, int64_t sbn,
                                                              int64_t sbk, void* __restrict__ C, int64_t ldc, int M,
                                                              int N, int K, int accumulate_bf16) {
  __shared__ float As[kRK][kRB + 4];
  __shared__ float Bs[kRK][kRB + 4];
  const int ntn = (N + kRB - 1) / kRB;
  const int m0 = (blockIdx.x / ntn) * kRB, n0 = (blockIdx.x % ntn) * kRB;
  const int tid = threadIdx.x, tm = tid >> 4, tn = tid & 15;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  const bool a_m_fast = sam == 1;   // which A axis is contiguous in memory (coalesced staging)
  const bool b_n_fast = sbn == 1;
  for (int k0 = 0; k0 < K; k0 += kRK) {
#pragma unroll
    for (int q = 0; q < kRB * kRK / 256; ++q) {
      const int i = tid + q * 256;
      const int mm = a_m_fast ? (i % kRB) : (i / kRK), kk = a_m_fast ? (i / kRB) : (i % kRK);
      const int m = m0 + mm, k = k0 + kk;
      As[kk][mm] = (m < M && k < K) ? A[(int64_t)m * sam + (int64_t)k * sak] : 0.f;
      const int nn = b_n_fast ? (i % kRB) : (i / kRK), kb = b_n_fast ? (i / kRB) : (i % kRK);
      const int n = n0 + nn, kq = k0 + kb;
      Bs[kb][nn] = (n < N && kq < K) ? bf2f(B[(int64_t)n * sbn + (int64_t)kq * sbk]) : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kRK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][tm * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tn * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + tm * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tn * 4 + j;
      if (n >= N) continue;
      if (accumulate_bf16) {
        uint16_t* c = (uint16_t*)C + (int64_t)m * ldc + n;
        *c = f2bf(bf2f(*c) + acc[i][j]);
      } else {
        ((float*)C)[(int64_t)m * ldc + n] = acc[i][j];
      }
    }
  }
}

static int launch_router_gemm(const float* A, int64_t sam, int64_t sak, const uint16_t* B, int64_t sbn, int64_t sbk,
                              void* C, int64_t ldc, int M, int N, int K, int acc_bf16, hipStream_t s) {
  const int64_t tiles = (int64_t)((M + kRB - 1) / kRB) * ((N + kRB - 1) / kRB);
  if (tiles == 0) return MOE_OK;
  if (tiles > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(router_gemm_f32_kernel, dim3((unsigned)tiles), dim3(256), 0, s, A, sam, sak, B, sbn, sbk, C, ldc,
                     M, N, K, acc_bf16);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_route_gemm_backward(const moe_problem* p, const void* x, const void* w_router, const float* d_logits,
                            float* dw_router, void* dx, hipStream_t stream) {
  int st = validate_routing(p);
  if (st) return st;
  if (p->dtype == MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (!x || !w_router || !d_logits || !dw_router) return MOE_ERR_INVALID_ARG;
  const int T = p->T, D = p->D, E = p->E;
  // dW_r[e][d] = sum_t d_logits[t][e] x[t][d]:  A(m = e, k = t) = d_logits[t E + e], B(n = d, k = t) = x[t D + d]
  if ((st = launch_router_gemm(d_logits, 1, E, (const uint16_t*)x, 1, D, dw_router, D, E, D, T, 0, stream))) return st;
  if (!dx) return MOE_OK;
  // dx[t][d] += sum_e d_logits[t][e] W_r[e][d]:  A(m = t, k = e) = d_logits[t E + e], B(n = d, k = e) = W_r[e D + d]
  return launch_router_gemm(d_logits, E, 1, (const uint16_t*)w_router, 1, D, dx, D, T, D, E, 1, stream);
}

}  // extern "C"
