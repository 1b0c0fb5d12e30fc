// Backward of the router projection logits = x W_r^T (the router of the Cursor blog
// "Mixture-of-Kittens: our open-source MoE megakernel for NVL72s", section "Overlapping
// computation and communication in MoE", whose logits moe_route_gemm computes):
//   dW_r [E][D] = d_logits^T x        (contraction over the T tokens)
//   dx   [T][D] += d_logits W_r       (contraction over the E experts, added to the experts' dx)
// d_logits is fp32 (nonzero only on each token's K chosen experts, as moe_backward writes it),
// x and W_r are bf16. Both products are formed exactly in fp32 (a bf16 times an fp32 value has
// at most 8 + 24 significant bits, so only the fp32 accumulation rounds), each output as one
// thread's fma chain in ascending k (token for dW_r, expert for dx): deterministic and
// independent of the launch shape. The kernels below take only the nonzero entries of d_logits;
// where the operands lack the alignment of their vector accesses, a dense strided FMA GEMM (64 x
// 64 outputs per workgroup, K slices of 32 staged through LDS) forms the same chains over every
// entry, with the same bits.
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

// Both products skip the zero entries of d_logits (moe_backward leaves K of each token's E entries
// nonzero). A zero entry contributes an exact zero product, and adding it leaves an fp32 sum
// unchanged (up to the sign of an all-zero sum), so taking the nonzero entries in the dense
// kernel's order (ascending expert for dx, ascending token for dW_r) with the same fma gives its
// result bit for bit, at about K/E of its work.

// dx[t][:] += d_logits[t][:] W_r, one wavefront per token. The wavefront lists the token's
// nonzero (expert, value) pairs in ascending expert order in LDS (one ballot per 64 experts), then
// walks 512-column blocks (8 columns per lane, 16-byte loads of W_r and dx), issuing the W_r rows
// of up to 8 list entries before their fmas.
__global__ __launch_bounds__(256) void router_dx_sparse_kernel(const float* __restrict__ dl,
                                                               const uint16_t* __restrict__ w,
                                                               uint16_t* __restrict__ dx, int T, int D, int E) {
  __shared__ int s_e[4][1024];
  __shared__ float s_v[4][1024];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;   // wave-uniform; no workgroup barrier below
  const float* drow = dl + (int64_t)t * E;
  int n = 0;
  for (int b = 0; b * 64 < E; ++b) {
    const int e = b * 64 + lane;
    const float v = e < E ? drow[e] : 0.f;
    const uint64_t m = __ballot(v != 0.f);
    if (v != 0.f) {
      const int pos = n + __popcll(m & ((1ull << lane) - 1));
      s_e[wv][pos] = e;
      s_v[wv][pos] = v;
    }
    n += __popcll(m);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int c0 = 0; c0 < D; c0 += 512) {
    const int col = c0 + lane * 8;
    const bool ok = col < D;   // D % 8 == 0: a lane's 8 columns are all in range or none
    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.f;
    for (int j0 = 0; j0 < n; j0 += 8) {
      uint4 q[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        q[j] = (ok && j0 + j < n) ? *reinterpret_cast<const uint4*>(w + (int64_t)s_e[wv][j0 + j] * D + col)
                                  : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j0 + j >= n) break;
        const float d = s_v[wv][j0 + j];
        const uint32_t u[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[2 * k] = fmaf(d, __uint_as_float(u[k] << 16), acc[2 * k]);
          acc[2 * k + 1] = fmaf(d, __uint_as_float(u[k] & 0xffff0000u), acc[2 * k + 1]);
        }
      }
    }
    if (ok) {
      uint4* p = reinterpret_cast<uint4*>(dx + (int64_t)t * D + col);
      const uint4 q = *p;
      const uint32_t u[4] = {q.x, q.y, q.z, q.w};
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint16_t lo = f2bf(__uint_as_float(u[k] << 16) + acc[2 * k]);
        const uint16_t hi = f2bf(__uint_as_float(u[k] & 0xffff0000u) + acc[2 * k + 1]);
        o[k] = (uint32_t)lo | ((uint32_t)hi << 16);
      }
      *p = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

// dW_r[e][:] = sum over tokens t of d_logits[t][e] x[t][:], one workgroup per 8 experts and
// 512-column block (2 columns per thread). Per segment of 1024 tokens the workgroup reads its 8
// columns of d_logits once (all 32 loads of a thread in flight together) and lists, per expert,
// its nonzero (token, value) pairs in ascending token order; then it walks the 8 lists one after
// another, loading each listed token's x row block (two batches of 32 tokens in flight per thread)
// into that expert's sum.
constexpr int kDwSeg = 1024, kDwBatch = 16;
__global__ __launch_bounds__(256) void router_dw_sparse_kernel(const float* __restrict__ dl,
                                                               const uint16_t* __restrict__ x,
                                                               float* __restrict__ dw, int T, int D, int E) {
  __shared__ int2 s_l[8][kDwSeg];     // per expert: (token, value bits)
  __shared__ int s_cnt[4][8];
  const int nblk = (D + 511) / 512;
  const int e0 = (blockIdx.x / nblk) * 8, col = (blockIdx.x % nblk) * 512 + threadIdx.x * 2;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool ok = col < D;   // D % 2 == 0
  constexpr int R = kDwSeg / 256;
  float acc[8][2];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k][0] = acc[k][1] = 0.f;
  // 16-byte reads of a token's 8 values where d_logits rows and this group are 16-byte aligned
  const bool v16 = e0 + 8 <= E && (E % 4) == 0 && ((uintptr_t)dl % 16) == 0;
  for (int t0 = 0; t0 < T; t0 += kDwSeg) {
    float v[R][8];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int t = t0 + r * 256 + tid;
      if (v16) {
        const float4 a = t < T ? *reinterpret_cast<const float4*>(dl + (int64_t)t * E + e0) : make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 b = t < T ? *reinterpret_cast<const float4*>(dl + (int64_t)t * E + e0 + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
        v[r][0] = a.x; v[r][1] = a.y; v[r][2] = a.z; v[r][3] = a.w;
        v[r][4] = b.x; v[r][5] = b.y; v[r][6] = b.z; v[r][7] = b.w;
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) v[r][k] = (t < T && e0 + k < E) ? dl[(int64_t)t * E + e0 + k] : 0.f;
      }
    }
    int n[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) n[k] = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint64_t bm[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        bm[k] = __ballot(v[r][k] != 0.f);
        if (lane == 0) s_cnt[wv][k] = __popcll(bm[k]);
      }
      __syncthreads();
      const int t = t0 + r * 256 + tid;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        int base = n[k];
        for (int q = 0; q < wv; ++q) base += s_cnt[q][k];
        if (v[r][k] != 0.f) s_l[k][base + __popcll(bm[k] & ((1ull << lane) - 1))] = make_int2(t, __float_as_int(v[r][k]));
        n[k] += s_cnt[0][k] + s_cnt[1][k] + s_cnt[2][k] + s_cnt[3][k];
      }
      __syncthreads();   // s_cnt is rewritten next round; the lists are complete after the last
    }
    // batches of kDwBatch entries, two in flight: batch b + 1 loads while batch b is summed
    auto load = [&](int k, int j0, uint32_t (&xv)[kDwBatch], float (&dv)[kDwBatch]) {
#pragma unroll
      for (int j = 0; j < kDwBatch; ++j) {
        const int2 en = j0 + j < n[k] ? s_l[k][j0 + j] : make_int2(0, 0);
        dv[j] = __int_as_float(en.y);
        xv[j] = (ok && j0 + j < n[k]) ? *reinterpret_cast<const uint32_t*>(x + (int64_t)en.x * D + col) : 0u;
      }
    };
    auto sum = [&](int k, int j0, const uint32_t (&xv)[kDwBatch], const float (&dv)[kDwBatch]) {
#pragma unroll
      for (int j = 0; j < kDwBatch; ++j) {
        if (j0 + j >= n[k]) break;
        acc[k][0] = fmaf(dv[j], __uint_as_float(xv[j] << 16), acc[k][0]);
        acc[k][1] = fmaf(dv[j], __uint_as_float(xv[j] & 0xffff0000u), acc[k][1]);
      }
    };
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t xa[kDwBatch], xb[kDwBatch];
      float da[kDwBatch], db[kDwBatch];
      if (n[k] > 0) load(k, 0, xa, da);
      for (int j0 = 0; j0 < n[k]; j0 += 2 * kDwBatch) {
        if (j0 + kDwBatch < n[k]) load(k, j0 + kDwBatch, xb, db);
        sum(k, j0, xa, da);
        if (j0 + kDwBatch >= n[k]) break;
        if (j0 + 2 * kDwBatch < n[k]) load(k, j0 + 2 * kDwBatch, xa, da);
        sum(k, j0 + kDwBatch, xb, db);
      }
    }
    __syncthreads();   // every thread is past the lists before the next segment rewrites them
  }
  if (ok) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (e0 + k < E) *reinterpret_cast<float2*>(dw + (int64_t)(e0 + k) * D + col) = make_float2(acc[k][0], acc[k][1]);
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
  const bool sparse = !(p->flags & MOE_FLAG_ROUTER_BWD_DENSE);
  if (sparse && ((uintptr_t)x % 4 == 0) && ((uintptr_t)dw_router % 8 == 0) && D % 2 == 0) {
    const int64_t wgs = (int64_t)((E + 7) / 8) * ((D + 511) / 512);
    hipLaunchKernelGGL(router_dw_sparse_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, d_logits,
                       (const uint16_t*)x, dw_router, T, D, E);
    MOE_LAUNCH_CHECK();
  } else {
    // dW_r[e][d] = sum_t d_logits[t][e] x[t][d]:  A(m = e, k = t) = d_logits[t E + e], B(n = d, k = t) = x[t D + d]
    if ((st = launch_router_gemm(d_logits, 1, E, (const uint16_t*)x, 1, D, dw_router, D, E, D, T, 0, stream))) return st;
  }
  if (!dx) return MOE_OK;
  if (sparse && ((uintptr_t)w_router | (uintptr_t)dx) % 16 == 0 && D % 8 == 0) {
    hipLaunchKernelGGL(router_dx_sparse_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, stream, d_logits,
                       (const uint16_t*)w_router, (uint16_t*)dx, T, D, E);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
  }
  // dx[t][d] += sum_e d_logits[t][e] W_r[e][d]:  A(m = t, k = e) = d_logits[t E + e], B(n = d, k = e) = W_r[e D + d]
  return launch_router_gemm(d_logits, E, 1, (const uint16_t*)w_router, 1, D, dx, D, T, D, E, 1, stream);
}

}  // extern "C"
