// Row movement kernels: dispatch into expert-contiguous slots, the fixed-order combine, and the
// MX quantiser. All are HBM-bound row copies with 16-byte vector accesses.
//
// Dispatch is the one-GPU analogue of the pull dispatch (sparsenotes page "Mixture-of-Kittens:
// MoE Megakernel for NVL72s", section "Pull dispatch, push combine"): the destination slot j
// reads its source row perm[j] / K. Combine is the source side's weighted sum over the
// per-route rows y[t*K + k] that the push combine wrote (Cursor blog "Mixture-of-Kittens: our
// open-source MoE megakernel for NVL72s", section "Scheduling", where one table serves both
// exchanges), summed in a fixed order with no atomics (sparsenotes page, "The production
// details", on determinism).
#include "common.h"
#include "mx_codec.h"

namespace moe {

// ---------------------------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------------------------
// One wavefront per destination slot; 16-byte chunks.
__global__ __launch_bounds__(256) void dispatch_kernel(const uint4* __restrict__ x,
                                                       const int32_t* __restrict__ perm, int K,
                                                       int chunks_per_row, int64_t begin,
                                                       int64_t count, uint4* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= count) return;
  const int64_t src = perm[begin + j] / K;
  const uint4* s = x + src * chunks_per_row;
  uint4* d = out + j * chunks_per_row;
  // 8 loads in flight per lane before their stores (a D = 7168 row is 14 chunks per lane)
  int c = lane;
  for (; c + 7 * 64 < chunks_per_row; c += 8 * 64) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = s[c + u * 64];
#pragma unroll
    for (int u = 0; u < 8; ++u) d[c + u * 64] = v[u];
  }
  for (; c < chunks_per_row; c += 64) d[c] = s[c];
}

// MXFP8 dispatch: one lane per 32-element block of the row.
__global__ __launch_bounds__(256) void dispatch_mx_kernel(const uint16_t* __restrict__ x,
                                                          const int32_t* __restrict__ perm, int K,
                                                          int D, int64_t begin, int64_t count,
                                                          uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ sc) {
  const int lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= count) return;
  const int64_t src = perm[begin + j] / K;
  const int nb = D / 32;
  for (int b = lane; b < nb; b += 64) {
    const uint4* s = reinterpret_cast<const uint4*>(x + src * D + b * 32);
    float v[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 u = s[c];
      uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * c + 2 * i] = __uint_as_float(w[i] << 16);
        v[8 * c + 2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    }
    uint32_t p[8];
    sc[j * nb + b] = (uint8_t)mx_block(v, p);
    uint4* d = reinterpret_cast<uint4*>(q + j * D + b * 32);
    d[0] = make_uint4(p[0], p[1], p[2], p[3]);
    d[1] = make_uint4(p[4], p[5], p[6], p[7]);
  }
}

// Token-major dispatch of the whole routed range: one wavefront per token reads its row of x once
// and writes it to the token's K slots inv_perm[t*K + k] (the same bytes as the slot-major gather,
// with x read from HBM once instead of once per route).
// The slot rows are stored with nontemporal (streaming) stores: nothing reads them again before the
// grouped GEMM, and 0.94 GB of slots at the DeepSeek-V3 shape would only evict other lines from the
// caches (measured 0.60 -> 0.72 of HBM peak at T = 8192, K = 8, D = 7168).
__global__ __launch_bounds__(256) void dispatch_tokens_kernel(const uint4* __restrict__ x,
                                                              const int32_t* __restrict__ inv_perm, int T, int K,
                                                              int chunks_per_row, uint4* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const u32x4* s = reinterpret_cast<const u32x4*>(x) + (int64_t)t * chunks_per_row;
  u32x4* o = reinterpret_cast<u32x4*>(out);
  const int32_t* slots = inv_perm + (int64_t)t * K;
  int c = lane;
  for (; c + 7 * 64 < chunks_per_row; c += 8 * 64) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = s[c + u * 64];
    for (int k = 0; k < K; ++k) {
      u32x4* d = o + (int64_t)slots[k] * chunks_per_row;
#pragma unroll
      for (int u = 0; u < 8; ++u) __builtin_nontemporal_store(v[u], d + c + u * 64);
    }
  }
  for (; c < chunks_per_row; c += 64) {
    const u32x4 v = s[c];
    for (int k = 0; k < K; ++k) __builtin_nontemporal_store(v, o + (int64_t)slots[k] * chunks_per_row + c);
  }
}

// Token-major MXFP8 dispatch: one wavefront per token quantises each 32-wide block of its row
// once and writes the codes and the scale byte to the token's K slots. The codes are exchanged
// across lanes first so that every store instruction covers 1 KB of whole lines: stored as each
// lane's own two 16-byte halves, nontemporal stores left gaps in every line and were slower
// (0.59 -> 0.80 ms at T = 32768).
__global__ __launch_bounds__(256) void dispatch_tokens_mx_kernel(const uint16_t* __restrict__ x,
                                                                 const int32_t* __restrict__ inv_perm, int T,
                                                                 int K, int D, uint8_t* __restrict__ q,
                                                                 uint8_t* __restrict__ sc) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int32_t* slots = inv_perm + (int64_t)t * K;
  const int nb = D / 32;
  for (int base = 0; base < nb; base += 64) {
    // lane quantises block b = base + lane
    const int b = base + lane;
    u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    uint8_t e = 127;
    if (b < nb) {
      const uint4* s = reinterpret_cast<const uint4*>(x + (int64_t)t * D + b * 32);
      float v[32];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint4 u = s[c];
        uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[8 * c + 2 * i] = __uint_as_float(w[i] << 16);
          v[8 * c + 2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
      }
      uint32_t p[8];
      e = (uint8_t)mx_block(v, p);
      lo = u32x4{p[0], p[1], p[2], p[3]};
      hi = u32x4{p[4], p[5], p[6], p[7]};
    }
    // Lane l then stores 16-byte chunk l of the 64 blocks' 2 KB of codes (block base + l / 2,
    // half l % 2) and chunk 64 + l (block base + 32 + l / 2), so each store instruction writes
    // 1 KB of whole lines and nontemporal stores can be used.
    const int s0 = lane >> 1, s1 = 32 + (lane >> 1);
    u32x4 c0, c1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t l0 = __shfl(lo[i], s0, 64), h0 = __shfl(hi[i], s0, 64);
      const uint32_t l1 = __shfl(lo[i], s1, 64), h1 = __shfl(hi[i], s1, 64);
      c0[i] = (lane & 1) ? h0 : l0;
      c1[i] = (lane & 1) ? h1 : l1;
    }
    const bool v0 = base + s0 < nb, v1 = base + s1 < nb;
    for (int k = 0; k < K; ++k) {
      const int64_t j = slots[k];
      if (b < nb) sc[j * nb + b] = e;
      u32x4* d = reinterpret_cast<u32x4*>(q + j * D + (int64_t)base * 32);
      if (v0) __builtin_nontemporal_store(c0, d + lane);
      if (v1) __builtin_nontemporal_store(c1, d + 64 + lane);
    }
  }
}

int launch_dispatch_tokens(const void* x, int dtype, const int32_t* inv_perm, int T, int K, int D, void* x_slot,
                           uint8_t* x_slot_sc, hipStream_t s) {
  if (T <= 0) return MOE_OK;
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (dtype == MOE_MXFP8) {
    hipLaunchKernelGGL(dispatch_tokens_mx_kernel, grid, block, 0, s, (const uint16_t*)x, inv_perm, T, K, D,
                       (uint8_t*)x_slot, x_slot_sc);
  } else {
    const int cpr = (int)(D * elt_bytes(dtype) / 16);
    hipLaunchKernelGGL(dispatch_tokens_kernel, grid, block, 0, s, (const uint4*)x, inv_perm, T, K, cpr,
                       (uint4*)x_slot);
  }
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

int launch_dispatch(const void* x, int dtype, const int32_t* perm, int K, int D, int64_t begin,
                    int64_t count, void* x_slot, uint8_t* x_slot_sc, hipStream_t s) {
  if (count <= 0) return MOE_OK;
  dim3 grid((unsigned)((count + 3) / 4)), block(256);
  if (dtype == MOE_MXFP8) {
    hipLaunchKernelGGL(dispatch_mx_kernel, grid, block, 0, s, (const uint16_t*)x, perm, K, D, begin,
                       count, (uint8_t*)x_slot, x_slot_sc);
  } else {
    const int cpr = (int)(D * elt_bytes(dtype) / 16);
    hipLaunchKernelGGL(dispatch_kernel, grid, block, 0, s, (const uint4*)x, perm, K, cpr, begin,
                       count, (uint4*)x_slot);
  }
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

// ---------------------------------------------------------------------------------------------
// combine: out[t] = shared[t] + sum_k w[t,k] * y[t*K+k], fp32, k ascending, one rounding
// ---------------------------------------------------------------------------------------------
// One wavefront per token. KC > 0: K = KC known at compile time; each lane takes 4 chunks of 8
// columns at a time and issues the 4 (K + 1) row loads together. KC = 0: any K, one chunk at a
// time. The per-route rows are read once, with nontemporal loads (0.61 -> 0.77 of HBM peak at
// T = 8192, K = 8, D = 7168). Same sum order either way: shared output first, then k ascending,
// fp32, one rounding.
__device__ __forceinline__ void bf16x8_to_f32(const u32x4 u, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(u[i] << 16);
    f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ void fma_bf16x8(const float g, const u32x4 u, float* acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] = fmaf(g, __uint_as_float(u[i] << 16), acc[2 * i]);
    acc[2 * i + 1] = fmaf(g, __uint_as_float(u[i] & 0xffff0000u), acc[2 * i + 1]);
  }
}

__device__ __forceinline__ u32x4 pack_bf16x8(const float* acc) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (uint32_t)f2bf(acc[2 * i]) | ((uint32_t)f2bf(acc[2 * i + 1]) << 16);
  return o;
}

template <int KC>
__global__ __launch_bounds__(256) void combine_bf16_kernel(const uint16_t* __restrict__ y,
                                                           const uint16_t* __restrict__ sh,
                                                           const float* __restrict__ w,
                                                           uint16_t* __restrict__ out, int T,
                                                           int K_, int D) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int chunks = D / 8;
  const u32x4* shr = sh ? reinterpret_cast<const u32x4*>(sh + (size_t)t * D) : nullptr;
  u32x4* orow = reinterpret_cast<u32x4*>(out + (size_t)t * D);
  if constexpr (KC > 0) {
    constexpr int U = 4;
    const u32x4* yr = reinterpret_cast<const u32x4*>(y + (size_t)t * KC * D);
    float g[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) g[k] = w[(size_t)t * KC + k];
    for (int c0 = lane; c0 < chunks; c0 += 64 * U) {
      u32x4 sv[U], yv[U][KC];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * 64;
        if (c < chunks) {
          sv[u] = shr ? shr[c] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
          for (int k = 0; k < KC; ++k) yv[u][k] = __builtin_nontemporal_load(yr + (size_t)k * chunks + c);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + u * 64;
        if (c >= chunks) break;
        float acc[8];
        bf16x8_to_f32(sv[u], acc);      // +0.0 when there is no shared expert
#pragma unroll
        for (int k = 0; k < KC; ++k) fma_bf16x8(g[k], yv[u][k], acc);
        orow[c] = pack_bf16x8(acc);
      }
    }
  } else {
    const int K = K_;
    const u32x4* yr = reinterpret_cast<const u32x4*>(y + (size_t)t * K * D);
    for (int c = lane; c < chunks; c += 64) {
      float acc[8];
      bf16x8_to_f32(shr ? shr[c] : u32x4{0u, 0u, 0u, 0u}, acc);
      for (int k = 0; k < K; ++k) fma_bf16x8(w[(size_t)t * K + k], __builtin_nontemporal_load(yr + (size_t)k * chunks + c), acc);
      orow[c] = pack_bf16x8(acc);
    }
  }
}

__global__ __launch_bounds__(256) void combine_f32_kernel(const float* __restrict__ y,
                                                          const float* __restrict__ sh,
                                                          const float* __restrict__ w,
                                                          float* __restrict__ out, int T, int K,
                                                          int D) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)T * D) return;
  const int64_t t = i / D, d = i % D;
  float acc = sh ? sh[i] : 0.f;
  for (int k = 0; k < K; ++k) acc = fmaf(w[t * K + k], y[(t * K + k) * D + d], acc);
  out[i] = acc;
}

int launch_combine(const void* y_routes, const void* shared_out, const float* topk_w, void* out,
                   int T, int K, int D, int dtype, hipStream_t s) {
  if (dtype == MOE_F32) {
    int64_t n = (int64_t)T * D;
    hipLaunchKernelGGL(combine_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const float*)y_routes, (const float*)shared_out, topk_w, (float*)out, T, K, D);
  } else {
    const dim3 grid((T + 3) / 4), block(256);
    const uint16_t* yr = (const uint16_t*)y_routes;
    const uint16_t* sh = (const uint16_t*)shared_out;
    uint16_t* o = (uint16_t*)out;
    switch (K) {
      case 8: hipLaunchKernelGGL(combine_bf16_kernel<8>, grid, block, 0, s, yr, sh, topk_w, o, T, K, D); break;
      case 6: hipLaunchKernelGGL(combine_bf16_kernel<6>, grid, block, 0, s, yr, sh, topk_w, o, T, K, D); break;
      case 4: hipLaunchKernelGGL(combine_bf16_kernel<4>, grid, block, 0, s, yr, sh, topk_w, o, T, K, D); break;
      case 2: hipLaunchKernelGGL(combine_bf16_kernel<2>, grid, block, 0, s, yr, sh, topk_w, o, T, K, D); break;
      default: hipLaunchKernelGGL(combine_bf16_kernel<0>, grid, block, 0, s, yr, sh, topk_w, o, T, K, D); break;
    }
  }
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

// ---------------------------------------------------------------------------------------------
// MX quantiser for whole matrices (offline weights): one thread per 32-element block
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quantize_mx_kernel(const uint16_t* __restrict__ src,
                                                          int64_t nblocks, uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ sc) {
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nblocks; b += (int64_t)gridDim.x * 256) {
    const uint4* s = reinterpret_cast<const uint4*>(src + b * 32);
    float v[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 u = s[c];
      uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * c + 2 * i] = __uint_as_float(w[i] << 16);
        v[8 * c + 2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    }
    uint32_t p[8];
    sc[b] = (uint8_t)mx_block(v, p);
    uint4* d = reinterpret_cast<uint4*>(q + b * 32);
    d[0] = make_uint4(p[0], p[1], p[2], p[3]);
    d[1] = make_uint4(p[4], p[5], p[6], p[7]);
  }
}

int launch_quantize_mx(const uint16_t* src, int64_t rows, int cols, uint8_t* q, uint8_t* sc,
                       hipStream_t s) {
  const int64_t nb = rows * (cols / 32);
  if (nb == 0) return MOE_OK;
  int64_t grid = (nb + 255) / 256;
  if (grid > 65536) grid = 65536;
  hipLaunchKernelGGL(quantize_mx_kernel, dim3((unsigned)grid), dim3(256), 0, s, src, nb, q, sc);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
