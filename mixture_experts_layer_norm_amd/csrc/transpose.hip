// Transposes and small row kernels of the backward pass.
//
// The weight-gradient GEMMs contract over the rows of one expert (dW = sum_j p_j q_j^T), so
// they read activations transposed, [features][rows], with each expert's rows starting at a
// multiple of 64 and the gap filled with zeros; every K step of those GEMMs is then a full,
// aligned 64-wide step. poff[e] (padded offsets) = sum over earlier experts of their row
// counts rounded up to 64.
#include "common.h"

namespace moe {

// Group bookkeeping from caller row offsets: a sanitised copy (offsets[0] taken as 0, every
// offset clamped to [previous, rows], so no later kernel can index past the buffers; a change
// sets the sticky error word), the m-tile prefix (kGemmBM rows) and the offsets padded to a
// multiple of `pad` (64 for the bf16 weight gradients, 128 for the MXFP8 ones).
__global__ __launch_bounds__(1024) void group_prefix_kernel(const int32_t* __restrict__ offsets, int G, int rows,
                                                            int32_t* __restrict__ clean, int32_t* __restrict__ tile_off,
                                                            int32_t* __restrict__ poff, int32_t* err, int pad) {
  __shared__ int sv[1024], sa[1024], sb[1024];
  const int t = threadIdx.x;
  const int raw = t < G ? offsets[t + 1] : 0;
  int v = t < G ? min(max(raw, 0), rows) : 0;
  sv[t] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {   // running maximum makes the offsets monotone
    const int o = t >= off ? sv[t - off] : 0;
    __syncthreads();
    sv[t] = max(sv[t], o);
    __syncthreads();
  }
  v = sv[t];
  const int prev = t == 0 ? 0 : sv[t - 1];
  if (t < G && (v != raw || (t == 0 && offsets[0] != 0))) atomicOr(err, 2);
  const int n = t < G ? v - prev : 0;
  sa[t] = t < G ? (n + kGemmBM - 1) / kGemmBM : 0;
  sb[t] = t < G ? (n + pad - 1) / pad * pad : 0;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int a = t >= off ? sa[t - off] : 0;
    const int b = t >= off ? sb[t - off] : 0;
    __syncthreads();
    sa[t] += a;
    sb[t] += b;
    __syncthreads();
  }
  if (t < G) {
    clean[t + 1] = v;
    tile_off[t + 1] = sa[t];
    poff[t + 1] = sb[t];
  }
  if (t == 0) {
    clean[0] = 0;
    tile_off[0] = 0;
    poff[0] = 0;
  }
}

// Groups ranked by their K extent (poff[g+1] - poff[g]) in decreasing order, ties to the lower
// index: order[rank] = group. The K-grouped GEMM deals its tiles in this order, longest first.
__global__ __launch_bounds__(1024) void group_order_kernel(const int32_t* __restrict__ poff, int G,
                                                           int32_t* __restrict__ order) {
  __shared__ int sz[1024];
  const int t = threadIdx.x;
  sz[t] = t < G ? poff[t + 1] - poff[t] : -1;
  __syncthreads();
  if (t >= G) return;
  const int mine = sz[t];
  int rank = 0;
  for (int u = 0; u < G; ++u) {
    const int o = sz[u];
    rank += (o > mine) || (o == mine && u < t);
  }
  order[rank] = t;
}

int launch_group_order(const int32_t* poff, int G, int32_t* order, hipStream_t s) {
  if (G < 1 || G > 1024) return MOE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(group_order_kernel, dim3(1), dim3(1024), 0, s, poff, G, order);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

int launch_group_prefix(const int32_t* offsets, int G, int rows, int32_t* clean, int32_t* tile_off, int32_t* poff,
                        int32_t* err, hipStream_t s, int pad) {
  hipLaunchKernelGGL(group_prefix_kernel, dim3(1), dim3(1024), 0, s, offsets, G, rows, clean, tile_off, poff, err, pad);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

// Grouped transpose into the padded layout. Source rows j of group e (offsets[e] <= j <
// offsets[e+1]) become columns poff[e] + (j - offsets[e]) of out [W][ldo]; columns in a group's
// padding become 0. Modes:
//   TR_COPY:   out = src[j][c]
//   TR_SWIGLU: out = scale[j] * SiLU(src[j][c]) * src2[j][c]  (gated activation from fp32 a, u;
//              scale optional); with split_lo the remainder v - bf16(v) goes to rows W..2W-1
// TR_COPY may read its rows through a row map: source row rmap[j] / rdiv instead of j (the
// layer backward reads x and dout rows through the schedule instead of slot copies).
// 64 x 64 tiles through LDS; each tile lies inside one group (poff is 64-aligned).
template <int MODE>
__global__ __launch_bounds__(256) void transpose_pad_kernel(const uint16_t* __restrict__ src,
                                                            const uint16_t* __restrict__ src2,
                                                            const float* __restrict__ scale, int64_t lds,
                                                            int W, const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ poff, int G,
                                                            uint16_t* __restrict__ out, int64_t ldo, int split_lo,
                                                            const int32_t* __restrict__ rmap, int rdiv) {
  __shared__ uint16_t tile[64][66];
  __shared__ uint16_t tile_lo[64][66];
  const int p0 = blockIdx.x * 64;          // padded column block
  const int c0 = blockIdx.y * 64;          // feature block
  if (p0 >= poff[G]) return;
  int lo = 0, hi = G - 1;                  // group holding padded column p0
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (poff[mid] <= p0) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int n = offsets[e + 1] - offsets[e];
  const int jbase = offsets[e] + (p0 - poff[e]);   // source row of padded column p0
  const int valid = min(64, n - (p0 - poff[e]));   // source rows present in this tile
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  // read 64 source rows x 64 features (coalesced along features)
  for (int r = ty; r < 64; r += 4) {
    uint16_t v = 0, vlo = 0;
    if (r < valid && c0 + tx < W) {
      const int64_t j = jbase + r;
      if (MODE == TR_COPY) v = src[(rmap ? (int64_t)(rmap[j] / rdiv) : j) * lds + c0 + tx];
      if (MODE == TR_SWIGLU) {
        const float* fa = reinterpret_cast<const float*>(src);
        const float* fu = reinterpret_cast<const float*>(src2);
        float f = silu_f(fa[j * lds + c0 + tx]) * fu[j * lds + c0 + tx];
        if (scale) f *= scale[j];
        v = f2bf_split(f);
        vlo = f2bf(f - bf2f(v));
      }
    }
    tile[r][tx] = v;
    tile_lo[r][tx] = vlo;
  }
  __syncthreads();
  // write 64 features x 64 padded columns (coalesced along columns); the low halves go W rows below
  for (int c = ty; c < 64; c += 4) {
    if (c0 + c < W) {
      out[(int64_t)(c0 + c) * ldo + p0 + tx] = tile[tx][c];
      if (split_lo) out[(int64_t)(W + c0 + c) * ldo + p0 + tx] = tile_lo[tx][c];
    }
  }
}

// TR_COPY of bf16 rows with 16-byte accesses on both sides: 64 padded columns x 64 features per
// workgroup; each thread loads 8 consecutive features of a source row and stores 8 consecutive
// padded columns of one output row. W % 8 == 0, lds % 8 == 0, ldo % 8 == 0.
__global__ __launch_bounds__(256) void transpose_pad_copy16_kernel(const uint16_t* __restrict__ src, int64_t lds,
                                                                   int W, const int32_t* __restrict__ offsets,
                                                                   const int32_t* __restrict__ poff, int G,
                                                                   uint16_t* __restrict__ out, int64_t ldo,
                                                                   const int32_t* __restrict__ rmap, int rdiv) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];
  const int p0 = blockIdx.x * 64;          // padded column block
  const int c0 = blockIdx.y * 64;          // feature block
  if (p0 >= poff[G]) return;
  int lo = 0, hi = G - 1;                  // group holding padded column p0
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (poff[mid] <= p0) lo = mid; else hi = mid - 1;
  }
  const int n = offsets[lo + 1] - offsets[lo];
  const int jbase = offsets[lo] + (p0 - poff[lo]);
  const int valid = min(64, n - (p0 - poff[lo]));
  const int t = threadIdx.x, q = t & 7, rr = t >> 3;   // chunk of 8, row in a pass of 32
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int r = rr + 32 * pass;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < valid && c0 + q * 8 < W) {
      const int64_t j = rmap ? (int64_t)(rmap[jbase + r] / rdiv) : (int64_t)(jbase + r);
      v = *reinterpret_cast<const u32x4*>(src + j * lds + c0 + q * 8);
    }
    *reinterpret_cast<u32x4*>(&tile[r][q * 8]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int c = rr + 32 * pass;            // feature within the block
    if (c0 + c >= W) continue;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = (uint32_t)tile[q * 8 + 2 * k][c] | ((uint32_t)tile[q * 8 + 2 * k + 1][c] << 16);
    u32x4 o = {w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4*>(out + (int64_t)(c0 + c) * ldo + p0 + q * 8) = o;
  }
}

int launch_transpose_pad(int mode, const void* src, const void* src2, const float* scale, int64_t lds, int W,
                         const int32_t* offsets, const int32_t* poff, int G, int64_t max_padded, void* out,
                         int64_t ldo, hipStream_t s, int split_lo, const int32_t* rmap, int rdiv) {
  if (mode != TR_COPY && mode != TR_SWIGLU) return MOE_ERR_INVALID_ARG;
  if (rmap && mode != TR_COPY) return MOE_ERR_UNSUPPORTED;
  dim3 grid((unsigned)((max_padded + 63) / 64), (unsigned)((W + 63) / 64)), block(256);
  const uint16_t* a = (const uint16_t*)src;
  const uint16_t* b = (const uint16_t*)src2;
  uint16_t* o = (uint16_t*)out;
  const bool v16 = mode == TR_COPY && !split_lo && W % 8 == 0 && lds % 8 == 0 && ldo % 8 == 0 &&
                   ((uintptr_t)src & 15) == 0 && ((uintptr_t)out & 15) == 0;
  if (v16)
    hipLaunchKernelGGL(transpose_pad_copy16_kernel, grid, block, 0, s, a, lds, W, offsets, poff, G, o, ldo, rmap, rdiv);
  else if (mode == TR_COPY)
    hipLaunchKernelGGL(transpose_pad_kernel<TR_COPY>, grid, block, 0, s, a, b, scale, lds, W, offsets, poff, G, o, ldo, split_lo, rmap, rdiv);
  else
    hipLaunchKernelGGL(transpose_pad_kernel<TR_SWIGLU>, grid, block, 0, s, a, b, scale, lds, W, offsets, poff, G, o, ldo, split_lo, nullptr, 1);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}


// dg[j] = sum over n-tiles of the per-tile partial <h, dh'> (fixed order)
__global__ __launch_bounds__(256) void row_sum_kernel(const float* __restrict__ part, int64_t rows, int ntn,
                                                      float* __restrict__ out) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= rows) return;
  float s = 0.f;
  for (int t = 0; t < ntn; ++t) s += part[j * ntn + t];
  out[j] = s;
}

int launch_row_sum(const float* part, int64_t rows, int ntn, float* out, hipStream_t s) {
  if (rows == 0) return MOE_OK;
  hipLaunchKernelGGL(row_sum_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, part, rows, ntn, out);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

// g_slot[j] = topk_w[perm[j]]  (router weight of each slot)
__global__ __launch_bounds__(256) void gather_f32_kernel(const float* __restrict__ src, const int32_t* __restrict__ idx,
                                                         int64_t n, float* __restrict__ out) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j < n) out[j] = src[idx[j]];
}

int launch_gather_f32(const float* src, const int32_t* idx, int64_t n, float* out, hipStream_t s) {
  if (n == 0) return MOE_OK;
  hipLaunchKernelGGL(gather_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, idx, n, out);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

// Router backward, one wavefront per token: d_topk_w[t][k] = dg_slot[inv_perm[t*K + k]] and
// d_logits[t][e] = g_e (dg_e - sum_j g_j dg_j) on the chosen experts, 0 elsewhere. This is the
// derivative of g_i = exp(l_i) / sum_{j chosen} exp(l_j) (the softmax denominator cancels).
__global__ __launch_bounds__(256) void router_backward_kernel(const float* __restrict__ dg_slot,
                                                              const int32_t* __restrict__ inv_perm,
                                                              const int32_t* __restrict__ topk_idx,
                                                              const float* __restrict__ topk_w, int T, int E,
                                                              int K, float* __restrict__ d_topk_w,
                                                              float* __restrict__ d_logits) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float dg = 0.f, g = 0.f;
  int e = -1;
  if (lane < K) {
    dg = dg_slot[inv_perm[(int64_t)t * K + lane]];
    g = topk_w[(int64_t)t * K + lane];
    e = topk_idx[(int64_t)t * K + lane];
    d_topk_w[(int64_t)t * K + lane] = dg;
  }
  if (!d_logits) return;
  // inner = sum_k g_k dg_k, summed in k order on every lane
  float inner = 0.f;
  for (int k = 0; k < K; ++k) inner = fmaf(__shfl(g, k, 64), __shfl(dg, k, 64), inner);
  const float mine = g * (dg - inner);
  for (int c = lane; c < E; c += 64) {
    float v = 0.f;
    for (int k = 0; k < K; ++k) {
      const int ek = __shfl(e, k, 64);
      const float vk = __shfl(mine, k, 64);
      if (ek == c) v = vk;
    }
    d_logits[(int64_t)t * E + c] = v;
  }
}

int launch_router_backward(const float* dg_slot, const int32_t* inv_perm, const int32_t* topk_idx,
                           const float* topk_w, int T, int E, int K, float* d_topk_w, float* d_logits,
                           hipStream_t s) {
  hipLaunchKernelGGL(router_backward_kernel, dim3((T + 3) / 4), dim3(256), 0, s, dg_slot, inv_perm, topk_idx,
                     topk_w, T, E, K, d_topk_w, d_logits);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

// Reverse dispatch: dx[t] = dx_shared[t] + sum_k dx_slot[inv_perm[t*K + k]], fp32, k ascending.
__global__ __launch_bounds__(256) void reverse_dispatch_kernel(const uint16_t* __restrict__ dxs,
                                                               const int32_t* __restrict__ inv_perm,
                                                               const uint16_t* __restrict__ dsh,
                                                               uint16_t* __restrict__ dx, int T, int K, int D) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  for (int c = lane; c < D / 8; c += 64) {
    float acc[8];
    if (dsh) {
      u32x4 u = reinterpret_cast<const u32x4*>(dsh + (int64_t)t * D)[c];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __uint_as_float(u[i] << 16);
        acc[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    }
    for (int k = 0; k < K; ++k) {
      const int64_t j = inv_perm[(int64_t)t * K + k];
      u32x4 u = reinterpret_cast<const u32x4*>(dxs + j * D)[c];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += __uint_as_float(u[i] << 16);
        acc[2 * i + 1] += __uint_as_float(u[i] & 0xffff0000u);
      }
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (uint32_t)f2bf(acc[2 * i]) | ((uint32_t)f2bf(acc[2 * i + 1]) << 16);
    reinterpret_cast<u32x4*>(dx + (int64_t)t * D)[c] = o;
  }
}

int launch_reverse_dispatch(const void* dx_slot, const int32_t* inv_perm, const void* dx_shared, void* dx, int T,
                            int K, int D, hipStream_t s) {
  hipLaunchKernelGGL(reverse_dispatch_kernel, dim3((T + 3) / 4), dim3(256), 0, s, (const uint16_t*)dx_slot, inv_perm,
                     (const uint16_t*)dx_shared, (uint16_t*)dx, T, K, D);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
