// Operand preparation of the MXFP8 expert backward (sparsenotes page "Mixture-of-Kittens: MoE
// Megakernel for NVL72s", "The production details": the routed experts train in MXFP8). Every
// backward GEMM takes both operands quantised along its own contraction dimension (OCP MX v1.0,
// blocks of 32), so besides the row quantiser three kernels are needed:
//
//   * mx_requant_t_kernel: a forward MX weight [R][C] (blocks along C) dequantised and quantised
//     again along R into its transpose [C][R] (W_down along D for dgrad-down, W_gate / W_up
//     along I for dgrad-up);
//   * mx_quant_t_kernel: an activation of the slot rows, grouped by expert, transposed and
//     quantised along the slots: [cols][padded slots], each expert's slots starting at a multiple
//     of 128 (one K slice of the MX GEMM), the padding zeros. Blocks start at the expert's first
//     slot. Sources: x, g * dy, h = SiLU(a) u, or [da | du];
//   * mx_swiglu_bwd_kernel: the SwiGLU backward of one slot row from the replayed a, u and the
//     dgrad-down output dh' (all fp32): da, du (fp32, and quantised along I for dgrad-up), h
//     (fp32) and the router-weight gradient dg = <h, dh'> summed in a fixed order.
#include "common.h"
#include "mx_codec.h"

namespace moe {

// Column pass shared by both transposing quantisers: tile[32][256] fp32 in LDS holds 32
// consecutive rows of the source block; thread c quantises column c0 + c (32 values down the
// rows) and writes 32 codes at q_row + p0 and the scale byte at sc_row[p0 / 32].
__device__ __forceinline__ void quantise_column(const float (*tile)[257], int c, uint8_t* q_row, uint8_t* sc_byte) {
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = tile[i][c];
  uint32_t p[8];
  *sc_byte = (uint8_t)mx_block(v, p);
  u32x4* d = reinterpret_cast<u32x4*>(q_row);
  d[0] = u32x4{p[0], p[1], p[2], p[3]};
  d[1] = u32x4{p[4], p[5], p[6], p[7]};
}

// grid (R / 32, ceil(C / 256), G), 256 threads. src [G][R][C] codes + [G][R][C/32] scales;
// out row c of batch g at out + g * out_bstride + c * ldo + col0 (codes, along R) and the scales
// at osc + g * osc_bstride + c * (ldo / 32) + col0 / 32.
__global__ __launch_bounds__(256) void mx_requant_t_kernel(const uint8_t* __restrict__ src, const uint8_t* __restrict__ ssc,
                                                           int R, int C, uint8_t* __restrict__ out, uint8_t* __restrict__ osc,
                                                           int64_t ldo, int64_t col0, int64_t out_bstride,
                                                           int64_t osc_bstride) {
  __shared__ float tile[32][257];
  const int tid = threadIdx.x, g = blockIdx.z;
  const int r0 = blockIdx.x * 32, c0 = blockIdx.y * 256;
  const uint8_t* s = src + (int64_t)g * R * C;
  const uint8_t* sc = ssc + (int64_t)g * R * (C / 32);
  // 32 rows x 256 codes = 512 chunks of 16 codes, 2 per thread
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int qd = tid + 256 * k, i = qd >> 4, cc = (qd & 15) * 16;
    if (c0 + cc < C) {
      const int64_t r = r0 + i;
      const u32x4 w = *reinterpret_cast<const u32x4*>(s + r * C + c0 + cc);
      const float scale = e8m0_value(sc[r * (C / 32) + (c0 + cc) / 32]);
#pragma unroll
      for (int b = 0; b < 16; ++b) tile[i][cc + b] = e4m3_value((w[b >> 2] >> (8 * (b & 3))) & 0xffu) * scale;
    }
  }
  __syncthreads();
  const int c = c0 + tid;
  if (c < C)
    quantise_column(tile, tid, out + (int64_t)g * out_bstride + (int64_t)c * ldo + col0 + r0,
                    osc + (int64_t)g * osc_bstride + (int64_t)c * (ldo / 32) + (col0 + r0) / 32);
}

// grid (max padded slots / 32, ceil(W / 256)), 256 threads. Slot block [p0, p0 + 32) lies in the
// group g with poff[g] <= p0 < poff[g + 1]; its source rows are offs[g] + p0 - poff[g] + i while
// below offs[g + 1] (zeros past it). Output row c (source column) at q + c * ldo + p0, scales at
// sc + c * (ldo / 32) + p0 / 32.
__global__ __launch_bounds__(256) void mx_quant_t_kernel(int mode, const void* __restrict__ src, const float* __restrict__ src2,
                                                         const float* __restrict__ rscale, int64_t lds, int W,
                                                         const int32_t* __restrict__ offs, const int32_t* __restrict__ poff,
                                                         int G, uint8_t* __restrict__ q, uint8_t* __restrict__ sc,
                                                         int64_t ldo) {
  __shared__ float tile[32][257];
  const int tid = threadIdx.x;
  const int p0 = blockIdx.x * 32, c0 = blockIdx.y * 256;
  if (p0 >= poff[G]) return;
  int lo = 0, hi = G - 1;   // last group with poff[g] <= p0 (empty groups have poff[g] == poff[g + 1])
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (poff[mid] <= p0) lo = mid; else hi = mid - 1;
  }
  const int64_t rbase = (int64_t)offs[lo] + (p0 - poff[lo]);
  const int64_t rend = offs[lo + 1];
  if (mode == MXT_F32 || mode == MXT_SWIGLU) {
    // 32 rows x 64 chunks of 4 floats, 8 per thread
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int qd = tid + 256 * k, i = qd >> 6, cc = (qd & 63) * 4;
      const int64_t r = rbase + i;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (r < rend && c0 + cc < W) {
        v = *reinterpret_cast<const f32x4*>((const float*)src + r * lds + c0 + cc);
        if (mode == MXT_SWIGLU) {
          const f32x4 u = *reinterpret_cast<const f32x4*>(src2 + r * lds + c0 + cc);
#pragma unroll
          for (int b = 0; b < 4; ++b) v[b] = silu_f(v[b]) * u[b];
        }
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) tile[i][cc + b] = v[b];
    }
  } else {
    // bf16: 32 rows x 32 chunks of 8, 4 per thread; MXT_BF16_SCALED multiplies by rscale[row]
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int qd = tid + 256 * k, i = qd >> 5, cc = (qd & 31) * 8;
      const int64_t r = rbase + i;
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (r < rend && c0 + cc < W) {
        const u32x4 w = *reinterpret_cast<const u32x4*>((const uint16_t*)src + r * lds + c0 + cc);
        const float f = mode == MXT_BF16_SCALED ? rscale[r] : 1.f;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          v[2 * b] = __uint_as_float(w[b] << 16) * f;
          v[2 * b + 1] = __uint_as_float(w[b] & 0xffff0000u) * f;
        }
      }
#pragma unroll
      for (int b = 0; b < 8; ++b) tile[i][cc + b] = v[b];
    }
  }
  __syncthreads();
  const int c = c0 + tid;
  if (c < W) quantise_column(tile, tid, q + (int64_t)c * ldo + p0, sc + (int64_t)c * (ldo / 32) + p0 / 32);
}

// One wavefront per slot row j < n: lane l takes the 32-element blocks b = l, l + 64, ... of the
// I columns. da, du -> daf [n][2I] (fp32) and, quantised per block along I, dq [n][2I] codes +
// dsc [n][2I / 32] (du blocks after the I / 32 da blocks); h -> hf [n][I]; dg[j] = <h, dh'>
// (per-lane sums in column order, then a fixed butterfly across the wavefront).
__global__ __launch_bounds__(256) void mx_swiglu_bwd_kernel(const float* __restrict__ a, const float* __restrict__ u,
                                                            const float* __restrict__ dhp, const float* __restrict__ g,
                                                            int64_t n, int I, float* __restrict__ hf,
                                                            float* __restrict__ daf, uint8_t* __restrict__ dq,
                                                            uint8_t* __restrict__ dsc, float* __restrict__ dg) {
  const int lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= n) return;
  const float gj = g[j];
  const int nb = I / 32;
  float part = 0.f;
  for (int b = lane; b < nb; b += 64) {
    const int64_t e0 = j * I + b * 32;
    float da[32], du[32];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const f32x4 av = *reinterpret_cast<const f32x4*>(a + e0 + 4 * c);
      const f32x4 uv = *reinterpret_cast<const f32x4*>(u + e0 + 4 * c);
      const f32x4 pv = *reinterpret_cast<const f32x4*>(dhp + e0 + 4 * c);
      f32x4 hv;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float x = av[k], s = sigmoid_f(x), sa = x * s;
        hv[k] = sa * uv[k];
        part = fmaf(hv[k], pv[k], part);
        const float dh = gj * pv[k];
        da[4 * c + k] = dh * uv[k] * s * (1.f + x * (1.f - s));
        du[4 * c + k] = dh * sa;
      }
      *reinterpret_cast<f32x4*>(hf + e0 + 4 * c) = hv;
    }
    const int64_t d0 = j * 2 * I + b * 32;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      *reinterpret_cast<f32x4*>(daf + d0 + 4 * c) = f32x4{da[4 * c], da[4 * c + 1], da[4 * c + 2], da[4 * c + 3]};
      *reinterpret_cast<f32x4*>(daf + d0 + I + 4 * c) = f32x4{du[4 * c], du[4 * c + 1], du[4 * c + 2], du[4 * c + 3]};
    }
    uint32_t p[8];
    dsc[j * (2 * nb) + b] = (uint8_t)mx_block(da, p);
    u32x4* qd = reinterpret_cast<u32x4*>(dq + d0);
    qd[0] = u32x4{p[0], p[1], p[2], p[3]};
    qd[1] = u32x4{p[4], p[5], p[6], p[7]};
    dsc[j * (2 * nb) + nb + b] = (uint8_t)mx_block(du, p);
    qd = reinterpret_cast<u32x4*>(dq + d0 + I);
    qd[0] = u32x4{p[0], p[1], p[2], p[3]};
    qd[1] = u32x4{p[4], p[5], p[6], p[7]};
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
  if (lane == 0) dg[j] = part;
}

int launch_mx_requant_t(const uint8_t* src, const uint8_t* ssc, int G, int R, int C, uint8_t* out, uint8_t* osc,
                        int64_t ldo, int64_t col0, int64_t out_bstride, int64_t osc_bstride, hipStream_t s) {
  if (G <= 0 || R <= 0 || C <= 0) return MOE_OK;
  if (R % 32 || C % 32 || ldo % 32 || col0 % 32) return MOE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(mx_requant_t_kernel, dim3(R / 32, (C + 255) / 256, G), dim3(256), 0, s, src, ssc, R, C, out, osc,
                     ldo, col0, out_bstride, osc_bstride);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

int launch_mx_quant_t(int mode, const void* src, const float* src2, const float* rscale, int64_t lds, int W,
                      const int32_t* offs, const int32_t* poff, int G, int64_t max_padded, uint8_t* q, uint8_t* sc,
                      int64_t ldo, hipStream_t s) {
  if (max_padded <= 0 || W <= 0) return MOE_OK;
  if (max_padded % 32 || ldo % 128 || W % 8 || lds % 8) return MOE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(mx_quant_t_kernel, dim3((unsigned)(max_padded / 32), (W + 255) / 256), dim3(256), 0, s, mode, src,
                     src2, rscale, lds, W, offs, poff, G, q, sc, ldo);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

int launch_mx_swiglu_bwd(const float* a, const float* u, const float* dhp, const float* g, int64_t n, int I, float* hf,
                         float* daf, uint8_t* dq, uint8_t* dsc, float* dg, hipStream_t s) {
  if (n <= 0) return MOE_OK;
  if (I % 32) return MOE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(mx_swiglu_bwd_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, s, a, u, dhp, g, n, I, hf, daf,
                     dq, dsc, dg);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
