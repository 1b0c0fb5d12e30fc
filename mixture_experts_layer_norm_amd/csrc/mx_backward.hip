// Operand preparation of the MXFP8 expert backward (sparsenotes page "Mixture-of-Kittens: MoE
// Megakernel for NVL72s", "The production details": the routed experts train in MXFP8). Every
// backward GEMM takes both operands quantised along its own contraction dimension (OCP MX v1.0,
// blocks of 32), so besides the row quantiser three kernels are needed:
//
//   * mx_requant_t_kernel: a forward MX weight [R][C] (blocks along C) dequantised and quantised
//     again along R into its transpose [C][R] (W_down along D for dgrad-down, W_gate / W_up
//     along I for dgrad-up);
//   * mx_quant_t_kernel: a bf16 activation of the slot rows (x, or dy scaled by g), grouped by
//     expert, transposed and quantised along the slots: [cols][padded slots], each expert's slots
//     starting at a multiple of 128 (one K slice of the MX GEMM), the padding zeros, blocks from
//     the expert's first slot; in the same pass the unscaled rows quantised along the features
//     (the dgrad operands Q_D(x), Q_D(dy)), so each is read once;
//   * mx_swiglu_bwd_t_kernel: the SwiGLU backward on a tile of 32 slots x 256 units from the
//     replayed a, u and the dgrad-down output dh' (all fp32): da, du quantised along I for
//     dgrad-up, and h, da, du quantised along the slots (the weight-gradient operands) from
//     registers, so neither h nor [da | du] goes through HBM in fp32; the router-weight gradient
//     dg = <h, dh'> as per-tile partial sums in a fixed order.
#include "common.h"
#include "mx_codec.h"

namespace moe {

// Workgroups are dealt round-robin to the 8 XCDs (workgroup b runs on XCD b % 8), each with its
// own L2. The transposing kernels write each 128-byte line of an output row in 32-byte pieces
// from neighbouring slot blocks; taking the tiles XCD-contiguously (XCD x takes tiles
// [x per, (x + 1) per), slot block fastest) keeps the pieces of a line in one L2 so they leave it
// as one line. Returns false for padding workgroups.
__device__ __forceinline__ bool xcd_tile(int nsb, int ntiles, int& sb, int& ct) {
  const int per = (ntiles + 7) >> 3;
  const int logical = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (logical >= ntiles) return false;
  sb = logical % nsb;
  ct = logical / nsb;
  return true;
}

static inline unsigned xcd_grid(int64_t ntiles) { return (unsigned)((ntiles + 7) / 8 * 8); }

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

// (max padded slots / 128) x ceil(W / 64) tiles (xcd_tile), 256 threads: a bf16 source block of
// 128 padded slot positions (one group's: poff is 128-aligned) x 64 features. Rows are
// offs[g] + p - poff[g] while below offs[g + 1]; past that the block holds zeros. Outputs:
//   * along the slots: feature c's 32-slot blocks -> q + c * ldo + p (codes) and
//     sc + c * (ldo / 32) + p / 32 (scales); with rscale the values are rscale[row] * src; four
//     neighbouring threads write one 128-byte line of an output row;
//   * along the features (rq != nullptr): each valid row's two 32-feature blocks -> rq + row * W +
//     c0 (codes) and rsc + row * (W / 32) + c0 / 32 (scales), from the unscaled source.
// With rmap, slot row r is read from source row rmap[r] / rdiv (the layer backward reads x and
// dout through the schedule instead of slot copies); outputs stay indexed by slot.
// The tile stays bf16 in LDS (18.5 KB, so 8 workgroups share a CU and their loads overlap): row r
// at halfword r * 72 + (r / 32) * 16, which puts the four 32-slot blocks a column read touches on
// different banks.
__global__ __launch_bounds__(256) void mx_quant_t_kernel(const uint16_t* __restrict__ src, const float* __restrict__ rscale,
                                                         int64_t lds, int W, const int32_t* __restrict__ offs,
                                                         const int32_t* __restrict__ poff, int G, uint8_t* __restrict__ q,
                                                         uint8_t* __restrict__ sc, int64_t ldo, uint8_t* __restrict__ rq,
                                                         uint8_t* __restrict__ rsc, int nsb, int ntiles,
                                                         const int32_t* __restrict__ rmap, int rdiv) {
  constexpr int P = 72;       // halfwords per tile row (64 + 8)
  __shared__ __attribute__((aligned(16))) uint16_t tile[128 * P + 64];
  __shared__ float rs[128];   // row scales of the block (1 without rscale or past the group's end)
  const int tid = threadIdx.x;
  int sb, ct;
  if (!xcd_tile(nsb, ntiles, sb, ct)) return;
  const int p0 = sb * 128, c0 = ct * 64;
  if (p0 >= poff[G]) return;
  int lo = 0, hi = G - 1;   // last group with poff[g] <= p0 (empty groups have poff[g] == poff[g + 1])
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (poff[mid] <= p0) lo = mid; else hi = mid - 1;
  }
  const int64_t rbase = (int64_t)offs[lo] + (p0 - poff[lo]);
  const int64_t rend = offs[lo + 1];
  auto at = [](int r, int c) { return r * P + (r >> 5) * 16 + c; };
  if (tid < 128) rs[tid] = (rscale && rbase + tid < rend) ? rscale[rbase + tid] : 1.f;
  // 128 rows x 8 chunks of 8 bf16, 4 per thread, stored as 16-byte LDS writes
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int qd = tid + 256 * k, i = qd >> 3, cc = (qd & 7) * 8;
    const int64_t r = rbase + i;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (r < rend && c0 + cc < W) {
      const int64_t sr = rmap ? (int64_t)(rmap[r] / rdiv) : r;   // source row of slot r
      w = *reinterpret_cast<const u32x4*>(src + sr * lds + c0 + cc);
    }
    *reinterpret_cast<u32x4*>(&tile[at(i, cc)]) = w;
  }
  __syncthreads();
  uint32_t pk[8];
  if (rq) {
    // along the features: row i, block b (unscaled source)
    const int i = tid >> 1, b = tid & 1;
    const int64_t r = rbase + i;
    if (r < rend && c0 + 32 * b < W) {
      float v[32];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(&tile[at(i, 32 * b + 8 * j)]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[8 * j + 2 * e] = __uint_as_float(w[e] << 16);
          v[8 * j + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
      }
      rsc[r * (W / 32) + c0 / 32 + b] = (uint8_t)mx_block(v, pk);
      u32x4* d = reinterpret_cast<u32x4*>(rq + r * W + c0 + 32 * b);
      d[0] = u32x4{pk[0], pk[1], pk[2], pk[3]};
      d[1] = u32x4{pk[4], pk[5], pk[6], pk[7]};
    }
  }
  {
    // along the slots: feature c, slot block k
    const int c = tid >> 2, k = tid & 3;
    if (c0 + c < W) {
      float v[32];
#pragma unroll
      for (int j = 0; j < 32; ++j)
        v[j] = __uint_as_float((uint32_t)tile[at(32 * k + j, c)] << 16) * rs[32 * k + j];
      sc[(int64_t)(c0 + c) * (ldo / 32) + (p0 >> 5) + k] = (uint8_t)mx_block(v, pk);
      u32x4* d = reinterpret_cast<u32x4*>(q + (int64_t)(c0 + c) * ldo + p0 + 32 * k);
      d[0] = u32x4{pk[0], pk[1], pk[2], pk[3]};
      d[1] = u32x4{pk[4], pk[5], pk[6], pk[7]};
    }
  }
}

// (max padded slots / 32) x ceil(I / 256) tiles (xcd_tile), 256 threads; thread t owns unit c = 256 ct + t of
// the 32 slots [p0, p0 + 32) of one group (rows as in mx_quant_t_kernel, zeros past the group's
// end). Per valid row: da, du quantised along I (32-unit blocks = 32-lane groups, amax by
// shuffles), staged in LDS and written as 16-byte chunks into dq [n][2I] and the scale bytes into
// dsc [n][2I / 32] (du after da); per unit: the 32 values of h, da, du down the
// slots quantised into hq / daq (rows c and I + c of [2I][ldo]) with their scales; per row and
// unit tile: part[r][ct] = sum over the tile's units of h dh' (wavefront butterflies, then the four
// wavefronts in order).
__global__ __launch_bounds__(256) void mx_swiglu_bwd_t_kernel(const float* __restrict__ a, const float* __restrict__ u,
                                                              const float* __restrict__ dhp, const float* __restrict__ g,
                                                              int I, const int32_t* __restrict__ offs,
                                                              const int32_t* __restrict__ poff, int G,
                                                              uint8_t* __restrict__ dq, uint8_t* __restrict__ dsc,
                                                              uint8_t* __restrict__ hq, uint8_t* __restrict__ hsc,
                                                              uint8_t* __restrict__ daq, uint8_t* __restrict__ dasc,
                                                              int64_t ldo, float* __restrict__ part, int ntn, int nsb,
                                                              int ntiles) {
  __shared__ float wsum[4][32];
  __shared__ __attribute__((aligned(16))) uint8_t rowq[32][512];   // row-quantised da | du codes of the tile
  __shared__ uint8_t rows_sc[32][16];                               // and their scale bytes
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int sb, ct;
  if (!xcd_tile(nsb, ntiles, sb, ct)) return;
  const int p0 = sb * 32;
  if (p0 >= poff[G]) return;
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (poff[mid] <= p0) lo = mid; else hi = mid - 1;
  }
  const int64_t rbase = (int64_t)offs[lo] + (p0 - poff[lo]);
  const int64_t rend = offs[lo + 1];
  const int c = ct * 256 + tid;
  const bool cv = c < I;                 // whole 32-lane groups agree (I % 32 == 0)
  const int nb = I / 32;
  float hv[32], dav[32], duv[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int64_t r = rbase + i;
    const bool rv = r < rend;            // uniform across the workgroup
    float h = 0.f, da = 0.f, du = 0.f, pr = 0.f;
    if (rv && cv) {
      const float x = a[r * I + c], uu = u[r * I + c], p = dhp[r * I + c];
      const float sg = sigmoid_f(x), sa = x * sg;
      h = sa * uu;
      pr = h * p;
      const float dh = g[r] * p;
      da = dh * uu * sg * (1.f + x * (1.f - sg));
      du = dh * sa;
    }
    hv[i] = h;
    dav[i] = da;
    duv[i] = du;
    if (rv) {
      // row quantisation along I: the 32 lanes of this lane group hold one block of da and of du
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const float v = half ? du : da;
        float amax = fabsf(v);
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
        uint32_t code = 0, sbyte = 127;
        if (amax > 0.f) {
          const int se = mx_shared_exp(amax);
          sbyte = (uint32_t)(se + 127);
          code = e4m3_code(v * __uint_as_float((uint32_t)(127 - se) << 23));
        }
        rowq[i][half * 256 + tid] = (uint8_t)code;
        if ((lane & 31) == 0) rows_sc[i][half * 8 + tid / 32] = (uint8_t)sbyte;
      }
      float s = pr;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
      if (lane == 0) wsum[wave][i] = s;
    }
  }
  if (cv) {
    uint32_t pk[8];
    u32x4* d;
    hsc[(int64_t)c * (ldo / 32) + p0 / 32] = (uint8_t)mx_block(hv, pk);
    d = reinterpret_cast<u32x4*>(hq + (int64_t)c * ldo + p0);
    d[0] = u32x4{pk[0], pk[1], pk[2], pk[3]};
    d[1] = u32x4{pk[4], pk[5], pk[6], pk[7]};
    dasc[(int64_t)c * (ldo / 32) + p0 / 32] = (uint8_t)mx_block(dav, pk);
    d = reinterpret_cast<u32x4*>(daq + (int64_t)c * ldo + p0);
    d[0] = u32x4{pk[0], pk[1], pk[2], pk[3]};
    d[1] = u32x4{pk[4], pk[5], pk[6], pk[7]};
    dasc[(int64_t)(I + c) * (ldo / 32) + p0 / 32] = (uint8_t)mx_block(duv, pk);
    d = reinterpret_cast<u32x4*>(daq + (int64_t)(I + c) * ldo + p0);
    d[0] = u32x4{pk[0], pk[1], pk[2], pk[3]};
    d[1] = u32x4{pk[4], pk[5], pk[6], pk[7]};
  }
  __syncthreads();
  if (tid < 32 && rbase + tid < rend)
    part[(rbase + tid) * ntn + ct] = ((wsum[0][tid] + wsum[1][tid]) + wsum[2][tid]) + wsum[3][tid];
  // row-quantised codes: 16-byte chunks of the valid rows (32 rows x 2 halves x 16 chunks)
  const int cw = min(256, I - ct * 256);   // units of this tile (a multiple of 32)
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int qd = tid + 256 * k, i = qd >> 5, half = (qd >> 4) & 1, ch = qd & 15;
    const int64_t r = rbase + i;
    if (r < rend && ch * 16 < cw)
      *reinterpret_cast<u32x4*>(dq + r * 2 * I + half * I + ct * 256 + ch * 16) =
          *reinterpret_cast<const u32x4*>(&rowq[i][half * 256 + ch * 16]);
  }
  if (tid < 64) {
    const int i = tid >> 1, half = tid & 1;
    const int64_t r = rbase + i;
    if (r < rend)
      for (int b = 0; b < cw / 32; ++b) dsc[r * 2 * nb + half * nb + ct * 8 + b] = rows_sc[i][half * 8 + b];
  }
}

int launch_mx_swiglu_bwd_t(const float* a, const float* u, const float* dhp, const float* g, int I, const int32_t* offs,
                           const int32_t* poff, int G, int64_t max_padded, uint8_t* dq, uint8_t* dsc, uint8_t* hq,
                           uint8_t* hsc, uint8_t* daq, uint8_t* dasc, int64_t ldo, float* part, hipStream_t s) {
  if (max_padded <= 0) return MOE_OK;
  if (I % 32 || max_padded % 32 || ldo % 128) return MOE_ERR_UNSUPPORTED;
  const int ntn = (I + 255) / 256, nsb = (int)(max_padded / 32), ntiles = nsb * ntn;
  hipLaunchKernelGGL(mx_swiglu_bwd_t_kernel, dim3(xcd_grid(ntiles)), dim3(256), 0, s, a, u, dhp, g, I, offs, poff, G, dq,
                     dsc, hq, hsc, daq, dasc, ldo, part, ntn, nsb, ntiles);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
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

int launch_mx_quant_t(const uint16_t* src, const float* rscale, int64_t lds, int W, const int32_t* offs,
                      const int32_t* poff, int G, int64_t max_padded, uint8_t* q, uint8_t* sc, int64_t ldo, uint8_t* rq,
                      uint8_t* rsc, hipStream_t s, const int32_t* rmap, int rdiv) {
  if (max_padded <= 0 || W <= 0) return MOE_OK;
  if (max_padded % 128 || ldo % 128 || W % 32 || lds % 8) return MOE_ERR_UNSUPPORTED;
  const int nsb = (int)(max_padded / 128), ntiles = nsb * ((W + 63) / 64);
  hipLaunchKernelGGL(mx_quant_t_kernel, dim3(xcd_grid(ntiles)), dim3(256), 0, s, src, rscale, lds, W, offs, poff, G, q,
                     sc, ldo, rq, rsc, nsb, ntiles, rmap, rdiv);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
