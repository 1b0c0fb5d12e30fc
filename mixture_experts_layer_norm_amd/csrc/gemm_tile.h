// One workgroup tile of the grouped GEMMs (shared by the standalone kernels and the persistent
// pipeline). See gemm.hip for the tiling.
#pragma once
#include "common.h"

namespace moe {

namespace gemm_detail {
constexpr int BM = kGemmBM;   // 256 rows per m-tile
constexpr int BK = 64;
constexpr int PITCH = BK + 8; // bf16 per LDS row (16 B of padding)
}  // namespace gemm_detail

// LDS of one tile: two buffers of 256 A rows + 256 B rows, PITCH bf16 each
constexpr int kGemmSmemElems = 2 * (2 * kGemmBM) * (64 + 8);

struct TileCoord {
  int grp, r0, rows, nt;
};

using namespace gemm_detail;

// Find the (group, first row, valid rows) of m-tile mt; false when mt is past the last tile.
__device__ __forceinline__ bool locate_tile(const Grouped& g, int mt, TileCoord& tc) {
  if (g.row_off) {
    const int total = g.tile_off[g.groups];
    if (mt >= total) return false;
    int lo = 0, hi = g.groups - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (g.tile_off[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    tc.grp = lo;
    tc.r0 = g.row_off[lo] + (mt - g.tile_off[lo]) * BM;
    tc.rows = min(BM, g.row_off[lo + 1] - tc.r0);
  } else {
    tc.grp = 0;
    tc.r0 = mt * BM;
    if (tc.r0 >= g.M) return false;
    tc.rows = min(BM, g.M - tc.r0);
  }
  return true;
}

// Computes one workgroup tile: rows tc.r0 .. tc.r0 + tc.rows - 1 of group tc.grp, n-tile tc.nt,
// K steps [k0, k0 + 64 nk) (times two with a.two_pass). smem holds 2 x (256 + 256) x 72 bf16.
template <int EPI, bool KG, int WN>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, const TileCoord& tc, int k0, int nk, int ntn,
                                          uint16_t* smem) {
  constexpr int WAVES_N = 4, WM = 128, BN = WAVES_N * WN;
  constexpr int NT = 512;
  constexpr int MI = WM / 32, NJ = WN / 32;
  constexpr int A_T = BM * PITCH, B_T = BN * PITCH;
  constexpr int RPP = NT / 8;                       // rows staged per pass (8 chunks of 16 B per row)
  constexpr int AL = BM / RPP, BL = BN / RPP;       // 16-byte chunks per thread per K step
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int lrow = tid >> 3, lchunk = tid & 7;

  // element offsets of the rows this thread stages (A rows lrow + RPP i, B rows likewise)
  const uint16_t* abase0 = (const uint16_t*)a.A + k0 + lchunk * 8;
  uint32_t aoff[AL];
#pragma unroll
  for (int i = 0; i < AL; ++i) {
    const int rr = lrow + RPP * i;
    const int r = tc.r0 + min(rr, tc.rows - 1);
    const int64_t src = (!KG && a.a_gather) ? (int64_t)(a.a_gather[r] / a.a_div) : (int64_t)r;
    aoff[i] = (uint32_t)(src * a.lda);
  }
  const uint16_t* bbase0[2];
  bbase0[0] = (const uint16_t*)a.B + (KG ? 0 : (int64_t)tc.grp * a.b_group_stride) + k0 + lchunk * 8;
  bbase0[1] = (EPI == EPI_SWIGLU || EPI == EPI_SAVE_AU)
                  ? (const uint16_t*)a.B2 + (int64_t)tc.grp * a.b_group_stride + k0 + lchunk * 8
                  : bbase0[0];
  // K step kt < nk1 reads the first pass, kt >= nk1 the second (operands shifted by the split offsets)
  const int nk1 = nk;
  if (a.two_pass) nk *= 2;
  uint32_t boff[BL];
  bool bup[BL];
#pragma unroll
  for (int i = 0; i < BL; ++i) {
    const int rr = lrow + RPP * i;
    int64_t wrow;
    if (EPI == EPI_SWIGLU || EPI == EPI_SAVE_AU) {
      // per wave column block: NJ/2 blocks of gate rows, then the matching NJ/2 blocks of up rows
      const int half = rr / WN, q = (rr % WN) / 32;
      bup[i] = q >= NJ / 2;
      wrow = (int64_t)tc.nt * (BN / 2) + half * (WN / 2) + (bup[i] ? q - NJ / 2 : q) * 32 + (rr & 31);
    } else {
      bup[i] = false;
      wrow = (int64_t)tc.nt * BN + rr;
    }
    wrow = wrow < a.N ? wrow : a.N - 1;          // partial last n-tile: clamp, results unused
    boff[i] = (uint32_t)(wrow * a.ldb);
  }

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // row blocks of this wave that hold at least one valid row
  const int wrows = tc.rows - wm * WM;
  u32x4 ra[AL], rb[BL];
  const int st_off = lrow * PITCH + lchunk * 8;   // this thread's LDS store offset (+ RPP i rows)
  if (nk > 0) {
#pragma unroll
    for (int i = 0; i < AL; ++i) ra[i] = *reinterpret_cast<const u32x4*>(abase0 + aoff[i]);
#pragma unroll
    for (int i = 0; i < BL; ++i) rb[i] = *reinterpret_cast<const u32x4*>(bbase0[bup[i]] + boff[i]);
#pragma unroll
    for (int i = 0; i < AL; ++i) *reinterpret_cast<u32x4*>(smem + st_off + RPP * i * PITCH) = ra[i];
#pragma unroll
    for (int i = 0; i < BL; ++i) *reinterpret_cast<u32x4*>(smem + A_T + st_off + RPP * i * PITCH) = rb[i];
  }
  __syncthreads();
  const int a_rd = (wm * WM + (lane & 31)) * PITCH + (lane >> 5) * 8;
  const int b_rd = (wn * WN + (lane & 31)) * PITCH + (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) {
      const bool second = kt + 1 >= nk1;
      const int ko = (second ? kt + 1 - nk1 : kt + 1) * BK;
      const uint16_t* ab = second ? abase0 + a.a_seg_shift : abase0;
      const int64_t bsh = second ? a.b_seg_shift : 0;
#pragma unroll
      for (int i = 0; i < AL; ++i) ra[i] = *reinterpret_cast<const u32x4*>(ab + aoff[i] + ko);
#pragma unroll
      for (int i = 0; i < BL; ++i) rb[i] = *reinterpret_cast<const u32x4*>(bbase0[bup[i]] + bsh + boff[i] + ko);
    }
    const uint16_t* As = smem + buf * (A_T + B_T);
    const uint16_t* Bs = As + A_T;
    bf16x8 af[2][MI], bfr[2][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i) af[0][i] = *reinterpret_cast<const bf16x8*>(As + a_rd + i * 32 * PITCH);
#pragma unroll
    for (int j = 0; j < NJ; ++j) bfr[0][j] = *reinterpret_cast<const bf16x8*>(Bs + b_rd + j * 32 * PITCH);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < BK / 16) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
          af[cur ^ 1][i] = *reinterpret_cast<const bf16x8*>(As + a_rd + i * 32 * PITCH + (kk + 1) * 16);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          bfr[cur ^ 1][j] = *reinterpret_cast<const bf16x8*>(Bs + b_rd + j * 32 * PITCH + (kk + 1) * 16);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        if (i * 32 < wrows) {
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][i], bfr[cur][j], acc[i][j], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < nk) {
      uint16_t* An = smem + (buf ^ 1) * (A_T + B_T);
#pragma unroll
      for (int i = 0; i < AL; ++i) *reinterpret_cast<u32x4*>(An + st_off + RPP * i * PITCH) = ra[i];
#pragma unroll
      for (int i = 0; i < BL; ++i) *reinterpret_cast<u32x4*>(An + A_T + st_off + RPP * i * PITCH) = rb[i];
    }
    __syncthreads();
  }

  // epilogue. Accumulator slot r of lane l: row (r/4)*8 + (l/32)*4 + r%4, column l%32.
  const int ccol = lane & 31;
  float* part = reinterpret_cast<float*>(smem);   // EPI_DGRAD: [BM][WAVES_N] partials (LDS is free now)
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int lr = wm * WM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      const bool ok = lr < tc.rows;
      const int row = tc.r0 + lr;
      if (EPI == EPI_SWIGLU || EPI == EPI_SAVE_AU) {
        if (!ok) continue;
#pragma unroll
        for (int j = 0; j < NJ / 2; ++j) {
          const int64_t col = (int64_t)tc.nt * (BN / 2) + wn * (WN / 2) + j * 32 + ccol;
          if (col >= a.N) continue;
          const float gt = acc[i][j][r], up = acc[i][j + NJ / 2][r];
          if (EPI == EPI_SWIGLU) {
            const float h = silu_f(gt) * up;
            if (a.c_f32) ((float*)a.C)[(int64_t)row * a.ldc + col] = h;
            else ((uint16_t*)a.C)[(int64_t)row * a.ldc + col] = f2bf(h);
          } else {
            ((float*)a.C)[(int64_t)row * a.ldc + col] = gt;
            ((float*)a.C2)[(int64_t)row * a.ldc + col] = up;
          }
        }
      } else if (EPI == EPI_DGRAD) {
        float p = 0.f;
        if (ok) {
          const float gj = a.row_scale ? a.row_scale[row] : 1.f;
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const int64_t col = (int64_t)tc.nt * BN + wn * WN + j * 32 + ccol;
            if (col >= a.N) continue;
            const float av = a.ea[(int64_t)row * a.lde + col];
            const float uv = a.eu[(int64_t)row * a.lde + col];
            const float sg = sigmoid_f(av);
            const float sl = av * sg;
            const float dhp = acc[i][j][r];
            p = fmaf(sl * uv, dhp, p);
            const float dh = gj * dhp;
            const float da = dh * uv * sg * (1.f + av * (1.f - sg));
            const float du = dh * sl;
            const uint16_t dah = f2bf(da), duh = f2bf(du);
            uint16_t* c1 = (uint16_t*)a.C + (int64_t)row * a.ldc + col;
            uint16_t* c2 = (uint16_t*)a.C2 + (int64_t)row * a.ldc + col;
            *c1 = dah;
            *c2 = duh;
            if (a.lo_off) {
              c1[a.lo_off] = f2bf(da - bf2f(dah));
              c2[a.lo_off] = f2bf(du - bf2f(duh));
            }
          }
        }
        // sum over the 32 columns this row has in each block (lanes with the same lane / 32)
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) p += __shfl_xor(p, off, 64);
        if (ccol == 0) part[lr * WAVES_N + wn] = p;
      } else {
        if (!ok) continue;
        if (KG) {
          const bool hi = a.C2 && row >= a.m_split;
          float* cb = (float*)(hi ? a.C2 : a.C) + (int64_t)tc.grp * a.c_group_stride;
          const int64_t orow = hi ? row - a.m_split : row;
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const int64_t col = (int64_t)tc.nt * BN + wn * WN + j * 32 + ccol;
            if (col < a.N) cb[orow * a.ldc + col] = acc[i][j][r];
          }
        } else {
          const int64_t orow = a.c_scatter ? (int64_t)a.c_scatter[row] : (int64_t)row;
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const int64_t col = (int64_t)tc.nt * BN + wn * WN + j * 32 + ccol;
            if (col >= a.N) continue;
            if (a.c_f32) ((float*)a.C)[orow * a.ldc + col] = acc[i][j][r];
            else ((uint16_t*)a.C)[orow * a.ldc + col] = f2bf(acc[i][j][r]);
          }
        }
      }
    }
  }
  if (EPI == EPI_DGRAD) {
    __syncthreads();
    if (tid < tc.rows) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES_N; ++w) s += part[tid * WAVES_N + w];
      a.row_partial[(int64_t)(tc.r0 + tid) * ntn + tc.nt] = s;
    }
  }
}


}  // namespace moe
