// Grouped GEMMs of the expert FFN on gfx950 MFMA.
//
// Per expert (group) g with rows R_g of the expert-contiguous slot buffer:
//   up/gate:  h = SiLU(X W_gate^T) (*) (X W_up^T)          (EPI_SWIGLU, output [rows][I])
//   down:     y = h W_down^T, row j stored at c_scatter[j]  (EPI_STORE,  output [rows][D])
// which is the expert FFN E_i(x) = W_down(SiLU(W_gate x) (*) W_up x) of the Cursor blog
// "Mixture-of-Kittens: our open-source MoE megakernel for NVL72s", section "Overlapping
// computation and communication in MoE". Both operands are K-contiguous (activations [rows][K],
// weights [N][K]), the layout MFMA fragments want.
//
// Tiling (bf16): 256 threads = 4 wavefronts in a 2x2 grid, workgroup tile 128 rows x 128
// weight rows, K step 64, LDS double-buffered (2 x 36 KB, rows padded by 16 B so that the
// fragment reads of 32 rows hit distinct bank groups). Each wavefront owns a 64 x 64 block of
// the product as 2 x 2 v_mfma_f32_32x32x16_bf16 accumulators (fp32). For SwiGLU the weight tile
// interleaves 32 gate rows and the 32 up rows of the same h columns, so a lane holds the gate
// and up value of the same (row, column) in the same accumulator slot and the epilogue needs no
// data exchange.
//
// Workgroup -> tile mapping: tiles are numbered (m-tile major, n-tile minor) and dealt out so
// that each XCD (workgroups are placed round-robin over the 8 XCDs) gets a contiguous range,
// which keeps an expert's activation rows and weight tiles in that XCD's L2.
#include "common.h"

namespace moe {

namespace {
constexpr int BM = kGemmBM;   // 128
constexpr int BN = 128;       // weight rows per tile
constexpr int BK = 64;
constexpr int PITCH = BK + 8; // bf16 per LDS row
constexpr int A_TILE = BM * PITCH;
constexpr int B_TILE = BN * PITCH;
}  // namespace

struct TileCoord {
  int grp, r0, rows, nt;
};

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

template <int EPI>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(GemmArgs a, Grouped g, int ntn) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (A_TILE + B_TILE)];
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int logical = (bid & 7) * (nb >> 3) + (bid >> 3);
  TileCoord tc;
  tc.nt = logical % ntn;
  if (!locate_tile(g, logical / ntn, tc)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = tid >> 3, lchunk = tid & 7;

  // global row pointers of the 4 A rows and 4 B rows this thread stages
  const uint16_t* aptr[4];
  const uint16_t* bptr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = lrow + 32 * i;
    int r = tc.r0 + min(rr, tc.rows - 1);
    int64_t src = a.a_gather ? (int64_t)(a.a_gather[r] / a.a_div) : (int64_t)r;
    aptr[i] = (const uint16_t*)a.A + src * a.lda + lchunk * 8;
    const uint16_t* wb;
    int64_t wrow;
    if (EPI == EPI_SWIGLU) {
      const int blk = rr >> 5;                 // 0: gate, 1: up (wn 0), 2: gate, 3: up (wn 1)
      wb = (const uint16_t*)((blk & 1) ? a.B2 : a.B);
      wrow = (int64_t)tc.nt * 64 + (blk >> 1) * 32 + (rr & 31);
    } else {
      wb = (const uint16_t*)a.B;
      wrow = (int64_t)tc.nt * BN + rr;
    }
    bptr[i] = wb + (int64_t)tc.grp * a.b_group_stride + wrow * a.ldb + lchunk * 8;
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 ra[4], rb[4];
  const int nk = a.K / BK;

  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = *reinterpret_cast<const uint4*>(aptr[i] + kt * BK);
      rb[i] = *reinterpret_cast<const uint4*>(bptr[i] + kt * BK);
    }
  };
  auto lstore = [&](int buf) {
    uint16_t* As = smem + buf * (A_TILE + B_TILE);
    uint16_t* Bs = As + A_TILE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint4*>(As + (lrow + 32 * i) * PITCH + lchunk * 8) = ra[i];
      *reinterpret_cast<uint4*>(Bs + (lrow + 32 * i) * PITCH + lchunk * 8) = rb[i];
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint16_t* As = smem + buf * (A_TILE + B_TILE);
    const uint16_t* Bs = As + A_TILE;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int col = kk * 16 + (lane >> 5) * 8;
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const bf16x8*>(As + (wm * 64 + i * 32 + (lane & 31)) * PITCH + col);
        bfr[i] = *reinterpret_cast<const bf16x8*>(Bs + (wn * 64 + i * 32 + (lane & 31)) * PITCH + col);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue. Accumulator slot r of lane l: row (r/4)*8 + (l/32)*4 + r%4, column l%32.
  const int ccol = lane & 31;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int lr = wm * 64 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      if (lr >= tc.rows) continue;
      const int row = tc.r0 + lr;
      if (EPI == EPI_SWIGLU) {
        const float gt = acc[i][0][r], up = acc[i][1][r];
        const float h = silu_f(gt) * up;
        const int64_t col = (int64_t)tc.nt * 64 + wn * 32 + ccol;
        if (a.c_f32) ((float*)a.C)[(int64_t)row * a.ldc + col] = h;
        else ((uint16_t*)a.C)[(int64_t)row * a.ldc + col] = f2bf(h);
      } else {
        const int64_t orow = a.c_scatter ? (int64_t)a.c_scatter[row] : (int64_t)row;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t col = (int64_t)tc.nt * BN + wn * 64 + j * 32 + ccol;
          if (a.c_f32) ((float*)a.C)[orow * a.ldc + col] = acc[i][j][r];
          else ((uint16_t*)a.C)[orow * a.ldc + col] = f2bf(acc[i][j][r]);
        }
      }
    }
  }
}

static int64_t grid_blocks(int64_t mtiles, int ntn) {
  int64_t n = mtiles * ntn;
  return (n + 7) / 8 * 8;
}

int launch_gemm_bf16(const GemmArgs& a, const Grouped& g, Epi epi, hipStream_t s) {
  const int ntn = (epi == EPI_SWIGLU) ? a.N / 64 : a.N / BN;
  const int64_t mt = g.row_off ? g.max_mtiles : (g.M + BM - 1) / BM;
  const int64_t nb = grid_blocks(mt, ntn);
  if (nb == 0) return MOE_OK;
  if (nb > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  if (epi == EPI_SWIGLU)
    hipLaunchKernelGGL(gemm_bf16_kernel<EPI_SWIGLU>, dim3((unsigned)nb), dim3(256), 0, s, a, g, ntn);
  else
    hipLaunchKernelGGL(gemm_bf16_kernel<EPI_STORE>, dim3((unsigned)nb), dim3(256), 0, s, a, g, ntn);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

// ---------------------------------------------------------------------------------------------
// fp32 path (plain FMA, any sizes): 128-row m-tiles, 64 product columns per tile (SwiGLU: 32 h
// columns, gate and up side by side), K step 16, each thread 8 rows x 4 columns.
// ---------------------------------------------------------------------------------------------
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a, Grouped g, int ntn) {
  constexpr int FBK = 16;
  __shared__ float As[FBK][BM + 4];
  __shared__ float Bs[FBK][64 + 4];
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int logical = (bid & 7) * (nb >> 3) + (bid >> 3);
  TileCoord tc;
  tc.nt = logical % ntn;
  if (!locate_tile(g, logical / ntn, tc)) return;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const float* A = (const float*)a.A;
  float acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  const int hcols = (EPI == EPI_SWIGLU) ? 32 : 64;
  for (int k0 = 0; k0 < a.K; k0 += FBK) {
    // stage A: 128 rows x 16 k
    for (int i = tid; i < BM * FBK; i += 256) {
      const int rr = i / FBK, kk = i % FBK;
      float v = 0.f;
      if (rr < tc.rows && k0 + kk < a.K) {
        const int r = tc.r0 + rr;
        const int64_t src = a.a_gather ? (int64_t)(a.a_gather[r] / a.a_div) : (int64_t)r;
        v = A[src * a.lda + k0 + kk];
      }
      As[kk][rr] = v;
    }
    // stage B: 64 product columns x 16 k
    for (int i = tid; i < 64 * FBK; i += 256) {
      const int cc = i / FBK, kk = i % FBK;
      float v = 0.f;
      const float* wb;
      int64_t wrow;
      if (EPI == EPI_SWIGLU) {
        wb = (const float*)(cc < 32 ? a.B : a.B2);
        wrow = (int64_t)tc.nt * 32 + (cc & 31);
      } else {
        wb = (const float*)a.B;
        wrow = (int64_t)tc.nt * 64 + cc;
      }
      if (wrow < a.N && k0 + kk < a.K) v = wb[(int64_t)tc.grp * a.b_group_stride + wrow * a.ldb + k0 + kk];
      Bs[kk][cc] = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      float av[8], bv[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) av[i] = As[kk][ty * 8 + i];
      if (EPI == EPI_SWIGLU) {
        bv[0] = Bs[kk][tx * 2]; bv[1] = Bs[kk][tx * 2 + 1];
        bv[2] = Bs[kk][32 + tx * 2]; bv[3] = Bs[kk][32 + tx * 2 + 1];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  (void)hcols;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int lr = ty * 8 + i;
    if (lr >= tc.rows) continue;
    const int row = tc.r0 + lr;
    if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col = (int64_t)tc.nt * 32 + tx * 2 + j;
        if (col < a.N) ((float*)a.C)[(int64_t)row * a.ldc + col] = silu_f(acc[i][j]) * acc[i][2 + j];
      }
    } else {
      const int64_t orow = a.c_scatter ? (int64_t)a.c_scatter[row] : (int64_t)row;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = (int64_t)tc.nt * 64 + tx * 4 + j;
        if (col < a.N) ((float*)a.C)[orow * a.ldc + col] = acc[i][j];
      }
    }
  }
}

int launch_gemm_f32(const GemmArgs& a, const Grouped& g, Epi epi, hipStream_t s) {
  const int hc = (epi == EPI_SWIGLU) ? 32 : 64;
  const int ntn = (a.N + hc - 1) / hc;
  const int64_t mt = g.row_off ? g.max_mtiles : (g.M + BM - 1) / BM;
  const int64_t nb = grid_blocks(mt, ntn);
  if (nb == 0) return MOE_OK;
  if (epi == EPI_SWIGLU)
    hipLaunchKernelGGL(gemm_f32_kernel<EPI_SWIGLU>, dim3((unsigned)nb), dim3(256), 0, s, a, g, ntn);
  else
    hipLaunchKernelGGL(gemm_f32_kernel<EPI_STORE>, dim3((unsigned)nb), dim3(256), 0, s, a, g, ntn);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
