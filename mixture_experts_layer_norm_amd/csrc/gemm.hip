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
// Tiling (bf16): 512 threads = 8 wavefronts in a 2 x 4 grid, workgroup tile 256 rows x 256 weight
// rows, K slices 64 wide staged into LDS by LDS-direct loads (two 64 KB stages, the next slice
// loading while the current one multiplies; 16-byte chunks XOR-swizzled within each row, see
// gemm_tile.h). Each wavefront owns a 128 x 64 block of the product as 4 x 2
// v_mfma_f32_32x32x16_bf16 accumulators (fp32), reading its fragments straight from the
// swizzled LDS rows. For SwiGLU the weight tile interleaves 32 gate rows and the 32 up rows of
// the same h columns, so a lane holds the gate and up value of the same (row, column) in the same
// accumulator slot and the epilogue needs no data exchange. 256-row m-tiles read each expert's
// weights once for up to 256 routed rows; row blocks past an expert's last row skip their MFMAs.
//
// Workgroup -> tile mapping: tiles are numbered group by group (inside a group in blocks of 4
// m-tiles, n-tile major inside a block, see decode_grouped_tile) and dealt out so that each XCD
// (workgroups are placed round-robin over the 8 XCDs) gets a contiguous range, which keeps an
// expert's activation rows and weight tiles in that XCD's L2. The split is over the tiles that
// exist (read on the device), not over the launched upper bound, so that every XCD gets an
// equal share even when the routing leaves most of the bound empty.
#include "gemm_tile.h"

namespace moe {

// Workgroup tile 256 rows x BN weight rows, 8 wavefronts in a 2 (rows) x 4 (columns) grid; each
// wavefront owns a 128 x WN block as (128/32) x (WN/32) v_mfma_f32_32x32x16_bf16 accumulators.
// Row blocks of 32 that lie past the group's last row skip their MFMAs (a wave-uniform branch),
// so a sparsely filled tile costs only the streaming of its weight tile.
template <int EPI, bool KG, int WN, int WAVES_N, int BKE, bool BT = false>
__global__ __launch_bounds__(128 * WAVES_N, 1) void gemm_bf16_kernel(GemmArgs a, Grouped g, int ntn, int mtn) {
  constexpr int BK = SliceCfg<BKE>::BK;
  // EPI_DGRAD keeps its [BM][WAVES_N] fp32 row partials past the 128 KB of operand staging
  __shared__ __attribute__((aligned(16))) uint16_t smem[kGemmSmemElems + (EPI == EPI_DGRAD ? 2 * BM * WAVES_N : 0)];
  // The grid is an upper bound (grouped tile counts are known only on the device); the valid
  // tiles are split evenly over the 8 XCDs, each taking a contiguous range of them.
  // K-grouped tiles differ in length by their group's K extent: they are dealt in launch order
  // (workgroups start in blockIdx order as CUs free up), groups longest first, so that the
  // in-order dispatch balances the CUs like a longest-first schedule.
  const int valid = (KG ? g.groups * mtn : (g.row_off ? g.tile_off[g.groups] : mtn)) * ntn;
  const int per_xcd = (valid + 7) >> 3;
  const int bid = blockIdx.x;
  if (!KG && (bid >> 3) >= per_xcd) return;
  const int logical = KG ? bid : (bid & 7) * per_xcd + (bid >> 3);
  if (logical >= valid) return;
  TileCoord tc;
  int k0 = 0, nk;
  if (KG) {
    const int per = mtn * ntn;
    const int rank = logical / per;
    if (rank >= g.groups) return;
    tc.grp = a.k_order ? a.k_order[rank] : rank;
    const int rem = logical - rank * per;
    tc.nt = rem % ntn;
    tc.r0 = (rem / ntn) * BM;
    tc.rows = min(BM, a.M - tc.r0);
    k0 = a.k_off[tc.grp];
    nk = (a.k_off[tc.grp + 1] - k0) / BK;
  } else {
    if (!decode_grouped_tile(g, logical, ntn, mtn, tc)) return;
    nk = a.K / BK;
  }

  gemm_tile<EPI, KG, WN, WAVES_N, BKE, BT>(a, tc, k0, nk, ntn, smem);
}

// Persistent form of the grouped GEMMs (every epilogue; grouped, dense and K-grouped tiles): one
// workgroup per CU loops over tiles (persistent_tiles) instead of one workgroup per tile. The
// tiles and their order are those of gemm_bf16_kernel: for grouped and dense tiles one ticket
// counter per XCD range, a workgroup starting with its own XCD's range (workgroups are placed
// round-robin over the 8 XCDs); for K-grouped tiles one counter over the dealing order (longest
// groups first). Each tile is computed by exactly one workgroup with the same summation order as
// the per-tile launch, so the results are bitwise those of gemm_bf16_kernel whatever the grid and
// the timing. budget, budget_ind: the workgroup budget word (nullable), see persistent_tiles.
template <int EPI, bool KG, int WN, int WAVES_N, int BKE, bool BT = false>
__global__ __launch_bounds__(128 * WAVES_N, 1) void gemm_bf16_persistent_kernel(GemmArgs a, Grouped g, int ntn,
                                                                                  int mtn, int32_t* tickets,
                                                                                  const int32_t* budget,
                                                                                  int budget_ind) {
  static_assert(!(KG && EPI != EPI_STORE), "K-grouped tiles store fp32 weight gradients");
  constexpr int BK = SliceCfg<BKE>::BK;
  constexpr int kExtra = EPI == EPI_DGRAD ? 2 * BM * WAVES_N : 0;   // EPI_DGRAD's row partials
  __shared__ __attribute__((aligned(16))) uint16_t smem[kGemmSmemElems + kExtra + 8];
  // K-grouped: every (group, m-tile, n-tile) in launch order (longest groups first), one counter;
  // grouped / dense: the XCD ranges of gemm_bf16_kernel, one counter each
  const int valid = KG ? g.groups * mtn * ntn : (g.row_off ? g.tile_off[g.groups] : mtn) * ntn;
  // the next ticket fetched during the epilogue: the forward's GEMMs (see persistent_tiles)
  constexpr bool kEarly = !KG && !BT && (EPI == EPI_SWIGLU || EPI == EPI_STORE);
  persistent_tiles<kEarly>(valid, KG ? valid : (valid + 7) >> 3, KG ? 1 : 8, KG ? 0 : (int)(blockIdx.x & 7), tickets,
                           budget, budget_ind, reinterpret_cast<int*>(smem + kGemmSmemElems + kExtra),
                           [&](int cur, auto& ti, auto& hook) {
    // A per-tile copy of the arguments the tile reads, opaque like the thread index, so that
    // nothing the tile derives from them is hoisted out of the loop and held across the K loop.
    GemmArgs la = a;
    asm volatile("" : "+s"(la.A), "+s"(la.B), "+s"(la.B2), "+s"(la.C), "+s"(la.C2), "+s"(la.a_gather),
                 "+s"(la.c_scatter));
    asm volatile("" : "+s"(la.lda), "+s"(la.ldb), "+s"(la.ldc), "+s"(la.b_group_stride), "+s"(la.a_seg_shift),
                 "+s"(la.b_seg_shift));
    asm volatile("" : "+s"(la.N), "+s"(la.K), "+s"(la.a_div), "+s"(la.c_f32), "+s"(la.two_pass), "+s"(la.b_split));
    TileCoord tc;
    int k0 = 0, nk = la.K / BK;
    bool ok = true;
    if (KG) {
      // as gemm_bf16_kernel: tile `cur` of the groups in dealing order
      const int per = mtn * ntn;
      const int rank = cur / per;
      tc.grp = la.k_order ? la.k_order[rank] : rank;
      const int rem = cur - rank * per;
      tc.nt = rem % ntn;
      tc.r0 = (rem / ntn) * BM;
      tc.rows = min(BM, la.M - tc.r0);
      k0 = la.k_off[tc.grp];
      nk = (la.k_off[tc.grp + 1] - k0) / BK;
    } else {
      ok = decode_grouped_tile(g, cur, ntn, mtn, tc);
    }
    if (ok) gemm_tile<EPI, KG, WN, WAVES_N, BKE, BT>(la, tc, k0, nk, ntn, smem, ti(), hook);
  });
}

// Zeroes the 8 ticket counters of a persistent launch (a kernel, not a memset, so that the
// launch sequence can be captured into a graph).
__global__ void zero_tickets_kernel(int32_t* t) {
  if (threadIdx.x < 8) t[threadIdx.x] = 0;
}

int launch_zero_tickets(int32_t* tickets, hipStream_t s) {
  hipLaunchKernelGGL(zero_tickets_kernel, dim3(1), dim3(64), 0, s, tickets);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

static int64_t grid_blocks(int64_t mtiles, int ntn) {
  int64_t n = mtiles * ntn;
  return (n + 7) / 8 * 8;
}

// Every epilogue uses 8 wavefronts with 128 x 64 wavefront tiles: a workgroup covers 256 weight
// rows (the SwiGLU tiles: 128 h columns, each as a gate row and an up row).
constexpr int kWN = 64;
constexpr int kTileCols = 4 * kWN;

int gemm_tile_cols(Epi epi) { return (epi == EPI_SWIGLU || epi == EPI_SAVE_AU) ? kTileCols / 2 : kTileCols; }

// Grid of the persistent form for a launch of at most nb tiles, or nw = 0 for the per-tile form:
// one workgroup per CU (a multiple of 8, so that every XCD holds the same number), at most one
// per possible tile, taken when forced or when the launch has at least kPersistMinTilesPerWg
// tiles per workgroup. Measured on the DSV3 forward (T=8192, 256 experts: at most 32 and 56
// tiles per workgroup) the persistent form is 5% faster than the per-tile launch, and on one
// expert-parallel rank's share (14 and 25) faster too; at the mid shape (6 and 8) 3% slower, the
// counters' zeroing launch and each tile's ticket costing more than the workgroup launches they
// replace.
int persistent_grid(int64_t nb, const Persist* pc, int64_t& nw) {
  nw = 0;
  if (!pc || !pc->tickets) return MOE_OK;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MOE_ERR_HIP;
  int64_t w = (int64_t)(ncu > 8 ? ncu : 8) / 8 * 8;
  if (w > nb) w = nb;
  if (pc->force || nb >= (int64_t)kPersistMinTilesPerWg * w) nw = w;
  return MOE_OK;
}

int launch_gemm_bf16(const GemmArgs& a, const Grouped& g, Epi epi, hipStream_t s, const Persist* pc) {
  const int tcols = gemm_tile_cols(epi);
  const int ntn = (a.N + tcols - 1) / tcols;
  const int64_t mt = g.row_off ? g.max_mtiles : (g.M + BM - 1) / BM;
  const int64_t nb = grid_blocks(mt, ntn);
  if (nb == 0) return MOE_OK;
  if (nb > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  const int mtn = g.row_off ? 0 : (int)mt;   // dense mode: the exact m-tile count
  if (a.b_kmajor && ((epi != EPI_STORE && epi != EPI_DGRAD) || a.N % 8 || a.ldb % 8 || a.b_seg_shift ||
                     a.K % 64 || (a.b_split && (a.b_split % 64 || !a.B2))))
    return MOE_ERR_UNSUPPORTED;
  int64_t nw = 0;
  int st;
  if ((st = persistent_grid(nb, pc, nw))) return st;
  if (nw > 0) {
    if ((st = launch_zero_tickets(pc->tickets, s))) return st;
    const dim3 pg((unsigned)nw), pb(512);
    if (a.b_kmajor) {
      if (epi == EPI_STORE)
        hipLaunchKernelGGL((gemm_bf16_persistent_kernel<EPI_STORE, false, kWN, 4, 64, true>), pg, pb, 0, s, a, g, ntn, mtn, pc->tickets, pc->budget, (int)pc->budget_indirect);
      else
        hipLaunchKernelGGL((gemm_bf16_persistent_kernel<EPI_DGRAD, false, kWN, 4, 64, true>), pg, pb, 0, s, a, g, ntn, mtn, pc->tickets, pc->budget, (int)pc->budget_indirect);
    } else {
      switch (epi) {
        case EPI_SWIGLU: hipLaunchKernelGGL((gemm_bf16_persistent_kernel<EPI_SWIGLU, false, kWN, 4, 64>), pg, pb, 0, s, a, g, ntn, mtn, pc->tickets, pc->budget, (int)pc->budget_indirect); break;
        case EPI_STORE: hipLaunchKernelGGL((gemm_bf16_persistent_kernel<EPI_STORE, false, kWN, 4, 64>), pg, pb, 0, s, a, g, ntn, mtn, pc->tickets, pc->budget, (int)pc->budget_indirect); break;
        case EPI_SAVE_AU: hipLaunchKernelGGL((gemm_bf16_persistent_kernel<EPI_SAVE_AU, false, kWN, 4, 64>), pg, pb, 0, s, a, g, ntn, mtn, pc->tickets, pc->budget, (int)pc->budget_indirect); break;
        case EPI_DGRAD: hipLaunchKernelGGL((gemm_bf16_persistent_kernel<EPI_DGRAD, false, kWN, 4, 64>), pg, pb, 0, s, a, g, ntn, mtn, pc->tickets, pc->budget, (int)pc->budget_indirect); break;
      }
    }
    MOE_LAUNCH_CHECK();
    return MOE_OK;
  }
  dim3 grid((unsigned)nb), block(512);
  if (a.b_kmajor) {
    if (epi == EPI_STORE)
      hipLaunchKernelGGL((gemm_bf16_kernel<EPI_STORE, false, kWN, 4, 64, true>), grid, block, 0, s, a, g, ntn, mtn);
    else
      hipLaunchKernelGGL((gemm_bf16_kernel<EPI_DGRAD, false, kWN, 4, 64, true>), grid, block, 0, s, a, g, ntn, mtn);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
  }
  switch (epi) {
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_bf16_kernel<EPI_SWIGLU, false, kWN, 4, 64>), grid, block, 0, s, a, g, ntn, mtn); break;
    case EPI_STORE: hipLaunchKernelGGL((gemm_bf16_kernel<EPI_STORE, false, kWN, 4, 64>), grid, block, 0, s, a, g, ntn, mtn); break;
    case EPI_SAVE_AU: hipLaunchKernelGGL((gemm_bf16_kernel<EPI_SAVE_AU, false, kWN, 4, 64>), grid, block, 0, s, a, g, ntn, mtn); break;
    case EPI_DGRAD: hipLaunchKernelGGL((gemm_bf16_kernel<EPI_DGRAD, false, kWN, 4, 64>), grid, block, 0, s, a, g, ntn, mtn); break;
  }
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

// Weight-gradient GEMM: for each group, C_g[M][N] = sum over k in the group's range of
// A[m][k] * B[n][k], written once (fp32), with no split-K and no atomics.
int launch_gemm_bf16_kgroup(const GemmArgs& a, int groups, hipStream_t s, const Persist* pc) {
  const int ntn = (a.N + kTileCols - 1) / kTileCols, mtn = (a.M + BM - 1) / BM;
  Grouped g;
  g.groups = groups;
  const int64_t nb = grid_blocks((int64_t)groups * mtn, ntn);
  if (nb == 0) return MOE_OK;
  int64_t nw = 0;
  int st;
  if ((st = persistent_grid(nb, pc, nw))) return st;
  if (nw > 0) {
    if ((st = launch_zero_tickets(pc->tickets, s))) return st;
    hipLaunchKernelGGL((gemm_bf16_persistent_kernel<EPI_STORE, true, kWN, 4, 64>), dim3((unsigned)nw), dim3(512), 0, s,
                       a, g, ntn, mtn, pc->tickets, pc->budget, (int)pc->budget_indirect);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
  }
  hipLaunchKernelGGL((gemm_bf16_kernel<EPI_STORE, true, kWN, 4, 64>), dim3((unsigned)nb), dim3(512), 0, s, a, g, ntn, mtn);
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
  __shared__ float As[FBK][BM + 4];   // BM = 256 rows; thread (tx, ty) owns rows ty*16 .. ty*16+15
  __shared__ float Bs[FBK][64 + 4];
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int logical = (bid & 7) * (nb >> 3) + (bid >> 3);
  TileCoord tc;
  tc.nt = logical % ntn;
  if (!locate_tile(g, logical / ntn, tc)) return;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const float* A = (const float*)a.A;
  float acc[16][4];
#pragma unroll
  for (int i = 0; i < 16; ++i)
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
      float av[16], bv[4];
#pragma unroll
      for (int i = 0; i < 16; ++i) av[i] = As[kk][ty * 16 + i];
      if (EPI == EPI_SWIGLU) {
        bv[0] = Bs[kk][tx * 2]; bv[1] = Bs[kk][tx * 2 + 1];
        bv[2] = Bs[kk][32 + tx * 2]; bv[3] = Bs[kk][32 + tx * 2 + 1];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  (void)hcols;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int lr = ty * 16 + i;
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
