// MXFP8 grouped GEMMs on gfx950's block-scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// The sparsenotes page "Mixture-of-Kittens: MoE Megakernel for NVL72s" ("The production details")
// runs the routed experts in MXFP8 with activation quantisation fused into dispatch, the grouped
// GEMMs and the gated activation; the shared expert stays BF16. Operands here are OCP MX v1.0:
// E4M3 bytes with one E8M0 scale byte per 32 elements along the contraction dimension.
//
//   up/gate:  h = SiLU(X W_gate^T) (*) (X W_up^T), quantised to MXFP8 along I in the epilogue
//   down:     y = h W_down^T (bf16), row j stored at c_scatter[j]
// With a_gather, A row j (codes and scales) is row a_gather[j] / a_div: the up/gate GEMM reads the
// E4M3 token rows through the schedule instead of per-slot copies.
//
// Tiling matches the BF16 kernel byte for byte: 256 rows x 256 weight rows, 8 wavefronts of
// 128 x 64, and the same LDS staging (gemm_tile.h): a K slice of 128 fp8 values is a 128-byte row,
// copied from HBM straight into LDS (global_load_lds_dwordx4), 2 stages, chunks swizzled by
// (r >> 1) & 7; two scaled MFMAs (K = 64 each) per slice. Operand layout of the scaled 32x32x64
// MFMA (lane l, lane group q = l / 32, row or column l % 32): bytes 0-15 of a lane's 32 hold K
// block 0 of the instruction and bytes 16-31 K block 1 (32 values each); lane group q supplies K
// values [16q, 16q+16) of each block and the E8M0 scale of block q. Scale words (4 bytes = the 4
// blocks of one row and slice) are copied into LDS beside the slice (one 4-byte LDS-direct load
// per wavefront), and each lane shifts its byte into place.
#include "gemm_tile.h"
#include "mx_codec.h"

namespace moe {

// The K loop of an MX tile: 2 LDS stages. In step kt, once slice kt and its scale words have
// landed and the barrier has made every thread's copies visible, slice kt + 1 and its scale words
// are issued and the two scaled MFMAs of slice kt run for this wave's first NACT row blocks. The
// scale words of a slice (one 32-bit word = 4 blocks per tile row, A rows then B rows) are copied
// into LDS too: wavefront w copies the words of 64 tile rows, one 4-byte load per lane.
template <int EPI, int NACT, int NL>
__device__ __forceinline__ void mx_k_loop(const StageSrc<NL>& src, uint8_t* sm, uint32_t* scl, int nk, int wave,
                                          int a_rd, int b_rd, int sw, int q, const uint32_t* sc_src, int a_srow,
                                          int b_srow, f32x16 (&acc)[4][2]) {
  using C = SliceCfg<64>;
  constexpr int MI = 4, NJ = 2;
  // this wave's scale-word copy: words sc_src[kt] of its row into scl[stage][64 wave + lane]
  auto issue_scales = [&](int kt, int stage) __attribute__((always_inline)) {
    __builtin_amdgcn_global_load_lds((const void*)(sc_src + kt), (lds_void*)(scl + stage * 512 + 64 * wave), 4, 0, 0);
  };
  stage_issue<NL, 64>(src, 0, sm, 0, wave);
  issue_scales(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    MOE_WAIT_VMCNT(0);
    slice_barrier();
    if (kt + 1 < nk) {
      stage_issue<NL, 64>(src, kt + 1, sm, (kt + 1) & 1, wave);
      issue_scales(kt + 1, (kt + 1) & 1);
    }
    const uint32_t* scs = scl + (kt & 1) * 512;
    uint32_t sa[MI], sb[NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i) sa[i] = scs[a_srow + i * 32];
#pragma unroll
    for (int j = 0; j < NJ; ++j) sb[j] = scs[256 + b_srow + j * 32];
    const uint8_t* As = sm + (kt & 1) * C::STAGE_BYTES + a_rd;
    const uint8_t* Bs = sm + (kt & 1) * C::STAGE_BYTES + BM * C::ROWB + b_rd;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int clo = ((4 * s + q) ^ sw) * 16, chi = ((4 * s + 2 + q) ^ sw) * 16;
      i32x8 af[NACT > 0 ? NACT : 1], bfr[NJ];
#pragma unroll
      for (int i = 0; i < NACT; ++i) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(As + i * 32 * C::ROWB + clo);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(As + i * 32 * C::ROWB + chi);
        af[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(Bs + j * 32 * C::ROWB + clo);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(Bs + j * 32 * C::ROWB + chi);
        bfr[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
      __builtin_amdgcn_sched_barrier(0);
      const int shift = 8 * (2 * s + q);
#pragma unroll
      for (int i = 0; i < NACT; ++i) {
        const int sca = (int)((sa[i] >> shift) & 0xffu);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int scb = (int)((sb[j] >> shift) & 0xffu);
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bfr[j], acc[i][j], 0, 0, 0, sca, 0, scb);
        }
      }
    }
  }
}

// An output tile of the MX GEMMs: n-tile nt of group grp, tile rows [r0, r0 + rows), nk K slices
// of 128 from k0; kbl scale bytes per A row (and per B row unless KG).
struct MxTile {
  int nt, grp, r0, rows, k0, nk;
  int64_t kbl;
};

// Tile `logical` of a launch: KG (weight gradients) in launch order n-tile fastest, then m-tile,
// then group (groups in k_order, longest K first), group grp contracting k in [k_off[grp],
// k_off[grp+1]); otherwise the grouped (or dense) tiles of decode_grouped_tile. False: no tile.
template <bool KG>
__device__ __forceinline__ bool mx_decode(const GemmArgs& a, const Grouped& g, int ntn, int logical, MxTile& t) {
  if (KG) {
    const int mtn = (a.M + BM - 1) / BM;
    if (logical >= g.groups * mtn * ntn) return false;
    const int gi = logical / (mtn * ntn), rem = logical - gi * mtn * ntn;
    t.grp = a.k_order ? a.k_order[gi] : gi;
    const int mt = rem / ntn;
    t.nt = rem - mt * ntn;
    t.r0 = mt * BM;
    t.rows = min(BM, a.M - t.r0);
    t.k0 = a.k_off[t.grp];
    t.nk = (a.k_off[t.grp + 1] - t.k0) / 128;
    t.kbl = a.lda / 32;
  } else {
    TileCoord tc;
    if (!decode_grouped_tile(g, logical, ntn, (g.M + BM - 1) / BM, tc)) return false;
    t.nt = tc.nt; t.grp = tc.grp; t.r0 = tc.r0; t.rows = tc.rows;
    t.k0 = 0;
    t.nk = a.K / 128;                            // 128-wide K slices
    t.kbl = a.K / 32;
  }
  return true;
}

// LDS of an MX tile: the two operand stages, then 2 x 512 scale words
constexpr int kMxSmemElems = kGemmSmemElems + 2048;

// One tile; tid: the thread index (the persistent kernel passes one rebuilt per tile); hook() runs
// between the K loop and the epilogue (see gemm_tile).
template <int EPI, bool KG, class Hook = NoHook>
__device__ __forceinline__ void mx_tile(const GemmArgs& a, const uint8_t* __restrict__ a_sc,
                                        const uint8_t* __restrict__ b_sc, const uint8_t* __restrict__ b2_sc,
                                        int64_t sc_group_stride, uint8_t* __restrict__ h_sc, const MxTile& t,
                                        uint8_t* sm, int tid, Hook hook = Hook{}) {
  using C = SliceCfg<64>;
  constexpr int WAVES_N = 4, WM = 128, WN = 64, BN = WAVES_N * WN;
  constexpr int MI = WM / 32, NJ = WN / 32;
  constexpr int NL = BM / (C::RPI * 8);   // loads per operand per slice per wavefront
  constexpr bool PAIRED = EPI == EPI_SWIGLU || EPI == EPI_SAVE_AU;   // gate and up rows in one tile
  const int nt = t.nt, grp = t.grp, r0 = t.r0, rows = t.rows, nk = t.nk, k0 = t.k0;
  const int64_t kbl = t.kbl;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  // Copies as 16-bit units (2 fp8 each): row offsets in units of lda / 2.
  StageSrc<NL> src;
  src.abase = (const uint16_t*)((const uint8_t*)a.A + k0);
  src.bbase[0] = (const uint16_t*)((const uint8_t*)a.B + (KG ? 0 : (int64_t)grp * a.b_group_stride) + k0);
  src.bbase[1] = PAIRED ? (const uint16_t*)((const uint8_t*)a.B2 + (int64_t)grp * a.b_group_stride) : src.bbase[0];
  src.nk1 = nk;
  src.a_shift = 0;
  src.b_shift = 0;
  {
    const int left = __builtin_amdgcn_readfirstlane(rows) - C::RPI * NL * __builtin_amdgcn_readfirstlane(wave);
    src.na = left <= 0 ? 0 : min(NL, (left + C::RPI - 1) / C::RPI);
  }
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int rr = C::RPI * (NL * wave + j) + lane / C::CPR;
    const int ch = (lane % C::CPR) ^ C::swz(rr);
    const int r = r0 + min(rr, rows - 1);
    const int64_t sr = (!KG && a.a_gather) ? (int64_t)(*gmem(a.a_gather + r) / a.a_div) : (int64_t)r;
    src.aoff[j] = (uint32_t)(sr * (a.lda / 2) + ch * 8);
    int64_t wrow;
    if (PAIRED) {
      const int wc = rr / WN, qq = (rr % WN) / 32;
      src.bup[j] = qq >= NJ / 2;
      wrow = (int64_t)nt * (BN / 2) + wc * (WN / 2) + (src.bup[j] ? qq - NJ / 2 : qq) * 32 + (rr & 31);
    } else {
      src.bup[j] = false;
      wrow = (int64_t)nt * BN + rr;
    }
    wrow = wrow < a.N ? wrow : a.N - 1;
    src.boff[j] = (uint32_t)(wrow * (a.ldb / 2) + ch * 8);
  }
  // Scale words: wavefront w < 4 copies those of A tile rows 64 w + lane, w >= 4 those of B tile
  // rows 64 (w - 4) + lane (in the B tile's row order), one 32-bit word (4 blocks) per slice.
  uint32_t* scl = reinterpret_cast<uint32_t*>(sm + 2 * C::STAGE_BYTES);   // 2 x 512 scale words past the stages
  const uint32_t* sc_src;
  {
    const int tr = 64 * (wave & 3) + lane;   // tile row whose words this lane copies
    if (wave < 4) {
      const int r = r0 + min(tr, rows - 1);
      const int64_t sr = (!KG && a.a_gather) ? (int64_t)(*gmem(a.a_gather + r) / a.a_div) : (int64_t)r;
      sc_src = reinterpret_cast<const uint32_t*>(a_sc + sr * kbl + k0 / 32);
    } else {
      int64_t wrow;
      bool up = false;
      if (PAIRED) {
        const int wc = tr / WN, qq = (tr % WN) / 32;
        up = qq >= NJ / 2;
        wrow = (int64_t)nt * (BN / 2) + wc * (WN / 2) + (up ? qq - NJ / 2 : qq) * 32 + (tr & 31);
      } else {
        wrow = (int64_t)nt * BN + tr;
      }
      wrow = wrow < a.N ? wrow : a.N - 1;
      const uint8_t* base = (up ? b2_sc : b_sc) + (KG ? 0 : (int64_t)grp * sc_group_stride);
      sc_src = reinterpret_cast<const uint32_t*>(base + wrow * (KG ? (int64_t)(a.ldb / 32) : kbl) + k0 / 32);
    }
  }
  const int q = lane >> 5;

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int a_rd = (wm * WM + (lane & 31)) * C::ROWB;
  const int b_rd = (wn * WN + (lane & 31)) * C::ROWB;
  const int sw = C::swz(lane & 31);
  const int a_srow = wm * WM + (lane & 31), b_srow = wn * WN + (lane & 31);   // tile rows of this lane's scales
  const int wrows_u = rows - (__builtin_amdgcn_readfirstlane(wave) / WAVES_N) * WM;
  const int nact = wrows_u <= 0 ? 0 : min(MI, (wrows_u + 31) / 32);
  if (nk > 0) switch (nact) {
    case 0: mx_k_loop<EPI, 0, NL>(src, sm, scl, nk, wave, a_rd, b_rd, sw, q, sc_src, a_srow, b_srow, acc); break;
    case 1: mx_k_loop<EPI, 1, NL>(src, sm, scl, nk, wave, a_rd, b_rd, sw, q, sc_src, a_srow, b_srow, acc); break;
    case 2: mx_k_loop<EPI, 2, NL>(src, sm, scl, nk, wave, a_rd, b_rd, sw, q, sc_src, a_srow, b_srow, acc); break;
    case 3: mx_k_loop<EPI, 3, NL>(src, sm, scl, nk, wave, a_rd, b_rd, sw, q, sc_src, a_srow, b_srow, acc); break;
    default: mx_k_loop<EPI, 4, NL>(src, sm, scl, nk, wave, a_rd, b_rd, sw, q, sc_src, a_srow, b_srow, acc); break;
  }
  hook();

  const int ccol = lane & 31;
  const int tid512 = tid;
  if (KG || EPI == EPI_SAVE_AU || (EPI == EPI_STORE && a.c_f32)) {
    // fp32 outputs, element stores (the 32 lanes of a lane group cover 32 consecutive columns).
    // Accumulator slot r of lane l: tile row (r / 4) 8 + (l / 32) 4 + r % 4, column l % 32.
#pragma clang loop unroll(full)
    for (int i = 0; i < MI; ++i)
#pragma clang loop unroll(full)
      for (int r = 0; r < 16; ++r) {
        const int lr = wm * WM + i * 32 + (r >> 2) * 8 + q * 4 + (r & 3);
        if (lr >= rows) continue;
        const int64_t row = r0 + lr;
        if (EPI == EPI_SAVE_AU && !KG) {
          const int64_t col = (int64_t)nt * (BN / 2) + wn * (WN / 2) + ccol;
          if (col < a.N) {
            *gmem((float*)a.C + row * a.ldc + col) = acc[i][0][r];
            *gmem((float*)a.C2 + row * a.ldc + col) = acc[i][1][r];
          }
        } else {
          float* out = (float*)a.C;
          int64_t orow = row;
          if (KG) {
            if (a.m_split > 0 && row >= a.m_split) {
              out = (float*)a.C2;
              orow = row - a.m_split;
            }
            out += (int64_t)grp * a.c_group_stride;
          }
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const int64_t col = (int64_t)nt * BN + wn * WN + j * 32 + ccol;
            if (col < a.N) {
              auto o = gmem(out + orow * a.ldc + col);
              *o = acc[i][j][r] + (a.c_accumulate ? *o : 0.f);
            }
          }
        }
      }
    return;
  }
  __syncthreads();   // every wavefront is done with the staged slices: LDS holds the output tile now
  if (EPI == EPI_SWIGLU) {
    // E4M3 h tile (256 rows x 128 bytes) through LDS, then 16-byte stores (4 per thread instead of
    // 64 single bytes). Chunk c of row r at c ^ (2 ((r >> 2) & 3)): rows r and r + 4 of one LDS
    // write instruction fall on different banks. The E8M0 bytes go straight out.
#pragma clang loop unroll(full)
    for (int i = 0; i < MI; ++i)
#pragma clang loop unroll(full)
      for (int r = 0; r < 16; ++r) {
        const int lr = wm * WM + i * 32 + (r >> 2) * 8 + q * 4 + (r & 3);
        const int row = r0 + lr;
        // one 32-column MX block per (row, wavefront): amax over the 32 lanes of this lane group
        const int c = wn * (WN / 2) + ccol;
        const float h = silu_f(acc[i][0][r]) * acc[i][1][r];
        float amax = fabsf(h);
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
        uint32_t code = 0, sbyte = 127;
        if (amax > 0.f) {
          int eb = (int)((__float_as_uint(amax) >> 23) & 0xffu);
          int se = eb - 127 - 8;
          se = se < -127 ? -127 : (se > 127 ? 127 : se);
          sbyte = (uint32_t)(se + 127);
          code = e4m3_code(h * __uint_as_float((uint32_t)(127 - se) << 23));
        }
        sm[lr * 128 + (((c >> 4) ^ (((lr >> 2) & 3) << 1)) << 4) + (c & 15)] = (uint8_t)code;
        const int64_t col = (int64_t)nt * (BN / 2) + c;
        if (ccol == 0 && lr < rows && col < a.N) *gmem(h_sc + (int64_t)row * (a.ldc / 32) + col / 32) = (uint8_t)sbyte;
      }
    __syncthreads();
#pragma unroll 4
    for (int qq = tid512; qq < BM * 8; qq += 512) {
      const int lr = qq >> 3, c = qq & 7;
      if (lr >= rows) break;
      const int64_t col = (int64_t)nt * (BN / 2) + c * 16;
      if (col >= a.N) continue;
      const u32x4 v = *reinterpret_cast<const u32x4*>(sm + lr * 128 + ((c ^ (((lr >> 2) & 3) << 1)) << 4));
      *gmem(reinterpret_cast<u32x4*>((uint8_t*)a.C + (int64_t)(r0 + lr) * a.ldc + col)) = v;
    }
  } else {
    // BF16 output tile through LDS (512-byte rows, chunk c of row r at c ^ (4 ((r >> 2) & 3))),
    // then 16-byte stores to the (scattered) output rows, whose indices are loaded first (a load
    // between two stores would make the second wait for every earlier one)
    constexpr int NS = BM * 32 / 512;
    int32_t orow[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const int row = r0 + min((tid512 >> 5) + k * 16, rows - 1);
      orow[k] = a.c_scatter ? *gmem(a.c_scatter + row) : row;
    }
#pragma clang loop unroll(full)
    for (int i = 0; i < MI; ++i)
#pragma clang loop unroll(full)
      for (int r = 0; r < 16; ++r) {
        const int lr = wm * WM + i * 32 + (r >> 2) * 8 + q * 4 + (r & 3);
        const int sw4 = ((lr >> 2) & 3) << 2;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int c = wn * WN + j * 32 + ccol;
          *reinterpret_cast<uint16_t*>(sm + lr * 512 + (((c >> 3) ^ sw4) << 4) + (c & 7) * 2) = f2bf(acc[i][j][r]);
        }
      }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const int qq = tid512 + k * 512;
      const int lr = qq >> 5, c = qq & 31;
      if (lr >= rows) break;
      const int64_t col = (int64_t)nt * BN + c * 8;
      if (col >= a.N) continue;
      const u32x4 v = *reinterpret_cast<const u32x4*>(sm + lr * 512 + ((c ^ (((lr >> 2) & 3) << 2)) << 4));
      *gmem(reinterpret_cast<u32x4*>((uint16_t*)a.C + (int64_t)orow[k] * a.ldc + col)) = v;
    }
  }
}

// One workgroup per tile: tile `blockIdx.x` in launch order (KG), or the tiles that exist
// (known on the device) split evenly over the 8 XCDs, contiguous per XCD.
template <int EPI, bool KG>
__global__ __launch_bounds__(512, 1) void gemm_mx_kernel(GemmArgs a, const uint8_t* __restrict__ a_sc,
                                                         const uint8_t* __restrict__ b_sc,
                                                         const uint8_t* __restrict__ b2_sc, int64_t sc_group_stride,
                                                         uint8_t* __restrict__ h_sc, Grouped g, int ntn) {
  __shared__ __attribute__((aligned(16))) uint16_t smem_u16[kMxSmemElems];
  int logical = blockIdx.x;
  if (!KG) {
    const int valid = (g.row_off ? g.tile_off[g.groups] : (g.M + BM - 1) / BM) * ntn;
    const int per_xcd = (valid + 7) >> 3;
    const int bid = blockIdx.x;
    if ((bid >> 3) >= per_xcd) return;
    logical = (bid & 7) * per_xcd + (bid >> 3);
    if (logical >= valid) return;
  }
  MxTile t;
  if (!mx_decode<KG>(a, g, ntn, logical, t)) return;
  mx_tile<EPI, KG>(a, a_sc, b_sc, b2_sc, sc_group_stride, h_sc, t, reinterpret_cast<uint8_t*>(smem_u16),
                   (int)threadIdx.x);
}

// Persistent form (persistent_tiles): the tiles and their dealing order of gemm_mx_kernel, one
// workgroup per CU; each tile is the same workgroup sum, so the results are bitwise those of the
// per-tile launch. budget, budget_ind: the workgroup budget word (nullable), see persistent_tiles.
template <int EPI, bool KG>
__global__ __launch_bounds__(512, 1) void gemm_mx_persistent_kernel(GemmArgs a, const uint8_t* __restrict__ a_sc,
                                                                    const uint8_t* __restrict__ b_sc,
                                                                    const uint8_t* __restrict__ b2_sc,
                                                                    int64_t sc_group_stride,
                                                                    uint8_t* __restrict__ h_sc, Grouped g, int ntn,
                                                                    int32_t* tickets, const int32_t* budget,
                                                                    int budget_ind) {
  __shared__ __attribute__((aligned(16))) uint16_t smem_u16[kMxSmemElems + 4];
  const int valid = KG ? g.groups * ((a.M + BM - 1) / BM) * ntn
                       : (g.row_off ? g.tile_off[g.groups] : (g.M + BM - 1) / BM) * ntn;
  persistent_tiles<!KG>(valid, KG ? valid : (valid + 7) >> 3, KG ? 1 : 8, KG ? 0 : (int)(blockIdx.x & 7), tickets,
                        budget, budget_ind, reinterpret_cast<int*>(smem_u16 + kMxSmemElems),
                        [&](int cur, auto& ti, auto& hook) {
    // per-tile opaque copies of the arguments (nothing derived from them is held across tiles)
    GemmArgs la = a;
    const uint8_t *la_sc = a_sc, *lb_sc = b_sc, *lb2_sc = b2_sc;
    uint8_t* lh_sc = h_sc;
    int64_t lsgs = sc_group_stride;
    asm volatile("" : "+s"(la.A), "+s"(la.B), "+s"(la.B2), "+s"(la.C), "+s"(la.C2), "+s"(la.c_scatter),
                 "+s"(la.a_gather), "+s"(la.a_div));
    asm volatile("" : "+s"(la_sc), "+s"(lb_sc), "+s"(lb2_sc), "+s"(lh_sc), "+s"(lsgs));
    asm volatile("" : "+s"(la.lda), "+s"(la.ldb), "+s"(la.ldc), "+s"(la.b_group_stride), "+s"(la.N), "+s"(la.K));
    MxTile t;
    if (mx_decode<KG>(la, g, ntn, cur, t))
      mx_tile<EPI, KG>(la, la_sc, lb_sc, lb2_sc, lsgs, lh_sc, t, reinterpret_cast<uint8_t*>(smem_u16), ti(), hook);
  });
}

// a_sc / b_sc / b2_sc: E8M0 scales of A [rows][K/32] and of the weights [G][N][K/32]. pc: may
// run as the persistent kernel (see Persist).
int launch_gemm_mx(const GemmArgs& a, const uint8_t* a_sc, const uint8_t* b_sc, const uint8_t* b2_sc,
                   int64_t sc_group_stride, uint8_t* h_sc, const Grouped& g, Epi epi, hipStream_t s,
                   const Persist* pc) {
  if (epi != EPI_SWIGLU && epi != EPI_STORE && epi != EPI_SAVE_AU) return MOE_ERR_UNSUPPORTED;
  const bool paired = epi == EPI_SWIGLU || epi == EPI_SAVE_AU;
  const int tcols = paired ? 128 : 256;
  const int ntn = (a.N + tcols - 1) / tcols;
  const int64_t mt = g.row_off ? g.max_mtiles : (g.M + BM - 1) / BM;
  int64_t nb = mt * ntn;
  nb = (nb + 7) / 8 * 8;
  if (nb == 0) return MOE_OK;
  if (nb > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  // the bf16 / E4M3 epilogues write whole 16-byte chunks of output rows; fp32 ones single words
  const int64_t rowb = epi == EPI_SWIGLU ? 1 : (epi == EPI_SAVE_AU || a.c_f32) ? 4 : 2;
  if ((reinterpret_cast<uintptr_t>(a.C) | (a.ldc * rowb) | (a.N * rowb)) & 15) return MOE_ERR_MISALIGNED;
  int64_t nw = 0;
  int st;
  if ((st = persistent_grid(nb, pc, nw))) return st;
  if (nw > 0) {
    if ((st = launch_zero_tickets(pc->tickets, s))) return st;
    const dim3 pg((unsigned)nw), pb(512);
    if (epi == EPI_SWIGLU)
      hipLaunchKernelGGL((gemm_mx_persistent_kernel<EPI_SWIGLU, false>), pg, pb, 0, s, a, a_sc, b_sc, b2_sc,
                         sc_group_stride, h_sc, g, ntn, pc->tickets, pc->budget, (int)pc->budget_indirect);
    else if (epi == EPI_SAVE_AU)
      hipLaunchKernelGGL((gemm_mx_persistent_kernel<EPI_SAVE_AU, false>), pg, pb, 0, s, a, a_sc, b_sc, b2_sc,
                         sc_group_stride, h_sc, g, ntn, pc->tickets, pc->budget, (int)pc->budget_indirect);
    else
      hipLaunchKernelGGL((gemm_mx_persistent_kernel<EPI_STORE, false>), pg, pb, 0, s, a, a_sc, b_sc, b2_sc,
                         sc_group_stride, h_sc, g, ntn, pc->tickets, pc->budget, (int)pc->budget_indirect);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
  }
  if (epi == EPI_SWIGLU)
    hipLaunchKernelGGL((gemm_mx_kernel<EPI_SWIGLU, false>), dim3((unsigned)nb), dim3(512), 0, s, a, a_sc, b_sc, b2_sc,
                       sc_group_stride, h_sc, g, ntn);
  else if (epi == EPI_SAVE_AU)
    hipLaunchKernelGGL((gemm_mx_kernel<EPI_SAVE_AU, false>), dim3((unsigned)nb), dim3(512), 0, s, a, a_sc, b_sc, b2_sc,
                       sc_group_stride, h_sc, g, ntn);
  else
    hipLaunchKernelGGL((gemm_mx_kernel<EPI_STORE, false>), dim3((unsigned)nb), dim3(512), 0, s, a, a_sc, b_sc, b2_sc,
                       sc_group_stride, h_sc, g, ntn);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

int launch_gemm_mx_kgroup(const GemmArgs& a, const uint8_t* a_sc, const uint8_t* b_sc, int groups, hipStream_t s,
                          const Persist* pc) {
  if (groups <= 0 || a.M <= 0 || a.N <= 0) return MOE_OK;
  if ((a.lda | a.ldb) % 128 || a.ldc % 4 || (reinterpret_cast<uintptr_t>(a.C) & 15) ||
      (a.C2 && (reinterpret_cast<uintptr_t>(a.C2) & 15)))
    return MOE_ERR_MISALIGNED;
  const int ntn = (a.N + BM - 1) / BM, mtn = (a.M + BM - 1) / BM;
  const int64_t nb = (int64_t)groups * mtn * ntn;
  if (nb > 0x7fffffff) return MOE_ERR_UNSUPPORTED;
  Grouped g;
  g.groups = groups;
  int64_t nw = 0;
  int st;
  if ((st = persistent_grid(nb, pc, nw))) return st;
  if (nw > 0) {
    if ((st = launch_zero_tickets(pc->tickets, s))) return st;
    hipLaunchKernelGGL((gemm_mx_persistent_kernel<EPI_STORE, true>), dim3((unsigned)nw), dim3(512), 0, s, a, a_sc,
                       b_sc, b_sc, (int64_t)0, (uint8_t*)nullptr, g, ntn, pc->tickets, pc->budget, (int)pc->budget_indirect);
    MOE_LAUNCH_CHECK();
    return MOE_OK;
  }
  hipLaunchKernelGGL((gemm_mx_kernel<EPI_STORE, true>), dim3((unsigned)nb), dim3(512), 0, s, a, a_sc, b_sc, b_sc,
                     (int64_t)0, (uint8_t*)nullptr, g, ntn);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

}  // namespace moe
