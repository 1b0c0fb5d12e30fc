// One workgroup tile of the bf16 grouped GEMMs (and the operand staging the MXFP8 GEMM shares).
// See gemm.hip for the tiling.
//
// Operand staging: global_load_lds_dwordx4 copies 16 bytes per lane from HBM straight into LDS
// (no register staging, no LDS store instructions). One such instruction of a wavefront fills
// 1 KB of LDS in lane order, i.e. 8 rows of one 64-wide K slice (128 B rows). Two LDS stages of
// 256 A rows and 256 B rows (128 KB); the next slice loads while the current one multiplies.
// Within a row the 16-byte chunks are stored XOR-swizzled (chunk c of row r at position
// c ^ ((r >> 1) & 7)), chosen by measured LDS bank conflicts on gfx950 for this kernel's
// fragment-read pattern (it reads conflict-free; e.g. r & 7 or no swizzle do not).
#pragma once
#include "common.h"

namespace moe {

namespace gemm_detail {
constexpr int kCachePolicyNT = 2;          // cache-policy operand of a gfx950 load: nt (streaming)
constexpr int BM = kGemmBM;                 // 256 rows per m-tile (and 256 B rows per tile)

// Shape of one staged K slice: BKE bf16 per row.
template <int BKE>
struct SliceCfg {
  static_assert(BKE == 64, "64-wide K slices");
  static constexpr int BK = BKE;                      // K elements per slice
  static constexpr int STAGES = 2;                    // LDS stages (loads run one slice ahead)
  static constexpr int ROWB = BKE * 2;                // bytes per staged row
  static constexpr int CPR = ROWB / 16;               // 16-byte chunks per row
  static constexpr int RPI = 1024 / ROWB;             // rows filled by one wavefront load
  static constexpr int KSTEPS = BKE / 16;             // MFMA K steps per slice
  static constexpr int STAGE_BYTES = 2 * BM * ROWB;   // A rows, then B rows
  __device__ static __forceinline__ int swz(int row) { return (row >> 1) & 7; }
};
}  // namespace gemm_detail

// LDS of one tile: two 64 KB stages
constexpr int kGemmSmemElems = 2 * gemm_detail::SliceCfg<64>::STAGE_BYTES / 2;

struct TileCoord {
  int grp, r0, rows, nt;
};

using namespace gemm_detail;

// Rows per m-tile of a group of n rows cut into m = ceil(n / BM) m-tiles: the rows are shared out
// evenly (in multiples of 32) instead of m - 1 full tiles and a remainder. The m-tiles of one group
// stream the same weight rows; with equal row counts they advance at the same rate, so the
// copies that run side by side stay close enough in K for the second read of each weight slice
// to hit the L2. ceil(n / (32 m)) * 32 <= BM, and (m - 1) times it stays below n: no tile is empty.
__device__ __forceinline__ int group_tile_rows(int n, int m) {
  return m <= 1 ? BM : ((n + 32 * m - 1) / (32 * m)) * 32;
}

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
    const int per = group_tile_rows(g.row_off[lo + 1] - g.row_off[lo], g.tile_off[lo + 1] - g.tile_off[lo]);
    tc.r0 = g.row_off[lo] + (mt - g.tile_off[lo]) * per;
    tc.rows = min(per, g.row_off[lo + 1] - tc.r0);
  } else {
    tc.grp = 0;
    tc.r0 = mt * BM;
    if (tc.r0 >= g.M) return false;
    tc.rows = min(BM, g.M - tc.r0);
  }
  return true;
}

// Largest g < groups with off[g] <= q (off non-decreasing, off[0] = 0, groups <= 4096): the
// group of m-tile q. Two rounds of 64 loads across the wavefront and a ballot each, instead of a
// binary search whose ~log2(groups) dependent loads would sit in front of every tile's first
// K slice. Wave-uniform result.
__device__ __forceinline__ int find_group(const int32_t* __restrict__ off, int groups, int q) {
  // lane id from the lane count, so that no caller keeps the thread index register live for it
  const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int step = (groups + 63) >> 6;
  const int i1 = lane * step;
  const bool p1 = i1 < groups && off[i1] <= q;
  const uint64_t m1 = __ballot(p1);                       // lanes 0 .. L1 (lane 0 always: off[0] = 0)
  const int base = (63 - __builtin_clzll(m1)) * step;
  const int i2 = base + lane;
  const bool p2 = lane < step && i2 < groups && off[i2] <= q;
  const uint64_t m2 = __ballot(p2);
  return base + (63 - __builtin_clzll(m2));
}

// Tile `logical` of a grouped (or dense) GEMM with ntn n-tiles per group (dense: one group of mtn
// m-tiles). The tiles of group grp occupy logical [tile_off[grp] * ntn, tile_off[grp + 1] * ntn).
// An XCD runs about 32 tiles at a time, consecutive in this order, and only tiles running close
// together reuse each other's K slices from the L2. Order: blocks of up to kMtGroup = 4 m-tiles,
// n-tile major inside a block, i.e. (m0,n0) (m1,n0) (m2,n0) (m3,n0) (m0,n1) ... then (m4,n0) ...
// The m-tiles of one expert hold equal row counts and advance together, so a window of 32 tiles
// holds 4 m-tiles x 8 n-tiles: 12 operand tiles fetched per 32 tiles, against 18 (2 x 16) for
// pairs of m-tiles (an expert of 4 or more m-tiles fetches each weight tile once per 4 m-tiles). Measured against pairs (bitwise equal outputs): DSV3 forward 9.37 ->
// 9.19 ms, the MXFP8 forward at T = 32768 19.2 -> 19.0 ms, the expert-parallel share unchanged;
// blocks of 8 are no better.
constexpr int kMtGroup = 4;
__device__ __forceinline__ bool decode_grouped_tile(const Grouped& g, int logical, int ntn, int mtn, TileCoord& tc) {
  int grp = 0, t0 = 0, nmt = mtn;
  if (g.row_off) {
    grp = find_group(g.tile_off, g.groups, logical / ntn);
    t0 = g.tile_off[grp];
    nmt = g.tile_off[grp + 1] - t0;
  }
  const int rem = logical - t0 * ntn;
  tc.grp = grp;
  const int blk = rem / (kMtGroup * ntn);
  const int h = min(kMtGroup, nmt - kMtGroup * blk);
  const int r2 = rem - blk * kMtGroup * ntn;
  tc.nt = r2 / h;
  const int mt = kMtGroup * blk + r2 % h;
  const int rbase = g.row_off ? g.row_off[grp] : 0;
  const int rend = g.row_off ? g.row_off[grp + 1] : g.M;
  const int per = g.row_off ? group_tile_rows(rend - rbase, nmt) : BM;
  tc.r0 = rbase + mt * per;
  tc.rows = min(per, rend - tc.r0);
  return tc.rows > 0;
}

typedef __attribute__((address_space(3))) void lds_void;

// The global-memory view of a pointer. The persistent kernels pass their arguments through an
// empty asm (so that nothing derived from them is held across tiles), which hides where the
// pointers came from; their accesses then compile to flat instructions, which count against the
// LDS counter as well as the vector-memory one, so that every LDS wait of an epilogue also waits
// for the stores in flight. Every output and index the GEMMs access is in global memory.
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gmem(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

// s_waitcnt with only the vector-memory counter constrained (expcnt, lgkmcnt left at maximum)
#define MOE_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))

// Where this thread's 16-byte chunks come from: per load instruction a row offset (fixed for the
// tile) and a chunk within the K slice; the K slice is added per stage.
template <int NL>
struct StageSrc {
  const uint16_t* abase;
  const uint16_t* bbase[2];
  uint32_t aoff[NL];    // element offsets (row * ld + chunk * 8) of this lane's A loads
  uint32_t boff[NL];    // and B loads
  bool bup[NL];         // B load from the second weight matrix (W_up)
  int nk1;              // K slices of the first pass; later slices read the second pass
  int64_t a_shift, b_shift;
  int na;               // A loads issued per slice (2-stage slices skip loads of rows past the tile's end)
  bool b_nt = false;    // weight loads carry the non-temporal cache policy
  int64_t bk_stride = 0;   // k-major B: elements per K row
  int b_split = 0;         // k-major B: K rows >= b_split come from bbase[1]
};

// k-major B tile in LDS: 64 K rows of the tile's 256 N columns (512 bytes per row), 16-byte chunk c
// of row k stored at position c ^ bt_swz(k), so that one transposing fragment read (4 rows x 16
// columns per 16 lanes, rows 8 apart for the other half-wave) uses every bank at most twice.
__device__ __forceinline__ int bt_swz(int k) { return 4 * (k & 3); }

// Issues the 2 NL LDS-direct loads of this thread for K slice kt into LDS stage `stage`: A rows
// RPI (NL wave + j) .. + RPI - 1 and the same B rows, for j < NL.
template <int NL, int BKE, bool BT = false>
__device__ __forceinline__ void stage_issue(const StageSrc<NL>& s, int kt, uint8_t* smem, int stage, int wave) {
  using C = SliceCfg<BKE>;
  const bool second = kt >= s.nk1;
  const int ko = (second ? kt - s.nk1 : kt) * C::BK;
  const uint16_t* ab = (second ? s.abase + s.a_shift : s.abase) + ko;
  const int64_t bsh = (second ? s.b_shift : 0) + ko;
  if (BT) {
    // k-major B: K rows ko .. ko + 63 (from the second matrix past b_split), 2 rows per load
    uint8_t* base = smem + stage * C::STAGE_BYTES + wave * (NL * 1024);
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      if (C::STAGES == 2 && j >= s.na) break;
      __builtin_amdgcn_global_load_lds((const void*)(ab + s.aoff[j]), (lds_void*)(base + j * 1024), 16, 0, 0);
    }
    const bool up = s.b_split && ko >= s.b_split;
    const uint16_t* bk = up ? s.bbase[1] + (int64_t)(ko - s.b_split) * s.bk_stride : s.bbase[0] + (int64_t)ko * s.bk_stride;
#pragma unroll
    for (int j = 0; j < NL; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(bk + s.boff[j]), (lds_void*)(base + BM * C::ROWB + j * 1024), 16, 0, 0);
    return;
  }
  uint8_t* base = smem + stage * C::STAGE_BYTES + wave * (NL * 1024);
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    // With 2 stages every wait drains all loads (vmcnt 0), so the count per slice may vary.
    // The skipped rows hold stale LDS; they feed only accumulator rows the epilogue drops.
    if (C::STAGES == 2 && j >= s.na) break;
    __builtin_amdgcn_global_load_lds((const void*)(ab + s.aoff[j]), (lds_void*)(base + j * 1024), 16, 0, 0);
  }
  if (s.b_nt) {
    // non-temporal: weight slices that no other tile of this launch will ask for soon
#pragma unroll
    for (int j = 0; j < NL; ++j)
      __builtin_amdgcn_global_load_lds((const void*)((s.bup[j] ? s.bbase[1] : s.bbase[0]) + bsh + s.boff[j]),
                                       (lds_void*)(base + BM * C::ROWB + j * 1024), 16, 0, kCachePolicyNT);
  } else {
#pragma unroll
    for (int j = 0; j < NL; ++j)
      __builtin_amdgcn_global_load_lds((const void*)((s.bup[j] ? s.bbase[1] : s.bbase[0]) + bsh + s.boff[j]),
                                       (lds_void*)(base + BM * C::ROWB + j * 1024), 16, 0, 0);
  }
}


// Fragments of one K slice for this wave: its first NACT row blocks of A and its NJ column
// blocks of B, for the two 16-wide K steps of the slice.
template <int NACT, int NJ, int KS>
struct Frags {
  bf16x8 a[KS][NACT > 0 ? NACT : 1];
  bf16x8 b[KS][NJ];
};

// Reads the fragments of one LDS stage. a_rd / b_rd: byte offsets of this lane's row; sw: its
// chunk swizzle; half: which 8 of the 16 K values of an MFMA step the lane supplies.
template <int NACT, int NJ, int BKE>
__device__ __forceinline__ void frag_read(const uint8_t* st, int a_rd, int b_rd, int sw, int half,
                                          Frags<NACT, NJ, SliceCfg<BKE>::KSTEPS>& f) {
  using C = SliceCfg<BKE>;
  const uint8_t* As = st + a_rd;
  const uint8_t* Bs = st + BM * C::ROWB + b_rd;
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk) {
    const int c = ((kk * 2 + half) ^ sw) * 16;
#pragma unroll
    for (int i = 0; i < NACT; ++i) f.a[kk][i] = *reinterpret_cast<const bf16x8*>(As + i * 32 * C::ROWB + c);
#pragma unroll
    for (int j = 0; j < NJ; ++j) f.b[kk][j] = *reinterpret_cast<const bf16x8*>(Bs + j * 32 * C::ROWB + c);
  }
}

// The same with a k-major B tile: each B fragment (8 consecutive K of one N column) is two
// transposing reads (ds_read_b64_tr_b16: within each 16 lanes, lane i receives element i, i + 16,
// i + 32, i + 48 of the 64 the 16 lanes read, so lanes 4 j + b reading 4 columns 4 b .. 4 b + 3
// of K row j deliver to lane i the 4 K values of column i). b_tr[j]: this lane's byte offset for
// column block j at K step 0; K step kk adds 16 kk rows, the second read 4 more.
template <int NACT, int NJ, int BKE>
__device__ __forceinline__ void frag_read_bt(const uint8_t* st, int a_rd, const int (&b_tr)[NJ], int sw, int half,
                                             Frags<NACT, NJ, SliceCfg<BKE>::KSTEPS>& f) {
  using C = SliceCfg<BKE>;
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const uint8_t* As = st + a_rd;
  const uint8_t* Bs = st + BM * C::ROWB;
#pragma unroll
  for (int kk = 0; kk < C::KSTEPS; ++kk) {
    const int c = ((kk * 2 + half) ^ sw) * 16;
#pragma unroll
    for (int i = 0; i < NACT; ++i) f.a[kk][i] = *reinterpret_cast<const bf16x8*>(As + i * 32 * C::ROWB + c);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const uint8_t* p = Bs + b_tr[j] + kk * 16 * 512;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p + 4 * 512));
      f.b[kk][j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
}

// MFMAs of one K slice: NACT x NJ blocks of 32 x 32 over the slice's 16-wide K steps.
template <int MI, int NJ, int NACT, int KS>
__device__ __forceinline__ void frag_mfma(const Frags<NACT, NJ, KS>& f, f32x16 (&acc)[MI][NJ]) {
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
#pragma unroll
    for (int i = 0; i < NACT; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[kk][i], f.b[kk][j], acc[i][j], 0, 0, 0);
}

// Waits until at most `pending` K slices of this thread's loads are outstanding (2 NL loads each).
template <int NL>
__device__ __forceinline__ void wait_slices(int pending) {
  if (pending >= 2) MOE_WAIT_VMCNT(4 * NL);
  else if (pending == 1) MOE_WAIT_VMCNT(2 * NL);
  else MOE_WAIT_VMCNT(0);
}

// Barrier between K slices: this wave's LDS reads have landed, then all waves meet. No fence, so
// the later slices' loads stay in flight; the empty asm statements stop the compiler moving LDS
// accesses across.
__device__ __forceinline__ void slice_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The K loop of one tile. LDS stage s holds K slice kt with kt = s mod STAGES. In step kt,
// once slice kt has landed (this thread's loads: only the slices issued after it may be
// pending) and the barrier has made every thread's loads visible (and ended every wave's reads
// of slice kt - 1), the stage of slice kt - 1 is refilled with slice kt + STAGES - 1, then the
// fragments of slice kt are read and multiplied. NACT (active row blocks of this wave) is a
// compile-time constant so that the loop has no divergent branches around the MFMAs.
template <int MI, int NJ, int NACT, int NL, int BKE, bool BT = false>
__device__ __forceinline__ void k_loop(const StageSrc<NL>& src, uint8_t* sm, int nk, int wave, int a_rd,
                                       int b_rd, int sw, int half, f32x16 (&acc)[MI][NJ], const int (&b_tr)[NJ]) {
  using C = SliceCfg<BKE>;
  constexpr int ST = C::STAGES;
  for (int s = 0; s < ST - 1; ++s)
    if (s < nk) stage_issue<NL, BKE, BT>(src, s, sm, s, wave);
  for (int kt = 0; kt < nk; ++kt) {
    wait_slices<NL>(min(ST - 2, nk - 1 - kt));
    slice_barrier();
    if (!BT && kt + ST - 1 < nk) stage_issue<NL, BKE>(src, kt + ST - 1, sm, (kt + ST - 1) % ST, wave);
    Frags<NACT, NJ, C::KSTEPS> f;
    if (BT) {
      // The transposing reads carry no alias information, so the compiler would make them wait
      // for every outstanding LDS-direct copy, the next slice's included: the next slice's
      // copies are issued after them instead (they still run under this slice's MFMAs).
      frag_read_bt<NACT, NJ, BKE>(sm + (kt % ST) * C::STAGE_BYTES, a_rd, b_tr, sw, half, f);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + ST - 1 < nk) stage_issue<NL, BKE, true>(src, kt + ST - 1, sm, (kt + ST - 1) % ST, wave);
    } else {
      frag_read<NACT, NJ, BKE>(sm + (kt % ST) * C::STAGE_BYTES, a_rd, b_rd, sw, half, f);
    }
    // every fragment read of the slice ahead of its MFMAs: one LDS latency per slice
    __builtin_amdgcn_sched_barrier(0);
    frag_mfma<MI, NJ, NACT, C::KSTEPS>(f, acc);
  }
}

// A tile's hook between its K loop and its epilogue (the persistent loop fetches its next ticket
// there); the per-tile kernels pass none.
struct NoHook {
  __device__ void operator()() const {}
};

// Computes one workgroup tile: rows tc.r0 .. tc.r0 + tc.rows - 1 of group tc.grp, n-tile tc.nt,
// K slices [k0, k0 + 32 nk) (times two with a.two_pass). smem holds kGemmSmemElems bf16. hook()
// runs once every wave is past the K loop, before the epilogue.
template <int EPI, bool KG, int WN, int WAVES_N, int BKE, bool BT = false, class Hook = NoHook>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, const TileCoord& tc, int k0, int nk, int ntn,
                                          uint16_t* smem, int tid_in = -1, Hook hook = Hook{}) {
  static_assert(!BT || ((EPI == EPI_STORE || EPI == EPI_DGRAD) && !KG), "k-major B: grouped dgrad GEMMs");
  using C = SliceCfg<BKE>;
  constexpr int WM = 128, BN = WAVES_N * WN;
  constexpr int NWAVES = 2 * WAVES_N, NL = BM / (C::RPI * NWAVES);   // wavefronts; loads per operand per slice
  constexpr int MI = WM / 32, NJ = WN / 32;
  static_assert(BN == BM, "A and B stages have the same row count");
  // tid_in: the thread index as the caller holds it (a persistent caller passes one the compiler
  // cannot see as loop-invariant, so that the tile's lane-dependent addresses are not hoisted out
  // of its tile loop and kept live across the K loop)
  const int tid = tid_in >= 0 ? tid_in : (int)threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: per-wave bases stay in SGPRs
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  uint8_t* sm = reinterpret_cast<uint8_t*>(smem);

  // This lane's loads: row RPI (NL wave + j) + lane / CPR of A and of B, chunk position lane % CPR
  // holding logical chunk (lane % CPR) ^ f(row).
  StageSrc<NL> src;
  src.abase = (const uint16_t*)a.A + k0;
  src.bbase[0] = (const uint16_t*)a.B + (KG ? 0 : (int64_t)tc.grp * a.b_group_stride) + k0;
  src.bbase[1] = (EPI == EPI_SWIGLU || EPI == EPI_SAVE_AU)
                     ? (const uint16_t*)a.B2 + (int64_t)tc.grp * a.b_group_stride + k0
                     : src.bbase[0];
  if (BT) {
    // k-major B: K rows of the group's matrix (rows >= b_split from the second one)
    src.bbase[0] = (const uint16_t*)a.B + (int64_t)tc.grp * a.b_group_stride;
    src.bbase[1] = a.B2 ? (const uint16_t*)a.B2 + (int64_t)tc.grp * a.b_group_stride : src.bbase[0];
    src.bk_stride = a.ldb;
    src.b_split = a.b_split;
  }
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int rr = C::RPI * (NL * wave + j) + lane / C::CPR;
    const int ch = (lane % C::CPR) ^ C::swz(rr);
    const int r = tc.r0 + min(rr, tc.rows - 1);
    const int64_t srow = (!KG && a.a_gather) ? (int64_t)(*gmem(a.a_gather + r) / a.a_div) : (int64_t)r;
    src.aoff[j] = (uint32_t)(srow * a.lda + ch * 8);
    int64_t wrow;
    if (EPI == EPI_SWIGLU || EPI == EPI_SAVE_AU) {
      // per wave column block: NJ/2 blocks of gate rows, then the matching NJ/2 blocks of up rows
      const int blk = rr / WN, q = (rr % WN) / 32;
      src.bup[j] = q >= NJ / 2;
      wrow = (int64_t)tc.nt * (BN / 2) + blk * (WN / 2) + (src.bup[j] ? q - NJ / 2 : q) * 32 + (rr & 31);
    } else {
      src.bup[j] = false;
      wrow = (int64_t)tc.nt * BN + rr;
    }
    wrow = wrow < a.N ? wrow : a.N - 1;          // partial last n-tile: clamp, results unused
    src.boff[j] = (uint32_t)(wrow * a.ldb + ch * 8);
    if (BT) {
      // K row kr of the slice, position lane % 32 of its 32 chunks holding chunk c = position ^ swz
      // (N columns 8 c .. 8 c + 7 of the tile; past N clamped, results unused)
      const int kr = 2 * (NL * wave + j) + (lane >> 5);
      const int c = (lane & 31) ^ bt_swz(kr);
      int64_t n = (int64_t)tc.nt * BN + 8 * c;
      n = n < a.N - 8 ? n : a.N - 8;
      src.boff[j] = (uint32_t)(kr * a.ldb + n);
    }
  }
  // K slice kt < nk1 reads the first pass, kt >= nk1 the second (operands shifted by the split offsets)
  src.nk1 = nk;
  {
    // wave-uniform: A loads j of this wave start at row RPI (NL wave + j)
    const int left = __builtin_amdgcn_readfirstlane(tc.rows) - C::RPI * NL * __builtin_amdgcn_readfirstlane(wave);
    src.na = left <= 0 ? 0 : min(NL, (left + C::RPI - 1) / C::RPI);
  }
  // The routed down GEMM's weight tile (256 of D rows x I) is read by the m-tiles of one expert,
  // which the tile order runs side by side, and by no tile after them; streaming it past the L2's retention
  // keeps the activation rows that the expert's other n-tiles re-read. Measured on the DSV3
  // forward: down 3.17 -> 3.12 ms under its routing, 2.52 -> 2.33 ms with 256 slots per expert
  // (bitwise equal). On the up/gate GEMM the same policy measured no faster.
  src.b_nt = EPI == EPI_STORE && !KG && a.c_scatter != nullptr;
  src.a_shift = a.a_seg_shift;
  src.b_shift = a.b_seg_shift;
  if (a.two_pass) nk *= 2;

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int a_rd = (wm * WM + (lane & 31)) * C::ROWB;
  const int b_rd = (wn * WN + (lane & 31)) * C::ROWB;
  const int sw = C::swz(lane & 31), half = lane >> 5;
  // k-major B: this lane's transposing-read offsets per column block (16-lane group g reads K rows
  // 8 (g / 2) + (lane % 16) / 4 and columns 16 (g % 2) + 4 (lane % 4) of the block)
  int b_tr[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int g = (lane >> 4) & 3, sl = lane & 15;
    const int kr = 8 * (g >> 1) + (sl >> 2);
    const int ncol = wn * WN + j * 32 + 16 * (g & 1) + 4 * (sl & 3);
    b_tr[j] = BT ? kr * 512 + ((((ncol >> 3) ^ bt_swz(kr))) << 4) + (ncol & 7) * 2 : 0;
  }

  static_assert(4 * NL <= 63, "vmcnt range");
  // wave-uniform count of this wave's row blocks that hold a valid row
  const int wrows_u = tc.rows - (__builtin_amdgcn_readfirstlane(wave) / WAVES_N) * WM;
  const int nact = wrows_u <= 0 ? 0 : min(MI, (wrows_u + 31) / 32);
  static_assert(MI == 4, "row-block dispatch below assumes 4 row blocks per wave");
  switch (nact) {
    case 0: k_loop<MI, NJ, 0, NL, BKE, BT>(src, sm, nk, wave, a_rd, b_rd, sw, half, acc, b_tr); break;
    case 1: k_loop<MI, NJ, 1, NL, BKE, BT>(src, sm, nk, wave, a_rd, b_rd, sw, half, acc, b_tr); break;
    case 2: k_loop<MI, NJ, 2, NL, BKE, BT>(src, sm, nk, wave, a_rd, b_rd, sw, half, acc, b_tr); break;
    case 3: k_loop<MI, NJ, 3, NL, BKE, BT>(src, sm, nk, wave, a_rd, b_rd, sw, half, acc, b_tr); break;
    default: k_loop<MI, NJ, 4, NL, BKE, BT>(src, sm, nk, wave, a_rd, b_rd, sw, half, acc, b_tr); break;
  }
  __syncthreads();
  hook();

  // epilogue. Accumulator slot r of lane l: row (r/4)*8 + (l/32)*4 + r%4, column l%32.
  const int ccol = lane & 31;
  if (EPI == EPI_STORE && !KG && !a.c_f32 && ((reinterpret_cast<uintptr_t>(a.C) | (a.ldc * 2) | (a.N * 2)) & 15) == 0) {
    // BF16 tile through LDS (free now), then whole 16-byte chunks to the output rows (16-byte
    // aligned rows and N a multiple of 8): 16 stores per thread instead of 128 two-byte ones. Chunk c of tile row r sits at c ^ (4 ((r >> 2) & 3))
    // so the two rows one store instruction writes (r and r + 4) use different banks.
    static_assert(BN * 2 == 512, "one tile row is 32 chunks of 16 bytes");
    // Output rows of this thread's NS chunk stores (tile rows tid / 32 + k NT / 32), loaded before
    // the tile goes through LDS: a scatter load between two stores would make the second store
    // wait for every earlier one (vector-memory waits count stores too).
    constexpr int NT = NWAVES * 64, NS = BM * 32 / NT;
    int32_t orow[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const int row = tc.r0 + min((tid >> 5) + k * (NT / 32), tc.rows - 1);
      orow[k] = a.c_scatter ? *gmem(a.c_scatter + row) : row;
    }
#pragma clang loop unroll(full)
    for (int i = 0; i < MI; ++i)
#pragma clang loop unroll(full)
      for (int r = 0; r < 16; ++r) {
        const int lr = wm * WM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
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
      const int q = tid + k * NT;
      const int lr = q >> 5, c = q & 31;
      if (lr >= tc.rows) break;           // rows grow with q
      const int64_t col = (int64_t)tc.nt * BN + c * 8;
      if (col >= a.N) continue;
      const u32x4 v = *reinterpret_cast<const u32x4*>(sm + lr * 512 + ((c ^ (((lr >> 2) & 3) << 2)) << 4));
      *gmem(reinterpret_cast<u32x4*>((uint16_t*)a.C + (int64_t)orow[k] * a.ldc + col)) = v;
    }
    return;
  }
  if (EPI == EPI_SWIGLU && !a.c_f32 && ((reinterpret_cast<uintptr_t>(a.C) | (a.ldc * 2) | (a.N * 2)) & 15) == 0) {
    // h tile (BM x BN/2 BF16, 256-byte rows) through LDS the same way, 8 chunk stores per thread
    static_assert(BN == 256, "h tile rows are 16 chunks of 16 bytes");
#pragma clang loop unroll(full)
    for (int i = 0; i < MI; ++i)
#pragma clang loop unroll(full)
      for (int r = 0; r < 16; ++r) {
        const int lr = wm * WM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int sw4 = ((lr >> 2) & 3) << 2;
#pragma unroll
        for (int j = 0; j < NJ / 2; ++j) {
          const int c = wn * (WN / 2) + j * 32 + ccol;
          const float h = silu_f(acc[i][j][r]) * acc[i][j + NJ / 2][r];
          *reinterpret_cast<uint16_t*>(sm + lr * 256 + (((c >> 3) ^ sw4) << 4) + (c & 7) * 2) = f2bf(h);
        }
      }
    __syncthreads();
    constexpr int NT = NWAVES * 64;
#pragma unroll 4
    for (int q = tid; q < BM * 16; q += NT) {
      const int lr = q >> 4, c = q & 15;
      if (lr >= tc.rows) break;
      const int64_t col = (int64_t)tc.nt * (BN / 2) + c * 8;
      if (col >= a.N) continue;
      const u32x4 v = *reinterpret_cast<const u32x4*>(sm + lr * 256 + ((c ^ (((lr >> 2) & 3) << 2)) << 4));
      *gmem(reinterpret_cast<u32x4*>((uint16_t*)a.C + (int64_t)(tc.r0 + lr) * a.ldc + col)) = v;
    }
    return;
  }
  if (EPI == EPI_DGRAD && a.lo_off % 8 == 0 &&
      ((reinterpret_cast<uintptr_t>(a.ea) | reinterpret_cast<uintptr_t>(a.eu) | reinterpret_cast<uintptr_t>(a.C) |
        reinterpret_cast<uintptr_t>(a.C2) | (a.lde * 4) | (a.ldc * 2) | (a.N * 2)) & 15) == 0) {
    // SwiGLU backward through LDS, in 4 rounds of 64 tile rows (row block i of both wavefront
    // rows). Per round: a and u (fp32) of those rows are copied into LDS with 16-byte loads; each
    // lane reads its elements, computes da, du and their low halves, and writes the four BF16
    // values back into the 8 bytes it read; then whole 16-byte chunks of each output row go out.
    // Same arithmetic and the same partial-sum order as the element-wise epilogue below. The row
    // partials <h, dh'> sit past the 128 KB of staging (the kernel allocates them for DGRAD).
    float* part = reinterpret_cast<float*>(smem + kGemmSmemElems);   // [BM][WAVES_N]
    uint8_t* la = sm;                 // a: 64 rows x 1 KB (256 fp32), chunk c of row r at c ^ (8 ((r >> 2) & 1))
    uint8_t* lu = sm + 65536;         // u: the same
    constexpr int NT = NWAVES * 64;
#pragma clang loop unroll(full)
    for (int i = 0; i < MI; ++i) {
      if (i > 0) __syncthreads();     // the previous round's stores have read their chunks
      // LDS-direct copies, one 1 KB row per wavefront instruction: lane l fills position l of the
      // row, i.e. chunk l ^ swizzle (columns past N are left out)
#pragma unroll
      for (int t = 0; t < 64 / NWAVES; ++t) {
        const int rl = __builtin_amdgcn_readfirstlane(wave) * (64 / NWAVES) + t;
        const int lr = (rl >> 5) * WM + i * 32 + (rl & 31);
        const int c = lane ^ (((rl >> 2) & 1) << 3);
        const int64_t col = (int64_t)tc.nt * BN + c * 4;
        if (lr < tc.rows && col < a.N) {
          const int64_t ge = (int64_t)(tc.r0 + lr) * a.lde + col;
          __builtin_amdgcn_global_load_lds((const void*)(a.ea + ge), (lds_void*)(la + rl * 1024), 16, 0, 0);
          __builtin_amdgcn_global_load_lds((const void*)(a.eu + ge), (lds_void*)(lu + rl * 1024), 16, 0, 0);
        }
      }
      MOE_WAIT_VMCNT(0);
      __syncthreads();
#pragma clang loop unroll(full)
      for (int r = 0; r < 16; ++r) {
        const int rsub = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int rl = wm * 32 + rsub, lr = wm * WM + i * 32 + rsub;
        const bool ok = lr < tc.rows;
        const int row = tc.r0 + lr;
        const float gj = (ok && a.row_scale) ? *gmem(a.row_scale + row) : 1.f;
        float p = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int cl = wn * WN + j * 32 + ccol;
          const int pos = rl * 1024 + (((cl >> 2) ^ (((rl >> 2) & 1) << 3)) << 4) + (cl & 3) * 4;
          const float av = *reinterpret_cast<const float*>(la + pos);
          const float uv = *reinterpret_cast<const float*>(lu + pos);
          const float sg = sigmoid_f(av);
          const float sl = av * sg;
          const float dhp = acc[i][j][r];
          if (ok && (int64_t)tc.nt * BN + cl < a.N) p = fmaf(sl * uv, dhp, p);
          const float dh = gj * dhp;
          const float da = dh * uv * sg * (1.f + av * (1.f - sg));
          const float du = dh * sl;
          const uint16_t dah = f2bf_split(da), duh = f2bf_split(du);
          *reinterpret_cast<uint32_t*>(la + pos) = (uint32_t)dah | ((uint32_t)duh << 16);
          *reinterpret_cast<uint32_t*>(lu + pos) =
              (uint32_t)f2bf(da - bf2f(dah)) | ((uint32_t)f2bf(du - bf2f(duh)) << 16);
        }
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) p += __shfl_xor(p, off, 64);
        if (ccol == 0) part[lr * WAVES_N + wn] = p;
      }
      __syncthreads();
#pragma unroll 1
      for (int q = tid; q < 64 * 32; q += NT) {
        const int rl = q >> 5, g8 = q & 31;
        const int lr = (rl >> 5) * WM + i * 32 + (rl & 31);
        const int64_t col = (int64_t)tc.nt * BN + g8 * 8;
        if (lr >= tc.rows || col >= a.N) continue;
        const int sw = ((rl >> 2) & 1) << 3;
        const int p0 = rl * 1024 + (((2 * g8) ^ sw) << 4), p1 = rl * 1024 + (((2 * g8 + 1) ^ sw) << 4);
        const uint4 h0 = *reinterpret_cast<const uint4*>(la + p0), h1 = *reinterpret_cast<const uint4*>(la + p1);
        const int64_t o = (int64_t)(tc.r0 + lr) * a.ldc + col;
        // element e of the 8 holds (da | du << 16): the low halves are da, the high halves du
        *gmem(reinterpret_cast<u32x4*>((uint16_t*)a.C + o)) =
            u32x4{(h0.x & 0xffffu) | (h0.y << 16), (h0.z & 0xffffu) | (h0.w << 16),
                  (h1.x & 0xffffu) | (h1.y << 16), (h1.z & 0xffffu) | (h1.w << 16)};
        *gmem(reinterpret_cast<u32x4*>((uint16_t*)a.C2 + o)) =
            u32x4{(h0.x >> 16) | (h0.y & 0xffff0000u), (h0.z >> 16) | (h0.w & 0xffff0000u),
                  (h1.x >> 16) | (h1.y & 0xffff0000u), (h1.z >> 16) | (h1.w & 0xffff0000u)};
        if (a.lo_off) {
          const uint4 l0 = *reinterpret_cast<const uint4*>(lu + p0), l1 = *reinterpret_cast<const uint4*>(lu + p1);
          *gmem(reinterpret_cast<u32x4*>((uint16_t*)a.C + o + a.lo_off)) =
              u32x4{(l0.x & 0xffffu) | (l0.y << 16), (l0.z & 0xffffu) | (l0.w << 16),
                    (l1.x & 0xffffu) | (l1.y << 16), (l1.z & 0xffffu) | (l1.w << 16)};
          *gmem(reinterpret_cast<u32x4*>((uint16_t*)a.C2 + o + a.lo_off)) =
              u32x4{(l0.x >> 16) | (l0.y & 0xffff0000u), (l0.z >> 16) | (l0.w & 0xffff0000u),
                    (l1.x >> 16) | (l1.y & 0xffff0000u), (l1.z >> 16) | (l1.w & 0xffff0000u)};
        }
      }
    }
    __syncthreads();
    if (tid < tc.rows) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES_N; ++w) sum += part[tid * WAVES_N + w];
      *gmem(a.row_partial + (int64_t)(tc.r0 + tid) * ntn + tc.nt) = sum;
    }
    return;
  }
  float* part = reinterpret_cast<float*>(smem);   // EPI_DGRAD: [BM][WAVES_N] partials (LDS is free now)
  // fully unrolled: the accumulators must be indexed with constants to stay in registers
#pragma clang loop unroll(full)
  for (int i = 0; i < MI; ++i) {
#pragma clang loop unroll(full)
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
            if (a.c_f32) *gmem(((float*)a.C) + (int64_t)row * a.ldc + col) = h;
            else *gmem(((uint16_t*)a.C) + (int64_t)row * a.ldc + col) = f2bf(h);
          } else {
            *gmem(((float*)a.C) + (int64_t)row * a.ldc + col) = gt;
            *gmem(((float*)a.C2) + (int64_t)row * a.ldc + col) = up;
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
            const uint16_t dah = f2bf_split(da), duh = f2bf_split(du);
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
        // bound the loads the scheduler hoists ahead (it would otherwise spill)
        __builtin_amdgcn_sched_barrier(0);
      } else {
        if (!ok) continue;
        if (KG) {
          const bool hi = a.C2 && row >= a.m_split;
          float* cb = (float*)(hi ? a.C2 : a.C) + (int64_t)tc.grp * a.c_group_stride;
          const int64_t orow = hi ? row - a.m_split : row;
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const int64_t col = (int64_t)tc.nt * BN + wn * WN + j * 32 + ccol;
            // nontemporal: nothing reads dW again in this call (layer backward 57.95 -> 57.03 ms at
            // the DSV3 shape; staging the tile through LDS for 16-byte stores measured no faster)
            if (col < a.N) __builtin_nontemporal_store(acc[i][j][r], gmem(cb + orow * a.ldc + col));
          }
        } else {
          const int64_t orow = a.c_scatter ? (int64_t)a.c_scatter[row] : (int64_t)row;
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const int64_t col = (int64_t)tc.nt * BN + wn * WN + j * 32 + ccol;
            if (col >= a.N) continue;
            if (a.c_f32) *gmem(((float*)a.C) + orow * a.ldc + col) = acc[i][j][r];
            else *gmem(((uint16_t*)a.C) + orow * a.ldc + col) = f2bf(acc[i][j][r]);
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
      *gmem(a.row_partial + (int64_t)(tc.r0 + tid) * ntn + tc.nt) = s;
    }
  }
}


// The tile loop of the persistent GEMMs (one workgroup per CU, looping over tiles instead of one
// workgroup per tile). Tiles are dealt from ticket counters, one per range of per_range
// consecutive tiles (nrange ranges, counters tickets[0 .. nrange-1]): a workgroup starts with
// range `home` and moves on to the following ones once it finds a range used up, so workgroups
// that finish early take over the rest. body(tile, ti, hook) computes tile `tile`, calling ti() for
// the thread index and hook() between its K loop and its epilogue (with EARLY the hook fetches the
// next ticket, below). Workgroups never wait for one another; the only shared state is the
// counters. The loop keeps no per-lane value live across a tile (the tile itself uses the whole register
// budget): the thread index is rebuilt per tile from the lane count and the wavefront's scalar
// index, and thread 0's position in the ranges is kept in LDS, in the two ints at ctl (past the
// tile's own LDS use, in the same array: as separate __shared__ objects the compiler could not
// tell them from the staging buffers and guarded every fragment read with a wait for all
// outstanding LDS-direct copies).
// budget (nullable): a word polled between tiles (the sharing of the sparsenotes page
// "Mixture-of-Kittens: MoE Megakernel for NVL72s", section "The production details": the
// persistent kernel hands processors back to another stream's work). While it holds v > 0,
// workgroups with index >= v take no further tile and exit once their current tile is done;
// the others go on until every tile is taken. The word is read, never written. budget_ind: budget
// points at the word's address (8 bytes; null: no limit) instead of the word.
template <bool EARLY, class Body>
__device__ __forceinline__ void persistent_tiles(int valid, int per_range, int nrange, int home, int32_t* tickets,
                                                 const int32_t* budget, int budget_ind, int* ctl, Body&& body) {
  int& s_next = ctl[0];
  int& s_probe = ctl[1];
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  auto thread_index = [&]() -> int {
    int t = wave * 64 + (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(t));   // opaque per tile: the tile's lane-dependent addressing stays inside the loop
    return t;
  };
  auto take = [&]() -> int {   // thread 0 only
    if (budget) {
      const int32_t* word = budget_ind ? *reinterpret_cast<const int32_t* const volatile*>(budget) : budget;
      const int v = word ? __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) : 0;
      if (v > 0 && (int)blockIdx.x >= v) return -1;
    }
    int probe = s_probe;
    int got = -1;
    for (; probe < nrange; ++probe) {
      const int x = (home + probe) % nrange;
      const int lo = x * per_range, cnt = min(per_range, valid - lo);
      if (cnt <= 0) continue;
      const int i = __hip_atomic_fetch_add(tickets + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (i < cnt) {
        got = lo + i;
        break;
      }
    }
    s_probe = probe;
    return got;
  };
  if (threadIdx.x == 0) {
    s_probe = 0;
    s_next = take();
  }
  __syncthreads();
  int cur = __builtin_amdgcn_readfirstlane(s_next);   // uniform: the tile's coordinates stay scalar
  while (cur >= 0) {
    // EARLY: thread 0 fetches the next ticket while the tile's epilogue runs: early() (the tile's
    // hook, after its K loop) polls the budget and issues one fetch-add on the range it is in; the
    // result is used after the tile, so the atomic's round trip overlaps the epilogue. pend: the
    // raw ticket, -2 when the budget stops this workgroup, -3 when nothing was issued (then, and
    // without EARLY, take() after the tile). Measured on the DSV3 forward: up/gate 5.25 -> 5.17 ms,
    // down 2.76 -> 2.74 ms; on the backward's GEMMs (K-grouped, k-major B, fp32 epilogues) it
    // measured no faster and is not used there.
    // After the tile every thread is past its read of s_next (the tile's barriers) and, after the
    // barrier below, past the epilogue's LDS reads that the next tile's copies overwrite.
    if constexpr (EARLY) {
      int pend = -3, pend_x = 0;
      auto early = [&]() {
        if (thread_index() != 0) return;
        if (budget) {
          const int32_t* word = budget_ind ? *reinterpret_cast<const int32_t* const volatile*>(budget) : budget;
          const int v = word ? __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) : 0;
          if (v > 0 && (int)blockIdx.x >= v) {
            pend = -2;
            return;
          }
        }
        const int probe = s_probe;
        if (probe >= nrange) return;
        const int x = (home + probe) % nrange;
        if (min(per_range, valid - x * per_range) <= 0) return;
        pend_x = x;
        pend = __hip_atomic_fetch_add(tickets + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      };
      body(cur, thread_index, early);
      if (thread_index() == 0) {
        const int lo = pend_x * per_range, cnt = min(per_range, valid - lo);
        if (pend == -2) {
          s_next = -1;
        } else if (pend >= 0 && pend < cnt) {
          s_next = lo + pend;
        } else {
          if (pend >= 0) s_probe = s_probe + 1;   // that range is used up
          s_next = take();
        }
      }
    } else {
      NoHook none;
      body(cur, thread_index, none);
      if (thread_index() == 0) s_next = take();
    }
    __syncthreads();
    cur = __builtin_amdgcn_readfirstlane(s_next);
    __syncthreads();
  }
}

}  // namespace moe
