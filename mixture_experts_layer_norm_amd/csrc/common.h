// Internal declarations shared by the HIP sources of libmoe.so (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------------------------------------
// element types and vectors
// ---------------------------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;   // raw bf16 bits in memory

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN)
// float -> bf16 bits, round to nearest even; a NaN keeps its sign and top payload bits with the
// quiet bit set. gfx950's conversion instruction (v_cvt_pk_bf16_f32); over all 2^32 inputs it
// gives the bits of f2bf_split below.
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// The same rounding in integer arithmetic, for the high half of a split v = hi + lo with
// lo = v - hi: given the conversion instruction, the compiler sees hi as a float truncation of v
// and may fuse the product that forms v into the subtraction (lo then comes from the unrounded
// product); from integer operations it cannot, and lo is the residual of the fp32 v.
__device__ __forceinline__ uint16_t f2bf_split(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float silu_f(float a) { return a / (1.0f + __expf(-a)); }
__device__ __forceinline__ float sigmoid_f(float a) { return 1.0f / (1.0f + __expf(-a)); }

// ---------------------------------------------------------------------------------------------
// workspace layout (byte offsets from the workspace base)
// ---------------------------------------------------------------------------------------------
constexpr int kRouteRowsPerBlock = 2048;     // schedule: routes per histogram block
constexpr int kGemmBM = 256;                 // rows per grouped-GEMM m-tile
constexpr int kErrOffset = 0;                // sticky error word (int32)
// Byte offset, inside the error word's 256-byte block at the start of the forward workspace, of the
// persistent GEMMs' 8 ticket counters (the workgroup budget word sits at MOE_WS_CU_BUDGET_OFFSET).
constexpr size_t kTicketsOffset = 64;

struct WsLayout {
  size_t err;              // int32 error word
  size_t ctrl;             // reserved control words
  size_t blk_hist;         // [nblk][E] int32
  size_t tile_off;         // [E+1] int32  m-tile prefix for kGemmBM
  size_t grp_clean;        // [E+1] int32  sanitised caller offsets (expert-level entry)
  size_t grp_poff;         // [E+1] int32  64-padded offsets
  size_t x_slot;           // dispatched rows
  size_t x_slot_sc;        // MX scales of x_slot
  size_t h;                // gated activation
  size_t h_sc;             // MX scales of h
  size_t y_routes;         // per-route outputs [T*K][D]
  size_t sh_h;             // shared expert activation [T][I_s]
  size_t sh_out;           // shared expert output [T][D]
  size_t bwd;              // backward scratch start
  size_t total;
  size_t chunk_tiles;      // [C][E+1] int32 m-tile prefix of each chunk over experts
  size_t chunk_rowoff;     // [C][E+1] int32 experts' row ranges clamped to each chunk
  int64_t nblk;            // histogram blocks
  int64_t ring_rows;       // rows of x_slot / h held (chunk * stages, or T*K)
  int64_t chunk;           // rows per chunk
  int32_t stages;          // ring stages (1 when one chunk holds everything)
  int32_t chunks;          // C (1 when one chunk holds everything)
  bool chunked;            // chunk_rows selects the chunked ring
};

size_t elt_bytes(int dtype);
WsLayout ws_layout(const moe_problem& p);

int validate_problem(const moe_problem* p);
int validate_routing(const moe_problem* p);

// ---------------------------------------------------------------------------------------------
// launchers (each returns 0 or a moe_status; all enqueue on `s`)
// ---------------------------------------------------------------------------------------------
int launch_route_topk(const float* logits, int32_t* idx, float* w, int T, int E, int K, hipStream_t s);
int launch_route_topk_partials(const float* part, int S, int64_t part_stride, float* logits, int32_t* idx, float* w,
                               int T, int E, int K, hipStream_t s);
int launch_schedule(const int32_t* idx, int T, int K, int E, int32_t* counts, int32_t* offsets,
                    int32_t* perm, int32_t* inv_perm, int32_t* blk_hist, int32_t* tile_off,
                    int32_t* err, hipStream_t s);

int launch_dispatch_tokens(const void* x, int dtype, const int32_t* inv_perm, int T, int K, int D, void* x_slot,
                           uint8_t* x_slot_sc, hipStream_t s);
int launch_dispatch(const void* x, int dtype, const int32_t* perm, int K, int D, int64_t begin,
                    int64_t count, void* x_slot, uint8_t* x_slot_sc, hipStream_t s);
int launch_combine(const void* y_routes, const void* shared_out, const float* topk_w, void* out,
                   int T, int K, int D, int dtype, hipStream_t s);
int launch_group_order(const int32_t* poff, int G, int32_t* order, hipStream_t s);
int launch_group_prefix(const int32_t* offsets, int G, int rows, int32_t* clean, int32_t* tile_off, int32_t* poff,
                        int32_t* err, hipStream_t s, int pad = 64);
int launch_transpose_pad(int mode, const void* src, const void* src2, const float* scale, int64_t lds, int W,
                         const int32_t* offsets, const int32_t* poff, int G, int64_t max_padded, void* out,
                         int64_t ldo, hipStream_t s, int split_lo = 0, const int32_t* rmap = nullptr, int rdiv = 1);
int launch_row_sum(const float* part, int64_t rows, int ntn, float* out, hipStream_t s);
int launch_gather_f32(const float* src, const int32_t* idx, int64_t n, float* out, hipStream_t s);
int launch_router_backward(const float* dg_slot, const int32_t* inv_perm, const int32_t* topk_idx,
                           const float* topk_w, int T, int E, int K, float* d_topk_w, float* d_logits,
                           hipStream_t s);
int launch_reverse_dispatch(const void* dx_slot, const int32_t* inv_perm, const void* dx_shared, void* dx, int T,
                            int K, int D, hipStream_t s);
enum { TR_COPY = 0, TR_SWIGLU = 2 };   // TR_SWIGLU reads fp32 a and u
int launch_quantize_mx(const uint16_t* src, int64_t rows, int cols, uint8_t* q, uint8_t* sc,
                       hipStream_t s);
// MXFP8 backward operands (mx_backward.hip)
int launch_mx_requant_t(const uint8_t* src, const uint8_t* ssc, int G, int R, int C, uint8_t* out, uint8_t* osc,
                        int64_t ldo, int64_t col0, int64_t out_bstride, int64_t osc_bstride, hipStream_t s);
int launch_mx_quant_t(const uint16_t* src, const float* rscale, int64_t lds, int W, const int32_t* offs,
                      const int32_t* poff, int G, int64_t max_padded, uint8_t* q, uint8_t* sc, int64_t ldo, uint8_t* rq,
                      uint8_t* rsc, hipStream_t s, const int32_t* rmap = nullptr, int rdiv = 1);
int launch_mx_swiglu_bwd_t(const float* a, const float* u, const float* dhp, const float* g, int I, const int32_t* offs,
                           const int32_t* poff, int G, int64_t max_padded, uint8_t* dq, uint8_t* dsc, uint8_t* hq,
                           uint8_t* hsc, uint8_t* daq, uint8_t* dasc, int64_t ldo, float* part, hipStream_t s);

// grouped GEMM descriptor. The rows of group g are row_off[g] .. row_off[g+1]-1 of A (after the
// optional gather); m-tiles of kGemmBM rows are numbered by tile_off (prefix over groups). With
// row_off == nullptr there is one group of M rows.
struct Grouped {
  const int32_t* row_off = nullptr;
  const int32_t* tile_off = nullptr;
  int32_t groups = 1;
  int32_t M = 0;              // rows when row_off == nullptr
  int64_t max_mtiles = 0;     // host bound on the number of m-tiles (grid size)
};

// EPI_SWIGLU:   h = SiLU(gate) * up                       -> C
// EPI_STORE:    plain product (optional row scatter)       -> C (bf16 or fp32)
// EPI_SAVE_AU:  gate pre-activation a -> C, up projection u -> C2 (fp32)
// EPI_DGRAD:    product dh' = dY W_down; with a, u (ea, eu, fp32) and the row weight g:
//               da -> C, du -> C2 (bf16) and per-tile partial <h, dh'> -> row_partial
enum Epi { EPI_SWIGLU = 0, EPI_STORE = 1, EPI_SAVE_AU = 2, EPI_DGRAD = 3 };

struct GemmArgs {
  const void* A = nullptr; int64_t lda = 0;
  const int32_t* a_gather = nullptr; int32_t a_div = 1;  // A row r -> a_gather[r] / a_div
  const void* B = nullptr; const void* B2 = nullptr;     // B2: up-projection weights (SwiGLU)
  int64_t ldb = 0; int64_t b_group_stride = 0;           // elements
  int32_t N = 0;          // output columns (h columns for SwiGLU)
  int32_t K = 0;          // contraction length
  void* C = nullptr; int64_t ldc = 0;                    // output
  const int32_t* c_scatter = nullptr;                    // output row r -> c_scatter[r]
  int32_t c_f32 = 0;                                     // store fp32 instead of bf16
  void* C2 = nullptr;                                    // second output (see Epi)
  // K-grouped mode (weight gradients): group g contracts k in [k_off[g], k_off[g+1]) (multiples
  // of 64); A is [M][lda], B is [N][ldb] shared by all groups; the fp32 output of group g is
  // C + g * c_group_stride ([M][ldc]), or C2 + g * c_group_stride for rows >= m_split.
  const int32_t* k_off = nullptr;
  const int32_t* k_order = nullptr;   // groups in dealing order (longest K first); null: 0, 1, ...
  int32_t M = 0;
  int32_t m_split = 0;
  int64_t c_group_stride = 0;
  // EPI_DGRAD inputs
  const float* ea = nullptr;          // a [rows][lde]
  const float* eu = nullptr;          // u [rows][lde]
  int64_t lde = 0;
  const float* row_scale = nullptr;   // g per row
  float* row_partial = nullptr;       // [rows][N / 256]
  int64_t lo_off = 0;                 // EPI_DGRAD: also store the low halves (v - bf16(v)) at C + lo_off / C2 + lo_off
  // second K pass (hi/lo operand splitting): when nonzero, the K range is run twice, the second
  // time with A and B displaced by these element offsets, accumulating into the same tile
  int64_t a_seg_shift = 0, b_seg_shift = 0;
  // B stored k-major ([K][N] rows, N contiguous; bf16 grouped GEMMs with EPI_STORE / EPI_DGRAD):
  // the weights as they are, read through transposing LDS reads instead of a transposed copy.
  // K rows >= b_split (when nonzero) come from B2, row k - b_split.
  int32_t b_kmajor = 0;
  int32_t b_split = 0;
  int32_t two_pass = 0;
  int32_t c_accumulate = 0;           // fp32 outputs of the MXFP8 GEMM: C += product
};

// Persistent launch of the grouped GEMMs (gemm.hip, gemm_mx.hip): tickets, 8 int32 counters in device
// memory (zeroed by the launch); budget, the workgroup budget word (nullable, read only); force:
// always persistent, otherwise only where the launch holds at least kPersistMinTilesPerWg tiles
// per workgroup (its upper bound of tiles, known on the host).
struct Persist {
  int32_t* tickets = nullptr;
  const int32_t* budget = nullptr;
  bool force = false;
  bool budget_indirect = false;   // budget points at the address of the word (MOE_FLAG_CU_BUDGET_INDIRECT)
};
// The persistent GEMMs' budget control of a call: the workspace's budget word, or with
// MOE_FLAG_CU_BUDGET_INDIRECT its address slot; none without MOE_FLAG_CU_BUDGET. wsblock: the
// workspace's first (error-word) block.
inline void set_budget(Persist& pc, int32_t flags, char* wsblock) {
  pc.budget = nullptr;
  pc.budget_indirect = (flags & MOE_FLAG_CU_BUDGET_INDIRECT) != 0;
  if (flags & MOE_FLAG_CU_BUDGET)
    pc.budget = (const int32_t*)(wsblock + (pc.budget_indirect ? MOE_WS_CU_BUDGET_PTR_OFFSET : MOE_WS_CU_BUDGET_OFFSET));
}
constexpr int kPersistMinTilesPerWg = 12;
// Grid of the persistent form for a launch of at most nb tiles: nw workgroups, or nw = 0 for the
// per-tile form (pc null, or too few tiles per workgroup and not forced).
int persistent_grid(int64_t nb, const Persist* pc, int64_t& nw);
int launch_zero_tickets(int32_t* tickets, hipStream_t s);
// pc: may run as the persistent kernel (see Persist).
int launch_gemm_bf16(const GemmArgs& a, const Grouped& g, Epi epi, hipStream_t s, const Persist* pc = nullptr);
int launch_gemm_bf16_kgroup(const GemmArgs& a, int groups, hipStream_t s, const Persist* pc = nullptr);
int gemm_tile_cols(Epi epi);
int launch_chunk_tables(const int32_t* offsets, int E, int n, int b, int C, int32_t* ctile, int32_t* crow,
                        hipStream_t s);
// pc: may run as the persistent kernel, as launch_gemm_bf16.
int launch_gemm_mx(const GemmArgs& a, const uint8_t* a_sc, const uint8_t* b_sc, const uint8_t* b2_sc,
                   int64_t sc_group_stride, uint8_t* h_sc, const Grouped& g, Epi epi, hipStream_t s,
                   const Persist* pc = nullptr);
// K-grouped MXFP8 weight gradients: A [M][lda] and B [N][ldb] E4M3 along K with scales
// [M][lda / 32], [N][ldb / 32]; group g contracts k in [k_off[g], k_off[g+1]) (multiples of 128);
// fp32 output as launch_gemm_bf16_kgroup.
int launch_gemm_mx_kgroup(const GemmArgs& a, const uint8_t* a_sc, const uint8_t* b_sc, int groups, hipStream_t s,
                         const Persist* pc = nullptr);
// h [n4 * 4] bf16 = SiLU(a) u from fp32 a, u, with the SwiGLU GEMM epilogue's arithmetic.
int launch_swiglu_rows(const float* a, const float* u, int64_t n4, uint16_t* h, hipStream_t s);
// The same under MXFP8: nblk blocks of 32 along I -> E4M3 codes q and E8M0 scales sc, as the
// MXFP8 SwiGLU GEMM epilogue quantises h.
int launch_swiglu_rows_mx(const float* a, const float* u, int64_t nblk, uint8_t* q, uint8_t* sc, hipStream_t s);
int launch_gemm_f32(const GemmArgs& a, const Grouped& g, Epi epi, hipStream_t s);

}  // namespace moe

#define MOE_LAUNCH_CHECK()                                  \
  do {                                                      \
    hipError_t e_ = hipGetLastError();                      \
    if (e_ != hipSuccess) return MOE_ERR_HIP;               \
  } while (0)
