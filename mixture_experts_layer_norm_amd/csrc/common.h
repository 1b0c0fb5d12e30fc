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
typedef uint16_t bf16_t;   // raw bf16 bits in memory

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint16_t f2bf(float f) {
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
constexpr int kGemmBM = 128;                 // rows per grouped-GEMM m-tile
constexpr int kErrOffset = 0;                // sticky error word (int32)

struct WsLayout {
  size_t err;              // int32 error word
  size_t ctrl;             // pipeline counters / flags
  size_t blk_hist;         // [nblk][E] int32
  size_t tile_off;         // [E+1] int32  m-tile prefix for kGemmBM
  size_t x_slot;           // dispatched rows
  size_t x_slot_sc;        // MX scales of x_slot
  size_t h;                // gated activation
  size_t h_sc;             // MX scales of h
  size_t y_routes;         // per-route outputs [T*K][D]
  size_t sh_h;             // shared expert activation [T][I_s]
  size_t sh_out;           // shared expert output [T][D]
  size_t bwd;              // backward scratch start
  size_t total;
  int64_t nblk;            // histogram blocks
  int64_t ring_rows;       // rows of x_slot / h held (chunk * stages, or T*K)
  int64_t chunk;           // rows per chunk
  int32_t stages;          // ring stages (1 when one chunk holds everything)
};

size_t elt_bytes(int dtype);
WsLayout ws_layout(const moe_problem& p);
int validate_problem(const moe_problem* p);

// ---------------------------------------------------------------------------------------------
// launchers (each returns 0 or a moe_status; all enqueue on `s`)
// ---------------------------------------------------------------------------------------------
int launch_route_topk(const float* logits, int32_t* idx, float* w, int T, int E, int K, hipStream_t s);
int launch_schedule(const int32_t* idx, int T, int K, int E, int32_t* counts, int32_t* offsets,
                    int32_t* perm, int32_t* inv_perm, int32_t* blk_hist, int32_t* tile_off,
                    int32_t* err, hipStream_t s);

int launch_dispatch(const void* x, int dtype, const int32_t* perm, int K, int D, int64_t begin,
                    int64_t count, void* x_slot, uint8_t* x_slot_sc, hipStream_t s);
int launch_combine(const void* y_routes, const void* shared_out, const float* topk_w, void* out,
                   int T, int K, int D, int dtype, hipStream_t s);
int launch_quantize_mx(const uint16_t* src, int64_t rows, int cols, uint8_t* q, uint8_t* sc,
                       hipStream_t s);

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

enum Epi { EPI_SWIGLU = 0, EPI_STORE = 1 };

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
};

int launch_gemm_bf16(const GemmArgs& a, const Grouped& g, Epi epi, hipStream_t s);
int launch_gemm_f32(const GemmArgs& a, const Grouped& g, Epi epi, hipStream_t s);

}  // namespace moe

#define MOE_LAUNCH_CHECK()                                  \
  do {                                                      \
    hipError_t e_ = hipGetLastError();                      \
    if (e_ != hipSuccess) return MOE_ERR_HIP;               \
  } while (0)
