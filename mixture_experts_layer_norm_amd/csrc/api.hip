// C ABI entry points: host-side validation, workspace carve-up and kernel orchestration.
// Every entry point checks its arguments before enqueuing anything and never synchronises.
#include <string.h>

#include <algorithm>

#include "common.h"

namespace moe {

size_t elt_bytes(int dtype) { return dtype == MOE_F32 ? 4 : 2; }

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static constexpr uint32_t kKnownFlags = MOE_FLAG_FUSED_GATHER | MOE_FLAG_PERSISTENT | MOE_FLAG_BWD_DGRAD_ONE_PASS |
                                        MOE_FLAG_BWD_WGRAD_LO_MXFP8 | MOE_FLAG_PERSISTENT_GEMM | MOE_FLAG_CU_BUDGET |
                                        MOE_FLAG_ROUTER_BWD_DENSE | MOE_FLAG_DISPATCH_COPY |
                                        MOE_FLAG_CU_BUDGET_INDIRECT;

// Extra checks of the entry points that route tokens (top-k over the E experts).
int validate_routing(const moe_problem* p) {
  int st = validate_problem(p);
  if (st) return st;
  if (p->K > p->E) return MOE_ERR_INVALID_ARG;
  if (p->K > 64) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int validate_problem(const moe_problem* p) {
  if (!p) return MOE_ERR_INVALID_ARG;
  if (p->T < 1 || p->D < 1 || p->I < 1 || p->E < 1 || p->K < 1 || p->I_shared < 0) return MOE_ERR_INVALID_ARG;
  if (p->dtype != MOE_F32 && p->dtype != MOE_BF16 && p->dtype != MOE_MXFP8) return MOE_ERR_INVALID_ARG;
  if (p->chunk_rows < 0 || p->ring_stages < 0 || p->ring_stages == 1 || p->ring_stages == 2) return MOE_ERR_INVALID_ARG;
  if ((uint32_t)p->flags & ~kKnownFlags) return MOE_ERR_INVALID_ARG;
  if ((p->flags & MOE_FLAG_CU_BUDGET) && !(p->flags & MOE_FLAG_PERSISTENT_GEMM)) return MOE_ERR_INVALID_ARG;
  if ((p->flags & MOE_FLAG_CU_BUDGET_INDIRECT) && !(p->flags & MOE_FLAG_CU_BUDGET)) return MOE_ERR_INVALID_ARG;
  if ((p->flags & MOE_FLAG_FUSED_GATHER) && (p->flags & MOE_FLAG_DISPATCH_COPY)) return MOE_ERR_INVALID_ARG;
  if (p->E > 1024) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)p->T * p->K >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  if (p->dtype == MOE_F32) {
    if (p->D % 4) return MOE_ERR_UNSUPPORTED;
  } else {
    if (p->D % 128 || p->I % 128 || p->I_shared % 128) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

WsLayout ws_layout(const moe_problem& p) {
  WsLayout L{};
  const int64_t n = (int64_t)p.T * p.K;
  const size_t act = elt_bytes(p.dtype);
  const bool mx = p.dtype == MOE_MXFP8;
  L.nblk = (n + kRouteRowsPerBlock - 1) / kRouteRowsPerBlock;
  L.chunk = n;
  L.stages = 1;
  L.chunks = 1;
  L.ring_rows = n;
  L.chunked = p.chunk_rows > 0 && (p.dtype == MOE_BF16 || p.dtype == MOE_MXFP8);
  if (L.chunked) {
    // b: multiple of 256 rows, at least n/1024 (at most 1024 chunks), at most n rounded up
    const int64_t nr = (n + 255) / 256 * 256;
    int64_t b = ((int64_t)p.chunk_rows + 255) / 256 * 256;
    const int64_t bmin = ((n + 1023) / 1024 + 255) / 256 * 256;
    b = b < bmin ? bmin : b;
    b = b > nr ? nr : b;
    L.chunk = b;
    L.chunks = (int32_t)((n + b - 1) / b);
    L.stages = p.ring_stages ? p.ring_stages : 3;
    L.ring_rows = (int64_t)(L.stages < L.chunks ? L.stages : L.chunks) * b;
  }
  size_t o = 0;
  L.err = o; o += 256;
  L.ctrl = o; o += 4096;
  L.blk_hist = o; o = align256(o + (size_t)L.nblk * p.E * 4);
  L.tile_off = o; o = align256(o + (size_t)(p.E + 1) * 4);
  L.grp_clean = o; o = align256(o + (size_t)(p.E + 1) * 4);
  L.grp_poff = o; o = align256(o + (size_t)(p.E + 1) * 4);
  // x rows for GEMM1: under MOE_FLAG_DISPATCH_COPY the dispatched slot rows (all of them, or a
  // ring of chunk stages); otherwise BF16 GEMM1 reads x itself through the schedule (no buffer) and
  // MXFP8 reads its T token rows quantised once. The MXFP8 expert-level forward quantises its
  // slot rows here too (up to T K of them).
  const bool copy = mx || (p.flags & MOE_FLAG_DISPATCH_COPY);
  const int64_t xrows = mx && L.ring_rows < p.T ? p.T : L.ring_rows;
  L.x_slot = o; o = align256(o + (copy ? (size_t)xrows * p.D * (mx ? 1 : act) : 0));
  L.x_slot_sc = o; o = align256(o + (mx ? (size_t)xrows * (p.D / 32) : 0));
  L.h = o; o = align256(o + (size_t)L.ring_rows * p.I * (mx ? 1 : act));
  L.h_sc = o; o = align256(o + (mx ? (size_t)L.ring_rows * (p.I / 32) : 0));
  L.y_routes = o; o = align256(o + (size_t)n * p.D * act);
  L.sh_h = o; o = align256(o + (size_t)p.T * p.I_shared * act);
  L.sh_out = o; o = align256(o + (p.I_shared > 0 ? (size_t)p.T * p.D * act : 0));
  L.chunk_tiles = o; o = align256(o + (L.chunked ? (size_t)L.chunks * (p.E + 1) * 4 : 0));
  L.chunk_rowoff = o; o = align256(o + (L.chunked ? (size_t)L.chunks * (p.E + 1) * 4 : 0));
  L.bwd = o;
  L.total = o;
  return L;
}

static bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15) == 0; }

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_MISALIGNED: return "MOE_ERR_MISALIGNED";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

int moe_workspace_size(const moe_problem* p, size_t* bytes) {
  int st = validate_problem(p);
  if (st) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = ws_layout(*p).total;
  return MOE_OK;
}

int moe_route_topk(const moe_problem* p, const float* logits, int32_t* topk_idx, float* topk_w,
                   hipStream_t stream) {
  int st = validate_routing(p);
  if (st) return st;
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
  return launch_route_topk(logits, topk_idx, topk_w, p->T, p->E, p->K, stream);
}

}  // extern "C"

namespace moe {

// Router GEMM split along D into S K-groups so that the T/256 x E/256 output tiles fill the
// chip: about 256 workgroups, at least one 64-wide K slice per group, at most 16 groups.
struct RouteGemmWs {
  int S;
  size_t err, k_off, part, total;
};

static RouteGemmWs route_gemm_ws(const moe_problem& p) {
  RouteGemmWs w{};
  const int mtn = (p.T + kGemmBM - 1) / kGemmBM, ntn = (p.E + 255) / 256, nkt = p.D / 64;
  const int want = (256 + mtn * ntn - 1) / (mtn * ntn);
  w.S = std::max(1, std::min(want, std::min(16, nkt)));
  w.err = 0;
  w.k_off = 256;
  w.part = 512;
  w.total = w.part + (((size_t)w.S * p.T * p.E * 4 + 255) / 256) * 256;
  return w;
}

__global__ void route_k_off_kernel(int S, int nkt, int32_t* k_off) {
  const int g = threadIdx.x;
  if (g <= S) k_off[g] = (int)(((int64_t)g * nkt / S) * 64);
}

}  // namespace moe

extern "C" {

int moe_route_gemm_workspace_size(const moe_problem* p, size_t* bytes) {
  int st = validate_routing(p);
  if (st) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = route_gemm_ws(*p).total;
  return MOE_OK;
}

int moe_route_gemm(const moe_problem* p, const void* x, const void* w_router, float* logits, int32_t* topk_idx,
                   float* topk_w, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = validate_routing(p);
  if (st) return st;
  if (p->dtype == MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (!x || !w_router || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_MISALIGNED;
  const RouteGemmWs W = route_gemm_ws(*p);
  if (!ws || ws_bytes < W.total) return MOE_ERR_WORKSPACE;
  char* wsb = (char*)ws;
  int32_t* k_off = (int32_t*)(wsb + W.k_off);
  float* part = (float*)(wsb + W.part);
  hipLaunchKernelGGL(route_k_off_kernel, dim3(1), dim3(64), 0, stream, W.S, p->D / 64, k_off);
  MOE_LAUNCH_CHECK();
  // partial logits: part[s][t][e] = sum over k in group s of x[t][k] w_router[e][k] (fp32)
  GemmArgs g;
  g.A = x; g.lda = p->D; g.B = w_router; g.ldb = p->D;
  g.M = p->T; g.N = p->E; g.K = p->D;
  g.C = part; g.ldc = p->E; g.c_group_stride = (int64_t)p->T * p->E;
  g.k_off = k_off;
  if ((st = launch_gemm_bf16_kgroup(g, W.S, stream))) return st;
  return launch_route_topk_partials(part, W.S, (int64_t)p->T * p->E, logits, topk_idx, topk_w, p->T, p->E, p->K,
                                    stream);
}

static int schedule_into(const moe_problem* p, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                         int32_t* perm, int32_t* inv_perm, char* ws, hipStream_t stream) {
  WsLayout L = ws_layout(*p);
  return launch_schedule(topk_idx, p->T, p->K, p->E, counts, offsets, perm, inv_perm,
                         (int32_t*)(ws + L.blk_hist), (int32_t*)(ws + L.tile_off),
                         (int32_t*)(ws + L.err), stream);
}

int moe_schedule(const moe_problem* p, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                 int32_t* perm, int32_t* inv_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = validate_routing(p);
  if (st) return st;
  if (!topk_idx || !counts || !offsets || !perm || !inv_perm) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < ws_layout(*p).total) return MOE_ERR_WORKSPACE;
  return schedule_into(p, topk_idx, counts, offsets, perm, inv_perm, (char*)ws, stream);
}

int moe_dispatch(const moe_problem* p, const void* x, const int32_t* perm, int64_t slot_begin,
                 int64_t slot_count, void* x_slot, uint8_t* x_slot_scales, hipStream_t stream) {
  int st = validate_problem(p);
  if (st) return st;
  if (!x || !perm || !x_slot) return MOE_ERR_INVALID_ARG;
  const int64_t n = (int64_t)p->T * p->K;
  if (slot_begin < 0 || slot_count < 0 || slot_begin + slot_count > n) return MOE_ERR_INVALID_ARG;
  if ((p->dtype == MOE_MXFP8) != (x_slot_scales != nullptr)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(x_slot)) return MOE_ERR_MISALIGNED;
  return launch_dispatch(x, p->dtype, perm, p->K, p->D, slot_begin, slot_count, x_slot, x_slot_scales, stream);
}

int moe_dispatch_tokens(const moe_problem* p, const void* x, const int32_t* inv_perm, void* x_slot,
                        uint8_t* x_slot_scales, hipStream_t stream) {
  int st = validate_problem(p);
  if (st) return st;
  if (!x || !inv_perm || !x_slot) return MOE_ERR_INVALID_ARG;
  if ((p->dtype == MOE_MXFP8) != (x_slot_scales != nullptr)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(x_slot)) return MOE_ERR_MISALIGNED;
  return launch_dispatch_tokens(x, p->dtype, inv_perm, p->T, p->K, p->D, x_slot, x_slot_scales, stream);
}

int moe_combine(const moe_problem* p, const void* y_routes, const void* shared_out,
                const float* topk_w, void* out, hipStream_t stream) {
  int st = validate_problem(p);
  if (st) return st;
  if (!y_routes || !topk_w || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y_routes) || !aligned16(out) || (shared_out && !aligned16(shared_out))) return MOE_ERR_MISALIGNED;
  return launch_combine(y_routes, shared_out, topk_w, out, p->T, p->K, p->D,
                        p->dtype == MOE_F32 ? MOE_F32 : MOE_BF16, stream);
}

int moe_quantize_mx(const void* src_bf16, int64_t rows, int32_t cols, uint8_t* q, uint8_t* scales,
                    hipStream_t stream) {
  if (!src_bf16 || !q || !scales || rows < 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
  if (cols % 32) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(src_bf16) || !aligned16(q)) return MOE_ERR_MISALIGNED;
  return launch_quantize_mx((const uint16_t*)src_bf16, rows, cols, q, scales, stream);
}

// Expert FFN over grouped rows: h = SwiGLU(A), y = h W_down^T (optionally scattered).
static int expert_ffn(int dtype, const Grouped& grp, const void* A, int64_t lda, const int32_t* gather,
                      int gather_div, const void* wg, const void* wu, const void* wd, int D, int I,
                      int64_t w_stride_up, int64_t w_stride_down, void* h, void* y,
                      const int32_t* scatter, hipStream_t stream, hipEvent_t mid = nullptr,
                      const Persist* pc = nullptr) {
  GemmArgs g1;
  g1.A = A; g1.lda = lda; g1.a_gather = gather; g1.a_div = gather_div;
  g1.B = wg; g1.B2 = wu; g1.ldb = D; g1.b_group_stride = w_stride_up;
  g1.N = I; g1.K = D; g1.C = h; g1.ldc = I;
  GemmArgs g2;
  g2.A = h; g2.lda = I;
  g2.B = wd; g2.ldb = I; g2.b_group_stride = w_stride_down;
  g2.N = D; g2.K = I; g2.C = y; g2.ldc = D; g2.c_scatter = scatter;
  int st;
  if (dtype == MOE_F32) {
    g1.c_f32 = 1; g2.c_f32 = 1;
    st = launch_gemm_f32(g1, grp, EPI_SWIGLU, stream);
    if (st) return st;
    if (mid && hipEventRecord(mid, stream) != hipSuccess) return MOE_ERR_HIP;
    return launch_gemm_f32(g2, grp, EPI_STORE, stream);
  }
  st = launch_gemm_bf16(g1, grp, EPI_SWIGLU, stream, pc);
  if (st) return st;
  if (mid && hipEventRecord(mid, stream) != hipSuccess) return MOE_ERR_HIP;
  return launch_gemm_bf16(g2, grp, EPI_STORE, stream, pc);
}

}  // extern "C"

// The forward, in order on `stream`. `ev` (moe_forward_stages) marks the stage boundaries.
static int forward_impl(const moe_problem* p, const void* x, const float* logits, const moe_weights* w,
                        void* out, const moe_routing* r, void* y_routes, void* shared_out, void* ws,
                        size_t ws_bytes, hipEvent_t* ev, hipStream_t stream, float* act_a = nullptr,
                        float* act_u = nullptr, const moe_lanes* lanes = nullptr) {
  int st = validate_routing(p);
  if (st) return st;
  static_assert(kTicketsOffset + 32 * MOE_MAX_LANES <= 256, "per-lane ticket counters in the error word's block");
  if (lanes) {
    if (lanes->count < 1 || lanes->count >= MOE_MAX_LANES || !lanes->streams || !lanes->events) return MOE_ERR_INVALID_ARG;
    const int S = p->ring_stages ? p->ring_stages : 3;
    for (int l = 0; l < lanes->count; ++l)
      if (!lanes->streams[l]) return MOE_ERR_INVALID_ARG;
    for (int e = 0; e < S + 1 + lanes->count; ++e)
      if (!lanes->events[e]) return MOE_ERR_INVALID_ARG;
  }
  const bool keep = act_a || act_u;
  if (keep && (!act_a || !act_u)) return MOE_ERR_INVALID_ARG;
  if (keep && (p->dtype == MOE_F32 || p->chunk_rows > 0)) return MOE_ERR_UNSUPPORTED;
  if (keep && (!aligned16(act_a) || !aligned16(act_u))) return MOE_ERR_MISALIGNED;
  if (!x || !logits || !w || !out || !r) return MOE_ERR_INVALID_ARG;
  if (!r->topk_idx || !r->topk_w || !r->counts || !r->offsets || !r->perm || !r->inv_perm) return MOE_ERR_INVALID_ARG;
  if (!w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_INVALID_ARG;
  if (p->I_shared > 0 && (!w->ws_gate || !w->ws_up || !w->ws_down)) return MOE_ERR_INVALID_ARG;
  const bool mx = p->dtype == MOE_MXFP8;
  if (mx && (!w->sc_gate || !w->sc_up || !w->sc_down)) return MOE_ERR_INVALID_ARG;
  if (p->flags & MOE_FLAG_PERSISTENT) return MOE_ERR_UNSUPPORTED;   // persistent chunk kernel is switched off
  if ((p->flags & MOE_FLAG_PERSISTENT_GEMM) && p->dtype == MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (p->chunk_rows > 0 && p->dtype == MOE_F32) return MOE_ERR_UNSUPPORTED;
  WsLayout L = ws_layout(*p);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(out) || !aligned16(ws) || (y_routes && !aligned16(y_routes)) ||
      (shared_out && !aligned16(shared_out)))
    return MOE_ERR_MISALIGNED;
  char* wsb = (char*)ws;
  const int64_t n = (int64_t)p->T * p->K;
  void* yr = y_routes ? y_routes : (void*)(wsb + L.y_routes);
  void* sho = p->I_shared > 0 ? (shared_out ? shared_out : (void*)(wsb + L.sh_out)) : nullptr;
  // persistent GEMMs (BF16 and MXFP8): ticket counters and the workgroup budget word in the error
  // word's block; taken where a launch has enough tiles per workgroup, always with the flag
  Persist pcs;
  const Persist* pc = nullptr;
  if (p->dtype != MOE_F32) {
    pcs.tickets = (int32_t*)(wsb + L.err + kTicketsOffset);
    pcs.force = (p->flags & MOE_FLAG_PERSISTENT_GEMM) != 0;
    set_budget(pcs, p->flags, wsb + L.err);
    pc = &pcs;
  }

#define MOE_MARK(i) \
  do { if (ev && hipEventRecord(ev[i], stream) != hipSuccess) return MOE_ERR_HIP; } while (0)
  MOE_MARK(MOE_STAGE_ROUTE);
  st = launch_route_topk(logits, r->topk_idx, r->topk_w, p->T, p->E, p->K, stream);
  if (st) return st;
  MOE_MARK(MOE_STAGE_SCHEDULE);
  st = schedule_into(p, r->topk_idx, r->counts, r->offsets, r->perm, r->inv_perm, wsb, stream);
  if (st) return st;

  // shared expert first: it does not depend on the schedule (with lanes: on lane 0 after the fork)
  MOE_MARK(MOE_STAGE_SHARED);
  auto shared_expert = [&](hipStream_t s_, const Persist* pc_) -> int {
    if (p->I_shared <= 0) return MOE_OK;
    Grouped gs;
    gs.M = p->T;
    return expert_ffn(p->dtype, gs, x, p->D, nullptr, 1, w->ws_gate, w->ws_up, w->ws_down, p->D, p->I_shared,
                      0, 0, wsb + L.sh_h, sho, nullptr, s_, nullptr, pc_);
  };
  const bool laned = lanes && L.chunked;
  if (!laned && (st = shared_expert(stream, pc))) return st;

  Grouped gr;
  gr.row_off = r->offsets;
  gr.tile_off = (const int32_t*)(wsb + L.tile_off);
  gr.groups = p->E;
  gr.max_mtiles = (n + kGemmBM - 1) / kGemmBM + p->E;
  if (L.chunked) {
    // Chunks of b routed slots through a ring of S stages, each carried through dispatch, up/gate
    // and down before the next (the Notes' "Granularity as a tunable" and "A ring buffer instead
    // of a host round-trip"); all tile bookkeeping is on the device (no host synchronisation).
    // Slot j of chunk c lives in ring row (c % S) b + (j - c b): each chunk's operands are
    // addressed through a base pointer displaced by (c % S) b - c b rows, so the kernels index
    // them by slot as in the unchunked path and every output tile is the same workgroup sum.
    const int64_t b = L.chunk;
    const int C = L.chunks, S = L.stages;
    int32_t* ctile = (int32_t*)(wsb + L.chunk_tiles);
    int32_t* crow = (int32_t*)(wsb + L.chunk_rowoff);
    st = launch_chunk_tables(r->offsets, p->E, (int)n, (int)b, C, ctile, crow, stream);
    if (st) return st;
    // Lanes: chunk c on lane c % NLn (lane 0 = `stream`), each lane with ticket counters of its
    // own; events[0 .. S-1] hand a ring stage from the lane that used it last to the next one,
    // events[S] forks the lanes, events[S + l] (l >= 1) joins lane l back.
    const int NLn = laned ? lanes->count + 1 : 1;
    hipStream_t ls[MOE_MAX_LANES];
    Persist lpc[MOE_MAX_LANES];
    ls[0] = stream;
    for (int l = 0; l < NLn; ++l) {
      if (l > 0) ls[l] = lanes->streams[l - 1];
      lpc[l] = pcs;
      if (pcs.tickets) lpc[l].tickets = pcs.tickets + 8 * l;
    }
    // Chunks read x through the schedule (the ring then holds only h): BF16 x as it is, MXFP8 its
    // T token rows quantised once up front (on `stream`, before the lanes fork). Under
    // MOE_FLAG_DISPATCH_COPY each chunk's rows are dispatched (MXFP8: quantising) into the ring.
    const bool gather_x = !(p->flags & MOE_FLAG_DISPATCH_COPY);
    const int64_t xrow = mx ? p->D : (int64_t)p->D * 2, hrow = mx ? p->I : (int64_t)p->I * 2;   // bytes per row
    uint8_t* xr = (uint8_t*)(wsb + L.x_slot);
    uint8_t* hr = (uint8_t*)(wsb + L.h);
    uint8_t* xs = (uint8_t*)(wsb + L.x_slot_sc);
    uint8_t* hs = (uint8_t*)(wsb + L.h_sc);
    auto quantize_tokens = [&]() -> int {
      return (mx && gather_x) ? launch_quantize_mx((const uint16_t*)x, p->T, p->D, xr, xs, stream) : MOE_OK;
    };
    if (NLn > 1) {
      if ((st = quantize_tokens())) return st;
      if (hipEventRecord(lanes->events[S], stream) != hipSuccess) return MOE_ERR_HIP;
      for (int l = 1; l < NLn; ++l)
        if (hipStreamWaitEvent(ls[l], lanes->events[S], 0) != hipSuccess) return MOE_ERR_HIP;
    }
    if (laned && (st = shared_expert(stream, pc))) return st;
    MOE_MARK(MOE_STAGE_DISPATCH);
    if (NLn == 1 && (st = quantize_tokens())) return st;
    for (int c = 0; c < C; ++c) {
      const int64_t c0 = c * b, rows = (n - c0) < b ? (n - c0) : b;
      const int64_t stage = (int64_t)(c % S) * b, shift = stage - c0;   // slot index -> ring row
      const int lane = c % NLn;
      hipStream_t cs = ls[lane];
      // A chunk's tile bound counts a partial tile per expert, so with many experts every chunk
      // passes the persistent rule; below 4 full m-tiles per chunk the per-tile form measured
      // faster (DSV3 shape with 3 extra lanes, b = 512: 12.7 vs 13.6 ms; from b = 2048 on the
      // persistent form is faster, 9.84 vs 10.47 ms at b = 32768).
      const Persist* cpc = (pc && (pcs.force || b >= 4 * kGemmBM)) ? &lpc[lane] : nullptr;
      // ring stage c % S was last read by chunk c - S (its up/gate and down): on another lane, wait
      if (NLn > 1 && c >= S && (c - S) % NLn != lane && hipStreamWaitEvent(cs, lanes->events[c % S], 0) != hipSuccess)
        return MOE_ERR_HIP;
      if (!gather_x) {
        st = launch_dispatch(x, p->dtype, r->perm, p->K, p->D, c0, rows, xr + stage * xrow,
                             mx ? xs + stage * (p->D / 32) : nullptr, cs);
        if (st) return st;
      }
      Grouped gc;
      gc.row_off = crow + (int64_t)c * (p->E + 1);
      gc.tile_off = ctile + (int64_t)c * (p->E + 1);
      gc.groups = p->E;
      gc.max_mtiles = (rows + kGemmBM - 1) / kGemmBM + p->E;
      if (mx) {
        GemmArgs g1;
        g1.A = gather_x ? xr : xr + shift * xrow; g1.lda = p->D; g1.B = w->w_gate; g1.B2 = w->w_up; g1.ldb = p->D;
        g1.b_group_stride = (int64_t)p->I * p->D; g1.N = p->I; g1.K = p->D; g1.C = hr + shift * hrow; g1.ldc = p->I;
        if (gather_x) { g1.a_gather = r->perm; g1.a_div = p->K; }
        st = launch_gemm_mx(g1, gather_x ? xs : xs + shift * (p->D / 32), w->sc_gate, w->sc_up,
                            (int64_t)p->I * (p->D / 32), hs + shift * (p->I / 32), gc, EPI_SWIGLU, cs, cpc);
        if (st) return st;
        GemmArgs g2;
        g2.A = hr + shift * hrow; g2.lda = p->I; g2.B = w->w_down; g2.ldb = p->I;
        g2.b_group_stride = (int64_t)p->D * p->I; g2.N = p->D; g2.K = p->I; g2.C = yr; g2.ldc = p->D;
        g2.c_scatter = r->perm;
        st = launch_gemm_mx(g2, hs + shift * (p->I / 32), w->sc_down, nullptr, (int64_t)p->D * (p->I / 32), nullptr,
                            gc, EPI_STORE, cs, cpc);
      } else {
        st = expert_ffn(p->dtype, gc, gather_x ? x : (const void*)(xr + shift * xrow), p->D,
                        gather_x ? r->perm : nullptr, gather_x ? p->K : 1, w->w_gate, w->w_up, w->w_down, p->D,
                        p->I, (int64_t)p->I * p->D, (int64_t)p->D * p->I, hr + shift * hrow, yr, r->perm, cs,
                        nullptr, cpc);
      }
      if (st) return st;
      if (NLn > 1 && c + S < C && (c + S) % NLn != lane && hipEventRecord(lanes->events[c % S], cs) != hipSuccess)
        return MOE_ERR_HIP;
    }
    for (int l = 1; l < NLn; ++l) {
      if (hipEventRecord(lanes->events[S + l], ls[l]) != hipSuccess) return MOE_ERR_HIP;
      if (hipStreamWaitEvent(stream, lanes->events[S + l], 0) != hipSuccess) return MOE_ERR_HIP;
    }
    MOE_MARK(MOE_STAGE_UP_GATE);
    MOE_MARK(MOE_STAGE_DOWN);
    MOE_MARK(MOE_STAGE_COMBINE);
    st = launch_combine(yr, sho, r->topk_w, out, p->T, p->K, p->D, p->dtype, stream);
    if (st) return st;
    MOE_MARK(MOE_STAGE_COUNT);
    return MOE_OK;
  }
  MOE_MARK(MOE_STAGE_DISPATCH);
  if (mx) {
    // x quantised (its token rows once, or per-slot copies under MOE_FLAG_DISPATCH_COPY), then the
    // two block-scaled grouped GEMMs (h quantised in the SwiGLU epilogue)
    uint8_t* xq = (uint8_t*)(wsb + L.x_slot);
    uint8_t* xs = (uint8_t*)(wsb + L.x_slot_sc);
    uint8_t* hq = (uint8_t*)(wsb + L.h);
    uint8_t* hs = (uint8_t*)(wsb + L.h_sc);
    // the T token rows quantised once, read by GEMM1 through the schedule (row j = token
    // perm[j] / K); under MOE_FLAG_DISPATCH_COPY quantised into per-slot copies instead
    const bool gather = !(p->flags & MOE_FLAG_DISPATCH_COPY);
    st = gather ? launch_quantize_mx((const uint16_t*)x, p->T, p->D, xq, xs, stream)
                : launch_dispatch_tokens(x, MOE_MXFP8, r->inv_perm, p->T, p->K, p->D, xq, xs, stream);
    if (st) return st;
    MOE_MARK(MOE_STAGE_UP_GATE);
    GemmArgs g1;
    g1.A = xq; g1.lda = p->D; g1.B = w->w_gate; g1.B2 = w->w_up; g1.ldb = p->D;
    if (gather) { g1.a_gather = r->perm; g1.a_div = p->K; }
    g1.b_group_stride = (int64_t)p->I * p->D; g1.N = p->I; g1.K = p->D; g1.C = hq; g1.ldc = p->I;
    if (keep) {
      // a, u to the caller in fp32 (the backward's replay GEMM), h quantised from them
      g1.C = act_a; g1.C2 = act_u;
      st = launch_gemm_mx(g1, xs, w->sc_gate, w->sc_up, (int64_t)p->I * (p->D / 32), nullptr, gr, EPI_SAVE_AU, stream, pc);
      if (st) return st;
      st = launch_swiglu_rows_mx(act_a, act_u, n * (p->I / 32), hq, hs, stream);
    } else {
      st = launch_gemm_mx(g1, xs, w->sc_gate, w->sc_up, (int64_t)p->I * (p->D / 32), hs, gr, EPI_SWIGLU, stream, pc);
    }
    if (st) return st;
    MOE_MARK(MOE_STAGE_DOWN);
    GemmArgs g2;
    g2.A = hq; g2.lda = p->I; g2.B = w->w_down; g2.ldb = p->I; g2.b_group_stride = (int64_t)p->D * p->I;
    g2.N = p->D; g2.K = p->I; g2.C = yr; g2.ldc = p->D; g2.c_scatter = r->perm;
    st = launch_gemm_mx(g2, hs, w->sc_down, nullptr, (int64_t)p->D * (p->I / 32), nullptr, gr, EPI_STORE, stream, pc);
    if (st) return st;
  } else {
    // GEMM1 reads x rows through the schedule (row j = x[perm[j] / K]) unless the slot copy is asked for
    const void* A = x;
    const int32_t* gather = r->perm;
    if (p->flags & MOE_FLAG_DISPATCH_COPY) {
      st = launch_dispatch_tokens(x, p->dtype, r->inv_perm, p->T, p->K, p->D, wsb + L.x_slot, nullptr, stream);
      if (st) return st;
      A = wsb + L.x_slot;
      gather = nullptr;
    }
    MOE_MARK(MOE_STAGE_UP_GATE);
    if (keep) {
      // a, u to the caller in fp32 (the backward's replay GEMM, in slot order), h from them, then down
      GemmArgs g1;
      g1.A = A; g1.lda = p->D; g1.a_gather = gather; g1.a_div = p->K;
      g1.B = w->w_gate; g1.B2 = w->w_up; g1.ldb = p->D; g1.b_group_stride = (int64_t)p->I * p->D;
      g1.N = p->I; g1.K = p->D; g1.C = act_a; g1.C2 = act_u; g1.ldc = p->I;
      if ((st = launch_gemm_bf16(g1, gr, EPI_SAVE_AU, stream))) return st;
      if ((st = launch_swiglu_rows(act_a, act_u, n * p->I / 4, (uint16_t*)(wsb + L.h), stream))) return st;
      GemmArgs g2;
      g2.A = wsb + L.h; g2.lda = p->I; g2.B = w->w_down; g2.ldb = p->I; g2.b_group_stride = (int64_t)p->D * p->I;
      g2.N = p->D; g2.K = p->I; g2.C = yr; g2.ldc = p->D; g2.c_scatter = r->perm;
      if ((st = launch_gemm_bf16(g2, gr, EPI_STORE, stream, pc))) return st;
    } else {
      st = expert_ffn(p->dtype, gr, A, p->D, gather, p->K, w->w_gate, w->w_up, w->w_down, p->D, p->I,
                      (int64_t)p->I * p->D, (int64_t)p->D * p->I, wsb + L.h, yr, r->perm, stream,
                      ev ? ev[MOE_STAGE_DOWN] : nullptr, pc);
      if (st) return st;
    }
  }
  MOE_MARK(MOE_STAGE_COMBINE);
  st = launch_combine(yr, sho, r->topk_w, out, p->T, p->K, p->D, p->dtype, stream);
  if (st) return st;
  MOE_MARK(MOE_STAGE_COUNT);
#undef MOE_MARK
  return MOE_OK;
}

extern "C" {

int moe_forward(const moe_problem* p, const void* x, const float* logits, const moe_weights* w,
                void* out, const moe_routing* r, void* y_routes, void* shared_out, void* ws,
                size_t ws_bytes, hipStream_t stream) {
  return forward_impl(p, x, logits, w, out, r, y_routes, shared_out, ws, ws_bytes, nullptr, stream);
}

int moe_forward_keep(const moe_problem* p, const void* x, const float* logits, const moe_weights* w, void* out,
                     const moe_routing* r, void* y_routes, void* shared_out, float* act_a, float* act_u, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  if (!act_a || !act_u) return MOE_ERR_INVALID_ARG;
  return forward_impl(p, x, logits, w, out, r, y_routes, shared_out, ws, ws_bytes, nullptr, stream, act_a, act_u);
}

int moe_forward_stages(const moe_problem* p, const void* x, const float* logits, const moe_weights* w,
                       void* out, const moe_routing* r, void* y_routes, void* shared_out, void* ws,
                       size_t ws_bytes, hipEvent_t* ev, hipStream_t stream) {
  return forward_impl(p, x, logits, w, out, r, y_routes, shared_out, ws, ws_bytes, ev, stream);
}

int moe_forward_lanes(const moe_problem* p, const void* x, const float* logits, const moe_weights* w, void* out,
                      const moe_routing* r, void* y_routes, void* shared_out, void* ws, size_t ws_bytes,
                      hipStream_t stream, const moe_lanes* lanes) {
  if (!lanes) return MOE_ERR_INVALID_ARG;
  return forward_impl(p, x, logits, w, out, r, y_routes, shared_out, ws, ws_bytes, nullptr, stream, nullptr,
                      nullptr, lanes);
}

}  // extern "C"
