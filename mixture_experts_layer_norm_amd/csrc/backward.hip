// Expert-level forward and the backward pass (host orchestration of the kernels).
//
// Backward of E(x) = W_down (SiLU(a) (*) u), a = W_gate x, u = W_up x, for slot rows weighted by
// g (each slot enters the layer output as g * E(x)), following the sparsenotes page
// "Mixture-of-Kittens: MoE Megakernel for NVL72s":
//   * "A ring buffer instead of a host round-trip": a and u are recomputed (replayed) from the
//     slot rows, unless the caller hands in the forward's kept fp32 a, u (the *_kept entry points,
//     filled by the *_keep forwards), which skips the replay GEMM;
//   * "The production details": the router-weight gradient dg = <h, dh'> with dh' = W_down^T dy,
//     so the down-projection output is never recomputed;
//   * "Pull dispatch, push combine": the backward reverse-combine gathers the output gradient
//     into slots (dy_slot[j] = dout[perm[j] / K]) and the reverse-dispatch sums each token's
//     slot gradients back (fixed order, no atomics).
// Steps per group of rows: replay (a, u in fp32); dgrad-down with the SwiGLU backward in its
// epilogue (da, du and per-tile <h, dh'> partials); dgrad-up over [da | du] with K = 2I (both
// read the weights in place, k-major); padded transposes of x, dy, g*h and [da | du]; K-grouped
// weight-gradient GEMMs.
// The weight-gradient operands that are not exact inputs (da, du, g*h) are carried as pairs of
// bf16 values hi + lo (lo = v - bf16(v)) and contracted in two K passes, so they lose ~2^-17
// relative instead of 2^-9: a weight gradient of an expert with a single slot is an outer
// product, and its largest elements would carry the whole 2^-9 rounding. dgrad-up does the same
// by default; with MOE_FLAG_BWD_DGRAD_ONE_PASS it contracts the bf16 da, du alone (every dx
// element sums 2I products with independent roundings, so the error stays within the BF16 bound;
// one K pass instead of two). x, dy and the weights are exact bf16 inputs.
#include <algorithm>

#include "common.h"
#include "mx_codec.h"

namespace moe {

static size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

struct BwdLayout {
  size_t err, offs, tile_off, poff, order, offs_s, tile_off_s, poff_s;
  size_t g_slot, dg_slot, x_slot, dy_slot, dx_slot, dx_sh;
  size_t act_a, act_u, dau, part, xT, dyT, ghT, dauT;
  size_t s_a, s_u, s_dau, s_part, s_xT, s_dyT, s_hT, s_dauT;
  // MXFP8 routed experts: E4M3 codes (q) and E8M0 scales (s) of every backward GEMM operand
  size_t mq_x, ms_x, mq_dy, ms_dy, m_dhp, mq_dau, ms_dau, mq_wdT, ms_wdT, mq_wguT, ms_wguT;
  size_t mq_xT, ms_xT, mq_gdyT, ms_gdyT, mq_hT, ms_hT, mq_dauT, ms_dauT;
  // fp32: dh', h, da, du of the routed rows and of the shared expert's rows
  size_t f_dh, f_h, f_da, f_du, sf_dh, sf_h, sf_da, sf_du;
  // BF16: the weight gradients' second K pass in MXFP8 (low halves and the exact operands, all
  // quantised along the slots), routed and shared
  size_t lq_dau, ls_dau, lq_gh, ls_gh, lq_x, ls_x, lq_dy, ls_dy;
  size_t slq_dau, sls_dau, slq_gh, sls_gh, slq_x, sls_x, slq_dy, sls_dy;
  size_t total;
  int64_t n, Spad, Tpad;
  int pad, pad_s;          // group alignment of the slot axis: routed, shared
  bool lo_mx, lo_mx_s;     // BF16 weight gradients' low-half pass in MXFP8: routed, shared
};

// Under MOE_FLAG_BWD_WGRAD_LO_MXFP8 the BF16 weight gradients take their low-half pass in MXFP8
// (a second, accumulating pass over the fp32 dW), where a group's K is long enough on average to
// repay reading and writing dW once more.
static bool wgrad_lo_mx(const moe_problem& p, int64_t rows, int64_t groups) {
  return (p.flags & MOE_FLAG_BWD_WGRAD_LO_MXFP8) && rows >= 4096 * groups;
}

// Workspace of the backward for up to n = T*K slot rows (bf16). kept: the caller hands in the
// routed a, u (the *_kept entry points), so no room is reserved for replaying them.
static BwdLayout bwd_layout(const moe_problem& p, bool kept = false) {
  BwdLayout L{};
  const int64_t n = (int64_t)p.T * p.K, T = p.T, D = p.D, I = p.I, E = p.E, Is = p.I_shared;
  L.n = n;
  L.lo_mx = p.dtype == MOE_BF16 && wgrad_lo_mx(p, n, E);
  L.lo_mx_s = p.dtype != MOE_F32 && Is > 0 && wgrad_lo_mx(p, T, 1);   // the shared expert is BF16 under MXFP8
  L.pad = p.dtype == MOE_MXFP8 || L.lo_mx ? 128 : 64;               // 128: one MX K slice
  L.pad_s = L.lo_mx_s ? 128 : 64;
  L.Spad = (n + L.pad * E + L.pad - 1) / L.pad * L.pad;
  L.Tpad = L.lo_mx_s ? (T + 127) / 128 * 128 : (T + 127) / 64 * 64;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = al256(o + bytes); return at; };
  L.err = take(256 + 4096);
  L.offs = take((E + 1) * 4); L.tile_off = take((E + 1) * 4); L.poff = take((E + 1) * 4);
  L.order = take(E * 4);
  L.offs_s = take(8); L.tile_off_s = take(8); L.poff_s = take(8);
  const int64_t eb = p.dtype == MOE_F32 ? 4 : 2;   // bytes per activation element
  L.g_slot = take(n * 4); L.dg_slot = take(n * 4);
  // slot copies of x and dout: the BF16 and MXFP8 layer backwards read both through the schedule
  // instead (unless MOE_FLAG_DISPATCH_COPY); fp32 copies them
  const bool copy = p.dtype == MOE_F32 || (p.flags & MOE_FLAG_DISPATCH_COPY);
  L.x_slot = take(copy ? n * D * eb : 0); L.dy_slot = take(copy ? n * D * eb : 0); L.dx_slot = take(n * D * eb);
  L.dx_sh = take(T * D * eb);
  // replayed a, u; left out when the caller keeps them (offsets then unused)
  L.act_a = take(kept ? 0 : n * I * 4); L.act_u = take(kept ? 0 : n * I * 4);
  if (p.dtype == MOE_F32) {
    L.f_dh = take(n * I * 4); L.f_h = take(n * I * 4); L.f_da = take(n * I * 4); L.f_du = take(n * I * 4);
    if (Is > 0) {
      L.s_a = take(T * Is * 4); L.s_u = take(T * Is * 4);
      L.sf_dh = take(T * Is * 4); L.sf_h = take(T * Is * 4); L.sf_da = take(T * Is * 4); L.sf_du = take(T * Is * 4);
    }
    L.total = o;
    return L;
  }
  if (p.dtype == MOE_MXFP8) {
    // rows quantised along D; dgrad-down output and h, [da | du] in fp32; [da | du] along I;
    // weights re-quantised transposed; slot-axis operands [features][Spad], experts 128-aligned
    const int64_t S = L.Spad;
    L.mq_x = take(n * D); L.ms_x = take(n * D / 32); L.mq_dy = take(n * D); L.ms_dy = take(n * D / 32);
    L.m_dhp = take(n * I * 4); L.part = take(n * ((I + 255) / 256) * 4);
    L.mq_dau = take(n * 2 * I); L.ms_dau = take(n * 2 * I / 32);
    L.mq_wdT = take(E * I * D); L.ms_wdT = take(E * I * D / 32);
    L.mq_wguT = take(E * D * 2 * I); L.ms_wguT = take(E * D * 2 * I / 32);
    L.mq_xT = take(D * S); L.ms_xT = take(D * S / 32); L.mq_gdyT = take(D * S); L.ms_gdyT = take(D * S / 32);
    L.mq_hT = take(I * S); L.ms_hT = take(I * S / 32); L.mq_dauT = take(2 * I * S); L.ms_dauT = take(2 * I * S / 32);
  } else {
    // [da | du | da_lo | du_lo] bf16; transposed padded x, dy, [g*h | lo], [da|du|lo]
    L.dau = take(n * 4 * I * 2);
    L.part = take(n * ((I + 127) / 128) * 4);
    L.xT = take(D * L.Spad * 2); L.dyT = take(D * L.Spad * 2); L.ghT = take(2 * I * L.Spad * 2);
    L.dauT = take(4 * I * L.Spad * 2);
    const int64_t S = L.Spad;
    if (L.lo_mx) {
      L.lq_dau = take(2 * I * S); L.ls_dau = take(2 * I * S / 32); L.lq_gh = take(I * S); L.ls_gh = take(I * S / 32);
      L.lq_x = take(D * S); L.ls_x = take(D * S / 32); L.lq_dy = take(D * S); L.ls_dy = take(D * S / 32);
    }
  }
  if (Is > 0) {
    L.s_a = take(T * Is * 4); L.s_u = take(T * Is * 4); L.s_dau = take(T * 4 * Is * 2);
    L.s_part = take(T * ((Is + 127) / 128) * 4);
    L.s_xT = take(D * L.Tpad * 2); L.s_dyT = take(D * L.Tpad * 2); L.s_hT = take(2 * Is * L.Tpad * 2);
    L.s_dauT = take(4 * Is * L.Tpad * 2);
    const int64_t S = L.Tpad;
    if (L.lo_mx_s) {
      L.slq_dau = take(2 * Is * S); L.sls_dau = take(2 * Is * S / 32); L.slq_gh = take(Is * S);
      L.sls_gh = take(Is * S / 32); L.slq_x = take(D * S); L.sls_x = take(D * S / 32); L.slq_dy = take(D * S);
      L.sls_dy = take(D * S / 32);
    }
  }
  L.total = o;
  return L;
}

struct CoreBufs {
  void *act_a, *act_u, *dau, *xT, *dyT, *ghT, *dauT;   // the dgrad GEMMs read the weights in place, k-major
  float* part;
  int64_t Spad;
  int32_t* order;   // [G] dealing order of the K-grouped GEMMs (null for one group)
  // MXFP8 codes and scales of the weight gradients' second pass: [da | du] and g*h low halves,
  // x and dy, each [features][Spad] along the slots (all null: both passes in BF16)
  uint8_t *q_dau, *s_dau, *q_gh, *s_gh, *q_x, *s_x, *q_dy, *s_dy;
  const Persist* pc = nullptr;   // persistent GEMM control, see launch_gemm_bf16
};

// Backward of one set of groups (routed experts, or the shared expert as one group).
// rows: x_rows/dy_rows [n][D] grouped by offs (sanitised, device) with m-tile prefix tile_off
// and padded offsets poff; with row_map, row j of either is row row_map[j] / row_div of x_rows /
// dy_rows (the layer backward reads x and dout through the schedule, no slot copies). g_rows may
// be null (weight 1). Outputs dx_rows [n][D] bf16, dg_rows [n] fp32 (nullable), dW (fp32).
static int core_backward(int G, int64_t n_cap, int D, int I, const void* x_rows, const void* dy_rows,
                         const float* g_rows, const int32_t* offs, const int32_t* tile_off, const int32_t* poff,
                         const void* wg, const void* wu, const void* wd, void* dx_rows, float* dg_rows,
                         float* dw_gate, float* dw_up, float* dw_down, const CoreBufs& b, hipStream_t s,
                         bool dgrad_one_pass, bool replay = true, const int32_t* row_map = nullptr,
                         int row_div = 1) {
  int st;
  // The dgrad GEMMs contract the weights along their row axis (dh' = dy W_down over D, dx =
  // [da | du] [W_gate; W_up] over I): they read them in place, k-major, through transposing LDS
  // reads (before: transposed copies of every weight per call, 9.2 ms of the DSV3 backward even
  // with 16-byte transposes).

  Grouped grp;
  grp.row_off = offs;
  grp.tile_off = tile_off;
  grp.groups = G;
  grp.max_mtiles = (n_cap + kGemmBM - 1) / kGemmBM + G;

  // replay: a = x W_gate^T, u = x W_up^T (kept in fp32); skipped when the forward kept them
  if (replay) {
    GemmArgs r;
    r.A = x_rows; r.lda = D; r.a_gather = row_map; r.a_div = row_div;
    r.B = wg; r.B2 = wu; r.ldb = D; r.b_group_stride = (int64_t)I * D;
    r.N = I; r.K = D; r.C = b.act_a; r.C2 = b.act_u; r.ldc = I;
    if ((st = launch_gemm_bf16(r, grp, EPI_SAVE_AU, s, b.pc))) return st;
  }

  // dgrad-down + SwiGLU backward: dh' = dy W_down; da, du (as bf16 hi/lo pairs); partial <h, dh'>
  GemmArgs d;
  d.A = dy_rows; d.lda = D; d.a_gather = row_map; d.a_div = row_div;
  d.B = wd; d.ldb = I; d.b_group_stride = (int64_t)D * I; d.b_kmajor = 1;
  d.N = I; d.K = D; d.C = b.dau; d.C2 = (uint16_t*)b.dau + I; d.ldc = 4 * I; d.lo_off = 2 * I;
  d.ea = (const float*)b.act_a; d.eu = (const float*)b.act_u; d.lde = I;
  d.row_scale = g_rows; d.row_partial = b.part;
  if ((st = launch_gemm_bf16(d, grp, EPI_DGRAD, s, b.pc))) return st;
  const int ntn_d = (I + gemm_tile_cols(EPI_DGRAD) - 1) / gemm_tile_cols(EPI_DGRAD);
  if (dg_rows && (st = launch_row_sum(b.part, n_cap, ntn_d, dg_rows, s))) return st;

  // dgrad-up: dx = [da | du] [W_gate; W_up]: K rows < I from W_gate, the rest from W_up
  GemmArgs u;
  u.A = b.dau; u.lda = 4 * I; u.B = wg; u.B2 = wu; u.b_split = I; u.ldb = D; u.b_group_stride = (int64_t)I * D;
  u.b_kmajor = 1;
  u.N = D; u.K = 2 * I; u.C = dx_rows; u.ldc = D;
  if (!dgrad_one_pass) { u.two_pass = 1; u.a_seg_shift = 2 * I; }   // high halves, then low halves
  if ((st = launch_gemm_bf16(u, grp, EPI_STORE, s, b.pc))) return st;

  // padded transposes for the weight gradients: x and dy exact; g*h and [da|du] as hi/lo rows
  const int64_t Sp = b.Spad;
  if ((st = launch_transpose_pad(TR_COPY, x_rows, nullptr, nullptr, D, D, offs, poff, G, Sp, b.xT, Sp, s, 0, row_map,
                                 row_div)))
    return st;
  if ((st = launch_transpose_pad(TR_COPY, dy_rows, nullptr, nullptr, D, D, offs, poff, G, Sp, b.dyT, Sp, s, 0, row_map,
                                 row_div)))
    return st;
  if ((st = launch_transpose_pad(TR_SWIGLU, b.act_a, b.act_u, g_rows, I, I, offs, poff, G, Sp, b.ghT, Sp, s, 1)))
    return st;
  if ((st = launch_transpose_pad(TR_COPY, b.dau, nullptr, nullptr, 4 * I, 4 * I, offs, poff, G, Sp, b.dauT, Sp, s)))
    return st;

  // weight-gradient tiles of the longest groups first
  if (G > 1 && b.order && (st = launch_group_order(poff, G, b.order, s))) return st;
  const int32_t* order = G > 1 ? b.order : nullptr;
  if (!b.q_dy) {
    // both halves in one K loop: B = g*h high rows then low rows; A = [da; du] high rows then low
    GemmArgs w1;   // dW_down[g] = sum_j dy_j (g_j h_j)^T   -> [D][I]
    w1.A = b.dyT; w1.lda = Sp; w1.B = b.ghT; w1.ldb = Sp; w1.k_off = poff; w1.M = D; w1.N = I;
    w1.C = dw_down; w1.ldc = I; w1.c_group_stride = (int64_t)D * I;
    w1.two_pass = 1; w1.b_seg_shift = (int64_t)I * Sp; w1.k_order = order;
    if ((st = launch_gemm_bf16_kgroup(w1, G, s, b.pc))) return st;
    GemmArgs w2;   // [dW_gate; dW_up][g] = sum_j [da_j; du_j] x_j^T -> rows < I: dW_gate, rows >= I: dW_up
    w2.A = b.dauT; w2.lda = Sp; w2.B = b.xT; w2.ldb = Sp; w2.k_off = poff; w2.M = 2 * I; w2.N = D;
    w2.C = dw_gate; w2.C2 = dw_up; w2.m_split = I; w2.ldc = D; w2.c_group_stride = (int64_t)I * D;
    w2.two_pass = 1; w2.a_seg_shift = (int64_t)2 * I * Sp; w2.k_order = order;
    return launch_gemm_bf16_kgroup(w2, G, s, b.pc);
  }
  // MOE_FLAG_BWD_WGRAD_LO_MXFP8 on long groups: the high halves in BF16, then the low halves in
  // MXFP8 added into the same fp32 outputs. A low half is below 2^-8 of its value, so the E4M3 rounding of the second pass (its
  // operands quantised along the slots) costs about 2^-12 relative, with half the bytes and twice
  // the MFMA rate of a second BF16 pass.
  if ((st = launch_quantize_mx((const uint16_t*)b.dyT, D, (int)Sp, b.q_dy, b.s_dy, s))) return st;
  if ((st = launch_quantize_mx((const uint16_t*)b.xT, D, (int)Sp, b.q_x, b.s_x, s))) return st;
  if ((st = launch_quantize_mx((const uint16_t*)b.ghT + (int64_t)I * Sp, I, (int)Sp, b.q_gh, b.s_gh, s))) return st;
  if ((st = launch_quantize_mx((const uint16_t*)b.dauT + (int64_t)2 * I * Sp, 2 * I, (int)Sp, b.q_dau, b.s_dau, s)))
    return st;
  // dW_down[g] = sum_j dy_j (g_j h_j)^T   -> [D][I]
  GemmArgs w1;
  w1.A = b.dyT; w1.lda = Sp; w1.B = b.ghT; w1.ldb = Sp; w1.k_off = poff; w1.M = D; w1.N = I;
  w1.C = dw_down; w1.ldc = I; w1.c_group_stride = (int64_t)D * I; w1.k_order = order;
  if ((st = launch_gemm_bf16_kgroup(w1, G, s, b.pc))) return st;
  GemmArgs m1 = w1;
  m1.A = b.q_dy; m1.B = b.q_gh; m1.c_accumulate = 1;
  if ((st = launch_gemm_mx_kgroup(m1, b.s_dy, b.s_gh, G, s, b.pc))) return st;
  // [dW_gate; dW_up][g] = sum_j [da_j; du_j] x_j^T -> rows < I: dW_gate, rows >= I: dW_up
  GemmArgs w2;
  w2.A = b.dauT; w2.lda = Sp; w2.B = b.xT; w2.ldb = Sp; w2.k_off = poff; w2.M = 2 * I; w2.N = D;
  w2.C = dw_gate; w2.C2 = dw_up; w2.m_split = I; w2.ldc = D; w2.c_group_stride = (int64_t)I * D; w2.k_order = order;
  if ((st = launch_gemm_bf16_kgroup(w2, G, s, b.pc))) return st;
  GemmArgs m2 = w2;
  m2.A = b.q_dau; m2.B = b.q_x; m2.c_accumulate = 1;
  return launch_gemm_mx_kgroup(m2, b.s_dau, b.s_x, G, s, b.pc);
}

// MXFP8 backward of the routed groups (the shared expert stays BF16). Weights are the forward's
// MX tensors: W_gate, W_up [G][I][D] and W_down [G][D][I] with scales along their last axis.
// Every GEMM takes both operands quantised along its own contraction dimension (blocks of 32):
//   replay     a, u (fp32)   = Q_D(x) W_gate^T, Q_D(x) W_up^T
//   dgrad-down dh' (fp32)    = Q_D(dy) Q_D(W_down^T)
//   SwiGLU     da, du, h (fp32, registers only): Q_I([da | du]), Q_n(h), Q_n([da | du]), dg = <h, dh'>
//   dgrad-up   dx (bf16)     = Q_I([da | du]) Q_I([W_gate^T | W_up^T])^T
//   wgrad      dW_down = Q_n(g dy)^T Q_n(h), [dW_gate; dW_up] = Q_n([da | du])^T Q_n(x)
// with Q_n along each group's slots (poff: offsets padded to 128, one MX K slice).
static int core_backward_mx(int G, int64_t n_cap, int D, int I, const void* x_rows, const void* dy_rows,
                            const float* g_rows, const int32_t* offs, const int32_t* tile_off, const int32_t* poff,
                            const moe_weights* w, void* dx_rows, float* dg_rows, float* dw_gate, float* dw_up,
                            float* dw_down, char* ws, const BwdLayout& L, hipStream_t s, const Persist* pc,
                            const float* kept_a = nullptr, const float* kept_u = nullptr,
                            const int32_t* row_map = nullptr, int row_div = 1) {
  int st;
  auto B = [&](size_t off) { return (uint8_t*)(ws + off); };
  auto F = [&](size_t off) { return (float*)(ws + off); };
  // a, u: the forward's (kept, read only) or replayed into the workspace
  float* act_a = kept_a ? const_cast<float*>(kept_a) : F(L.act_a);
  float* act_u = kept_a ? const_cast<float*>(kept_u) : F(L.act_u);
  const int64_t S = L.Spad, ID = (int64_t)I * D;
  // weights re-quantised along the backward contraction axis
  if ((st = launch_mx_requant_t((const uint8_t*)w->w_down, w->sc_down, G, D, I, B(L.mq_wdT), B(L.ms_wdT), D, 0, ID, ID / 32, s))) return st;
  if ((st = launch_mx_requant_t((const uint8_t*)w->w_gate, w->sc_gate, G, I, D, B(L.mq_wguT), B(L.ms_wguT), 2 * I, 0, 2 * ID, 2 * ID / 32, s)))
    return st;
  if ((st = launch_mx_requant_t((const uint8_t*)w->w_up, w->sc_up, G, I, D, B(L.mq_wguT), B(L.ms_wguT), 2 * I, I, 2 * ID, 2 * ID / 32, s)))
    return st;
  // x and dy: along D (dgrad operands) and, in the same pass, x and g dy along the slots
  // (weight-gradient operands)
  if ((st = launch_mx_quant_t((const uint16_t*)x_rows, nullptr, D, D, offs, poff, G, S, B(L.mq_xT), B(L.ms_xT), S,
                              B(L.mq_x), B(L.ms_x), s, row_map, row_div)))
    return st;
  if ((st = launch_mx_quant_t((const uint16_t*)dy_rows, g_rows, D, D, offs, poff, G, S, B(L.mq_gdyT), B(L.ms_gdyT), S,
                              B(L.mq_dy), B(L.ms_dy), s, row_map, row_div)))
    return st;

  Grouped grp;
  grp.row_off = offs;
  grp.tile_off = tile_off;
  grp.groups = G;
  grp.max_mtiles = (n_cap + kGemmBM - 1) / kGemmBM + G;
  if (!kept_a) {
    GemmArgs r;   // replay
    r.A = B(L.mq_x); r.lda = D; r.B = w->w_gate; r.B2 = w->w_up; r.ldb = D; r.b_group_stride = ID;
    r.N = I; r.K = D; r.C = act_a; r.C2 = act_u; r.ldc = I;
    if ((st = launch_gemm_mx(r, B(L.ms_x), w->sc_gate, w->sc_up, ID / 32, nullptr, grp, EPI_SAVE_AU, s, pc))) return st;
  }
  GemmArgs d;   // dgrad-down
  d.A = B(L.mq_dy); d.lda = D; d.B = B(L.mq_wdT); d.ldb = D; d.b_group_stride = ID;
  d.N = I; d.K = D; d.C = F(L.m_dhp); d.ldc = I; d.c_f32 = 1;
  if ((st = launch_gemm_mx(d, B(L.ms_dy), B(L.ms_wdT), nullptr, ID / 32, nullptr, grp, EPI_STORE, s, pc))) return st;
  // SwiGLU backward: [da | du] quantised along I (dgrad-up), h and [da | du] along the slots
  // (weight gradients), dg from per-tile partial sums
  if ((st = launch_mx_swiglu_bwd_t(act_a, act_u, F(L.m_dhp), g_rows, I, offs, poff, G, S, B(L.mq_dau),
                                   B(L.ms_dau), B(L.mq_hT), B(L.ms_hT), B(L.mq_dauT), B(L.ms_dauT), S, F(L.part), s)))
    return st;
  if ((st = launch_row_sum(F(L.part), n_cap, (I + 255) / 256, dg_rows, s))) return st;
  GemmArgs u;   // dgrad-up, K = 2I
  u.A = B(L.mq_dau); u.lda = 2 * I; u.B = B(L.mq_wguT); u.ldb = 2 * I; u.b_group_stride = 2 * ID;
  u.N = D; u.K = 2 * I; u.C = dx_rows; u.ldc = D;
  if ((st = launch_gemm_mx(u, B(L.ms_dau), B(L.ms_wguT), nullptr, 2 * ID / 32, nullptr, grp, EPI_STORE, s, pc)))
    return st;

  int32_t* order = G > 1 ? (int32_t*)(ws + L.order) : nullptr;
  if (order && (st = launch_group_order(poff, G, order, s))) return st;
  GemmArgs w1;  // dW_down [G][D][I]
  w1.A = B(L.mq_gdyT); w1.lda = S; w1.B = B(L.mq_hT); w1.ldb = S; w1.k_off = poff; w1.k_order = order;
  w1.M = D; w1.N = I; w1.C = dw_down; w1.ldc = I; w1.c_group_stride = ID;
  if ((st = launch_gemm_mx_kgroup(w1, B(L.ms_gdyT), B(L.ms_hT), G, s, pc))) return st;
  GemmArgs w2;  // [dW_gate; dW_up] [G][I][D] each
  w2.A = B(L.mq_dauT); w2.lda = S; w2.B = B(L.mq_xT); w2.ldb = S; w2.k_off = poff; w2.k_order = order;
  w2.M = 2 * I; w2.N = D; w2.C = dw_gate; w2.C2 = dw_up; w2.m_split = I; w2.ldc = D; w2.c_group_stride = ID;
  return launch_gemm_mx_kgroup(w2, B(L.ms_dauT), B(L.ms_xT), G, s, pc);
}

int core_backward_f32(int G, int64_t n_cap, int64_t max_rows, int D, int I, const float* x_rows, const float* dy_rows,
                      const float* g_rows, const int32_t* offs, const float* wg, const float* wu, const float* wd,
                      float* dx_rows, float* dg_rows, float* dw_gate, float* dw_up, float* dw_down, float* sa, float* su,
                      float* sdh, float* sh, float* sda, float* sdu, hipStream_t s);
int launch_reverse_dispatch_f32(const float* dx_slot, const int32_t* inv_perm, const float* dx_shared, float* dx, int T,
                                int K, int D, hipStream_t s);

static bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }

static CoreBufs routed_bufs(char* ws, const BwdLayout& L) {
  auto u = [&](size_t o) { return L.lo_mx ? (uint8_t*)(ws + o) : nullptr; };
  return CoreBufs{ws + L.act_a, ws + L.act_u, ws + L.dau, ws + L.xT, ws + L.dyT,
                  ws + L.ghT, ws + L.dauT, (float*)(ws + L.part), L.Spad, (int32_t*)(ws + L.order),
                  u(L.lq_dau), u(L.ls_dau), u(L.lq_gh), u(L.ls_gh), u(L.lq_x), u(L.ls_x), u(L.lq_dy), u(L.ls_dy)};
}
static CoreBufs shared_bufs(char* ws, const BwdLayout& L) {
  auto u = [&](size_t o) { return L.lo_mx_s ? (uint8_t*)(ws + o) : nullptr; };
  return CoreBufs{ws + L.s_a, ws + L.s_u, ws + L.s_dau, ws + L.s_xT, ws + L.s_dyT,
                  ws + L.s_hT, ws + L.s_dauT, (float*)(ws + L.s_part), L.Tpad, nullptr,
                  u(L.slq_dau), u(L.sls_dau), u(L.slq_gh), u(L.sls_gh), u(L.slq_x), u(L.sls_x), u(L.slq_dy),
                  u(L.sls_dy)};
}

// Persistent GEMM control of a backward call: the ticket counters and the budget word
// sit in the first block of the backward workspace, as in the forward's.
static Persist bwd_persist(const moe_problem* p, char* wsb, const BwdLayout& L) {
  Persist pc;
  pc.tickets = (int32_t*)(wsb + L.err + kTicketsOffset);
  pc.force = (p->flags & MOE_FLAG_PERSISTENT_GEMM) != 0;
  set_budget(pc, p->flags, wsb + L.err);
  return pc;
}

// one group of T rows for the shared expert: offsets {0, T}
__global__ void single_group_kernel(int rows, int32_t* offs) {
  offs[0] = 0;
  offs[1] = rows;
}

static int shared_backward(const moe_problem* p, const void* x, const void* dy, const moe_weights* w,
                           const moe_grads* dw, void* dx, char* wsb, const BwdLayout& L, hipStream_t s,
                           const float* kept_a = nullptr, const float* kept_u = nullptr) {
  int32_t* o = (int32_t*)(wsb + L.offs_s);
  hipLaunchKernelGGL(single_group_kernel, dim3(1), dim3(1), 0, s, p->T, o);
  MOE_LAUNCH_CHECK();
  if (p->dtype == MOE_F32) {
    auto F = [&](size_t off) { return (float*)(wsb + off); };
    return core_backward_f32(1, p->T, p->T, p->D, p->I_shared, (const float*)x, (const float*)dy, nullptr, o,
                             (const float*)w->ws_gate, (const float*)w->ws_up, (const float*)w->ws_down, (float*)dx,
                             nullptr, dw->dws_gate, dw->dws_up, dw->dws_down, F(L.s_a), F(L.s_u), F(L.sf_dh), F(L.sf_h),
                             F(L.sf_da), F(L.sf_du), s);
  }
  int st = launch_group_prefix(o, 1, p->T, o, (int32_t*)(wsb + L.tile_off_s), (int32_t*)(wsb + L.poff_s),
                               (int32_t*)(wsb + L.err), s, L.pad_s);
  if (st) return st;
  CoreBufs cb = shared_bufs(wsb, L);
  const Persist pc = bwd_persist(p, wsb, L);
  cb.pc = &pc;
  if (kept_a) {
    cb.act_a = const_cast<float*>(kept_a);   // read only from here on
    cb.act_u = const_cast<float*>(kept_u);
  }
  return core_backward(1, p->T, p->D, p->I_shared, x, dy, nullptr, o, (int32_t*)(wsb + L.tile_off_s),
                       (int32_t*)(wsb + L.poff_s), w->ws_gate, w->ws_up, w->ws_down, dx, nullptr, dw->dws_gate,
                       dw->dws_up, dw->dws_down, cb, s, (p->flags & MOE_FLAG_BWD_DGRAD_ONE_PASS) != 0, !kept_a);
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_backward_workspace_size(const moe_problem* p, size_t* bytes) {
  int st = validate_problem(p);
  if (st) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = bwd_layout(*p).total;
  return MOE_OK;
}

int moe_backward_kept_workspace_size(const moe_problem* p, size_t* bytes) {
  int st = validate_problem(p);
  if (st) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  if (p->dtype == MOE_F32) return MOE_ERR_UNSUPPORTED;
  *bytes = bwd_layout(*p, true).total;
  return MOE_OK;
}

}  // extern "C"

namespace moe {

// h = bf16(SiLU(a) u) from the kept fp32 a, u: the arithmetic of the SwiGLU GEMM epilogue, so h
// (and y) are bitwise those of the fused path.
__global__ __launch_bounds__(256) void swiglu_rows_kernel(const float* __restrict__ a, const float* __restrict__ u,
                                                          int64_t n4, uint16_t* __restrict__ h) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const float4 va = reinterpret_cast<const float4*>(a)[i], vu = reinterpret_cast<const float4*>(u)[i];
    const uint32_t lo = (uint32_t)f2bf(silu_f(va.x) * vu.x) | ((uint32_t)f2bf(silu_f(va.y) * vu.y) << 16);
    const uint32_t hi = (uint32_t)f2bf(silu_f(va.z) * vu.z) | ((uint32_t)f2bf(silu_f(va.w) * vu.w) << 16);
    reinterpret_cast<uint2*>(h)[i] = make_uint2(lo, hi);
  }
}

int launch_swiglu_rows(const float* a, const float* u, int64_t n4, uint16_t* h, hipStream_t s) {
  if (n4 <= 0) return MOE_OK;
  const unsigned nb = (unsigned)std::min<int64_t>((n4 + 255) / 256, 16384);
  hipLaunchKernelGGL(swiglu_rows_kernel, dim3(nb), dim3(256), 0, s, a, u, n4, h);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

// The same from the kept a, u under MXFP8: h = SiLU(a) u in fp32, quantised along I in blocks of
// 32 (E4M3 codes, E8M0 scales) exactly as the MXFP8 SwiGLU GEMM epilogue does. One thread per
// block; blocks are row-major over [rows][I / 32].
__global__ __launch_bounds__(256) void swiglu_rows_mx_kernel(const float* __restrict__ a, const float* __restrict__ u,
                                                             int64_t nblk, uint8_t* __restrict__ q,
                                                             uint8_t* __restrict__ sc) {
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nblk; b += (int64_t)gridDim.x * 256) {
    const float4* pa = reinterpret_cast<const float4*>(a + b * 32);
    const float4* pu = reinterpret_cast<const float4*>(u + b * 32);
    float v[32];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float4 va = pa[k], vu = pu[k];
      v[4 * k] = silu_f(va.x) * vu.x;
      v[4 * k + 1] = silu_f(va.y) * vu.y;
      v[4 * k + 2] = silu_f(va.z) * vu.z;
      v[4 * k + 3] = silu_f(va.w) * vu.w;
    }
    uint32_t p[8];
    sc[b] = (uint8_t)mx_block(v, p);
    u32x4* d = reinterpret_cast<u32x4*>(q + b * 32);
    d[0] = u32x4{p[0], p[1], p[2], p[3]};
    d[1] = u32x4{p[4], p[5], p[6], p[7]};
  }
}

int launch_swiglu_rows_mx(const float* a, const float* u, int64_t nblk, uint8_t* q, uint8_t* sc, hipStream_t s) {
  if (nblk <= 0) return MOE_OK;
  const unsigned nb = (unsigned)std::min<int64_t>((nblk + 255) / 256, 16384);
  hipLaunchKernelGGL(swiglu_rows_mx_kernel, dim3(nb), dim3(256), 0, s, a, u, nblk, q, sc);
  MOE_LAUNCH_CHECK();
  return MOE_OK;
}

static int experts_forward_impl(const moe_problem* p, int64_t slots, const void* x_slot, const int32_t* offsets,
                                const moe_weights* w, void* y_slot, const void* x_local, void* shared_out,
                                float* act_a, float* act_u, float* sact_a, float* sact_u, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  int st = validate_problem(p);
  if (st) return st;
  // the slots arrive dispatched: nothing to carry through a ring (its layout would also be too
  // small for all slots)
  if (p->chunk_rows > 0) return MOE_ERR_UNSUPPORTED;
  const bool keep = act_a || act_u;
  if (keep && (!act_a || !act_u)) return MOE_ERR_INVALID_ARG;
  if (!sact_a != !sact_u || (sact_a && !keep)) return MOE_ERR_INVALID_ARG;
  if (keep && p->dtype == MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (p->I_shared == 0) sact_a = sact_u = nullptr;
  if (keep && (!al16(act_a) || !al16(act_u) || p->I % 4)) return MOE_ERR_MISALIGNED;
  if (sact_a && (!al16(sact_a) || !al16(sact_u) || p->I_shared % 4)) return MOE_ERR_MISALIGNED;
  const bool mx = p->dtype == MOE_MXFP8;
  // the non-MX path runs the bf16 MFMA GEMMs, or the fp32 FMA GEMMs under MOE_F32
  const bool f32 = p->dtype == MOE_F32;
  if ((p->flags & MOE_FLAG_PERSISTENT_GEMM) && p->dtype == MOE_F32) return MOE_ERR_UNSUPPORTED;
  // BF16 and MXFP8: the up/gate and down GEMMs run persistent where they have enough tiles per workgroup
  // (always with MOE_FLAG_PERSISTENT_GEMM), their ticket counters in the workspace's first block
  Persist pcs;
  const Persist* pc = nullptr;
  if (p->dtype != MOE_F32 && ws) {
    pcs.tickets = (int32_t*)((char*)ws + kTicketsOffset);
    pcs.force = (p->flags & MOE_FLAG_PERSISTENT_GEMM) != 0;
    set_budget(pcs, p->flags, (char*)ws);
    pc = &pcs;
  }
  auto gemm = [f32, pc](const GemmArgs& a, const Grouped& g, Epi e, hipStream_t s) {
    return f32 ? launch_gemm_f32(a, g, e, s) : launch_gemm_bf16(a, g, e, s, pc);
  };
  if (!x_slot || !offsets || !w || !y_slot || !w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_INVALID_ARG;
  if (mx && (!w->sc_gate || !w->sc_up || !w->sc_down)) return MOE_ERR_INVALID_ARG;
  if (slots < 0 || slots > (int64_t)p->T * p->K) return MOE_ERR_INVALID_ARG;
  if (p->I_shared > 0 && (!x_local || !shared_out || !w->ws_gate || !w->ws_up || !w->ws_down)) return MOE_ERR_INVALID_ARG;
  WsLayout L = ws_layout(*p);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!al16(x_slot) || !al16(y_slot) || !al16(ws) || (x_local && !al16(x_local)) || (shared_out && !al16(shared_out)))
    return MOE_ERR_MISALIGNED;
  char* wsb = (char*)ws;
  // sanitised offsets + m-tile prefix
  int32_t* clean = (int32_t*)(wsb + L.grp_clean);
  int32_t* poff = (int32_t*)(wsb + L.grp_poff);
  if ((st = launch_group_prefix(offsets, p->E, (int)slots, clean, (int32_t*)(wsb + L.tile_off), poff,
                                (int32_t*)(wsb + L.err), stream)))
    return st;
  Grouped gr;
  gr.row_off = clean;
  gr.tile_off = (const int32_t*)(wsb + L.tile_off);
  gr.groups = p->E;
  gr.max_mtiles = (slots + kGemmBM - 1) / kGemmBM + p->E;
  if (mx) {
    // slot rows quantised along D, then the forward's two block-scaled GEMMs (h quantised along I
    // in the SwiGLU epilogue)
    uint8_t* xq = (uint8_t*)(wsb + L.x_slot);
    uint8_t* xs = (uint8_t*)(wsb + L.x_slot_sc);
    uint8_t* hq = (uint8_t*)(wsb + L.h);
    uint8_t* hs = (uint8_t*)(wsb + L.h_sc);
    if ((st = launch_quantize_mx((const uint16_t*)x_slot, slots, p->D, xq, xs, stream))) return st;
    GemmArgs m1;
    m1.A = xq; m1.lda = p->D; m1.B = w->w_gate; m1.B2 = w->w_up; m1.ldb = p->D;
    m1.b_group_stride = (int64_t)p->I * p->D; m1.N = p->I; m1.K = p->D; m1.C = hq; m1.ldc = p->I;
    if (keep) {
      // a, u to the caller in fp32 (the backward's replay GEMM), then h quantised from them
      m1.C = act_a; m1.C2 = act_u;
      if ((st = launch_gemm_mx(m1, xs, w->sc_gate, w->sc_up, (int64_t)p->I * (p->D / 32), nullptr, gr, EPI_SAVE_AU,
                               stream, pc)))
        return st;
      const int64_t nblk = slots * (p->I / 32);
      if (nblk > 0) {
        const unsigned nb = (unsigned)std::min<int64_t>((nblk + 255) / 256, 16384);
        hipLaunchKernelGGL(swiglu_rows_mx_kernel, dim3(nb), dim3(256), 0, stream, act_a, act_u, nblk, hq, hs);
        MOE_LAUNCH_CHECK();
      }
    } else if ((st = launch_gemm_mx(m1, xs, w->sc_gate, w->sc_up, (int64_t)p->I * (p->D / 32), hs, gr, EPI_SWIGLU,
                                    stream, pc))) {
      return st;
    }
    GemmArgs m2;
    m2.A = hq; m2.lda = p->I; m2.B = w->w_down; m2.ldb = p->I; m2.b_group_stride = (int64_t)p->D * p->I;
    m2.N = p->D; m2.K = p->I; m2.C = y_slot; m2.ldc = p->D;
    if ((st = launch_gemm_mx(m2, hs, w->sc_down, nullptr, (int64_t)p->D * (p->I / 32), nullptr, gr, EPI_STORE, stream,
                             pc)))
      return st;
  } else {
  GemmArgs g1;
  g1.A = x_slot; g1.lda = p->D; g1.B = w->w_gate; g1.B2 = w->w_up; g1.ldb = p->D;
  g1.b_group_stride = (int64_t)p->I * p->D; g1.N = p->I; g1.K = p->D; g1.C = wsb + L.h; g1.ldc = p->I;
  if (keep) {
    // a, u to the caller in fp32 (the backward's replay GEMM), then h from them
    g1.C = act_a; g1.C2 = act_u;
    if ((st = gemm(g1, gr, EPI_SAVE_AU, stream))) return st;
    const int64_t n4 = slots * p->I / 4;
    if (n4 > 0) {
      const unsigned nb = (unsigned)std::min<int64_t>((n4 + 255) / 256, 16384);
      hipLaunchKernelGGL(swiglu_rows_kernel, dim3(nb), dim3(256), 0, stream, act_a, act_u, n4, (uint16_t*)(wsb + L.h));
      MOE_LAUNCH_CHECK();
    }
  } else if ((st = gemm(g1, gr, EPI_SWIGLU, stream))) {
    return st;
  }
  GemmArgs g2;
  g2.A = wsb + L.h; g2.lda = p->I; g2.B = w->w_down; g2.ldb = p->I; g2.b_group_stride = (int64_t)p->D * p->I;
  g2.N = p->D; g2.K = p->I; g2.C = y_slot; g2.ldc = p->D;
  if ((st = gemm(g2, gr, EPI_STORE, stream))) return st;
  }
  if (p->I_shared > 0) {
    Grouped gs;
    gs.M = p->T;
    GemmArgs s1;
    s1.A = x_local; s1.lda = p->D; s1.B = w->ws_gate; s1.B2 = w->ws_up; s1.ldb = p->D; s1.N = p->I_shared;
    s1.K = p->D; s1.C = wsb + L.sh_h; s1.ldc = p->I_shared;
    if (sact_a) {
      // the shared expert's a, u to the caller as well, h from them (BF16 even under MXFP8)
      s1.C = sact_a; s1.C2 = sact_u;
      if ((st = launch_gemm_bf16(s1, gs, EPI_SAVE_AU, stream))) return st;
      const int64_t n4 = (int64_t)p->T * p->I_shared / 4;
      const unsigned nb = (unsigned)std::min<int64_t>((n4 + 255) / 256, 16384);
      hipLaunchKernelGGL(swiglu_rows_kernel, dim3(nb), dim3(256), 0, stream, sact_a, sact_u, n4,
                         (uint16_t*)(wsb + L.sh_h));
      MOE_LAUNCH_CHECK();
    } else if ((st = gemm(s1, gs, EPI_SWIGLU, stream))) {
      return st;
    }
    GemmArgs s2;
    s2.A = wsb + L.sh_h; s2.lda = p->I_shared; s2.B = w->ws_down; s2.ldb = p->I_shared; s2.N = p->D;
    s2.K = p->I_shared; s2.C = shared_out; s2.ldc = p->D;
    if ((st = gemm(s2, gs, EPI_STORE, stream))) return st;
  }
  return MOE_OK;
}

static int experts_backward_impl(const moe_problem* p, int64_t slots, const void* x_slot, const int32_t* offsets,
                                 const float* g_slot, const void* dy_slot, const moe_weights* w, void* dx_slot,
                                 float* dg_slot, const moe_grads* dw, const void* x_local, const void* dy_local,
                                 void* dx_local, const float* act_a, const float* act_u, const float* sact_a,
                                 const float* sact_u, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = validate_problem(p);
  if (st) return st;
  const bool kept = act_a || act_u;
  if (kept && (!act_a || !act_u)) return MOE_ERR_INVALID_ARG;
  if (!sact_a != !sact_u || (sact_a && !kept)) return MOE_ERR_INVALID_ARG;
  if (kept && p->dtype == MOE_F32) return MOE_ERR_UNSUPPORTED;
  if (p->I_shared == 0) sact_a = sact_u = nullptr;
  const bool mx = p->dtype == MOE_MXFP8, f32 = p->dtype == MOE_F32;
  if (!x_slot || !offsets || !g_slot || !dy_slot || !w || !dx_slot || !dg_slot || !dw) return MOE_ERR_INVALID_ARG;
  if (!w->w_gate || !w->w_up || !w->w_down || !dw->dw_gate || !dw->dw_up || !dw->dw_down) return MOE_ERR_INVALID_ARG;
  if (mx && (!w->sc_gate || !w->sc_up || !w->sc_down)) return MOE_ERR_INVALID_ARG;
  if (slots < 0 || slots > (int64_t)p->T * p->K) return MOE_ERR_INVALID_ARG;
  if (p->I_shared > 0 && (!x_local || !dy_local || !dx_local || !w->ws_gate || !w->ws_up || !w->ws_down ||
                          !dw->dws_gate || !dw->dws_up || !dw->dws_down))
    return MOE_ERR_INVALID_ARG;
  BwdLayout L = bwd_layout(*p, kept);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!al16(x_slot) || !al16(dy_slot) || !al16(dx_slot) || !al16(ws) || (x_local && !al16(x_local)) ||
      (dy_local && !al16(dy_local)) || (dx_local && !al16(dx_local)))
    return MOE_ERR_MISALIGNED;
  if (kept && (!al16(act_a) || !al16(act_u) || p->I % 4)) return MOE_ERR_MISALIGNED;
  if (sact_a && (!al16(sact_a) || !al16(sact_u) || p->I_shared % 4)) return MOE_ERR_MISALIGNED;
  char* wsb = (char*)ws;
  int32_t* offs = (int32_t*)(wsb + L.offs);
  if ((st = launch_group_prefix(offsets, p->E, (int)slots, offs, (int32_t*)(wsb + L.tile_off),
                                (int32_t*)(wsb + L.poff), (int32_t*)(wsb + L.err), stream, L.pad)))
    return st;
  if (f32) {
    auto F = [&](size_t off) { return (float*)(wsb + off); };
    if ((st = core_backward_f32(p->E, slots, slots, p->D, p->I, (const float*)x_slot, (const float*)dy_slot, g_slot,
                                offs, (const float*)w->w_gate, (const float*)w->w_up, (const float*)w->w_down,
                                (float*)dx_slot, dg_slot, dw->dw_gate, dw->dw_up, dw->dw_down, F(L.act_a), F(L.act_u),
                                F(L.f_dh), F(L.f_h), F(L.f_da), F(L.f_du), stream)))
      return st;
  } else if (mx) {
    const Persist pc = bwd_persist(p, wsb, L);
    if ((st = core_backward_mx(p->E, slots, p->D, p->I, x_slot, dy_slot, g_slot, offs, (int32_t*)(wsb + L.tile_off),
                               (int32_t*)(wsb + L.poff), w, dx_slot, dg_slot, dw->dw_gate, dw->dw_up, dw->dw_down, wsb,
                               L, stream, &pc, act_a, act_u)))
      return st;
  } else {
    CoreBufs cb = routed_bufs(wsb, L);
    const Persist pc = bwd_persist(p, wsb, L);
    cb.pc = &pc;
    if (kept) {
      cb.act_a = const_cast<float*>(act_a);   // read only from here on
      cb.act_u = const_cast<float*>(act_u);
    }
    if ((st = core_backward(p->E, slots, p->D, p->I, x_slot, dy_slot, g_slot, offs, (int32_t*)(wsb + L.tile_off),
                            (int32_t*)(wsb + L.poff), w->w_gate, w->w_up, w->w_down, dx_slot, dg_slot, dw->dw_gate,
                            dw->dw_up, dw->dw_down, cb, stream, (p->flags & MOE_FLAG_BWD_DGRAD_ONE_PASS) != 0,
                            !kept)))
      return st;
  }
  if (p->I_shared > 0) return shared_backward(p, x_local, dy_local, w, dw, dx_local, wsb, L, stream, sact_a, sact_u);
  return MOE_OK;
}

}  // namespace moe

extern "C" {

int moe_experts_forward(const moe_problem* p, int64_t slots, const void* x_slot, const int32_t* offsets,
                        const moe_weights* w, void* y_slot, const void* x_local, void* shared_out,
                        void* ws, size_t ws_bytes, hipStream_t stream) {
  return experts_forward_impl(p, slots, x_slot, offsets, w, y_slot, x_local, shared_out, nullptr, nullptr, nullptr,
                              nullptr, ws, ws_bytes, stream);
}

int moe_experts_forward_keep(const moe_problem* p, int64_t slots, const void* x_slot, const int32_t* offsets,
                             const moe_weights* w, void* y_slot, const void* x_local, void* shared_out,
                             float* act_a, float* act_u, float* shared_act_a, float* shared_act_u, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  if (!act_a || !act_u) return MOE_ERR_INVALID_ARG;
  return experts_forward_impl(p, slots, x_slot, offsets, w, y_slot, x_local, shared_out, act_a, act_u, shared_act_a,
                              shared_act_u, ws, ws_bytes, stream);
}

int moe_experts_backward(const moe_problem* p, int64_t slots, const void* x_slot, const int32_t* offsets,
                         const float* g_slot, const void* dy_slot, const moe_weights* w, void* dx_slot,
                         float* dg_slot, const moe_grads* dw, const void* x_local, const void* dy_local,
                         void* dx_local, void* ws, size_t ws_bytes, hipStream_t stream) {
  return experts_backward_impl(p, slots, x_slot, offsets, g_slot, dy_slot, w, dx_slot, dg_slot, dw, x_local,
                               dy_local, dx_local, nullptr, nullptr, nullptr, nullptr, ws, ws_bytes, stream);
}

int moe_experts_backward_kept(const moe_problem* p, int64_t slots, const void* x_slot, const int32_t* offsets,
                              const float* g_slot, const void* dy_slot, const moe_weights* w, void* dx_slot,
                              float* dg_slot, const moe_grads* dw, const void* x_local, const void* dy_local,
                              void* dx_local, const float* act_a, const float* act_u, const float* shared_act_a,
                              const float* shared_act_u, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!act_a || !act_u) return MOE_ERR_INVALID_ARG;
  return experts_backward_impl(p, slots, x_slot, offsets, g_slot, dy_slot, w, dx_slot, dg_slot, dw, x_local,
                               dy_local, dx_local, act_a, act_u, shared_act_a, shared_act_u, ws, ws_bytes, stream);
}

static int backward_impl(const moe_problem* p, const void* dout, const void* x, const float* logits,
                         const moe_weights* w, const moe_routing* r, void* dx, const moe_grads* dw, float* d_topk_w,
                         float* d_logits, const float* act_a, const float* act_u, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  int st = validate_routing(p);
  if (st) return st;
  const bool kept = act_a || act_u;
  if (kept && (!act_a || !act_u)) return MOE_ERR_INVALID_ARG;
  if (kept && p->dtype == MOE_F32) return MOE_ERR_UNSUPPORTED;
  (void)logits;   // the routing state of the forward carries everything the backward needs
  const bool mx = p->dtype == MOE_MXFP8, f32 = p->dtype == MOE_F32;
  if (!dout || !x || !w || !r || !dx || !dw || !d_topk_w) return MOE_ERR_INVALID_ARG;
  if (mx && (!w->sc_gate || !w->sc_up || !w->sc_down)) return MOE_ERR_INVALID_ARG;
  if (!r->topk_idx || !r->topk_w || !r->offsets || !r->perm || !r->inv_perm) return MOE_ERR_INVALID_ARG;
  if (!w->w_gate || !w->w_up || !w->w_down || !dw->dw_gate || !dw->dw_up || !dw->dw_down) return MOE_ERR_INVALID_ARG;
  if (p->I_shared > 0 && (!w->ws_gate || !w->ws_up || !w->ws_down || !dw->dws_gate || !dw->dws_up || !dw->dws_down))
    return MOE_ERR_INVALID_ARG;
  BwdLayout L = bwd_layout(*p, kept);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!al16(dout) || !al16(x) || !al16(dx) || !al16(ws)) return MOE_ERR_MISALIGNED;
  if (kept && (!al16(act_a) || !al16(act_u))) return MOE_ERR_MISALIGNED;
  char* wsb = (char*)ws;
  const int64_t n = L.n;
  // reverse-combine (pull dout into slots) and replayed dispatch of x: copies for fp32 and under
  // MOE_FLAG_DISPATCH_COPY; otherwise the BF16 GEMMs and transposes, and the MXFP8 quantisers, read
  // slot row j from dout / x row perm[j] / K directly
  const bool copy = p->dtype == MOE_F32 || (p->flags & MOE_FLAG_DISPATCH_COPY);
  const int adt = f32 ? MOE_F32 : MOE_BF16;   // activations stay bf16 under MXFP8 until quantised
  if (copy) {
    if ((st = launch_dispatch(dout, adt, r->perm, p->K, p->D, 0, n, wsb + L.dy_slot, nullptr, stream))) return st;
    if ((st = launch_dispatch(x, adt, r->perm, p->K, p->D, 0, n, wsb + L.x_slot, nullptr, stream))) return st;
  }
  if ((st = launch_gather_f32(r->topk_w, r->perm, n, (float*)(wsb + L.g_slot), stream))) return st;
  int32_t* offs = (int32_t*)(wsb + L.offs);
  if ((st = launch_group_prefix(r->offsets, p->E, (int)n, offs, (int32_t*)(wsb + L.tile_off),
                                (int32_t*)(wsb + L.poff), (int32_t*)(wsb + L.err), stream, L.pad)))
    return st;
  if (f32) {
    auto F = [&](size_t off) { return (float*)(wsb + off); };
    if ((st = core_backward_f32(p->E, n, n, p->D, p->I, F(L.x_slot), F(L.dy_slot), F(L.g_slot), offs,
                                (const float*)w->w_gate, (const float*)w->w_up, (const float*)w->w_down, F(L.dx_slot),
                                F(L.dg_slot), dw->dw_gate, dw->dw_up, dw->dw_down, F(L.act_a), F(L.act_u), F(L.f_dh),
                                F(L.f_h), F(L.f_da), F(L.f_du), stream)))
      return st;
  } else if (mx) {
    const Persist pc = bwd_persist(p, wsb, L);
    if ((st = core_backward_mx(p->E, n, p->D, p->I, copy ? (const void*)(wsb + L.x_slot) : x,
                               copy ? (const void*)(wsb + L.dy_slot) : dout, (float*)(wsb + L.g_slot), offs,
                               (int32_t*)(wsb + L.tile_off), (int32_t*)(wsb + L.poff), w, wsb + L.dx_slot,
                               (float*)(wsb + L.dg_slot), dw->dw_gate, dw->dw_up, dw->dw_down, wsb, L, stream, &pc,
                               act_a, act_u, copy ? nullptr : r->perm, p->K)))
      return st;
  } else {
    CoreBufs cb = routed_bufs(wsb, L);
    const Persist pc = bwd_persist(p, wsb, L);
    cb.pc = &pc;
    if (kept) {
      cb.act_a = const_cast<float*>(act_a);   // read only from here on
      cb.act_u = const_cast<float*>(act_u);
    }
    if ((st = core_backward(p->E, n, p->D, p->I, copy ? (const void*)(wsb + L.x_slot) : x,
                            copy ? (const void*)(wsb + L.dy_slot) : dout, (float*)(wsb + L.g_slot), offs,
                            (int32_t*)(wsb + L.tile_off), (int32_t*)(wsb + L.poff), w->w_gate, w->w_up, w->w_down,
                            wsb + L.dx_slot, (float*)(wsb + L.dg_slot), dw->dw_gate, dw->dw_up, dw->dw_down, cb,
                            stream, (p->flags & MOE_FLAG_BWD_DGRAD_ONE_PASS) != 0, !kept,
                            copy ? nullptr : r->perm, p->K)))
      return st;
  }
  if ((st = launch_router_backward((float*)(wsb + L.dg_slot), r->inv_perm, r->topk_idx, r->topk_w, p->T, p->E, p->K,
                                   d_topk_w, d_logits, stream)))
    return st;
  void* dsh = nullptr;
  if (p->I_shared > 0) {
    dsh = wsb + L.dx_sh;
    if ((st = shared_backward(p, x, dout, w, dw, dsh, wsb, L, stream))) return st;
  }
  // reverse-dispatch: dx[t] = dx_shared[t] + sum_k dx_slot[inv_perm[t*K + k]]
  if (f32)
    return launch_reverse_dispatch_f32((const float*)(wsb + L.dx_slot), r->inv_perm, (const float*)dsh, (float*)dx,
                                       p->T, p->K, p->D, stream);
  return launch_reverse_dispatch(wsb + L.dx_slot, r->inv_perm, dsh, dx, p->T, p->K, p->D, stream);
}

int moe_backward(const moe_problem* p, const void* dout, const void* x, const float* logits, const moe_weights* w,
                 const moe_routing* r, void* dx, const moe_grads* dw, float* d_topk_w, float* d_logits, void* ws,
                 size_t ws_bytes, hipStream_t stream) {
  return backward_impl(p, dout, x, logits, w, r, dx, dw, d_topk_w, d_logits, nullptr, nullptr, ws, ws_bytes, stream);
}

int moe_backward_kept(const moe_problem* p, const void* dout, const void* x, const float* logits,
                      const moe_weights* w, const moe_routing* r, void* dx, const moe_grads* dw, float* d_topk_w,
                      float* d_logits, const float* act_a, const float* act_u, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  if (!act_a || !act_u) return MOE_ERR_INVALID_ARG;
  return backward_impl(p, dout, x, logits, w, r, dx, dw, d_topk_w, d_logits, act_a, act_u, ws, ws_bytes, stream);
}

}  // extern "C"
