/*
 * moe.h - C ABI of the MI355X (gfx950) MoE layer library (libmoe.so).
 *
 * One DeepSeek-V3-style mixture-of-experts layer on one GPU, as defined by the Cursor blog post
 * "Mixture-of-Kittens: our open-source MoE megakernel for NVL72s", section "Overlapping
 * computation and communication in MoE" (notation and MoE layer equation):
 *
 *     MoE(x, s) = E_shared(x) + sum_{i in E} g_i E_i(x),      g_i = s_i / sum_{j in E} s_j,
 *     E_i(x)    = W_down^(i) ( SiLU(W_gate^(i) x) (*) W_up^(i) x ),
 *
 * with s = softmax(router logits) over all routed experts and E the top-K routed experts.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Ownership: the caller owns every pointer. Tensor and workspace pointers are device
 *   pointers (hipMalloc'd memory of the current device); structs are host memory read during
 *   the call only. The library allocates nothing, creates no streams or events, and keeps no
 *   state between calls, except that moe_schedule_noalloc keeps, per device, the address of its
 *   static scratch array.
 * - Asynchrony: a call validates its arguments on the host, then only enqueues kernels on
 *   `stream`. It never synchronises, never copies device data to the host and never blocks.
 * - Errors: MOE_OK (0) or a negative moe_status. Argument errors are detected on the host
 *   before anything is enqueued (no device work happens then). A kernel launch failure returns
 *   MOE_ERR_HIP. Data errors only the device can see (an expert id out of range in a
 *   caller-supplied topk_idx) are clamped so that no access goes out of bounds, and set the
 *   sticky error word at byte offset 0 of the workspace (int32, nonzero = error) without
 *   faulting; the caller may read it asynchronously after the call.
 * - Layouts are row-major. Element types: MOE_F32 = float, MOE_BF16 = bfloat16 (uint16 bits),
 *   MOE_MXFP8 = OCP E4M3 bytes with one E8M0 scale byte per 32 elements along the contraction
 *   dimension (OCP Microscaling Formats v1.0).
 * - Determinism: for identical inputs and problem descriptors, every output is bitwise
 *   identical from run to run, and independent of chunk_rows and of how many workgroups run:
 *   no floating-point atomics are used and every sum has a fixed order.
 * - Re-entrancy: calls are re-entrant; concurrent calls need separate workspaces.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,   /* null pointer, non-positive size, K outside [1, E], ... */
  MOE_ERR_UNSUPPORTED = -2,   /* valid but not implemented (a size the kernels do not tile) */
  MOE_ERR_WORKSPACE = -3,     /* workspace null or smaller than moe_workspace_size() */
  MOE_ERR_MISALIGNED = -4,    /* a tensor pointer not 16-byte aligned */
  MOE_ERR_HIP = -5            /* a HIP launch error (hipGetLastError after enqueue) */
} moe_status;

typedef enum moe_dtype {
  MOE_F32 = 0,     /* fp32 storage and arithmetic */
  MOE_BF16 = 1,    /* bf16 storage, fp32 accumulation */
  MOE_MXFP8 = 2    /* routed experts in MXFP8 (E4M3 + E8M0 per 32), shared expert and x in bf16 */
} moe_dtype;

/* Problem descriptor. T tokens of dimension D; E routed experts of intermediate size I, K per
 * token; one shared expert of intermediate size I_shared (0 = none).
 * Size limits: E <= 1024; T*K < 2^31; the routing entry points (route_topk, schedule, forward,
 * backward) also need K <= min(E, 64) (the expert-level entry points use K only as slots per
 * token). BF16/MXFP8 need D % 128 == 0 and
 * I % 128 == 0 (I_shared likewise); MOE_F32 needs D % 4 == 0.
 * chunk_rows (b): rows of the expert-contiguous routed buffer that one chunk carries through
 *   dispatch and the whole expert FFN before the next (Notes "Mixture-of-Kittens: MoE Megakernel
 *   for NVL72s", section "Granularity as a tunable"). 0 means one chunk of all T*K rows; other
 *   values are rounded up to a multiple of 256 and clamped to [max(256, T*K/1024), T*K]. With
 *   chunks, h lives in a ring of ring_stages chunk stages (BF16 and MXFP8), and so do the
 *   dispatched rows under MOE_FLAG_DISPATCH_COPY (otherwise chunks read x through the schedule:
 *   BF16 x itself, MXFP8 its token rows quantised once). moe_forward / moe_forward_stages return
 *   MOE_ERR_UNSUPPORTED for chunk_rows > 0 under MOE_F32, as do moe_forward_keep and the
 *   expert-level forwards (their slots are not carried through a ring). The backward entry
 *   points do not chunk: they accept the forward's problem descriptor and ignore chunk_rows and
 *   ring_stages.
 * ring_stages: macrobatch ring depth (Notes, section "A ring buffer instead of a host
 *   round-trip"); 0 selects 3. Ignored when one chunk holds every row.
 * flags: bitwise OR of MOE_FLAG_* below; any other bit is MOE_ERR_INVALID_ARG. */
typedef struct moe_problem {
  int32_t T, D, I, E, K, I_shared;
  int32_t dtype;
  int32_t chunk_rows;
  int32_t ring_stages;
  int32_t flags;
} moe_problem;

/* The forwards (moe_forward, moe_forward_stages, moe_forward_keep, moe_forward_lanes; chunks too)
 * read the x rows of the routed up/gate GEMM through the schedule (row j of expert-slot order is
 * x[perm[j] / K]) instead of a dispatched copy: the pages' pull dispatch done by the GEMM's own
 * operand loads, with no copy pass (DSV3 shape: 9.41 against 9.66 ms per forward). Under
 * MOE_MXFP8 the T token rows are quantised once (E4M3 codes and E8M0 scales per 32) and the
 * block-scaled GEMM reads codes and scales the same way (T = 32768: the dispatch stage 0.50 ->
 * 0.11 ms). This is the default; MOE_FLAG_FUSED_GATHER names it and is accepted. The BF16 layer
 * backward (moe_backward, moe_backward_kept) reads x and dout the same way in its GEMMs and
 * transposes (DSV3 shape: 45.3 against 45.7 ms, and no 2 T K D-element slot buffers in its
 * workspace), the MXFP8 layer backward in its quantisers. MOE_FLAG_DISPATCH_COPY instead writes
 * the expert-contiguous slot copies first (as the fp32 backward always does) and runs on them; the
 * outputs are the same bits. Both flags together: MOE_ERR_INVALID_ARG. */
#define MOE_FLAG_FUSED_GATHER 0x1
#define MOE_FLAG_DISPATCH_COPY 0x100000
/* Bits 0x2, 0x8, 0x10, 0x20 and 0xff00 are reserved (they selected tuning variants that measured
 * no faster and were removed); a problem that sets one, or any bit not defined here, is rejected. */
/* moe_backward / moe_experts_backward under MOE_BF16: contract dgrad-up (dx = [da | du] [W_gate |
 * W_up]) over the bf16 da, du in one K pass instead of over their hi + lo halves in two. Each dx
 * element sums 2I products whose roundings are independent; measured max |d| of dx reaches
 * 2.5e-2 RMS (the worst element at 0.73 of its bound tau RMS + half a BF16 ulp of the value)
 * against 1.6e-2 (0.44) with both passes; about 4 ms faster on one EP=64 rank's share. */
#define MOE_FLAG_BWD_DGRAD_ONE_PASS 0x40
/* moe_backward / moe_experts_backward: the bf16 weight gradients' second K pass (over the low
 * halves of g*h and [da | du]) in MXFP8 instead of BF16, added into the fp32 dW by a second
 * grouped GEMM over operands quantised along the slots. Taken only where the groups average at
 * least 4096 rows (routed: T*K >= 4096 E; shared expert: T >= 4096, also under MOE_MXFP8), since
 * it reads and writes dW once more; otherwise the flag changes nothing. The low halves keep
 * about 4 significant bits, so dW carries about 2^-13 relative error per product: measured max
 * |d| of dW at 7e-4 RMS against 2e-5 with both passes in BF16 (both far inside tau = 2e-2).
 * moe_backward_workspace_size grows by the quantised operands, (3 I + 2 D) * 33/32 bytes per
 * padded slot (routed) and (3 I_shared + 2 D) * 33/32 per padded token (shared), where taken. */
#define MOE_FLAG_BWD_WGRAD_LO_MXFP8 0x80
/* Run the chunked path (chunk_rows > 0) as one persistent work-queue kernel instead of three
 * launches per chunk. Currently disabled: a call with this flag returns MOE_ERR_UNSUPPORTED. */
#define MOE_FLAG_PERSISTENT 0x4
/* Persistent grouped GEMMs (MOE_BF16 and MOE_MXFP8; the sparsenotes page "Mixture-of-Kittens: MoE
 * Megakernel for NVL72s", sections "Granularity as a tunable" and "The production details"): the
 * up/gate and down GEMMs (BF16 or block-scaled) of the forward entry points (moe_forward, moe_forward_stages, moe_forward_keep, and the
 * expert-level moe_experts_forward, moe_experts_forward_keep; routed and shared expert) can run as
 * persistent kernels, one workgroup per CU taking 256 x 256 tiles from ticket counters kept in
 * the first 256 bytes of the workspace, instead of one workgroup per tile. Without this flag a
 * GEMM runs persistent where it has at least 12 tiles per workgroup (e.g. the routed GEMMs at
 * T = 8192, 256 experts, K = 8), per tile otherwise; with it, always. Each tile is computed by one
 * workgroup in the same order either way, so every output is bitwise the same. Workgroups never
 * wait for each other. MOE_F32 forwards with the flag: MOE_ERR_UNSUPPORTED. The backward entry
 * points apply the same rule to their GEMMs (replay, dgrad-down, dgrad-up, K-grouped weight
 * gradients; BF16, and block-scaled under MOE_MXFP8), with the counters in their own workspace's
 * first 256 bytes. */
#define MOE_FLAG_PERSISTENT_GEMM 0x10000
/* With MOE_FLAG_PERSISTENT_GEMM (alone: MOE_ERR_INVALID_ARG): between tiles, the persistent GEMMs
 * read the int32 workgroup budget at byte offset MOE_WS_CU_BUDGET_OFFSET of the workspace the call
 * is given (forward or backward workspace). While
 * it holds v > 0, workgroups with index >= v take no further tile and end after their current
 * one, handing their CUs to other work on the GPU (the Notes' "The production details": the
 * kernel yields processors to a higher-priority stream); the workgroups below v take every
 * remaining tile, so the outputs are unchanged. v <= 0: no limit. The caller owns the word: it
 * must initialise it before the call (the workspace is otherwise uninitialised); the library only
 * reads it. Set before the call, it partitions the GPU: the persistent GEMMs use v workgroups and
 * leave the other CUs to other streams (e.g. collectives). It may also be changed while the call
 * runs, and takes effect at each workgroup's next tile boundary; but a copy or stream write-value
 * enqueued on another stream can itself wait for a free CU before it lands, so a write meant to
 * free CUs quickly belongs before the call. With this flag every forward GEMM runs persistent
 * (MOE_FLAG_PERSISTENT_GEMM); the other kernels (routing, dispatch, combine) are short, run one
 * workgroup per block, and do not read the word. */
#define MOE_FLAG_CU_BUDGET 0x20000
#define MOE_WS_CU_BUDGET_OFFSET 4
/* With MOE_FLAG_CU_BUDGET (alone: MOE_ERR_INVALID_ARG): the budget word is not the one in the
 * workspace but the one whose address the 8 bytes at byte offset MOE_WS_CU_BUDGET_PTR_OFFSET of the
 * workspace hold (8-byte aligned; a null address: no limit). It may live in any memory the GPU
 * reads, e.g. pinned host memory allocated coherent (hipHostMalloc with hipHostMallocCoherent),
 * which the host can store to while the call runs: the persistent GEMMs read the word with
 * system-scope loads between tiles, so the store takes effect at each workgroup's next tile
 * boundary with no GPU work of its own (a copy or write-value on another stream would itself wait
 * for a free CU). The caller writes the address into the workspace before the call and keeps the
 * word alive until the call's work is done; the library only reads both. */
#define MOE_FLAG_CU_BUDGET_INDIRECT 0x200000
#define MOE_WS_CU_BUDGET_PTR_OFFSET 8
/* moe_route_gemm_backward: d_logits has dense terms (e.g. from an auxiliary loss on the router),
 * so both products run on the dense kernel instead of skipping zero entries. The results are the
 * same bits either way; only the speed differs (DSV3 shape: 0.48 ms skipping zeros at K = 8 of 256
 * nonzero per row and 2.4 ms dense; a fully dense d_logits takes 8.8 ms skipping zeros). */
#define MOE_FLAG_ROUTER_BWD_DENSE 0x80000

/* Expert weights (device pointers). Routed: w_gate, w_up [E][I][D]; w_down [E][D][I].
 * Shared: ws_gate, ws_up [I_shared][D]; ws_down [D][I_shared] (always bf16 under MOE_MXFP8).
 * MXFP8 only: routed weights are E4M3 bytes with scales sc_gate, sc_up [E][I][D/32] and
 * sc_down [E][D][I/32] (E8M0 bytes), as produced by moe_quantize_mx. */
typedef struct moe_weights {
  const void *w_gate, *w_up, *w_down;
  const void *ws_gate, *ws_up, *ws_down;
  const uint8_t *sc_gate, *sc_up, *sc_down;
} moe_weights;

/* Routing state written by the forward and read by the backward (device pointers).
 * topk_idx [T][K] int32 and topk_w [T][K] float: the K chosen experts per token in descending
 * logit order (ties to the lower index) and their weights g. counts [E], offsets [E+1]
 * (exclusive scan of counts), perm [T*K] (slot -> route id t*K+k) and inv_perm [T*K]
 * (route id -> slot). Slots of expert e are offsets[e] .. offsets[e+1]-1, in route order. */
typedef struct moe_routing {
  int32_t *topk_idx;
  float *topk_w;
  int32_t *counts;
  int32_t *offsets;
  int32_t *perm;
  int32_t *inv_perm;
} moe_routing;

/* Weight gradients, fp32, same shapes as the weights (shared ones may be NULL when
 * I_shared == 0). Overwritten, not accumulated; an expert with no rows gets exact zeros. */
typedef struct moe_grads {
  float *dw_gate, *dw_up, *dw_down;
  float *dws_gate, *dws_up, *dws_down;
} moe_grads;

/* Human-readable name of a status code (static string). */
const char *moe_status_string(int status);

/* Bytes of device workspace that moe_schedule and the forwards (moe_forward, moe_forward_stages,
 * moe_forward_keep, moe_forward_lanes) need for `p` (moe_backward: moe_backward_workspace_size).
 * Writes *bytes; returns MOE_OK or MOE_ERR_INVALID_ARG.
 * The first 256 bytes hold the sticky error word (offset 0, int32). */
int moe_workspace_size(const moe_problem *p, size_t *bytes);

/* Bytes of device workspace that moe_backward and moe_experts_backward need for `p` (the
 * expert-level backward takes p->T * p->K as its slot capacity). Same conventions as above. */
int moe_backward_workspace_size(const moe_problem *p, size_t *bytes);

/* Bytes of device workspace that moe_backward_kept and moe_experts_backward_kept need for `p`:
 * the above less the 2 * T * K * I * 4 bytes the replay of the routed a, u would fill (the caller
 * holds them). The replaying backwards refuse a workspace of only this size (MOE_ERR_WORKSPACE).
 * MOE_F32: MOE_ERR_UNSUPPORTED (no kept path). */
int moe_backward_kept_workspace_size(const moe_problem *p, size_t *bytes);

/* Top-K selection and router weights (Blog, "Overlapping computation and communication in
 * MoE": the router picks the top-k routed experts and weights them with g_i = s_i / sum s_j).
 * logits [T][E] fp32 -> topk_idx [T][K] int32, topk_w [T][K] fp32. One wavefront per token;
 * selection compares the fp32 logits (a total order: larger first, lower index on ties,
 * -0.0 == +0.0, NaN below -inf), g is computed in fp32 as exp(l_k - l_max) / sum. Inputs are
 * expected to have at least K non-NaN logits per token (otherwise g is NaN). */
int moe_route_topk(const moe_problem *p, const float *logits, int32_t *topk_idx, float *topk_w,
                   hipStream_t stream);

/* Router GEMM fused with the top-K selection (the logits of the Blog's "Overlapping computation
 * and communication in MoE" computed in the library): logits[t][e] = sum_d x[t][d] w_router[e][d]
 * from BF16 x [T][D] and w_router [E][D] with fp32 accumulation, split along D into K-groups
 * whose fp32 partial products are summed in group order (deterministic), then moe_route_topk's
 * selection and weights on those logits. logits [T][E] fp32 receives them (nullable);
 * topk_idx [T][K], topk_w [T][K] as moe_route_topk. BF16 problems only (MOE_ERR_UNSUPPORTED for
 * MOE_F32; under MOE_MXFP8 x is the BF16 input). x and w_router 16-byte aligned. Needs `ws` of
 * moe_route_gemm_workspace_size bytes (the split-K partials). */
int moe_route_gemm(const moe_problem *p, const void *x, const void *w_router, float *logits,
                   int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of device workspace moe_route_gemm needs for `p`. */
int moe_route_gemm_workspace_size(const moe_problem *p, size_t *bytes);

/* Backward of moe_route_gemm's projection logits = x W_r^T (the router of the Blog's
 * "Overlapping computation and communication in MoE"; the router-gradient step of the Notes'
 * "The production details" continued through the projection): from d_logits [T][E] fp32 (as
 * moe_backward writes it), dw_router [E][D] fp32 = d_logits^T x (overwritten) and, when dx is
 * not NULL, dx [T][D] (BF16, the experts' input gradient from moe_backward) += d_logits W_r,
 * summed in fp32 onto the stored value and rounded once. x [T][D], w_router [E][D] BF16.
 * Products are exact in fp32; each output is one thread's fp32 sum in ascending token (dw) or
 * expert (dx) order: deterministic. Zero entries of d_logits are skipped: their products are
 * exact zeros, so the sums are those over every entry (up to the sign of an all-zero sum), at
 * about K/E of the work; a NaN or infinite x or W_r element meets only the nonzero entries. With
 * x 4-byte, dw_router 8-byte and w_router and dx 16-byte aligned the zero-skipping kernels run
 * (unless MOE_FLAG_ROUTER_BWD_DENSE), otherwise a dense kernel with the same sums. BF16 and MXFP8 problems (x is BF16 under both);
 * MOE_F32: MOE_ERR_UNSUPPORTED. No workspace. */
int moe_route_gemm_backward(const moe_problem *p, const void *x, const void *w_router, const float *d_logits,
                            float *dw_router, void *dx, hipStream_t stream);

/* Device-side histogram + exclusive scan + stable placement: the one-source-rank case of the
 * pull schedule (Blog, "Scheduling"; sort key from the Notes, section "Pull dispatch, push
 * combine"). topk_idx [T][K] -> counts [E], offsets [E+1], perm [T*K], inv_perm [T*K], with
 * the layout documented at moe_routing. Bit-exact and independent of launch shape. No host
 * synchronisation: counts stay on the device. Needs `ws` of moe_workspace_size bytes. */
int moe_schedule(const moe_problem *p, const int32_t *topk_idx, int32_t *counts, int32_t *offsets,
                 int32_t *perm, int32_t *inv_perm, void *ws, size_t ws_bytes, hipStream_t stream);

/* moe_schedule for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same outputs, bit for bit, with no
 * workspace argument. Its scratch (per-block histograms and the m-tile prefix) is a static device
 * array of 2 MiB + 8 KiB that each GPU holds from the first call until the process ends; the
 * first call on a device also looks up that array's address there (the library's only
 * host-side state, kept per device). Sizes beyond the array -- ceil(T*K / 2048) * E > 2^19,
 * e.g. more than 2^20 routes with E = 1024 or 2^22 with E = 256 -- return MOE_ERR_UNSUPPORTED
 * before anything is enqueued. error_word: a caller-owned device int32 that receives the sticky
 * error bits moe_schedule puts at workspace offset 0 (bit 0: an expert id out of range, counted
 * as expert 0); never cleared by the library. Calls that overlap on one GPU share the array and
 * race: serialise them (one stream, or an event between streams). */
int moe_schedule_noalloc(const moe_problem *p, const int32_t *topk_idx, int32_t *counts, int32_t *offsets,
                         int32_t *perm, int32_t *inv_perm, int32_t *error_word, hipStream_t stream);

/* Pull-dispatch schedule of rank `rank` among R source ranks (Blog, "Scheduling"; region order
 * from the Notes, "Pull dispatch, push combine"). routing [R][N][K] int32 (device): global expert
 * of route k of token i on source rank r, in [0, R*L); rank c owns experts [c*L, (c+1)*L).
 * Outputs (device): counts [L] routes per local expert, src_counts [L][R] routes per (local
 * expert, source rank), offsets [L+1] exclusive scan of counts (offsets[L] = routes this rank
 * pulls), and for slot p < offsets[L] the source of the route it holds: phi_src[p] (source rank)
 * and phi_idx[p] (i*K + k on that rank). Inside the region of expert l the routes are ordered by
 * (ordinal, source rank), the ordinal being the number of earlier routes (in (i, k) order) from
 * the same source rank to l; so slot offsets[l] + q holds, for q < sum_r min(M[l][r], o + 1),
 * ordinal o's routes in source-rank order. route_pos [R*N*K] (nullable) receives each route's
 * slot, or -1 for routes owned by another rank. phi_src / phi_idx must hold R*N*K entries (the
 * worst case). Bit-exact and independent of launch shape; no host synchronisation. At R = 1 this
 * is moe_schedule's permutation (phi_idx = perm). Expert ids outside [0, R*L) set bit 0 of the
 * sticky error word (the first int32 of `ws`, never cleared by the library) and count as expert
 * 0. Needs `ws` of moe_pull_schedule_workspace_size bytes. Returns MOE_ERR_UNSUPPORTED when
 * R*L > 1024 or R*N*K >= 2^31. */
int moe_pull_schedule(int32_t R, int32_t N, int32_t K, int32_t L, int32_t rank, const int32_t *routing,
                      int32_t *counts, int32_t *src_counts, int32_t *offsets, int32_t *phi_src,
                      int32_t *phi_idx, int32_t *route_pos, void *ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of device workspace moe_pull_schedule needs for (R, N, K, L). */
int moe_pull_schedule_workspace_size(int32_t R, int32_t N, int32_t K, int32_t L, size_t *bytes);

/* Dispatch (the one-GPU analogue of the pull dispatch, Notes "Pull dispatch, push combine"):
 * x_slot[j - slot_begin] = x[perm[j] / K] for j in [slot_begin, slot_begin + slot_count).
 * x [T][D] in the activation type (bf16, or f32 under MOE_F32). Under MOE_MXFP8 the rows are
 * quantised on the way (Notes, "The production details": quantisation fused into dispatch):
 * x_slot gets E4M3 bytes [slot_count][D] and x_slot_scales E8M0 bytes [slot_count][D/32];
 * otherwise x_slot_scales must be NULL. */
int moe_dispatch(const moe_problem *p, const void *x, const int32_t *perm, int64_t slot_begin,
                 int64_t slot_count, void *x_slot, uint8_t *x_slot_scales, hipStream_t stream);

/* The same dispatch over all T*K slots, token-major: each token's row of x is read once (and
 * under MOE_MXFP8 quantised once) and written to its K slots x_slot[inv_perm[t*K + k]]
 * (inv_perm as produced by moe_schedule, a bijection onto [0, T*K)). Identical bytes to
 * moe_dispatch over the whole range; this is the form moe_forward uses when it dispatches all
 * slots at once. x_slot_scales: E8M0 bytes [T*K][D/32] under MOE_MXFP8, NULL otherwise
 * (MOE_ERR_INVALID_ARG if that does not hold). */
int moe_dispatch_tokens(const moe_problem *p, const void *x, const int32_t *inv_perm, void *x_slot,
                        uint8_t *x_slot_scales, hipStream_t stream);

/* Deterministic combine (Blog, weighted sum after the combine; Notes "The production details"
 * on determinism): out[t] = shared_out[t] + sum_{k=0}^{K-1} topk_w[t][k] * y_routes[t*K + k],
 * accumulated in fp32 in exactly that order and rounded once. y_routes [T*K][D] (route order),
 * shared_out [T][D] or NULL, out [T][D]; activation type (bf16, or f32 under MOE_F32). */
int moe_combine(const moe_problem *p, const void *y_routes, const void *shared_out,
                const float *topk_w, void *out, hipStream_t stream);

/* Whole forward: route (moe_route_topk) -> schedule (moe_schedule) -> dispatch into
 * expert-contiguous ring slots -> grouped up/gate GEMM with the SwiGLU epilogue -> grouped down
 * GEMM whose epilogue stores row j at route perm[j] -> shared expert -> combine.
 * x [T][D], logits [T][E] fp32, out [T][D]. `routing` (all six pointers) receives the routing
 * state for the backward. y_routes [T*K][D] and shared_out [T][D] are optional (NULL: kept in
 * the workspace); when given they receive the per-route expert outputs and the shared expert
 * output. */
int moe_forward(const moe_problem *p, const void *x, const float *logits, const moe_weights *w,
                void *out, const moe_routing *routing, void *y_routes, void *shared_out,
                void *ws, size_t ws_bytes, hipStream_t stream);

/* Concurrent chunk lanes for the chunked forward (Notes "Mixture-of-Kittens: MoE Megakernel for
 * NVL72s", section "Granularity as a tunable": small chunks stay cheap only when the work of
 * several chunks is in flight at once). Lane 0 is the call's `stream`; lanes 1 .. count are the
 * caller's `streams[0 .. count-1]` (streams of the current device at the default priority; the
 * library creates none). `events` holds S + 1 + count events created by the caller on the current
 * device (hipEventCreateWithFlags with hipEventDisableTiming suggested), where S is the
 * problem's ring depth (ring_stages, 0 meaning 3): events[0 .. S-1] mark ring stages free again,
 * events[S] forks the lanes from `stream`, events[S+1 ..] join them back. */
#define MOE_MAX_LANES 4
typedef struct moe_lanes {
  int32_t count;          /* extra lanes, 1 .. MOE_MAX_LANES - 1 */
  hipStream_t *streams;   /* [count] */
  hipEvent_t *events;     /* [S + 1 + count] */
} moe_lanes;

/* moe_forward whose routed chunks run on several streams at once. After the routing, the
 * schedule and the chunk tables (on `stream`), the lanes fork from `stream`; chunk c (dispatch,
 * up/gate, down) runs on lane c mod (count + 1), and the shared expert first on lane 0. Chunk c
 * reuses the ring stage of chunk c - S: when that chunk ran on another lane, chunk c's dispatch
 * waits (hipStreamWaitEvent) for the event recorded after that chunk's down GEMM. The lanes join
 * `stream` before the combine, so `stream` orders the whole call as for moe_forward: the caller
 * may synchronise or capture `stream` alone (a graph captured from `stream` takes in the lanes'
 * work through the fork and join events). Each lane's persistent GEMMs take tiles from ticket
 * counters of their own in the workspace's first 256 bytes. Outputs are bitwise those of
 * moe_forward for the same problem: every output tile is the same workgroup sum. With one chunk
 * (chunk_rows == 0) the lanes only fork and join. Requirements as moe_forward (chunk_rows > 0
 * under MOE_F32: MOE_ERR_UNSUPPORTED); lanes NULL, count outside
 * [1, MOE_MAX_LANES - 1], or a NULL stream or event: MOE_ERR_INVALID_ARG. Overlapping calls on
 * the same events or workspace race. The lanes overlap only where `stream` and the lane streams
 * sit on distinct hardware queues. HIP binds a stream to one of GPU_MAX_HW_QUEUES queues (4 by
 * default) when the stream first receives work, and streams beyond that share queues (measured
 * through rocprofv3's queue ids and the run times), so lanes may run one after the other (same
 * outputs, less overlap). Give lanes streams that received work before any other stream but
 * `stream`, e.g. one small kernel each at start-up, or raise GPU_MAX_HW_QUEUES. */
int moe_forward_lanes(const moe_problem *p, const void *x, const float *logits, const moe_weights *w,
                      void *out, const moe_routing *routing, void *y_routes, void *shared_out,
                      void *ws, size_t ws_bytes, hipStream_t stream, const moe_lanes *lanes);

/* Stage boundaries of the forward, for moe_forward_stages. Event i is recorded on `stream`
 * just before stage i; event MOE_STAGE_COUNT just after the last stage. */
enum moe_stage {
  MOE_STAGE_ROUTE = 0,      /* moe_route_topk */
  MOE_STAGE_SCHEDULE = 1,   /* histogram + scan + placement */
  MOE_STAGE_SHARED = 2,     /* shared expert (up/gate + SwiGLU, down) */
  MOE_STAGE_DISPATCH = 3,   /* rows into expert-contiguous slots (skipped under FUSED_GATHER) */
  MOE_STAGE_UP_GATE = 4,    /* routed grouped GEMM W_gate/W_up + SwiGLU epilogue */
  MOE_STAGE_DOWN = 5,       /* routed grouped GEMM W_down + scatter epilogue */
  MOE_STAGE_COMBINE = 6,    /* fixed-order weighted sum */
  MOE_STAGE_COUNT = 7
};

/* moe_forward with timing hooks: identical work and outputs; if `stage_events` is not NULL it
 * holds MOE_STAGE_COUNT + 1 events created by the caller (hipEventCreate), recorded on `stream`
 * at the stage boundaries above so that hipEventElapsedTime gives per-stage device time. */
int moe_forward_stages(const moe_problem *p, const void *x, const float *logits,
                       const moe_weights *w, void *out, const moe_routing *routing,
                       void *y_routes, void *shared_out, void *ws, size_t ws_bytes,
                       hipEvent_t *stage_events, hipStream_t stream);

/* Whole backward of the layer (Notes, "Pull dispatch, push combine": reverse-combine and
 * reverse-dispatch; "A ring buffer instead of a host round-trip": the forward activations are
 * recomputed, not stored; "The production details": the router gradient as <h, W_down^T dY>).
 * Inputs: dout [T][D], x [T][D], logits [T][E], weights, and the routing state of the forward.
 * Outputs: dx [T][D] (activation type: BF16, fp32 under MOE_F32), weight gradients (fp32),
 * d_topk_w [T][K] fp32 (gradient w.r.t. g) and d_logits [T][E] fp32 (nullable). MOE_BF16;
 * MOE_MXFP8 with the forward's MX weights (routed experts as in moe_experts_backward; the shared
 * expert in BF16); MOE_F32 with every operand fp32 (plain FMA GEMMs, for small problems). */
int moe_backward(const moe_problem *p, const void *dout, const void *x, const float *logits,
                 const moe_weights *w, const moe_routing *routing, void *dx, const moe_grads *dw,
                 float *d_topk_w, float *d_logits, void *ws, size_t ws_bytes, hipStream_t stream);

/* moe_forward that also hands the routed pre-activations to the caller, for moe_backward_kept:
 * act_a, act_u [T*K][I] fp32 (16-byte aligned) receive a = x W_gate^T and u = x W_up^T per slot
 * in the schedule's slot order, with the backward replay's own GEMM; h is formed from them with
 * the fused epilogue's arithmetic, so every output is bitwise that of moe_forward. The pages'
 * replay (sparsenotes page "Mixture-of-Kittens: MoE Megakernel for NVL72s", "The production
 * details") recomputes a, u; on one GPU 2 T K I 4 bytes of HBM buy that GEMM back. MOE_BF16 and
 * MOE_MXFP8 (a, u of the block-scaled GEMM; h quantised along I from them as the epilogue does)
 * with chunk_rows == 0 (otherwise MOE_ERR_UNSUPPORTED); null act_a or act_u: MOE_ERR_INVALID_ARG. */
int moe_forward_keep(const moe_problem *p, const void *x, const float *logits, const moe_weights *w,
                     void *out, const moe_routing *routing, void *y_routes, void *shared_out,
                     float *act_a, float *act_u, void *ws, size_t ws_bytes, hipStream_t stream);

/* moe_backward reading the routed a, u that moe_forward_keep wrote for the same x, routing and
 * weights instead of replaying them; every output bitwise that of moe_backward. The shared expert
 * replays its own. MOE_BF16 and MOE_MXFP8 (MOE_F32: MOE_ERR_UNSUPPORTED); act_a, act_u non-null
 * (MOE_ERR_INVALID_ARG) and 16-byte aligned (MOE_ERR_MISALIGNED). `ws` holds
 * moe_backward_kept_workspace_size bytes. */
int moe_backward_kept(const moe_problem *p, const void *dout, const void *x, const float *logits,
                      const moe_weights *w, const moe_routing *routing, void *dx, const moe_grads *dw,
                      float *d_topk_w, float *d_logits, const float *act_a, const float *act_u,
                      void *ws, size_t ws_bytes, hipStream_t stream);

/* Expert-level forward of one expert-parallel rank's share (Blog, "Overlapping computation and
 * communication in MoE": EP sharding gives each rank a few routed experts plus the shared
 * expert). Slots arrive already grouped by local expert, as a pull dispatch lands them.
 * p->E = local experts, p->T = local tokens (rows of the shared expert), p->T * p->K = slot
 * capacity (slots <= T*K). Offsets outside [0, slots] or decreasing are clamped (error word
 * set) so that no access leaves the buffers. `ws` holds moe_workspace_size bytes.
 * x_slot [slots][D], offsets [E+1] device int32 (expert e owns rows offsets[e]..offsets[e+1]-1,
 * offsets[E] == slots) -> y_slot [slots][D] = E_e(x_slot) (unweighted; the source applies g).
 * x_local [T][D] -> shared_out [T][D] (skipped when I_shared == 0). MOE_BF16, MOE_F32 (fp32
 * tensors and weights, plain FMA GEMMs), or MOE_MXFP8:
 * x_slot stays BF16 and is quantised along D inside the call, the routed weights are the MX
 * tensors of moe_weights (E4M3 + E8M0 scales per 32 along their last axis), h is quantised
 * along I before the down projection, and the shared expert runs in BF16. */
int moe_experts_forward(const moe_problem *p, int64_t slots, const void *x_slot,
                        const int32_t *offsets, const moe_weights *w, void *y_slot,
                        const void *x_local, void *shared_out, void *ws, size_t ws_bytes,
                        hipStream_t stream);

/* Backward of moe_experts_forward where slot j contributes g_slot[j] * E_e(x_slot[j]) against
 * the upstream gradient dy_slot[j]. Outputs dx_slot [slots][D] (bf16), dg_slot [slots] fp32
 * (= <dy_slot[j], E_e(x_slot[j])>), routed and shared weight gradients (fp32) and dx_local
 * [T][D] (bf16, fp32 under MOE_F32; shared expert path with upstream dy_local [T][D]). `ws` holds
 * moe_backward_workspace_size bytes (which depend on p->dtype).
 * MOE_MXFP8 (sparsenotes page "Mixture-of-Kittens: MoE Megakernel for NVL72s", "The production
 * details": the routed experts train in MXFP8): every routed GEMM takes both operands quantised
 * (OCP MX, blocks of 32) along its own contraction dimension: the replay a, u from Q_D(x_slot);
 * dh' = Q_D(dy) Q_D(W_down^T); the SwiGLU backward in fp32 with dg = <h, dh'>; dx_slot =
 * Q_I([da | du]) Q_I([W_gate | W_up]^T)^T; dW_down = Q_n(g dy)^T Q_n(h) and [dW_gate; dW_up] =
 * Q_n([da | du])^T Q_n(x) with Q_n along each expert's slots (blocks from its first slot). The
 * weights are the forward's MX tensors, dequantised and quantised again along the backward
 * contraction axis inside the call; the shared expert runs in BF16. */
int moe_experts_backward(const moe_problem *p, int64_t slots, const void *x_slot,
                         const int32_t *offsets, const float *g_slot, const void *dy_slot,
                         const moe_weights *w, void *dx_slot, float *dg_slot, const moe_grads *dw,
                         const void *x_local, const void *dy_local, void *dx_local,
                         void *ws, size_t ws_bytes, hipStream_t stream);

/* moe_experts_forward that also hands the routed experts' pre-activations to the caller, so
 * that moe_experts_backward_kept can skip its replay of them. act_a, act_u: [slots][I] fp32
 * device buffers (16-byte aligned, I % 4 == 0) that receive a = x_slot W_gate^T and
 * u = x_slot W_up^T with the backward replay's own GEMM, bitwise; h = SiLU(a) u is then formed
 * from them with the fused epilogue's arithmetic, so y_slot and shared_out are bitwise those of
 * moe_experts_forward. The replay the pages describe (sparsenotes page "Mixture-of-Kittens: MoE
 * Megakernel for NVL72s", "The production details") recomputes a, u; on one GPU that is pure
 * extra work, and 2 * slots * I * 4 bytes of HBM buy it back. MOE_BF16 and MOE_MXFP8 (a, u
 * from the block-scaled GEMM over Q_D(x_slot), h quantised along I from them as the fused
 * epilogue does); MOE_F32: MOE_ERR_UNSUPPORTED; null act_a or act_u: MOE_ERR_INVALID_ARG.
 * shared_act_a, shared_act_u: the same for the shared expert, [T][I_shared] fp32 (BF16 GEMM under
 * both dtypes), or both null to let the backward replay the shared expert; ignored when
 * I_shared == 0; only one of the two given: MOE_ERR_INVALID_ARG. */
int moe_experts_forward_keep(const moe_problem *p, int64_t slots, const void *x_slot,
                             const int32_t *offsets, const moe_weights *w, void *y_slot,
                             const void *x_local, void *shared_out, float *act_a, float *act_u,
                             float *shared_act_a, float *shared_act_u, void *ws, size_t ws_bytes,
                             hipStream_t stream);

/* moe_experts_backward reading the routed a, u that moe_experts_forward_keep wrote for the same
 * x_slot, offsets and weights, instead of replaying them; every output is bitwise that of
 * moe_experts_backward. The shared expert reads shared_act_a, shared_act_u when given (both
 * or neither), and replays its own otherwise. MOE_BF16 and MOE_MXFP8 (the buffers of
 * moe_experts_forward_keep under the same dtype); act buffers 16-byte aligned with I % 4 == 0
 * (MOE_ERR_MISALIGNED). `ws` holds moe_backward_kept_workspace_size bytes. */
int moe_experts_backward_kept(const moe_problem *p, int64_t slots, const void *x_slot,
                              const int32_t *offsets, const float *g_slot, const void *dy_slot,
                              const moe_weights *w, void *dx_slot, float *dg_slot, const moe_grads *dw,
                              const void *x_local, const void *dy_local, void *dx_local,
                              const float *act_a, const float *act_u, const float *shared_act_a,
                              const float *shared_act_u, void *ws, size_t ws_bytes, hipStream_t stream);

/* MX quantiser (OCP Microscaling v1.0; the Notes' MXFP8, "The production details"): src
 * [rows][cols] bf16 -> q [rows][cols] E4M3 bytes and scales [rows][cols/32] E8M0 bytes, blocks
 * of 32 along each row. Scale 2^(floor(log2 amax) - 8) clamped to [2^-127, 2^127]; elements
 * rounded to nearest-even and saturated to +-448; an all-zero block gets scale byte 127.
 * cols % 32 == 0. Used offline for the weights, and by dispatch for activations. */
int moe_quantize_mx(const void *src_bf16, int64_t rows, int32_t cols, uint8_t *q, uint8_t *scales,
                    hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
