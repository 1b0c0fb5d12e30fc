"""fp64 reference of the MoE layer (routing, schedule, experts, combine, backward).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's CPU baseline,
never by the library path.

Notation follows the Blog's section "Overlapping computation and communication in MoE":
D model dimension, I expert intermediate dimension, E the set of top-k routed experts of a token,
s the router weights, g_i = s_i / sum_{j in E} s_j, and

    MoE(x, s) = E_shared(x) + sum_{i in E} g_i * E_i(x),
    E_i(x)    = W_down^(i) ( SiLU(W_gate^(i) x) (*) W_up^(i) x ),

with W_up, W_gate in R^{I x D} and W_down in R^{D x I}. Arrays here are row-major with one token
per row, so W x becomes X @ W.T.

Readings where the pages leave a step open:
* the router weights s are the softmax of the router logits over all experts;
* the top-k set is chosen on the logits (the same set as on s, since softmax is monotone),
  in descending order with ties going to the lower expert index; -0.0 equals +0.0 and a NaN
  logit ranks below -inf;
* the route id of the k-th choice of token i is i*K + k.
"""
from __future__ import annotations

import numpy as np


def sigmoid(a):
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(over='ignore'):
        return 1.0 / (1.0 + np.exp(-a))


def silu(a):
    """SiLU(a) = a * sigmoid(a)  (the gated activation of the Blog's MoE equation)."""
    a = np.asarray(a, dtype=np.float64)
    return a * sigmoid(a)


# ----------------------------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------------------------
def route_topk(logits: np.ndarray, K: int) -> np.ndarray:
    """Top-K expert ids per token, [T, K] int32.

    Blog, "Overlapping computation and communication in MoE": the router picks the top-k routed
    experts of each token. Order: larger logit first; equal logits by lower expert index; NaN
    after every number.
    """
    l = np.asarray(logits, dtype=np.float64)
    T, E = l.shape
    nan = np.isnan(l)
    neg = np.where(nan, 0.0, -l)        # ascending -l == descending l; -0.0 == +0.0 here
    ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((ids, neg, nan), axis=-1)   # last key is the primary key
    return order[:, :K].astype(np.int32)


def routing_weights(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """g[t, k] = s_i / sum_{j in E} s_j for i = idx[t, k], with s = softmax(logits[t]) over all
    experts (Blog, "Overlapping computation and communication in MoE", MoE layer equation).
    A NaN logit gets s = 0."""
    l = np.asarray(logits, dtype=np.float64)
    l = np.where(np.isnan(l), -np.inf, l)
    m = np.max(l, axis=1, keepdims=True)
    z = np.exp(l - m)
    s = z / z.sum(axis=1, keepdims=True)
    s_sel = np.take_along_axis(s, idx.astype(np.int64), axis=1)
    return s_sel / s_sel.sum(axis=1, keepdims=True)


# ----------------------------------------------------------------------------------------------
# schedule
# ----------------------------------------------------------------------------------------------
def schedule(idx: np.ndarray, E: int):
    """One rank's schedule when every expert is local (R = 1).

    The Blog's "Scheduling" section builds, per local expert, a contiguous region of the
    destination buffer (region offsets are the exclusive scan of the per-expert counts), and
    fills each region with that expert's routes. With a single source rank the Notes' sort key
    (local expert, per-source ordinal, source rank) is (expert, route order), i.e. a stable sort
    of the route ids by expert.

    Returns counts [E], offsets [E+1] (exclusive scan, offsets[E] = T*K), perm [T*K]
    (slot -> route id i*K+k) and inv_perm [T*K] (route id -> slot), all int32.
    """
    flat = np.asarray(idx, dtype=np.int64).ravel()
    counts = np.bincount(flat, minlength=E)[:E]
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind='stable')
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    return (counts.astype(np.int32), offsets.astype(np.int32), perm.astype(np.int32),
            inv.astype(np.int32))


def pull_schedule(routing: np.ndarray, rank: int, L: int):
    """Pull-dispatch schedule of rank ``rank`` for R source ranks (Blog, "Scheduling").

    routing[r, i, k] is the global expert of route k of token i on source rank r; rank c owns
    global experts [c*L, (c+1)*L). Output: per-local-expert counts T [L], per (expert, source)
    counts M [L, R], region offsets S [L] and the table Phi [sum T, 2] of (src_rank, src_index)
    with src_index = i*K + k.

    Order inside a region, by definition (Notes, "Pull dispatch, push combine"): routes sorted by
    (local expert, per-source ordinal, source rank), where the ordinal of a route is how many
    earlier routes (in (i, k) order) of the same source rank went to the same local expert.
    """
    R, N, K = routing.shape
    routes = []        # (local expert, ordinal, source rank, src_index)
    ordinal = {}
    for r in range(R):
        for i in range(N):
            for k in range(K):
                e = int(routing[r, i, k])
                if e // L != rank:
                    continue
                le = e - rank * L
                o = ordinal.get((le, r), 0)
                ordinal[(le, r)] = o + 1
                routes.append((le, o, r, i * K + k))
    Tc = np.zeros(L, dtype=np.int64)
    M = np.zeros((L, R), dtype=np.int64)
    for le, _, r, _ in routes:
        Tc[le] += 1
        M[le, r] += 1
    S = np.zeros(L, dtype=np.int64)
    S[1:] = np.cumsum(Tc)[:-1]
    routes.sort(key=lambda q: (q[0], q[1], q[2]))
    phi = np.array([(q[2], q[3]) for q in routes], dtype=np.int64).reshape(-1, 2)
    return Tc, M, S, phi


# ----------------------------------------------------------------------------------------------
# experts
# ----------------------------------------------------------------------------------------------
def swiglu_expert(X, w_gate, w_up, w_down, return_parts=False):
    """E(x) = W_down (SiLU(W_gate x) (*) W_up x) on rows X [n, D] (Blog, MoE layer equation)."""
    X = np.asarray(X, dtype=np.float64)
    A = X @ np.asarray(w_gate, dtype=np.float64).T
    U = X @ np.asarray(w_up, dtype=np.float64).T
    H = silu(A) * U
    Y = H @ np.asarray(w_down, dtype=np.float64).T
    if return_parts:
        return Y, A, U, H
    return Y


def moe_forward(x, logits, w_gate, w_up, w_down, K, ws_gate=None, ws_up=None, ws_down=None,
                h_transform=None):
    """MoE(x, s) for every row of x (Blog, "Overlapping computation and communication in MoE").

    Returns (out [T, D], idx [T, K], g [T, K], y [T, K, D] per-route expert outputs,
    shared [T, D] or None), all fp64 except idx. ``w_*`` may be arrays [E, ...] or callables
    e -> array (to stream large weights). ``h_transform`` (optional) maps the fp64 gated
    activation before the down projection (the MXFP8 path quantises it there).
    """
    x = np.asarray(x, dtype=np.float64)
    T, D = x.shape
    idx = route_topk(logits, K)
    g = routing_weights(logits, idx)
    y = np.zeros((T, K, D), dtype=np.float64)
    E = np.asarray(logits).shape[1]
    get = lambda w, e: w(e) if callable(w) else w[e]
    for e in range(E):
        t, k = np.nonzero(idx == e)
        if t.size == 0:
            continue
        Xe = x[t]
        A = Xe @ np.asarray(get(w_gate, e), dtype=np.float64).T
        U = Xe @ np.asarray(get(w_up, e), dtype=np.float64).T
        H = silu(A) * U
        if h_transform is not None:
            H = h_transform(H)
        y[t, k] = H @ np.asarray(get(w_down, e), dtype=np.float64).T
    out = np.einsum('tk,tkd->td', g, y)
    sh = None
    if ws_gate is not None:
        sh = swiglu_expert(x, ws_gate, ws_up, ws_down)
        out = out + sh
    return out, idx, g, y, sh


def combine(shared, y_routes, g):
    """out[t] = shared[t] + sum_k g[t, k] * y[t*K + k] (Blog, weighted sum after the combine)."""
    T, K = g.shape
    yr = np.asarray(y_routes, dtype=np.float64).reshape(T, K, -1)
    out = np.einsum('tk,tkd->td', np.asarray(g, dtype=np.float64), yr)
    if shared is not None:
        out = out + np.asarray(shared, dtype=np.float64)
    return out


# ----------------------------------------------------------------------------------------------
# backward
# ----------------------------------------------------------------------------------------------
def _expert_backward(X, dY, w_gate, w_up, w_down):
    """Backward of E(x) on rows X with output gradient dY (both [n, .]), fp64.

    Returns dX [n, D], dW_gate [I, D], dW_up [I, D], dW_down [D, I], H [n, I], dH [n, I].
    """
    Wg = np.asarray(w_gate, dtype=np.float64)
    Wu = np.asarray(w_up, dtype=np.float64)
    Wd = np.asarray(w_down, dtype=np.float64)
    A = X @ Wg.T
    U = X @ Wu.T
    sg = sigmoid(A)
    Sa = A * sg
    H = Sa * U
    dH = dY @ Wd
    dA = dH * U * sg * (1.0 + A * (1.0 - sg))
    dU = dH * Sa
    dX = dA @ Wg + dU @ Wu
    return dX, dA.T @ X, dU.T @ X, dY.T @ H, H, dH


def d_logits_from_dg(g, idx, dg, E):
    """Gradient w.r.t. the router logits. With s = softmax(l), g_i = s_i / sum_{j in sel} s_j =
    exp(l_i) / sum_{j in sel} exp(l_j), so dl_i = g_i (dg_i - sum_j g_j dg_j) on the selected
    experts and 0 elsewhere (top-k selection is piecewise constant)."""
    T, K = g.shape
    inner = (g * dg).sum(axis=1, keepdims=True)
    dsel = g * (dg - inner)
    out = np.zeros((T, E), dtype=np.float64)
    np.put_along_axis(out, idx.astype(np.int64), dsel, axis=1)
    return out


def moe_backward(x, logits, w_gate, w_up, w_down, K, dout, ws_gate=None, ws_up=None, ws_down=None):
    """Gradients of sum(dout * MoE(x, s)) for the whole layer.

    Returns dict with dx [T, D], dW_gate/dW_up [E, I, D], dW_down [E, D, I], dg [T, K],
    d_logits [T, E], and dWs_* for the shared expert. The router-weight gradient dg[t, k] is
    <dout[t], E_i(x_t)>, which equals <H_i, W_down^T (dout)> (Notes, "The production details",
    the SonicMoE identity that avoids materialising the down-projection output).
    """
    x = np.asarray(x, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    T, D = x.shape
    E = np.asarray(logits).shape[1]
    idx = route_topk(logits, K)
    g = routing_weights(logits, idx)
    I = np.asarray(w_gate[0]).shape[0]
    dx = np.zeros((T, D))
    dWg = np.zeros((E, I, D))
    dWu = np.zeros((E, I, D))
    dWd = np.zeros((E, D, I))
    dg = np.zeros((T, K))
    for e in range(E):
        t, k = np.nonzero(idx == e)
        if t.size == 0:
            continue
        dY = g[t, k][:, None] * dout[t]
        dX, a, b, c, H, dH = _expert_backward(x[t], dY, w_gate[e], w_up[e], w_down[e])
        dx[t] += dX
        dWg[e], dWu[e], dWd[e] = a, b, c
        # <H, W_down^T dout> with the unweighted output gradient
        dg[t, k] = np.einsum('ni,ni->n', H, dout[t] @ np.asarray(w_down[e], dtype=np.float64))
    res = dict(dx=dx, dW_gate=dWg, dW_up=dWu, dW_down=dWd, dg=dg, idx=idx, g=g,
               d_logits=d_logits_from_dg(g, idx, dg, E))
    if ws_gate is not None:
        dXs, a, b, c, _, _ = _expert_backward(x, dout, ws_gate, ws_up, ws_down)
        res['dx'] = dx + dXs
        res['dWs_gate'], res['dWs_up'], res['dWs_down'] = a, b, c
    return res


def router_logits(x, w_router):
    """Router projection: logits[t, e] = <x[t], W_r[e]> with W_r [E, D] (the router of the Blog's
    "Overlapping computation and communication in MoE", whose softmax gives the weights s)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w_router, dtype=np.float64).T


def router_backward(x, w_router, d_logits):
    """Backward of router_logits given the gradient w.r.t. the logits [T, E] (d_logits_from_dg):
    dW_r = d_logits^T x [E, D] and the router's share of the input gradient dx = d_logits W_r
    [T, D], to be added to the experts' (the logits are linear in both x and W_r)."""
    dl = np.asarray(d_logits, dtype=np.float64)
    return dl.T @ np.asarray(x, dtype=np.float64), dl @ np.asarray(w_router, dtype=np.float64)


# ----------------------------------------------------------------------------------------------
# expert-level entry (slots already grouped by expert: one expert-parallel rank's share)
# ----------------------------------------------------------------------------------------------
def experts_forward(x_slot, counts, w_gate, w_up, w_down):
    """Unweighted expert outputs per slot: rows offsets[e]..offsets[e+1] of x_slot go to expert e.
    (The router weight is applied by the source rank's weighted sum, Blog "Scheduling".)"""
    x_slot = np.asarray(x_slot, dtype=np.float64)
    y = np.zeros_like(x_slot)
    off = np.concatenate([[0], np.cumsum(counts)])
    for e in range(len(counts)):
        a, b = off[e], off[e + 1]
        if b > a:
            y[a:b] = swiglu_expert(x_slot[a:b], w_gate[e], w_up[e], w_down[e])
    return y


def experts_backward(x_slot, counts, g, dy_slot, w_gate, w_up, w_down):
    """Backward of the share: each slot's output enters the loss as g_j * E_e(x_j) against the
    upstream gradient dy_slot[j] (the reverse-combine of the source's output gradient).

    Returns dx_slot [S, D], dg [S] = <dy_j, E_e(x_j)>, dW_gate/dW_up [E, I, D], dW_down [E, D, I].
    """
    x_slot = np.asarray(x_slot, dtype=np.float64)
    dy_slot = np.asarray(dy_slot, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    S, D = x_slot.shape
    E = len(counts)
    I = np.asarray(w_gate[0]).shape[0]
    off = np.concatenate([[0], np.cumsum(counts)])
    dx = np.zeros((S, D))
    dg = np.zeros(S)
    dWg = np.zeros((E, I, D))
    dWu = np.zeros((E, I, D))
    dWd = np.zeros((E, D, I))
    for e in range(E):
        a, b = off[e], off[e + 1]
        if b <= a:
            continue
        dYw = g[a:b, None] * dy_slot[a:b]
        dX, p, q, r, H, _ = _expert_backward(x_slot[a:b], dYw, w_gate[e], w_up[e], w_down[e])
        dx[a:b], dWg[e], dWu[e], dWd[e] = dX, p, q, r
        dg[a:b] = np.einsum('ni,ni->n', H, dy_slot[a:b] @ np.asarray(w_down[e], dtype=np.float64))
    return dict(dx_slot=dx, dg=dg, dW_gate=dWg, dW_up=dWu, dW_down=dWd)


def shared_backward(x, dy, ws_gate, ws_up, ws_down):
    """Backward of the shared expert (no router weight): dx, dW_gate, dW_up, dW_down."""
    dX, a, b, c, _, _ = _expert_backward(np.asarray(x, dtype=np.float64), np.asarray(dy, dtype=np.float64),
                                         ws_gate, ws_up, ws_down)
    return dict(dx=dX, dW_gate=a, dW_up=b, dW_down=c)


# ----------------------------------------------------------------------------------------------
# MXFP8 expert-level forward and backward
# ----------------------------------------------------------------------------------------------
# The Notes ("The production details") run the routed experts in MXFP8 in training, forward and
# backward, without saying which operand is quantised along which axis. Reading taken here: every
# grouped GEMM quantises both of its operands along its own contraction dimension (OCP MX blocks of
# 32); activations are quantised from their high-precision values (bf16 inputs, the fp32 replay
# a, u, h and the fp32 SwiGLU backward); the weights exist only as the forward's MX tensors, so
# the backward re-quantises their dequantised values along its contraction axis. Along the slot
# axis (weight gradients) the blocks start at each expert's first slot, the last one zero-padded.
def mx_along(v, axis, quantize=True):
    """MX round trip of v [n, m] along `axis` (0: down each column, 1: along each row). Blocks of
    32 from index 0; a short last block is padded with zeros, which changes no block maximum."""
    v = np.asarray(v, dtype=np.float64)
    if not quantize:
        return v
    from .mx import mx_roundtrip, MX_BLOCK
    w = v if axis == 1 else v.T
    n = w.shape[1]
    pad = (-n) % MX_BLOCK
    if pad:
        w = np.concatenate([w, np.zeros((w.shape[0], pad))], axis=1)
    r = mx_roundtrip(w)[:, :n]
    return r if axis == 1 else r.T


def _mx_weights(wq, sc):
    from .mx import mx_dequantize
    return mx_dequantize(np.asarray(wq, dtype=np.uint8), np.asarray(sc, dtype=np.uint8))


def experts_forward_mx(x_slot, counts, wq_gate, sc_gate, wq_up, sc_up, wq_down, sc_down, quantize=True):
    """MXFP8 experts on slot rows (one expert-parallel rank's share): x quantised along D, the
    gated activation h along I before the down projection; weights are the MX tensors
    [E, I, D] (gate, up; blocks along D) and [E, D, I] (down; blocks along I). Unweighted outputs
    per slot. quantize=False skips the activation round trips (the fp64 path on the same weights)."""
    return experts_forward_mx_w(x_slot, counts, _mx_weights(wq_gate, sc_gate), _mx_weights(wq_up, sc_up),
                                _mx_weights(wq_down, sc_down), quantize)


def experts_forward_mx_w(x_slot, counts, Wg, Wu, Wd, quantize=True):
    """experts_forward_mx on already dequantised MX weights Wg, Wu [E, I, D], Wd [E, D, I]."""
    x_slot = np.asarray(x_slot, dtype=np.float64)
    y = np.zeros_like(x_slot)
    off = np.concatenate([[0], np.cumsum(counts)])
    for e in range(len(counts)):
        a, b = off[e], off[e + 1]
        if b <= a:
            continue
        Xq = mx_along(x_slot[a:b], 1, quantize)
        H = silu(Xq @ Wg[e].T) * (Xq @ Wu[e].T)
        y[a:b] = mx_along(H, 1, quantize) @ Wd[e].T
    return y


def experts_backward_mx(x_slot, counts, g, dy_slot, wq_gate, sc_gate, wq_up, sc_up, wq_down, sc_down,
                        quantize=True):
    """Backward of experts_forward_mx with router weights g per slot (each slot enters the loss as
    g_j E_e(x_j) against dy_slot[j]), every GEMM in MXFP8 as read above:

        replay     a = Q_D(x) W_gate^T,  u = Q_D(x) W_up^T,  h = SiLU(a) u
        dgrad-down dh' = Q_D(dy) Q_D(W_down)                  (W_down [D, I] quantised down D)
        dg         <h, dh'>                                    (fp64 here, fp32 on the device)
        SwiGLU     dh = g dh',  da = dh u sig(a)(1 + a(1 - sig(a))),  du = dh SiLU(a)
        dgrad-up   dx = Q_I(da) Q_I(W_gate) + Q_I(du) Q_I(W_up)    (W [I, D] quantised down I)
        wgrad      dW_down = Q_n(g dy)^T Q_n(h),  dW_gate = Q_n(da)^T Q_n(x),  dW_up = Q_n(du)^T Q_n(x)

    with Q_n blocks along the expert's slots. quantize=False makes every Q the identity, which is
    experts_backward on the dequantised weights."""
    return experts_backward_mx_w(x_slot, counts, g, dy_slot, _mx_weights(wq_gate, sc_gate), _mx_weights(wq_up, sc_up),
                                 _mx_weights(wq_down, sc_down), quantize)


def experts_backward_mx_w(x_slot, counts, g, dy_slot, Wg, Wu, Wd, quantize=True, return_parts=False):
    """experts_backward_mx on already dequantised MX weights Wg, Wu [E, I, D], Wd [E, D, I]. Row i
    of dW_gate / dW_up and column i of dW_down depend only on rows i of Wg, Wu and column i of Wd
    (every quantisation they meet runs down a single column), so they can be had from the
    restriction to that unit. return_parts adds, per expert, the unquantised operands that are
    computed rather than given (h, da, du, g dy) under 'parts'."""
    x_slot = np.asarray(x_slot, dtype=np.float64)
    dy_slot = np.asarray(dy_slot, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    Wg, Wu, Wd = (np.asarray(w, dtype=np.float64) for w in (Wg, Wu, Wd))
    S, D = x_slot.shape
    E = len(counts)
    I = Wg.shape[1]
    off = np.concatenate([[0], np.cumsum(counts)])
    q = lambda v, ax: mx_along(v, ax, quantize)
    parts = {}
    dx = np.zeros((S, D))
    dg = np.zeros(S)
    dWg = np.zeros((E, I, D))
    dWu = np.zeros((E, I, D))
    dWd = np.zeros((E, D, I))
    for e in range(E):
        a, b = off[e], off[e + 1]
        if b <= a:
            continue
        X, dy, ge = x_slot[a:b], dy_slot[a:b], g[a:b, None]
        Xq = q(X, 1)
        A = Xq @ Wg[e].T
        U = Xq @ Wu[e].T
        sg = sigmoid(A)
        Sa = A * sg
        H = Sa * U
        dhp = q(dy, 1) @ q(Wd[e], 0)
        dg[a:b] = np.einsum('ni,ni->n', H, dhp)
        dh = ge * dhp
        dA = dh * U * sg * (1.0 + A * (1.0 - sg))
        dU = dh * Sa
        dx[a:b] = q(dA, 1) @ q(Wg[e], 0) + q(dU, 1) @ q(Wu[e], 0)
        dWd[e] = q(ge * dy, 0).T @ q(H, 0)
        Xn = q(X, 0)
        dWg[e] = q(dA, 0).T @ Xn
        dWu[e] = q(dU, 0).T @ Xn
        if return_parts:
            parts[e] = dict(H=H, dA=dA, dU=dU, gdy=ge * dy)
    res = dict(dx_slot=dx, dg=dg, dW_gate=dWg, dW_up=dWu, dW_down=dWd)
    if return_parts:
        res['parts'] = parts
    return res


def moe_forward_mx(x, logits, w_gate, w_up, w_down, K, ws_gate=None, ws_up=None, ws_down=None, quantize=True,
                   return_h=False):
    """The whole layer with the routed experts in MXFP8 (Notes, "The production details": activation
    quantisation fused into dispatch, the grouped GEMMs and the gated activation; the shared expert
    stays in BF16).

    Routing and combine are those of moe_forward (Blog, MoE layer equation). Each routed slot carries
    its token's row of x quantised along D (dispatch copies and quantises token rows, so a slot's
    blocks are its token's); the gated activation h of a slot is quantised along I before the down
    projection. w_gate, w_up [E, I, D] and w_down [E, D, I] are the dequantised MX weights (arrays,
    or callables e -> array to stream them); the shared expert works on the unquantised x with its
    own (BF16-valued) weights. quantize=False skips both activation round trips, which is moe_forward
    on the same weights.

    Returns (out [T, D], idx [T, K], g [T, K], y [T, K, D] per-route outputs, shared [T, D] or None);
    with return_h also a dict e -> (t, k, H) of each expert's unquantised gated activation rows (the
    values whose quantisation decisions the device takes in fp32)."""
    x = np.asarray(x, dtype=np.float64)
    T, D = x.shape
    E = np.asarray(logits).shape[1]
    idx = route_topk(logits, K)
    g = routing_weights(logits, idx)
    xq = mx_along(x, 1, quantize)
    get = lambda w, e: w(e) if callable(w) else w[e]
    y = np.zeros((T, K, D))
    hs = {}
    for e in range(E):
        t, k = np.nonzero(idx == e)
        if t.size == 0:
            continue
        Xe = xq[t]
        H = silu(Xe @ np.asarray(get(w_gate, e), dtype=np.float64).T) * (Xe @ np.asarray(get(w_up, e), dtype=np.float64).T)
        y[t, k] = mx_along(H, 1, quantize) @ np.asarray(get(w_down, e), dtype=np.float64).T
        if return_h:
            hs[e] = (t, k, H)
    out = np.einsum('tk,tkd->td', g, y)
    sh = None
    if ws_gate is not None:
        sh = swiglu_expert(x, ws_gate, ws_up, ws_down)
        out = out + sh
    res = (out, idx, g, y, sh)
    return res + (hs,) if return_h else res
