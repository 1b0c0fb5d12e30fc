"""Pins of the oracle's forward and backward: brute force, dense-FFN reduction against torch's
own CPU ops, finite differences and the router-gradient identity. CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def tiny_layer(seed, T=6, D=5, I=3, E=4, K=2, shared=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, D))
    lg = rng.standard_normal((T, E)).astype(np.float32)
    wg = rng.standard_normal((E, I, D)) / math.sqrt(D)
    wu = rng.standard_normal((E, I, D)) / math.sqrt(D)
    wd = rng.standard_normal((E, D, I)) / math.sqrt(I)
    sh = (rng.standard_normal((I, D)), rng.standard_normal((I, D)), rng.standard_normal((D, I))) if shared else (None,) * 3
    return x, lg, wg, wu, wd, sh


def brute_forward(x, lg, wg, wu, wd, K, sh):
    """Per-token pure-Python loops of MoE(x, s) with the Blog's equation."""
    T, D = x.shape
    E, I, _ = wg.shape
    out = np.zeros((T, D))

    def ffn(xt, g_, u_, d_):
        h = []
        for r in range(len(g_)):
            a = sum(g_[r][c] * xt[c] for c in range(D))
            b = sum(u_[r][c] * xt[c] for c in range(D))
            h.append(a / (1.0 + math.exp(-a)) * b)
        return [sum(d_[c][r] * h[r] for r in range(len(h))) for c in range(D)]

    for t in range(T):
        row = [float(v) for v in lg[t]]
        sel = sorted(range(E), key=lambda e: (-row[e], e))[:K]
        z = [math.exp(row[e] - max(row)) for e in sel]
        g = [v / sum(z) for v in z]
        acc = [0.0] * D
        for gi, e in zip(g, sel):
            y = ffn(x[t], wg[e], wu[e], wd[e])
            acc = [a + gi * b for a, b in zip(acc, y)]
        if sh[0] is not None:
            y = ffn(x[t], sh[0], sh[1], sh[2])
            acc = [a + b for a, b in zip(acc, y)]
        out[t] = acc
    return out


@pytest.mark.parametrize('seed', [0, 1])
def test_forward_brute_force(seed):
    x, lg, wg, wu, wd, sh = tiny_layer(seed)
    out, idx, g, y, shv = oracle.moe_forward(x, lg, wg, wu, wd, 2, *sh)
    np.testing.assert_allclose(out, brute_forward(x, lg, wg, wu, wd, 2, sh), rtol=1e-12, atol=1e-12)
    # combine of the per-route outputs reproduces the layer output
    np.testing.assert_allclose(oracle.combine(shv, y.reshape(-1, x.shape[1]), g), out, rtol=1e-13, atol=1e-13)


def test_dense_reduction_against_torch():
    """E = 1, K = 1: g = 1 and the layer is E_shared(x) + E_0(x), two plain SwiGLU FFNs,
    evaluated here with torch's CPU matmul and SiLU."""
    cfg = synth.scaled(synth.TINY, 'dense', E=1, K=1)
    L = synth.host_layer(cfg)
    out, idx, g, _, _ = oracle.moe_forward(L.x, L.logits, L.w_gate, L.w_up, L.w_down, 1,
                                           L.ws_gate, L.ws_up, L.ws_down)
    assert np.all(idx == 0) and np.all(g == 1.0)
    X = torch.from_numpy(L.x).double()
    F = torch.nn.functional

    def ffn(wg_, wu_, wd_):
        wg_, wu_, wd_ = (torch.from_numpy(np.asarray(w)).double() for w in (wg_, wu_, wd_))
        return (F.silu(X @ wg_.T) * (X @ wu_.T)) @ wd_.T

    ref = ffn(L.w_gate[0], L.w_up[0], L.w_down[0]) + ffn(L.ws_gate, L.ws_up, L.ws_down)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_experts_forward_matches_layer():
    """Slot-level entry (share): gathering the layer's routes by expert and running
    experts_forward gives the same per-route outputs as moe_forward."""
    x, lg, wg, wu, wd, _ = tiny_layer(3, T=9, E=5, K=3, shared=False)
    out, idx, g, y, _ = oracle.moe_forward(x, lg, wg, wu, wd, 3)
    counts, offsets, perm, inv = oracle.schedule(idx, 5)
    ys = oracle.experts_forward(x[perm // 3], counts, wg, wu, wd)
    np.testing.assert_allclose(ys[inv].reshape(9, 3, -1), y, rtol=1e-13, atol=1e-13)


def _fd(f, arr, eps=1e-6):
    g = np.zeros_like(arr)
    it = np.nditer(arr, flags=['multi_index'])
    for _ in it:
        i = it.multi_index
        old = arr[i]
        arr[i] = old + eps
        fp = f()
        arr[i] = old - eps
        fm = f()
        arr[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


def test_backward_finite_differences():
    x, lg, wg, wu, wd, sh = tiny_layer(5, T=5, D=4, I=3, E=4, K=2)
    lg = lg.astype(np.float64)
    sg, su, sd = (np.array(a) for a in sh)
    dout = np.random.default_rng(9).standard_normal(x.shape)
    idx0 = oracle.route_topk(lg, 2)

    def loss():
        assert np.array_equal(oracle.route_topk(lg, 2), idx0), 'selection changed under the step'
        return float((dout * oracle.moe_forward(x, lg, wg, wu, wd, 2, sg, su, sd)[0]).sum())

    res = oracle.moe_backward(x, lg, wg, wu, wd, 2, dout, sg, su, sd)
    for name, arr in [('dx', x), ('dW_gate', wg), ('dW_up', wu), ('dW_down', wd),
                      ('d_logits', lg), ('dWs_gate', sg), ('dWs_up', su), ('dWs_down', sd)]:
        fd = _fd(loss, arr)
        an = res[name]
        err = np.max(np.abs(fd - an)) / max(np.max(np.abs(fd)), 1e-12)
        assert err < 1e-6, (name, err)
    # d_logits vanish off the selected set
    mask = np.zeros_like(lg, dtype=bool)
    np.put_along_axis(mask, idx0.astype(np.int64), True, axis=1)
    assert np.all(res['d_logits'][~mask] == 0)


def test_router_gradient_identity():
    """dg[t, k] = <dout[t], E_i(x_t)> (the loss gradient w.r.t. g) equals <H, W_down^T dout>."""
    x, lg, wg, wu, wd, _ = tiny_layer(6, T=7, E=5, K=3, shared=False)
    dout = np.random.default_rng(1).standard_normal(x.shape)
    out, idx, g, y, _ = oracle.moe_forward(x, lg, wg, wu, wd, 3)
    res = oracle.moe_backward(x, lg, wg, wu, wd, 3, dout)
    np.testing.assert_allclose(res['dg'], np.einsum('td,tkd->tk', dout, y), rtol=1e-12, atol=1e-13)


def test_experts_backward_finite_differences():
    rng = np.random.default_rng(4)
    S, D, I, E = 7, 4, 3, 3
    counts = np.array([3, 0, 4])
    xs = rng.standard_normal((S, D))
    g = rng.random(S)
    dy = rng.standard_normal((S, D))
    wg = rng.standard_normal((E, I, D))
    wu = rng.standard_normal((E, I, D))
    wd = rng.standard_normal((E, D, I))

    def loss():
        return float((dy * g[:, None] * oracle.experts_forward(xs, counts, wg, wu, wd)).sum())

    res = oracle.experts_backward(xs, counts, g, dy, wg, wu, wd)
    for name, arr in [('dx_slot', xs), ('dg', g), ('dW_gate', wg), ('dW_up', wu), ('dW_down', wd)]:
        fd = _fd(loss, arr)
        err = np.max(np.abs(fd - res[name])) / max(np.max(np.abs(fd)), 1e-12)
        assert err < 1e-6, (name, err)
    assert np.all(res['dW_gate'][1] == 0) and np.all(res['dW_down'][1] == 0)


def test_shared_backward_finite_differences():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((4, 3))
    dy = rng.standard_normal((4, 3))
    wg, wu, wd = rng.standard_normal((2, 3)), rng.standard_normal((2, 3)), rng.standard_normal((3, 2))

    def loss():
        return float((dy * oracle.swiglu_expert(x, wg, wu, wd)).sum())

    res = oracle.shared_backward(x, dy, wg, wu, wd)
    for name, arr in [('dx', x), ('dW_gate', wg), ('dW_up', wu), ('dW_down', wd)]:
        fd = _fd(loss, arr)
        assert np.max(np.abs(fd - res[name])) < 1e-6 * max(1, np.max(np.abs(fd))), name
