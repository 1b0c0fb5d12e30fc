"""Pins of the oracle's router backward (dW_r = d_logits^T x, dx_router = d_logits W_r). CPU only.

The layer's loss sum(dout * MoE(x, logits)) with logits = x W_r^T is differentiated by central
finite differences in fp64 through the whole layer (routing, experts, shared expert, combine)
and compared with the analytic gradients: dW_r = router_backward(...)[0] with d_logits from
moe_backward, and dx = moe_backward's dx + router_backward(...)[1]. The routing must not change
under the perturbations (checked), so the top-k selection is constant there.
"""
import numpy as np

import oracle


def _layer(seed, T=7, D=8, I=6, E=5, K=2, Is=4):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, D))
    wr = rng.standard_normal((E, D)) / np.sqrt(D)
    wg, wu = rng.standard_normal((E, I, D)) / np.sqrt(D), rng.standard_normal((E, I, D)) / np.sqrt(D)
    wd = rng.standard_normal((E, D, I)) / np.sqrt(I)
    sg, su, sd = rng.standard_normal((Is, D)) / np.sqrt(D), rng.standard_normal((Is, D)) / np.sqrt(D), rng.standard_normal((D, Is)) / np.sqrt(Is)
    dout = rng.standard_normal((T, D))
    return x, wr, (wg, wu, wd), (sg, su, sd), dout, K


def _loss(x, wr, w, ws, dout, K):
    lg = oracle.router_logits(x, wr)
    out, idx, *_ = oracle.moe_forward(x, lg, *w, K, *ws)
    return float(np.sum(dout * out)), idx


def test_router_backward_matches_central_differences_through_the_layer():
    for seed in range(3):
        x, wr, w, ws, dout, K = _layer(seed)
        lg = oracle.router_logits(x, wr)
        g = oracle.moe_backward(x, lg, *w, K, dout, *ws)
        dwr, dxr = oracle.router_backward(x, wr, g['d_logits'])
        dx_total = g['dx'] + dxr
        _, idx0 = _loss(x, wr, w, ws, dout, K)
        eps = 1e-6
        for arr, grad in ((wr, dwr), (x, dx_total)):
            num = np.zeros_like(arr)
            for i in np.ndindex(arr.shape):
                keep = arr[i]
                arr[i] = keep + eps
                lp, ip = _loss(x, wr, w, ws, dout, K)
                arr[i] = keep - eps
                lm, im = _loss(x, wr, w, ws, dout, K)
                arr[i] = keep
                assert np.array_equal(ip, idx0) and np.array_equal(im, idx0), 'routing changed under the perturbation'
                num[i] = (lp - lm) / (2 * eps)
            rel = np.abs(num - grad).max() / np.abs(grad).max()
            assert rel < 1e-6, (seed, rel)


def test_router_backward_closed_forms():
    """One token, one expert chosen out of two (K = 1, g = 1, d_logits = 0): no router gradient;
    K = E = 2 with equal logits gives g = 1/2 each and d_logit_i = (dg_i - dg_j) / 4."""
    x = np.array([[1.0, 2.0]])
    wr = np.array([[0.5, -0.25], [1.0, 1.0]])
    dl = np.array([[3.0, -1.0]])
    dwr, dxr = oracle.router_backward(x, wr, dl)
    np.testing.assert_array_equal(dwr, [[3.0, 6.0], [-1.0, -2.0]])
    np.testing.assert_array_equal(dxr, [[0.5, -1.75]])
    g = np.array([[0.5, 0.5]])
    idx = np.array([[0, 1]])
    np.testing.assert_allclose(oracle.d_logits_from_dg(g, idx, np.array([[1.0, 3.0]]), 2), [[-0.5, 0.5]], rtol=0, atol=1e-15)
