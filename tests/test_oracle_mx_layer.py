"""Pins of the oracle's whole-layer MXFP8 forward (oracle.moe_forward_mx). CPU only.

* With quantisation off it is moe_forward on the same weights (pinned by brute force and the
  dense reduction in test_oracle_experts.py).
* It equals the expert-level MXFP8 forward (whose quantisation axes test_oracle_mx_axes.py fixes
  by hand) run on the dispatched slots, followed by the combine: the layer quantises each token's
  row once and every slot of that token carries the same blocks.
* A closed form with one expert: the routed path sees x quantised along D, the shared expert the
  unquantised x, and the two differ by a worked-out amount.
"""
import numpy as np

import oracle
from test_oracle_mx_axes import case_x_along_D, S, D


def _layer(seed, T=96, Dd=64, Ii=64, E=6, K=2, Is=32):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, Dd))
    logits = rng.standard_normal((T, E))
    deq = lambda s: oracle.mx_roundtrip(rng.standard_normal(s) / np.sqrt(s[-1]))
    w = [deq((E, Ii, Dd)), deq((E, Ii, Dd)), deq((E, Dd, Ii))]
    ws = [rng.standard_normal((Is, Dd)) / 8, rng.standard_normal((Is, Dd)) / 8, rng.standard_normal((Dd, Is)) / 6]
    return x, logits, w, ws, K


def test_unquantised_is_moe_forward():
    x, logits, w, ws, K = _layer(1)
    got = oracle.moe_forward_mx(x, logits, *w, K, *ws, quantize=False)
    ref = oracle.moe_forward(x, logits, *w, K, *ws)
    np.testing.assert_array_equal(got[1], ref[1])
    for a, b in zip((got[0], got[2], got[3], got[4]), (ref[0], ref[2], ref[3], ref[4])):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_equals_expert_level_forward_on_dispatched_slots():
    x, logits, w, ws, K = _layer(2)
    T, E = logits.shape
    out, idx, g, y, sh = oracle.moe_forward_mx(x, logits, *w, K, *ws)
    counts, offsets, perm, inv = oracle.schedule(idx, E)
    y_slot = oracle.experts_forward_mx_w(x[perm // K], counts, *w)
    np.testing.assert_allclose(y.reshape(T * K, -1), y_slot[inv], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out, oracle.combine(sh, y_slot[inv], g), rtol=1e-12, atol=1e-12)
    assert np.abs(y - oracle.moe_forward_mx(x, logits, *w, K, *ws, quantize=False)[3]).max() > 1e-3


def test_closed_form_routed_quantised_shared_not():
    """One expert, K = 1 (g = 1), the x of the expert-level case x[:, 0] = 2^20, x[:, d>0] = 1:
    the routed output is 2048 (x's ones flushed along D). The shared expert gets W_gate column 0
    = 2^-14 (else 2), W_up column 0 = 2^-20 (else 1), W_down = 1 and the unquantised x:
    a = 64 + 31 * 2 = 126, u = 1 + 31 = 32, h = 4032, output 32 * 4032 = 129024. Total 131072;
    a shared expert on quantised x would give 2048 + 2048 = 4096."""
    x, wg, wu, wd = case_x_along_D()
    logits = np.zeros((S, 1))
    ws_gate, ws_up, ws_down = wg[0], wu[0], wd[0]
    out, idx, g, y, sh = oracle.moe_forward_mx(x, logits, wg, wu, wd, 1, ws_gate, ws_up, ws_down)
    assert np.all(idx == 0) and np.all(g == 1.0)
    np.testing.assert_array_equal(y[:, 0], np.full((S, D), 2048.0))
    np.testing.assert_array_equal(sh, np.full((S, D), 129024.0))
    np.testing.assert_array_equal(out, np.full((S, D), 131072.0))


def test_token_outputs_depend_on_their_own_token_only():
    x, logits, w, ws, K = _layer(3)
    base = oracle.moe_forward_mx(x, logits, *w, K, *ws)[0]
    x2 = x.copy()
    x2[17] *= 2.0 ** 12
    got = oracle.moe_forward_mx(x2, logits, *w, K, *ws)[0]
    keep = np.arange(len(x)) != 17
    np.testing.assert_array_equal(got[keep], base[keep])


def test_return_h_holds_the_unquantised_gated_activation():
    x, logits, w, ws, K = _layer(4)
    *_, hs = oracle.moe_forward_mx(x, logits, *w, K, *ws, return_h=True)
    xq = oracle.mx_roundtrip(x)
    for e, (t, k, H) in hs.items():
        A = xq[t] @ w[0][e].T
        np.testing.assert_allclose(H, oracle.silu(A) * (xq[t] @ w[1][e].T), rtol=1e-13, atol=1e-13)
