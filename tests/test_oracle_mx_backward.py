"""Pins of the oracle's MXFP8 expert-level forward and backward (CPU only).

* The per-axis MX round trip (blocks of 32 from index 0, short last block zero-padded) is checked
  block by block against the row quantiser, whose bytes are pinned by the golden cases.
* With every quantisation switched off, the MXFP8 forward and backward reduce to the fp64
  experts_forward / experts_backward on the same (dequantised) weights; those are pinned by
  brute force and central finite differences. A dropped term, a wrong sign or a transposed
  operand in the quantised formulas breaks this reduction.
* With quantisation on, each operand moves by at most 2^-4 of its block's scale range, so the
  gradients stay within a few percent of the unquantised ones (a bound, not parity).
"""
import math

import numpy as np
import pytest

import oracle


def _mx_weights(rng, E, R, C, std):
    w = rng.standard_normal((E, R, C)) * std
    q, sc = oracle.mx_quantize(w)
    return q, sc


def _share(seed, S=70, D=64, I=32, counts=(37, 0, 33)):
    rng = np.random.default_rng(seed)
    E = len(counts)
    x = rng.standard_normal((S, D))
    dy = rng.standard_normal((S, D))
    g = rng.random(S)
    wg = _mx_weights(rng, E, I, D, 1 / math.sqrt(D))
    wu = _mx_weights(rng, E, I, D, 1 / math.sqrt(D))
    wd = _mx_weights(rng, E, D, I, 1 / math.sqrt(I))
    return x, dy, g, np.array(counts), wg, wu, wd


@pytest.mark.parametrize('n,m', [(70, 5), (32, 3), (5, 64), (1, 33)])
def test_mx_along_blockwise(n, m):
    rng = np.random.default_rng(n * 100 + m)
    v = rng.standard_normal((n, m)) * np.exp(rng.standard_normal((n, m)))
    r0 = oracle.mx_along(v, 0)
    for c in range(m):
        for b0 in range(0, n, 32):
            blk = np.zeros(32)
            seg = v[b0:b0 + 32, c]
            blk[:len(seg)] = seg
            np.testing.assert_array_equal(r0[b0:b0 + 32, c], oracle.mx_roundtrip(blk[None])[0, :len(seg)])
    if m % 32 == 0 or m < 32:
        r1 = oracle.mx_along(v, 1)
        np.testing.assert_array_equal(r1, oracle.mx_along(v.T, 0).T)
    # values already on the grid of their block stay put
    grid = oracle.mx_roundtrip(np.pad(v[:, :1].T, ((0, 0), (0, (-n) % 32))))[0, :n]
    np.testing.assert_array_equal(oracle.mx_along(grid[:, None], 0)[:, 0], grid)


def test_forward_mx_reduces_to_fp64_without_quantisation():
    x, dy, g, counts, wg, wu, wd = _share(0)
    deq = [oracle.mx_dequantize(*w) for w in (wg, wu, wd)]
    ref = oracle.experts_forward(x, counts, *deq)
    got = oracle.experts_forward_mx(x, counts, *wg, *wu, *wd, quantize=False)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_backward_mx_reduces_to_fp64_without_quantisation():
    x, dy, g, counts, wg, wu, wd = _share(1)
    deq = [oracle.mx_dequantize(*w) for w in (wg, wu, wd)]
    ref = oracle.experts_backward(x, counts, g, dy, *deq)
    got = oracle.experts_backward_mx(x, counts, g, dy, *wg, *wu, *wd, quantize=False)
    for k in ('dx_slot', 'dg', 'dW_gate', 'dW_up', 'dW_down'):
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-11, atol=1e-11, err_msg=k)


def test_backward_mx_close_to_fp64_and_zero_for_empty_expert():
    x, dy, g, counts, wg, wu, wd = _share(2)
    deq = [oracle.mx_dequantize(*w) for w in (wg, wu, wd)]
    ref = oracle.experts_backward(x, counts, g, dy, *deq)
    got = oracle.experts_backward_mx(x, counts, g, dy, *wg, *wu, *wd)
    for k in ('dx_slot', 'dg', 'dW_gate', 'dW_up', 'dW_down'):
        rel = np.linalg.norm(got[k] - ref[k]) / np.linalg.norm(ref[k])
        assert 1e-4 < rel < 0.15, (k, rel)      # quantised, but only by the E4M3 rounding
    for k in ('dW_gate', 'dW_up', 'dW_down'):
        assert np.all(got[k][1] == 0)


def test_backward_mx_unit_restriction():
    """Row i of dW_gate / dW_up and column i of dW_down from the expert restricted to unit i (rows
    i of W_gate, W_up, column i of W_down) equal those of the whole expert: every quantisation on
    their path runs down a single column. The full-size GPU test samples units this way."""
    x, dy, g, counts, wg, wu, wd = _share(3, S=45, counts=(45,))
    Wg, Wu, Wd = (oracle.mx_dequantize(*w) for w in (wg, wu, wd))
    full = oracle.experts_backward_mx_w(x, counts, g, dy, Wg, Wu, Wd)
    for i in (0, 7, 31):
        ru = oracle.experts_backward_mx_w(x, counts, g, dy, Wg[:, i:i + 1], Wu[:, i:i + 1], Wd[:, :, i:i + 1])
        np.testing.assert_allclose(ru['dW_gate'][0, 0], full['dW_gate'][0, i], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(ru['dW_up'][0, 0], full['dW_up'][0, i], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(ru['dW_down'][0, :, 0], full['dW_down'][0, :, i], rtol=1e-12, atol=1e-12)
