"""Pins of the quantisation axes in the oracle's MXFP8 experts (forward and backward). CPU only.

The Notes ("The production details") train the routed experts in MXFP8 without saying which
operand is quantised along which axis; the reading taken is that every grouped GEMM quantises both
operands along its own contraction dimension (OCP MX v1.0 blocks of 32). These cases fix that
reading with values worked out by hand, independently of the oracle's code:

* Every case has one expert, 32 slots, D = I = 32, so each quantisation axis holds exactly one
  block of 32. The pre-activations are at least 40, where sigmoid(a) rounds to 1.0 in fp64, so
  SiLU(a) = a and the SwiGLU backward reduces to da = dh u, du = dh a: every intermediate value
  is a small integer or a power of two, and the expected outputs are exact.
* In each case one operand carries a spike: along one axis a block holds 2^20 next to values
  2^-20 of it, which the E4M3 grid flushes to zero (their quotient by the block scale is at
  most 2^-12, below half the smallest subnormal 2^-9); along the other axis every block is
  uniform and quantises exactly. Quantising along the wrong axis, or not at all, therefore
  changes the result by a known amount that the expected value excludes.

Block scale arithmetic (OCP MX v1.0, the oracle's encoder pinned by tests/golden/mx_cases.txt):
scale = 2^(floor(log2 amax) - 8); a value v is stored as RNE_E4M3(v / scale) * scale.
"""
import numpy as np
import pytest

import oracle

S = D = I = 32
COUNTS = np.array([S])


def ones(*shape):
    return np.ones(shape)


# ----------------------------------------------------------------------------------------------
# forward: y = Q_I(h) W_down^T with h = SiLU(Q_D(x) W_gate^T) * (Q_D(x) W_up^T)
# ----------------------------------------------------------------------------------------------
def case_h_along_I():
    """x = 1 and W_gate = 2 give a = 32 * 2 = 64 everywhere (SiLU(64) = 64). W_up row 0 = 2^15,
    other rows 2^-5, so u[:, 0] = 32 * 2^15 = 2^20 and u[:, i>0] = 1; h[:, 0] = 2^26, h[:, i>0] = 64.
    Along I each row of h is (2^26, 64, ..., 64): scale 2^18, 64 / 2^18 = 2^-12 flushes, so
    Q_I(h) row = (2^26, 0, ..., 0). Along the slots every column is uniform (exact).
    W_down[:, 0] = 2^-20, W_down[:, i>0] = 1: y = 2^26 * 2^-20 = 64 with h along I;
    64 + 31 * 64 = 2048 with h along the slots or unquantised."""
    wg = 2 * ones(1, I, D)
    wu = np.full((1, I, D), 2.0 ** -5)
    wu[0, 0, :] = 2.0 ** 15
    wd = ones(1, D, I)
    wd[0, :, 0] = 2.0 ** -20
    return ones(S, D), wg, wu, wd


def case_x_along_D():
    """x[:, 0] = 2^20, x[:, d>0] = 1. Along D each row is (2^20, 1, ..., 1): scale 2^12, the ones
    flush (2^-12), Q_D(x) row = (2^20, 0, ..., 0); along the slots the columns are uniform (exact).
    W_gate[:, 0] = 2^-14, else 2: a = 2^20 * 2^-14 = 64 (126 if the ones survived).
    W_up[:, 0] = 2^-20, else 1: u = 1 (32 if the ones survived). h = 64 exactly (uniform rows);
    W_down = 1: y = 32 * 64 = 2048. Unquantised: h = 126 * 32 = 4032, y = 32 * 4032 = 129024."""
    x = ones(S, D)
    x[:, 0] = 2.0 ** 20
    wg = 2 * ones(1, I, D)
    wg[0, :, 0] = 2.0 ** -14
    wu = ones(1, I, D)
    wu[0, :, 0] = 2.0 ** -20
    return x, wg, wu, ones(1, D, I)


def test_forward_h_quantised_along_I():
    x, wg, wu, wd = case_h_along_I()
    y = oracle.experts_forward_mx_w(x, COUNTS, wg, wu, wd)
    np.testing.assert_array_equal(y, np.full((S, D), 64.0))
    np.testing.assert_array_equal(oracle.experts_forward_mx_w(x, COUNTS, wg, wu, wd, quantize=False),
                                  np.full((S, D), 2048.0))


def test_forward_x_quantised_along_D():
    x, wg, wu, wd = case_x_along_D()
    np.testing.assert_array_equal(oracle.experts_forward_mx_w(x, COUNTS, wg, wu, wd), np.full((S, D), 2048.0))
    np.testing.assert_array_equal(oracle.experts_forward_mx_w(x, COUNTS, wg, wu, wd, quantize=False),
                                  np.full((S, D), 129024.0))


# ----------------------------------------------------------------------------------------------
# backward. With g = 1 unless stated and a >= 40:  dh' = Q_D(dy) Q_D(W_down);  dg = <h, dh'>;
# da = g dh' u;  du = g dh' a;  dx = Q_I(da) Q_I(W_gate) + Q_I(du) Q_I(W_up);
# dW_down = Q_n(g dy)^T Q_n(h);  dW_gate = Q_n(da)^T Q_n(x);  dW_up = Q_n(du)^T Q_n(x)
# (Q_n along the slots; the weights as given, re-quantised along the backward contraction axis).
# ----------------------------------------------------------------------------------------------
def backward(x, g, dy, wg, wu, wd, quantize=True):
    return oracle.experts_backward_mx_w(x, COUNTS, g, dy, wg, wu, wd, quantize=quantize)


def test_backward_da_along_I_for_dgrad_and_along_slots_for_wgrad():
    """x = 1, W_gate = 2: a = 64. W_up row 0 = 2^10, other rows 1: u[:, 0] = 2^15, u[:, i>0] = 32.
    dy = 1, W_down[:, 0] = 2^10, other columns 1: dh'[:, 0] = 2^15, dh'[:, i>0] = 32.
    da = dh' u: column 0 = 2^30, others 1024 -- each row a spike along I, each column uniform.
    du = dh' a: 2^21 and 2048 (powers of two: exact on either axis).
    dx = Q_I(da) W_gate + du W_up (W_gate = 2 and W_up columns (2^10, 1, ..) exact along I):
      Q_I(da) row = (2^30, 0, ..): dx = 2^30 * 2 + 2^21 * 2^10 + 31 * 2048 = 2^32 + 63488;
      with da along the slots (exact) or unquantised, 31 * 1024 * 2 = 63488 more.
    dW_gate = Q_n(da)^T x: columns of da uniform, so exact: 32 * 2^30 = 2^35 (row 0), 32 * 1024
      = 32768 (others); da along I in the weight gradient would zero rows i > 0.
    dg = <h, dh'> with h = 64 u: 2^21 * 2^15 + 31 * 2^11 * 32 = 2^36 + 2031616."""
    wg = 2 * ones(1, I, D)
    wu = ones(1, I, D)
    wu[0, 0, :] = 2.0 ** 10
    wd = ones(1, D, I)
    wd[0, :, 0] = 2.0 ** 10
    r = backward(ones(S, D), ones(S), ones(S, D), wg, wu, wd)
    np.testing.assert_array_equal(r['dx_slot'], np.full((S, D), 2.0 ** 32 + 63488))
    np.testing.assert_array_equal(r['dg'], np.full(S, 2.0 ** 36 + 2031616))
    want_dwg = np.full((1, I, D), 32768.0)
    want_dwg[0, 0] = 2.0 ** 35
    np.testing.assert_array_equal(r['dW_gate'], want_dwg)
    r0 = backward(ones(S, D), ones(S), ones(S, D), wg, wu, wd, quantize=False)
    np.testing.assert_array_equal(r0['dx_slot'], np.full((S, D), 2.0 ** 32 + 2 * 63488))


def test_backward_w_gate_quantised_along_I_for_dgrad():
    """x = 1 on columns 1..16 and 0 elsewhere; W_gate = 4 except column 0 = (2^20, 1, .., 1) (rows
    i = 0, 1, ..); W_up = 2^-4 on columns 1..16, else 0. Then a = 16 * 4 = 64, u = 16 * 2^-4 = 1,
    independent of column 0 (x is 0 there). dy = 1, W_down = 1: dh' = 32; da = 32, du = 2048.
    Q_I(W_gate) (down each column): column 0 = (2^20, 1, ..) -> (2^20, 0, ..); other columns exact.
    dx[:, 0] = 32 * 2^20 = 2^25 (W_up column 0 is 0); dx[:, 1..16] = 32*32*4 + 2048*32*2^-4 = 8192;
    dx[:, 17..31] = 4096. Quantised along D instead, row 0 = (2^20, 4, ..) flushes its fours
    (4 / 2^12 = 2^-10, a tie that rounds to even zero) and keeps column 0's ones:
    dx[:, 0] = 32 (2^20 + 31) = 2^25 + 992, dx[:, 1..16] = 8064, dx[:, 17..31] = 3968."""
    x = np.zeros((S, D))
    x[:, 1:17] = 1
    wg = 4 * ones(1, I, D)
    wg[0, :, 0] = 1
    wg[0, 0, 0] = 2.0 ** 20
    wu = np.zeros((1, I, D))
    wu[0, :, 1:17] = 2.0 ** -4
    r = backward(x, ones(S), ones(S, D), wg, wu, ones(1, D, I))
    want = np.full(D, 4096.0)
    want[0] = 2.0 ** 25
    want[1:17] = 8192
    np.testing.assert_array_equal(r['dx_slot'], np.broadcast_to(want, (S, D)))
    np.testing.assert_array_equal(r['dg'], np.full(S, 65536.0))       # <h, dh'> = 32 * 64 * 32
    r0 = backward(x, ones(S), ones(S, D), wg, wu, ones(1, D, I), quantize=False)
    np.testing.assert_array_equal(r0['dx_slot'][:, 0], np.full(S, 2.0 ** 25 + 992))


def test_backward_w_up_quantised_along_I_for_dgrad():
    """The W_gate case with the roles of the two projections swapped: x = 1 on columns 1..16;
    W_up = 2^-4 there, column 0 = (2^20, 1, .., 1), 0 elsewhere; W_gate = 4 on columns 1..16, 0
    elsewhere. a = 64, u = 1, dh' = 32, da = 32, du = 2048. Q_I(W_up) column 0 -> (2^20, 0, ..):
    dx[:, 0] = 2048 * 2^20 = 2^31; dx[:, 1..16] = 32*32*4 + 2048*32*2^-4 = 8192; dx[:, 17..31] = 0.
    Along D, row 0 of W_up flushes its 2^-4 entries and column 0 keeps its ones:
    dx[:, 0] = 2048 (2^20 + 31) = 2^31 + 63488 (as unquantised), dx[:, 1..16] = 8064."""
    x = np.zeros((S, D))
    x[:, 1:17] = 1
    wu = np.zeros((1, I, D))
    wu[0, :, 1:17] = 2.0 ** -4
    wu[0, :, 0] = 1
    wu[0, 0, 0] = 2.0 ** 20
    wg = np.zeros((1, I, D))
    wg[0, :, 1:17] = 4
    r = backward(x, ones(S), ones(S, D), wg, wu, ones(1, D, I))
    want = np.zeros(D)
    want[0] = 2.0 ** 31
    want[1:17] = 8192
    np.testing.assert_array_equal(r['dx_slot'], np.broadcast_to(want, (S, D)))
    r0 = backward(x, ones(S), ones(S, D), wg, wu, ones(1, D, I), quantize=False)
    np.testing.assert_array_equal(r0['dx_slot'][:, 0], np.full(S, 2.0 ** 31 + 63488))


def test_backward_du_along_I_for_dgrad_and_along_slots_for_wgrad():
    """The da case with the roles swapped: x = 1; W_gate row 0 = 2^11, other rows 2: a[:, 0] = 2^16,
    a[:, i>0] = 64; W_up = 2^-5: u = 1, h = a. dy = 1, W_down[:, 0] = 2^10, other columns 1:
    dh'[:, 0] = 2^15, dh'[:, i>0] = 32. du = dh' a: 2^31 and 2048 (a spike along I, uniform
    columns); da = dh' u: 2^15 and 32 (powers of two, exact either way).
    dx = Q_I(da) W_gate + Q_I(du) W_up (both weights exact along I): Q_I(du) row = (2^31, 0, ..),
      dx = 2^15 2^11 + 31*32*2 + 2^31 2^-5 = 2^27 + 1984 (unquantised: 31*2048*2^-5 = 1984 more).
    dW_up = Q_n(du)^T x: exact along the slots: 32 * 2^31 = 2^36 (row 0), 32 * 2048 = 65536.
    dg = <h, dh'> = 2^16 2^15 + 31 * 64 * 32 = 2^31 + 63488."""
    wg = 2 * ones(1, I, D)
    wg[0, 0, :] = 2.0 ** 11
    wu = np.full((1, I, D), 2.0 ** -5)
    wd = ones(1, D, I)
    wd[0, :, 0] = 2.0 ** 10
    r = backward(ones(S, D), ones(S), ones(S, D), wg, wu, wd)
    np.testing.assert_array_equal(r['dx_slot'], np.full((S, D), 2.0 ** 27 + 1984))
    want = np.full((1, I, D), 65536.0)
    want[0, 0] = 2.0 ** 36
    np.testing.assert_array_equal(r['dW_up'], want)
    np.testing.assert_array_equal(r['dg'], np.full(S, 2.0 ** 31 + 63488))
    r0 = backward(ones(S, D), ones(S), ones(S, D), wg, wu, wd, quantize=False)
    np.testing.assert_array_equal(r0['dx_slot'], np.full((S, D), 2.0 ** 27 + 3968))


def _b3_weights():
    wg = 2 * ones(1, I, D)                   # a = 64
    wu = np.full((1, I, D), 2.0 ** -5)       # u = 1, h = 64
    return wg, wu


def test_backward_dy_along_D_for_dgrad_and_along_slots_for_wgrad():
    """x = 1, a = 64, u = 1, h = 64; W_down = 1; dy[:, 0] = 2^20, dy[:, d>0] = 1.
    Q_D(dy) row = (2^20, 0, ..) so dh' = 2^20 and dg = 32 * 64 * 2^20 = 2^31 (with the ones kept,
    2^31 + 63488). dW_down = Q_n(dy)^T h: the columns of dy are uniform (exact along the slots):
    dW_down[0, :] = 32 * 2^20 * 64 = 2^31, dW_down[d>0, :] = 32 * 64 = 2048; dy along D there
    would zero rows d > 0. da = 2^20, du = 2^26: dx = 32 * 2^20 * 2 + 32 * 2^26 * 2^-5 = 2^27."""
    wg, wu = _b3_weights()
    dy = ones(S, D)
    dy[:, 0] = 2.0 ** 20
    r = backward(ones(S, D), ones(S), dy, wg, wu, ones(1, D, I))
    np.testing.assert_array_equal(r['dg'], np.full(S, 2.0 ** 31))
    want = np.full((1, D, I), 2048.0)
    want[0, 0] = 2.0 ** 31
    np.testing.assert_array_equal(r['dW_down'], want)
    np.testing.assert_array_equal(r['dx_slot'], np.full((S, D), 2.0 ** 27))
    r0 = backward(ones(S, D), ones(S), dy, wg, wu, ones(1, D, I), quantize=False)
    np.testing.assert_array_equal(r0['dg'], np.full(S, 2.0 ** 31 + 63488))


def test_backward_w_down_quantised_along_D_for_dgrad():
    """As above with dy = 1 and W_down row 0 = 2^20 (W_down is [D, I]): down each column the
    block is (2^20, 1, .., 1) -> (2^20, 0, ..), so dh' = 2^20 and dg = 2^31; along I the rows are
    uniform (exact) and dh' = 2^20 + 31, dg = 2^31 + 63488."""
    wg, wu = _b3_weights()
    wd = ones(1, D, I)
    wd[0, 0, :] = 2.0 ** 20
    r = backward(ones(S, D), ones(S), ones(S, D), wg, wu, wd)
    np.testing.assert_array_equal(r['dg'], np.full(S, 2.0 ** 31))
    np.testing.assert_array_equal(r['dx_slot'], np.full((S, D), 2.0 ** 27))
    np.testing.assert_array_equal(r['dW_down'], np.full((1, D, I), 2048.0))


def test_backward_x_h_and_gdy_along_slots_for_wgrad():
    """Slot 0 is scaled: x[0] = 2^20 (x[j>0] = 1), g[0] = 2^-20 (g[j>0] = 1), dy = 1, W_down = 1,
    W_gate = 2, W_up = 2^-5. a[0] = 2^26, a[j] = 64; u[0] = 2^20, u[j] = 1; h[0] = 2^46, h[j] = 64;
    dh' = 32; dh = g dh': 2^-15 and 32, so da = dh u = 32 and du = dh a = 2048 in every slot.
    Along the slots x's columns are (2^20, 1, ..) -> (2^20, 0, ..): dW_gate = 32 * 2^20 = 2^25,
    dW_up = 2048 * 2^20 = 2^31 (x along D is exact and adds 31 * 32 = 992, resp. 63488).
    h's columns (2^46, 64, ..) -> (2^46, 0, ..) and g dy's columns (2^-20, 1, ..) -> (0, 1, ..):
    dW_down = 0 (h along I would give 31 * 64 = 1984, g dy along D 2^-20 * 2^46 = 2^26).
    dx = 32 * 32 * 2 + 2048 * 32 * 2^-5 = 4096; dg = <h, dh'> = 2^56 (slot 0), 65536 (others)."""
    x = ones(S, D)
    x[0] = 2.0 ** 20
    g = ones(S)
    g[0] = 2.0 ** -20
    wg, wu = _b3_weights()
    r = backward(x, g, ones(S, D), wg, wu, ones(1, D, I))
    np.testing.assert_array_equal(r['dW_gate'], np.full((1, I, D), 2.0 ** 25))
    np.testing.assert_array_equal(r['dW_up'], np.full((1, I, D), 2.0 ** 31))
    np.testing.assert_array_equal(r['dW_down'], np.zeros((1, D, I)))
    np.testing.assert_array_equal(r['dx_slot'], np.full((S, D), 4096.0))
    want_dg = np.full(S, 65536.0)
    want_dg[0] = 2.0 ** 56
    np.testing.assert_array_equal(r['dg'], want_dg)
    r0 = backward(x, g, ones(S, D), wg, wu, ones(1, D, I), quantize=False)
    np.testing.assert_array_equal(r0['dW_down'], np.full((1, D, I), 2.0 ** 26 + 1984))


# ----------------------------------------------------------------------------------------------
# invariants: the forward output and the slot gradients of slot j depend on slot j alone (every
# activation block in those paths lies inside one slot's row); the weight gradients do not
# ----------------------------------------------------------------------------------------------
def _random_share(seed, S=70, Dd=64, Ii=64, counts=(40, 30)):
    rng = np.random.default_rng(seed)
    E = len(counts)
    x = rng.standard_normal((S, Dd))
    dy = rng.standard_normal((S, Dd))
    g = rng.random(S)
    w = [oracle.mx_roundtrip(rng.standard_normal(s) / np.sqrt(s[-1])) for s in ((E, Ii, Dd), (E, Ii, Dd), (E, Dd, Ii))]
    return x, dy, g, np.array(counts), w


@pytest.mark.parametrize('j', [0, 33, 69])
def test_slot_outputs_depend_on_their_own_slot_only(j):
    x, dy, g, counts, (wg, wu, wd) = _random_share(5)
    base_y = oracle.experts_forward_mx_w(x, counts, wg, wu, wd)
    base = oracle.experts_backward_mx_w(x, counts, g, dy, wg, wu, wd)
    x2, dy2, g2 = x.copy(), dy.copy(), g.copy()
    x2[j] *= 2.0 ** 12        # large enough to own every block it would share with another slot
    dy2[j] *= 2.0 ** 12
    g2[j] = 0.5
    y = oracle.experts_forward_mx_w(x2, counts, wg, wu, wd)
    r = oracle.experts_backward_mx_w(x2, counts, g2, dy2, wg, wu, wd)
    keep = np.arange(len(x)) != j
    np.testing.assert_array_equal(y[keep], base_y[keep])
    np.testing.assert_array_equal(r['dx_slot'][keep], base['dx_slot'][keep])
    np.testing.assert_array_equal(r['dg'][keep], base['dg'][keep])
    e = int(np.searchsorted(np.cumsum(counts), j, side='right'))
    assert not np.array_equal(r['dW_gate'][e], base['dW_gate'][e])   # the weight gradients do see it
