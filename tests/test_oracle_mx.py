"""Pins of the oracle's MXFP8 encoder: hand-worked blocks, torch's float8_e4m3fn conversion
(a library routine) for in-range values, and the round-trip error bound. CPU only."""
import os

import numpy as np
import torch

import oracle


def test_mx_golden(golden_dir):
    n = 0
    for line in open(os.path.join(golden_dir, 'mx_cases.txt')):
        line = line.split('#')[0]
        if '|' not in line:
            continue
        a, b, c = [p.strip() for p in line.split('|')]
        v = np.zeros(32)
        for kv in a.split():
            i, x = kv.split('=')
            v[int(i)] = eval(x, {'__builtins__': {}}, {})
        want = np.zeros(32, dtype=np.uint8)
        for kv in c.split():
            i, x = kv.split('=')
            want[int(i)] = int(x, 16)
        q, s = oracle.mx_quantize(v[None])
        assert int(s[0, 0]) == int(b), line
        assert np.array_equal(q[0], want), (line, q[0])
        n += 1
    assert n >= 8


def test_e4m3_against_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.1, 1, 30, 200)])
    v = np.clip(v, -448, 448)
    v = np.concatenate([v, [0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -6]])
    ours = oracle.e4m3_encode(oracle.e4m3_round(v))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.e4m3_decode(codes)
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
    # every finite code re-encodes to itself (except -0 / +0 both valid)
    fin = ~np.isnan(ours)
    assert np.array_equal(oracle.e4m3_encode(ours[fin]), codes[fin])


def test_mx_saturation_and_error_bound():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((64, 256)) * np.exp(rng.standard_normal((64, 1)) * 4)
    q, s = oracle.mx_quantize(v)
    d = oracle.mx_dequantize(q, s)
    blk = v.reshape(64, 8, 32)
    amax = np.abs(blk).max(-1)
    scale = np.ldexp(1.0, s.astype(np.int32) - 127)
    # the scale puts amax in [256, 512) before saturation
    assert np.all((amax / scale >= 256) & (amax / scale < 512))
    # error: half a quantum of the element's binade, or the saturation gap for the top binade
    err = np.abs(d - v).reshape(64, 8, 32)
    y = np.abs(blk) / scale[..., None]
    e = np.maximum(np.floor(np.log2(np.maximum(y, 1e-300))), -6)
    bound = np.where(y > 448, y - 448, 2.0 ** (e - 4)) * scale[..., None]
    assert np.all(err <= bound * (1 + 1e-12))
    assert np.all(np.abs(oracle.e4m3_decode(q)) <= 448)


def test_mx_bf16_inputs_exact_power_of_two_and_clamp():
    v = np.zeros((3, 32))
    v[0, 0] = 4.0                 # amax exact power of two -> 4 / 2^-6 = 256
    v[1, :] = 1.0
    v[1, 7] = 1.96875             # top of the binade -> 504 -> saturates to 448
    q, s = oracle.mx_quantize(v)
    assert list(s[:, 0]) == [127 - 6, 127 - 8, 127]
    assert q[0, 0] == 0x78 and q[1, 7] == 0x7E and q[1, 0] == 0x78
    assert np.all(q[2] == 0)
