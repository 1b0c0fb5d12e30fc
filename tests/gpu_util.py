"""Helpers for the GPU parity tests: run the library on synthetic inputs and compare with the oracle.

Only tests import this module. It calls the library through its C ABI binding.
"""
from __future__ import annotations

import numpy as np
import torch

import synth

TOL = {'f32': 1e-4, 'bf16': 2e-2, 'mxfp8': 3e-2}


def half_ulp_bf16(v):
    """Half a unit in the last place of |v| in BF16 (8 significant bits): the rounding error of
    storing v as BF16."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    _, ex = np.frexp(np.where(a > 0, a, 1.0))        # a = m * 2^ex, m in [0.5, 1)
    return np.where(a > 0, np.ldexp(1.0, (ex - 1 - 8).astype(np.int32)), 0.0)


def mx_choice_allowance(H, eps=2.0 ** -13):
    """Per-element size of the alternative MXFP8 decisions for a gated activation H [rows][I].

    The kernel takes the quantisation decision (block scale and E4M3 code) on its fp32 value of
    h, the oracle on its fp64 value; they agree except where the value sits within rounding
    distance of a decision boundary, where either neighbour is a correct result. Perturbing H by
    a relative eps both ways finds those elements; the returned array holds, per element, the
    largest change of the dequantised value over the alternatives (0 where the decision is
    unambiguous)."""
    import oracle
    H = np.asarray(H, dtype=np.float64)
    base = oracle.mx_roundtrip(H)
    delta = np.zeros_like(H)
    for s in (1.0 + eps, 1.0 - eps):
        delta = np.maximum(delta, np.abs(oracle.mx_roundtrip(H * s) - base))
    # element-wise perturbations with the block scale held: codes that flip on their own
    q, sc = oracle.mx_quantize(H)
    scale = np.repeat(np.ldexp(1.0, sc.astype(np.int32) - 127), 32, axis=-1)
    for s in (1.0 + eps, 1.0 - eps):
        alt = oracle.e4m3_decode(oracle.e4m3_encode(oracle.e4m3_round(H * s / scale))) * scale
        delta = np.maximum(delta, np.abs(alt - base))
    return delta


def assert_close_rms(got, ref, tau, what='', stored_bf16=False, allowance=None):
    """|got - ref| <= tau * RMS(ref) element by element over the whole tensor.

    For a tensor stored as BF16 the bound per element is tau * RMS(ref) + half a BF16 ulp of
    ref[i]: the arithmetic error plus the rounding of the storage format itself, which alone
    exceeds 2e-2 * RMS for elements beyond 8 * RMS. `allowance` (same shape, optional) adds the
    effect of alternative quantisation decisions that are equally correct."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f'{what}: non-finite output'
    if not ref.size:
        return 0.0
    rms = float(np.sqrt(np.mean(ref ** 2)))
    d = np.abs(got - ref)
    bound = tau * rms + (half_ulp_bf16(ref) if stored_bf16 else 0.0) + 1e-30
    if allowance is not None:
        bound = bound + np.asarray(allowance, dtype=np.float64)
    bad = d > bound
    i = int(np.argmax(d - bound))
    assert not bad.any(), (f'{what}: {int(bad.sum())} elements out of bound; worst |d| = {d.flat[i]:.3e} at ref '
                           f'{ref.flat[i]:.3e} (tau*RMS = {tau * rms:.3e})')
    ratio = float(d.max() / rms) if rms else 0.0
    used = float(np.max(d / bound))
    print(f'  {what}: max|d|/RMS = {ratio:.2e} (tau {tau:g}); worst element at {used:.2f} of its bound', flush=True)
    return ratio


def frac_beyond(got, ref, tau, stored_bf16=False):
    """Share of elements with |got - ref| > tau * RMS(ref) (+ half a BF16 ulp of ref for a tensor
    stored as BF16), with no allowance for alternative quantisation decisions. Genuine decision
    flips touch few elements; a wrong axis, a dropped term or a transposed operand moves most."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    bound = tau * rms + (half_ulp_bf16(ref) if stored_bf16 else 0.0)
    return float(np.mean(np.abs(got - ref) > bound)) if ref.size else 0.0


def t2np(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype != torch.int32 else t.cpu().numpy()


def dtype_of(cfg):
    return torch.float32 if cfg.dtype == 'f32' else torch.bfloat16


class ForwardRun:
    """Runs moe_forward once on a DeviceLayer and keeps every output tensor."""

    def __init__(self, m, L: synth.DeviceLayer, flags=0, chunk_rows=0, ring_stages=0, want_parts=True):
        cfg = L.cfg
        dev = L.x.device
        self.p = m.problem(cfg.T, cfg.D, cfg.I, cfg.E, cfg.K, cfg.I_shared, cfg.dtype, chunk_rows, ring_stages, flags)
        T, K, D, E = cfg.T, cfg.K, cfg.D, cfg.E
        dt = L.x.dtype
        self.topk_idx = torch.empty((T, K), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T, K), dtype=torch.float32, device=dev)
        self.counts = torch.empty((E,), dtype=torch.int32, device=dev)
        self.offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
        self.perm = torch.empty((T * K,), dtype=torch.int32, device=dev)
        self.inv_perm = torch.empty((T * K,), dtype=torch.int32, device=dev)
        self.out = torch.empty((T, D), dtype=dt, device=dev)
        self.y_routes = torch.empty((T * K, D), dtype=dt, device=dev) if want_parts else None
        self.shared_out = torch.empty((T, D), dtype=dt, device=dev) if (want_parts and cfg.I_shared) else None
        self.ws = torch.zeros((m.workspace_size(self.p),), dtype=torch.uint8, device=dev)
        self.weights = m.make_weights(L.w_gate, L.w_up, L.w_down, L.ws_gate, L.ws_up, L.ws_down)
        self.routing = m.make_routing(self.topk_idx, self.topk_w, self.counts, self.offsets, self.perm,
                                      self.inv_perm)
        self.m, self.L = m, L

    def __call__(self):
        self.m.forward(self.p, self.L.x, self.L.logits, self.weights, self.out, self.routing, self.ws,
                       self.y_routes, self.shared_out)
        return self

    def lanes(self, streams, events):
        """moe_forward_lanes on the current stream plus `streams`."""
        self.m.forward_lanes(self.p, self.L.x, self.L.logits, self.weights, self.out, self.routing, self.ws,
                             streams, events, self.y_routes, self.shared_out)
        return self


class PinnedWord:
    """A coherent pinned host int32 (hipHostMalloc with hipHostMallocCoherent, through the HIP runtime
    torch has loaded): `value` reads and stores it from the host, `device_address` is what a kernel
    reads. Free with close() once no queued work reads it."""

    def __init__(self):
        import ctypes
        with open('/proc/self/maps') as f:
            paths = sorted({line.split()[-1] for line in f if 'libamdhip64' in line})
        assert paths, 'HIP runtime not loaded'
        self._hip = ctypes.CDLL(paths[0])
        self._ptr, dptr = ctypes.c_void_p(), ctypes.c_void_p()
        assert self._hip.hipHostMalloc(ctypes.byref(self._ptr), ctypes.c_size_t(64), ctypes.c_uint(0x40000000)) == 0
        assert self._hip.hipHostGetDevicePointer(ctypes.byref(dptr), self._ptr, ctypes.c_uint(0)) == 0
        self.device_address = dptr.value
        self._word = ctypes.c_int32.from_address(self._ptr.value)
        self._word.value = 0

    @property
    def value(self):
        return self._word.value

    @value.setter
    def value(self, v):
        self._word.value = v

    def close(self):
        if self._ptr is not None:
            self._hip.hipHostFree(self._ptr)
            self._ptr = None
