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


def assert_close_rms(got, ref, tau, what='', stored_bf16=False):
    """|got - ref| <= tau * RMS(ref) element by element over the whole tensor.

    For a tensor stored as BF16 the bound per element is tau * RMS(ref) + half a BF16 ulp of
    ref[i]: the arithmetic error plus the rounding of the storage format itself, which alone
    exceeds 2e-2 * RMS for elements beyond 8 * RMS."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f'{what}: non-finite output'
    if not ref.size:
        return 0.0
    rms = float(np.sqrt(np.mean(ref ** 2)))
    d = np.abs(got - ref)
    bound = tau * rms + (half_ulp_bf16(ref) if stored_bf16 else 0.0) + 1e-30
    bad = d > bound
    i = int(np.argmax(d - bound))
    assert not bad.any(), (f'{what}: {int(bad.sum())} elements out of bound; worst |d| = {d.flat[i]:.3e} at ref '
                           f'{ref.flat[i]:.3e} (tau*RMS = {tau * rms:.3e})')
    return float(d.max() / rms) if rms else 0.0


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
        self.ws = torch.empty((m.workspace_size(self.p),), dtype=torch.uint8, device=dev)
        self.weights = m.make_weights(L.w_gate, L.w_up, L.w_down, L.ws_gate, L.ws_up, L.ws_down)
        self.routing = m.make_routing(self.topk_idx, self.topk_w, self.counts, self.offsets, self.perm,
                                      self.inv_perm)
        self.m, self.L = m, L

    def __call__(self):
        self.m.forward(self.p, self.L.x, self.L.logits, self.weights, self.out, self.routing, self.ws,
                       self.y_routes, self.shared_out)
        return self
