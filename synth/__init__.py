"""Seeded synthetic inputs for the MoE layer, shared by the oracle tests and the GPU path.

This module only draws random numbers, rounds them to the storage format, and lays them out.
It holds none of the layer's arithmetic (no routing, no expert FFN, no combine): both sides
receive the same bytes from here and compute everything else on their own.

Two generators:

* ``host``: numpy ``PCG64(SeedSequence([cfg_seed, tensor_id, expert_id]))``, fp32 draws.
  Used for every size the CPU oracle handles whole.
* ``device``: torch's Philox generator on ``cuda:0``, seeded with
  ``cfg_seed * 1_000_003 + tensor_id * 4099 + expert_id``. Used for the full-size layers
  (22.5 GB of BF16 weights at the DeepSeek-V3 shape), which a host generator fills too
  slowly. The oracle reads back exactly the slices it needs.

Storage rounding: fp32 draws are rounded to BF16 with round-to-nearest-even. On the host this
is the usual bit trick; on the device it is torch's own ``.to(torch.bfloat16)`` (also RNE).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# tensor ids (part of the seed)
TID_X, TID_WR, TID_BIAS, TID_WGATE, TID_WUP, TID_WDOWN = 0, 1, 2, 3, 4, 5
TID_SGATE, TID_SUP, TID_SDOWN, TID_DOUT, TID_G, TID_GUMBEL = 6, 7, 8, 9, 10, 11
TID_XSLOT, TID_XLOCAL, TID_DYLOCAL = 12, 13, 14


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """Shape of one MoE layer workload. ``dtype`` is the storage/compute format of the path."""
    name: str
    T: int          # tokens
    D: int          # model dimension
    I: int          # routed expert intermediate dimension
    E: int          # routed experts
    K: int          # experts per token
    I_shared: int   # shared expert intermediate dimension (0: no shared expert)
    dtype: str      # 'f32' | 'bf16' | 'mxfp8'
    seed: int
    router: str = 'gaussian'     # 'gaussian' | 'gaussian_bias' | 'zipf_gumbel'
    bias_var: float = 0.0        # variance of the per-expert router bias ('gaussian_bias')
    zipf_s: float = 1.0          # Zipf exponent ('zipf_gumbel')

    @property
    def slots(self) -> int:
        return self.T * self.K


# The five workloads. Names describe the shapes.
TINY = LayerConfig('tiny_f32_T256_D128_I64_E8_K2', 256, 128, 64, 8, 2, 64, 'f32', 1)
MID = LayerConfig('mid_bf16_T4096_D2048_I768_E128_K8', 4096, 2048, 768, 128, 8, 768, 'bf16', 2)
DSV3 = LayerConfig('dsv3_bf16_T8192_D7168_I2048_E256_K8', 8192, 7168, 2048, 256, 8, 2048, 'bf16', 3,
                   router='gaussian_bias', bias_var=0.5)
MXFP8 = LayerConfig('dsv3_mxfp8_T32768_D7168_I2048_E256_K8', 32768, 7168, 2048, 256, 8, 2048,
                    'mxfp8', 5, router='zipf_gumbel', zipf_s=1.0)


@dataclasses.dataclass(frozen=True)
class EPShareConfig:
    """One expert-parallel rank's share: slots already grouped by local expert."""
    name: str
    tokens: int       # local tokens (shared expert rows)
    D: int
    I: int
    E_local: int
    K: int
    I_shared: int
    zipf_s: float
    seed: int

    @property
    def slots(self) -> int:
        return self.tokens * self.K


EP_SHARE = EPShareConfig('ep64_share_bf16_S57344_D7168_I2048_E4', 7168, 7168, 2048, 4, 8, 2048, 1.2, 4)

CONFIGS = {c.name: c for c in (TINY, MID, DSV3, MXFP8)}


# ----------------------------------------------------------------------------------------------
# host generator
# ----------------------------------------------------------------------------------------------
def host_rng(cfg_seed: int, tensor_id: int, expert_id: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_seed, tensor_id, expert_id])))


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 -> nearest BF16 value (ties to even), returned as fp32. Finite inputs only."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """BF16-valued fp32 array -> its uint16 bit pattern (exact)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def host_normal(cfg_seed, tensor_id, shape, std, expert_id=0, bf16=False) -> np.ndarray:
    v = host_rng(cfg_seed, tensor_id, expert_id).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        v = (v * np.float32(std)).astype(np.float32)
    return round_bf16(v) if bf16 else v


def zipf_counts(total: int, n: int, s: float) -> np.ndarray:
    """Split ``total`` items over ``n`` bins with Zipf(s) shares p_e ~ 1/(e+1)^s, by largest remainder.

    Bin 0 is the most popular. Remainder ties go to the lower bin index.
    """
    p = 1.0 / np.arange(1, n + 1, dtype=np.float64) ** s
    p /= p.sum()
    raw = p * total
    base = np.floor(raw).astype(np.int64)
    rem = total - int(base.sum())
    order = np.lexsort((np.arange(n), -(raw - base)))
    base[order[:rem]] += 1
    return base


def router_logits_host(cfg: LayerConfig, x: np.ndarray) -> np.ndarray:
    """Synthetic router logits [T, E] in fp32, computed in fp64 from the seeded draws.

    'gaussian':      x . W_r^T with W_r ~ N(0, 1/D)           (near-uniform expert load)
    'gaussian_bias': the same plus a per-expert bias ~ N(0, bias_var)   (mild skew)
    'zipf_gumbel':   ln p_e + G with p_e ~ 1/(e+1)^s and G ~ Gumbel(0, 1) i.i.d.; the top-k of
                     these is a draw without replacement from the Zipf popularity
    """
    T, E, D = cfg.T, cfg.E, cfg.D
    if cfg.router == 'zipf_gumbel':
        u = host_rng(cfg.seed, TID_GUMBEL).random((T, E))
        gum = -np.log(-np.log(np.clip(u, 1e-300, 1.0)))
        lp = -cfg.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
        return (lp[None, :] + gum).astype(np.float32)
    wr = host_normal(cfg.seed, TID_WR, (E, D), 1.0 / math.sqrt(D))
    lg = x.astype(np.float64) @ wr.astype(np.float64).T
    if cfg.router == 'gaussian_bias':
        lg = lg + host_normal(cfg.seed, TID_BIAS, (E,), math.sqrt(cfg.bias_var)).astype(np.float64)[None, :]
    return lg.astype(np.float32)


@dataclasses.dataclass
class HostLayer:
    """All inputs of one layer as host arrays (fp32 arrays holding BF16 values for BF16 configs)."""
    cfg: LayerConfig
    x: np.ndarray          # [T, D]
    logits: np.ndarray     # [T, E] fp32
    w_gate: np.ndarray     # [E, I, D]
    w_up: np.ndarray       # [E, I, D]
    w_down: np.ndarray     # [E, D, I]
    ws_gate: np.ndarray | None   # [I_s, D]
    ws_up: np.ndarray | None     # [I_s, D]
    ws_down: np.ndarray | None   # [D, I_s]


def host_layer(cfg: LayerConfig) -> HostLayer:
    """Whole-layer inputs on the host. Weights ~ N(0, 1/fan_in), x ~ N(0, 1)."""
    bf = cfg.dtype != 'f32'
    T, D, I, E, Is = cfg.T, cfg.D, cfg.I, cfg.E, cfg.I_shared
    x = host_normal(cfg.seed, TID_X, (T, D), 1.0, bf16=bf)
    logits = router_logits_host(cfg, x)
    wg = np.stack([host_normal(cfg.seed, TID_WGATE, (I, D), 1 / math.sqrt(D), e, bf) for e in range(E)])
    wu = np.stack([host_normal(cfg.seed, TID_WUP, (I, D), 1 / math.sqrt(D), e, bf) for e in range(E)])
    wd = np.stack([host_normal(cfg.seed, TID_WDOWN, (D, I), 1 / math.sqrt(I), e, bf) for e in range(E)])
    if Is > 0:
        sg = host_normal(cfg.seed, TID_SGATE, (Is, D), 1 / math.sqrt(D), 0, bf)
        su = host_normal(cfg.seed, TID_SUP, (Is, D), 1 / math.sqrt(D), 0, bf)
        sd = host_normal(cfg.seed, TID_SDOWN, (D, Is), 1 / math.sqrt(Is), 0, bf)
    else:
        sg = su = sd = None
    return HostLayer(cfg, x, logits, wg, wu, wd, sg, su, sd)


def host_dout(cfg: LayerConfig, rows: int) -> np.ndarray:
    """Upstream gradient dOut ~ N(0, 1), [rows, D], rounded like the activations."""
    return host_normal(cfg.seed, TID_DOUT, (rows, cfg.D), 1.0, bf16=cfg.dtype != 'f32')


def tie_logits(logits: np.ndarray, step: float = 0.25) -> np.ndarray:
    """Round logits to multiples of ``step`` so that many exact ties appear."""
    return (np.round(logits.astype(np.float64) / step) * step).astype(np.float32)


def scaled(cfg: LayerConfig, name: str, **kw) -> LayerConfig:
    """A smaller layer with the same recipe (for parity tests the oracle finishes in seconds)."""
    return dataclasses.replace(cfg, name=name, **kw)


# ----------------------------------------------------------------------------------------------
# EP-share inputs (slots already expert-contiguous)
# ----------------------------------------------------------------------------------------------
@dataclasses.dataclass
class HostShare:
    cfg: EPShareConfig
    counts: np.ndarray     # [E_local] int64
    x_slot: np.ndarray     # [S, D]
    g: np.ndarray          # [S] fp32 ~ U(0, 1)
    dy_slot: np.ndarray    # [S, D]
    x_local: np.ndarray    # [tokens, D]
    dy_local: np.ndarray   # [tokens, D]
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray
    ws_gate: np.ndarray
    ws_up: np.ndarray
    ws_down: np.ndarray


def host_share(cfg: EPShareConfig) -> HostShare:
    S, D, I, E, Is = cfg.slots, cfg.D, cfg.I, cfg.E_local, cfg.I_shared
    counts = zipf_counts(S, E, cfg.zipf_s)
    x_slot = host_normal(cfg.seed, TID_XSLOT, (S, D), 1.0, bf16=True)
    g = host_rng(cfg.seed, TID_G).random(S, dtype=np.float32)
    dy = host_normal(cfg.seed, TID_DOUT, (S, D), 1.0, bf16=True)
    xl = host_normal(cfg.seed, TID_XLOCAL, (cfg.tokens, D), 1.0, bf16=True)
    dyl = host_normal(cfg.seed, TID_DYLOCAL, (cfg.tokens, D), 1.0, bf16=True)
    wg = np.stack([host_normal(cfg.seed, TID_WGATE, (I, D), 1 / math.sqrt(D), e, True) for e in range(E)])
    wu = np.stack([host_normal(cfg.seed, TID_WUP, (I, D), 1 / math.sqrt(D), e, True) for e in range(E)])
    wd = np.stack([host_normal(cfg.seed, TID_WDOWN, (D, I), 1 / math.sqrt(I), e, True) for e in range(E)])
    sg = host_normal(cfg.seed, TID_SGATE, (Is, D), 1 / math.sqrt(D), 0, True)
    su = host_normal(cfg.seed, TID_SUP, (Is, D), 1 / math.sqrt(D), 0, True)
    sd = host_normal(cfg.seed, TID_SDOWN, (D, Is), 1 / math.sqrt(Is), 0, True)
    return HostShare(cfg, counts, x_slot, g, dy, xl, dyl, wg, wu, wd, sg, su, sd)


# ----------------------------------------------------------------------------------------------
# device generator (full-size layers)
# ----------------------------------------------------------------------------------------------
def device_seed(cfg_seed: int, tensor_id: int, expert_id: int = 0) -> int:
    return cfg_seed * 1_000_003 + tensor_id * 4099 + expert_id


def device_normal(cfg_seed, tensor_id, shape, std, expert_id=0, dtype=None, device='cuda'):
    """N(0, std^2) draws from torch's Philox generator on `device`, rounded to `dtype` (RNE)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(device_seed(cfg_seed, tensor_id, expert_id))
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        v.mul_(std)
    return v.to(dtype) if dtype is not None else v


@dataclasses.dataclass
class DeviceLayer:
    """All inputs of one layer as device tensors (bf16 for BF16/MXFP8 configs, fp32 for f32)."""
    cfg: LayerConfig
    x: object
    logits: object        # fp32 [T, E]
    w_gate: object        # [E, I, D]
    w_up: object
    w_down: object        # [E, D, I]
    ws_gate: object
    ws_up: object
    ws_down: object


def device_layer(cfg: LayerConfig, device='cuda') -> DeviceLayer:
    """Full-size inputs generated on the device, expert by expert. Same recipe as host_layer
    (distributions and router construction), different generator (Philox)."""
    import torch
    dt = torch.float32 if cfg.dtype == 'f32' else torch.bfloat16
    T, D, I, E, Is = cfg.T, cfg.D, cfg.I, cfg.E, cfg.I_shared
    x = device_normal(cfg.seed, TID_X, (T, D), 1.0, dtype=dt, device=device)
    if cfg.router == 'zipf_gumbel':
        g = torch.Generator(device=device)
        g.manual_seed(device_seed(cfg.seed, TID_GUMBEL))
        u = torch.rand((T, E), generator=g, device=device, dtype=torch.float64).clamp_(min=1e-300)
        lp = -cfg.zipf_s * torch.log(torch.arange(1, E + 1, device=device, dtype=torch.float64))
        logits = (lp[None, :] - torch.log(-torch.log(u))).to(torch.float32)
    else:
        wr = device_normal(cfg.seed, TID_WR, (E, D), 1.0 / math.sqrt(D), device=device).double()
        lg = x.double() @ wr.T
        if cfg.router == 'gaussian_bias':
            lg += device_normal(cfg.seed, TID_BIAS, (E,), math.sqrt(cfg.bias_var), device=device).double()[None, :]
        logits = lg.to(torch.float32)
        del wr, lg
    wg = torch.empty((E, I, D), dtype=dt, device=device)
    wu = torch.empty((E, I, D), dtype=dt, device=device)
    wd = torch.empty((E, D, I), dtype=dt, device=device)
    for e in range(E):
        wg[e] = device_normal(cfg.seed, TID_WGATE, (I, D), 1 / math.sqrt(D), e, dt, device)
        wu[e] = device_normal(cfg.seed, TID_WUP, (I, D), 1 / math.sqrt(D), e, dt, device)
        wd[e] = device_normal(cfg.seed, TID_WDOWN, (D, I), 1 / math.sqrt(I), e, dt, device)
    if Is > 0:
        sg = device_normal(cfg.seed, TID_SGATE, (Is, D), 1 / math.sqrt(D), 0, dt, device)
        su = device_normal(cfg.seed, TID_SUP, (Is, D), 1 / math.sqrt(D), 0, dt, device)
        sd = device_normal(cfg.seed, TID_SDOWN, (D, Is), 1 / math.sqrt(Is), 0, dt, device)
    else:
        sg = su = sd = None
    return DeviceLayer(cfg, x, logits, wg, wu, wd, sg, su, sd)


def to_device(L: HostLayer, device='cuda') -> DeviceLayer:
    """Upload a host layer (exact: host BF16-valued fp32 arrays convert to bf16 without rounding)."""
    import torch
    dt = torch.float32 if L.cfg.dtype == 'f32' else torch.bfloat16

    def up(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device=device).to(dt)

    return DeviceLayer(L.cfg, up(L.x), torch.from_numpy(L.logits).to(device), up(L.w_gate), up(L.w_up),
                       up(L.w_down), up(L.ws_gate), up(L.ws_up), up(L.ws_down))


def device_share(cfg: EPShareConfig, device='cuda') -> HostShare:
    """Full-size share inputs generated on the device (same recipe as host_share, Philox draws);
    the fields hold device tensors (bf16, g fp32) and `counts` the host array."""
    import torch
    S, D, I, E, Is = cfg.slots, cfg.D, cfg.I, cfg.E_local, cfg.I_shared
    bf = torch.bfloat16
    counts = zipf_counts(S, E, cfg.zipf_s)
    x_slot = device_normal(cfg.seed, TID_XSLOT, (S, D), 1.0, dtype=bf, device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(device_seed(cfg.seed, TID_G))
    g = torch.rand((S,), generator=gen, device=device, dtype=torch.float32)
    dy = device_normal(cfg.seed, TID_DOUT, (S, D), 1.0, dtype=bf, device=device)
    xl = device_normal(cfg.seed, TID_XLOCAL, (cfg.tokens, D), 1.0, dtype=bf, device=device)
    dyl = device_normal(cfg.seed, TID_DYLOCAL, (cfg.tokens, D), 1.0, dtype=bf, device=device)
    wg = torch.stack([device_normal(cfg.seed, TID_WGATE, (I, D), 1 / math.sqrt(D), e, bf, device) for e in range(E)])
    wu = torch.stack([device_normal(cfg.seed, TID_WUP, (I, D), 1 / math.sqrt(D), e, bf, device) for e in range(E)])
    wd = torch.stack([device_normal(cfg.seed, TID_WDOWN, (D, I), 1 / math.sqrt(I), e, bf, device) for e in range(E)])
    sg = device_normal(cfg.seed, TID_SGATE, (Is, D), 1 / math.sqrt(D), 0, bf, device)
    su = device_normal(cfg.seed, TID_SUP, (Is, D), 1 / math.sqrt(D), 0, bf, device)
    sd = device_normal(cfg.seed, TID_SDOWN, (D, Is), 1 / math.sqrt(Is), 0, bf, device)
    return HostShare(cfg, counts, x_slot, g, dy, xl, dyl, wg, wu, wd, sg, su, sd)
