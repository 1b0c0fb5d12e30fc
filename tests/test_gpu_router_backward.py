"""GPU parity of the router backward (moe_route_gemm_backward: dW_r = d_logits^T x and
dx += d_logits W_r) against the oracle's router_backward.

* Small-integer x, W_r and d_logits: every product and partial sum is exact in fp32, so dW_r is
  compared bit for bit and dx against the oracle's exact sum rounded once to BF16 (RNE).
* Normal inputs: dW_r (fp32) within 1e-4 RMS of the oracle; dx within 1e-4 RMS plus the BF16
  rounding of its stored value.
* The whole layer through the router: logits from moe_route_gemm, moe_forward, moe_backward, then
  moe_route_gemm_backward, against the oracle's layer backward plus router_backward (BF16 path:
  2e-2 RMS; dx is rounded twice, once by moe_backward and once here, so its bound carries two
  half-ulps of BF16).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL, assert_close_rms, half_ulp_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope='module')
def m():
    import mixture_experts_layer_norm_amd as mod
    return mod


def bf(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(torch.bfloat16)


def sparse_dlogits(rng, T, E, K, ints):
    """d_logits as moe_backward writes them: nonzero only on K experts per token."""
    dl = np.zeros((T, E), dtype=np.float32)
    cols = np.stack([rng.permutation(E)[:K] for _ in range(T)])
    vals = rng.integers(-8, 9, (T, K)).astype(np.float32) if ints else rng.standard_normal((T, K)).astype(np.float32)
    np.put_along_axis(dl, cols, vals, axis=1)
    return dl


def run(m, x, w, dl, dx0):
    T, D = x.shape
    E = w.shape[0]
    p = m.problem(T, D, 128, E, 1, 0, 'bf16')
    dw = torch.full((E, D), float('nan'), dtype=torch.float32, device='cuda')
    dx = bf(dx0)
    m.route_gemm_backward(p, bf(x), bf(w), torch.from_numpy(dl).cuda(), dw, dx)
    torch.cuda.synchronize()
    return dw.cpu().numpy().astype(np.float64), dx.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize('T,D,E,K', [(300, 256, 16, 2), (513, 1024, 300, 6), (8192, 7168, 256, 8)])
def test_router_backward_exact_integers(m, T, D, E, K):
    rng = np.random.default_rng(T + D)
    x = rng.integers(-4, 5, (T, D)).astype(np.float64)
    w = rng.integers(-4, 5, (E, D)).astype(np.float64)
    dl = sparse_dlogits(rng, T, E, K, True)
    dx0 = rng.integers(-64, 65, (T, D)).astype(np.float64)
    dw, dx = run(m, x, w, dl, dx0)
    rdw, rdx = oracle.router_backward(x, w, dl)
    assert np.array_equal(dw, rdw)
    assert np.array_equal(dx, synth.round_bf16(dx0 + rdx).astype(np.float64))


@pytest.mark.parametrize('T,D,E,K', [(777, 2048, 128, 8), (4096, 7168, 256, 8)])
def test_router_backward_normal_inputs(m, T, D, E, K):
    rng = np.random.default_rng(7 * T)
    x = synth.round_bf16(rng.standard_normal((T, D))).astype(np.float64)
    w = synth.round_bf16(rng.standard_normal((E, D)) / np.sqrt(D)).astype(np.float64)
    dl = sparse_dlogits(rng, T, E, K, False)
    dx0 = synth.round_bf16(rng.standard_normal((T, D)) * 0.05).astype(np.float64)
    dw, dx = run(m, x, w, dl, dx0)
    rdw, rdx = oracle.router_backward(x, w, dl)
    assert_close_rms(dw, rdw, TOL['f32'], 'dW_r')
    assert_close_rms(dx, dx0 + rdx, TOL['f32'], 'dx + router term', True)


def test_layer_backward_through_the_router(m):
    """Layer with its router: small-integer x and W_r keep the logits exact, so routing and the
    oracle agree bit for bit; the experts' weights are normal."""
    cfg = synth.scaled(synth.DSV3, 'router_bwd_T300_D256_I256_E16_K4', T=300, D=256, I=256, E=16, K=4, I_shared=256)
    H = synth.host_layer(cfg)
    T, D, E, K = cfg.T, cfg.D, cfg.E, cfg.K
    rng = np.random.default_rng(11)
    x = rng.integers(-3, 4, (T, D)).astype(np.float64)
    wr = rng.integers(-2, 3, (E, D)).astype(np.float64) / 16.0
    p = m.problem(T, D, cfg.I, E, K, cfg.I_shared, 'bf16')
    xt, wrt = bf(x), bf(wr)
    lg = torch.empty((T, E), dtype=torch.float32, device='cuda')
    rt = [torch.empty((T, K), dtype=torch.int32, device='cuda'), torch.empty((T, K), dtype=torch.float32, device='cuda'),
          torch.empty((E,), dtype=torch.int32, device='cuda'), torch.empty((E + 1,), dtype=torch.int32, device='cuda'),
          torch.empty((T * K,), dtype=torch.int32, device='cuda'), torch.empty((T * K,), dtype=torch.int32, device='cuda')]
    ws_r = torch.zeros((m.route_gemm_workspace_size(p),), dtype=torch.uint8, device='cuda')
    m.route_gemm(p, xt, wrt, lg, rt[0], rt[1], ws_r)
    # the weight tensors must outlive every call: make_weights keeps only their device pointers
    wts = [bf(getattr(H, k)) for k in ('w_gate', 'w_up', 'w_down', 'ws_gate', 'ws_up', 'ws_down')]
    W = m.make_weights(*wts)
    out = torch.empty((T, D), dtype=torch.bfloat16, device='cuda')
    ws = torch.zeros((m.workspace_size(p),), dtype=torch.uint8, device='cuda')
    m.forward(p, xt, lg, W, out, m.make_routing(*rt), ws)
    dout = synth.round_bf16(rng.standard_normal((T, D))).astype(np.float64)
    gr = dict(dw_gate=torch.empty((E, cfg.I, D), device='cuda'), dw_up=torch.empty((E, cfg.I, D), device='cuda'),
              dw_down=torch.empty((E, D, cfg.I), device='cuda'), dws_gate=torch.empty((cfg.I_shared, D), device='cuda'),
              dws_up=torch.empty((cfg.I_shared, D), device='cuda'), dws_down=torch.empty((D, cfg.I_shared), device='cuda'))
    dx = torch.empty((T, D), dtype=torch.bfloat16, device='cuda')
    dtw = torch.empty((T, K), dtype=torch.float32, device='cuda')
    dlg = torch.empty((T, E), dtype=torch.float32, device='cuda')
    wsb = torch.zeros((m.backward_workspace_size(p),), dtype=torch.uint8, device='cuda')
    m.backward(p, bf(dout), xt, lg, W, m.make_routing(*rt), dx, m.make_grads(**gr), dtw, dlg, wsb)
    dx_experts = dx.float().cpu().numpy().astype(np.float64)
    dwr = torch.full((E, D), float('nan'), dtype=torch.float32, device='cuda')
    m.route_gemm_backward(p, xt, wrt, dlg, dwr, dx)
    torch.cuda.synchronize()
    logits = oracle.router_logits(x, wr)
    assert np.array_equal(lg.cpu().numpy().astype(np.float64), logits)      # exact in fp32
    ref = oracle.moe_backward(x, logits, H.w_gate, H.w_up, H.w_down, K, dout, H.ws_gate, H.ws_up, H.ws_down)
    assert np.array_equal(rt[0].cpu().numpy(), ref['idx'])
    rdw, rdx = oracle.router_backward(x, wr, ref['d_logits'])
    assert_close_rms(dwr.cpu().numpy(), rdw, TOL['bf16'], 'layer dW_r')
    # the experts' dx (moe_backward) first, then the router's increment on top of it
    assert_close_rms(dx_experts, ref['dx'], TOL['bf16'], 'layer dx of the experts', True)
    inc = dx.float().cpu().numpy().astype(np.float64) - dx_experts
    assert_close_rms(inc, rdx, TOL['bf16'], 'router increment of dx', False,
                     half_ulp_bf16(dx_experts + rdx) + 1e-30)
    want = ref['dx'] + rdx
    got = dx.float().cpu().numpy().astype(np.float64)
    rms = float(np.sqrt(np.mean(want ** 2)))
    bound = TOL['bf16'] * rms + half_ulp_bf16(want) + half_ulp_bf16(dx_experts)
    worst = float(np.max(np.abs(got - want) / bound))
    print(f'  layer dx with router: max|d|/RMS = {np.abs(got - want).max() / rms:.2e}; worst at {worst:.2f} of bound',
          flush=True)
    assert worst <= 1.0
    # deterministic: a second router backward onto the experts' dx gives the same bits
    dx2 = torch.from_numpy(dx_experts.astype(np.float32)).cuda().to(torch.bfloat16)
    dwr2 = torch.empty_like(dwr)
    m.route_gemm_backward(p, xt, wrt, dlg, dwr2, dx2)
    torch.cuda.synchronize()
    assert torch.equal(dwr, dwr2) and torch.equal(dx, dx2)


@pytest.mark.parametrize('T,D,E,density', [(1000, 1024, 64, 0.1), (300, 256, 300, 1.0), (2048, 7168, 256, 8 / 256)])
def test_router_backward_sparse_kernels_equal_dense_bitwise(m, T, D, E, density):
    """Aligned operands take the kernels that skip zero d_logits entries; the same values stored at
    misaligned addresses, or MOE_FLAG_ROUTER_BWD_DENSE, take the dense FMA kernel. Skipping exact-zero products leaves every fp32
    sum unchanged, so both give the same bits: sparse, dense (every entry nonzero) and signed-zero
    d_logits, E a multiple of 4 or not."""
    print(f'[router bwd] sparse = dense T={T} D={D} E={E} density={density:.3f}', flush=True)
    g = torch.Generator(device='cuda')
    g.manual_seed(T + E)
    x = torch.randn((T, D), device='cuda', generator=g).to(torch.bfloat16)
    w = (torch.randn((E, D), device='cuda', generator=g) / np.sqrt(D)).to(torch.bfloat16)
    keep = torch.rand((T, E), device='cuda', generator=g) < density
    dl = torch.where(keep, torch.randn((T, E), device='cuda', generator=g), torch.zeros((T, E), device='cuda'))
    dl[::7, ::5] = -0.0                       # negative zeros are zeros too
    dx0 = (torch.randn((T, D), device='cuda', generator=g) * 0.05).to(torch.bfloat16)
    p = m.problem(T, D, 128, E, 1, 0, 'bf16')

    def shifted(t, elems):
        """A copy of t whose data starts `elems` elements past an aligned allocation."""
        buf = torch.empty(t.numel() + elems, dtype=t.dtype, device='cuda')
        v = buf[elems:].view(t.shape)
        v.copy_(t)
        return v

    dw1 = torch.full((E, D), float('nan'), device='cuda')
    dx1 = dx0.clone()
    m.route_gemm_backward(p, x, w, dl, dw1, dx1)
    xs, ws_, dxs = shifted(x, 1), shifted(w, 1), shifted(dx0, 1)
    dw2 = shifted(torch.full((E, D), float('nan'), device='cuda'), 1)
    assert xs.data_ptr() % 4 and ws_.data_ptr() % 16 and dxs.data_ptr() % 16 and dw2.data_ptr() % 8
    m.route_gemm_backward(p, xs, ws_, dl, dw2, dxs)
    # MOE_FLAG_ROUTER_BWD_DENSE selects the dense kernel on aligned operands too
    pd = m.problem(T, D, 128, E, 1, 0, 'bf16', flags=m.MOE_FLAG_ROUTER_BWD_DENSE)
    dw3 = torch.full((E, D), float('nan'), device='cuda')
    dx3 = dx0.clone()
    m.route_gemm_backward(pd, x, w, dl, dw3, dx3)
    torch.cuda.synchronize()
    assert torch.equal(dw1, dw2) and torch.equal(dw1, dw3)
    assert torch.equal(dx1, dxs) and torch.equal(dx1, dx3)
