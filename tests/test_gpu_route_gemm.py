"""GPU parity of the fused router (moe_route_gemm: router GEMM split along D + top-K) against
the oracle: logits = x W_r^T, top-K and routing weights. With small-integer inputs every partial
sum is exact in fp32, so logits and the selected experts are compared bit for bit; with normal
inputs the logits are held to the fp32 tolerance and the selection to the oracle's order wherever
the oracle's logits are not within that tolerance of a tie."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, assert_close_rms

pytestmark = pytest.mark.gpu


@pytest.fixture(scope='module')
def m():
    import mixture_experts_layer_norm_amd as mod
    return mod


def run(m, x, w, K):
    T, D = x.shape
    E = w.shape[0]
    p = m.problem(T, D, 128, E, K, 0, 'bf16')
    dev = 'cuda'
    xt = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev).to(torch.bfloat16)
    wt = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(dev).to(torch.bfloat16)
    lg = torch.full((T, E), float('nan'), dtype=torch.float32, device=dev)
    idx = torch.full((T, K), -1, dtype=torch.int32, device=dev)
    g = torch.full((T, K), float('nan'), dtype=torch.float32, device=dev)
    ws = torch.zeros((m.route_gemm_workspace_size(p),), dtype=torch.uint8, device=dev)
    m.route_gemm(p, xt, wt, lg, idx, g, ws)
    torch.cuda.synchronize()
    return lg.cpu().numpy(), idx.cpu().numpy(), g.cpu().numpy()


@pytest.mark.parametrize('T,D,E,K', [(300, 256, 16, 2), (777, 2048, 256, 8), (8192, 7168, 256, 8),
                                     (513, 1024, 300, 6)])
def test_route_gemm_exact_integers(m, T, D, E, K):
    rng = np.random.default_rng(T + D + E)
    x = rng.integers(-3, 4, (T, D)).astype(np.float64)
    w = rng.integers(-3, 4, (E, D)).astype(np.float64)
    lg, idx, g = run(m, x, w, K)
    ref = x @ w.T                         # integers below 2^24: exact in fp32 in any order
    assert np.array_equal(lg.astype(np.float64), ref)
    ridx = oracle.route_topk(ref, K)      # ties (frequent with integers) to the lower index
    assert np.array_equal(idx, ridx)
    rg = oracle.routing_weights(ref, ridx)
    assert np.max(np.abs(g - rg)) <= 1e-6


def test_route_gemm_normal_inputs(m):
    T, D, E, K = 1000, 7168, 256, 8
    rng = np.random.default_rng(7)
    x = rng.standard_normal((T, D)).astype(np.float32)
    w = (rng.standard_normal((E, D)) / np.sqrt(D)).astype(np.float32)
    # the bf16 values both sides use
    xb = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    wb = torch.from_numpy(w).to(torch.bfloat16).float().numpy().astype(np.float64)
    lg, idx, g = run(m, xb, wb, K)
    ref = xb @ wb.T
    assert_close_rms(lg.astype(np.float64), ref, TOL['f32'], 'router logits')
    tol = TOL['f32'] * float(np.sqrt(np.mean(ref ** 2)))
    srt = np.sort(ref, axis=1)[:, ::-1]
    kth = srt[:, K - 1]
    # every chosen expert is within tol of the oracle's top K
    chosen = np.take_along_axis(ref, idx.astype(np.int64), axis=1)
    assert np.all(chosen >= kth[:, None] - tol)
    assert all(len(set(r)) == K for r in idx.tolist())
    # tokens without a near-tie at any of the first K + 1 ranks: identical selection and order
    gaps = np.min(np.abs(np.diff(srt[:, :K + 1], axis=1)), axis=1)
    clear = gaps > 2 * tol
    assert clear.mean() > 0.5
    ridx = oracle.route_topk(ref, K)
    assert np.array_equal(idx[clear], ridx[clear])
    rg = oracle.routing_weights(ref, ridx)
    assert np.max(np.abs(g[clear] - rg[clear])) <= 1e-4
