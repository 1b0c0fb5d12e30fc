"""GPU parity of top-k routing and the schedule against the oracle: bit-exact indices, counts,
offsets and permutation; router weights within the fp32 tolerance."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL, assert_close_rms

pytestmark = pytest.mark.gpu


@pytest.fixture(scope='module')
def m():
    import mixture_experts_layer_norm_amd as mod
    return mod


def run_route(m, logits_np, K):
    T, E = logits_np.shape
    p = m.problem(T, 128, 128, E, K, 0, 'bf16')
    lg = torch.from_numpy(np.ascontiguousarray(logits_np)).cuda()
    idx = torch.empty((T, K), dtype=torch.int32, device='cuda')
    w = torch.empty((T, K), dtype=torch.float32, device='cuda')
    m.route_topk(p, lg, idx, w)
    counts = torch.empty((E,), dtype=torch.int32, device='cuda')
    offsets = torch.empty((E + 1,), dtype=torch.int32, device='cuda')
    perm = torch.empty((T * K,), dtype=torch.int32, device='cuda')
    inv = torch.empty((T * K,), dtype=torch.int32, device='cuda')
    ws = torch.zeros((m.workspace_size(p),), dtype=torch.uint8, device='cuda')
    m.schedule(p, idx, counts, offsets, perm, inv, ws)
    torch.cuda.synchronize()
    err = int(ws[:4].view(torch.int32).item())
    return [t.cpu().numpy() for t in (idx, w, counts, offsets, perm, inv)] + [err]


def check_route(m, lg, K):
    idx, w, counts, offsets, perm, inv, err = run_route(m, lg, K)
    E = lg.shape[1]
    ridx = oracle.route_topk(lg, K)
    assert np.array_equal(idx, ridx), 'top-k indices differ'
    rg = oracle.routing_weights(lg, ridx)
    assert_close_rms(w, rg, TOL['f32'], 'g')
    rc, ro, rp, ri = oracle.schedule(ridx, E)
    assert np.array_equal(counts, rc) and np.array_equal(offsets, ro)
    assert np.array_equal(perm, rp) and np.array_equal(inv, ri)
    assert err == 0


def synth_logits(cfg):
    if cfg.router == 'zipf_gumbel':
        return synth.router_logits_host(cfg, None)
    x = synth.host_normal(cfg.seed, synth.TID_X, (cfg.T, cfg.D), 1.0, bf16=cfg.dtype != 'f32')
    return synth.router_logits_host(cfg, x)


@pytest.mark.parametrize('cfg', [synth.TINY, synth.MID, synth.DSV3, synth.MXFP8], ids=lambda c: c.name)
def test_route_and_schedule_configs(m, cfg):
    print(f'[route] {cfg.name}', flush=True)
    check_route(m, synth_logits(cfg), cfg.K)


def test_route_ties(m):
    lg = synth.tie_logits(synth_logits(synth.TINY))
    check_route(m, lg, 2)
    lg = synth.tie_logits(synth_logits(synth.MID), 0.5)
    check_route(m, lg, 8)


@pytest.mark.parametrize('T,E,K', [(1, 1, 1), (1, 8, 8), (37, 8, 8), (513, 100, 7), (300, 1024, 64),
                                   (4099, 256, 8), (2048 * 3 + 5, 64, 1)])
def test_route_edge_shapes(m, T, E, K):
    rng = np.random.default_rng(T * 131 + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    check_route(m, lg, K)


def test_route_special_values(m):
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((64, 16)).astype(np.float32)
    lg[0] = 0.0
    lg[0, ::2] = -0.0
    lg[1, 3] = np.nan
    lg[2, :] = -np.inf
    lg[2, [5, 9, 11, 12]] = [1.0, 1.0, -2.0, 3.0]
    lg[3, :8] = np.inf
    lg[3, 8:] = 1.0
    idx, w, *_ = run_route(m, lg, 4)
    assert np.array_equal(idx, oracle.route_topk(lg, 4))


def test_schedule_skewed_all_to_one_expert(m):
    """Every token prefers expert 3 and 7: two experts take all routes, the rest stay empty."""
    T, E, K = 5000, 32, 2
    lg = np.full((T, E), -1.0, dtype=np.float32)
    lg[:, 3] = 2.0
    lg[:, 7] = 1.0
    check_route(m, lg, K)


def test_schedule_bitwise_repeatable(m):
    lg = synth_logits(synth.DSV3)
    a = run_route(m, lg, 8)
    for _ in range(5):
        b = run_route(m, lg, 8)
        for u, v in zip(a, b):
            assert np.array_equal(u, v)


def test_schedule_out_of_range_ids_set_error_word(m):
    """A caller-supplied expert id outside [0, E) is clamped and reported, never dereferenced."""
    T, E, K = 100, 8, 2
    p = m.problem(T, 128, 128, E, K, 0, 'bf16')
    idx = torch.randint(0, E, (T, K), dtype=torch.int32, device='cuda')
    idx[7, 1] = 99
    idx[8, 0] = -3
    counts = torch.empty((E,), dtype=torch.int32, device='cuda')
    offsets = torch.empty((E + 1,), dtype=torch.int32, device='cuda')
    perm = torch.empty((T * K,), dtype=torch.int32, device='cuda')
    inv = torch.empty((T * K,), dtype=torch.int32, device='cuda')
    ws = torch.zeros((m.workspace_size(p),), dtype=torch.uint8, device='cuda')
    m.schedule(p, idx, counts, offsets, perm, inv, ws)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) != 0
    pc = perm.cpu().numpy()
    assert sorted(pc.tolist()) == list(range(T * K))
    assert int(counts.sum().item()) == T * K
