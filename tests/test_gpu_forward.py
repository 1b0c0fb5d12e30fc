"""GPU parity of the forward path (dispatch, grouped GEMMs + SwiGLU, down projection with the
scatter epilogue, shared expert, combine) against the fp64 oracle, plus determinism."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL, ForwardRun, assert_close_rms, t2np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope='module')
def m():
    import mixture_experts_layer_norm_amd as mod
    return mod


SMALL_BF16 = synth.scaled(synth.DSV3, 'small_bf16_T300_D256_I256_E16_K4', T=300, D=256, I=256, E=16, K=4,
                          I_shared=256)
DENSE_F32 = synth.scaled(synth.TINY, 'dense_f32_E1_K1', E=1, K=1)
DENSE_BF16 = synth.scaled(synth.MID, 'dense_bf16_E1_K1', T=200, D=256, I=128, E=1, K=1, I_shared=128)
NOSHARED_BF16 = synth.scaled(synth.MID, 'noshared_bf16', T=257, D=384, I=256, E=12, K=3, I_shared=0)
ONE_TOKEN = synth.scaled(synth.MID, 'one_token_bf16', T=1, D=256, I=128, E=8, K=2, I_shared=128)


def oracle_forward(H: synth.HostLayer):
    return oracle.moe_forward(H.x, H.logits, H.w_gate, H.w_up, H.w_down, H.cfg.K, H.ws_gate, H.ws_up, H.ws_down)


def check_forward(m, cfg, flags=0, chunk_rows=0):
    print(f'[forward] {cfg.name} flags={flags} chunk={chunk_rows}', flush=True)
    H = synth.host_layer(cfg)
    L = synth.to_device(H)
    run = ForwardRun(m, L, flags=flags, chunk_rows=chunk_rows)()
    torch.cuda.synchronize()
    out, idx, g, y, sh = oracle_forward(H)
    tau = TOL[cfg.dtype]
    bf = cfg.dtype != 'f32'
    assert np.array_equal(run.topk_idx.cpu().numpy(), idx)
    assert_close_rms(t2np(run.topk_w), g, TOL['f32'], 'g')
    # per-route expert outputs in route order (push-combine destinations)
    assert_close_rms(t2np(run.y_routes), y.reshape(cfg.T * cfg.K, cfg.D), tau, 'y_routes', bf)
    if cfg.I_shared:
        assert_close_rms(t2np(run.shared_out), sh, tau, 'shared_out', bf)
    assert_close_rms(t2np(run.out), out, tau, 'out', bf)
    return run


@pytest.mark.parametrize('cfg', [synth.TINY, DENSE_F32, SMALL_BF16, DENSE_BF16, NOSHARED_BF16, ONE_TOKEN],
                         ids=lambda c: c.name)
def test_forward_small(m, cfg):
    check_forward(m, cfg)


def test_forward_tiny_ties(m):
    """Tie-heavy logits (multiples of 0.25): routing stays bit-exact and the layer matches."""
    H = synth.host_layer(synth.TINY)
    H.logits = synth.tie_logits(H.logits)
    L = synth.to_device(H)
    run = ForwardRun(m, L)()
    torch.cuda.synchronize()
    out, idx, *_ = oracle_forward(H)
    assert np.array_equal(run.topk_idx.cpu().numpy(), idx)
    assert_close_rms(t2np(run.out), out, TOL['f32'], 'out')


def test_forward_mid(m):
    check_forward(m, synth.MID)


@pytest.mark.parametrize('cfg', [SMALL_BF16, DENSE_F32], ids=lambda c: c.name)
def test_forward_gather_matches_dispatch_copy_bitwise(m, cfg):
    """The default forward reads x through the schedule; MOE_FLAG_DISPATCH_COPY writes the slot copy
    first. Same rows, same GEMM tiles: the same bits (MOE_FLAG_FUSED_GATHER names the default)."""
    H = synth.host_layer(cfg)
    L = synth.to_device(H)
    a = ForwardRun(m, L)()
    b = ForwardRun(m, L, flags=m.MOE_FLAG_DISPATCH_COPY)()
    c = ForwardRun(m, L, flags=m.MOE_FLAG_FUSED_GATHER)()
    torch.cuda.synchronize()
    assert b.ws.numel() > a.ws.numel()      # the copy needs the slot buffer
    for r in (b, c):
        assert torch.equal(a.out, r.out) and torch.equal(a.y_routes, r.y_routes)


def test_forward_bitwise_deterministic(m):
    H = synth.host_layer(SMALL_BF16)
    L = synth.to_device(H)
    run = ForwardRun(m, L)
    ref = run().out.clone()
    for _ in range(20):
        run()
        assert torch.equal(run.out, ref)


@pytest.mark.parametrize('D', [256, 4096, 7168])
def test_dispatch_standalone(m, D):
    """moe_dispatch copies rows x[perm[j] / K] exactly (perm from the oracle's schedule); rows of
    4096 and 7168 columns take the 8-loads-in-flight loop plus its tail."""
    cfg = synth.scaled(SMALL_BF16, f'dispatch_D{D}', D=D)
    H = synth.host_layer(cfg)
    _, _, perm, _ = oracle.schedule(oracle.route_topk(H.logits, cfg.K), cfg.E)
    p = m.problem(cfg.T, cfg.D, cfg.I, cfg.E, cfg.K, cfg.I_shared, cfg.dtype)
    x = torch.from_numpy(H.x).cuda().to(torch.bfloat16)
    perm_d = torch.from_numpy(perm).cuda()
    n = cfg.T * cfg.K
    for begin, count in [(0, n), (5, n - 5), (n - 1, 1), (17, 0)]:
        x_slot = torch.empty((max(count, 1), cfg.D), dtype=torch.bfloat16, device='cuda')
        m.dispatch(p, x, perm_d, begin, count, x_slot)
        torch.cuda.synchronize()
        if count:
            assert np.array_equal(t2np(x_slot[:count]), H.x[perm[begin:begin + count] // cfg.K])
    # token-major form over the whole range: same bytes
    inv = np.empty_like(perm)
    inv[perm] = np.arange(n, dtype=perm.dtype)
    x_tok = torch.empty((n, cfg.D), dtype=torch.bfloat16, device='cuda')
    m.dispatch_tokens(p, x, torch.from_numpy(inv).cuda(), x_tok)
    torch.cuda.synchronize()
    assert np.array_equal(t2np(x_tok), H.x[perm // cfg.K])


@pytest.mark.parametrize('dtype,shared,K,D', [('bf16', True, 6, 256), ('bf16', False, 6, 256), ('f32', True, 6, 256),
                                             ('bf16', True, 12, 256), ('bf16', True, 8, 4096)])
def test_combine_standalone(m, dtype, shared, K, D):
    """moe_combine against the oracle's weighted sum, on seeded per-route rows and weights (K <= 8
    keeps the weights in registers; K > 8 takes the general loop)."""
    T = 333
    bf = dtype == 'bf16'
    y = synth.host_normal(77, 0, (T * K, D), 1.0, bf16=bf)
    sh = synth.host_normal(77, 1, (T, D), 1.0, bf16=bf) if shared else None
    g = synth.host_rng(77, 2).random((T, K), dtype=np.float32)
    p = m.problem(T, D, 128, 16, K, 128 if shared else 0, dtype)
    tdt = torch.bfloat16 if bf else torch.float32
    yd = torch.from_numpy(y).cuda().to(tdt)
    shd = torch.from_numpy(sh).cuda().to(tdt) if shared else None
    out = torch.empty((T, D), dtype=tdt, device='cuda')
    m.combine(p, yd, shd, torch.from_numpy(g).cuda(), out)
    torch.cuda.synchronize()
    ref = oracle.combine(sh, y, g)
    assert_close_rms(t2np(out), ref, 1e-5, 'combine', bf)
    out2 = torch.empty_like(out)
    m.combine(p, yd, shd, torch.from_numpy(g).cuda(), out2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


@pytest.mark.slow
def test_forward_dsv3_full_size_sampled(m):
    """DeepSeek-V3 shape (T=8192, D=7168, I=2048, E=256, K=8, shared I=2048) in the launch
    configuration the benchmark times. Routing and schedule checked in full; against the oracle:
    the layer output of 256 sampled tokens, and the per-route expert outputs y of two whole
    experts, the hottest one (its rows span several m-tiles, the last one partial) and the
    smallest non-empty one."""
    cfg = synth.DSV3
    print('[forward] dsv3 full size: generating inputs', flush=True)
    L = synth.device_layer(cfg)
    run = ForwardRun(m, L, want_parts=True)()
    torch.cuda.synchronize()
    lg = L.logits.cpu().numpy()
    idx = oracle.route_topk(lg, cfg.K)
    assert np.array_equal(run.topk_idx.cpu().numpy(), idx)
    counts, offsets, perm, inv = oracle.schedule(idx, cfg.E)
    assert np.array_equal(run.perm.cpu().numpy(), perm)
    cache = {}

    def weights(e):
        if e not in cache:
            cache.clear()       # one expert at a time: the oracle visits experts in order
            cache[e] = tuple(w[e].float().cpu().numpy() for w in (L.w_gate, L.w_up, L.w_down))
        return cache[e]

    # whole experts: every route of the hottest and of the smallest non-empty expert
    nz = np.nonzero(counts)[0]
    for e in (int(np.argmax(counts)), int(nz[np.argmin(counts[nz])])):
        routes = perm[offsets[e]:offsets[e + 1]]
        print(f'[forward] dsv3 y_routes of expert {e} ({routes.size} routes)', flush=True)
        xs = L.x[torch.from_numpy(routes // cfg.K).cuda()].float().cpu().numpy()
        ref = oracle.swiglu_expert(xs, *weights(e))
        got = run.y_routes[torch.from_numpy(routes).cuda()].float().cpu().numpy()
        assert_close_rms(got, ref, TOL['bf16'], f'dsv3 y_routes expert {e}', True)
    toks = np.sort(np.random.default_rng(0).choice(cfg.T, 256, replace=False))
    xs = L.x[torch.from_numpy(toks).cuda()].float().cpu().numpy()
    print(f'[forward] dsv3 oracle on {len(toks)} tokens, {len(set(idx[toks].ravel().tolist()))} experts', flush=True)
    out, *_ = oracle.moe_forward(xs, lg[toks], lambda e: weights(e)[0], lambda e: weights(e)[1],
                                 lambda e: weights(e)[2], cfg.K, L.ws_gate.float().cpu().numpy(),
                                 L.ws_up.float().cpu().numpy(), L.ws_down.float().cpu().numpy())
    got = run.out[torch.from_numpy(toks).cuda()].float().cpu().numpy()
    assert_close_rms(got, out, TOL['bf16'], 'dsv3 sampled out', True)


def chunked_equals_unchunked(m, chunk, stages, flags=0):
    print(f'[chunked] chunk={chunk} stages={stages} flags={flags}', flush=True)
    L = synth.to_device(synth.host_layer(SMALL_BF16))
    a = ForwardRun(m, L)()
    b = ForwardRun(m, L, chunk_rows=chunk, ring_stages=stages, flags=flags)()
    torch.cuda.synchronize()
    assert int(b.ws[:4].view(torch.int32).item()) == 0
    assert torch.equal(a.y_routes, b.y_routes)
    assert torch.equal(a.shared_out, b.shared_out)
    assert torch.equal(a.out, b.out)


@pytest.mark.parametrize('chunk,stages', [(256, 3), (512, 3), (256, 4), (768, 5), (1 << 20, 3)])
def test_chunked_ring_bitwise_equals_unchunked(m, chunk, stages):
    """Chunks of `chunk` routed slots carried through a ring of `stages` chunk buffers give bitwise
    the same per-route rows, shared output and layer output as the unchunked path: every output
    tile is one workgroup's fixed-order sum, whatever the chunking."""
    chunked_equals_unchunked(m, chunk, stages)


@pytest.mark.parametrize('chunk,stages', [(256, 3), (768, 5)])
def test_chunked_ring_dispatch_copy_bitwise_equals_unchunked(m, chunk, stages):
    """The same with MOE_FLAG_DISPATCH_COPY: each chunk's x rows dispatched into its ring stage
    instead of read through the schedule."""
    chunked_equals_unchunked(m, chunk, stages, flags=m.MOE_FLAG_DISPATCH_COPY)


@pytest.mark.skip(reason='the persistent work-queue chunk kernel hung on MI355X twice (second time after '
                         'bounding its waits); its cause is not yet shown, so the path is switched off and '
                         'MOE_FLAG_PERSISTENT returns MOE_ERR_UNSUPPORTED')
@pytest.mark.parametrize('chunk,stages', [(256, 3), (768, 5)])
def test_persistent_pipeline_bitwise_equals_unchunked(m, chunk, stages):
    chunked_equals_unchunked(m, chunk, stages, flags=m.MOE_FLAG_PERSISTENT)


def test_chunked_ring_mid_parity(m):
    """Chunked ring at the mid shape (T=4096, E=128, K=8) against the oracle."""
    check_forward(m, synth.MID, chunk_rows=512)


def test_forward_stages_equals_forward(m):
    """moe_forward_stages (stage events recorded between the launches) gives the same bits as
    moe_forward, also when calls on the same stream interleave."""
    L = synth.to_device(synth.host_layer(SMALL_BF16))
    a = ForwardRun(m, L)
    b = ForwardRun(m, L)
    events = [torch.cuda.Event(enable_timing=True) for _ in range(len(m.STAGES) + 1)]
    for e in events:
        e.record()
    outs = []
    for _ in range(3):
        a()
        m.forward_stages(b.p, L.x, L.logits, b.weights, b.out, b.routing, b.ws, events, b.y_routes, b.shared_out)
        torch.cuda.synchronize()
        assert torch.equal(a.out, b.out) and torch.equal(a.shared_out, b.shared_out)
        outs.append(a.out.clone())
    assert all(torch.equal(outs[0], o) for o in outs[1:])


