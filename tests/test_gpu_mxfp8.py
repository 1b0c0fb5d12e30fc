"""GPU parity of the MXFP8 path: the quantiser and the quantising dispatch bit-exact against the
oracle's OCP MX encoder, and the MXFP8 forward against the oracle run on the same quantised
values in fp64 (h quantised before the down projection; shared expert in BF16)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL, assert_close_rms, frac_beyond, mx_choice_allowance, t2np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope='module')
def m():
    import mixture_experts_layer_norm_amd as mod
    return mod


def bf(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(torch.bfloat16)


def u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


@pytest.mark.parametrize('rows,cols', [(1, 32), (37, 256), (512, 7168)])
def test_quantize_mx_bit_exact(m, rows, cols):
    rng = np.random.default_rng(rows)
    v = rng.standard_normal((rows, cols)).astype(np.float32) * np.exp(rng.standard_normal((rows, 1)) * 6).astype(np.float32)
    v[0, :32] = 0.0                                      # an all-zero block
    if cols >= 64:
        v[0, 32:64] = 1.0                                # amax an exact power of two
        v[0, 40] = 1.96875                               # saturates to 448
    if rows > 1:
        v[1, :] *= 1e-38                                 # tiny (bf16 subnormal range)
    v = synth.round_bf16(v)
    q = torch.empty((rows, cols), dtype=torch.uint8, device='cuda')
    sc = torch.empty((rows, cols // 32), dtype=torch.uint8, device='cuda')
    m.quantize_mx(bf(v), q, sc)
    torch.cuda.synchronize()
    rq, rs = oracle.mx_quantize(v.astype(np.float64))
    assert np.array_equal(sc.cpu().numpy(), rs)
    assert np.array_equal(q.cpu().numpy(), rq)


MX_SMALL = synth.scaled(synth.MXFP8, 'small_mxfp8_T300_D256_I256_E16_K4', T=300, D=256, I=256, E=16, K=4,
                        I_shared=256)


def mx_layer(cfg):
    H = synth.host_layer(cfg)
    q = {k: oracle.mx_quantize(getattr(H, k).astype(np.float64)) for k in ('w_gate', 'w_up', 'w_down')}
    return H, q


def run_mx_forward(m, H, q, act=None, chunk_rows=0, ring_stages=0, lanes=None, flags=0, budget=None):
    """moe_forward in MXFP8; with act = [a, u] buffers, moe_forward_keep; with lanes = (streams,
    events), moe_forward_lanes; budget: the workgroup budget word's value."""
    cfg = H.cfg
    T, K, D, E = cfg.T, cfg.K, cfg.D, cfg.E
    p = m.problem(T, D, cfg.I, E, K, cfg.I_shared, 'mxfp8', chunk_rows, ring_stages, flags)
    tensors = dict(x=bf(H.x), logits=torch.from_numpy(H.logits).cuda(),
                   wq=[u8(q[k][0]) for k in ('w_gate', 'w_up', 'w_down')],
                   ws=[bf(H.ws_gate), bf(H.ws_up), bf(H.ws_down)],
                   sc=[u8(q[k][1]) for k in ('w_gate', 'w_up', 'w_down')])
    W = m.make_weights(*tensors['wq'], *tensors['ws'], *tensors['sc'])
    rt = [torch.empty((T, K), dtype=torch.int32, device='cuda'), torch.empty((T, K), dtype=torch.float32, device='cuda'),
          torch.empty((E,), dtype=torch.int32, device='cuda'), torch.empty((E + 1,), dtype=torch.int32, device='cuda'),
          torch.empty((T * K,), dtype=torch.int32, device='cuda'), torch.empty((T * K,), dtype=torch.int32, device='cuda')]
    out = torch.empty((T, D), dtype=torch.bfloat16, device='cuda')
    yr = torch.empty((T * K, D), dtype=torch.bfloat16, device='cuda')
    ws = torch.zeros((m.workspace_size(p),), dtype=torch.uint8, device='cuda')
    if budget is not None:
        ws[m.MOE_WS_CU_BUDGET_OFFSET:m.MOE_WS_CU_BUDGET_OFFSET + 4].view(torch.int32).fill_(budget)
    if lanes is not None:
        m.forward_lanes(p, tensors['x'], tensors['logits'], W, out, m.make_routing(*rt), ws, *lanes, y_routes=yr)
    elif act is None:
        m.forward(p, tensors['x'], tensors['logits'], W, out, m.make_routing(*rt), ws, y_routes=yr)
    else:
        m.forward_keep(p, tensors['x'], tensors['logits'], W, out, m.make_routing(*rt), *act, ws, y_routes=yr)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0
    return out, yr, rt, p, tensors


def oracle_mx_forward(x, logits, deq, K, ws_gate, ws_up, ws_down):
    """oracle.moe_forward_mx, plus the per-element allowance for equally correct alternative h
    decisions (see gpu_util.mx_choice_allowance), propagated through |W_down| to y and through g
    to out. deq: the oracle's own dequantised MX weights (dict of arrays or callables e -> array)."""
    get = lambda w, e: w(e) if callable(w) else w[e]
    out, idx, g, y, sh, hs = oracle.moe_forward_mx(x, logits, deq['w_gate'], deq['w_up'], deq['w_down'], K,
                                                   ws_gate, ws_up, ws_down, return_h=True)
    ya = np.zeros_like(y)
    for e, (t, k, H) in hs.items():
        ya[t, k] = mx_choice_allowance(H) @ np.abs(np.asarray(get(deq['w_down'], e))).T
    out_allow = np.einsum('tk,tkd->td', g, ya)
    return out, idx, y, ya, out_allow


# Share of elements allowed beyond tau * RMS with no allowance for alternative decisions: genuine
# decision flips touch few elements, a wrong axis or a dropped term moves most of them.
MAX_FRAC_BEYOND = 5e-3


def test_mx_dispatch_bit_exact(m):
    cfg = MX_SMALL
    H = synth.host_layer(cfg)
    idx = oracle.route_topk(H.logits, cfg.K)
    _, _, perm, inv = oracle.schedule(idx, cfg.E)
    n = cfg.T * cfg.K
    p = m.problem(cfg.T, cfg.D, cfg.I, cfg.E, cfg.K, cfg.I_shared, 'mxfp8')
    xq = torch.empty((n, cfg.D), dtype=torch.uint8, device='cuda')
    xs = torch.empty((n, cfg.D // 32), dtype=torch.uint8, device='cuda')
    m.dispatch(p, bf(H.x), torch.from_numpy(perm).cuda(), 0, n, xq, xs)
    torch.cuda.synchronize()
    rq, rs = oracle.mx_quantize(H.x[perm // cfg.K].astype(np.float64))
    assert np.array_equal(xs.cpu().numpy(), rs) and np.array_equal(xq.cpu().numpy(), rq)
    # token-major form (the forward's slot copies under MOE_FLAG_DISPATCH_COPY): same bytes
    xq.fill_(0xAA)
    xs.fill_(0xAA)
    m.dispatch_tokens(p, bf(H.x), torch.from_numpy(inv).cuda(), xq, xs)
    torch.cuda.synchronize()
    assert np.array_equal(xs.cpu().numpy(), rs) and np.array_equal(xq.cpu().numpy(), rq)


@pytest.mark.parametrize('T,D', [(37, 7168), (64, 2176)])
def test_mx_dispatch_tokens_wide_rows(m, T, D):
    """Token-major MXFP8 dispatch on rows of 224 and 68 blocks (more blocks than lanes, ragged),
    block magnitudes spread over 2^-20 .. 2^19 so the scale bytes vary."""
    K, E = 3, 8
    rng = np.random.default_rng(11)
    mag = np.exp2(rng.integers(-20, 20, (T, D // 32))).repeat(32, axis=1)
    x = synth.round_bf16(rng.standard_normal((T, D)) * mag)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    _, _, perm, inv = oracle.schedule(idx, E)
    n = T * K
    p = m.problem(T, D, 128, E, K, 0, 'mxfp8')
    xq = torch.full((n, D), 0xAA, dtype=torch.uint8, device='cuda')
    xs = torch.full((n, D // 32), 0xAA, dtype=torch.uint8, device='cuda')
    m.dispatch_tokens(p, bf(x), torch.from_numpy(inv).cuda(), xq, xs)
    torch.cuda.synchronize()
    rq, rs = oracle.mx_quantize(x[perm // K].astype(np.float64))
    assert np.array_equal(xs.cpu().numpy(), rs) and np.array_equal(xq.cpu().numpy(), rq)


def test_mx_forward_small(m):
    H, q = mx_layer(MX_SMALL)
    out, yr, rt, *_ = run_mx_forward(m, H, q)
    deq = {k: oracle.mx_dequantize(*q[k]) for k in q}
    ref, idx, y, ya, oa = oracle_mx_forward(H.x, H.logits, deq, MX_SMALL.K, H.ws_gate, H.ws_up, H.ws_down)
    assert np.array_equal(rt[0].cpu().numpy(), idx)
    D = MX_SMALL.D
    assert_close_rms(t2np(out), ref, TOL['mxfp8'], 'mx out', True, oa)
    assert_close_rms(t2np(yr), y.reshape(-1, D), TOL['mxfp8'], 'mx y_routes', True, ya.reshape(-1, D))
    for name, got, want in (('out', t2np(out), ref), ('y_routes', t2np(yr), y.reshape(-1, D))):
        fb = frac_beyond(got, want, TOL['mxfp8'], True)
        print(f'  mx {name}: share beyond tau*RMS without allowance = {fb:.2e}', flush=True)
        assert fb < MAX_FRAC_BEYOND, (name, fb)


@pytest.mark.parametrize('flags', [0, 0x100000], ids=['gather', 'dispatch_copy'])
@pytest.mark.parametrize('chunk,stages', [(256, 3), (512, 4), (768, 5), (1 << 20, 3)])
def test_mx_chunked_ring_bitwise_equals_unchunked(m, chunk, stages, flags):
    """The MXFP8 forward through the chunked ring (the up/gate GEMM reads the token rows quantised
    once through the schedule, h goes through ring stage c mod S; with MOE_FLAG_DISPATCH_COPY each
    chunk's rows are quantised into its ring stage first) gives the unchunked path's bits."""
    H, q = mx_layer(MX_SMALL)
    a, ya, *_ = run_mx_forward(m, H, q)
    b, yb, _, p, _ = run_mx_forward(m, H, q, chunk_rows=chunk, ring_stages=stages, flags=flags)
    assert torch.equal(a, b) and torch.equal(ya, yb)


def test_mx_gather_matches_dispatch_copy_bitwise(m):
    """The default MXFP8 forward quantises the T token rows once and the block-scaled up/gate GEMM
    reads codes and scales through the schedule; MOE_FLAG_DISPATCH_COPY quantises per-slot copies
    first (the same codes: a slot's row is its token's row). Same bits, also with a, u kept
    (moe_forward_keep); MOE_FLAG_FUSED_GATHER names the default."""
    H, q = mx_layer(MX_SMALL)
    cfg = H.cfg
    n = cfg.T * cfg.K
    runs = {}
    for name, flags in (('gather', 0), ('copy', m.MOE_FLAG_DISPATCH_COPY), ('named', m.MOE_FLAG_FUSED_GATHER)):
        runs[name] = run_mx_forward(m, H, q, flags=flags)
    for name in ('copy', 'named'):
        assert torch.equal(runs['gather'][0], runs[name][0]) and torch.equal(runs['gather'][1], runs[name][1]), name
    kept = []
    for flags in (0, m.MOE_FLAG_DISPATCH_COPY):
        act = [torch.full((n, cfg.I), float('nan'), device='cuda') for _ in range(2)]
        out, yr, *_ = run_mx_forward(m, H, q, act, flags=flags)
        kept.append((out, yr, act))
    assert torch.equal(kept[0][0], runs['gather'][0]) and torch.equal(kept[1][0], runs['gather'][0])
    for u, v in zip(kept[0][2], kept[1][2]):
        assert torch.equal(u, v)


def test_mx_forward_deterministic(m):
    H, q = mx_layer(MX_SMALL)
    a, *_ = run_mx_forward(m, H, q)
    b, *_ = run_mx_forward(m, H, q)
    assert torch.equal(a, b)


@pytest.mark.slow
def test_mx_forward_full_size_sampled(m):
    """MXFP8 at T=32768, D=7168, I=2048, E=256, K=8 (Zipf expert popularity): weights quantised on
    the device, 64 sampled tokens (all routed to expert 0, their experts drawn from a small popular
    set) checked against the oracle on its own quantisation of the same weights (the device
    quantiser is checked bit-exact on those experts first)."""
    cfg = synth.MXFP8
    print('[mxfp8] generating full-size inputs', flush=True)
    L = synth.device_layer(cfg)
    E, I, D, T, K = cfg.E, cfg.I, cfg.D, cfg.T, cfg.K
    wq = {k: torch.empty(getattr(L, k).shape, dtype=torch.uint8, device='cuda') for k in ('w_gate', 'w_up', 'w_down')}
    ws = {k: torch.empty(getattr(L, k).shape[:-1] + (getattr(L, k).shape[-1] // 32,), dtype=torch.uint8, device='cuda')
          for k in ('w_gate', 'w_up', 'w_down')}
    for k in wq:
        m.quantize_mx(getattr(L, k), wq[k], ws[k])
    p = m.problem(T, D, I, E, K, cfg.I_shared, 'mxfp8')
    W = m.make_weights(wq['w_gate'], wq['w_up'], wq['w_down'], L.ws_gate, L.ws_up, L.ws_down,
                       ws['w_gate'], ws['w_up'], ws['w_down'])
    rt = [torch.empty((T, K), dtype=torch.int32, device='cuda'), torch.empty((T, K), dtype=torch.float32, device='cuda'),
          torch.empty((E,), dtype=torch.int32, device='cuda'), torch.empty((E + 1,), dtype=torch.int32, device='cuda'),
          torch.empty((T * K,), dtype=torch.int32, device='cuda'), torch.empty((T * K,), dtype=torch.int32, device='cuda')]
    out = torch.empty((T, D), dtype=torch.bfloat16, device='cuda')
    wsp = torch.empty((m.workspace_size(p),), dtype=torch.uint8, device='cuda')
    m.forward(p, L.x, L.logits, W, out, m.make_routing(*rt), wsp)
    torch.cuda.synchronize()
    lg = L.logits.cpu().numpy()
    idx = oracle.route_topk(lg, K)
    assert np.array_equal(rt[0].cpu().numpy(), idx)
    toks = pick_tokens_few_experts(idx, 64)
    used = sorted(set(idx[toks].ravel().tolist()))
    assert 0 in used
    print(f'[mxfp8] oracle on {len(toks)} tokens, {len(used)} experts', flush=True)
    deq = {k: {} for k in ('w_gate', 'w_up', 'w_down')}

    def quantize_expert(ke):
        k, e = ke
        rq, rs = oracle.mx_quantize(getattr(L, k)[e].float().cpu().numpy().astype(np.float64))
        same = np.array_equal(wq[k][e].cpu().numpy(), rq) and np.array_equal(ws[k][e].cpu().numpy(), rs)
        return k, e, same, oracle.mx_dequantize(rq, rs)

    # the oracle's own quantisation of every weight it uses (numpy releases the GIL in its array
    # operations, so a few host threads share the work); the device codes must match bit for bit
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(8) as pool:
        for k, e, same, d in pool.map(quantize_expert, [(k, e) for k in deq for e in used]):
            assert same, (k, e)
            deq[k][e] = d
    x = L.x[torch.from_numpy(toks).cuda()].float().cpu().numpy().astype(np.float64)
    ref, _, _, _, oa = oracle_mx_forward(x, lg[toks], {k: (lambda e, k=k: deq[k][e]) for k in deq}, K,
                                         L.ws_gate.float().cpu().numpy(), L.ws_up.float().cpu().numpy(),
                                         L.ws_down.float().cpu().numpy())
    got = out[torch.from_numpy(toks).cuda()].float().cpu().numpy()
    assert_close_rms(got, ref, TOL['mxfp8'], 'mx full sampled', True, oa)
    fb = frac_beyond(got, ref, TOL['mxfp8'], True)
    print(f'  mx full sampled: share beyond tau*RMS without allowance = {fb:.2e}', flush=True)
    assert fb < MAX_FRAC_BEYOND, fb


def pick_tokens_few_experts(idx, n):
    """n tokens whose K experts all lie among the M most popular ones (expert ids 0 .. M-1 under
    the Zipf routing), with the smallest M that offers n such tokens that route to expert 0; the
    host oracle's cost grows with the number of distinct experts it has to quantise."""
    top = idx.max(axis=1)
    has0 = (idx == 0).any(axis=1)
    for M in range(idx.shape[1], idx.max() + 2):
        cand = np.nonzero((top < M) & has0)[0]
        if cand.size >= n:
            return np.sort(cand[:n])
    raise AssertionError('routing offers too few tokens')
