"""GPU parity of the expert-level forward/backward (one expert-parallel rank's share) and of the
whole-layer backward against the fp64 oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL, ForwardRun, assert_close_rms, t2np

pytestmark = pytest.mark.gpu
TAU = TOL['bf16']


@pytest.fixture(scope='module')
def m():
    import mixture_experts_layer_norm_amd as mod
    return mod


def bf(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(torch.bfloat16)


def share_inputs(cfg, counts):
    """Seeded share inputs with given per-expert slot counts (sum <= tokens * K)."""
    S = int(sum(counts))
    base = synth.host_share(dataclasses.replace(cfg))
    return base, S


SMALL_SHARE = synth.EPShareConfig('small_share_bf16_T100_K5_D256_I256_E3', tokens=100, D=256, I=256, E_local=3, K=5,
                                  I_shared=128, zipf_s=1.2, seed=41)


def run_share(m, H, counts, flags=0, keep=False, keep_shared=True):
    cfg = H.cfg
    S = int(sum(counts))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    p = m.problem(cfg.tokens, cfg.D, cfg.I, cfg.E_local, cfg.K, cfg.I_shared, 'bf16', flags=flags)
    W = m.make_weights(*(bf(a) for a in (H.w_gate, H.w_up, H.w_down, H.ws_gate, H.ws_up, H.ws_down)))
    keep = [W]
    dev = {k: bf(getattr(H, k)[:S] if k in ('x_slot', 'dy_slot') else getattr(H, k))
           for k in ('x_slot', 'dy_slot', 'x_local', 'dy_local', 'w_gate', 'w_up', 'w_down', 'ws_gate', 'ws_up',
                     'ws_down')}
    W = m.make_weights(dev['w_gate'], dev['w_up'], dev['w_down'], dev['ws_gate'], dev['ws_up'], dev['ws_down'])
    off_d = torch.from_numpy(offsets).cuda()
    g_d = torch.from_numpy(H.g[:S].copy()).cuda()
    y = torch.empty((S, cfg.D), dtype=torch.bfloat16, device='cuda')
    sh = torch.empty((cfg.tokens, cfg.D), dtype=torch.bfloat16, device='cuda')
    ws = torch.zeros((m.workspace_size(p),), dtype=torch.uint8, device='cuda')
    E, I, D, Is = cfg.E_local, cfg.I, cfg.D, cfg.I_shared
    if keep:
        act = [torch.full((S, I), float('nan'), device='cuda') for _ in range(2)]
        act += [torch.full((cfg.tokens, Is), float('nan'), device='cuda') if keep_shared else None for _ in range(2)]
        m.experts_forward_keep(p, S, dev['x_slot'], off_d, W, y, dev['x_local'], sh, *act, ws)
    else:
        m.experts_forward(p, S, dev['x_slot'], off_d, W, y, dev['x_local'], sh, ws)
    dxs = torch.empty((S, D), dtype=torch.bfloat16, device='cuda')
    dg = torch.empty((S,), dtype=torch.float32, device='cuda')
    gr = dict(dw_gate=torch.empty((E, I, D), device='cuda'), dw_up=torch.empty((E, I, D), device='cuda'),
              dw_down=torch.empty((E, D, I), device='cuda'), dws_gate=torch.empty((Is, D), device='cuda'),
              dws_up=torch.empty((Is, D), device='cuda'), dws_down=torch.empty((D, Is), device='cuda'))
    G = m.make_grads(**gr)
    dxl = torch.empty((cfg.tokens, D), dtype=torch.bfloat16, device='cuda')
    # the kept backward runs in exactly the smaller workspace that leaves out the replay's a, u
    wsb = torch.zeros(((m.backward_kept_workspace_size if keep else m.backward_workspace_size)(p),),
                      dtype=torch.uint8, device='cuda')
    if keep:
        m.experts_backward_kept(p, S, dev['x_slot'], off_d, g_d, dev['dy_slot'], W, dxs, dg, G, dev['x_local'],
                                dev['dy_local'], dxl, *act, wsb)
    else:
        m.experts_backward(p, S, dev['x_slot'], off_d, g_d, dev['dy_slot'], W, dxs, dg, G, dev['x_local'],
                           dev['dy_local'], dxl, wsb)
    torch.cuda.synchronize()
    err = int(wsb[:4].view(torch.int32).item())
    return dict(y=y, sh=sh, dx_slot=dxs, dg=dg, dx_local=dxl, err=err, **gr)


# Groups of 4096+ slots on average: with MOE_FLAG_BWD_WGRAD_LO_MXFP8 the weight gradients'
# low-half pass runs in MXFP8 (routed and shared expert), as it does on the full-size share.
LONG_SHARE = synth.EPShareConfig('long_share_bf16_T4096_K3_D256_I256_E3', tokens=4096, D=256, I=256, E_local=3, K=3,
                                 I_shared=128, zipf_s=1.2, seed=43)


@pytest.mark.parametrize('counts', [[300, 0, 157], [1, 257, 242], [0, 0, 500]], ids=['empty_mid', 'ragged', 'one_hot'])
def test_experts_forward_backward_small(m, counts):
    check_share(m, SMALL_SHARE, counts)


@pytest.mark.parametrize('lo_mx', [False, True], ids=['bf16', 'lo_mxfp8'])
@pytest.mark.parametrize('counts', [[6000, 0, 4321], [1, 7003, 5284]], ids=['empty_mid', 'ragged'])
def test_experts_forward_backward_long_groups(m, counts, lo_mx):
    check_share(m, LONG_SHARE, counts, m.MOE_FLAG_BWD_WGRAD_LO_MXFP8 if lo_mx else 0)


@pytest.mark.parametrize('keep_shared', [True, False], ids=['shared_kept', 'shared_replayed'])
@pytest.mark.parametrize('flags', [0, 0x40], ids=['default', 'one_pass'])
@pytest.mark.parametrize('counts', [[300, 0, 157], [1, 257, 242], [0, 0, 500]], ids=['empty_mid', 'ragged', 'one_hot'])
def test_experts_keep_activations_bitwise(m, counts, flags, keep_shared):
    """moe_experts_forward_keep + moe_experts_backward_kept: a, u handed from the forward to the
    backward instead of replayed (routed, and the shared expert's too or not); every output
    bitwise that of the replaying pair."""
    H = synth.host_share(SMALL_SHARE)
    a = run_share(m, H, counts, flags, keep=True, keep_shared=keep_shared)
    b = run_share(m, H, counts, flags)
    assert a['err'] == 0
    for k in ('y', 'sh', 'dx_slot', 'dg', 'dw_gate', 'dw_up', 'dw_down', 'dws_gate', 'dws_up', 'dws_down', 'dx_local'):
        assert torch.equal(a[k], b[k]), k


def test_wgrad_lo_mxfp8_short_groups_unchanged(m):
    """On groups shorter than 4096 rows on average the flag leaves every output bitwise unchanged."""
    H = synth.host_share(SMALL_SHARE)
    a = run_share(m, H, [300, 0, 157], flags=m.MOE_FLAG_BWD_WGRAD_LO_MXFP8)
    b = run_share(m, H, [300, 0, 157])
    for k in ('dx_slot', 'dg', 'dw_gate', 'dw_up', 'dw_down', 'dws_gate', 'dws_up', 'dws_down', 'dx_local'):
        assert torch.equal(a[k], b[k]), k


def check_share(m, cfg, counts, flags=0):
    print(f'[backward] share {cfg.name} counts={counts} flags={flags:#x}', flush=True)
    H = synth.host_share(cfg)
    S = int(sum(counts))
    r = run_share(m, H, counts, flags)
    assert r['err'] == 0
    c = np.array(counts)
    y = oracle.experts_forward(H.x_slot[:S], c, H.w_gate, H.w_up, H.w_down)
    assert_close_rms(t2np(r['y']), y, TAU, 'y_slot', True)
    sh = oracle.swiglu_expert(H.x_local, H.ws_gate, H.ws_up, H.ws_down)
    assert_close_rms(t2np(r['sh']), sh, TAU, 'shared_out', True)
    ref = oracle.experts_backward(H.x_slot[:S], c, H.g[:S], H.dy_slot[:S], H.w_gate, H.w_up, H.w_down)
    assert_close_rms(t2np(r['dx_slot']), ref['dx_slot'], TAU, 'dx_slot', True)
    assert_close_rms(t2np(r['dg']), ref['dg'], TAU, 'dg')
    for k in ('dW_gate', 'dW_up', 'dW_down'):
        got = t2np(r[k.replace('dW', 'dw')])
        assert_close_rms(got, ref[k], TAU, k)
        for e in range(len(counts)):
            if counts[e] == 0:
                assert np.all(got[e] == 0), f'{k}[{e}] of an empty expert must be exact zeros'
    rs = oracle.shared_backward(H.x_local, H.dy_local, H.ws_gate, H.ws_up, H.ws_down)
    assert_close_rms(t2np(r['dx_local']), rs['dx'], TAU, 'dx_local', True)
    for k in ('dW_gate', 'dW_up', 'dW_down'):
        assert_close_rms(t2np(r[k.replace('dW', 'dws')]), rs[k], TAU, 'shared ' + k)


def test_experts_backward_deterministic(m):
    H = synth.host_share(SMALL_SHARE)
    a = run_share(m, H, [300, 0, 157])
    b = run_share(m, H, [300, 0, 157])
    for k in ('dx_slot', 'dg', 'dw_gate', 'dw_up', 'dw_down', 'dws_down', 'dx_local'):
        assert torch.equal(a[k], b[k]), k


LAYER_BWD = synth.scaled(synth.DSV3, 'layer_bwd_bf16_T300_D256_I256_E16_K4', T=300, D=256, I=256, E=16, K=4,
                         I_shared=128)


# Three experts over 6144 tokens x 2 routes: groups long enough for MOE_FLAG_BWD_WGRAD_LO_MXFP8
# (routed and shared expert) on the whole-layer backward.
LAYER_LONG = synth.scaled(LAYER_BWD, 'layer_bwd_long_T6144_E3_K2', T=6144, E=3, K=2)


@pytest.mark.parametrize('cfg,flags', [(LAYER_BWD, 0), (synth.scaled(LAYER_BWD, 'layer_bwd_noshared', I_shared=0, T=130,
                                                                     K=2), 0), (LAYER_LONG, 0x80)],
                         ids=['layer_bwd', 'noshared', 'long_lo_mxfp8'])
def test_layer_backward(m, cfg, flags):
    print(f'[backward] layer {cfg.name} flags={flags:#x}', flush=True)
    H = synth.host_layer(cfg)
    L = synth.to_device(H)
    run = ForwardRun(m, L, flags=flags, want_parts=False)()
    dout_h = synth.host_dout(cfg, cfg.T)
    dout = bf(dout_h)
    E, I, D, Is, T, K = cfg.E, cfg.I, cfg.D, cfg.I_shared, cfg.T, cfg.K
    gr = dict(dw_gate=torch.empty((E, I, D), device='cuda'), dw_up=torch.empty((E, I, D), device='cuda'),
              dw_down=torch.empty((E, D, I), device='cuda'))
    if Is:
        gr.update(dws_gate=torch.empty((Is, D), device='cuda'), dws_up=torch.empty((Is, D), device='cuda'),
                  dws_down=torch.empty((D, Is), device='cuda'))
    G = m.make_grads(**gr)
    dx = torch.empty((T, D), dtype=torch.bfloat16, device='cuda')
    dtw = torch.empty((T, K), dtype=torch.float32, device='cuda')
    dlg = torch.empty((T, E), dtype=torch.float32, device='cuda')
    wsb = torch.zeros((m.backward_workspace_size(run.p),), dtype=torch.uint8, device='cuda')
    m.backward(run.p, dout, L.x, L.logits, run.weights, run.routing, dx, G, dtw, dlg, wsb)
    torch.cuda.synchronize()
    ref = oracle.moe_backward(H.x, H.logits, H.w_gate, H.w_up, H.w_down, K, dout_h, H.ws_gate, H.ws_up, H.ws_down)
    assert_close_rms(t2np(dx), ref['dx'], TAU, 'dx', True)
    assert_close_rms(t2np(dtw), ref['dg'], TAU, 'd_topk_w')
    assert_close_rms(t2np(dlg), ref['d_logits'], TAU, 'd_logits')
    for k in ('dW_gate', 'dW_up', 'dW_down'):
        assert_close_rms(t2np(gr[k.replace('dW', 'dw')]), ref[k], TAU, k)
    if Is:
        for k in ('dWs_gate', 'dWs_up', 'dWs_down'):
            assert_close_rms(t2np(gr[k.replace('dWs', 'dws')]), ref[k], TAU, k)
    # off the selected experts d_logits is exactly zero
    mask = np.zeros((T, E), dtype=bool)
    np.put_along_axis(mask, ref['idx'].astype(np.int64), True, axis=1)
    assert np.all(t2np(dlg)[~mask] == 0)


def run_share_device(m, D_):
    """experts_forward + experts_backward on device-generated share inputs (full size)."""
    cfg = D_.cfg
    S, E, I, D, Is = cfg.slots, cfg.E_local, cfg.I, cfg.D, cfg.I_shared
    offsets = torch.from_numpy(np.concatenate([[0], np.cumsum(D_.counts)]).astype(np.int32)).cuda()
    p = m.problem(cfg.tokens, D, I, E, cfg.K, Is, 'bf16')
    W = m.make_weights(D_.w_gate, D_.w_up, D_.w_down, D_.ws_gate, D_.ws_up, D_.ws_down)
    y = torch.empty((S, D), dtype=torch.bfloat16, device='cuda')
    sh = torch.empty((cfg.tokens, D), dtype=torch.bfloat16, device='cuda')
    ws = torch.zeros((m.workspace_size(p),), dtype=torch.uint8, device='cuda')
    m.experts_forward(p, S, D_.x_slot, offsets, W, y, D_.x_local, sh, ws)
    dxs = torch.empty((S, D), dtype=torch.bfloat16, device='cuda')
    dg = torch.empty((S,), dtype=torch.float32, device='cuda')
    gr = dict(dw_gate=torch.empty((E, I, D), device='cuda'), dw_up=torch.empty((E, I, D), device='cuda'),
              dw_down=torch.empty((E, D, I), device='cuda'), dws_gate=torch.empty((Is, D), device='cuda'),
              dws_up=torch.empty((Is, D), device='cuda'), dws_down=torch.empty((D, Is), device='cuda'))
    G = m.make_grads(**gr)
    dxl = torch.empty((cfg.tokens, D), dtype=torch.bfloat16, device='cuda')
    wsb = torch.zeros((m.backward_workspace_size(p),), dtype=torch.uint8, device='cuda')
    m.experts_backward(p, S, D_.x_slot, offsets, D_.g, D_.dy_slot, W, dxs, dg, G, D_.x_local, D_.dy_local, dxl, wsb)
    torch.cuda.synchronize()
    return dict(y=y, sh=sh, dx_slot=dxs, dg=dg, dx_local=dxl, err=int(wsb[:4].view(torch.int32).item()), **gr)


def h64(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.slow
def test_ep_share_full_size_sampled(m):
    """One EP=64 rank's share at the DSV3 shape (4 local experts, Zipf(1.2) loads over 57,344
    slots, shared expert on 7,168 tokens), forward + backward on the device. Checked against the
    oracle on samples it can afford: whole slots (y, dx, dg depend on their own slot only), whole
    shared-expert rows, and single intermediate units i, for which the expert restricted to unit i
    (rows i of W_gate, W_up and column i of W_down) gives exactly row i of dW_gate, dW_up and
    column i of dW_down over all of the expert's slots."""
    cfg = synth.EP_SHARE
    print('[ep_share] generating full-size share inputs', flush=True)
    D_ = synth.device_share(cfg)
    r = run_share_device(m, D_)
    assert r['err'] == 0
    off = np.concatenate([[0], np.cumsum(D_.counts)])
    rng = np.random.default_rng(7)
    # whole slots, 16 per expert: its first and last slot and 14 drawn at random
    slots = np.concatenate([np.unique(np.concatenate([[off[e], off[e + 1] - 1],
                                                      rng.choice(np.arange(off[e] + 1, off[e + 1] - 1), 14,
                                                                 replace=False)]))
                            for e in range(cfg.E_local)])
    cnt = np.full(cfg.E_local, 16)
    assert slots.size == 16 * cfg.E_local
    idx = torch.from_numpy(slots).cuda()
    xs, dys, gs = h64(D_.x_slot[idx]), h64(D_.dy_slot[idx]), D_.g[idx].cpu().numpy().astype(np.float64)
    wg, wu, wd = h64(D_.w_gate), h64(D_.w_up), h64(D_.w_down)
    print('[ep_share] oracle on sampled slots', flush=True)
    y = oracle.experts_forward(xs, cnt, wg, wu, wd)
    assert_close_rms(h64(r['y'][idx]), y, TAU, 'ep y_slot sampled', True)
    ref = oracle.experts_backward(xs, cnt, gs, dys, wg, wu, wd)
    assert_close_rms(h64(r['dx_slot'][idx]), ref['dx_slot'], TAU, 'ep dx_slot sampled', True)
    assert_close_rms(r['dg'][idx].cpu().numpy(), ref['dg'], TAU, 'ep dg sampled')
    # single units i of every expert, over all its slots: units at both edges of the first and
    # last 128-column tile of h and four drawn at random
    for e in range(cfg.E_local):
        a, b = int(off[e]), int(off[e + 1])
        X, DY = h64(D_.x_slot[a:b]), h64(D_.dy_slot[a:b])
        G = D_.g[a:b].cpu().numpy().astype(np.float64)
        for i in np.concatenate([[0, 127, 128, cfg.I - 1], rng.choice(np.arange(129, cfg.I - 1), 4, replace=False)]):
            print(f'[ep_share] oracle on expert {e} unit {i} ({b - a} slots)', flush=True)
            ru = oracle.experts_backward(X, np.array([b - a]), G, DY, wg[e:e + 1, i:i + 1], wu[e:e + 1, i:i + 1],
                                         wd[e:e + 1, :, i:i + 1])
            assert_close_rms(r['dw_gate'][e, i].cpu().numpy(), ru['dW_gate'][0, 0], TAU, f'ep dW_gate[{e},{i}]')
            assert_close_rms(r['dw_up'][e, i].cpu().numpy(), ru['dW_up'][0, 0], TAU, f'ep dW_up[{e},{i}]')
            assert_close_rms(r['dw_down'][e, :, i].cpu().numpy(), ru['dW_down'][0, :, 0], TAU, f'ep dW_down[{e},:,{i}]')
    # shared expert: sampled rows of its output and input gradient, sampled units of its weight gradients
    rows = np.sort(rng.choice(cfg.tokens, 4, replace=False))
    ridx = torch.from_numpy(rows).cuda()
    sg, su, sd = h64(D_.ws_gate), h64(D_.ws_up), h64(D_.ws_down)
    xl, dyl = h64(D_.x_local), h64(D_.dy_local)
    assert_close_rms(h64(r['sh'][ridx]), oracle.swiglu_expert(xl[rows], sg, su, sd), TAU, 'ep shared_out sampled',
                     True)
    rs = oracle.shared_backward(xl[rows], dyl[rows], sg, su, sd)
    assert_close_rms(h64(r['dx_local'][ridx]), rs['dx'], TAU, 'ep shared dx sampled', True)
    for i in rng.choice(cfg.I_shared, 2, replace=False):
        ru = oracle.shared_backward(xl, dyl, sg[i:i + 1], su[i:i + 1], sd[:, i:i + 1])
        assert_close_rms(r['dws_gate'][i].cpu().numpy(), ru['dW_gate'][0], TAU, f'ep shared dW_gate[{i}]')
        assert_close_rms(r['dws_up'][i].cpu().numpy(), ru['dW_up'][0], TAU, f'ep shared dW_up[{i}]')
        assert_close_rms(r['dws_down'][:, i].cpu().numpy(), ru['dW_down'][:, 0], TAU, f'ep shared dW_down[:,{i}]')


def test_layer_backward_f32_tiny(m):
    """Whole-layer backward on the tiny fp32 configuration (T=256, D=128, I=64, 8 experts top-2 +
    shared): every gradient within 1e-4 RMS of the fp64 oracle, zero d_logits off the selection."""
    cfg = synth.TINY
    print(f'[backward] layer {cfg.name}', flush=True)
    H = synth.host_layer(cfg)
    L = synth.to_device(H)
    run = ForwardRun(m, L, want_parts=False)()
    dout_h = synth.host_dout(cfg, cfg.T)
    dout = torch.from_numpy(np.ascontiguousarray(dout_h, dtype=np.float32)).cuda()
    E, I, D, Is, T, K = cfg.E, cfg.I, cfg.D, cfg.I_shared, cfg.T, cfg.K
    gr = dict(dw_gate=torch.full((E, I, D), float('nan'), device='cuda'),
              dw_up=torch.full((E, I, D), float('nan'), device='cuda'),
              dw_down=torch.full((E, D, I), float('nan'), device='cuda'), dws_gate=torch.empty((Is, D), device='cuda'),
              dws_up=torch.empty((Is, D), device='cuda'), dws_down=torch.empty((D, Is), device='cuda'))
    dx = torch.empty((T, D), dtype=torch.float32, device='cuda')
    dtw = torch.empty((T, K), dtype=torch.float32, device='cuda')
    dlg = torch.empty((T, E), dtype=torch.float32, device='cuda')
    wsb = torch.zeros((m.backward_workspace_size(run.p),), dtype=torch.uint8, device='cuda')
    m.backward(run.p, dout, L.x, L.logits, run.weights, run.routing, dx, m.make_grads(**gr), dtw, dlg, wsb)
    torch.cuda.synchronize()
    assert int(wsb[:4].view(torch.int32).item()) == 0
    tau = TOL['f32']
    ref = oracle.moe_backward(H.x, H.logits, H.w_gate, H.w_up, H.w_down, K, dout_h, H.ws_gate, H.ws_up, H.ws_down)
    assert_close_rms(t2np(dx), ref['dx'], tau, 'f32 dx')
    assert_close_rms(t2np(dtw), ref['dg'], tau, 'f32 d_topk_w')
    assert_close_rms(t2np(dlg), ref['d_logits'], tau, 'f32 d_logits')
    for k in ('dW_gate', 'dW_up', 'dW_down'):
        assert_close_rms(t2np(gr[k.replace('dW', 'dw')]), ref[k], tau, 'f32 ' + k)
    for k in ('dWs_gate', 'dWs_up', 'dWs_down'):
        assert_close_rms(t2np(gr[k.replace('dWs', 'dws')]), ref[k], tau, 'f32 ' + k)
    mask = np.zeros((T, E), dtype=bool)
    np.put_along_axis(mask, ref['idx'].astype(np.int64), True, axis=1)
    assert np.all(t2np(dlg)[~mask] == 0)


@pytest.mark.parametrize('counts', [[300, 0, 157], [1, 257, 242]], ids=['empty_mid', 'ragged'])
def test_experts_forward_backward_f32(m, counts):
    """Expert-level forward + backward in fp32 on the small share (1e-4 RMS against fp64),
    exact zeros for an empty expert's weight gradients, bitwise repeatable."""
    H = synth.host_share(SMALL_SHARE)
    cfg = H.cfg
    S = int(sum(counts))
    E, I, D, Is = cfg.E_local, cfg.I, cfg.D, cfg.I_shared
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    p = m.problem(cfg.tokens, D, I, E, cfg.K, Is, 'f32')
    wts = [f(getattr(H, k)) for k in ('w_gate', 'w_up', 'w_down', 'ws_gate', 'ws_up', 'ws_down')]
    W = m.make_weights(*wts)   # the binding keeps raw pointers: wts must outlive every call
    off_d = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).cuda()
    xs, dys, xl, dyl = f(H.x_slot[:S]), f(H.dy_slot[:S]), f(H.x_local), f(H.dy_local)
    g_d = torch.from_numpy(H.g[:S].copy()).cuda()

    def run():
        y = torch.empty((S, D), device='cuda')
        sh = torch.empty((cfg.tokens, D), device='cuda')
        ws = torch.zeros((m.workspace_size(p),), dtype=torch.uint8, device='cuda')
        m.experts_forward(p, S, xs, off_d, W, y, xl, sh, ws)
        dxs = torch.empty((S, D), device='cuda')
        dg = torch.empty((S,), device='cuda')
        gr = dict(dw_gate=torch.full((E, I, D), float('nan'), device='cuda'),
                  dw_up=torch.full((E, I, D), float('nan'), device='cuda'),
                  dw_down=torch.full((E, D, I), float('nan'), device='cuda'),
                  dws_gate=torch.empty((Is, D), device='cuda'), dws_up=torch.empty((Is, D), device='cuda'),
                  dws_down=torch.empty((D, Is), device='cuda'))
        dxl = torch.empty((cfg.tokens, D), device='cuda')
        wsb = torch.zeros((m.backward_workspace_size(p),), dtype=torch.uint8, device='cuda')
        m.experts_backward(p, S, xs, off_d, g_d, dys, W, dxs, dg, m.make_grads(**gr), xl, dyl, dxl, wsb)
        torch.cuda.synchronize()
        assert int(wsb[:4].view(torch.int32).item()) == 0
        return dict(y=y, sh=sh, dx_slot=dxs, dg=dg, dx_local=dxl, **gr)

    print(f'[backward] f32 share counts={counts}', flush=True)
    r = run()
    tau = TOL['f32']
    c = np.array(counts)
    assert_close_rms(t2np(r['y']), oracle.experts_forward(H.x_slot[:S], c, H.w_gate, H.w_up, H.w_down), tau, 'f32 y')
    assert_close_rms(t2np(r['sh']), oracle.swiglu_expert(H.x_local, H.ws_gate, H.ws_up, H.ws_down), tau, 'f32 sh')
    ref = oracle.experts_backward(H.x_slot[:S], c, H.g[:S], H.dy_slot[:S], H.w_gate, H.w_up, H.w_down)
    assert_close_rms(t2np(r['dx_slot']), ref['dx_slot'], tau, 'f32 dx_slot')
    assert_close_rms(t2np(r['dg']), ref['dg'], tau, 'f32 dg')
    for k in ('dW_gate', 'dW_up', 'dW_down'):
        got = t2np(r[k.replace('dW', 'dw')])
        assert_close_rms(got, ref[k], tau, 'f32 ' + k)
        for e in range(len(counts)):
            if counts[e] == 0:
                assert np.all(got[e] == 0), f'{k}[{e}] of an empty expert must be exact zeros'
    rs = oracle.shared_backward(H.x_local, H.dy_local, H.ws_gate, H.ws_up, H.ws_down)
    assert_close_rms(t2np(r['dx_local']), rs['dx'], tau, 'f32 shared dx')
    for k in ('dW_gate', 'dW_up', 'dW_down'):
        assert_close_rms(t2np(r[k.replace('dW', 'dws')]), rs[k], tau, 'f32 shared ' + k)
    r2 = run()
    for k in ('dx_slot', 'dg', 'dw_gate', 'dw_up', 'dw_down', 'dx_local'):
        assert torch.equal(r[k], r2[k]), k


@pytest.mark.parametrize('counts', [[300, 0, 157], [1, 257, 242]], ids=['empty_mid', 'ragged'])
def test_experts_backward_dgrad_one_pass(m, counts):
    """MOE_FLAG_BWD_DGRAD_ONE_PASS: dgrad-up over the bf16 da, du in one K pass. dx_slot and
    dx_local stay within the BF16 bound; the other outputs are computed as without the flag."""
    print(f'[backward] one-pass dgrad-up, share counts={counts}', flush=True)
    H = synth.host_share(SMALL_SHARE)
    S = int(sum(counts))
    r = run_share(m, H, counts, flags=m.MOE_FLAG_BWD_DGRAD_ONE_PASS)
    assert r['err'] == 0
    c = np.array(counts)
    ref = oracle.experts_backward(H.x_slot[:S], c, H.g[:S], H.dy_slot[:S], H.w_gate, H.w_up, H.w_down)
    assert_close_rms(t2np(r['dx_slot']), ref['dx_slot'], TAU, 'one-pass dx_slot', True)
    rs = oracle.shared_backward(H.x_local, H.dy_local, H.ws_gate, H.ws_up, H.ws_down)
    assert_close_rms(t2np(r['dx_local']), rs['dx'], TAU, 'one-pass dx_local', True)
    base = run_share(m, H, counts)
    for k in ('dg', 'dw_gate', 'dw_up', 'dw_down', 'dws_down'):
        assert torch.equal(r[k], base[k]), k


def layer_fwd_bwd(m, cfg, flags, keep):
    """One layer forward (moe_forward, or moe_forward_keep) and backward (moe_backward, or
    moe_backward_kept) on `cfg`; every output."""
    H = synth.host_layer(cfg)
    L = synth.to_device(H)
    E, I, D, Is, T, K = cfg.E, cfg.I, cfg.D, cfg.I_shared, cfg.T, cfg.K
    dout = bf(synth.host_dout(cfg, T))
    run = ForwardRun(m, L, flags=flags, want_parts=False)
    act = [torch.full((T * K, I), float('nan'), device='cuda') for _ in range(2)]
    if keep:
        m.forward_keep(run.p, L.x, L.logits, run.weights, run.out, run.routing, *act, run.ws)
    else:
        run()
    gr = dict(dw_gate=torch.empty((E, I, D), device='cuda'), dw_up=torch.empty((E, I, D), device='cuda'),
              dw_down=torch.empty((E, D, I), device='cuda'), dws_gate=torch.empty((Is, D), device='cuda'),
              dws_up=torch.empty((Is, D), device='cuda'), dws_down=torch.empty((D, Is), device='cuda'))
    G = m.make_grads(**gr)
    dx = torch.empty((T, D), dtype=torch.bfloat16, device='cuda')
    dtw = torch.empty((T, K), dtype=torch.float32, device='cuda')
    dlg = torch.empty((T, E), dtype=torch.float32, device='cuda')
    wsb = torch.zeros(((m.backward_kept_workspace_size if keep else m.backward_workspace_size)(run.p),),
                      dtype=torch.uint8, device='cuda')
    if keep:
        m.backward_kept(run.p, dout, L.x, L.logits, run.weights, run.routing, dx, G, dtw, dlg, *act, wsb)
    else:
        m.backward(run.p, dout, L.x, L.logits, run.weights, run.routing, dx, G, dtw, dlg, wsb)
    torch.cuda.synchronize()
    return dict(out=run.out.clone(), perm=run.perm.clone(), dx=dx, dtw=dtw, dlg=dlg, **gr), wsb.numel()


@pytest.mark.parametrize('flags', [0, 0x100000, 0x40], ids=['gather', 'dispatch_copy', 'one_pass'])
def test_layer_keep_activations_bitwise(m, flags):
    """moe_forward_keep + moe_backward_kept: the routed a, u handed from the layer forward to the
    layer backward instead of replayed; every output bitwise that of moe_forward + moe_backward."""
    print(f'[backward] layer keep {LAYER_BWD.name} flags={flags:#x}', flush=True)
    res = [layer_fwd_bwd(m, LAYER_BWD, flags, keep)[0] for keep in (False, True)]
    for k in res[0]:
        assert torch.equal(res[0][k], res[1][k]), k


@pytest.mark.parametrize('keep', [False, True], ids=['replay', 'kept'])
@pytest.mark.parametrize('extra', [0, 0x40 | 0x80], ids=['default', 'one_pass_lo_mxfp8'])
def test_layer_gather_equals_dispatch_copy_bitwise(m, keep, extra):
    """The BF16 layer forward and backward read x and dout rows through the schedule (GEMM operand
    loads and the weight gradients' transposes); MOE_FLAG_DISPATCH_COPY makes the slot copies
    first. Same rows in the same order: every output is the same bits, and the gathering
    backward needs no slot buffers."""
    print(f'[backward] layer gather vs copy keep={keep} flags={extra:#x}', flush=True)
    a, wa = layer_fwd_bwd(m, LAYER_BWD, extra, keep)
    b, wb = layer_fwd_bwd(m, LAYER_BWD, extra | 0x100000, keep)
    n = LAYER_BWD.T * LAYER_BWD.K
    assert wb - wa >= 2 * n * LAYER_BWD.D * 2
    for k in a:
        assert torch.equal(a[k], b[k]), k
