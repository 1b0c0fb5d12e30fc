"""GPU parity of the MXFP8 expert-level forward and backward (one expert-parallel rank's share)
against the oracle run in fp64 on the same quantised values (every backward GEMM operand
quantised along its contraction dimension; the shared expert in BF16)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import TOL, assert_close_rms, frac_beyond, mx_choice_allowance, t2np

pytestmark = pytest.mark.gpu
TAU = TOL['mxfp8']


@pytest.fixture(scope='module')
def m():
    import mixture_experts_layer_norm_amd as mod
    return mod


def bf(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(torch.bfloat16)


def u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


SMALL = synth.EPShareConfig('small_share_mxfp8_T100_K5_D256_I256_E3', tokens=100, D=256, I=256, E_local=3, K=5,
                            I_shared=128, zipf_s=1.2, seed=43)


def run_share_mx(m, H, q, counts, dev_w=None, flags=0, keep=False):
    """experts_forward + experts_backward in MXFP8 on host share inputs; q: MX bytes of the weights."""
    cfg = H.cfg
    S = int(sum(counts))
    E, I, D, Is = cfg.E_local, cfg.I, cfg.D, cfg.I_shared
    p = m.problem(cfg.tokens, D, I, E, cfg.K, Is, 'mxfp8', flags=flags)
    dev = dict(x_slot=bf(H.x_slot[:S]), dy_slot=bf(H.dy_slot[:S]), x_local=bf(H.x_local), dy_local=bf(H.dy_local),
               ws=[bf(H.ws_gate), bf(H.ws_up), bf(H.ws_down)],
               wq=[u8(q[k][0]) for k in ('w_gate', 'w_up', 'w_down')],
               sc=[u8(q[k][1]) for k in ('w_gate', 'w_up', 'w_down')])
    W = m.make_weights(*dev['wq'], *dev['ws'], *dev['sc'])
    off_d = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).cuda()
    g_d = torch.from_numpy(H.g[:S].copy()).cuda()
    y = torch.empty((S, D), dtype=torch.bfloat16, device='cuda')
    sh = torch.empty((cfg.tokens, D), dtype=torch.bfloat16, device='cuda')
    ws = torch.zeros((m.workspace_size(p),), dtype=torch.uint8, device='cuda')
    if keep:
        act = [torch.full((S, I), float('nan'), device='cuda') for _ in range(2)]
        act += [torch.full((cfg.tokens, Is), float('nan'), device='cuda') for _ in range(2)]
        m.experts_forward_keep(p, S, dev['x_slot'], off_d, W, y, dev['x_local'], sh, *act, ws)
    else:
        m.experts_forward(p, S, dev['x_slot'], off_d, W, y, dev['x_local'], sh, ws)
    dxs = torch.empty((S, D), dtype=torch.bfloat16, device='cuda')
    dg = torch.empty((S,), dtype=torch.float32, device='cuda')
    gr = dict(dw_gate=torch.full((E, I, D), float('nan'), device='cuda'),
              dw_up=torch.full((E, I, D), float('nan'), device='cuda'),
              dw_down=torch.full((E, D, I), float('nan'), device='cuda'), dws_gate=torch.empty((Is, D), device='cuda'),
              dws_up=torch.empty((Is, D), device='cuda'), dws_down=torch.empty((D, Is), device='cuda'))
    G = m.make_grads(**gr)
    dxl = torch.empty((cfg.tokens, D), dtype=torch.bfloat16, device='cuda')
    wsb = torch.full(((m.backward_kept_workspace_size if keep else m.backward_workspace_size)(p),), 0x7f,
                     dtype=torch.uint8, device='cuda')
    wsb[:4].zero_()
    if keep:
        m.experts_backward_kept(p, S, dev['x_slot'], off_d, g_d, dev['dy_slot'], W, dxs, dg, G, dev['x_local'],
                                dev['dy_local'], dxl, *act, wsb)
    else:
        m.experts_backward(p, S, dev['x_slot'], off_d, g_d, dev['dy_slot'], W, dxs, dg, G, dev['x_local'],
                           dev['dy_local'], dxl, wsb)
    torch.cuda.synchronize()
    err = int(wsb[:4].view(torch.int32).item())
    return dict(y=y, sh=sh, dx_slot=dxs, dg=dg, dx_local=dxl, err=err, **gr)


def y_allowance(x, counts, Wg, Wu, Wd):
    """Per-element allowance on the forward output for equally correct h decisions."""
    off = np.concatenate([[0], np.cumsum(counts)])
    ya = np.zeros_like(x)
    for e in range(len(counts)):
        a, b = off[e], off[e + 1]
        if b > a:
            Xq = oracle.mx_along(x[a:b], 1)
            Hm = oracle.silu(Xq @ Wg[e].T) * (Xq @ Wu[e].T)
            ya[a:b] = mx_choice_allowance(Hm) @ np.abs(Wd[e]).T
    return ya


def allow_along(V, axis):
    """mx_choice_allowance of V [n, m] quantised along `axis` (short last block zero-padded)."""
    V = np.asarray(V, dtype=np.float64)
    Wt = V if axis == 1 else V.T
    n = Wt.shape[1]
    pad = (-n) % 32
    if pad:
        Wt = np.concatenate([Wt, np.zeros((Wt.shape[0], pad))], axis=1)
    a = mx_choice_allowance(Wt)[:, :n]
    return a if axis == 1 else a.T


def backward_allowance(ref, x, counts, Wg, Wu, Wd, units=None, Xn=None):
    """Per-element allowance on dx_slot and the weight gradients for equally correct quantisation
    decisions on the operands the device computes in fp32 (da, du along I for dgrad-up; da, du,
    h and g dy along the slots for the weight gradients). units: restrict to one unit (the unit
    test of the full-size share), ref then being the restricted oracle run."""
    off = np.concatenate([[0], np.cumsum(counts)])
    al = {k: np.zeros_like(ref[k]) for k in ('dx_slot', 'dW_gate', 'dW_up', 'dW_down')}
    mq = oracle.mx_along
    for e, P in ref['parts'].items():
        a, b = off[e], off[e + 1]
        Xa = np.abs(mq(x[a:b], 0)) if Xn is None else np.abs(Xn)
        aA, aU = allow_along(P['dA'], 0), allow_along(P['dU'], 0)
        al['dW_gate'][e] = aA.T @ Xa
        al['dW_up'][e] = aU.T @ Xa
        al['dW_down'][e] = allow_along(P['gdy'], 0).T @ np.abs(mq(P['H'], 0)) + \
            np.abs(mq(P['gdy'], 0)).T @ allow_along(P['H'], 0)
        if units is None:
            al['dx_slot'][a:b] = allow_along(P['dA'], 1) @ np.abs(mq(Wg[e], 0)) + \
                allow_along(P['dU'], 1) @ np.abs(mq(Wu[e], 0))
    return al


@pytest.mark.parametrize('counts', [[300, 0, 157], [1, 257, 242], [0, 0, 500], [129, 128, 127]],
                         ids=['empty_mid', 'ragged_single', 'one_hot', 'around_128'])
def test_mx_experts_forward_backward_small(m, counts):
    print(f'[mx backward] share counts={counts}', flush=True)
    H = synth.host_share(SMALL)
    q = {k: oracle.mx_quantize(getattr(H, k).astype(np.float64)) for k in ('w_gate', 'w_up', 'w_down')}
    S = int(sum(counts))
    r = run_share_mx(m, H, q, counts)
    assert r['err'] == 0
    c = np.array(counts)
    Wg, Wu, Wd = (oracle.mx_dequantize(*q[k]) for k in ('w_gate', 'w_up', 'w_down'))
    xs, dys, gs = H.x_slot[:S].astype(np.float64), H.dy_slot[:S].astype(np.float64), H.g[:S].astype(np.float64)
    y = oracle.experts_forward_mx_w(xs, c, Wg, Wu, Wd)
    assert_close_rms(t2np(r['y']), y, TAU, 'mx y_slot', True, y_allowance(xs, c, Wg, Wu, Wd))
    ref = oracle.experts_backward_mx_w(xs, c, gs, dys, Wg, Wu, Wd, return_parts=True)
    al = backward_allowance(ref, xs, c, Wg, Wu, Wd)
    assert_close_rms(t2np(r['dx_slot']), ref['dx_slot'], TAU, 'mx dx_slot', True, al['dx_slot'])
    assert_close_rms(t2np(r['dg']), ref['dg'], TAU, 'mx dg')
    for k in ('dW_gate', 'dW_up', 'dW_down'):
        got = t2np(r[k.replace('dW', 'dw')])
        assert_close_rms(got, ref[k], TAU, 'mx ' + k, False, al[k])
        for e in range(len(counts)):
            if counts[e] == 0:
                assert np.all(got[e] == 0), f'{k}[{e}] of an empty expert must be exact zeros'
    # without any allowance, only a small share of elements may sit beyond tau * RMS
    fr = {'dx_slot': frac_beyond(t2np(r['dx_slot']), ref['dx_slot'], TAU, True)}
    for k in ('dW_gate', 'dW_up', 'dW_down'):
        fr[k] = frac_beyond(t2np(r[k.replace('dW', 'dw')]), ref[k], TAU)
    print('  share beyond tau*RMS without allowance:', {k: f'{v:.2e}' for k, v in fr.items()}, flush=True)
    assert max(fr.values()) < 0.005, fr
    # the shared expert stays BF16
    rs = oracle.shared_backward(H.x_local, H.dy_local, H.ws_gate, H.ws_up, H.ws_down)
    assert_close_rms(t2np(r['dx_local']), rs['dx'], TOL['bf16'], 'shared dx_local', True)
    for k in ('dW_gate', 'dW_up', 'dW_down'):
        assert_close_rms(t2np(r[k.replace('dW', 'dws')]), rs[k], TOL['bf16'], 'shared ' + k)


def test_mx_experts_backward_deterministic(m):
    H = synth.host_share(SMALL)
    q = {k: oracle.mx_quantize(getattr(H, k).astype(np.float64)) for k in ('w_gate', 'w_up', 'w_down')}
    a = run_share_mx(m, H, q, [300, 0, 157])
    b = run_share_mx(m, H, q, [300, 0, 157])
    for k in ('y', 'dx_slot', 'dg', 'dw_gate', 'dw_up', 'dw_down', 'dws_down', 'dx_local'):
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize('counts', [[300, 0, 157], [1, 257, 242], [129, 128, 127]],
                         ids=['empty_mid', 'ragged_single', 'around_128'])
def test_mx_experts_keep_activations_bitwise(m, counts):
    """moe_experts_forward_keep + moe_experts_backward_kept under MXFP8: a, u from the forward's
    block-scaled GEMM, h quantised from them outside the GEMM; every output bitwise that of the
    fused forward and the replaying backward."""
    H = synth.host_share(SMALL)
    q = {k: oracle.mx_quantize(getattr(H, k).astype(np.float64)) for k in ('w_gate', 'w_up', 'w_down')}
    a = run_share_mx(m, H, q, counts, keep=True)
    b = run_share_mx(m, H, q, counts)
    assert a['err'] == 0
    for k in ('y', 'sh', 'dx_slot', 'dg', 'dw_gate', 'dw_up', 'dw_down', 'dws_gate', 'dws_up', 'dws_down', 'dx_local'):
        assert torch.equal(a[k], b[k]), k


def test_mx_shared_expert_wgrad_lo_mxfp8(m):
    """MOE_FLAG_BWD_WGRAD_LO_MXFP8 under MOE_MXFP8 with 4096 local tokens: the BF16 shared
    expert's weight gradients take their low-half pass in MXFP8 and stay within the BF16 bar; the
    routed experts (short groups here) are bitwise as without the flag."""
    cfg = dataclasses.replace(SMALL, name='share_mxfp8_T4096_K1_D256_I256_E3', tokens=4096, K=1)
    H = synth.host_share(cfg)
    q = {k: oracle.mx_quantize(getattr(H, k).astype(np.float64)) for k in ('w_gate', 'w_up', 'w_down')}
    counts = [300, 0, 157]
    r = run_share_mx(m, H, q, counts, flags=m.MOE_FLAG_BWD_WGRAD_LO_MXFP8)
    base = run_share_mx(m, H, q, counts)
    assert r['err'] == 0
    for k in ('y', 'dx_slot', 'dg', 'dw_gate', 'dw_up', 'dw_down', 'dx_local'):
        assert torch.equal(r[k], base[k]), k
    rs = oracle.shared_backward(H.x_local, H.dy_local, H.ws_gate, H.ws_up, H.ws_down)
    for k in ('dW_gate', 'dW_up', 'dW_down'):
        assert_close_rms(t2np(r[k.replace('dW', 'dws')]), rs[k], TOL['bf16'], 'shared lo-MXFP8 ' + k)


def h64(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.slow
def test_mx_ep_share_full_size_sampled(m):
    """One EP=64 rank's share at the DeepSeek-V3 shape in MXFP8 (4 local experts, Zipf(1.2) loads
    over 57,344 slots): weights quantised on the device and checked bit-exact against the oracle's
    encoder, then whole sampled slots (y, dx_slot, dg) and single intermediate units i of the
    largest and smallest expert (row i of dW_gate / dW_up, column i of dW_down over all the
    expert's slots) against the oracle. The unit checks use the two smaller experts (8,109 and
    5,741 slots, 64 and 45 K slices of the K-grouped GEMM): the oracle's quantisation of a whole
    expert's x along both axes is the slow part of this test on the host."""
    cfg = synth.EP_SHARE
    print('[mx ep_share] generating full-size share inputs', flush=True)
    D_ = synth.device_share(cfg)
    S, E, I, D, Is = cfg.slots, cfg.E_local, cfg.I, cfg.D, cfg.I_shared
    wq = {k: torch.empty(getattr(D_, k).shape, dtype=torch.uint8, device='cuda') for k in ('w_gate', 'w_up', 'w_down')}
    wsc = {k: torch.empty(getattr(D_, k).shape[:-1] + (getattr(D_, k).shape[-1] // 32,), dtype=torch.uint8,
                          device='cuda') for k in ('w_gate', 'w_up', 'w_down')}
    for k in wq:
        m.quantize_mx(getattr(D_, k), wq[k], wsc[k])
    deq = {}
    for k in wq:
        rq, rs = oracle.mx_quantize(h64(getattr(D_, k)))
        assert np.array_equal(wq[k].cpu().numpy(), rq) and np.array_equal(wsc[k].cpu().numpy(), rs), k
        deq[k] = oracle.mx_dequantize(rq, rs)
    offsets = torch.from_numpy(np.concatenate([[0], np.cumsum(D_.counts)]).astype(np.int32)).cuda()
    p = m.problem(cfg.tokens, D, I, E, cfg.K, Is, 'mxfp8')
    W = m.make_weights(wq['w_gate'], wq['w_up'], wq['w_down'], D_.ws_gate, D_.ws_up, D_.ws_down,
                       wsc['w_gate'], wsc['w_up'], wsc['w_down'])
    y = torch.empty((S, D), dtype=torch.bfloat16, device='cuda')
    sh = torch.empty((cfg.tokens, D), dtype=torch.bfloat16, device='cuda')
    ws = torch.zeros((m.workspace_size(p),), dtype=torch.uint8, device='cuda')
    print('[mx ep_share] forward + backward', flush=True)
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
    assert int(wsb[:4].view(torch.int32).item()) == 0
    off = np.concatenate([[0], np.cumsum(D_.counts)])
    rng = np.random.default_rng(9)
    slots = np.concatenate([np.sort(rng.choice(np.arange(off[e], off[e + 1]), 3, replace=False)) for e in range(E)])
    cnt = np.full(E, 3)
    idx = torch.from_numpy(slots).cuda()
    xs, dys, gs = h64(D_.x_slot[idx]), h64(D_.dy_slot[idx]), D_.g[idx].cpu().numpy().astype(np.float64)
    Wg, Wu, Wd = deq['w_gate'], deq['w_up'], deq['w_down']
    print('[mx ep_share] oracle on sampled slots', flush=True)
    yr = oracle.experts_forward_mx_w(xs, cnt, Wg, Wu, Wd)
    assert_close_rms(h64(y[idx]), yr, TAU, 'mx ep y_slot sampled', True, y_allowance(xs, cnt, Wg, Wu, Wd))
    ref = oracle.experts_backward_mx_w(xs, cnt, gs, dys, Wg, Wu, Wd, return_parts=True)
    al = backward_allowance(ref, xs, cnt, Wg, Wu, Wd)
    assert_close_rms(h64(dxs[idx]), ref['dx_slot'], TAU, 'mx ep dx_slot sampled', True, al['dx_slot'])
    assert_close_rms(dg[idx].cpu().numpy(), ref['dg'], TAU, 'mx ep dg sampled')
    for e in (E - 2, E - 1):
        a, b = int(off[e]), int(off[e + 1])
        X, DY = h64(D_.x_slot[a:b]), h64(D_.dy_slot[a:b])
        Ge = D_.g[a:b].cpu().numpy().astype(np.float64)
        Xn = oracle.mx_along(X, 0)
        for i in rng.choice(I, 1, replace=False):
            print(f'[mx ep_share] oracle on expert {e} unit {i} ({b - a} slots)', flush=True)
            ru = oracle.experts_backward_mx_w(X, np.array([b - a]), Ge, DY, Wg[e:e + 1, i:i + 1], Wu[e:e + 1, i:i + 1],
                                              Wd[e:e + 1, :, i:i + 1], return_parts=True)
            au = backward_allowance(ru, X, np.array([b - a]), None, None, None, units=True, Xn=Xn)
            assert_close_rms(gr['dw_gate'][e, i].cpu().numpy(), ru['dW_gate'][0, 0], TAU, f'mx ep dW_gate[{e},{i}]',
                             False, au['dW_gate'][0, 0])
            assert_close_rms(gr['dw_up'][e, i].cpu().numpy(), ru['dW_up'][0, 0], TAU, f'mx ep dW_up[{e},{i}]', False,
                             au['dW_up'][0, 0])
            assert_close_rms(gr['dw_down'][e, :, i].cpu().numpy(), ru['dW_down'][0, :, 0], TAU,
                             f'mx ep dW_down[{e},:,{i}]', False, au['dW_down'][0, :, 0])


def test_mx_layer_backward(m):
    """Whole-layer moe_backward in MXFP8 after the MXFP8 forward: the oracle's expert backward on
    the dispatched slots (schedule of the oracle's own routing), reverse-dispatched and summed with
    the BF16 shared expert's input gradient; router gradients from dg."""
    from test_gpu_mxfp8 import MX_SMALL, mx_layer, run_mx_forward
    cfg = MX_SMALL
    print(f'[mx backward] layer {cfg.name}', flush=True)
    H, q = mx_layer(cfg)
    out, yr, rt, p, tensors = run_mx_forward(m, H, q)
    T, K, D, E, I, Is = cfg.T, cfg.K, cfg.D, cfg.E, cfg.I, cfg.I_shared
    dout_h = synth.host_dout(cfg, T)
    W = m.make_weights(*tensors['wq'], *tensors['ws'], *tensors['sc'])
    gr = dict(dw_gate=torch.full((E, I, D), float('nan'), device='cuda'),
              dw_up=torch.full((E, I, D), float('nan'), device='cuda'),
              dw_down=torch.full((E, D, I), float('nan'), device='cuda'), dws_gate=torch.empty((Is, D), device='cuda'),
              dws_up=torch.empty((Is, D), device='cuda'), dws_down=torch.empty((D, Is), device='cuda'))
    dx = torch.empty((T, D), dtype=torch.bfloat16, device='cuda')
    dtw = torch.empty((T, K), dtype=torch.float32, device='cuda')
    dlg = torch.empty((T, E), dtype=torch.float32, device='cuda')
    wsb = torch.zeros((m.backward_workspace_size(p),), dtype=torch.uint8, device='cuda')
    m.backward(p, bf(dout_h), tensors['x'], tensors['logits'], W, m.make_routing(*rt), dx, m.make_grads(**gr), dtw,
               dlg, wsb)
    torch.cuda.synchronize()
    assert int(wsb[:4].view(torch.int32).item()) == 0
    idx = oracle.route_topk(H.logits, K)
    g = oracle.routing_weights(H.logits, idx)
    counts, _, perm, inv = oracle.schedule(idx, E)
    x64, d64 = H.x.astype(np.float64), dout_h.astype(np.float64)
    Wg, Wu, Wd = (oracle.mx_dequantize(*q[k]) for k in ('w_gate', 'w_up', 'w_down'))
    xs, dys, gs = x64[perm // K], d64[perm // K], g.ravel()[perm]
    ref = oracle.experts_backward_mx_w(xs, counts, gs, dys, Wg, Wu, Wd, return_parts=True)
    al = backward_allowance(ref, xs, counts, Wg, Wu, Wd)
    rs = oracle.shared_backward(x64, d64, H.ws_gate, H.ws_up, H.ws_down)
    dx_ref = ref['dx_slot'][inv].reshape(T, K, D).sum(axis=1) + rs['dx']
    dx_al = al['dx_slot'][inv].reshape(T, K, D).sum(axis=1)
    assert_close_rms(t2np(dx), dx_ref, TAU, 'mx layer dx', True, dx_al)
    dg = ref['dg'][inv].reshape(T, K)
    assert_close_rms(t2np(dtw), dg, TAU, 'mx layer d_topk_w')
    dl = oracle.d_logits_from_dg(g, idx, dg, E)
    assert_close_rms(t2np(dlg), dl, TAU, 'mx layer d_logits')
    mask = np.zeros((T, E), dtype=bool)
    np.put_along_axis(mask, idx.astype(np.int64), True, axis=1)
    assert np.all(t2np(dlg)[~mask] == 0)
    for k in ('dW_gate', 'dW_up', 'dW_down'):
        assert_close_rms(t2np(gr[k.replace('dW', 'dw')]), ref[k], TAU, 'mx layer ' + k, False, al[k])
    fr = {'dx': frac_beyond(t2np(dx), dx_ref, TAU, True)}
    for k in ('dW_gate', 'dW_up', 'dW_down'):
        fr[k] = frac_beyond(t2np(gr[k.replace('dW', 'dw')]), ref[k], TAU)
    print('  share beyond tau*RMS without allowance:', {k: f'{v:.2e}' for k, v in fr.items()}, flush=True)
    assert max(fr.values()) < 0.005, fr
    for k in ('dW_gate', 'dW_up', 'dW_down'):
        assert_close_rms(t2np(gr[k.replace('dW', 'dws')]), rs[k], TOL['bf16'], 'mx layer shared ' + k)


def run_mx_layer(m, H, q, keep=False, flags=0, budget=None):
    """moe_forward + moe_backward in MXFP8 (keep: moe_forward_keep + moe_backward_kept), every
    output; budget: the workgroup budget word's value in both workspaces."""
    from test_gpu_mxfp8 import run_mx_forward
    cfg = H.cfg
    T, K, D, E, I, Is = cfg.T, cfg.K, cfg.D, cfg.E, cfg.I, cfg.I_shared
    dout = bf(synth.host_dout(cfg, T))
    act = [torch.full((T * K, I), float('nan'), device='cuda') for _ in range(2)] if keep else None
    out, yr, rt, p, tensors = run_mx_forward(m, H, q, act, flags=flags, budget=budget)
    W = m.make_weights(*tensors['wq'], *tensors['ws'], *tensors['sc'])
    gr = dict(dw_gate=torch.empty((E, I, D), device='cuda'), dw_up=torch.empty((E, I, D), device='cuda'),
              dw_down=torch.empty((E, D, I), device='cuda'), dws_gate=torch.empty((Is, D), device='cuda'),
              dws_up=torch.empty((Is, D), device='cuda'), dws_down=torch.empty((D, Is), device='cuda'))
    dx = torch.empty((T, D), dtype=torch.bfloat16, device='cuda')
    dtw = torch.empty((T, K), dtype=torch.float32, device='cuda')
    dlg = torch.empty((T, E), dtype=torch.float32, device='cuda')
    wsb = torch.zeros(((m.backward_kept_workspace_size if keep else m.backward_workspace_size)(p),),
                      dtype=torch.uint8, device='cuda')
    if budget is not None:
        wsb[m.MOE_WS_CU_BUDGET_OFFSET:m.MOE_WS_CU_BUDGET_OFFSET + 4].view(torch.int32).fill_(budget)
    args = (p, dout, tensors['x'], tensors['logits'], W, m.make_routing(*rt), dx, m.make_grads(**gr), dtw, dlg)
    if keep:
        m.backward_kept(*args, *act, wsb)
    else:
        m.backward(*args, wsb)
    torch.cuda.synchronize()
    assert int(wsb[:4].view(torch.int32).item()) == 0
    return dict(out=out, yr=yr, dx=dx, dtw=dtw, dlg=dlg, **gr)


def test_mx_layer_keep_activations_bitwise(m):
    """moe_forward_keep + moe_backward_kept in MXFP8: the routed a, u of the block-scaled GEMM
    handed to the layer backward instead of replayed; every output bitwise that of moe_forward +
    moe_backward."""
    from test_gpu_mxfp8 import MX_SMALL, mx_layer
    H, q = mx_layer(MX_SMALL)
    res = [run_mx_layer(m, H, q, keep) for keep in (False, True)]
    for k in res[0]:
        assert torch.equal(res[0][k], res[1][k]), k


def test_mx_layer_gather_equals_dispatch_copy_bitwise(m):
    """The MXFP8 layer backward quantises x and g dout straight from the token rows through the
    schedule; MOE_FLAG_DISPATCH_COPY dispatches slot copies first. Same bits in every output, with
    a, u replayed or kept."""
    from test_gpu_mxfp8 import MX_SMALL, mx_layer
    H, q = mx_layer(MX_SMALL)
    for keep in (False, True):
        a = run_mx_layer(m, H, q, keep)
        b = run_mx_layer(m, H, q, keep, m.MOE_FLAG_DISPATCH_COPY)
        for k in a:
            assert torch.equal(a[k], b[k]), (keep, k)
