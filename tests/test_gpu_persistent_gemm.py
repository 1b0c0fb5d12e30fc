"""GPU tests of the persistent grouped GEMMs (MOE_FLAG_PERSISTENT_GEMM) and of the workgroup
budget word polled between their tiles (MOE_FLAG_CU_BUDGET).

Each tile of the persistent kernels is one workgroup's fixed-order sum, as in the per-tile
launch, so every output must equal the per-tile launch's bit for bit: whatever the grid, the
order in which workgroups take tiles, and however many workgroups the budget leaves working
(down to one), including a budget changed from another stream while the call runs. The
per-tile launch itself is checked against the oracle in test_gpu_forward.py."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import ForwardRun, PinnedWord

pytestmark = pytest.mark.gpu

SMALL_BF16 = synth.scaled(synth.DSV3, 'small_bf16_T300_D256_I256_E16_K4', T=300, D=256, I=256, E=16, K=4,
                          I_shared=256)
NOSHARED_BF16 = synth.scaled(synth.MID, 'noshared_bf16', T=257, D=384, I=256, E=12, K=3, I_shared=0)


@pytest.fixture(scope='module')
def m():
    import mixture_experts_layer_norm_amd as mod
    return mod


def set_budget(run, m, v):
    run.ws[m.MOE_WS_CU_BUDGET_OFFSET:m.MOE_WS_CU_BUDGET_OFFSET + 4].view(torch.int32).fill_(v)


def same(a, b):
    assert torch.equal(a.out, b.out)
    if a.y_routes is not None:
        assert torch.equal(a.y_routes, b.y_routes)
    if a.shared_out is not None:
        assert torch.equal(a.shared_out, b.shared_out)
    assert int(b.ws[:4].view(torch.int32).item()) == 0


@pytest.mark.parametrize('cfg', [SMALL_BF16, NOSHARED_BF16, synth.MID], ids=lambda c: c.name)
def test_persistent_gemm_bitwise_equals_per_tile(m, cfg):
    print(f'[persistent] {cfg.name}', flush=True)
    L = synth.to_device(synth.host_layer(cfg))
    a = ForwardRun(m, L)()
    b = ForwardRun(m, L, flags=m.MOE_FLAG_PERSISTENT_GEMM)
    for _ in range(3):
        b()
        torch.cuda.synchronize()
        same(a, b)


@pytest.mark.parametrize('chunk,stages', [(256, 3), (768, 4)])
def test_persistent_gemm_chunked_ring(m, chunk, stages):
    print(f'[persistent] chunked {chunk} {stages}', flush=True)
    L = synth.to_device(synth.host_layer(SMALL_BF16))
    a = ForwardRun(m, L)()
    b = ForwardRun(m, L, chunk_rows=chunk, ring_stages=stages, flags=m.MOE_FLAG_PERSISTENT_GEMM)()
    torch.cuda.synchronize()
    same(a, b)


def test_persistent_gemm_keep_forward(m):
    """moe_forward_keep with the flag: its down GEMM runs persistent; a, u and every output equal
    the per-tile keep forward's."""
    print('[persistent] keep forward', flush=True)
    cfg = SMALL_BF16
    L = synth.to_device(synth.host_layer(cfg))
    n = cfg.T * cfg.K
    runs, acts = [], []
    for flags in (0, m.MOE_FLAG_PERSISTENT_GEMM):
        r = ForwardRun(m, L, flags=flags)
        aa = torch.empty((n, cfg.I), dtype=torch.float32, device='cuda')
        uu = torch.empty((n, cfg.I), dtype=torch.float32, device='cuda')
        m.forward_keep(r.p, L.x, L.logits, r.weights, r.out, r.routing, aa, uu, r.ws, r.y_routes, r.shared_out)
        runs.append(r)
        acts.append((aa, uu))
    torch.cuda.synchronize()
    same(runs[0], runs[1])
    assert torch.equal(acts[0][0], acts[1][0]) and torch.equal(acts[0][1], acts[1][1])


@pytest.mark.parametrize('budget', [1, 3, 8, 37, 1000, 0, -4])
def test_cu_budget_preset(m, budget):
    """A budget set before the call: workgroups at or above it take no tile, the others take all
    of them (v <= 0: no limit)."""
    print(f'[budget] preset {budget}', flush=True)
    L = synth.to_device(synth.host_layer(synth.MID))
    a = ForwardRun(m, L)()
    b = ForwardRun(m, L, flags=m.MOE_FLAG_PERSISTENT_GEMM | m.MOE_FLAG_CU_BUDGET)
    set_budget(b, m, budget)
    b()
    torch.cuda.synchronize()
    same(a, b)
    assert int(b.ws[m.MOE_WS_CU_BUDGET_OFFSET:m.MOE_WS_CU_BUDGET_OFFSET + 4].view(torch.int32).item()) == budget


def test_cu_budget_changed_from_another_stream(m):
    """The budget is lowered by a copy on a second stream while the forward runs on the first,
    then raised again: the outputs are unchanged, whenever the copies land."""
    print('[budget] changed during the call', flush=True)
    L = synth.to_device(synth.host_layer(synth.MID))
    a = ForwardRun(m, L)()
    b = ForwardRun(m, L, flags=m.MOE_FLAG_PERSISTENT_GEMM | m.MOE_FLAG_CU_BUDGET)
    set_budget(b, m, 0)
    torch.cuda.synchronize()
    word = b.ws[m.MOE_WS_CU_BUDGET_OFFSET:m.MOE_WS_CU_BUDGET_OFFSET + 4].view(torch.int32)
    side = torch.cuda.Stream()
    for v in (16, 1, 64):
        host = torch.tensor([v], dtype=torch.int32).pin_memory()
        b()
        with torch.cuda.stream(side):
            word.copy_(host, non_blocking=True)
        torch.cuda.synchronize()
        same(a, b)
        assert int(word.item()) == v
        set_budget(b, m, 0)
        torch.cuda.synchronize()


def test_cu_budget_host_word(m):
    """MOE_FLAG_CU_BUDGET_INDIRECT: the budget word in coherent pinned host memory, its address in the
    workspace. Set before the call (0: no limit, 2, 1) and stored by the host while the call runs
    (after the launch, before the synchronisation): the outputs equal the per-tile forward's; a
    null address means no limit. The word is only read."""
    print('[budget] host word', flush=True)
    L = synth.to_device(synth.host_layer(synth.MID))
    a = ForwardRun(m, L)()
    b = ForwardRun(m, L, flags=m.MOE_FLAG_PERSISTENT_GEMM | m.MOE_FLAG_CU_BUDGET | m.MOE_FLAG_CU_BUDGET_INDIRECT)
    slot = b.ws[m.MOE_WS_CU_BUDGET_PTR_OFFSET:m.MOE_WS_CU_BUDGET_PTR_OFFSET + 8].view(torch.int64)
    hw = PinnedWord()
    try:
        slot.fill_(0)                       # null address: no limit
        b()
        torch.cuda.synchronize()
        same(a, b)
        slot.fill_(hw.device_address)
        for v in (0, 2, 1):
            hw.value = v
            b()
            torch.cuda.synchronize()
            same(a, b)
            assert hw.value == v
        for v in (1, 5, 0):
            hw.value = 0
            b()
            hw.value = v                    # stored while the forward may still run
            torch.cuda.synchronize()
            same(a, b)
        torch.cuda.synchronize()
    finally:
        hw.close()


def test_persistent_gemm_full_size_dsv3(m):
    """DSV3 shape (T=8192, 256 experts, 6,700-odd up/gate tiles): the persistent forward, with and
    without a budget of 64 workgroups, equals the per-tile forward bit for bit."""
    print('[persistent] DSV3 full size', flush=True)
    L = synth.device_layer(synth.DSV3)
    a = ForwardRun(m, L, want_parts=False)()
    b = ForwardRun(m, L, flags=m.MOE_FLAG_PERSISTENT_GEMM | m.MOE_FLAG_CU_BUDGET, want_parts=False)
    for v in (0, 64):
        set_budget(b, m, v)
        b()
        torch.cuda.synchronize()
        assert torch.equal(a.out, b.out), v
        assert int(b.ws[:4].view(torch.int32).item()) == 0
    del L
    torch.cuda.empty_cache()


@pytest.mark.parametrize('budget', [None, 2])
def test_persistent_gemm_experts_forward(m, budget):
    """moe_experts_forward (slots already grouped by expert, one expert-parallel rank's share):
    forced persistent GEMMs, with or without a budget of 2 workgroups, equal the per-tile launch
    bit for bit; so does the automatic choice on a share large enough to take it."""
    print(f'[persistent] experts forward budget={budget}', flush=True)
    rng = np.random.default_rng(5)
    T, D, I, E, K, Is = 640, 256, 256, 4, 8, 256
    counts = np.array([2100, 1500, 0, 1400])
    S = int(counts.sum())
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)

    def bf(shape, scale):
        return (torch.from_numpy(rng.standard_normal(shape).astype(np.float32)) * scale).cuda().to(torch.bfloat16)
    x_slot, x_local = bf((S, D), 1.0), bf((T, D), 1.0)
    wts = [bf((E, I, D), D ** -0.5), bf((E, I, D), D ** -0.5), bf((E, D, I), I ** -0.5),
           bf((Is, D), D ** -0.5), bf((Is, D), D ** -0.5), bf((D, Is), Is ** -0.5)]
    W = m.make_weights(*wts)
    off_d = torch.from_numpy(offsets).cuda()
    outs = []
    flag_sets = [0, m.MOE_FLAG_PERSISTENT_GEMM | (m.MOE_FLAG_CU_BUDGET if budget else 0)]
    for flags in flag_sets:
        p = m.problem(T, D, I, E, K, Is, 'bf16', 0, 0, flags)
        ws = torch.zeros((m.workspace_size(p),), dtype=torch.uint8, device='cuda')
        if budget:
            ws[m.MOE_WS_CU_BUDGET_OFFSET:m.MOE_WS_CU_BUDGET_OFFSET + 4].view(torch.int32).fill_(budget)
        y = torch.empty((S, D), dtype=torch.bfloat16, device='cuda')
        sh = torch.empty((T, D), dtype=torch.bfloat16, device='cuda')
        m.experts_forward(p, S, x_slot, off_d, W, y, x_local, sh, ws)
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32).item()) == 0
        outs.append((y, sh))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize('cfg,budget', [(SMALL_BF16, None), (SMALL_BF16, 3), (NOSHARED_BF16, None)],
                         ids=['small', 'small_budget3', 'noshared'])
def test_persistent_gemm_layer_backward(m, cfg, budget):
    """moe_backward with forced persistent GEMMs (replay, dgrad-down with the SwiGLU backward,
    dgrad-up, K-grouped weight gradients; routed and shared): every gradient equals the per-tile
    backward's bit for bit, also with a budget of 3 workgroups."""
    print(f'[persistent] layer backward {cfg.name} budget={budget}', flush=True)
    L = synth.to_device(synth.host_layer(cfg))
    T, D, I, E, K, Is = cfg.T, cfg.D, cfg.I, cfg.E, cfg.K, cfg.I_shared
    rng = np.random.default_rng(3)
    dout = torch.from_numpy(rng.standard_normal((T, D)).astype(np.float32)).cuda().to(torch.bfloat16)
    res = []
    for flags in (0, m.MOE_FLAG_PERSISTENT_GEMM | (m.MOE_FLAG_CU_BUDGET if budget else 0)):
        run = ForwardRun(m, L, flags=flags)()
        shapes = ((E, I, D), (E, I, D), (E, D, I)) + (((Is, D), (Is, D), (D, Is)) if Is else ())
        gr = [torch.full(sh, float('nan'), device='cuda') for sh in shapes]
        G = m.make_grads(*gr)
        dx = torch.empty((T, D), dtype=torch.bfloat16, device='cuda')
        dtw = torch.empty((T, K), dtype=torch.float32, device='cuda')
        dlg = torch.empty((T, E), dtype=torch.float32, device='cuda')
        wsb = torch.zeros((m.backward_workspace_size(run.p),), dtype=torch.uint8, device='cuda')
        if budget:
            wsb[m.MOE_WS_CU_BUDGET_OFFSET:m.MOE_WS_CU_BUDGET_OFFSET + 4].view(torch.int32).fill_(budget)
        m.backward(run.p, dout, L.x, L.logits, run.weights, run.routing, dx, G, dtw, dlg, wsb)
        torch.cuda.synchronize()
        assert int(wsb[:4].view(torch.int32).item()) == 0
        res.append([dx, dtw, dlg] + gr)
    for a, b in zip(*res):
        assert torch.equal(a, b)


# MXFP8: the block-scaled GEMMs (forward, replay, dgrad, K-grouped weight gradients) have the same
# persistent form; forced, with or without a budget, every output equals the per-tile launch's.
@pytest.mark.parametrize('budget', [None, 3])
def test_persistent_mx_layer_forward_backward(m, budget):
    from test_gpu_mxfp8 import MX_SMALL, mx_layer
    from test_gpu_mxfp8_backward import run_mx_layer
    print(f'[persistent] mxfp8 layer forward + backward budget={budget}', flush=True)
    H, q = mx_layer(MX_SMALL)
    a = run_mx_layer(m, H, q)
    flags = m.MOE_FLAG_PERSISTENT_GEMM | (m.MOE_FLAG_CU_BUDGET if budget else 0)
    for keep in (False, True):
        b = run_mx_layer(m, H, q, keep, flags, budget)
        for k in a:
            assert torch.equal(a[k], b[k]), (keep, k)


@pytest.mark.parametrize('chunk,stages', [(256, 3), (512, 4)])
def test_persistent_mx_chunked_ring(m, chunk, stages):
    from test_gpu_mxfp8 import MX_SMALL, mx_layer, run_mx_forward
    print(f'[persistent] mxfp8 chunked {chunk} {stages}', flush=True)
    H, q = mx_layer(MX_SMALL)
    a, ya, *_ = run_mx_forward(m, H, q)
    b, yb, *_ = run_mx_forward(m, H, q, chunk_rows=chunk, ring_stages=stages, flags=m.MOE_FLAG_PERSISTENT_GEMM)
    assert torch.equal(a, b) and torch.equal(ya, yb)


@pytest.mark.parametrize('counts', [[300, 0, 157], [1, 257, 242]], ids=['empty_mid', 'ragged_single'])
def test_persistent_mx_experts(m, counts):
    """moe_experts_forward + moe_experts_backward in MXFP8 (one expert-parallel rank's share)."""
    import oracle
    from test_gpu_mxfp8_backward import SMALL, run_share_mx
    print(f'[persistent] mxfp8 experts {counts}', flush=True)
    H = synth.host_share(SMALL)
    q = {k: oracle.mx_quantize(getattr(H, k).astype(np.float64)) for k in ('w_gate', 'w_up', 'w_down')}
    a = run_share_mx(m, H, q, counts)
    b = run_share_mx(m, H, q, counts, flags=m.MOE_FLAG_PERSISTENT_GEMM)
    assert a['err'] == 0 and b['err'] == 0
    for k in ('y', 'sh', 'dx_slot', 'dg', 'dw_gate', 'dw_up', 'dw_down', 'dws_gate', 'dws_up', 'dws_down', 'dx_local'):
        assert torch.equal(a[k], b[k]), k
