"""The library's calls only enqueue kernels on the given stream (no allocation, memset, copy or
synchronisation), so a caller can capture them into a HIP graph. Each replay is checked bitwise
against the eager result, with eager work of the program in between and the outputs poisoned
before every replay."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import ForwardRun

pytestmark = pytest.mark.gpu

CFG = synth.scaled(synth.DSV3, 'graph_bf16_T512_D1024_I512_E32_K4', T=512, D=1024, I=512, E=32, K=4, I_shared=256)


@pytest.fixture(scope='module')
def m():
    import mixture_experts_layer_norm_amd as mod
    return mod


def test_forward_and_backward_graph_replay_bitwise(m):
    print(f'[graph] {CFG.name}', flush=True)
    H = synth.host_layer(CFG)
    L = synth.to_device(H)
    run = ForwardRun(m, L, want_parts=False)
    E, I, D, Is, T, K = CFG.E, CFG.I, CFG.D, CFG.I_shared, CFG.T, CFG.K
    dout = torch.from_numpy(np.ascontiguousarray(synth.host_dout(CFG, T), dtype=np.float32)).cuda().to(torch.bfloat16)
    gr = dict(dw_gate=torch.empty((E, I, D), device='cuda'), dw_up=torch.empty((E, I, D), device='cuda'),
              dw_down=torch.empty((E, D, I), device='cuda'), dws_gate=torch.empty((Is, D), device='cuda'),
              dws_up=torch.empty((Is, D), device='cuda'), dws_down=torch.empty((D, Is), device='cuda'))
    G = m.make_grads(**gr)
    dx = torch.empty((T, D), dtype=torch.bfloat16, device='cuda')
    dtw = torch.empty((T, K), dtype=torch.float32, device='cuda')
    dlg = torch.empty((T, E), dtype=torch.float32, device='cuda')
    wsb = torch.zeros((m.backward_workspace_size(run.p),), dtype=torch.uint8, device='cuda')

    def step():
        run()
        m.backward(run.p, dout, L.x, L.logits, run.weights, run.routing, dx, G, dtw, dlg, wsb)

    outs = lambda: [run.out, run.topk_idx, run.perm, dx, dtw, dlg] + list(gr.values())
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs()]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on the capture side stream, as torch recommends
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs():                    # eager work between replays: poison every output
            if t.dtype.is_floating_point:
                t.fill_(float('nan'))
            else:
                t.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(['out', 'topk_idx', 'perm', 'dx', 'd_topk_w', 'd_logits'] + list(gr), outs(), ref):
            assert torch.equal(a, b), f'replay {rep}: {name} differs from the eager result'
    del g


def test_keep_activations_graph_replay_bitwise(m):
    """moe_forward_keep + moe_backward_kept captured into one graph: replays bitwise equal to the
    eager run, the kept a, u buffers poisoned before every replay."""
    print(f'[graph] keep {CFG.name}', flush=True)
    H = synth.host_layer(CFG)
    L = synth.to_device(H)
    run = ForwardRun(m, L, want_parts=False)
    E, I, D, Is, T, K = CFG.E, CFG.I, CFG.D, CFG.I_shared, CFG.T, CFG.K
    dout = torch.from_numpy(np.ascontiguousarray(synth.host_dout(CFG, T), dtype=np.float32)).cuda().to(torch.bfloat16)
    gr = dict(dw_gate=torch.empty((E, I, D), device='cuda'), dw_up=torch.empty((E, I, D), device='cuda'),
              dw_down=torch.empty((E, D, I), device='cuda'), dws_gate=torch.empty((Is, D), device='cuda'),
              dws_up=torch.empty((Is, D), device='cuda'), dws_down=torch.empty((D, Is), device='cuda'))
    G = m.make_grads(**gr)
    dx = torch.empty((T, D), dtype=torch.bfloat16, device='cuda')
    dtw = torch.empty((T, K), dtype=torch.float32, device='cuda')
    dlg = torch.empty((T, E), dtype=torch.float32, device='cuda')
    act = [torch.empty((T * K, I), device='cuda') for _ in range(2)]
    wsb = torch.zeros((m.backward_kept_workspace_size(run.p),), dtype=torch.uint8, device='cuda')

    def step():
        m.forward_keep(run.p, L.x, L.logits, run.weights, run.out, run.routing, *act, run.ws)
        m.backward_kept(run.p, dout, L.x, L.logits, run.weights, run.routing, dx, G, dtw, dlg, *act, wsb)

    outs = lambda: [run.out, dx, dtw, dlg] + act + list(gr.values())
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs():
            t.fill_(float('nan'))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs(), ref)):
            assert torch.equal(a, b), f'replay {rep}: output {i} differs from the eager result'
    del g
