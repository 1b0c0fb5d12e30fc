"""moe_forward_lanes: the chunked forward with its chunks spread over several streams gives bitwise
the outputs of the unchunked moe_forward (every output tile is one workgroup's fixed-order sum,
whichever stream runs it), with and without cross-lane ring-stage events, with persistent GEMMs
on several lanes at once, under MXFP8, captured into a graph, and at the DSV3 shape."""
import pytest
import torch

import synth
from gpu_util import ForwardRun

pytestmark = pytest.mark.gpu

SMALL_BF16 = synth.scaled(synth.DSV3, 'small_bf16_T300_D256_I256_E16_K4', T=300, D=256, I=256, E=16, K=4,
                          I_shared=256)


@pytest.fixture(scope='module')
def m():
    import mixture_experts_layer_norm_amd as mod
    return mod


def make_lanes(m, p, count):
    streams = [torch.cuda.Stream() for _ in range(count)]
    events = [torch.cuda.Event() for _ in range(m.lane_event_count(p, count))]
    for e in events:
        e.record()                       # creates the event
    torch.cuda.synchronize()
    return streams, events


def assert_same(a, b, what):
    assert int(b.ws[:4].view(torch.int32).item()) == 0, what
    assert torch.equal(a.y_routes, b.y_routes), what
    if a.shared_out is not None:
        assert torch.equal(a.shared_out, b.shared_out), what
    assert torch.equal(a.out, b.out), what


# (chunk rows b, ring stages S, extra lanes): S % (lanes + 1) == 0 keeps each stage on one lane;
# otherwise stages pass between lanes through the stage events; the last case has one chunk.
@pytest.mark.parametrize('chunk,stages,count', [(256, 3, 1), (256, 4, 3), (256, 3, 2), (256, 5, 3), (512, 4, 1),
                                                (768, 3, 3), (1 << 20, 3, 2)])
def test_lanes_bitwise_equal_unchunked(m, chunk, stages, count):
    print(f'[lanes] {SMALL_BF16.name} chunk={chunk} stages={stages} lanes={count}', flush=True)
    L = synth.to_device(synth.host_layer(SMALL_BF16))
    a = ForwardRun(m, L)()
    b = ForwardRun(m, L, chunk_rows=chunk, ring_stages=stages)
    streams, events = make_lanes(m, b.p, count)
    for rep in range(3):                 # the same events and workspace, call after call
        b.out.fill_(float('nan'))
        b.y_routes.fill_(float('nan'))
        b.lanes(streams, events)
        torch.cuda.synchronize()
        assert_same(a, b, f'rep {rep}')


def test_lanes_dispatch_copy(m):
    """Lanes with each chunk's x rows dispatched into the ring (MOE_FLAG_DISPATCH_COPY): stage
    events then guard x copies as well as h."""
    print(f'[lanes] {SMALL_BF16.name} dispatch copy', flush=True)
    L = synth.to_device(synth.host_layer(SMALL_BF16))
    a = ForwardRun(m, L)()
    b = ForwardRun(m, L, chunk_rows=256, ring_stages=3, flags=m.MOE_FLAG_DISPATCH_COPY)
    streams, events = make_lanes(m, b.p, 3)
    for rep in range(3):
        b.lanes(streams, events)
        torch.cuda.synchronize()
        assert_same(a, b, f'rep {rep}')


def test_lanes_with_persistent_gemms(m):
    """Every GEMM forced persistent: the lanes' launches run at once, each on its own counters."""
    print(f'[lanes] {SMALL_BF16.name} persistent', flush=True)
    L = synth.to_device(synth.host_layer(SMALL_BF16))
    a = ForwardRun(m, L)()
    b = ForwardRun(m, L, chunk_rows=256, ring_stages=4, flags=m.MOE_FLAG_PERSISTENT_GEMM)
    streams, events = make_lanes(m, b.p, 3)
    for rep in range(3):
        b.lanes(streams, events)
        torch.cuda.synchronize()
        assert_same(a, b, f'rep {rep}')


def test_mx_lanes_bitwise_equal_unchunked(m):
    from test_gpu_mxfp8 import MX_SMALL, mx_layer, run_mx_forward
    print(f'[lanes] {MX_SMALL.name} mxfp8', flush=True)
    H, q = mx_layer(MX_SMALL)
    a, ya, *_ = run_mx_forward(m, H, q)
    for chunk, stages, count in ((256, 3, 2), (512, 4, 3)):
        p = m.problem(MX_SMALL.T, MX_SMALL.D, MX_SMALL.I, MX_SMALL.E, MX_SMALL.K, MX_SMALL.I_shared, 'mxfp8', chunk,
                      stages)
        b, yb, *_ = run_mx_forward(m, H, q, chunk_rows=chunk, ring_stages=stages, lanes=make_lanes(m, p, count))
        assert torch.equal(a, b) and torch.equal(ya, yb), (chunk, stages, count)


def test_lanes_graph_replay_bitwise(m):
    """Captured from the current stream, the lanes join the graph through the fork event and
    leave it through the join events; replays (outputs poisoned in between) give the eager bits."""
    print(f'[lanes] {SMALL_BF16.name} graph', flush=True)
    L = synth.to_device(synth.host_layer(SMALL_BF16))
    a = ForwardRun(m, L)()
    b = ForwardRun(m, L, chunk_rows=256, ring_stages=3)
    streams, events = make_lanes(m, b.p, 2)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        b.lanes(streams, events)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        b.lanes(streams, events)
    torch.cuda.synchronize()
    for rep in range(4):
        b.out.fill_(float('nan'))
        b.y_routes.fill_(float('nan'))
        b.shared_out.fill_(float('nan'))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same(a, b, f'replay {rep}')
    del g


@pytest.mark.parametrize('chunk,stages,count', [(512, 8, 3), (4096, 4, 3)])
def test_lanes_dsv3_full_size(m, chunk, stages, count):
    """At the DSV3 shape (T=8192, D=7168, I=2048, E=256, K=8, one shared expert)."""
    print(f'[lanes] {synth.DSV3.name} chunk={chunk} stages={stages} lanes={count}', flush=True)
    L = synth.device_layer(synth.DSV3)
    a = ForwardRun(m, L)()
    b = ForwardRun(m, L, chunk_rows=chunk, ring_stages=stages)
    b.lanes(*make_lanes(m, b.p, count))
    torch.cuda.synchronize()
    assert_same(a, b, 'dsv3')
