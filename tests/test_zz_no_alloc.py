"""moe_schedule_noalloc (scratch in a static device array, no workspace) against moe_schedule
(scratch in the caller's workspace): bitwise equal counts, offsets, perm and inv_perm on two calls
in a row, the second smaller than the first, so the second call runs over the first one's
leftovers in the array; and the same error bit for an out-of-range expert id."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope='module')
def m():
    import mixture_experts_layer_norm_amd as mod
    return mod


def routing(seed, T, K, E, skew):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)) + skew * rng.standard_normal(E)
    return oracle.route_topk(logits, K)


def both(m, idx, E, bad=None):
    T, K = idx.shape
    p = m.problem(T, 128, 128, E, K, 0, 'bf16')
    d = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
    if bad is not None:
        d.view(-1)[bad] = E + 3
    outs = []
    for noalloc in (False, True):
        o = [torch.full((E,), -7, dtype=torch.int32, device='cuda'), torch.full((E + 1,), -7, dtype=torch.int32, device='cuda'),
             torch.full((T * K,), -7, dtype=torch.int32, device='cuda'), torch.full((T * K,), -7, dtype=torch.int32, device='cuda')]
        err = torch.zeros((1,), dtype=torch.int32, device='cuda')
        if noalloc:
            m.schedule_noalloc(p, d, *o, err)
        else:
            ws = torch.zeros((m.workspace_size(p),), dtype=torch.uint8, device='cuda')
            m.schedule(p, d, *o, ws)
            err = ws[:4].view(torch.int32)
        torch.cuda.synchronize()
        outs.append([t.cpu().numpy() for t in o] + [int(err.item())])
    return outs


def test_noalloc_schedule_equals_workspace_schedule_twice(m):
    # first call: 72,000 routes over 256 experts (36 histogram blocks); second: 1,200 routes over 64
    for seed, T, K, E, skew in ((1, 9000, 8, 256, 0.7), (2, 300, 4, 64, 0.0)):
        ref, got = both(m, routing(seed, T, K, E, skew), E)
        for a, b, name in zip(ref, got, ('counts', 'offsets', 'perm', 'inv_perm', 'error word')):
            assert np.array_equal(a, b), name
        c, off, perm, inv = oracle.schedule(routing(seed, T, K, E, skew), E)
        assert np.array_equal(got[2], perm) and np.array_equal(got[0], c)


def test_noalloc_schedule_reports_out_of_range_ids(m):
    ref, got = both(m, routing(3, 257, 3, 16, 0.3), 16, bad=[5, 400])
    assert ref[4] == 1 and got[4] == 1
    for a, b in zip(ref[:4], got[:4]):
        assert np.array_equal(a, b)
