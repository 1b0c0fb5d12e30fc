"""The C ABI library loads, exports every entry point include/moe.h declares, and rejects bad
arguments on the host (no GPU work is done on these paths). CPU only."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, 'include', 'moe.h')).read()
    src = re.sub(r'/\*.*?\*/', '', src, flags=re.S)
    return sorted(set(re.findall(r'\b(moe_[a-z_0-9]+)\s*\(', src)))


def test_header_declares_the_boundary():
    syms = declared_symbols()
    for name in ('moe_route_topk', 'moe_schedule', 'moe_dispatch', 'moe_combine', 'moe_forward',
                 'moe_backward', 'moe_experts_forward', 'moe_experts_backward', 'moe_quantize_mx',
                 'moe_workspace_size', 'moe_status_string'):
        assert name in syms


def test_library_exports_every_declared_symbol():
    import mixture_experts_layer_norm_amd as m
    lib = ctypes.CDLL(m.LIB_PATH)
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert set(declared_symbols()) == set(m.EXPORTED)


def test_status_strings():
    import mixture_experts_layer_norm_amd as m
    for code, name in m.STATUS.items():
        assert m.status_string(code) == name


def test_workspace_size_and_validation():
    import mixture_experts_layer_norm_amd as m
    p = m.problem(8192, 7168, 2048, 256, 8, 2048, 'bf16')
    n = m.workspace_size(p)
    assert n > 8192 * 8 * 7168 * 2      # holds at least the per-route outputs
    bad = [
        m.problem(0, 128, 64, 8, 2),            # T < 1
        m.problem(16, 128, 64, 8, 0),           # K < 1
        m.problem(16, 128, 64, 8, 2, dtype=7),  # unknown dtype
        m.problem(16, 128, 64, 8, 2, ring_stages=2),
    ]
    for p in bad:
        with pytest.raises(m.MoeError) as ei:
            m.workspace_size(p)
        assert ei.value.status == -1
    for p in (m.problem(16, 100, 128, 8, 2, dtype='bf16'),    # D not a multiple of 128
              m.problem(16, 128, 64, 2000, 2, dtype='bf16')):  # E > 1024
        with pytest.raises(m.MoeError) as ei:
            m.workspace_size(p)
        assert ei.value.status == -2
    # routing entry points also need K <= min(E, 64); the expert-level ones use K as slots/token
    lib = m._lib
    assert lib.moe_route_topk(ctypes.byref(m.problem(16, 128, 128, 8, 9)), 16, 16, 16, None) == -1
    assert lib.moe_route_topk(ctypes.byref(m.problem(16, 128, 128, 100, 65)), 16, 16, 16, None) == -2
    assert m.workspace_size(m.problem(7168, 7168, 2048, 4, 8, 2048)) > 0   # 4 local experts, 8 slots/token


def test_entry_points_reject_null_and_small_workspace_without_gpu():
    """These calls return on the host before any HIP call (no device is present here)."""
    import mixture_experts_layer_norm_amd as m
    lib = m._lib
    p = m.problem(16, 128, 64, 8, 2, 64, 'f32')
    P = ctypes.byref(p)
    assert lib.moe_route_topk(P, None, None, None, None) == -1
    assert lib.moe_schedule(P, 16, 16, 16, 16, 16, None, 0, None) == -3
    assert lib.moe_schedule(P, 16, 16, 16, 16, 16, 256, 1, None) == -3
    assert lib.moe_dispatch(P, 16, 16, 0, 10 ** 6, 16, None, None) == -1       # past T*K
    assert lib.moe_dispatch(P, 16, 16, 0, 4, 16, 16, None) == -1              # scales without MXFP8
    assert lib.moe_dispatch(P, 8, 16, 0, 4, 16, None, None) == -4             # misaligned x
    assert lib.moe_combine(P, None, None, None, None, None) == -1
    assert lib.moe_dispatch_tokens(P, 16, None, 16, None, None) == -1
    assert lib.moe_dispatch_tokens(P, 16, 16, 16, 16, None) == -1        # scales without MXFP8
    assert lib.moe_dispatch_tokens(P, 8, 16, 16, None, None) == -4      # misaligned x
    pm = m.problem(16, 128, 128, 8, 2, 128, 'mxfp8')
    assert lib.moe_dispatch_tokens(ctypes.byref(pm), 16, 16, 16, None, None) == -1   # MXFP8 needs scales
    assert lib.moe_quantize_mx(16, 4, 48, 16, 16, None) == -2                 # cols % 32
    # fused router: fp32 refused, null pointers, workspace size
    pb = m.problem(16, 128, 128, 8, 2, 128, 'bf16')
    assert lib.moe_route_gemm(P, 16, 16, 16, 16, 16, 16, 1 << 30, None) == -2            # MOE_F32
    assert lib.moe_route_gemm(ctypes.byref(pb), None, 16, 16, 16, 16, 16, 1 << 30, None) == -1
    assert lib.moe_route_gemm(ctypes.byref(pb), 16, 16, 16, 16, 16, 16, 8, None) == -3   # workspace
    assert lib.moe_route_gemm_workspace_size(ctypes.byref(pb), None) == -1
    # pull schedule: R, rank, R*L limit, null pointers, workspace size
    nb = ctypes.c_size_t(0)
    assert lib.moe_pull_schedule_workspace_size(8, 64, 8, 32, ctypes.byref(nb)) == 0 and nb.value > 256
    assert lib.moe_pull_schedule_workspace_size(8, 64, 8, 32, None) == -1
    a = (16,) * 7
    assert lib.moe_pull_schedule(0, 64, 8, 4, 0, *a, 16, 1 << 20, None) == -1          # R < 1
    assert lib.moe_pull_schedule(4, 64, 8, 4, 4, *a, 16, 1 << 20, None) == -1          # rank >= R
    assert lib.moe_pull_schedule(64, 64, 8, 32, 0, *a, 16, 1 << 20, None) == -2        # R*L > 1024
    assert lib.moe_pull_schedule(4, 64, 8, 4, 0, None, *a[1:], 16, 1 << 20, None) == -1
    assert lib.moe_pull_schedule(4, 64, 8, 4, 0, *a, 16, 8, None) == -3                # workspace too small
    w = m.Weights()
    r = m.Routing()
    assert lib.moe_forward(P, 16, 16, ctypes.byref(w), 16, ctypes.byref(r), None, None, None, 0, None) == -1
    # the persistent chunk kernel is switched off: the flag is refused before any launch
    pp = m.problem(16, 128, 128, 8, 2, 0, 'bf16', 256, 3, m.MOE_FLAG_PERSISTENT)
    for f in ('w_gate', 'w_up', 'w_down'):
        setattr(w, f, 256)
    for f in ('topk_idx', 'topk_w', 'counts', 'offsets', 'perm', 'inv_perm'):
        setattr(r, f, 256)
    assert lib.moe_forward(ctypes.byref(pp), 256, 256, ctypes.byref(w), 256, ctypes.byref(r), None, None, 256,
                           1 << 40, None) == -2


def test_one_hip_runtime_whatever_the_import_order():
    """Importing the binding before torch must not load a second HIP runtime into the process
    (torch's device pointers would be invalid in the library)."""
    import subprocess
    import sys
    code = ('import re, mixture_experts_layer_norm_amd, torch\n'
            'maps = open("/proc/self/maps").read()\n'
            'print(len(set(re.findall(r"\\S*/libamdhip64\\S*", maps))))\n')
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, '-c', code], capture_output=True, text=True, cwd=root, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == '1', r.stdout


def test_keep_activation_entry_points_reject_without_gpu():
    """moe_experts_forward_keep / moe_experts_backward_kept check on the host, before any HIP
    call: both activation buffers are required, and MOE_F32 is not supported."""
    import mixture_experts_layer_norm_amd as m
    lib = m._lib
    W, G = m.Weights(), m.Grads()
    fake = 1 << 20   # never dereferenced: every call below returns before touching memory
    cases = (('bf16', (fake, None, None, None), -1), ('mxfp8', (None, fake, None, None), -1),
             ('bf16', (fake, fake, fake, None), -1), ('f32', (fake, fake, None, None), -2))
    for dt, acts, code in cases:
        p = m.problem(100, 256, 256, 3, 5, 128, dt)
        assert lib.moe_experts_forward_keep(ctypes.byref(p), 0, fake, fake, ctypes.byref(W), fake, fake, fake,
                                            *acts, fake, 1 << 40, None) == code, (dt, acts)
        assert lib.moe_experts_backward_kept(ctypes.byref(p), 0, fake, fake, fake, fake, ctypes.byref(W), fake, fake,
                                             ctypes.byref(G), fake, fake, fake, *acts, fake, 1 << 40,
                                             None) == code, (dt, acts)


def test_removed_flag_bits_and_chunk_refusals_without_gpu():
    """Flag bits the library does not define are refused; chunk_rows is refused where no ring can
    hold the rows (fp32, the expert-level forward, the keep forward) instead of being ignored.
    Every call returns before any HIP call."""
    import mixture_experts_layer_norm_amd as m
    lib = m._lib
    n = ctypes.c_size_t()
    for bit in (0x2, 0x8, 0x10, 0x20, 0x100, 0x8000, 0x40000):
        p = m.problem(64, 128, 128, 8, 2, 0, 'bf16', 0, 0, bit)
        assert lib.moe_workspace_size(ctypes.byref(p), ctypes.byref(n)) == -1, hex(bit)
    fake = 1 << 20
    w, r = m.Weights(), m.Routing()
    for f in ('w_gate', 'w_up', 'w_down', 'sc_gate', 'sc_up', 'sc_down'):
        setattr(w, f, fake)
    for f in ('topk_idx', 'topk_w', 'counts', 'offsets', 'perm', 'inv_perm'):
        setattr(r, f, fake)
    p = m.problem(64, 128, 128, 8, 2, 0, 'f32', 256, 3)
    assert lib.moe_forward(ctypes.byref(p), fake, fake, ctypes.byref(w), fake, ctypes.byref(r), None, None, fake,
                           1 << 40, None) == -2
    for dt in ('bf16', 'mxfp8', 'f32'):
        p = m.problem(64, 128, 128, 8, 2, 0, dt, 512, 3)
        assert lib.moe_experts_forward(ctypes.byref(p), 64, fake, fake, ctypes.byref(w), fake, None, None, fake,
                                       1 << 40, None) == -2, dt
    p = m.problem(64, 128, 128, 8, 2, 0, 'bf16', 512, 3)
    assert lib.moe_forward_keep(ctypes.byref(p), fake, fake, ctypes.byref(w), fake, ctypes.byref(r), None, None,
                                fake, fake, fake, 1 << 40, None) == -2


def test_persistent_gemm_flags_without_gpu():
    """MOE_FLAG_CU_BUDGET needs MOE_FLAG_PERSISTENT_GEMM (invalid alone); the persistent GEMMs are
    BF16 and MXFP8 (MOE_F32: unsupported); checked on the host before any launch. The budget word
    sits inside the first 256 bytes of the forward workspace, with the error word."""
    import mixture_experts_layer_norm_amd as m
    lib = m._lib
    n = ctypes.c_size_t()
    p = m.problem(64, 128, 128, 8, 2, 0, 'bf16', 0, 0, m.MOE_FLAG_CU_BUDGET)
    assert lib.moe_workspace_size(ctypes.byref(p), ctypes.byref(n)) == -1
    p = m.problem(64, 128, 128, 8, 2, 0, 'bf16', 0, 0, m.MOE_FLAG_PERSISTENT_GEMM | m.MOE_FLAG_CU_BUDGET)
    assert lib.moe_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0 and n.value >= 256
    # the indirect budget word needs the budget; its address slot is 8-byte aligned, clear of the
    # error word and the budget word, and before the ticket counters (offset 64)
    p = m.problem(64, 128, 128, 8, 2, 0, 'bf16', 0, 0, m.MOE_FLAG_PERSISTENT_GEMM | m.MOE_FLAG_CU_BUDGET_INDIRECT)
    assert lib.moe_workspace_size(ctypes.byref(p), ctypes.byref(n)) == -1
    p = m.problem(64, 128, 128, 8, 2, 0, 'bf16', 0, 0,
                  m.MOE_FLAG_PERSISTENT_GEMM | m.MOE_FLAG_CU_BUDGET | m.MOE_FLAG_CU_BUDGET_INDIRECT)
    assert lib.moe_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
    assert m.MOE_WS_CU_BUDGET_PTR_OFFSET % 8 == 0 and m.MOE_WS_CU_BUDGET_PTR_OFFSET >= m.MOE_WS_CU_BUDGET_OFFSET + 4
    assert m.MOE_WS_CU_BUDGET_PTR_OFFSET + 8 <= 64
    p = m.problem(64, 128, 128, 8, 2, 0, 'bf16', 0, 0, m.MOE_FLAG_ROUTER_BWD_DENSE)   # a known bit
    assert lib.moe_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
    # the forward gathers x through the schedule by default; the slot copy is asked for, and needs
    # the slot buffer; asking for both is invalid
    p = m.problem(8192, 7168, 2048, 256, 8, 2048, 'bf16')
    gather = m.workspace_size(p)
    p = m.problem(8192, 7168, 2048, 256, 8, 2048, 'bf16', 0, 0, m.MOE_FLAG_DISPATCH_COPY)
    assert m.workspace_size(p) >= gather + 8192 * 8 * 7168 * 2
    p = m.problem(64, 128, 128, 8, 2, 0, 'bf16', 0, 0, m.MOE_FLAG_DISPATCH_COPY | m.MOE_FLAG_FUSED_GATHER)
    assert lib.moe_workspace_size(ctypes.byref(p), ctypes.byref(n)) == -1
    assert 4 <= m.MOE_WS_CU_BUDGET_OFFSET and m.MOE_WS_CU_BUDGET_OFFSET + 4 <= 64
    fake = 1 << 20
    w, r = m.Weights(), m.Routing()
    for f in ('w_gate', 'w_up', 'w_down', 'sc_gate', 'sc_up', 'sc_down'):
        setattr(w, f, fake)
    for f in ('topk_idx', 'topk_w', 'counts', 'offsets', 'perm', 'inv_perm'):
        setattr(r, f, fake)
    p = m.problem(64, 128, 128, 8, 2, 0, 'f32', 0, 0, m.MOE_FLAG_PERSISTENT_GEMM)
    assert lib.moe_forward(ctypes.byref(p), fake, fake, ctypes.byref(w), fake, ctypes.byref(r), None, None, fake,
                           1 << 40, None) == -2
    assert lib.moe_experts_forward(ctypes.byref(p), 64, fake, fake, ctypes.byref(w), fake, None, None, fake,
                                   1 << 40, None) == -2


def test_layer_keep_entry_points_reject_without_gpu():
    """moe_forward_keep / moe_backward_kept: F32 unsupported, both buffers required, both 16-byte
    aligned; checked on the host before any launch."""
    import mixture_experts_layer_norm_amd as m
    lib = m._lib
    fake = 1 << 20
    w, r, g = m.Weights(), m.Routing(), m.Grads()
    for f in ('w_gate', 'w_up', 'w_down', 'sc_gate', 'sc_up', 'sc_down'):
        setattr(w, f, fake)
    for f in ('topk_idx', 'topk_w', 'counts', 'offsets', 'perm', 'inv_perm'):
        setattr(r, f, fake)
    for f in ('dw_gate', 'dw_up', 'dw_down'):
        setattr(g, f, fake)
    cases = (('bf16', (fake, None), -1), ('mxfp8', (None, fake), -1), ('f32', (fake, fake), -2),
             ('bf16', (fake + 4, fake), -4), ('mxfp8', (fake, fake + 8), -4))
    for dt, acts, code in cases:
        p = m.problem(64, 128, 128, 8, 2, 0, dt)
        assert lib.moe_forward_keep(ctypes.byref(p), fake, fake, ctypes.byref(w), fake, ctypes.byref(r), None, None,
                                    *acts, fake, 1 << 40, None) == code, ('fwd', dt, acts)
        assert lib.moe_backward_kept(ctypes.byref(p), fake, fake, fake, ctypes.byref(w), ctypes.byref(r), fake,
                                     ctypes.byref(g), fake, None, *acts, fake, 1 << 40, None) == code, ('bwd', dt, acts)


def test_kept_backward_workspace_is_smaller_and_refused_by_the_replay():
    """moe_backward_kept_workspace_size leaves out the replayed a, u (2 T K I 4 bytes); the
    replaying backwards refuse a workspace of only that size (MOE_ERR_WORKSPACE, before any launch)."""
    import mixture_experts_layer_norm_amd as m
    lib = m._lib
    fake = 1 << 20
    w, r, g = m.Weights(), m.Routing(), m.Grads()
    for f in ('w_gate', 'w_up', 'w_down', 'sc_gate', 'sc_up', 'sc_down'):
        setattr(w, f, fake)
    for f in ('topk_idx', 'topk_w', 'counts', 'offsets', 'perm', 'inv_perm'):
        setattr(r, f, fake)
    for f in ('dw_gate', 'dw_up', 'dw_down'):
        setattr(g, f, fake)
    for dt in ('bf16', 'mxfp8'):
        p = m.problem(300, 256, 384, 16, 4, 0, dt)
        full, kept = m.backward_workspace_size(p), m.backward_kept_workspace_size(p)
        assert 0 <= full - kept - 2 * 300 * 4 * 384 * 4 <= 512, (dt, full, kept)
        assert lib.moe_backward(ctypes.byref(p), fake, fake, fake, ctypes.byref(w), ctypes.byref(r), fake,
                                ctypes.byref(g), fake, None, fake, kept, None) == -3, dt
        assert lib.moe_experts_backward(ctypes.byref(p), 1200, fake, fake, fake, fake, ctypes.byref(w), fake, fake,
                                        ctypes.byref(g), None, None, None, fake, kept, None) == -3, dt
    n = ctypes.c_size_t()
    assert lib.moe_backward_kept_workspace_size(ctypes.byref(m.problem(300, 256, 384, 16, 4, 0, 'f32')),
                                                ctypes.byref(n)) == -2


def test_schedule_noalloc_rejects_without_gpu():
    """moe_schedule_noalloc validates on the host before touching the device: null outputs or a
    null error word are INVALID_ARG; a routing whose histograms exceed the static scratch
    (ceil(T*K / 2048) * E > 2^19) is UNSUPPORTED."""
    import mixture_experts_layer_norm_amd as m
    lib = m._lib
    fake = 1 << 20
    p = m.problem(64, 128, 128, 8, 2, 0, 'bf16')
    assert lib.moe_schedule_noalloc(ctypes.byref(p), fake, fake, fake, fake, fake, None, None) == -1
    assert lib.moe_schedule_noalloc(ctypes.byref(p), None, fake, fake, fake, fake, fake, None) == -1
    big = m.problem(1 << 18, 128, 128, 1024, 8, 0, 'bf16')        # 2^21 routes, 1024 experts
    assert lib.moe_schedule_noalloc(ctypes.byref(big), fake, fake, fake, fake, fake, fake, None) == -2


def test_forward_lanes_rejects_without_gpu():
    """moe_forward_lanes validates its lanes on the host before any HIP call: NULL lanes, a lane
    count outside [1, MOE_MAX_LANES - 1], a NULL stream or any NULL among the S + 1 + count
    events is MOE_ERR_INVALID_ARG; the chunked path's own refusals (fp32, fused gather) stay."""
    import mixture_experts_layer_norm_amd as m
    lib = m._lib
    fake = 1 << 20
    w, r = m.Weights(), m.Routing()
    for f in ('w_gate', 'w_up', 'w_down'):
        setattr(w, f, fake)
    for f in ('topk_idx', 'topk_w', 'counts', 'offsets', 'perm', 'inv_perm'):
        setattr(r, f, fake)

    def call(p, count, streams, events):
        sarr = (ctypes.c_void_p * max(1, len(streams)))(*streams)
        earr = (ctypes.c_void_p * max(1, len(events)))(*events)
        lanes = m.Lanes(count, ctypes.cast(sarr, ctypes.POINTER(ctypes.c_void_p)),
                        ctypes.cast(earr, ctypes.POINTER(ctypes.c_void_p)))
        return lib.moe_forward_lanes(ctypes.byref(p), fake, fake, ctypes.byref(w), fake, ctypes.byref(r), None, None,
                                     fake, 1 << 40, None, ctypes.byref(lanes))

    p = m.problem(64, 128, 128, 8, 2, 0, 'bf16', 256, 3)
    assert lib.moe_forward_lanes(ctypes.byref(p), fake, fake, ctypes.byref(w), fake, ctypes.byref(r), None, None,
                                 fake, 1 << 40, None, None) == -1
    ev = [fake] * m.lane_event_count(p, 3)
    assert m.lane_event_count(p, 1) == 5
    for count in (0, -1, m.MOE_MAX_LANES):
        assert call(p, count, [fake] * 4, ev + [fake]) == -1, count
    assert call(p, 2, [fake, None], ev) == -1
    for hole in range(m.lane_event_count(p, 2)):
        e = list(ev)
        e[hole] = None
        assert call(p, 2, [fake, fake], e) == -1, hole
    p5 = m.problem(64, 128, 128, 8, 2, 0, 'bf16', 256, 5)   # S = 5: 5 + 1 + 1 events
    assert call(p5, 1, [fake], [fake] * 6 + [None]) == -1
    for f in ('sc_gate', 'sc_up', 'sc_down'):
        setattr(w, f, fake)
    q = m.problem(64, 128, 128, 8, 2, 0, 'f32', 256, 3)
    assert call(q, 1, [fake], [fake] * 5) == -2
