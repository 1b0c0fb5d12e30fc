"""Python binding of libmoe.so, the MI355X (gfx950) MoE layer library.

Argument marshalling only: every step runs in the HIP kernels of libmoe.so. Function names
match the C ABI in include/moe.h. Tensors are torch tensors on the current HIP device (torch is
used for device memory and streams); they are passed as raw device pointers. A nonzero status
raises MoeError. Importing this module fails loudly when libmoe.so has not been built.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, 'libmoe.so')

if not os.path.exists(LIB_PATH):
    raise ImportError(f'{LIB_PATH} is missing: build it with `python mixture_experts_layer_norm_amd/build.py` '
                      '(the library has no fallback path)')

# torch first: libmoe.so's libamdhip64.so.7 then resolves to the HIP runtime torch has loaded.
# Loaded the other way round, the process would hold two HIP runtimes and torch's device
# pointers and streams would be invalid in the library (every launch fails).
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

MOE_F32, MOE_BF16, MOE_MXFP8 = 0, 1, 2
MOE_FLAG_FUSED_GATHER = 0x1
MOE_FLAG_PERSISTENT = 0x4
MOE_FLAG_BWD_DGRAD_ONE_PASS = 0x40
MOE_FLAG_BWD_WGRAD_LO_MXFP8 = 0x80
MOE_FLAG_PERSISTENT_GEMM = 0x10000
MOE_FLAG_CU_BUDGET = 0x20000
MOE_FLAG_ROUTER_BWD_DENSE = 0x80000
MOE_FLAG_DISPATCH_COPY = 0x100000
MOE_WS_CU_BUDGET_OFFSET = 4
MOE_FLAG_CU_BUDGET_INDIRECT = 0x200000
MOE_WS_CU_BUDGET_PTR_OFFSET = 8
MOE_MAX_LANES = 4
STATUS = {0: 'MOE_OK', -1: 'MOE_ERR_INVALID_ARG', -2: 'MOE_ERR_UNSUPPORTED', -3: 'MOE_ERR_WORKSPACE',
          -4: 'MOE_ERR_MISALIGNED', -5: 'MOE_ERR_HIP'}
DTYPES = {'f32': MOE_F32, 'bf16': MOE_BF16, 'mxfp8': MOE_MXFP8}

EXPORTED = ('moe_status_string', 'moe_workspace_size', 'moe_route_topk', 'moe_schedule', 'moe_dispatch',
            'moe_dispatch_tokens',
            'moe_combine', 'moe_forward', 'moe_backward', 'moe_experts_forward', 'moe_experts_backward',
            'moe_experts_forward_keep', 'moe_experts_backward_kept', 'moe_forward_keep', 'moe_backward_kept',
            'moe_quantize_mx', 'moe_forward_stages', 'moe_backward_workspace_size', 'moe_pull_schedule',
            'moe_pull_schedule_workspace_size', 'moe_route_gemm', 'moe_route_gemm_workspace_size',
            'moe_backward_kept_workspace_size', 'moe_schedule_noalloc', 'moe_route_gemm_backward',
            'moe_forward_lanes')
STAGES = ('route', 'schedule', 'shared', 'dispatch', 'up_gate', 'down', 'combine')


class MoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f'{where} failed: {STATUS.get(status, status)}')


class Problem(ctypes.Structure):
    _fields_ = [('T', ctypes.c_int32), ('D', ctypes.c_int32), ('I', ctypes.c_int32), ('E', ctypes.c_int32),
                ('K', ctypes.c_int32), ('I_shared', ctypes.c_int32), ('dtype', ctypes.c_int32),
                ('chunk_rows', ctypes.c_int32), ('ring_stages', ctypes.c_int32), ('flags', ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ('w_gate', 'w_up', 'w_down', 'ws_gate', 'ws_up', 'ws_down',
                                                'sc_gate', 'sc_up', 'sc_down')]


class Routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ('topk_idx', 'topk_w', 'counts', 'offsets', 'perm', 'inv_perm')]


class Lanes(ctypes.Structure):
    _fields_ = [('count', ctypes.c_int32), ('streams', ctypes.POINTER(ctypes.c_void_p)),
                ('events', ctypes.POINTER(ctypes.c_void_p))]


class Grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ('dw_gate', 'dw_up', 'dw_down', 'dws_gate', 'dws_up', 'dws_down')]


_P = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t
_PP = ctypes.POINTER(Problem)
_sig = {
    'moe_status_string': (ctypes.c_char_p, [ctypes.c_int]),
    'moe_workspace_size': (ctypes.c_int, [_PP, ctypes.POINTER(_sz)]),
    'moe_backward_workspace_size': (ctypes.c_int, [_PP, ctypes.POINTER(_sz)]),
    'moe_backward_kept_workspace_size': (ctypes.c_int, [_PP, ctypes.POINTER(_sz)]),
    'moe_route_topk': (ctypes.c_int, [_PP, _P, _P, _P, _P]),
    'moe_schedule': (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _sz, _P]),
    'moe_schedule_noalloc': (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _P]),
    'moe_dispatch': (ctypes.c_int, [_PP, _P, _P, _i64, _i64, _P, _P, _P]),
    'moe_dispatch_tokens': (ctypes.c_int, [_PP, _P, _P, _P, _P, _P]),
    'moe_combine': (ctypes.c_int, [_PP, _P, _P, _P, _P, _P]),
    'moe_forward': (ctypes.c_int, [_PP, _P, _P, ctypes.POINTER(Weights), _P, ctypes.POINTER(Routing), _P, _P,
                                   _P, _sz, _P]),
    'moe_backward': (ctypes.c_int, [_PP, _P, _P, _P, ctypes.POINTER(Weights), ctypes.POINTER(Routing), _P,
                                    ctypes.POINTER(Grads), _P, _P, _P, _sz, _P]),
    'moe_forward_keep': (ctypes.c_int, [_PP, _P, _P, ctypes.POINTER(Weights), _P, ctypes.POINTER(Routing), _P, _P,
                                        _P, _P, _P, _sz, _P]),
    'moe_backward_kept': (ctypes.c_int, [_PP, _P, _P, _P, ctypes.POINTER(Weights), ctypes.POINTER(Routing), _P,
                                         ctypes.POINTER(Grads), _P, _P, _P, _P, _P, _sz, _P]),
    'moe_experts_forward': (ctypes.c_int, [_PP, _i64, _P, _P, ctypes.POINTER(Weights), _P, _P, _P, _P, _sz, _P]),
    'moe_experts_backward': (ctypes.c_int, [_PP, _i64, _P, _P, _P, _P, ctypes.POINTER(Weights), _P, _P,
                                            ctypes.POINTER(Grads), _P, _P, _P, _P, _sz, _P]),
    'moe_experts_forward_keep': (ctypes.c_int, [_PP, _i64, _P, _P, ctypes.POINTER(Weights), _P, _P, _P, _P, _P, _P,
                                                _P, _P, _sz, _P]),
    'moe_experts_backward_kept': (ctypes.c_int, [_PP, _i64, _P, _P, _P, _P, ctypes.POINTER(Weights), _P, _P,
                                                 ctypes.POINTER(Grads), _P, _P, _P, _P, _P, _P, _P, _P, _sz, _P]),
    'moe_quantize_mx': (ctypes.c_int, [_P, _i64, _i32, _P, _P, _P]),
    'moe_route_gemm': (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P, _sz, _P]),
    'moe_route_gemm_workspace_size': (ctypes.c_int, [_PP, ctypes.POINTER(ctypes.c_size_t)]),
    'moe_route_gemm_backward': (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, _P]),
    'moe_pull_schedule': (ctypes.c_int, [_i32, _i32, _i32, _i32, _i32, _P, _P, _P, _P, _P, _P, _P, _P, _sz, _P]),
    'moe_pull_schedule_workspace_size': (ctypes.c_int, [_i32, _i32, _i32, _i32, ctypes.POINTER(ctypes.c_size_t)]),
    'moe_forward_stages': (ctypes.c_int, [_PP, _P, _P, ctypes.POINTER(Weights), _P, ctypes.POINTER(Routing), _P,
                                          _P, _P, _sz, _P, _P]),
    'moe_forward_lanes': (ctypes.c_int, [_PP, _P, _P, ctypes.POINTER(Weights), _P, ctypes.POINTER(Routing), _P,
                                         _P, _P, _sz, _P, ctypes.POINTER(Lanes)]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def problem(T, D, I, E, K, I_shared=0, dtype='bf16', chunk_rows=0, ring_stages=0, flags=0) -> Problem:
    return Problem(T, D, I, E, K, I_shared, DTYPES.get(dtype, dtype), chunk_rows, ring_stages, flags)


def _ptr(t):
    """Device pointer of a tensor (or None -> NULL)."""
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(st, where):
    if st != 0:
        raise MoeError(st, where)


def status_string(st) -> str:
    return _lib.moe_status_string(st).decode()


def workspace_size(p: Problem) -> int:
    n = _sz(0)
    _check(_lib.moe_workspace_size(ctypes.byref(p), ctypes.byref(n)), 'moe_workspace_size')
    return n.value


def backward_workspace_size(p: Problem) -> int:
    n = _sz(0)
    _check(_lib.moe_backward_workspace_size(ctypes.byref(p), ctypes.byref(n)), 'moe_backward_workspace_size')
    return n.value


def backward_kept_workspace_size(p: Problem) -> int:
    n = ctypes.c_size_t()
    _check(_lib.moe_backward_kept_workspace_size(ctypes.byref(p), ctypes.byref(n)), 'moe_backward_kept_workspace_size')
    return n.value


def route_topk(p, logits, topk_idx, topk_w, stream=None):
    _check(_lib.moe_route_topk(ctypes.byref(p), _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _stream(stream)),
           'moe_route_topk')


def schedule(p, topk_idx, counts, offsets, perm, inv_perm, ws, stream=None):
    _check(_lib.moe_schedule(ctypes.byref(p), _ptr(topk_idx), _ptr(counts), _ptr(offsets), _ptr(perm),
                             _ptr(inv_perm), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           'moe_schedule')


def schedule_noalloc(p, topk_idx, counts, offsets, perm, inv_perm, error_word, stream=None):
    _check(_lib.moe_schedule_noalloc(ctypes.byref(p), _ptr(topk_idx), _ptr(counts), _ptr(offsets), _ptr(perm),
                                     _ptr(inv_perm), _ptr(error_word), _stream(stream)), 'moe_schedule_noalloc')


def dispatch(p, x, perm, slot_begin, slot_count, x_slot, x_slot_scales=None, stream=None):
    _check(_lib.moe_dispatch(ctypes.byref(p), _ptr(x), _ptr(perm), slot_begin, slot_count, _ptr(x_slot),
                             _ptr(x_slot_scales), _stream(stream)), 'moe_dispatch')


def dispatch_tokens(p, x, inv_perm, x_slot, x_slot_scales=None, stream=None):
    _check(_lib.moe_dispatch_tokens(ctypes.byref(p), _ptr(x), _ptr(inv_perm), _ptr(x_slot), _ptr(x_slot_scales),
                                    _stream(stream)), 'moe_dispatch_tokens')


def combine(p, y_routes, shared_out, topk_w, out, stream=None):
    _check(_lib.moe_combine(ctypes.byref(p), _ptr(y_routes), _ptr(shared_out), _ptr(topk_w), _ptr(out),
                            _stream(stream)), 'moe_combine')


def make_weights(w_gate, w_up, w_down, ws_gate=None, ws_up=None, ws_down=None, sc_gate=None, sc_up=None,
                 sc_down=None) -> Weights:
    return Weights(*(_ptr(t) for t in (w_gate, w_up, w_down, ws_gate, ws_up, ws_down, sc_gate, sc_up, sc_down)))


def make_routing(topk_idx, topk_w, counts, offsets, perm, inv_perm) -> Routing:
    return Routing(*(_ptr(t) for t in (topk_idx, topk_w, counts, offsets, perm, inv_perm)))


def make_grads(dw_gate, dw_up, dw_down, dws_gate=None, dws_up=None, dws_down=None) -> Grads:
    return Grads(*(_ptr(t) for t in (dw_gate, dw_up, dw_down, dws_gate, dws_up, dws_down)))


def forward(p, x, logits, weights: Weights, out, routing: Routing, ws, y_routes=None, shared_out=None,
            stream=None):
    _check(_lib.moe_forward(ctypes.byref(p), _ptr(x), _ptr(logits), ctypes.byref(weights), _ptr(out),
                            ctypes.byref(routing), _ptr(y_routes), _ptr(shared_out), _ptr(ws),
                            ws.numel() * ws.element_size(), _stream(stream)), 'moe_forward')


def forward_stages(p, x, logits, weights: Weights, out, routing: Routing, ws, events, y_routes=None,
                   shared_out=None, stream=None):
    """moe_forward with per-stage HIP events: `events` is a sequence of len(STAGES) + 1
    torch.cuda.Event(enable_timing=True) objects, recorded on the library's stream."""
    handles = [e.cuda_event for e in events]
    if len(handles) != len(STAGES) + 1 or not all(handles):
        raise ValueError('forward_stages needs len(STAGES) + 1 created events (record each once first)')
    arr = (ctypes.c_void_p * len(handles))(*handles)
    _check(_lib.moe_forward_stages(ctypes.byref(p), _ptr(x), _ptr(logits), ctypes.byref(weights), _ptr(out),
                                   ctypes.byref(routing), _ptr(y_routes), _ptr(shared_out), _ptr(ws),
                                   ws.numel() * ws.element_size(), arr, _stream(stream)), 'moe_forward_stages')


def lane_event_count(p, lanes):
    """Events moe_forward_lanes needs with `lanes` extra streams: ring depth + 1 + lanes."""
    return (p.ring_stages or 3) + 1 + lanes


def forward_lanes(p, x, logits, weights: Weights, out, routing: Routing, ws, streams, events, y_routes=None,
                  shared_out=None, stream=None):
    """moe_forward with the routed chunks spread over `stream` and the torch streams `streams`
    (1 .. MOE_MAX_LANES - 1 of them); `events` holds lane_event_count(p, len(streams))
    torch.cuda.Event objects, each recorded once so that it exists."""
    sh = [s.cuda_stream for s in streams]
    ev = [e.cuda_event for e in events]
    if not all(sh) or not all(ev):
        raise ValueError('forward_lanes needs created streams and events (record each event once first)')
    sarr = (ctypes.c_void_p * max(1, len(sh)))(*sh)
    earr = (ctypes.c_void_p * max(1, len(ev)))(*ev)
    if len(ev) < lane_event_count(p, len(sh)):
        raise ValueError(f'forward_lanes needs {lane_event_count(p, len(sh))} events')
    lanes = Lanes(len(sh), ctypes.cast(sarr, ctypes.POINTER(ctypes.c_void_p)), ctypes.cast(earr, ctypes.POINTER(ctypes.c_void_p)))
    _check(_lib.moe_forward_lanes(ctypes.byref(p), _ptr(x), _ptr(logits), ctypes.byref(weights), _ptr(out),
                                  ctypes.byref(routing), _ptr(y_routes), _ptr(shared_out), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream), ctypes.byref(lanes)),
           'moe_forward_lanes')


def backward(p, dout, x, logits, weights: Weights, routing: Routing, dx, grads: Grads, d_topk_w, d_logits, ws,
             stream=None):
    _check(_lib.moe_backward(ctypes.byref(p), _ptr(dout), _ptr(x), _ptr(logits), ctypes.byref(weights),
                             ctypes.byref(routing), _ptr(dx), ctypes.byref(grads), _ptr(d_topk_w), _ptr(d_logits),
                             _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), 'moe_backward')


def forward_keep(p, x, logits, weights: Weights, out, routing: Routing, act_a, act_u, ws, y_routes=None,
                 shared_out=None, stream=None):
    _check(_lib.moe_forward_keep(ctypes.byref(p), _ptr(x), _ptr(logits), ctypes.byref(weights), _ptr(out),
                                 ctypes.byref(routing), _ptr(y_routes), _ptr(shared_out), _ptr(act_a), _ptr(act_u),
                                 _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), 'moe_forward_keep')


def backward_kept(p, dout, x, logits, weights: Weights, routing: Routing, dx, grads: Grads, d_topk_w, d_logits,
                  act_a, act_u, ws, stream=None):
    _check(_lib.moe_backward_kept(ctypes.byref(p), _ptr(dout), _ptr(x), _ptr(logits), ctypes.byref(weights),
                                  ctypes.byref(routing), _ptr(dx), ctypes.byref(grads), _ptr(d_topk_w),
                                  _ptr(d_logits), _ptr(act_a), _ptr(act_u), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)), 'moe_backward_kept')


def experts_forward(p, slots, x_slot, offsets, weights: Weights, y_slot, x_local, shared_out, ws, stream=None):
    _check(_lib.moe_experts_forward(ctypes.byref(p), slots, _ptr(x_slot), _ptr(offsets), ctypes.byref(weights),
                                    _ptr(y_slot), _ptr(x_local), _ptr(shared_out), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)), 'moe_experts_forward')


def experts_backward(p, slots, x_slot, offsets, g_slot, dy_slot, weights: Weights, dx_slot, dg_slot, grads: Grads,
                     x_local, dy_local, dx_local, ws, stream=None):
    _check(_lib.moe_experts_backward(ctypes.byref(p), slots, _ptr(x_slot), _ptr(offsets), _ptr(g_slot),
                                     _ptr(dy_slot), ctypes.byref(weights), _ptr(dx_slot), _ptr(dg_slot),
                                     ctypes.byref(grads), _ptr(x_local), _ptr(dy_local), _ptr(dx_local), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)), 'moe_experts_backward')


def experts_forward_keep(p, slots, x_slot, offsets, weights: Weights, y_slot, x_local, shared_out, act_a, act_u,
                         shared_act_a, shared_act_u, ws, stream=None):
    _check(_lib.moe_experts_forward_keep(ctypes.byref(p), slots, _ptr(x_slot), _ptr(offsets), ctypes.byref(weights),
                                         _ptr(y_slot), _ptr(x_local), _ptr(shared_out), _ptr(act_a), _ptr(act_u),
                                         _ptr(shared_act_a), _ptr(shared_act_u), _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream(stream)), 'moe_experts_forward_keep')


def experts_backward_kept(p, slots, x_slot, offsets, g_slot, dy_slot, weights: Weights, dx_slot, dg_slot,
                          grads: Grads, x_local, dy_local, dx_local, act_a, act_u, shared_act_a, shared_act_u, ws,
                          stream=None):
    _check(_lib.moe_experts_backward_kept(ctypes.byref(p), slots, _ptr(x_slot), _ptr(offsets), _ptr(g_slot),
                                          _ptr(dy_slot), ctypes.byref(weights), _ptr(dx_slot), _ptr(dg_slot),
                                          ctypes.byref(grads), _ptr(x_local), _ptr(dy_local), _ptr(dx_local),
                                          _ptr(act_a), _ptr(act_u), _ptr(shared_act_a), _ptr(shared_act_u), _ptr(ws),
                                          ws.numel() * ws.element_size(), _stream(stream)),
           'moe_experts_backward_kept')


def quantize_mx(src_bf16, q, scales, stream=None):
    rows, cols = src_bf16.shape[0], src_bf16.shape[-1]
    rows = src_bf16.numel() // cols
    _check(_lib.moe_quantize_mx(_ptr(src_bf16), rows, cols, _ptr(q), _ptr(scales), _stream(stream)),
           'moe_quantize_mx')


def pull_schedule_workspace_size(R: int, N: int, K: int, L: int) -> int:
    n = _sz(0)
    _check(_lib.moe_pull_schedule_workspace_size(R, N, K, L, ctypes.byref(n)), 'moe_pull_schedule_workspace_size')
    return n.value


def pull_schedule(routing, rank, L, counts, src_counts, offsets, phi_src, phi_idx, ws, route_pos=None, stream=None):
    """routing: int32 [R, N, K] device tensor of global expert ids."""
    R, N, K = routing.shape
    _check(_lib.moe_pull_schedule(R, N, K, L, rank, _ptr(routing), _ptr(counts), _ptr(src_counts), _ptr(offsets),
                                  _ptr(phi_src), _ptr(phi_idx), _ptr(route_pos), _ptr(ws), ws.numel(),
                                  _stream(stream)), 'moe_pull_schedule')


def route_gemm_workspace_size(p: Problem) -> int:
    n = _sz(0)
    _check(_lib.moe_route_gemm_workspace_size(ctypes.byref(p), ctypes.byref(n)), 'moe_route_gemm_workspace_size')
    return n.value


def route_gemm(p, x, w_router, logits, topk_idx, topk_w, ws, stream=None):
    _check(_lib.moe_route_gemm(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(logits), _ptr(topk_idx), _ptr(topk_w),
                               _ptr(ws), ws.numel(), _stream(stream)), 'moe_route_gemm')


def route_gemm_backward(p, x, w_router, d_logits, dw_router, dx=None, stream=None):
    _check(_lib.moe_route_gemm_backward(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(d_logits), _ptr(dw_router),
                                        _ptr(dx), _stream(stream)), 'moe_route_gemm_backward')
