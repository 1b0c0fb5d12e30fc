#!/usr/bin/env python3
"""Throughput of the MoE layer hot path on one MI355X (gfx950).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3|mid|tiny]

A step is one moe_forward of the whole layer (routing, schedule, shared expert, dispatch, routed
grouped GEMMs with the SwiGLU and scatter epilogues, combine) on one batch of seeded synthetic
inputs already resident in HBM. W untimed steps, then K steps timed with HIP events on the
library's stream between two device synchronisations. Prints ONE JSON line.

The default workload is the DeepSeek-V3-shape BF16 forward: T=8192 tokens, D=7168, I=2048,
256 routed experts top-8 plus one shared expert (I=2048), router logits with a per-expert bias.

`roofline` covers the kernel with the largest device time per step, with its algorithmic bytes
and FLOPs per launch; `cpu_baseline` times the fp64 CPU oracle on a bounded sample of tokens of
the same workload (rank 0, one GPU only).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0       # MI355X dense BF16 MFMA, TFLOP/s
PEAK_MXFP8_TFLOPS = 5000.0      # MI355X dense FP8 (MX block-scaled) MFMA, TFLOP/s
PEAK_F32_TFLOPS = 157.3         # fp32 vector
PEAK_HBM_GBS = 8000.0           # HBM3E, GB/s
METRIC = 'MoE layer tokens/s (fwd, fwd+bwd) on 1 MI355X; % of MFMA peak'

# HBM traffic of the dominant kernel is read from its rocprofv3 counter summary, and only while the
# kernel sources are the ones the counters were taken on (hash recorded in the summary).
# the GEMM kernels and the host code that chooses their operands (gathered or copied rows) and forms
GEMM_SOURCES = ('mixture_experts_layer_norm_amd/csrc/gemm_tile.h', 'mixture_experts_layer_norm_amd/csrc/gemm.hip',
                'mixture_experts_layer_norm_amd/csrc/api.hip')
TRAFFIC_SUMMARY = {'up_gate': 'profiles/gemm_swiglu_routed_dsv3_T8192_hbm_traffic.md',
                   'down': 'profiles/gemm_down_routed_dsv3_T8192_hbm_traffic.md'}


def gemm_sources_hash():
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), 'rb') as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def routed_gemm_kernel(cfg, ntn, flags):
    """Which kernel the library launches for a routed BF16 GEMM with ntn n-tiles: the persistent
    one where the launch's upper bound of tiles is at least 12 per workgroup (one workgroup per CU),
    or with MOE_FLAG_PERSISTENT_GEMM; the per-tile one otherwise (the library's own rule)."""
    import torch
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    mt = (cfg.T * cfg.K + 255) // 256 + cfg.E
    nb = (mt * ntn + 7) // 8 * 8
    nw = min(max(ncu, 8) // 8 * 8, nb)
    return 'gemm_bf16_persistent_kernel' if (flags & 0x10000) or nb >= 12 * nw else 'gemm_bf16_kernel'


def measured_traffic(stage, flags, workload):
    """HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE) for `stage`, or None when no
    summary matches the current kernel sources, flags and workload."""
    rel = TRAFFIC_SUMMARY.get(stage)
    if rel is None or not os.path.exists(os.path.join(ROOT, rel)):
        return None
    kv = {}
    with open(os.path.join(ROOT, rel)) as f:
        for line in f:
            if line.startswith('- ') and ': ' in line:
                k, v = line[2:].split(': ', 1)
                kv[k.strip()] = v.strip().strip('`')
    try:
        if (kv.get('sources_sha256_16') != gemm_sources_hash() or int(kv.get('flags', -1)) != flags
                or kv.get('workload') != workload):
            return None
        return float(kv['traffic_bytes_per_launch'])
    except (KeyError, ValueError):
        return None


def stage_work(cfg, flags):
    """Algorithmic FLOPs and HBM bytes per launch of each forward stage."""
    T, D, I, E, K, Is = cfg.T, cfg.D, cfg.I, cfg.E, cfg.K, cfg.I_shared
    n = T * K
    b = 4 if cfg.dtype == 'f32' else 2
    fused = not (flags & 0x100000)   # GEMM1 reads x through the schedule unless the slot copy is asked for
    w = {}
    if cfg.dtype == 'mxfp8':
        # routed operands E4M3 (1 byte) + one E8M0 byte per 32; activations in, outputs BF16
        q = 1 + 1 / 32
        w['route'] = (0.0, T * cfg.E * 4 + T * K * 8)
        w['schedule'] = (0.0, n * 4 * 3)
        w['shared'] = (6.0 * T * D * Is, 3 * Is * D * 2 + 2 * T * D * 2 + 2 * T * Is * 2) if Is else (0.0, 0)
        # gathered (default): the T token rows quantised once, read by GEMM1 through the schedule
        w['dispatch'] = (0.0, T * D * 2 + (T * D * q if fused else n * D * q + n * 4))
        w['up_gate'] = (4.0 * n * D * I, 2 * E * I * D * q + (T if fused else n) * D * q + n * I * q)
        w['down'] = (2.0 * n * I * D, E * D * I * q + n * I * q + n * D * 2 + n * 4)
        w['combine'] = (0.0, n * D * 2 + (2 if Is else 1) * T * D * 2 + n * 4)
        return w
    w['route'] = (0.0, T * cfg.E * 4 + T * K * 8)
    w['schedule'] = (0.0, n * 4 * 3)
    w['shared'] = (6.0 * T * D * Is, 3 * Is * D * b + 2 * T * D * b + 2 * T * Is * b) if Is else (0.0, 0)
    w['dispatch'] = (0.0, 0 if fused else T * D * b + n * D * b + n * 4)
    w['up_gate'] = (4.0 * n * D * I, 2 * E * I * D * b + (T if fused else n) * D * b + n * I * b)
    w['down'] = (2.0 * n * I * D, E * D * I * b + n * I * b + n * D * b + n * 4)
    w['combine'] = (0.0, n * D * b + (2 if Is else 1) * T * D * b + n * 4)
    return w


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument('--gpus', type=int, default=1)
    ap.add_argument('--steps', type=int, default=50)
    ap.add_argument('--warmup', type=int, default=10)
    ap.add_argument('--workload', default='dsv3',
                    choices=['dsv3', 'mid', 'tiny', 'mxfp8', 'ep_share', 'ep_share_mxfp8', 'dsv3_layer'],
                    help='dsv3_layer: the DSV3-shape layer forward + backward as the step')
    ap.add_argument('--no-extra', action='store_true',
                    help='skip the expert-parallel share forward+backward reported under "extra"')
    ap.add_argument('--chunk-rows', type=int, default=0)
    ap.add_argument('--ring-stages', type=int, default=0, help='ring depth of the chunked path (0: 3)')
    ap.add_argument('--lanes', type=int, default=0,
                    help='extra streams for the chunked forward (moe_forward_lanes); 0: moe_forward')
    ap.add_argument('--flags', type=int, default=0)
    ap.add_argument('--keep-activations', action='store_true',
                    help='ep_share workloads: hand a, u from the forward to the backward instead of replaying')
    ap.add_argument('--no-cpu-baseline', action='store_true')
    ap.add_argument('--cpu-tokens', type=int, default=160, help='tokens in the CPU oracle sample')
    ap.add_argument('--calib-copy', action='store_true',
                    help='run one 1 GiB device-to-device copy before the timed region (HBM counter calibration)')
    args = ap.parse_args()
    if args.gpus != 1:
        print(f'bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU '
              'path: the expert-parallel sharding is described in DESIGN.md, not implemented.', file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import mixture_experts_layer_norm_amd as moe

    if args.workload in ('ep_share', 'ep_share_mxfp8'):
        dt = 'mxfp8' if args.workload == 'ep_share_mxfp8' else 'bf16'
        if args.calib_copy:
            calib_copy()
        print(json.dumps(bench_share(args.steps, args.warmup, args.flags, dt, keep=args.keep_activations)), flush=True)
        return
    if args.workload == 'dsv3_layer':
        torch.cuda.set_device(0)
        r = layer_fwd_bwd_leg(synth.DSV3, synth.device_layer(synth.DSV3), args.keep_activations, args.steps, args.warmup)
        print(json.dumps({'metric': METRIC, 'n_gpus': 1, 'higher_is_better': True, 'scaling': 'weak', 'dtype': 'bf16',
                          'data': 'synthetic', 'config': {'workload': r.pop('workload')}, **r}), flush=True)
        return
    cfg = {'dsv3': synth.DSV3, 'mid': synth.MID, 'tiny': synth.TINY, 'mxfp8': synth.MXFP8}[args.workload]
    torch.cuda.set_device(0)
    lane_streams_first()
    F = make_forward(cfg, args.chunk_rows, args.flags, args.ring_stages)
    L, p, weights, routing_t, routing, out, ws = F['L'], F['p'], F['weights'], F['routing_t'], F['routing'], F['out'], F['ws']
    T, D, K = cfg.T, cfg.D, cfg.K
    dev = 'cuda'
    stream = torch.cuda.current_stream()
    nst = len(moe.STAGES)

    lane_streams = LANE_STREAMS[:args.lanes]
    lane_events = [torch.cuda.Event() for _ in range(moe.lane_event_count(p, args.lanes) if args.lanes else 0)]
    for e in lane_events:
        e.record(stream)          # creates the HIP event

    def step(events=None):
        if events is None and args.lanes:
            moe.forward_lanes(p, L.x, L.logits, weights, out, routing, ws, lane_streams, lane_events, stream=stream)
        elif events is None:
            moe.forward(p, L.x, L.logits, weights, out, routing, ws, stream=stream)
        else:
            moe.forward_stages(p, L.x, L.logits, weights, out, routing, ws, events, stream=stream)

    if args.calib_copy:
        calib_copy()
    print(f'[bench] warmup {args.warmup}', file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps of moe_forward (every stage in order on this stream), bracketed by
    # device synchronisations
    n_attr = min(args.steps, 20)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(n_attr)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    for e in [t_start, t_end] + [e for row in evs for e in row]:
        e.record(stream)          # torch creates the HIP event on first record
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    # stage attribution: the same forward with HIP events between its stages (stages in order on the
    # library's stream, no overlap), outside the timed region
    for i in range(n_attr):
        step(evs[i])
    torch.cuda.synchronize()
    stage_ms = {s: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(n_attr)]))
                for j, s in enumerate(moe.STAGES)}
    print(f'[bench] {args.steps} steps: {ms_per_step:.3f} ms/step (wall {1e3 * wall / args.steps:.3f}); '
          f'stages {json.dumps({k: round(v, 4) for k, v in stage_ms.items()})}', file=sys.stderr, flush=True)

    n = T * K
    flops = 6.0 * n * cfg.D * cfg.I + 6.0 * T * cfg.D * cfg.I_shared
    peak = {'f32': PEAK_F32_TFLOPS, 'mxfp8': PEAK_MXFP8_TFLOPS}.get(cfg.dtype, PEAK_BF16_TFLOPS)
    tflops = flops / (ms_per_step * 1e-3) / 1e12

    work = stage_work(cfg, args.flags)   # chunks too read x through the schedule unless copies are asked for
    dom = max(stage_ms, key=stage_ms.get)
    f_dom, b_dom = work[dom]
    t_dom = stage_ms[dom] * 1e-3
    t_mfma = f_dom / (peak * 1e12)
    t_hbm = b_dom / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm:
        roof = {'bound': 'mfma', 'achieved': f_dom / t_dom / 1e12, 'peak': peak, 'unit': 'TFLOP/s'}
    else:
        roof = {'bound': 'hbm', 'achieved': b_dom / t_dom / 1e9, 'peak': PEAK_HBM_GBS, 'unit': 'GB/s'}
    roof['frac'] = roof['achieved'] / roof['peak']
    roof['traffic'] = measured_traffic(dom, args.flags, cfg.name)
    gk = {'mxfp8': 'gemm_mx_kernel', 'f32': 'gemm_f32_kernel'}.get(cfg.dtype, 'gemm_bf16_kernel')
    gku = gkd = gk
    if cfg.dtype == 'bf16' and not args.chunk_rows:
        gku = routed_gemm_kernel(cfg, cfg.I // 128, args.flags)
        gkd = routed_gemm_kernel(cfg, (cfg.D + 255) // 256, args.flags)
    roof['kernel'] = {'up_gate': f'{gku}<EPI_SWIGLU> (routed W_gate/W_up + SwiGLU)',
                      'down': f'{gkd}<EPI_STORE> (routed W_down + scatter)',
                      'shared': 'shared expert GEMMs', 'dispatch': 'dispatch_kernel',
                      'combine': 'combine_bf16_kernel', 'route': 'route_topk_kernel',
                      'schedule': 'sched_* kernels'}[dom]
    roof['stage'] = dom
    roof['avg_ms'] = stage_ms[dom]
    roof['algorithmic_flops'] = f_dom
    roof['algorithmic_bytes'] = b_dom
    roof['mfma_frac'] = f_dom / t_dom / 1e12 / peak
    roof['hbm_frac'] = b_dom / t_dom / 1e9 / PEAK_HBM_GBS

    pc = standalone_permute_combine(moe, p, cfg, L, routing_t, out, stream) if cfg.dtype == 'bf16' else None
    yl = None
    if not args.no_extra and args.workload == 'dsv3':
        # the same forward with persistent GEMMs that honour the workgroup budget word
        pb = moe.problem(T, D, cfg.I, cfg.E, K, cfg.I_shared, cfg.dtype, args.chunk_rows, 0,
                         args.flags | moe.MOE_FLAG_PERSISTENT_GEMM | moe.MOE_FLAG_CU_BUDGET)
        wsb = torch.zeros((moe.workspace_size(pb),), dtype=torch.uint8, device=dev)
        word = wsb[moe.MOE_WS_CU_BUDGET_OFFSET:moe.MOE_WS_CU_BUDGET_OFFSET + 4].view(torch.int32)

        def step_b():
            moe.forward(pb, L.x, L.logits, weights, out, routing, wsb, stream=stream)
        # and with the budget word in coherent pinned host memory, stored to by the host
        hip = hip_runtime()
        hw = pinned_host_word(hip)
        host_budget = None
        if hw is not None:
            ph = moe.problem(T, D, cfg.I, cfg.E, K, cfg.I_shared, cfg.dtype, args.chunk_rows, 0,
                             args.flags | moe.MOE_FLAG_PERSISTENT_GEMM | moe.MOE_FLAG_CU_BUDGET |
                             moe.MOE_FLAG_CU_BUDGET_INDIRECT)
            wsh = torch.zeros((moe.workspace_size(ph),), dtype=torch.uint8, device=dev)
            o = moe.MOE_WS_CU_BUDGET_PTR_OFFSET
            wsh[o:o + 8].view(torch.int64).fill_(hw[1])

            def step_h():
                moe.forward(ph, L.x, L.logits, weights, out, routing, wsh, stream=stream)
            host_budget = (step_h, hw[0], 224)
        yl = second_stream_latency(step, stream, budget=(step_b, word, 224), host_budget=host_budget)
        torch.cuda.synchronize()
        if hw is not None:
            del wsh
            hip.hipHostFree(hw[2])
        del wsb

    # per-step spread from the in-order run (sum of its stage events)
    per_step = np.array([evs[i][0].elapsed_time(evs[i][nst]) for i in range(n_attr)])

    cpu = None
    if not args.no_cpu_baseline and cfg.dtype != 'mxfp8':
        cpu = cpu_baseline(cfg, L, args.cpu_tokens)
    extra = None
    if not args.no_extra and args.workload == 'dsv3':
        rg = bench_route_gemm(moe, cfg, L.x, stream)
        chunks = chunk_leg(moe, cfg, L, weights, routing, stream, ms_per_step)
        del weights, ws, out, F
        torch.cuda.empty_cache()
        layer = {'layer_fwd_bwd': layer_fwd_bwd_leg(cfg, L, keep=False),
                 'layer_fwd_bwd_keep_activations': layer_fwd_bwd_leg(cfg, L, keep=True)}
        del L
        torch.cuda.empty_cache()
        extra = {'second_stream_latency': yl, 'chunked_forward': chunks, **layer,
                 'mid_forward': forward_leg(synth.MID, 20), 'mid_chunked_forward': mid_chunk_leg(),
                 'mxfp8_forward': forward_leg(synth.MXFP8, 5),
                 'ep_share_fwd_bwd': bench_share(max(5, args.steps // 5), 2, args.flags),
                 'ep_share_fwd_bwd_keep_activations': bench_share(max(5, args.steps // 5), 2, args.flags,
                                                                  keep=True),
                 'ep_share_fwd_bwd_dgrad_one_pass': bench_share(max(5, args.steps // 5), 2, args.flags | 0x40),
                 'ep_share_fwd_bwd_one_pass_lo_mxfp8': bench_share(max(5, args.steps // 5), 2,
                                                                  args.flags | 0x40 | 0x80),
                 'ep_share_fwd_bwd_keep_one_pass_lo_mxfp8': bench_share(max(5, args.steps // 5), 2,
                                                                       args.flags | 0x40 | 0x80, keep=True),
                 'ep_share_fwd_bwd_mxfp8': bench_share(max(5, args.steps // 5), 2, args.flags, 'mxfp8'),
                 'ep_share_fwd_bwd_mxfp8_keep_activations': bench_share(max(5, args.steps // 5), 2, args.flags,
                                                                        'mxfp8', keep=True),
                 'pull_schedule_ep8': bench_pull_schedule(moe, stream), 'route_gemm': rg}
        if not args.no_cpu_baseline:
            extra['cpu_baselines'] = cpu_oracle_extra(moe)

    line = {
        'metric': METRIC,
        'value': T / (ms_per_step * 1e-3),
        'unit': 'tokens/s',
        'n_gpus': 1,
        'steps': args.steps,
        'warmup': args.warmup,
        'ms_per_step': ms_per_step,
        'higher_is_better': True,
        'scaling': 'weak',
        'vs_baseline': None,
        'dtype': {'f32': 'f32', 'mxfp8': 'mxfp8 (e4m3 + e8m0 per 32), bf16 out'}.get(cfg.dtype, 'bf16'),
        'data': 'synthetic',
        'config': {'workload': f'{cfg.name} forward', 'T': T, 'D': cfg.D, 'I': cfg.I, 'E': cfg.E, 'K': K,
                   'I_shared': cfg.I_shared, 'router': cfg.router, 'chunk_rows': args.chunk_rows,
                   'ring_stages': args.ring_stages, 'lanes': args.lanes, 'flags': args.flags},
        'tflops': tflops,
        'mfma_peak_frac': tflops / peak,
        'stages_ms': stage_ms,
        'stages_note': 'stage times from a separate in-order run with HIP events between stages (no overlap)',
        'stages_sum_ms': float(sum(stage_ms.values())),
        'in_order_step_ms_p10_p50_p90': [float(np.percentile(per_step, q)) for q in (10, 50, 90)],
        'permute_combine_standalone': pc,
        'wall_ms_per_step': 1e3 * wall / args.steps,
        'roofline': roof,
        'cpu_baseline': cpu,
    }
    if extra is not None:
        line['extra'] = extra
    print(json.dumps(line), flush=True)


def standalone_permute_combine(moe, p, cfg, L, routing_t, out, stream, reps=20):
    """Dispatch and combine timed as standalone kernels on the full-size buffers of the workload
    (the routing of the last forward), against HBM peak with their algorithmic bytes: dispatch
    T*D*2 (x read once) + T*K*D*2 (slots written) + 4*T*K; combine T*K*D*2 + 2*T*D*2 + 4*T*K."""
    import torch
    T, D, K = cfg.T, cfg.D, cfg.K
    n = T * K
    xs = torch.empty((n, D), dtype=torch.bfloat16, device='cuda')
    ys = torch.empty((n, D), dtype=torch.bfloat16, device='cuda').normal_()
    sh = torch.empty((T, D), dtype=torch.bfloat16, device='cuda').normal_()
    res = {}
    for name, fn, nbytes in (
            ('dispatch', lambda: moe.dispatch_tokens(p, L.x, routing_t['inv_perm'], xs, stream=stream),
             T * D * 2 + n * D * 2 + 4 * n),
            ('dispatch_slot_major', lambda: moe.dispatch(p, L.x, routing_t['perm'], 0, n, xs, stream=stream),
             T * D * 2 + n * D * 2 + 4 * n),
            ('combine', lambda: moe.combine(p, ys, sh, routing_t['topk_w'], out, stream=stream),
             n * D * 2 + 2 * T * D * 2 + 4 * n)):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name] = {'ms': ms, 'algorithmic_bytes': nbytes, 'GB_s': nbytes / (ms * 1e-3) / 1e9,
                     'hbm_frac': nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    del xs, ys, sh
    return res


def bench_route_gemm(moe, cfg, x, stream, reps=20):
    """moe_route_gemm at the workload's shape: router GEMM (x [T][D] BF16 times a random
    w_router [E][D]) split along D, plus the top-K; 2*T*D*E FLOP."""
    import torch
    T, D, E, K = cfg.T, cfg.D, cfg.E, cfg.K
    g = torch.Generator(device='cuda')
    g.manual_seed(77)
    w = (torch.randn((E, D), generator=g, device='cuda') / D ** 0.5).to(torch.bfloat16)
    p = moe.problem(T, D, cfg.I, E, K, 0, 'bf16')
    lg = torch.empty((T, E), dtype=torch.float32, device='cuda')
    idx = torch.empty((T, K), dtype=torch.int32, device='cuda')
    gw = torch.empty((T, K), dtype=torch.float32, device='cuda')
    ws = torch.empty((moe.route_gemm_workspace_size(p),), dtype=torch.uint8, device='cuda')

    def fn():
        moe.route_gemm(p, x, w, lg, idx, gw, ws, stream=stream)
    for _ in range(3):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 2.0 * T * D * E
    res = {'workload': f'router GEMM + top-{K}, T={T} D={D} E={E}', 'ms': ms, 'tflops': flops / (ms * 1e-3) / 1e12}
    # its backward: dW_r = d_logits^T x and dx += d_logits W_r, with d_logits nonzero on each
    # token's K chosen experts as the layer backward writes it
    dl = torch.zeros((T, E), dtype=torch.float32, device='cuda')
    dl.scatter_(1, idx.long(), torch.randn((T, K), generator=g, device='cuda'))
    dw = torch.empty((E, D), dtype=torch.float32, device='cuda')
    dx = torch.zeros((T, D), dtype=torch.bfloat16, device='cuda')

    def fb():
        moe.route_gemm_backward(p, x, w, dl, dw, dx, stream=stream)
    for _ in range(2):
        fb()
    e0.record(stream)
    for _ in range(reps // 2):
        fb()
    e1.record(stream)
    torch.cuda.synchronize()
    mb = e0.elapsed_time(e1) / (reps // 2)
    # the kernels skip the zero entries of d_logits: T K nonzeros, 2 D FMAs each; algorithmic bytes
    # read d_logits, x and W_r once, read and write dx, write dW_r
    nnz_flops = 2 * 2.0 * T * K * D
    alg_bytes = T * E * 4 + T * D * 2 + E * D * 2 + 2 * T * D * 2 + E * D * 4
    res['backward'] = {'ms': mb, 'dense_equivalent_tflops': 2 * flops / (mb * 1e-3) / 1e12,
                       'nonzero_tflops': nnz_flops / (mb * 1e-3) / 1e12,
                       'algorithmic_bytes': alg_bytes,
                       'hbm_frac': alg_bytes / (mb * 1e-3) / 1e9 / PEAK_HBM_GBS,
                       'note': 'dW_r = d_logits^T x and dx += d_logits W_r with d_logits nonzero on K of E entries '
                               'per token; fp32 FMA over the nonzero entries only (bitwise the dense sums); '
                               'dense_equivalent_tflops counts the 4 T D E FLOP of the dense products'}
    return res


def bench_pull_schedule(moe, stream, R=8, N=8192, K=8, L=32, reps=20):
    """The R > 1 pull-dispatch schedule (moe_pull_schedule) at the DSV3 routing shape sharded over
    R = 8 ranks: routing [8][8192][8] over E = 256 experts (Gumbel-top-k on a mild Zipf
    popularity), rank 0's table of 32 local experts. Three launches; reported per call."""
    import torch
    E = R * L
    g = torch.Generator(device='cuda')
    g.manual_seed(4242)
    lp = -0.8 * torch.log(torch.arange(1, E + 1, device='cuda', dtype=torch.float32))
    u = torch.rand((R, N, E), generator=g, device='cuda').clamp_(min=1e-30)
    routing = torch.topk(lp - torch.log(-torch.log(u)), K, dim=2).indices.to(torch.int32).contiguous()
    del u
    n = R * N * K
    dev = 'cuda'
    counts = torch.empty((L,), dtype=torch.int32, device=dev)
    src = torch.empty((L, R), dtype=torch.int32, device=dev)
    offs = torch.empty((L + 1,), dtype=torch.int32, device=dev)
    phs = torch.empty((n,), dtype=torch.int32, device=dev)
    phi = torch.empty((n,), dtype=torch.int32, device=dev)
    pos = torch.empty((n,), dtype=torch.int32, device=dev)
    ws = torch.zeros((moe.pull_schedule_workspace_size(R, N, K, L),), dtype=torch.uint8, device=dev)

    def fn():
        moe.pull_schedule(routing, 0, L, counts, src, offs, phs, phi, ws, route_pos=pos, stream=stream)
    for _ in range(3):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    pulled = int(offs[L].item())
    return {'workload': f'pull schedule R={R} N={N} K={K} L={L} (rank 0)', 'ms': ms, 'routes': n,
            'routes_pulled': pulled, 'routes_per_s': n / (ms * 1e-3)}


def bench_share(steps, warmup, flags, dtype='bf16', keep=False):
    """Forward + backward of one expert-parallel rank's share at the DSV3 shape (4 local experts,
    57,344 slots with Zipf(1.2) loads, shared expert on 7,168 tokens): moe_experts_forward then
    moe_experts_backward per step, inputs resident in HBM. dtype 'mxfp8': the routed experts in
    MXFP8 forward and backward (weights quantised on the device beforehand, untimed), the shared
    expert in BF16. keep: the forward hands a, u (fp32, routed and shared expert) to the backward,
    which skips its replays (moe_experts_forward_keep / moe_experts_backward_kept). Returns a result dict."""
    import torch
    import synth
    import mixture_experts_layer_norm_amd as moe
    cfg = synth.EP_SHARE
    print(f'[bench] generating {cfg.name} on the device ({dtype})', file=sys.stderr, flush=True)
    D_ = synth.device_share(cfg)
    S, E, I, D, Is, T = cfg.slots, cfg.E_local, cfg.I, cfg.D, cfg.I_shared, cfg.tokens
    offsets = torch.from_numpy(np.concatenate([[0], np.cumsum(D_.counts)]).astype(np.int32)).cuda()
    p = moe.problem(T, D, I, E, cfg.K, Is, dtype, 0, 0, flags)
    if dtype == 'mxfp8':
        wq, wsc = [], []
        for k in ('w_gate', 'w_up', 'w_down'):
            wbf = getattr(D_, k)
            wq.append(torch.empty(wbf.shape, dtype=torch.uint8, device='cuda'))
            wsc.append(torch.empty(wbf.shape[:-1] + (wbf.shape[-1] // 32,), dtype=torch.uint8, device='cuda'))
            moe.quantize_mx(wbf, wq[-1], wsc[-1])
        W = moe.make_weights(*wq, D_.ws_gate, D_.ws_up, D_.ws_down, *wsc)
    else:
        W = moe.make_weights(D_.w_gate, D_.w_up, D_.w_down, D_.ws_gate, D_.ws_up, D_.ws_down)
    y = torch.empty((S, D), dtype=torch.bfloat16, device='cuda')
    sh = torch.empty((T, D), dtype=torch.bfloat16, device='cuda')
    ws = torch.empty((moe.workspace_size(p),), dtype=torch.uint8, device='cuda')
    dxs = torch.empty((S, D), dtype=torch.bfloat16, device='cuda')
    dg = torch.empty((S,), dtype=torch.float32, device='cuda')
    gr = [torch.empty(s_, device='cuda') for s_ in ((E, I, D), (E, I, D), (E, D, I), (Is, D), (Is, D), (D, Is))]
    G = moe.make_grads(*gr)
    dxl = torch.empty((T, D), dtype=torch.bfloat16, device='cuda')
    wsb = torch.empty((moe.backward_workspace_size(p),), dtype=torch.uint8, device='cuda')
    stream = torch.cuda.current_stream()

    act = [torch.empty(shp, device='cuda') for shp in ((S, I), (S, I), (T, Is), (T, Is))] if keep else None

    def fwd():
        if keep:
            moe.experts_forward_keep(p, S, D_.x_slot, offsets, W, y, D_.x_local, sh, *act, ws, stream=stream)
        else:
            moe.experts_forward(p, S, D_.x_slot, offsets, W, y, D_.x_local, sh, ws, stream=stream)

    def bwd():
        if keep:
            moe.experts_backward_kept(p, S, D_.x_slot, offsets, D_.g, D_.dy_slot, W, dxs, dg, G, D_.x_local,
                                      D_.dy_local, dxl, *act, wsb, stream=stream)
        else:
            moe.experts_backward(p, S, D_.x_slot, offsets, D_.g, D_.dy_slot, W, dxs, dg, G, D_.x_local,
                                 D_.dy_local, dxl, wsb, stream=stream)

    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for row in ev:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record(stream)
        fwd()
        ev[i][1].record(stream)
        bwd()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    f_ms = float(np.mean([r[0].elapsed_time(r[1]) for r in ev]))
    b_ms = float(np.mean([r[1].elapsed_time(r[2]) for r in ev]))
    ms = f_ms + b_ms
    flops_f = 6.0 * S * D * I + 6.0 * T * D * Is
    flops = 3.0 * flops_f
    print(f'[bench] ep share ({dtype}): fwd {f_ms:.3f} ms, bwd {b_ms:.3f} ms', file=sys.stderr, flush=True)
    # MXFP8: routed FLOPs priced at the MXFP8 peak, shared-expert FLOPs at the BF16 peak
    t_peak = (3.0 * 6.0 * S * D * I / (PEAK_MXFP8_TFLOPS if dtype == 'mxfp8' else PEAK_BF16_TFLOPS)
              + 3.0 * 6.0 * T * D * Is / PEAK_BF16_TFLOPS) / 1e12
    name = cfg.name.replace('bf16', dtype) if dtype != 'bf16' else cfg.name
    return {'workload': f'{name} forward+backward', 'dtype': dtype, 'flags': flags, 'keep_activations': keep, 'tokens': T, 'slots': S,
            'counts': D_.counts.tolist(), 'steps': steps, 'ms_per_step': ms, 'fwd_ms': f_ms, 'bwd_ms': b_ms,
            'value': T / (ms * 1e-3), 'unit': 'tokens/s', 'slots_per_s': S / (ms * 1e-3),
            'tflops': flops / (ms * 1e-3) / 1e12, 'mfma_peak_frac': t_peak / (ms * 1e-3),
            'fwd_tflops': flops_f / (f_ms * 1e-3) / 1e12, 'bwd_tflops': 2 * flops_f / (b_ms * 1e-3) / 1e12}


def second_stream_latency(step, stream, delays_ms=(1.0, 3.0, 8.0), trials=10, budget=None, host_budget=None):
    """Latency of a small kernel (an in-place add over 4 MB) enqueued on a second default-priority
    stream while moe_forward runs on the library's stream, `delay` ms after the forward was
    enqueued. Probes that did not start inside the forward are dropped.
    budget = (step_b, word, value): the forward `step_b` runs with MOE_FLAG_PERSISTENT_GEMM |
    MOE_FLAG_CU_BUDGET, and the second stream first copies `value` into its workgroup budget word
    `word` (a host-to-device copy, which needs no CU), then runs the probe; the latency counts from
    the copy. Workgroups at or above `value` end after their current tile and leave their CUs to
    the probe; the word is reset to 0 after each trial.
    host_budget = (step_h, host_word, value): the forward `step_h` runs with MOE_FLAG_CU_BUDGET_INDIRECT,
    its budget word in coherent pinned host memory (`host_word`, a ctypes c_int32); the host stores
    `value` into it right before enqueueing the probe (no GPU work at all) and resets it after each
    trial."""
    import torch
    other = torch.cuda.Stream()
    small = torch.zeros(1 << 20, device='cuda')

    def probe(pre=None):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(other)
        with torch.cuda.stream(other):
            if pre is not None:
                pre()
            small.add_(1.0)
        e1.record(other)
        return e0, e1

    alone = []
    for _ in range(trials):
        e0, e1 = probe()
        torch.cuda.synchronize()
        alone.append(e0.elapsed_time(e1) * 1e3)
    res = {'probe': 'in-place add over 1M fp32 on a second default-priority stream',
           'alone_us_median': float(np.median(alone))}

    def sweep(run, pre, reset):
        out = {}
        for d in delays_ms:
            lat = []
            for _ in range(trials):
                fa, fb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                fa.record(stream)
                run()
                fb.record(stream)
                time.sleep(d / 1e3)
                e0, e1 = probe(pre)
                torch.cuda.synchronize()
                if reset is not None:
                    reset()
                if fa.elapsed_time(e0) > 0 and e0.elapsed_time(fb) > 0:
                    lat.append(e0.elapsed_time(e1) * 1e3)
            out[f'after_{d:g}ms'] = ({'probes': len(lat), 'median_us': float(np.median(lat)),
                                      'max_us': float(np.max(lat))} if lat else {'probes': 0})
        return out

    res.update(sweep(step, None, None))
    if budget is not None:
        step_b, word, value = budget

        def reset():
            word.fill_(0)
            torch.cuda.synchronize()
        # budget set before the forward: its GEMMs use `value` workgroups, the rest stay free
        reset()
        word.fill_(value)
        torch.cuda.synchronize()
        res['cu_budget_preset'] = {'value': value, 'note': 'persistent GEMMs with MOE_FLAG_CU_BUDGET, budget set '
                                                           'before the forward', **sweep(step_b, None, None)}
        reset()
        # budget lowered while the forward runs, by a stream write-value operation on the second
        # stream (executed by the command processor, needs no CU)
        hip = hip_runtime()
        if hip is not None:
            def pre():
                hip.hipStreamWriteValue32(ctypes.c_void_p(other.cuda_stream), ctypes.c_void_p(word.data_ptr()),
                                          ctypes.c_uint32(value), ctypes.c_uint(0))
            res['cu_budget_dynamic'] = {'value': value, 'note': 'budget written by hipStreamWriteValue32 on the '
                                                                'second stream; latency from that write to the end '
                                                                'of the probe', **sweep(step_b, pre, reset)}
    if host_budget is not None:
        step_h, host_word, value = host_budget

        def pre_h():
            host_word.value = value

        def reset_h():
            host_word.value = 0
        reset_h()
        res['cu_budget_host'] = {'value': value, 'note': 'MOE_FLAG_CU_BUDGET_INDIRECT: budget word in coherent pinned '
                                                         'host memory, stored by the host right before the probe is '
                                                         'enqueued; latency from the probe stream\'s start event to '
                                                         'the end of the probe', **sweep(step_h, pre_h, reset_h)}
    return res


def pinned_host_word(hip):
    """A coherent pinned host int32 (hipHostMalloc with hipHostMallocCoherent), as (c_int32 view, device
    address, host pointer), or None."""
    if hip is None:
        return None
    ptr, dptr = ctypes.c_void_p(), ctypes.c_void_p()
    if hip.hipHostMalloc(ctypes.byref(ptr), ctypes.c_size_t(64), ctypes.c_uint(0x40000000)) != 0:
        return None
    if hip.hipHostGetDevicePointer(ctypes.byref(dptr), ptr, ctypes.c_uint(0)) != 0:
        hip.hipHostFree(ptr)
        return None
    word = ctypes.c_int32.from_address(ptr.value)
    word.value = 0
    return word, dptr.value, ptr


def hip_runtime():
    """The HIP runtime library this process has loaded (torch's), through ctypes, or None."""
    try:
        with open('/proc/self/maps') as f:
            paths = {line.split()[-1] for line in f if 'libamdhip64' in line}
        if not paths:
            return None
        lib = ctypes.CDLL(sorted(paths)[0])
        lib.hipStreamWriteValue32.restype = ctypes.c_int
        return lib
    except OSError:
        return None


def host_info():
    """What the CPU oracle runs on: CPU model, the cores this process may use, and the BLAS numpy
    calls (vendor, version and thread count as threadpoolctl reports them)."""
    model = 'unknown'
    try:
        with open('/proc/cpuinfo') as f:
            for line in f:
                if line.startswith('model name'):
                    model = line.split(':', 1)[1].strip()
                    break
    except OSError:
        pass
    blas = []
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get('user_api') == 'blas':
                blas.append({k: i.get(k) for k in ('internal_api', 'version', 'num_threads', 'threading_layer')})
    except Exception:  # pragma: no cover
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count()
    return {'cpu_model': model, 'cores_available': cores, 'blas': blas}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get('num_threads', 1) for i in threadpool_info() if i.get('user_api') == 'blas'), default=1)
    except Exception:  # pragma: no cover
        return os.cpu_count()


def cpu_baseline(cfg, L, ntok):
    """The fp64 oracle on `ntok` sampled tokens of the same layer, on the host cores. The weights
    of the experts these tokens use are copied to the host before the timed region."""
    import torch
    import oracle
    threads = blas_threads()
    rng = np.random.default_rng(1234)
    toks = np.sort(rng.choice(cfg.T, ntok, replace=False))
    lg = L.logits[torch.from_numpy(toks).cuda()].cpu().numpy()
    xs = L.x[torch.from_numpy(toks).cuda()].float().cpu().numpy()
    used = sorted(set(oracle.route_topk(lg, cfg.K).ravel().tolist()))
    print(f'[bench] cpu baseline: {ntok} tokens, {len(used)} experts to host', file=sys.stderr, flush=True)
    wg = {e: L.w_gate[e].float().cpu().numpy() for e in used}
    wu = {e: L.w_up[e].float().cpu().numpy() for e in used}
    wd = {e: L.w_down[e].float().cpu().numpy() for e in used}
    sh = [t.float().cpu().numpy() if t is not None else None for t in (L.ws_gate, L.ws_up, L.ws_down)]
    t0 = time.perf_counter()
    oracle.moe_forward(xs, lg, lambda e: wg[e], lambda e: wu[e], lambda e: wd[e], cfg.K, *sh)
    dt = time.perf_counter() - t0
    print(f'[bench] cpu baseline: {dt:.2f} s', file=sys.stderr, flush=True)
    return {'value': ntok / dt, 'unit': 'tokens/s', 'cores': threads, 'kind': 'oracle',
            'sample': f'{ntok} random tokens of the same layer (all their routed experts + shared), fp64 numpy, '
                      f'{len(used)} experts streamed; weights copied to host before timing',
            'seconds': dt, 'host': host_info()}


def calib_copy():
    """One elementwise kernel that reads exactly 1 GiB and writes exactly 1 GiB (torch.neg over 2^29
    int16): the yardstick the HBM traffic counters (FETCH_SIZE, WRITE_SIZE) are scaled by."""
    import torch
    src = torch.empty((1 << 29,), dtype=torch.int16, device='cuda')
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def make_forward(cfg, chunk_rows=0, flags=0, ring_stages=0):
    """Inputs of one moe_forward of configuration `cfg` generated on the device (seeded), with the
    routing state, output and workspace buffers; under MXFP8 the routed weights quantised on the
    device (E4M3 + E8M0 per 32 along K; the shared expert stays BF16)."""
    import torch
    import synth
    import mixture_experts_layer_norm_amd as moe
    print(f'[bench] generating {cfg.name} on the device', file=sys.stderr, flush=True)
    L = synth.device_layer(cfg)
    T, D, K, E = cfg.T, cfg.D, cfg.K, cfg.E
    dev = 'cuda'
    mx = None
    if cfg.dtype == 'mxfp8':
        mx = {}
        for k in ('w_gate', 'w_up', 'w_down'):
            wbf = getattr(L, k)
            q = torch.empty(wbf.shape, dtype=torch.uint8, device=dev)
            sc = torch.empty(wbf.shape[:-1] + (wbf.shape[-1] // 32,), dtype=torch.uint8, device=dev)
            moe.quantize_mx(wbf, q, sc)
            mx[k] = (q, sc)
        torch.cuda.synchronize()
    p = moe.problem(T, D, cfg.I, E, K, cfg.I_shared, cfg.dtype, chunk_rows, ring_stages, flags)
    routing_t = dict(topk_idx=torch.empty((T, K), dtype=torch.int32, device=dev),
                     topk_w=torch.empty((T, K), dtype=torch.float32, device=dev),
                     counts=torch.empty((E,), dtype=torch.int32, device=dev),
                     offsets=torch.empty((E + 1,), dtype=torch.int32, device=dev),
                     perm=torch.empty((T * K,), dtype=torch.int32, device=dev),
                     inv_perm=torch.empty((T * K,), dtype=torch.int32, device=dev))
    if mx is None:
        weights = moe.make_weights(L.w_gate, L.w_up, L.w_down, L.ws_gate, L.ws_up, L.ws_down)
    else:
        weights = moe.make_weights(mx['w_gate'][0], mx['w_up'][0], mx['w_down'][0], L.ws_gate, L.ws_up, L.ws_down,
                                   mx['w_gate'][1], mx['w_up'][1], mx['w_down'][1])
    return dict(L=L, p=p, mx=mx, weights=weights, routing_t=routing_t, routing=moe.make_routing(**routing_t),
                out=torch.empty((T, D), dtype=L.x.dtype, device=dev),
                ws=torch.empty((moe.workspace_size(p),), dtype=torch.uint8, device=dev))


def time_calls(fn, steps, warmup, stream):
    """Mean device time of fn() over `steps` calls after `warmup`, HIP events on `stream`."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


LANE_STREAMS = []


def lane_streams_first():
    """The lanes of moe_forward_lanes: three streams that receive work before any other stream
    but the default one. HIP binds a stream to one of its GPU_MAX_HW_QUEUES hardware queues (4 by
    default) when the stream first receives work, and later streams share those queues; two lanes
    on one queue run one after the other (measured: rocprofv3's queue ids, and b = 512 at the DSV3
    shape taking 18.8 instead of 12.8 ms when another stream was used first)."""
    import torch
    if not LANE_STREAMS:
        torch.zeros(1, device='cuda')                 # the default stream takes its queue first
        LANE_STREAMS.extend(torch.cuda.Stream() for _ in range(3))
        for s in LANE_STREAMS:
            with torch.cuda.stream(s):
                torch.zeros(1, device='cuda')         # first work: binds the stream to its queue
        torch.cuda.synchronize()


def chunk_leg(moe, cfg, L, weights, routing, stream, unchunked_ms, steps=10, warmup=2, bs=(512, 2048, 4096, 32768)):
    """The same DSV3 forward through the chunked ring at several chunk sizes b: in order on one
    stream (moe_forward, S = 3) and with the chunks spread over the stream and 3 more
    (moe_forward_lanes, S = 4); device time per step and its ratio to the unchunked forward."""
    import torch
    T, D, K = cfg.T, cfg.D, cfg.K
    out = torch.empty((T, D), dtype=L.x.dtype, device='cuda')
    main, lane_streams = stream, LANE_STREAMS[:3]
    res = {'unchunked_ms': unchunked_ms, 'lanes': 3, 'rows': []}
    for b in bs:
        row = {'b': b}
        for name, S, lanes in (('in_order', 3, 0), ('lanes', 4, 3)):
            p = moe.problem(T, D, cfg.I, cfg.E, K, cfg.I_shared, cfg.dtype, b, S, 0)
            ws = torch.empty((moe.workspace_size(p),), dtype=torch.uint8, device='cuda')
            if lanes:
                ev = [torch.cuda.Event() for _ in range(moe.lane_event_count(p, lanes))]
                for e in ev:
                    e.record(main)
                fn = lambda: moe.forward_lanes(p, L.x, L.logits, weights, out, routing, ws, lane_streams, ev,
                                               stream=main)
                ms = time_calls(fn, steps, warmup, main)
            else:
                fn = lambda: moe.forward(p, L.x, L.logits, weights, out, routing, ws, stream=stream)
                ms = time_calls(fn, steps, warmup, stream)
            row[f'{name}_ms'] = ms
            row[f'{name}_vs_unchunked'] = ms / unchunked_ms
            del ws
        res['rows'].append(row)
        print(f'[bench] chunked {cfg.name} b={b}: {json.dumps(row)}', file=sys.stderr, flush=True)
    best = min(res['rows'], key=lambda r: r['lanes_ms'])
    res['best_b'] = {'b': best['b'], 'lanes_ms': best['lanes_ms']}
    torch.cuda.empty_cache()
    return res


def mid_chunk_leg(steps=10):
    """The mid forward (T=4096, E=128) unchunked and chunked at b = 512 ... 4096."""
    import torch
    import synth
    import mixture_experts_layer_norm_amd as moe
    cfg = synth.MID
    F = make_forward(cfg)
    stream = torch.cuda.current_stream()
    ms = time_calls(lambda: moe.forward(F['p'], F['L'].x, F['L'].logits, F['weights'], F['out'], F['routing'],
                                        F['ws'], stream=stream), 20, 3, stream)
    res = chunk_leg(moe, cfg, F['L'], F['weights'], F['routing'], stream, ms, steps, bs=(512, 1024, 2048, 4096))
    del F
    torch.cuda.empty_cache()
    return res


def forward_leg(cfg, steps, warmup=3):
    """moe_forward of another configuration, timed like the headline (device time per step, inputs
    resident in HBM): mid BF16 at T=4096 and MXFP8 at T=32768."""
    import torch
    import mixture_experts_layer_norm_amd as moe
    F = make_forward(cfg)
    stream = torch.cuda.current_stream()
    ms = time_calls(lambda: moe.forward(F['p'], F['L'].x, F['L'].logits, F['weights'], F['out'], F['routing'],
                                        F['ws'], stream=stream), steps, warmup, stream)
    T, D, I, Is, n = cfg.T, cfg.D, cfg.I, cfg.I_shared, cfg.T * cfg.K
    routed, shared = 6.0 * n * D * I, 6.0 * T * D * Is
    if cfg.dtype == 'mxfp8':
        t_peak = routed / (PEAK_MXFP8_TFLOPS * 1e12) + shared / (PEAK_BF16_TFLOPS * 1e12)
    else:
        t_peak = (routed + shared) / (PEAK_BF16_TFLOPS * 1e12)
    del F
    torch.cuda.empty_cache()
    return {'workload': f'{cfg.name} forward', 'steps': steps, 'ms_per_step': ms, 'value': T / (ms * 1e-3),
            'unit': 'tokens/s', 'tflops': (routed + shared) / (ms * 1e-3) / 1e12,
            'mfma_peak_frac': t_peak / (ms * 1e-3),
            'peak_note': 'MXFP8: routed FLOPs at 5.0 PF, shared-expert FLOPs at 2.5 PF' if cfg.dtype == 'mxfp8'
            else 'BF16 at 2.5 PF'}


def layer_fwd_bwd_leg(cfg, L, keep, steps=5, warmup=2):
    """The whole layer forward + backward at `cfg` (moe_forward + moe_backward, or with keep
    moe_forward_keep + moe_backward_kept, which hand the routed a, u in fp32 to the backward instead
    of replaying them); the forward and backward device times per step and TFLOP/s counting the
    backward as twice the forward's FLOPs."""
    import torch
    import mixture_experts_layer_norm_amd as moe
    T, D, I, E, K, Is = cfg.T, cfg.D, cfg.I, cfg.E, cfg.K, cfg.I_shared
    dev = 'cuda'
    p = moe.problem(T, D, I, E, K, Is, cfg.dtype)
    rt = [torch.empty((T, K), dtype=torch.int32, device=dev), torch.empty((T, K), dtype=torch.float32, device=dev),
          torch.empty((E,), dtype=torch.int32, device=dev), torch.empty((E + 1,), dtype=torch.int32, device=dev),
          torch.empty((T * K,), dtype=torch.int32, device=dev), torch.empty((T * K,), dtype=torch.int32, device=dev)]
    R = moe.make_routing(*rt)
    W = moe.make_weights(L.w_gate, L.w_up, L.w_down, L.ws_gate, L.ws_up, L.ws_down)
    out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty((moe.workspace_size(p),), dtype=torch.uint8, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(4)
    dout = torch.randn((T, D), generator=g, device=dev).to(torch.bfloat16)
    gr = [torch.empty(s_, device=dev) for s_ in ((E, I, D), (E, I, D), (E, D, I), (Is, D), (Is, D), (D, Is))]
    G = moe.make_grads(*gr)
    dx = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    dtw = torch.empty((T, K), dtype=torch.float32, device=dev)
    dlg = torch.empty((T, E), dtype=torch.float32, device=dev)
    wsb = torch.empty(((moe.backward_kept_workspace_size if keep else moe.backward_workspace_size)(p),),
                      dtype=torch.uint8, device=dev)
    act = [torch.empty((T * K, I), device=dev) for _ in range(2)] if keep else None
    stream = torch.cuda.current_stream()

    def fwd():
        if keep:
            moe.forward_keep(p, L.x, L.logits, W, out, R, *act, ws, stream=stream)
        else:
            moe.forward(p, L.x, L.logits, W, out, R, ws, stream=stream)

    def bwd():
        if keep:
            moe.backward_kept(p, dout, L.x, L.logits, W, R, dx, G, dtw, dlg, *act, wsb, stream=stream)
        else:
            moe.backward(p, dout, L.x, L.logits, W, R, dx, G, dtw, dlg, wsb, stream=stream)

    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        fwd()
        ev[i][1].record(stream)
        bwd()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    f_ms = float(np.mean([r[0].elapsed_time(r[1]) for r in ev]))
    b_ms = float(np.mean([r[1].elapsed_time(r[2]) for r in ev]))
    flops_f = 6.0 * T * K * D * I + 6.0 * T * D * Is
    ms = f_ms + b_ms
    del ws, wsb, act, gr, G
    torch.cuda.empty_cache()
    return {'workload': f'{cfg.name} forward+backward' + (' (a, u kept)' if keep else ' (a, u replayed)'),
            'steps': steps, 'ms_per_step': ms, 'fwd_ms': f_ms, 'bwd_ms': b_ms, 'value': T / (ms * 1e-3),
            'unit': 'tokens/s', 'tflops': 3.0 * flops_f / (ms * 1e-3) / 1e12,
            'mfma_peak_frac': 3.0 * flops_f / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def cpu_oracle_extra(moe_mod):
    """The fp64 CPU oracle timed on the other configurations, each on a bounded sample (a few
    seconds of host work): the whole mid layer forward; one EP=64 rank's share forward+backward on
    128 slots per expert and 64 shared-expert tokens; the MXFP8 forward on 32 tokens whose experts
    lie in the smallest popular set (the weights' MX quantisation, offline in the recipe, is done by
    the oracle's encoder before the timed region)."""
    import torch
    import oracle
    import synth
    res = {}
    threads = blas_threads()
    # mid, whole layer
    L = synth.device_layer(synth.MID)
    h = lambda t: t.float().cpu().numpy() if t is not None else None
    x, lg = h(L.x), L.logits.cpu().numpy()
    w = [h(L.w_gate), h(L.w_up), h(L.w_down)]
    sh = [h(L.ws_gate), h(L.ws_up), h(L.ws_down)]
    del L
    torch.cuda.empty_cache()
    t0 = time.perf_counter()
    oracle.moe_forward(x, lg, *w, synth.MID.K, *sh)
    dt = time.perf_counter() - t0
    res['mid_forward'] = {'value': synth.MID.T / dt, 'unit': 'tokens/s', 'cores': threads, 'kind': 'oracle',
                          'sample': f'the whole {synth.MID.name} forward (all {synth.MID.T} tokens)', 'seconds': dt}
    del x, lg, w, sh
    # EP share, forward + backward on sampled slots
    cfg = synth.EP_SHARE
    D_ = synth.device_share(cfg)
    off = np.concatenate([[0], np.cumsum(D_.counts)])
    rng = np.random.default_rng(5)
    slots = np.concatenate([np.sort(rng.choice(np.arange(off[e], off[e + 1]), 128, replace=False))
                            for e in range(cfg.E_local)])
    rows = np.sort(rng.choice(cfg.tokens, 64, replace=False))
    si, ri = torch.from_numpy(slots).cuda(), torch.from_numpy(rows).cuda()
    xs, dys, gs = h(D_.x_slot[si]), h(D_.dy_slot[si]), D_.g[si].cpu().numpy().astype(np.float64)
    wg, wu, wd = h(D_.w_gate), h(D_.w_up), h(D_.w_down)
    xl, dyl = h(D_.x_local[ri]), h(D_.dy_local[ri])
    sg, su, sd = h(D_.ws_gate), h(D_.ws_up), h(D_.ws_down)
    del D_
    torch.cuda.empty_cache()
    cnt = np.full(cfg.E_local, 128)
    t0 = time.perf_counter()
    oracle.experts_forward(xs, cnt, wg, wu, wd)
    oracle.experts_backward(xs, cnt, gs, dys, wg, wu, wd)
    oracle.swiglu_expert(xl, sg, su, sd)
    oracle.shared_backward(xl, dyl, sg, su, sd)
    dt = time.perf_counter() - t0
    res['ep_share_fwd_bwd'] = {'value': 64 / dt, 'unit': 'tokens/s', 'slots_per_s': slots.size / dt,
                               'cores': threads, 'kind': 'oracle',
                               'sample': f'{cfg.name}: 128 slots per expert ({slots.size} slots, the routed work of 64 '
                                         f'tokens at the share\'s {cfg.slots // cfg.tokens} slots per token) and 64 '
                                         f'local tokens through the shared expert, forward+backward; value counts '
                                         f'those 64 tokens', 'seconds': dt}
    del xs, dys, gs, wg, wu, wd, xl, dyl, sg, su, sd
    # MXFP8 forward on tokens that use few experts
    cfg = synth.MXFP8
    L = synth.device_layer(cfg)
    lgm = L.logits.cpu().numpy()
    idx = oracle.route_topk(lgm, cfg.K)
    top, has0 = idx.max(axis=1), (idx == 0).any(axis=1)
    toks = None
    for M in range(cfg.K, cfg.E + 1):
        cand = np.nonzero((top < M) & has0)[0]
        if cand.size >= 32:
            toks = np.sort(cand[:32])
            break
    used = sorted(set(idx[toks].ravel().tolist()))
    ti = torch.from_numpy(toks).cuda()
    xm = h(L.x[ti])
    raw = {(k, e): getattr(L, k)[e].float().cpu().numpy() for k in ('w_gate', 'w_up', 'w_down') for e in used}
    shm = [h(L.ws_gate), h(L.ws_up), h(L.ws_down)]
    del L
    torch.cuda.empty_cache()
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(8) as pool:
        deq = dict(zip(raw.keys(), pool.map(lambda a: oracle.mx_dequantize(*oracle.mx_quantize(a.astype(np.float64))),
                                            raw.values())))
    del raw
    t0 = time.perf_counter()
    oracle.moe_forward_mx(xm, lgm[toks], lambda e: deq[('w_gate', e)], lambda e: deq[('w_up', e)],
                          lambda e: deq[('w_down', e)], cfg.K, *shm)
    dt = time.perf_counter() - t0
    res['mxfp8_forward'] = {'value': toks.size / dt, 'unit': 'tokens/s', 'cores': threads, 'kind': 'oracle',
                            'sample': f'{toks.size} tokens of {cfg.name} routed among its {len(used)} most popular '
                                      f'experts (x and h quantised in the timed region, weights before it)',
                            'seconds': dt}
    res['host'] = host_info()
    return res


if __name__ == '__main__':
    main()
