#!/usr/bin/env python3
"""SOCKET decode benchmark on one MI355X.

Default workload: Llama-3-8B-shaped decode at 131072 cached keys, batch 4,
32 query / 8 KV heads, d=128, bf16, L=32 tables of P=8 bits, tau=0.3,
k=4096, one fresh query per step (256 distinct steps). One "step" is one
call of socket_decode: soft bucket table, scores, deterministic top-k and
exact attention over the selected keys, for the whole batch of one layer.
To keep the 256 MB Infinity Cache from serving repeated steps, the steps
rotate over --layers independent copies of K, V, R and their hash cache.

Prints one JSON line: tokens/s (batch / step time), the fraction of HBM peak
implied by the algorithmic bytes of a step, per-stage times measured with
HIP events on the launch stream, the roofline of the dominant kernel and a
CPU baseline (the float64 oracle on a bounded sample of the same workload).
"""

from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode tokens/s at 128K ctx (hash-score+top-k+sparse attn); % HBM peak"
HBM_PEAK_GBS = 8000.0
# LDS read peak of the chip: 128 bytes per clock per CU, 256 CUs, 2.4 GHz
LDS_PEAK_GBS = 128 * 256 * 2.4


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3_8b_128k_b4")
    ap.add_argument("--layers", type=int, default=4,
                    help="independent KV caches the steps rotate over")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-stage-timing", action="store_true")
    ap.add_argument("--skip-prefill-hash", action="store_true",
                    help="leave out the prefill-hash timing (8 KV heads x 131072 keys, "
                         "L=64, P=8) reported beside the decode figure")
    ap.add_argument("--skip-dense", action="store_true",
                    help="leave out the dense flash-decode baseline (every key, same "
                         "caches and queries) reported beside the decode figure")
    ap.add_argument("--skip-decode-loop", action="store_true",
                    help="leave out the decode loop with one appended key per KV head "
                         "and step (eager, and the same steps as one HIP graph)")
    ap.add_argument("--loop-steps", type=int, default=64)
    ap.add_argument("--skip-group-shared", action="store_true",
                    help="leave out the GQA group-shared selection variant")
    ap.add_argument("--skip-ranking-study", action="store_true",
                    help="leave out the soft-versus-hard LSH ranking comparison")
    ap.add_argument("--skip-other-configs", action="store_true",
                    help="leave out the 32K (eager and graphed) and 1M-key decode legs")
    ap.add_argument("--skip-copy-reference", action="store_true",
                    help="skip timing a plain 1 GiB device copy")
    ap.add_argument("--skip-fallback", action="store_true",
                    help="leave out the timing of the selection's full-row fallback")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy a 1 GiB buffer 4 times (reference for HBM "
                         "byte counters) and exit")
    return ap.parse_args()


def algorithmic_bytes(w):
    """Compulsory bytes of one whole decode step: bucket ids and value norms
    of every key, the selected K and V rows of every query head, queries and
    outputs (intermediates such as tables and scores are not counted)."""
    e = w.elem_bytes
    rows = w.B * w.Hq
    keys = w.B * w.Hkv * w.N
    return keys * w.L + keys * 4 + rows * w.kk * 2 * w.d * e + 2 * rows * w.d * e


def decode_kernel_names(lib, w, ids, dt_code):
    """Kernels socket_decode enqueues for this workload, in order, as the
    library reports them (no score rows are requested)."""
    buf = ctypes.create_string_buffer(512)
    n = lib.socket_decode_kernels(ids.data_ptr(), dt_code, w.B, w.Hq, w.Hkv, w.d, w.N, w.N,
                                  w.L, w.P, w.k, 0, buf, len(buf))
    if n < 1:
        raise RuntimeError(f"socket_decode_kernels failed ({n})")
    return buf.value.decode().split(",")


def kernel_bytes(w, names):
    """Compulsory HBM bytes of one launch of each decode kernel (the score
    kernel reads the table from the table kernel, or builds it from the
    queries and hyperplanes when no table kernel runs)."""
    e = w.elem_bytes
    rows = w.B * w.Hq
    keys = w.B * w.Hkv * w.N
    kk = w.kk
    table = w.B * w.Hkv * (2 ** w.P) * w.L * w.G * 4
    table_in = table if "bucket_probs_kernel" in names else rows * w.d * e + w.d * w.C * e
    partial = 0  # intermediates between two kernels are not counted
    # the attention writes the output itself unless a merge kernel follows
    out_bytes = 0 if "attn_merge_kernel" in names else rows * w.d * e
    return {
        "bucket_probs_kernel": rows * w.d * e + w.d * w.C * e + table,
        "score_kernel": keys * w.L + keys * 4 + table_in,
        "topk_gather_kernel": 0,  # moves candidates between two kernels only
        "topk_select_kernel": rows * kk * 4,
        "iota_rows_kernel": rows * kk * 4,
        "sparse_attn_kernel": rows * kk * (2 * w.d * e + 4) + rows * w.d * e + out_bytes
        + partial,
        "attn_merge_kernel": rows * w.d * e,
    }


def _hip_runtime():
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                        ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return hip


def _hip_event(hip):
    ev = ctypes.c_void_p()
    rc = hip.hipEventCreate(ctypes.byref(ev))
    if rc != 0:
        raise RuntimeError(f"hipEventCreate failed ({rc})")
    return ev.value


# Inputs of the CPU baseline, set before the worker pool is forked so the
# workers share them copy-on-write (the GPU is not touched before the fork).
_CPU = {}


def _cpu_prefill_task(b):
    """Oracle prefill of sequence b (bucket ids and value norms); not timed."""
    from threadpoolctl import threadpool_limits

    import oracle as O

    c = _CPU
    with threadpool_limits(limits=1):
        return O.hash_keys(c["K"][b], c["R"], c["L"], c["P"]), O.value_norms(c["V"][b])


def _cpu_decode_task(t):
    """One oracle decode step of one sequence on one worker (one thread)."""
    from threadpoolctl import threadpool_limits

    import oracle as O

    step, b = t
    c = _CPU
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        O.decode(c["Q"][step][b:b + 1], c["K"][b], c["V"][b], c["R"], c["ids"][b], c["vn"][b],
                 c["L"], c["P"], c["tau"], c["k"])
        return time.perf_counter() - t0


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, steps=(0, 1, 127, 255)):
    """The float64 oracle's decode on the host's cores: every sequence of the
    batch at the given steps, one (step, sequence) per worker process with one
    thread each (the oracle as it stands, untuned). Inputs are the workload's
    seeded tensors drawn on the CPU (same shapes and distributions as the
    GPU's); the oracle's own prefill hashing is not timed. Runs before the
    GPU is touched, so the workers are forked from a process without a GPU
    context."""
    import multiprocessing as mp

    import numpy as np

    import synthetic as W

    steps = [s for s in steps if s < max(1, w.steps)]
    K, V = W.make_keys_values(w, "cpu", seed=0, layer=0)
    _CPU.update(
        K=[K[b:b + 1].double().numpy() for b in range(w.B)],
        V=[V[b:b + 1].double().numpy() for b in range(w.B)],
        R=W.make_hyperplanes(w, "cpu", seed=0, layer=0).double().numpy(),
        Q={s: W.make_query(w, "cpu", seed=0, step=s, layer=0).double().numpy() for s in steps},
        L=w.L, P=w.P, tau=float(np.float32(w.tau)), k=w.k)
    del K, V
    tasks = [(s, b) for s in steps for b in range(w.B)]
    workers = max(1, min(len(os.sched_getaffinity(0)), 16, len(tasks)))
    ctx = mp.get_context("fork")
    with ctx.Pool(min(workers, w.B)) as pool:           # prefill, not timed
        pre = pool.map(_cpu_prefill_task, range(w.B), chunksize=1)
    _CPU["ids"] = [p[0] for p in pre]
    _CPU["vn"] = [p[1] for p in pre]
    with ctx.Pool(workers) as pool:
        pool.map(abs, range(workers))                   # workers up before the clock
        t0 = time.perf_counter()
        busy = pool.map(_cpu_decode_task, tasks, chunksize=1)
        wall = time.perf_counter() - t0
    _CPU.clear()
    tokens = len(tasks)
    return {
        "value": tokens / wall,
        "unit": "tokens/s",
        "cores": workers,
        "kind": "oracle",
        "cpu_model": _cpu_model(),
        "host_cpus": len(os.sched_getaffinity(0)),
        "per_token_s_one_thread": round(sum(busy) / tokens, 3),
        "sample": (f"{w.name}: decode steps {steps} of all {w.B} sequences ({tokens} tokens, "
                   f"{w.Hq} heads x {w.N} keys each), numpy float64 oracle, one (step, "
                   f"sequence) per worker process, {workers} processes of one thread, "
                   f"{wall:.1f} s wall ({sum(busy):.1f} s of CPU work); inputs drawn on the "
                   f"CPU from the same seeded distributions, oracle prefill not timed"),
    }


MFMA_BF16_PEAK_TFLOPS = 2500.0


def prefill_hash(S, W, torch, dev, reps=10):
    """Mean time of socket_hash_keys on the prefill workload (all keys of 8
    KV heads, inputs resident), as throughput against the dense bf16 MFMA
    peak (2 * d * L * P flops per key) and HBM (K, V read; ids, norms
    written)."""
    w = W.WORKLOADS["prefill_hash_128k"]
    K, V = W.make_keys_values(w, dev, seed=0)
    R = W.make_hyperplanes(w, dev, seed=0)
    K, V = K.reshape(-1, w.N, w.d), V.reshape(-1, w.N, w.d)
    ids, vn = S.hash_keys(K, V, R, w.L, w.P)
    S.hash_keys(K, V, R, w.L, w.P, ids=ids, vnorm=vn)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        S.hash_keys(K, V, R, w.L, w.P, ids=ids, vnorm=vn)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nk = K.shape[0] * w.N
    flops = 2 * w.d * w.L * w.P * nk
    hbm = 2 * nk * w.d * w.elem_bytes + nk * w.L + nk * 4
    tflops = flops / (ms * 1e-3) / 1e12
    return {"workload": w.name, "keys": nk, "L": w.L, "P": w.P, "us_per_call": round(ms * 1e3, 2),
            "tflops": round(tflops, 1), "mfma_bf16_peak_tflops": MFMA_BF16_PEAK_TFLOPS,
            "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "hbm_gbs": round(hbm / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(hbm / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def make_layers(S, W, torch, w, dev, n_layers, n_q):
    """Independent caches (K, V, R, ids, vnorm) for n_layers rotated layers and
    n_q queries per layer, all resident on the device."""
    layers = []
    for layer in range(n_layers):
        K, V = W.make_keys_values(w, dev, seed=0, layer=layer)
        R = W.make_hyperplanes(w, dev, seed=0, layer=layer)
        ids, vn = S.hash_keys(K, V, R, w.L, w.P)
        layers.append((K, V, R, ids, vn))
        torch.cuda.synchronize()
    queries = [[W.make_query(w, dev, seed=0, step=s, layer=layer) for s in range(n_q)]
               for layer in range(n_layers)]
    return layers, queries


def decode_call_args(w, layers, queries, step, dt_code, out, idx, ws, ws_bytes, stream,
                     vnorm=None):
    """socket_decode's arguments for one step (rotating over the layers)."""
    layer = step % len(layers)
    K, V, R, ids, vn = layers[layer]
    if vnorm is not None:
        vn = vnorm[layer]
    Q = queries[layer][step % len(queries[layer])]
    return (Q.data_ptr(), K.data_ptr(), V.data_ptr(), R.data_ptr(), ids.data_ptr(),
            vn.data_ptr(), dt_code, w.B, w.Hq, w.Hkv, w.d, w.N, w.N, w.L, w.P, w.tau, w.k,
            out.data_ptr(), idx.data_ptr(), None, ws.data_ptr(), ws_bytes, stream)


def decode_leg(lib, S, W, torch, w, dev, layers, queries, steps, warmup, stage_timing=True,
               profiling=None, graph=False, vnorm=None):
    """Times `steps` socket_decode calls (after `warmup` untimed ones) with HIP
    events on the launch stream, then the same steps through
    socket_decode_profiled for per-kernel times (events recorded by each
    dispatch), and optionally the same steps replayed from one HIP graph.
    Returns the figures of the leg, including the roofline of its longest
    kernel (algorithmic bytes per launch / mean launch time)."""
    from soft_lsh_sparse_amd import _lib

    dt_code = _lib.DTYPE_BF16 if w.dtype == "bf16" else _lib.DTYPE_F32
    out = torch.empty((w.B, w.Hq, w.d), dtype=w.torch_dtype, device=dev)
    idx = torch.empty((w.B, w.Hq, w.kk), dtype=torch.int32, device=dev)
    ws_bytes = lib.socket_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.N, w.L, w.P, w.k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    total = warmup + steps
    arglist = [decode_call_args(w, layers, queries, s, dt_code, out, idx, ws, ws_bytes, stream,
                                vnorm) for s in range(total)]
    fn = lib.socket_decode
    for s in range(warmup):
        st = fn(*arglist[s])
        if st:
            _lib.check(st, "socket_decode")
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for s in range(warmup, total):
        fn(*arglist[s])
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / steps
    step_bytes = algorithmic_bytes(w)
    leg = {
        "workload": w.name,
        "ms_per_step": round(ms_per_step, 5),
        "tokens_per_s": round(w.B / (ms_per_step * 1e-3), 1),
        "hbm_peak_frac": round(step_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
        "algorithmic_bytes_per_step": step_bytes,
        "steps": steps,
        "layers_rotated": len(layers),
        "wall_s_timed": round(wall, 4),
        "kernel_ms": {},
        "roofline": None,
    }
    if graph:
        # the same steps captured in one HIP graph (launch overheads removed)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for s in range(warmup, total):
                a = list(arglist[s])
                a[-1] = side.cuda_stream
                fn(*a)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream().cuda_stream
            for s in range(warmup, total):
                a = list(arglist[s])
                a[-1] = cap
                st = fn(*a)
                if st:
                    _lib.check(st, "socket_decode (capture)")
        g.replay()
        torch.cuda.synchronize()
        ev0.record()
        g.replay()
        ev1.record()
        torch.cuda.synchronize()
        gms = ev0.elapsed_time(ev1) / steps
        del g
        leg["graph_ms_per_step"] = round(gms, 5)
        leg["graph_tokens_per_s"] = round(w.B / (gms * 1e-3), 1)
    if not stage_timing:
        return leg
    names = decode_kernel_names(lib, w, layers[0][3], dt_code)
    hip = _hip_runtime()
    n_ev = 2 * len(names)
    events = [[_hip_event(hip) for _ in range(n_ev)] for _ in range(steps)]
    ev_arrays = [(ctypes.c_void_p * n_ev)(*ev) for ev in events]
    prof = lib.socket_decode_profiled
    torch.cuda.synchronize()
    for i, s in enumerate(range(warmup, total)):
        st = prof(*arglist[s], ev_arrays[i], n_ev)
        if st:
            _lib.check(st, "socket_decode_profiled")
    torch.cuda.synchronize()
    kernel_ms = {}
    for j, name in enumerate(names):
        tot = 0.0
        for ev in events:
            ms = ctypes.c_float()
            rc = hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(ev[2 * j]),
                                         ctypes.c_void_p(ev[2 * j + 1]))
            if rc != 0:
                raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
            tot += ms.value
        kernel_ms[name] = tot / steps
    for ev in events:
        for e in ev:
            hip.hipEventDestroy(ctypes.c_void_p(e))
    kbytes = kernel_bytes(w, names)
    dom = max(kernel_ms, key=kernel_ms.get)
    # HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE summary
    # of this workload; None once the kernel's sources changed
    traffic = None
    if profiling is not None:
        traffic = profiling.load_traffic(
            os.path.join(ROOT, "profiles", f"decode_{w.name}_hbm_traffic.md"), dom)
    achieved = kbytes[dom] / (kernel_ms[dom] * 1e-3) / 1e9
    leg["kernel_ms"] = {k: round(v, 5) for k, v in kernel_ms.items()}
    leg["roofline"] = {
        "bound": "hbm",
        "kernel": dom,
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "algorithmic_bytes_per_launch": kbytes[dom],
        "avg_launch_ms": round(kernel_ms[dom], 5),
    }
    # the score kernel against its own bound, the LDS port: every key's L
    # table lookups for the G query heads of its KV head (4 bytes each),
    # over the kernel's mean duration, against 128 B/clk per CU
    if "score_kernel" in kernel_ms:
        lds_bytes = w.B * w.Hkv * w.N * w.L * w.G * 4
        lds_gbs = lds_bytes / (kernel_ms["score_kernel"] * 1e-3) / 1e9
        leg["score_lds_roofline"] = {
            "bound": "lds",
            "kernel": "score_kernel",
            "achieved": round(lds_gbs, 1),
            "peak": LDS_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(lds_gbs / LDS_PEAK_GBS, 4),
            "lds_lookup_bytes_per_launch": lds_bytes,
        }
    return leg


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); the SOCKET decode path here has no multi-GPU "
              f"implementation", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_copy": src.numel() * 4,
                          "copies": 4}), flush=True)
        return

    import soft_lsh_sparse_amd as S
    import synthetic as W
    from soft_lsh_sparse_amd import _lib, profiling

    # the CPU baseline first: its worker processes are forked before this
    # process touches the GPU
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(W.WORKLOADS[args.workload])

    lib = _lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = W.WORKLOADS[args.workload]
    assert w.decode, f"{w.name} is not a decode workload"
    dt_code = _lib.DTYPE_BF16 if w.dtype == "bf16" else _lib.DTYPE_F32

    # ---- the headline workload: caches for every rotated layer, queries for
    # every step, timed decode steps and per-kernel times
    n_q = max(1, min(w.steps, args.steps + args.warmup))
    layers, queries = make_layers(S, W, torch, w, dev, args.layers, n_q)
    leg = decode_leg(lib, S, W, torch, w, dev, layers, queries, args.steps, args.warmup,
                     stage_timing=not args.skip_stage_timing, profiling=profiling)
    ms_per_step = leg["ms_per_step"]
    tokens_per_s = leg["tokens_per_s"]
    step_bytes = leg["algorithmic_bytes_per_step"]
    hbm_frac = leg["hbm_peak_frac"]
    kernel_ms = leg["kernel_ms"]
    roofline = leg["roofline"]
    wall = leg["wall_s_timed"]
    out = torch.empty((w.B, w.Hq, w.d), dtype=w.torch_dtype, device=dev)
    idx = torch.empty((w.B, w.Hq, w.kk), dtype=torch.int32, device=dev)
    ws_bytes = lib.socket_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.N, w.L, w.P, w.k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    fn = lib.socket_decode
    total = args.warmup + args.steps
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)

    def decode_args(step):
        return decode_call_args(w, layers, queries, step, dt_code, out, idx, ws, ws_bytes, stream)

    # ---- dense baseline: exact attention over every key of the same
    # rotated caches and queries (the comparison SOCKET's speed-up is stated
    # against), timed the same way; its bytes are all K and V rows once per
    # KV head plus q and out
    dense = None
    if not args.skip_dense:
        dws_bytes = lib.socket_dense_attn_workspace_bytes(w.B, w.Hq, w.d, w.N)
        dws = torch.empty(dws_bytes, dtype=torch.uint8, device=dev)
        dfn = lib.socket_dense_attn

        def dense_args(step):
            layer = step % args.layers
            K, V = layers[layer][0], layers[layer][1]
            Q = queries[layer][step % n_q]
            return (Q.data_ptr(), K.data_ptr(), V.data_ptr(), dt_code, w.B, w.Hq, w.Hkv,
                    w.d, w.N, w.N, out.data_ptr(), dws.data_ptr(), dws_bytes, stream)

        dlist = [dense_args(s) for s in range(total)]
        for s in range(args.warmup):
            st = dfn(*dlist[s])
            if st:
                _lib.check(st, "socket_dense_attn")
        torch.cuda.synchronize()
        ev0.record()
        for s in range(args.warmup, total):
            dfn(*dlist[s])
        ev1.record()
        torch.cuda.synchronize()
        dense_ms = ev0.elapsed_time(ev1) / args.steps
        dense_bytes = (2 * w.B * w.Hkv * w.N * w.d + 2 * w.B * w.Hq * w.d) * w.elem_bytes
        dense_gbs = dense_bytes / (dense_ms * 1e-3) / 1e9
        dense = {
            "kernel": "dense_attn_kernel + attn_merge_kernel",
            "ms_per_step": round(dense_ms, 5),
            "tokens_per_s": round(w.B / (dense_ms * 1e-3), 1),
            "algorithmic_bytes_per_step": dense_bytes,
            "hbm_gbs": round(dense_gbs, 1),
            "hbm_frac": round(dense_gbs / HBM_PEAK_GBS, 4),
            "socket_speedup": round(dense_ms / ms_per_step, 3),
        }

    # ---- decode loop: every step appends one key per KV head (hashed alone,
    # n = 1 at its row) and decodes over the grown cache; the last T keys of
    # layer 0 are appended in turn (their values are the prefilled ones).
    # Timed eager, then the same T steps captured in one HIP graph.
    loop = None
    if not args.skip_decode_loop:
        T = max(1, min(args.loop_steps, w.N - 1))
        K0, V0, R0, ids0, vn0 = layers[0]
        n0 = w.N - T
        esz = w.elem_bytes
        hws_bytes = lib.socket_hash_keys_workspace_bytes(dt_code, w.B * w.Hkv, 1, w.d, w.L, w.P)
        hws = torch.empty(max(hws_bytes, 1), dtype=torch.uint8, device=dev)
        hfn = lib.socket_hash_keys

        def loop_calls(t, strm):
            o = n0 + t  # the appended row
            q = queries[0][t % n_q]
            h = (K0.data_ptr() + o * w.d * esz, V0.data_ptr() + o * w.d * esz, R0.data_ptr(),
                 dt_code, w.B * w.Hkv, 1, w.N, w.d, w.L, w.P, ids0.data_ptr() + o * w.L,
                 vn0.data_ptr() + o * 4, hws.data_ptr(), hws_bytes, strm)
            dd = (q.data_ptr(), K0.data_ptr(), V0.data_ptr(), R0.data_ptr(), ids0.data_ptr(),
                  vn0.data_ptr(), dt_code, w.B, w.Hq, w.Hkv, w.d, o + 1, w.N, w.L, w.P, w.tau,
                  w.k, out.data_ptr(), idx.data_ptr(), None, ws.data_ptr(), ws_bytes, strm)
            return h, dd

        def run_loop(strm):
            for t in range(T):
                h, dd = loop_calls(t, strm)
                st = hfn(*h)
                if st:
                    _lib.check(st, "socket_hash_keys")
                st = fn(*dd)
                if st:
                    _lib.check(st, "socket_decode")

        run_loop(stream)  # warm-up
        torch.cuda.synchronize()
        ev0.record()
        run_loop(stream)
        ev1.record()
        torch.cuda.synchronize()
        eager_ms = ev0.elapsed_time(ev1) / T
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run_loop(side.cuda_stream)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run_loop(torch.cuda.current_stream().cuda_stream)
        graph.replay()
        torch.cuda.synchronize()
        ev0.record()
        graph.replay()
        ev1.record()
        torch.cuda.synchronize()
        graph_ms = ev0.elapsed_time(ev1) / T
        del graph
        loop = {
            "steps": T,
            "keys_appended_per_step": w.B * w.Hkv,
            "context": [n0 + 1, w.N],
            "eager_ms_per_step": round(eager_ms, 5),
            "graph_ms_per_step": round(graph_ms, 5),
            "graph_tokens_per_s": round(w.B / (graph_ms * 1e-3), 1),
        }

    # ---- GQA group-shared variant (one index set per KV head from the
    # group's summed scores; one gather serves the G heads), timed like the
    # decode on the same rotated caches and queries
    group = None
    if not args.skip_group_shared:
        gws_bytes = lib.socket_decode_group_shared_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.N,
                                                                   w.L, w.P, w.k)
        gws = torch.empty(gws_bytes, dtype=torch.uint8, device=dev)
        gfn = lib.socket_decode_group_shared

        def group_args(step):
            a = list(decode_args(step))
            a[18] = None                 # idx_out: the variant's is [B, Hkv, kk]
            a[20], a[21] = gws.data_ptr(), gws_bytes
            return tuple(a)

        glist = [group_args(s_) for s_ in range(total)]
        for s_ in range(args.warmup):
            st = gfn(*glist[s_])
            if st:
                _lib.check(st, "socket_decode_group_shared")
        torch.cuda.synchronize()
        ev0.record()
        for s_ in range(args.warmup, total):
            gfn(*glist[s_])
        ev1.record()
        torch.cuda.synchronize()
        gms = ev0.elapsed_time(ev1) / args.steps
        group = {"ms_per_step": round(gms, 5), "tokens_per_s": round(w.B / (gms * 1e-3), 1),
                 "speedup_vs_per_head": round(ms_per_step / gms, 3),
                 "selection": "one shared top-k per KV head by the group's summed scores"}

    # ---- soft versus hard LSH scores (the tau -> 0 one-hot table) on layer
    # 0's cache and step 0's queries: per query row, the Pearson correlation
    # of the collision sum (score / value norm) with the true q . k / sqrt(d),
    # and the recall of the top-k keys by attention mass (q . k / sqrt(d) +
    # log |v|); means over the B * Hq rows. Analysis only, not the path.
    study = None
    if not args.skip_ranking_study:
        K0, V0, R0, ids0, vn0 = layers[0]
        q0 = queries[0][0]
        soft = S.score(S.bucket_probs(q0, R0, w.Hkv, w.L, w.P, w.tau), ids0, vn0, w.Hq)
        hard = S.score(S.hard_bucket_table(q0, R0, w.Hkv, w.L, w.P), ids0, vn0, w.Hq)
        G = w.Hq // w.Hkv
        kk = min(w.k, w.N)
        acc = {"pearson_soft": 0.0, "pearson_hard": 0.0, "recall_soft": 0.0, "recall_hard": 0.0}
        for b in range(w.B):
            kf = K0[b].float()                                   # [Hkv, N, d]
            qf = q0[b].float().view(w.Hkv, G, w.d).transpose(1, 2).contiguous()  # [Hkv, d, G]
            logit = torch.matmul(kf, qf).permute(0, 2, 1).reshape(w.Hq, w.N) / math.sqrt(w.d)
            vnr = vn0[b].repeat_interleave(G, dim=0)             # [Hq, N]
            mass = logit + torch.log(vnr.clamp_min(1e-30))
            top_true = torch.zeros_like(mass, dtype=torch.bool).scatter_(
                1, torch.topk(mass, kk, dim=1).indices, True)
            for name, sc in (("soft", soft[b]), ("hard", hard[b])):
                coll = sc / vnr.clamp_min(1e-30)
                x = coll - coll.mean(1, keepdim=True)
                y = logit - logit.mean(1, keepdim=True)
                r = (x * y).sum(1) / (x.norm(dim=1) * y.norm(dim=1)).clamp_min(1e-30)
                acc["pearson_" + name] += r.sum().item()
                sel = torch.topk(sc, kk, dim=1).indices
                acc["recall_" + name] += top_true.gather(1, sel).float().mean(1).sum().item()
        rows = w.B * w.Hq
        study = {k: round(v / rows, 4) for k, v in acc.items()}
        study.update({"rows": rows, "k": kk, "tau": w.tau})
        if w.planted > 0:
            # the planted keys (cos 0.9 with the step-0 query of the group's
            # first head): the share of them inside that head's top-k
            pos = W.planted_positions(w, seed=0, layer=0).to(dev)   # [B, Hkv, planted]
            for name, sc in (("soft", soft), ("hard", hard)):
                hit = 0.0
                for b in range(w.B):
                    for g in range(w.Hkv):
                        sel = torch.topk(sc[b, g * G], kk).indices
                        hit += torch.isin(pos[b, g], sel).float().mean().item()
                study["planted_recall_" + name] = round(hit / (w.B * w.Hkv), 4)

    # ---- the selection's full-row fallback, forced on every row: value norms
    # vanish except on the keys the score kernel samples for its thresholds
    # (the first 128 keys of every 1024 at this shape: 16 waves of 1024 keys
    # per block), so fewer than k keys reach the largest block threshold and
    # every row is scored again in full by the select kernel
    fallback = None
    if not args.skip_fallback and w.name == "llama3_8b_128k_b4":
        keep = (torch.arange(w.N, device=dev) % 1024) < 128
        vmask = [lay[4] * keep for lay in layers]
        fb = decode_leg(lib, S, W, torch, w, dev, layers, queries, min(args.steps, 20),
                        min(args.warmup, 3), stage_timing=not args.skip_stage_timing,
                        vnorm=vmask)
        fallback = {"ms_per_step": fb["ms_per_step"], "kernel_ms": fb["kernel_ms"],
                    "slowdown_vs_decode": round(fb["ms_per_step"] / ms_per_step, 2),
                    "rows_forced": w.B * w.Hq}
        del vmask

    # ---- the other decode configurations, one leg each: 32K keys (B=1,
    # 20 rotated layers so the 256 MB Infinity Cache cannot hold a step's
    # working set; eager and replayed from one HIP graph, since launches
    # weigh most there) and 1M keys (B=1, L=64, P=6, k=16384)
    others = None
    if not args.skip_other_configs and w.name == "llama3_8b_128k_b4":
        others = {}
        for name, n_layers, steps, warm, graph in (("llama3_8b_32k", 20, 64, 5, True),
                                                   ("llama3_8b_1m", 2, 8, 2, False)):
            ow = W.WORKLOADS[name]
            olayers, oq = make_layers(S, W, torch, ow, dev, n_layers, 1)
            others[name] = decode_leg(lib, S, W, torch, ow, dev, olayers, oq, steps, warm,
                                      stage_timing=not args.skip_stage_timing,
                                      profiling=profiling, graph=graph)
            del olayers, oq
            torch.cuda.empty_cache()

    # ---- prefill hashing (bf16 MFMA projections, fused sign packing and
    # value norms) on its own workload, reported beside the decode figure
    prefill = None
    if not args.skip_prefill_hash:
        prefill = prefill_hash(S, W, torch, dev)

    # ---- a plain device-to-device copy of 1 GiB on the same GPU, for scale:
    # the HBM rate a streaming copy reaches here (bytes read + written per
    # second), beside the 8 TB/s published peak every fraction is taken of
    copy_ref = None
    if not args.skip_copy_reference:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        reps = 10
        ev0.record()
        for _ in range(reps):
            dst.copy_(src)
        ev1.record()
        torch.cuda.synchronize()
        cms = ev0.elapsed_time(ev1) / reps
        cbytes = 2 * src.numel() * 4
        copy_ref = {
            "bytes_per_copy": cbytes,
            "ms": round(cms, 4),
            "gbs": round(cbytes / (cms * 1e-3) / 1e9, 1),
            "frac_of_peak": round(cbytes / (cms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        }
        del src, dst
        torch.cuda.empty_cache()


    rec = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d,
            "n_keys": w.N, "L": w.L, "P": w.P, "tau": w.tau, "k": w.k,
            "layers_rotated": args.layers,
        },
        "hbm_peak_frac": round(hbm_frac, 4),
        "algorithmic_bytes_per_step": step_bytes,
        "kernel_ms": {k: round(v, 5) for k, v in kernel_ms.items()},
        "roofline": roofline,
        "score_lds_roofline": leg.get("score_lds_roofline"),
        "dense_baseline": dense,
        "decode_loop": loop,
        "ranking_study": study,
        "group_shared_variant": group,
        "prefill_hash": prefill,
        "hbm_copy_reference": copy_ref,
        "select_fallback": fallback,
        "other_configs": others,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 4),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
