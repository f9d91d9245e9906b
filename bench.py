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
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode tokens/s at 128K ctx (hash-score+top-k+sparse attn); % HBM peak"
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3_8b_128k_b4")
    ap.add_argument("--layers", type=int, default=4,
                    help="independent KV caches the steps rotate over")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate budget of the CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-stage-timing", action="store_true")
    return ap.parse_args()


def algorithmic_bytes(w):
    """Compulsory bytes per step, whole step and per stage."""
    e = w.elem_bytes
    rows = w.B * w.Hq
    keys = w.B * w.Hkv * w.N
    kk = w.kk
    q_out = 2 * rows * w.d * e
    ids = keys * w.L
    norms = keys * 4
    gather = rows * kk * 2 * w.d * e
    scores = rows * w.N * 4
    table = w.B * w.Hkv * (2 ** w.P) * w.L * w.G * 4
    step = ids + norms + gather + q_out
    stages = {
        "bucket_probs": rows * w.d * e + w.d * w.C * e + table,
        "score": ids + norms + table + scores,
        "topk": scores + rows * kk * 4,
        "sparse_attn": gather + q_out + rows * kk * 4,
    }
    return step, stages


def cpu_baseline(w, budget_s):
    """Oracle decode on the host for a bounded sample of the workload."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle as O
    import synthetic as W

    Q, K, V, R = W.make_decode_inputs(w, "cpu", seed=0, step=0, layer=0)
    Q64 = Q.double().numpy()
    R64 = R.double().numpy()
    tau = float(np.float32(w.tau))
    done = 0
    elapsed = 0.0
    with threadpool_limits(limits=1):
        for b in range(w.B):
            K64 = K[b:b + 1].double().numpy()
            V64 = V[b:b + 1].double().numpy()
            ids = O.hash_keys(K64, R64, w.L, w.P)      # prefill, not timed
            vn = O.value_norms(V64)
            t0 = time.perf_counter()
            O.decode(Q64[b:b + 1], K64, V64, R64, ids, vn, w.L, w.P, tau, w.k)
            elapsed += time.perf_counter() - t0
            done += 1
            if elapsed >= budget_s:
                break
    return {
        "value": done / elapsed,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{w.name}: decode step 0 for batch elements 0..{done - 1} "
                   f"({done} tokens, {w.Hq} heads x {w.N} keys each), numpy float64 "
                   f"oracle, single thread, {elapsed:.1f} s timed (prefill hashing "
                   f"not timed)"),
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); the SOCKET decode path has no multi-GPU "
              f"implementation in this build", file=sys.stderr)
        sys.exit(2)

    import torch

    import soft_lsh_sparse_amd as S
    import synthetic as W
    from soft_lsh_sparse_amd import _lib

    lib = _lib.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = W.WORKLOADS[args.workload]
    assert w.decode, f"{w.name} is not a decode workload"
    dt_code = _lib.DTYPE_BF16 if w.dtype == "bf16" else _lib.DTYPE_F32

    # ---- setup: caches for every rotated layer, queries for every step
    layers = []
    for layer in range(args.layers):
        K, V = W.make_keys_values(w, dev, seed=0, layer=layer)
        R = W.make_hyperplanes(w, dev, seed=0, layer=layer)
        ids, vn = S.hash_keys(K, V, R, w.L, w.P)
        layers.append((K, V, R, ids, vn))
        torch.cuda.synchronize()
    n_q = max(1, min(w.steps, args.steps + args.warmup))
    queries = [[W.make_query(w, dev, seed=0, step=s, layer=layer)
                for s in range(n_q)] for layer in range(args.layers)]
    out = torch.empty((w.B, w.Hq, w.d), dtype=w.torch_dtype, device=dev)
    idx = torch.empty((w.B, w.Hq, w.kk), dtype=torch.int32, device=dev)
    ws_bytes = lib.socket_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, w.N, w.L,
                                                 w.P, w.k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def decode_args(step):
        layer = step % args.layers
        K, V, R, ids, vn = layers[layer]
        Q = queries[layer][step % n_q]
        return (Q.data_ptr(), K.data_ptr(), V.data_ptr(), R.data_ptr(),
                ids.data_ptr(), vn.data_ptr(), dt_code, w.B, w.Hq, w.Hkv, w.d,
                w.N, w.N, w.L, w.P, w.tau, w.k, out.data_ptr(), idx.data_ptr(),
                None, ws.data_ptr(), ws_bytes, stream)

    total = args.warmup + args.steps
    arglist = [decode_args(s) for s in range(total)]
    fn = lib.socket_decode

    for s in range(args.warmup):
        st = fn(*arglist[s])
        if st:
            _lib.check(st, "socket_decode")
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` decode steps
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for s in range(args.warmup, total):
        fn(*arglist[s])
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    tokens_per_s = w.B / (ms_per_step * 1e-3)

    step_bytes, stage_bytes = algorithmic_bytes(w)
    hbm_frac = step_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9)

    # ---- per-stage kernel times: the same kernels through the stage calls,
    # bracketed by HIP events on the launch stream
    stage_ms = {}
    roofline = None
    if not args.skip_stage_timing:
        table = torch.empty(w.B * w.Hkv * (2 ** w.P) * w.L * w.G, dtype=torch.float32,
                            device=dev)
        scores = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
        tws_b = lib.socket_topk_workspace_bytes(w.B * w.Hq, w.N, w.k)
        tws = torch.empty(max(tws_b, 1), dtype=torch.uint8, device=dev)
        aws_b = lib.socket_sparse_attn_workspace_bytes(w.B, w.Hq, w.d, w.kk)
        aws = torch.empty(aws_b, dtype=torch.uint8, device=dev)
        names = ["bucket_probs", "score", "topk", "sparse_attn"]
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i, s in enumerate(range(args.warmup, total)):
            layer = s % args.layers
            K, V, R, ids, vn = layers[layer]
            Q = queries[layer][s % n_q]
            e = evs[i]
            e[0].record()
            lib.socket_bucket_probs(Q.data_ptr(), R.data_ptr(), dt_code, w.B, w.Hq,
                                    w.Hkv, w.d, w.L, w.P, w.tau, table.data_ptr(),
                                    stream)
            e[1].record()
            lib.socket_score(table.data_ptr(), ids.data_ptr(), vn.data_ptr(), w.B,
                             w.Hq, w.Hkv, w.N, w.N, w.L, w.P, scores.data_ptr(),
                             stream)
            e[2].record()
            lib.socket_topk(scores.data_ptr(), w.B * w.Hq, w.N, w.k, idx.data_ptr(),
                            tws.data_ptr(), tws_b, stream)
            e[3].record()
            lib.socket_sparse_attn(Q.data_ptr(), K.data_ptr(), V.data_ptr(), dt_code,
                                   w.B, w.Hq, w.Hkv, w.d, w.N, idx.data_ptr(), w.kk,
                                   out.data_ptr(), aws.data_ptr(), aws_b, stream)
            e[4].record()
        torch.cuda.synchronize()
        for j, name in enumerate(names):
            stage_ms[name] = sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps
        # dominant single-kernel stage for the roofline (score is one kernel)
        dom = max(stage_ms, key=stage_ms.get)
        kernel = {"score": "score_kernel_rot", "bucket_probs": "bucket_probs_kernel",
                  "topk": "topk (zero+hist+filter+refine)",
                  "sparse_attn": "sparse_attn_kernel+attn_merge_kernel"}[dom]
        achieved = stage_bytes[dom] / (stage_ms[dom] * 1e-3) / 1e9
        roofline = {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "algorithmic_bytes_per_launch": stage_bytes[dom],
            "avg_launch_ms": round(stage_ms[dom], 5),
        }

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)

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
        "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 4),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
