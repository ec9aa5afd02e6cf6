"""Benchmark of one decode step of block top-k sparse attention on one MI355X.

One step = the whole hot path for one layer over one batch: refresh the summary
of the block holding the newest token, score and select the top-k blocks of
every (sequence, KV head), and attend the selected blocks with every query
head.  Steps cycle over `--layers` independent KV caches (distinct seeds), so
that the bytes a step touches were not touched by the previous steps and the
256 MB Infinity Cache does not serve them.  Inputs are resident in HBM before
timing starts.  The dense decode of the same shape is timed the same way.

Prints ONE JSON line (rank 0) with the throughput (sequences x steps per
second), the roofline of the dominant kernel (the sparse attention call), and
the fp64 oracle timed on the host as a CPU baseline.

    python bench.py [--steps K] [--warmup W] [--workload c2]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2", choices=["c2", "c3", "c4", "c5"])
    ap.add_argument("--layers", type=int, default=0, help="KV caches cycled over (0: auto)")
    ap.add_argument("--dense-steps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle time")
    return ap.parse_args()


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(each (sequence, KV head) row is independent; see DESIGN.md for how it would shard).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_attention_decode_ksa_amd as ksa
    from sparse_attention_decode_ksa_amd.inputs import WORKLOADS, as_numpy_bits, make_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    lib = ksa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOADS[args.workload]
    if w.plant == "tokens":
        raise SystemExit("the vote-union workload is measured with --workload c4 in a later build")
    B, Hq, Hkv, D, T, Bs, K = w.B, w.Hq, w.Hkv, w.D, w.T, w.Bs, w.top_k
    NB = (T + Bs - 1) // Bs
    keff = min(K, NB)
    elt = 2 if w.dtype == "bf16" else 4
    kv_layer_bytes = 2 * B * Hkv * w.cap * D * elt
    # bytes one step touches: the summaries and the selected K/V rows
    touched = B * Hkv * (NB + 2 * keff * Bs) * D * elt
    layers = args.layers or max(4, min(8, math.ceil(1.0e9 / touched)))

    # ---------------------------------------------------------------- inputs (resident in HBM)
    t0 = time.time()
    L = []
    for l in range(layers):
        x = make_inputs(w, device=dev, seed=w.seed * 1000 + l)
        s = torch.empty((B, Hkv, NB, D), dtype=x["k"].dtype, device=dev)
        ksa.ksa_block_summaries(x["k"], s, T, Bs)  # prefill: every block
        L.append(dict(q=x["q"], k=x["k"], v=x["v"], s=s,
                      idx=torch.empty((B, Hkv, keff), dtype=torch.int32, device=dev),
                      out=torch.empty((B, Hq, D), dtype=torch.float32, device=dev),
                      lse=torch.empty((B, Hq), dtype=torch.float32, device=dev),
                      dout=torch.empty((B, Hq, D), dtype=torch.float32, device=dev),
                      dlse=torch.empty((B, Hq), dtype=torch.float32, device=dev)))
    torch.cuda.synchronize()
    gen_s = time.time() - t0

    # ---------------------------------------------------------------- prepared C calls
    prob = ksa.Problem(B, Hq, Hkv, D, T, w.cap, Bs, ksa.KSA_BF16 if elt == 2 else ksa.KSA_F32, 0.0)
    pp = ctypes.byref(prob)
    ws_attn = ksa.ksa_workspace_bytes(prob, ksa.KSA_OP_SPARSE_BLOCKS, keff)
    ws_dense = ksa.ksa_workspace_bytes(prob, ksa.KSA_OP_DENSE, 0)
    ws = torch.empty(max(ws_attn, ws_dense, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    V = lambda t: ctypes.c_void_p(t.data_ptr())
    last_block = (T - 1) // Bs
    calls = []
    for x in L:
        sel = ksa.Selection(ksa.KSA_SEL_BLOCKS, V(x["idx"]).value, keff)
        x["sel"] = sel
        calls.append((
            (lib.ksa_block_summaries, (pp, V(x["k"]), V(x["s"]), last_block, 1, sp)),
            (lib.ksa_select_topk, (pp, V(x["q"]), V(x["s"]), K, V(x["idx"]), None, None, 0, sp)),
            (lib.ksa_sparse_decode, (pp, V(x["q"]), V(x["k"]), V(x["v"]), ctypes.byref(sel),
                                     V(x["out"]), V(x["lse"]), V(ws), ws.numel(), sp)),
            (lib.ksa_dense_decode, (pp, V(x["q"]), V(x["k"]), V(x["v"]), V(x["dout"]),
                                    V(x["dlse"]), V(ws), ws.numel(), sp)),
        ))

    def run(fn, a):
        st = fn(*a)
        if st != 0:
            raise RuntimeError("%s failed: %s" % (fn.__name__, ksa.ksa_status_string(st)))

    n_ev = args.steps
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]

    def sparse_steps(n, timed):
        for i in range(n):
            c = calls[i % layers]
            run(*c[0])
            run(*c[1])
            if timed:
                ev_a[i].record(stream)
            run(*c[2])
            if timed:
                ev_b[i].record(stream)

    # ---------------------------------------------------------------- sparse step
    sparse_steps(args.warmup, False)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    sparse_steps(args.steps, True)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    attn_ms = [a.elapsed_time(b) for a, b in zip(ev_a, ev_b)]
    attn_avg_ms = float(np.mean(attn_ms))

    # ---------------------------------------------------------------- dense step
    for i in range(min(3, args.dense_steps)):
        run(*calls[i % layers][3])
    torch.cuda.synchronize()
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record(stream)
    for i in range(args.dense_steps):
        run(*calls[i % layers][3])
    d1.record(stream)
    torch.cuda.synchronize()
    dense_ms = d0.elapsed_time(d1) / args.dense_steps

    # ---------------------------------------------------------------- bytes
    rows = B * Hkv
    tok_sel = keff * Bs
    attn_bytes = (rows * tok_sel * D * elt * 2            # selected K and V rows
                  + B * Hq * D * elt                      # q
                  + rows * keff * 4                       # block ids
                  + B * Hq * (D + 1) * 4)                 # out + lse
    select_bytes = rows * NB * D * elt + B * Hq * D * elt + rows * keff * 4
    summ_bytes = rows * (T - last_block * Bs) * D * elt + rows * D * elt
    step_bytes = attn_bytes + select_bytes + summ_bytes
    dense_bytes = rows * T * D * elt * 2 + B * Hq * D * elt + B * Hq * (D + 1) * 4
    achieved_gbps = attn_bytes / (attn_avg_ms * 1e-3) / 1e9

    traffic = None
    tr_path = os.path.join(ROOT, "profiles", "traffic_sparse_decode_%s.json" % w.name)
    if os.path.exists(tr_path):
        with open(tr_path) as f:
            tr = json.load(f)
        cur = source_hash([os.path.join(ROOT, "sparse_attention_decode_ksa_amd", "csrc", n)
                           for n in ("attention.hip", "ksa_device.h", "ksa_internal.h")])
        if tr.get("source_hash") == cur:
            traffic = tr.get("bytes_per_launch")

    # ---------------------------------------------------------------- CPU baseline (oracle)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        x = L[0]
        n_seq = B
        sl = slice(0, n_seq)
        qn, kn, vn = as_numpy_bits(x["q"][sl]), as_numpy_bits(x["k"][sl]), as_numpy_bits(x["v"][sl])
        summ = oracle.block_summaries(kn, T, Bs)  # prefill, untimed
        reps, tcpu = 0, 0.0
        while tcpu < args.cpu_seconds and reps < 50:
            c0 = time.time()
            oracle.block_summaries(kn, T, Bs, first_block=last_block, num_blocks=1, out=summ)
            raw, _ = oracle.group_scores(qn, summ, T, Bs, Tcap=w.cap)
            sel = oracle.topk(raw, K)
            oracle.attend_blocks(qn, kn, vn, T, Bs, sel)
            tcpu += time.time() - c0
            reps += 1
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
        cpu = {"value": n_seq * reps / tcpu, "unit": "seqs*steps/s", "cores": threads,
               "kind": "oracle",
               "sample": "%d full steps of all %d sequences of %s (fp64 C oracle, OpenMP), "
                         "inputs copied from the GPU" % (reps, n_seq, w.name)}

    value = B / (ms_step * 1e-3)
    dense_value = B / (dense_ms * 1e-3)
    line = {
        "metric": "sparse decode seqs*steps/s per layer (block top-k), with achieved HBM GB/s "
                  "(% of peak) vs dense",
        "value": round(value, 1),
        "unit": "seqs*steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if elt == 2 else "f32",
        "data": "synthetic (seeded N(0,1) K/V/q with planted blocks and outlier channels)",
        "config": {"workload": "%s: %s" % (w.name, w.description), "batch": B,
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "context": T,
                   "block_size": Bs, "top_k_blocks": K, "layers_cycled": layers,
                   "kv_bytes_per_layer": kv_layer_bytes},
        "step_gbps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "step_frac_of_peak": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "step_bytes": step_bytes,
        "dense": {"ms_per_step": round(dense_ms, 5), "value": round(dense_value, 1),
                  "gbps": round(dense_bytes / (dense_ms * 1e-3) / 1e9, 1)},
        "speedup_vs_dense": round(dense_ms / ms_step, 3),
        "roofline": {"kernel": "ksa_sparse_decode (block attention, split-K online softmax)",
                     "bound": "hbm", "achieved": round(achieved_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "avg_launch_ms": round(attn_avg_ms, 5),
                     "bytes_per_launch": attn_bytes},
        "cpu_baseline": cpu,
        "input_gen_s": round(gen_s, 2),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
