"""Benchmark of one decode step of sparse attention on one MI355X.

Block top-k workloads (c5 default, c2, c3): one step = refresh the summary of
the block holding the newest token, score and select the top-k blocks of every
(sequence, KV head), and attend the selected blocks with every query head.
--path fused (default) times that step as one ksa_block_topk_decode launch;
--path calls times it as ksa_block_summaries + ksa_select_topk +
ksa_sparse_decode.  The other path is run beside it and its outputs are
checked to be the same.
Vote-union workload (c4): one step = the selection layer's vote (all heads
score every history token, votes are pooled, the recency window appended) and
the attention over the shared set; the sparse-layer step (attention over a
set chosen earlier) is reported beside it.

The headline is --workload (c5: one GPU's share of the largest setting on the
pages, 34 GB of KV per layer); the workloads in --extra (c2, c3, c4) are timed
afterwards in the same process, each once the previous one's caches are
freed, and summarised under `configs`.

Steps cycle over several independent KV caches ("layers", distinct seeds) so
that a step's bytes were not touched by the steps just before it and the
256 MB Infinity Cache does not serve them.  Inputs are resident in HBM before
timing starts.  Dense decode of the same shape is timed the same way.

Order per workload: inputs; correctness checks (untimed: every layer's step,
the other path on the same inputs, HIP-graph capture and replay checked bit
for bit against the eager step); warm-up of at least --warmup steps and
--warm-seconds of wall time (the chip's clocks settle within ~15 ms of
sustained load); then the timed regions, each bracketed by
torch.cuda.synchronize() and HIP events on the stream the kernels run on
(every step is the plain C calls, launched from prepared ctypes arguments):
  1. K whole steps back to back                   -> value, ms_per_step
  2. K launches of the dominant call alone        -> roofline.achieved
     (for the fused path the step is that one call: region 1)
  3. dense decode steps                           -> dense, speedup_vs_dense
  4. K steps replayed from HIP graphs             -> graph_ms_per_step
  5. K steps with an event between consecutive steps -> step_ms_percentiles
     (p10 / p50 / p90 of single steps)
Then the oracle leg on the first sequences of layer 0 (copied from the GPU):
the step's outputs checked against the fp64 oracle (`parity`) and the oracle
timed on the host cores (`cpu_baseline`, headline only).
Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload c2|c3|c4|c5] [--path fused|calls]
    python bench.py --paged uniform|ragged [--workload c2|c3|c5]  # the step on a paged cache
    python bench.py --varlen [--workload c2|c3|c5]   # contiguous cache, one length per sequence
    python bench.py --schedule [--schedule-layers 36 --select-every 8]  # LessIsMore layers (c4)
    python bench.py --copy-probe      # a plain 1 GiB copy, to calibrate HBM counters
    python bench.py --trace-summary TRACE_DIR OUT_MD   # rocprofv3 kernel-trace durations
"""
from __future__ import annotations

import argparse
import ctypes
import gc
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
    ap.add_argument("--workload", default="c5", choices=["c2", "c3", "c4", "c5"],
                    help="the headline workload (default c5, the largest that fits one GPU)")
    ap.add_argument("--extra", default="c2,c3,c4",
                    help="workloads also timed in the same process, each after the previous "
                         "one's caches are freed (reported under `configs`; '' for none)")
    ap.add_argument("--extra-steps", type=int, default=100)
    ap.add_argument("--path", default="fused", choices=["fused", "calls"],
                    help="block top-k step as one fused launch or as the three separate calls")
    ap.add_argument("--layers", type=int, default=0, help="KV caches cycled over (0: auto)")
    ap.add_argument("--dense-steps", type=int, default=20)
    ap.add_argument("--warm-seconds", type=float, default=0.25,
                    help="least wall time of untimed warm-up before each timed workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle time")
    ap.add_argument("--paged", default="none", choices=["none", "uniform", "ragged"],
                    help="the step on a paged cache (random page order; for c4 the vote "
                         "path): every sequence at T, or lengths drawn in [T/2, T]")
    ap.add_argument("--varlen", action="store_true",
                    help="the one-launch step on the contiguous cache with one length per "
                         "sequence, drawn in [T/2, T] (ksa_block_topk_decode_varlen)")
    ap.add_argument("--schedule", action="store_true",
                    help="c4 shape: a LessIsMore layer schedule (2 dense layers, then a "
                         "selection layer every --select-every layers, sparse layers between), "
                         "amortized per layer")
    ap.add_argument("--schedule-layers", type=int, default=36)
    ap.add_argument("--select-every", type=int, default=8)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain copy of 1 GiB (counter calibration)")
    ap.add_argument("--read-probe", action="store_true",
                    help="only measure the read rate of each workload's access patterns with "
                         "the arithmetic taken away (libksa_probe.so), over a few launch shapes")
    ap.add_argument("--trace-summary", nargs=2, metavar=("TRACE_DIR", "OUT_MD"),
                    help="summarise the rocprofv3 --kernel-trace csv files under TRACE_DIR "
                         "(durations per kernel) into the markdown file OUT_MD")
    ap.add_argument("--counter-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                          "COPY_WRITE_CSV"),
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter_collection.csv files "
                         "(workload run, then the --copy-probe run) into "
                         "profiles/traffic_<kernel>_<workload>.json (kernel: block_topk_decode "
                         "for the fused path, else sparse_decode)")
    return ap.parse_args()


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# sources of the kernel each traffic record covers
KERNEL_SOURCES = {
    "sparse_decode": ("attention.hip", "ksa_attention.h", "ksa_device.h", "ksa_internal.h"),
    "block_topk_decode": ("decode_step.hip", "ksa_attention.h", "ksa_topk.h", "ksa_device.h",
                          "ksa_internal.h"),
}


def kernel_source_hash(kernel):
    return source_hash([os.path.join(ROOT, "sparse_attention_decode_ksa_amd", "csrc", n)
                        for n in KERNEL_SOURCES[kernel]])


def traffic_kernel(args, workload=None):
    workload = workload or args.workload
    return "block_topk_decode" if args.path == "fused" and workload != "c4" else "sparse_decode"


def counter_summary(args):
    """HBM bytes per launch of the timed path's dominant kernel (the fused step
    kernel, or the sparse attention kernel of the separate calls) from
    rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled
    by what the same counter reads for a plain copy of 1 GiB (bytes moved /
    counter bytes)."""
    import csv
    import statistics

    def per_kernel(path, want):
        vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
                if want(r["Kernel_Name"])]
        return statistics.median(vals), len(vals)

    fetch_csv, write_csv, cfetch_csv, cwrite_csv = args.counter_summary

    kernel = traffic_kernel(args)

    def template_args(base):
        return [t.strip() for t in base[base.index("<") + 1:base.index(">(")].split(",")]

    def is_sparse(name):
        base = name.replace("ksa::(anonymous namespace)::", "")
        if kernel == "block_topk_decode":
            return base.startswith("void block_topk_decode_kernel<")
        # the sparse attention kernel over a block (KIND 0) or token (KIND 1) list:
        # attn_partial_kernel<T, D, G, KIND> or attn_mfma_kernel<G, KIND, VK>
        kind = "1" if args.workload == "c4" else "0"
        if base.startswith("void attn_partial_kernel<"):
            return template_args(base)[3] == kind
        if base.startswith("void attn_mfma_kernel<"):
            return template_args(base)[1] == kind
        return False

    copy = lambda n: n == "__amd_rocclr_copyBuffer"
    f_kib, nf = per_kernel(fetch_csv, is_sparse)
    w_kib, nw_ = per_kernel(write_csv, is_sparse)
    cf_kib, _ = per_kernel(cfetch_csv, copy)
    cw_kib, _ = per_kernel(cwrite_csv, copy)
    gib = float(1 << 30)
    f_scale, w_scale = gib / (cf_kib * 1024.0), gib / (cw_kib * 1024.0)
    names = {"block_topk_decode": "ksa_block_topk_decode (fused step)",
             "sparse_decode": "ksa_sparse_decode"}
    out = {"workload": args.workload, "kernel": names[kernel],
           "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib,
           "dispatches": [nf, nw_], "copy_1GiB_fetch_kib": cf_kib, "copy_1GiB_write_kib": cw_kib,
           "fetch_scale": round(f_scale, 6), "write_scale": round(w_scale, 6),
           "bytes_per_launch": int(round(f_kib * 1024 * f_scale + w_kib * 1024 * w_scale)),
           "source_hash": kernel_source_hash(kernel)}
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kernel, args.workload))
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def trace_summary(args):
    """Durations per kernel from rocprofv3 --kernel-trace csv files (every
    *kernel_trace.csv under the directory), as a markdown table: launches,
    median, mean, min and max in microseconds, largest total time first."""
    import csv
    import glob
    import statistics

    tdir, out_md = args.trace_summary
    by = {}
    for p in sorted(glob.glob(os.path.join(tdir, "**", "*kernel_trace.csv"), recursive=True)):
        with open(p) as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"].replace("ksa::(anonymous namespace)::", "")
                name = name.split("(")[0] if name.startswith("void ") else name
                name = name[5:] if name.startswith("void ") else name
                us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                by.setdefault(name, []).append(us)
    rows = sorted(by.items(), key=lambda kv: -sum(kv[1]))
    lines = ["| kernel | launches | median us | mean us | min us | max us |",
             "|---|---|---|---|---|---|"]
    for name, v in rows:
        lines.append("| `%s` | %d | %.2f | %.2f | %.2f | %.2f |" % (
            name, len(v), statistics.median(v), sum(v) / len(v), min(v), max(v)))
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def copy_probe():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(10):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 10
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": round(ms, 4),
                      "gbps_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def read_probe(args):
    """Read rates of the step's access patterns with nothing computed: each
    workload's K/V (or summary, or K-history) rows read through
    libksa_probe.so with the attention kernels' lane layout, the same bytes as
    the real kernel and a few launch shapes each (waves per workgroup, splits
    per row, chunks of loads in flight per wave), cycling over caches that
    together exceed the 256 MB Infinity Cache.  One JSON line per pattern and
    shape, then a markdown table (best shape per pattern) on stderr."""
    import ctypes
    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_decode_ksa_amd", "libksa_probe.so"))
    P = ctypes.c_void_p
    lib.ksa_probe_read.argtypes = [P, P, ctypes.c_longlong, ctypes.c_int, P, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, P, P]
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    row_b = 256  # bf16 token row, D = 128

    def sorted_blocks(rows, nblocks, k, bs):
        # k distinct random blocks per row, ascending, expanded to their tokens
        ids = torch.rand((rows, nblocks), generator=g, device=dev).argsort(dim=1)[:, :k]
        ids = ids.sort(dim=1).values.to(torch.int32)
        tok = ids[:, :, None] * bs + torch.arange(bs, device=dev, dtype=torch.int32)
        return tok.reshape(rows, k * bs).contiguous()

    def token_set(B, hist, voted, window):
        ids = torch.rand((B, hist), generator=g, device=dev).argsort(dim=1)[:, :voted]
        ids = ids.sort(dim=1).values.to(torch.int32)
        rec = torch.arange(hist, hist + window, device=dev, dtype=torch.int32).expand(B, window)
        return torch.cat([ids, rec], dim=1).contiguous()

    # name, rows, capacity (tokens a row), two (K and V) or K alone, list maker
    # (rows_per_list, lists for one cache), launch shapes (waves, splits,
    # inflight; the real kernel's first), caches cycled
    pats = [
        ("c2 selected blocks (64 x 16 tokens, random 4 KB K and V blocks)", 512, 16384, True,
         lambda: (1, sorted_blocks(512, 1024, 64, 16)),
         [(8, 1, 1), (8, 1, 2), (8, 2, 1), (4, 1, 2), (8, 1, 4)], 4),
        ("c2 summaries (1024 per row, contiguous)", 512, 1024, False,
         lambda: (512, torch.arange(1024, device=dev, dtype=torch.int32)[None]),
         [(8, 1, 2), (8, 1, 4), (8, 2, 2)], 4),
        ("c2 dense (16384 tokens per row, contiguous K and V)", 512, 16384, True,
         lambda: (512, torch.arange(16384, device=dev, dtype=torch.int32)[None]),
         [(8, 8, 1), (8, 8, 2), (8, 16, 1)], 1),
        ("c3 selected blocks (64 x 32 tokens, random 8 KB K and V blocks)", 256, 32768, True,
         lambda: (1, sorted_blocks(256, 1024, 64, 32)),
         [(8, 1, 1), (8, 1, 2), (8, 2, 1), (8, 1, 4)], 4),
        ("c5 selected blocks (128 x 16 tokens, random 4 KB K and V blocks)", 2048, 32768, True,
         lambda: (1, sorted_blocks(2048, 2048, 128, 16)),
         [(4, 1, 1), (4, 1, 2), (8, 1, 1), (4, 1, 4)], 2),
        ("c4 shared token set (1536 random + 512 recent tokens, 256 B K and V rows)", 128, 20000, True,
         lambda: (8, token_set(16, 19488, 1536, 512)),
         [(8, 2, 1), (8, 2, 2), (8, 4, 1), (4, 4, 2), (8, 2, 4)], 4),
        ("c4 vote scorer's K history (19488 tokens per row, contiguous K)", 128, 20000, False,
         lambda: (128, torch.arange(19488, device=dev, dtype=torch.int32)[None]),
         [(4, 39, 2), (8, 20, 2), (8, 20, 4)], 1),
    ]
    best = []
    for name, rows, cap, two, make, shapes, ncache in pats:
        caches = []
        for _ in range(ncache):
            kk = torch.empty((rows, cap * row_b), dtype=torch.uint8, device=dev)
            vv = torch.empty_like(kk) if two else None
            rpl, lists = make()
            caches.append((kk, vv, rpl, lists))
        # the lists are made on the default stream and read on `stream`
        torch.cuda.synchronize()
        for _, _, rpl, lists in caches:
            assert lists.dtype == torch.int32 and lists.is_contiguous()
            assert lists.shape[0] * rpl >= rows and int(lists.min()) >= 0 and int(lists.max()) < cap
        ntok = caches[0][3].shape[1]
        bytes_call = rows * ntok * row_b * (2 if two else 1)
        top = None
        for waves, splits, inflight in shapes:
            sink = torch.empty(rows * splits * waves * 64, dtype=torch.int32, device=dev)

            def call(i):
                kk, vv, rpl, lists = caches[i % ncache]
                st = lib.ksa_probe_read(kk.data_ptr(), vv.data_ptr() if vv is not None else None,
                                        cap * row_b, cap, lists.data_ptr(), rpl, rows, ntok,
                                        splits, waves, inflight, sink.data_ptr(), sp)
                if st != 0:
                    raise RuntimeError("ksa_probe_read: status %d" % st)
            warm(torch, call, 4, 0.1)
            n = max(10, int(0.05 / max(bytes_call / 6.0e12, 1e-6)))
            ms = timed(torch, stream, n, call)
            gbps = bytes_call / (ms * 1e-3) / 1e9
            rec = {"pattern": name, "waves": waves, "splits": splits, "inflight": inflight,
                   "bytes_per_call": bytes_call, "us_per_call": round(ms * 1e3, 2),
                   "gbps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}
            print(json.dumps(rec), flush=True)
            if top is None or gbps > top["gbps"]:
                top = rec
        best.append(top)
        del caches
        torch.cuda.empty_cache()
    lines = ["| pattern | bytes per call | best shape (waves, splits, in flight) | us | GB/s | of 8 TB/s |",
             "|---|---|---|---|---|---|"]
    for r in best:
        lines.append("| %s | %.1f MB | %d, %d, %d | %.2f | %.0f | %.3f |" % (
            r["pattern"], r["bytes_per_call"] / 1e6, r["waves"], r["splits"], r["inflight"],
            r["us_per_call"], r["gbps"], r["frac_of_peak"]))
    print("\n".join(lines), file=sys.stderr, flush=True)


class Runner:
    """Prepared C calls: ctypes arguments built once, so a step costs a few
    microseconds of host time and the GPU never waits on Python."""

    def __init__(self, lib, ksa):
        self.lib, self.ksa = lib, ksa

    def run(self, call):
        fn, a = call
        st = fn(*a)
        if st != 0:
            raise RuntimeError("%s failed: %s" % (fn.__name__, self.ksa.ksa_status_string(st)))


def warm(torch, body, n, seconds):
    """n untimed calls of body(i), then more until `seconds` of wall time have
    passed: under a sudden sustained load the MI355X's clocks take some 15 ms
    to settle (the first ~30 c5 steps ran up to 28 % slower than the rest in
    a kernel trace), so a short warm-up would time the transient."""
    for i in range(n):
        body(i)
    torch.cuda.synchronize()
    t0, i = time.time(), n
    while time.time() - t0 < seconds:
        for _ in range(4):
            body(i)
            i += 1
        torch.cuda.synchronize()


def timed(torch, stream, n, body):
    """Time n calls of body(i) between two events; returns ms per call."""
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        body(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def per_step(torch, stream, n, body):
    """Time n calls of body(i) with an event between consecutive calls;
    returns the p10 / p50 / p90 of the per-call times in ms (the events add a
    little to each call, so region timing stays the headline)."""
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record(stream)
    for i in range(n):
        body(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    t = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(n))
    pick = lambda f: round(t[min(n - 1, int(f * n))], 5)
    return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9)}


def environment():
    """What the line was measured on: software versions, the GPU, the host CPU."""
    import platform

    import torch
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    cpu = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"torch": torch.__version__, "hip": torch.version.hip,
            "gpu": torch.cuda.get_device_name(0), "cpu_model": cpu,
            "host_threads": len(os.sched_getaffinity(0)), "python": platform.python_version()}


def input_checksum(torch, x):
    """sha256 (16 hex digits) of q and of a strided sample of 65536 elements
    of K and V: the same seed gives the same inputs."""
    h = hashlib.sha256()
    for name in ("q", "k", "v"):
        t = x[name].reshape(-1)
        step = max(1, t.numel() // 65536)
        s = t[::step].contiguous() if name != "q" else t.contiguous()
        s = s.view(torch.int16) if s.dtype == torch.bfloat16 else s.view(torch.int32)
        h.update(s.cpu().numpy().tobytes())
    return h.hexdigest()[:16]


REL_TIE = 1e-5  # near-tie gap, relative to the row's largest |relevance|


def block_parity(oracle, np, w, gpu_idx, gpu_out, gpu_lse, gpu_summ, qn, kn, vn):
    """The GPU's step on the first sequences against the fp64 oracle on the
    same bytes: summaries bitwise, selected blocks as sets (a difference is a
    near tie when the two blocks' relevances lie within REL_TIE of the row's
    largest |relevance|, else a mismatch), and the attention over the GPU's
    own selection (max abs error of out and lse)."""
    T, Bs, K = w.T, w.Bs, w.top_k
    NB = (T + Bs - 1) // Bs
    summ = oracle.block_summaries(kn, T, Bs)
    summ_exact = bool(np.array_equal(gpu_summ[:, :, :NB], summ[:, :, :NB]))
    raw, _ = oracle.group_scores(qn, summ, T, Bs, Tcap=w.cap)
    ref = oracle.topk(raw, K)
    rows = raw.reshape(-1, NB)
    gi, ri = gpu_idx.reshape(rows.shape[0], -1), ref.reshape(rows.shape[0], -1)
    near, bad = 0, 0
    for r in range(rows.shape[0]):
        a, b = set(gi[r].tolist()), set(ri[r].tolist())
        if a == b:
            continue
        tol = REL_TIE * np.abs(rows[r]).max()
        for j in a - b:
            if any(abs(rows[r, j] - rows[r, o]) < tol for o in b - a):
                near += 1
            else:
                bad += 1
    ro, rl = oracle.attend_blocks(qn, kn, vn, T, Bs, gpu_idx)
    return {"summaries_bitexact": summ_exact, "rows": int(rows.shape[0]),
            "near_tie_swaps": near, "mismatches": bad,
            "max_abs_err_out": float(np.abs(gpu_out - ro).max()),
            "max_abs_err_lse": float(np.abs(gpu_lse - rl).max())}


def vote_parity(oracle, np, w, gpu_tok, gpu_votes, gpu_out, gpu_lse, qn, kn, vn):
    """The vote-union step on the first sequences against the oracle: the
    GPU's token set must be the integer rule applied to the GPU's own votes;
    vote counts and sets are compared with the oracle's (they may differ
    only through per-head near ties at a head's threshold), and the attention
    over the GPU's set is compared with the oracle's."""
    T, N, W = w.T, w.token_budget, w.recent_window
    ref_tok, ref_votes = oracle.vote_select(qn, kn, T, N, W)
    rule = oracle.set_from_votes(gpu_votes.astype(np.int32), N, W)
    diff = sum(len(set(gpu_tok[b].tolist()) ^ set(ref_tok[b].tolist())) // 2
               for b in range(gpu_tok.shape[0]))
    ro, rl = oracle.attend_tokens(qn, kn, vn, T, gpu_tok)
    return {"sequences": int(gpu_tok.shape[0]),
            "set_is_rule_on_gpu_votes": bool(np.array_equal(rule, gpu_tok)),
            "vote_count_diffs": int(np.abs(gpu_votes.astype(np.int64) - ref_votes).sum()),
            "set_diffs_vs_oracle": int(diff),
            "max_abs_err_out": float(np.abs(gpu_out - ro).max()),
            "max_abs_err_lse": float(np.abs(gpu_lse - rl).max())}


def run_workload(args, name, headline):
    """One workload: layer caches resident in HBM, the correctness checks
    (untimed; they also bring the GPU to its working clocks), then the timed
    regions.  Returns the result dict (the headline's is the printed line)."""
    import numpy as np
    import torch

    import sparse_attention_decode_ksa_amd as ksa
    from sparse_attention_decode_ksa_amd.inputs import WORKLOADS, as_numpy_bits, make_inputs

    lib = ksa.load_library()
    R = Runner(lib, ksa)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOADS[name]
    vote = w.plant == "tokens"
    B, Hq, Hkv, D, T = w.B, w.Hq, w.Hkv, w.D, w.T
    elt = 2 if w.dtype == "bf16" else 4
    rows = B * Hkv
    steps = args.steps if headline else args.extra_steps
    warmup = args.warmup if headline else max(args.warmup, 5)
    if vote:
        N, W = w.token_budget, w.recent_window
        n_sel = min(N, T)
        Bs, K, NB, keff = 1, 0, T, 0
        touched = rows * (T - W) * D * elt + 2 * rows * n_sel * D * elt
    else:
        Bs, K = w.Bs, w.top_k
        NB = (T + Bs - 1) // Bs
        keff = min(K, NB)
        touched = rows * (NB + 2 * keff * Bs) * D * elt
    layers = args.layers or max(4, min(8, math.ceil(1.0e9 / touched)))

    # ---------------------------------------------------------------- inputs (resident in HBM)
    t0 = time.time()
    L = []
    for l in range(layers):
        x = make_inputs(w, device=dev, seed=w.seed * 1000 + l)
        x["out"] = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        x["lse"] = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        x["dout"] = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
        x["dlse"] = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        if vote:
            x["idx"] = torch.empty((B, n_sel), dtype=torch.int32, device=dev)
        else:
            x["s"] = torch.empty((B, Hkv, NB, D), dtype=x["k"].dtype, device=dev)
            ksa.ksa_block_summaries(x["k"], x["s"], T, Bs)  # prefill: every block
            x["idx"] = torch.empty((B, Hkv, keff), dtype=torch.int32, device=dev)
            # outputs of the path that is not the timed one
            x["out2"], x["lse2"] = torch.empty_like(x["out"]), torch.empty_like(x["lse"])
            x["idx2"] = torch.empty_like(x["idx"])
        L.append(x)
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    checksum = input_checksum(torch, L[0])

    # ---------------------------------------------------------------- prepared C calls
    prob = ksa.Problem(B, Hq, Hkv, D, T, w.cap, Bs, ksa.KSA_BF16 if elt == 2 else ksa.KSA_F32, 0.0)
    pp = ctypes.byref(prob)
    if vote:
        ws_sel = ksa.ksa_workspace_bytes(prob, ksa.KSA_OP_VOTE_SELECT, N)
        ws_attn = ksa.ksa_workspace_bytes(prob, ksa.KSA_OP_SPARSE_TOKENS, n_sel)
    else:
        ws_sel = ksa.ksa_workspace_bytes(prob, ksa.KSA_OP_SELECT_TOPK, K)
        ws_attn = ksa.ksa_workspace_bytes(prob, ksa.KSA_OP_SPARSE_BLOCKS, keff)
    ws_dense = ksa.ksa_workspace_bytes(prob, ksa.KSA_OP_DENSE, 0)
    wsel = ksa.new_workspace(ws_sel, dev)
    wat = ksa.new_workspace(max(ws_attn, ws_dense), dev)
    stream = torch.cuda.Stream(device=dev)  # every call and every capture runs here
    sp = ctypes.c_void_p(stream.cuda_stream)
    V = lambda t: ctypes.c_void_p(t.data_ptr())
    last_block = (T - 1) // Bs
    fused_path = args.path == "fused" and not vote
    for x in L:
        kind = ksa.KSA_SEL_TOKENS if vote else ksa.KSA_SEL_BLOCKS
        x["sel"] = ksa.Selection(kind, V(x["idx"]).value, n_sel if vote else keff)
        attn = (lib.ksa_sparse_decode, (pp, V(x["q"]), V(x["k"]), V(x["v"]), ctypes.byref(x["sel"]),
                                        V(x["out"]), V(x["lse"]), V(wat), wat.numel(), sp))
        dense = (lib.ksa_dense_decode, (pp, V(x["q"]), V(x["k"]), V(x["v"]), V(x["dout"]),
                                        V(x["dlse"]), V(wat), wat.numel(), sp))
        if vote:
            select = [(lib.ksa_vote_select, (pp, V(x["q"]), V(x["k"]), N, W, V(x["idx"]), None,
                                             V(wsel), wsel.numel(), sp))]
            fused = None
        else:
            # the separate calls write the *2 buffers when the fused step is timed
            o, l_, i_ = ((x["out2"], x["lse2"], x["idx2"]) if fused_path
                         else (x["out"], x["lse"], x["idx"]))
            x["sel"] = ksa.Selection(kind, V(i_).value, keff)
            attn = (lib.ksa_sparse_decode, (pp, V(x["q"]), V(x["k"]), V(x["v"]),
                                            ctypes.byref(x["sel"]), V(o), V(l_), V(wat),
                                            wat.numel(), sp))
            select = [(lib.ksa_block_summaries, (pp, V(x["k"]), V(x["s"]), last_block, 1, sp)),
                      (lib.ksa_select_topk, (pp, V(x["q"]), V(x["s"]), K, V(i_), None,
                                             V(wsel), wsel.numel(), sp))]
            o, l_, i_ = ((x["out"], x["lse"], x["idx"]) if fused_path
                         else (x["out2"], x["lse2"], x["idx2"]))
            fused = (lib.ksa_block_topk_decode, (pp, V(x["q"]), V(x["k"]), V(x["v"]), V(x["s"]), K,
                                                 1, V(i_), V(o), V(l_), sp))
        x["calls"] = dict(select=select, attn=attn, dense=dense, fused=fused)

    def calls_step(i):
        c = L[i % layers]["calls"]
        for s_ in c["select"]:
            R.run(s_)
        R.run(c["attn"])

    def fused_step(i):
        R.run(L[i % layers]["calls"]["fused"])

    step = fused_step if fused_path else calls_step
    other_step = None if vote else (calls_step if fused_path else fused_step)

    def attn_only(i):
        if fused_path:
            fused_step(i)
        else:
            R.run(L[i % layers]["calls"]["attn"])

    def select_only(i):
        for s_ in L[i % layers]["calls"]["select"]:
            R.run(s_)

    def dense_only(i):
        R.run(L[i % layers]["calls"]["dense"])

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fn()
        return g

    torch.cuda.synchronize()
    ms_graph = ms_attn = ms_select = ms_other = None
    with torch.cuda.stream(stream):
        # -------------------------------------------------------- checks (untimed)
        for l in range(layers):
            step(l)
        torch.cuda.synchronize()
        ref = [(x["out"].clone(), x["lse"].clone(), x["idx"].clone()) for x in L]
        if other_step is not None:
            # the other path on the same inputs: block ids bitwise, outputs bitwise
            # unless the separate attention is planned with another split (which
            # reorders its fp32 merge)
            for l in range(layers):
                other_step(l)
            torch.cuda.synchronize()
            for x in L:
                assert torch.equal(x["idx2"], x["idx"]), "fused step and separate calls select differently"
                assert float((x["out2"] - x["out"]).abs().max()) <= 1e-5 \
                    and float((x["lse2"] - x["lse"]).abs().max()) <= 1e-5, \
                    "fused step and separate calls differ"
        if headline:
            # graphs: one step per layer, and one whole cycle over the layers; a
            # replay reproduces the eager step bit for bit
            g_step = [capture(lambda l=l: step(l)) for l in range(layers)]
            g_cycle = capture(lambda: [step(l) for l in range(layers)])
            for x in L:
                x["out"].zero_(), x["lse"].zero_(), x["idx"].zero_()
            g_cycle.replay()
            torch.cuda.synchronize()
            for l, x in enumerate(L):
                assert torch.equal(x["out"], ref[l][0]) and torch.equal(x["lse"], ref[l][1]) \
                    and torch.equal(x["idx"], ref[l][2]), "graph replay differs from the eager step"

        # -------------------------------------------------------- timed regions
        warm(torch, step, warmup, args.warm_seconds)
        ms_step = timed(torch, stream, steps, step)             # region 1
        pct = per_step(torch, stream, steps, step)               # region 5
        if headline:
            full, rest = divmod(steps, layers)

            def graph_steps(i):
                if i < full:
                    g_cycle.replay()
                else:
                    g_step[i - full].replay()

            ms_graph = timed(torch, stream, full + rest, graph_steps) * (full + rest) / steps  # 4
            ms_select = timed(torch, stream, steps, select_only)
            if other_step is not None:
                ms_other = timed(torch, stream, steps, other_step)
        ms_attn = ms_step if fused_path else timed(torch, stream, steps, attn_only)     # 2
        warm(torch, dense_only, 1, args.warm_seconds)
        ms_dense = timed(torch, stream, args.dense_steps, dense_only)  # region 3
        for l in range(layers):  # layer caches back to the timed path's outputs
            step(l)
        torch.cuda.synchronize()

    # ---------------------------------------------------------------- algorithmic bytes
    q_bytes = B * Hq * D * elt
    out_bytes = B * Hq * (D + 1) * 4
    if vote:
        attn_bytes = rows * n_sel * D * elt * 2 + q_bytes + B * n_sel * 4 + out_bytes
        select_bytes = rows * (T - W) * D * elt + q_bytes + B * n_sel * 4
    else:
        attn_bytes = rows * keff * Bs * D * elt * 2 + q_bytes + rows * keff * 4 + out_bytes
        select_bytes = (rows * NB * D * elt + q_bytes + rows * keff * 4            # scoring + ids
                        + rows * (T - last_block * Bs) * D * elt + rows * D * elt)  # summary refresh
    step_bytes = attn_bytes + select_bytes
    dense_bytes = rows * T * D * elt * 2 + q_bytes + out_bytes
    dom_bytes = step_bytes if fused_path else attn_bytes
    achieved = dom_bytes / (ms_attn * 1e-3) / 1e9

    traffic = None
    tk = traffic_kernel(args, name)
    tr_path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (tk, w.name))
    if os.path.exists(tr_path):
        with open(tr_path) as f:
            tr = json.load(f)
        if tr.get("source_hash") == kernel_source_hash(tk):
            traffic = tr.get("bytes_per_launch")

    # ---------------------------------------------------------------- oracle leg (CPU baseline + parity)
    cpu = parity = None
    if not args.no_cpu_baseline:
        import oracle
        x = L[0]
        n_seq = min(B, 8 if headline else 2) if not vote else min(B, 4 if headline else 2)
        sl = slice(0, n_seq)
        qn, kn, vn = as_numpy_bits(x["q"][sl]), as_numpy_bits(x["k"][sl]), as_numpy_bits(x["v"][sl])
        g_out = x["out"][sl].cpu().numpy().astype(np.float64)
        g_lse = x["lse"][sl].cpu().numpy().astype(np.float64)
        if vote:
            # the timed vote writes no vote counts: one more untimed call with them
            votes = torch.empty((B, T), dtype=torch.uint8, device=dev)
            tok2 = torch.empty_like(x["idx"])
            R.run((lib.ksa_vote_select, (pp, V(x["q"]), V(x["k"]), N, W, V(tok2), V(votes),
                                         V(wsel), wsel.numel(), sp)))
            torch.cuda.synchronize()
            assert torch.equal(tok2, x["idx"]), "vote select is not repeatable"
            parity = vote_parity(oracle, np, w, x["idx"][sl].cpu().numpy(),
                                 votes[sl].cpu().numpy(), g_out, g_lse, qn, kn, vn)
        else:
            parity = block_parity(oracle, np, w, x["idx"][sl].cpu().numpy(), g_out, g_lse,
                                  as_numpy_bits(x["s"][sl]), qn, kn, vn)
        if headline:
            if not vote:
                summ = oracle.block_summaries(kn, T, Bs)  # prefill, untimed
            reps, tcpu = 0, 0.0
            while tcpu < args.cpu_seconds and reps < 50:
                c0 = time.time()
                if vote:
                    tok, _ = oracle.vote_select(qn, kn, T, N, W)
                    oracle.attend_tokens(qn, kn, vn, T, tok)
                else:
                    oracle.block_summaries(kn, T, Bs, first_block=last_block, num_blocks=1, out=summ)
                    raw, _ = oracle.group_scores(qn, summ, T, Bs, Tcap=w.cap)
                    oracle.attend_blocks(qn, kn, vn, T, Bs, oracle.topk(raw, K))
                tcpu += time.time() - c0
                reps += 1
            threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
            cpu = {"value": round(n_seq * reps / tcpu, 2), "unit": "seqs*steps/s", "cores": threads,
                   "kind": "oracle", "cpu_model": environment()["cpu_model"],
                   "sample": "%d full steps of %d of the %d sequences of %s (fp64 C oracle, OpenMP), "
                             "inputs copied from the GPU" % (reps, n_seq, B, w.name)}

    value = B / (ms_step * 1e-3)
    cfg = {"workload": "%s: %s" % (w.name, w.description), "batch": B, "q_heads": Hq,
           "kv_heads": Hkv, "head_dim": D, "context": T, "layers_cycled": layers,
           "input_sha256_16": checksum}
    if vote:
        cfg.update(token_budget=N, recent_window=W)
        dom = "ksa_sparse_decode (shared token set)"
    else:
        cfg.update(block_size=Bs, top_k_blocks=K, path=args.path)
        dom = ("ksa_block_topk_decode (refresh + score + top-k + attention, one launch)"
               if fused_path else "ksa_sparse_decode (selected blocks, split-K online softmax)")
    if vote:
        # the sparse layer (attention over a set chosen earlier) against 0.6 x T / N
        target = 0.6 * T / n_sel
        speedup = ms_dense / ms_attn
    else:
        target = 0.6 * T / (keff * Bs)
        speedup = ms_dense / ms_step
    line = {
        "metric": "sparse decode seqs*steps/s per layer, with achieved HBM GB/s (% of peak) vs dense",
        "value": round(value, 1),
        "unit": "seqs*steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "step_ms_percentiles": pct,
        "graph_ms_per_step": None if ms_graph is None else round(ms_graph, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if elt == 2 else "f32",
        "data": "synthetic (seeded N(0,1) K/V/q with planted structure)",
        "config": cfg,
        "step_bytes": step_bytes,
        "step_gbps": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "step_frac_of_peak": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "select": None if ms_select is None else
                  {"ms_eager": round(ms_select, 5),
                   "gbps": round(select_bytes / (ms_select * 1e-3) / 1e9, 1)},
        "dense": {"ms_per_step": round(ms_dense, 5), "value": round(B / (ms_dense * 1e-3), 1),
                  "gbps": round(dense_bytes / (ms_dense * 1e-3) / 1e9, 1)},
        "speedup_vs_dense": round(ms_dense / ms_step, 3),
        "speedup_target": {"value": round(target, 3), "measured": round(speedup, 3),
                           "on": "sparse layer" if vote else "step", "met": speedup >= target},
        # the step's bandwidth against what dense decode (a plain stream of K and V
        # over the same caches) reaches on this machine
        "step_frac_of_dense_gbps": round((step_bytes / ms_step) / (dense_bytes / ms_dense), 4),
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "avg_launch_ms": round(ms_attn, 5),
                     "bytes_per_launch": dom_bytes},
        "cpu_baseline": cpu,
        "parity": parity,
        "input_gen_s": round(gen_s, 2),
    }
    if ms_other is not None:
        line["other_path"] = {"path": "calls" if fused_path else "fused",
                              "ms_per_step": round(ms_other, 5),
                              "speedup_vs_dense": round(ms_dense / ms_other, 3)}
    if vote:
        line["sparse_layer_step"] = {"ms": round(ms_attn, 5), "value": round(B / (ms_attn * 1e-3), 1),
                                     "gbps": round(attn_bytes / (ms_attn * 1e-3) / 1e9, 1),
                                     "frac_of_peak": round(attn_bytes / (ms_attn * 1e-3) / 1e9
                                                           / HBM_PEAK_GBPS, 4),
                                     "speedup_vs_dense": round(ms_dense / ms_attn, 3)}
    return line


def compact(line):
    """The per-config summary kept in the headline's `configs`."""
    keep = ("value", "ms_per_step", "step_ms_percentiles", "step_gbps", "step_frac_of_peak",
            "speedup_vs_dense", "speedup_target", "step_frac_of_dense_gbps", "parity",
            "sparse_layer_step", "steps", "warmup")
    out = {k: line[k] for k in keep if k in line}
    out["workload"] = line["config"]["workload"]
    out["dense_ms"] = line["dense"]["ms_per_step"]
    out["roofline"] = {k: line["roofline"][k] for k in ("kernel", "achieved", "frac", "traffic",
                                                         "avg_launch_ms", "bytes_per_launch")}
    out["input_sha256_16"] = line["config"]["input_sha256_16"]
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(every (sequence, KV head) row is independent, so batch or KV-head sharding "
              "would need no communication; it is not built).", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    if args.read_probe:
        read_probe(args)
        return
    if args.paged != "none" or args.varlen:
        paged_main(args)
        return
    if args.schedule:
        schedule_main(args)
        return
    if args.counter_summary:
        counter_summary(args)
        return
    if args.trace_summary:
        trace_summary(args)
        return

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    line = run_workload(args, args.workload, headline=True)
    extra = [c for c in args.extra.split(",") if c and c != args.workload]
    if extra:
        line["configs"] = {}
        for c in extra:
            gc.collect()  # the previous workload's caches go back to the allocator
            torch.cuda.empty_cache()
            line["configs"][c] = compact(run_workload(args, c, headline=False))
    line["env"] = environment()
    print(json.dumps(line), flush=True)


def paged_main(args):
    """The block top-k decode step on a paged cache: every layer's K and V are
    stored as page pools in a seeded random page order (to_paged), each
    sequence has its own length (all T, or drawn in [T/2, T]), and the step
    is one ksa_paged_block_topk_decode launch; dense is ksa_paged_dense_decode.
    With --varlen the cache stays contiguous and the step is one
    ksa_block_topk_decode_varlen launch (lengths drawn in [T/2, T]); dense is
    then ksa_dense_decode with every sequence at T, reported for reference
    only (it reads more than the ragged batch holds, so no speedup is given)."""
    import numpy as np
    import torch

    import sparse_attention_decode_ksa_amd as ksa
    from sparse_attention_decode_ksa_amd.inputs import WORKLOADS, make_inputs, to_paged

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    lib = ksa.load_library()
    R = Runner(lib, ksa)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOADS[args.workload]
    if w.plant == "tokens":
        if args.varlen and args.paged == "none":
            raise SystemExit("--varlen times the block top-k step (c2, c3, c5)")
        return paged_vote_main(args, w)
    B, Hq, Hkv, D, T, Bs, K = w.B, w.Hq, w.Hkv, w.D, w.T, w.Bs, w.top_k
    elt = 2 if w.dtype == "bf16" else 4
    rows = B * Hkv
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed * 7 + 1)
    varlen = args.varlen and args.paged == "none"
    if args.paged == "ragged" or varlen:
        lens = torch.randint(T // 2, T + 1, (B,), generator=gen).tolist()
    else:
        lens = [T] * B
    nbc = (T + Bs - 1) // Bs
    touched = rows * (nbc + 2 * K * Bs) * D * elt
    layers = args.layers or max(4, min(8, math.ceil(1.0e9 / touched)))
    t0 = time.time()
    L = []
    for l in range(layers):
        x = make_inputs(w, device=dev, seed=w.seed * 1000 + l)
        if varlen:
            x.update(s=torch.empty((B, Hkv, (w.cap + Bs - 1) // Bs, D), dtype=x["k"].dtype,
                                   device=dev))
            ksa.ksa_block_summaries(x["k"], x["s"], T, Bs)
        else:
            kp, vp, table = to_paged(x["k"], x["v"], Bs, seed=w.seed * 1000 + l + 1)
            del x["k"], x["v"]
            x.update(kp=kp, vp=vp, table=table,
                     s=torch.empty((B, Hkv, table.shape[1], D), dtype=kp.dtype, device=dev))
        x.update(seq=torch.tensor(lens, dtype=torch.int32, device=dev),
                 out=torch.empty((B, Hq, D), dtype=torch.float32, device=dev),
                 lse=torch.empty((B, Hq), dtype=torch.float32, device=dev),
                 idx=torch.empty((B, Hkv, K), dtype=torch.int32, device=dev),
                 dout=torch.empty((B, Hq, D), dtype=torch.float32, device=dev),
                 dlse=torch.empty((B, Hq), dtype=torch.float32, device=dev))
        if not varlen:
            ksa.ksa_paged_block_summaries(x["kp"], x["s"], x["table"], x["seq"], max_len=T)
        L.append(x)
    torch.cuda.synchronize()
    gen_s = time.time() - t0

    prob = ksa.Problem(B, Hq, Hkv, D, T, w.cap if varlen else L[0]["table"].shape[1] * Bs, Bs,
                       ksa.KSA_BF16 if elt == 2 else ksa.KSA_F32, 0.0)
    pp = ctypes.byref(prob)
    stream = torch.cuda.Stream(device=dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    V = lambda t: ctypes.c_void_p(t.data_ptr())
    wsd = ksa.new_workspace(ksa.ksa_workspace_bytes(
        prob, ksa.KSA_OP_DENSE if varlen else ksa.KSA_OP_PAGED_DENSE, 0), dev)
    for x in L if varlen else []:
        x["step"] = (lib.ksa_block_topk_decode_varlen,
                     (pp, V(x["seq"]), V(x["q"]), V(x["k"]), V(x["v"]), V(x["s"]), K, 1,
                      V(x["idx"]), V(x["out"]), V(x["lse"]), sp))
        x["dense"] = (lib.ksa_dense_decode,
                      (pp, V(x["q"]), V(x["k"]), V(x["v"]), V(x["dout"]), V(x["dlse"]), V(wsd),
                       wsd.numel(), sp))
    for x in [] if varlen else L:
        x["pg"] = ksa.PagedKv(V(x["table"]).value, V(x["seq"]).value, x["table"].shape[1],
                              x["kp"].shape[0])
        pg = ctypes.byref(x["pg"])
        x["step"] = (lib.ksa_paged_block_topk_decode,
                     (pp, pg, V(x["q"]), V(x["kp"]), V(x["vp"]), V(x["s"]), K, 1, V(x["idx"]),
                      V(x["out"]), V(x["lse"]), sp))
        x["dense"] = (lib.ksa_paged_dense_decode,
                      (pp, pg, V(x["q"]), V(x["kp"]), V(x["vp"]), V(x["dout"]), V(x["dlse"]),
                       V(wsd), wsd.numel(), sp))

    def step(i):
        R.run(L[i % layers]["step"])

    def dense_only(i):
        R.run(L[i % layers]["dense"])

    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        warm(torch, step, args.warmup, args.warm_seconds)
        ms_step = timed(torch, stream, args.steps, step)
        pct = per_step(torch, stream, args.steps, step)
        warm(torch, dense_only, 1, args.warm_seconds)
        ms_dense = timed(torch, stream, args.dense_steps, dense_only)

    # algorithmic bytes of one step, from each row's length and its selected blocks
    x = L[0]
    ids = x["idx"].cpu().numpy().reshape(B, Hkv, K)
    tl = np.array(lens)
    nb = (tl + Bs - 1) // Bs
    sel_tok = 0
    for b in range(B):
        for g in range(Hkv):
            j = ids[b, g][ids[b, g] >= 0]
            sel_tok += int(np.minimum(Bs, tl[b] - j * Bs).sum())
    last_tok = int((tl - (nb - 1) * Bs).sum()) * Hkv
    q_bytes = B * Hq * D * elt
    out_bytes = B * Hq * (D + 1) * 4
    step_bytes = (int(nb.sum()) * Hkv * D * elt            # summaries scored
                  + last_tok * D * elt + rows * D * elt      # newest block refreshed
                  + sel_tok * D * elt * 2                    # selected K and V
                  + 2 * q_bytes + out_bytes + int(np.minimum(K, nb).sum()) * Hkv * 8 + B * 4)
    dense_bytes = (B * T if varlen else int(tl.sum())) * Hkv * D * elt * 2 + q_bytes + out_bytes
    achieved = step_bytes / (ms_step * 1e-3) / 1e9
    cfg = {"workload": "%s: %s" % (w.name, w.description), "batch": B, "q_heads": Hq,
           "kv_heads": Hkv, "head_dim": D, "context": T, "layers_cycled": layers,
           "block_size": Bs, "top_k_blocks": K, "paged": args.paged,
           "seq_len_mean": round(float(tl.mean()), 1), "seq_len_min": int(tl.min())}
    if varlen:
        cfg["varlen"] = True
    else:
        cfg["pages_per_layer"] = int(L[0]["kp"].shape[0])
    line = {
        "metric": "sparse decode seqs*steps/s per layer, with achieved HBM GB/s (% of peak) vs dense",
        "value": round(B / (ms_step * 1e-3), 1), "unit": "seqs*steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "step_ms_percentiles": pct,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if elt == 2 else "f32",
        "data": "synthetic (seeded N(0,1) K/V/q with planted structure)" +
                ("" if varlen else ", paged in a random page order"),
        "config": cfg, "step_bytes": step_bytes,
        "dense": {"ms_per_step": round(ms_dense, 5), "value": round(B / (ms_dense * 1e-3), 1),
                  "gbps": round(dense_bytes / (ms_dense * 1e-3) / 1e9, 1),
                  **({"note": "every sequence at T (reference only)"} if varlen else {})},
        "speedup_vs_dense": None if varlen else round(ms_dense / ms_step, 3),
        "roofline": {"kernel": ("ksa_block_topk_decode_varlen" if varlen else
                                "ksa_paged_block_topk_decode") +
                               " (refresh + score + top-k + attention, one launch)",
                     "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None, "avg_launch_ms": round(ms_step, 5),
                     "bytes_per_launch": step_bytes},
        "cpu_baseline": None,
        "input_gen_s": round(gen_s, 2),
    }
    print(json.dumps(line), flush=True)


def paged_vote_main(args, w):
    """The vote-union workload on a paged cache (pages of 16 tokens in a seeded
    random order, each sequence its own length): the selection step is
    ksa_paged_vote_select + ksa_paged_sparse_decode over the set; the sparse
    layer is the attention alone; the selection layer of the schedule is
    ksa_paged_vote_layer_decode (dense attention plus the vote); dense is
    ksa_paged_dense_decode."""
    import numpy as np
    import torch

    import sparse_attention_decode_ksa_amd as ksa
    from sparse_attention_decode_ksa_amd.inputs import make_inputs, to_paged

    lib = ksa.load_library()
    R = Runner(lib, ksa)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, Hq, Hkv, D, T = w.B, w.Hq, w.Hkv, w.D, w.T
    N, W, Bs = w.token_budget, w.recent_window, 16
    elt = 2 if w.dtype == "bf16" else 4
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed * 7 + 1)
    lens = (torch.randint(T // 2, T + 1, (B,), generator=gen).tolist() if args.paged == "ragged"
            else [T] * B)
    n_out = min(N, T)
    layers = args.layers or 4
    t0 = time.time()
    L = []
    for l in range(layers):
        x = make_inputs(w, device=dev, seed=w.seed * 1000 + l)
        kp, vp, table = to_paged(x["k"], x["v"], Bs, seed=w.seed * 1000 + l + 1)
        del x["k"], x["v"]
        x.update(kp=kp, vp=vp, table=table, seq=torch.tensor(lens, dtype=torch.int32, device=dev),
                 idx=torch.empty((B, n_out), dtype=torch.int32, device=dev),
                 out=torch.empty((B, Hq, D), dtype=torch.float32, device=dev),
                 lse=torch.empty((B, Hq), dtype=torch.float32, device=dev))
        L.append(x)
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    prob = ksa.Problem(B, Hq, Hkv, D, T, L[0]["table"].shape[1] * Bs, Bs,
                       ksa.KSA_BF16 if elt == 2 else ksa.KSA_F32, 0.0)
    pp = ctypes.byref(prob)
    stream = torch.cuda.Stream(device=dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    V = lambda t: ctypes.c_void_p(t.data_ptr())
    ws_v = ksa.new_workspace(ksa.ksa_workspace_bytes(prob, ksa.KSA_OP_VOTE_SELECT, N), dev)
    ws_a = ksa.new_workspace(max(1, ksa.ksa_workspace_bytes(prob, ksa.KSA_OP_SPARSE_TOKENS, n_out)), dev)
    ws_l = ksa.new_workspace(ksa.ksa_workspace_bytes(prob, ksa.KSA_OP_PAGED_VOTE_LAYER, N), dev)
    ws_d = ksa.new_workspace(max(1, ksa.ksa_workspace_bytes(prob, ksa.KSA_OP_PAGED_DENSE, 0)), dev)
    for x in L:
        x["pg"] = ksa.PagedKv(V(x["table"]).value, V(x["seq"]).value, x["table"].shape[1],
                              x["kp"].shape[0])
        pg = ctypes.byref(x["pg"])
        x["sel"] = ksa.Selection(ksa.KSA_SEL_TOKENS, V(x["idx"]).value, n_out)
        x["vote"] = (lib.ksa_paged_vote_select, (pp, pg, V(x["q"]), V(x["kp"]), N, W, V(x["idx"]),
                                                 None, V(ws_v), ws_v.numel(), sp))
        x["attn"] = (lib.ksa_paged_sparse_decode, (pp, pg, V(x["q"]), V(x["kp"]), V(x["vp"]),
                                                   ctypes.byref(x["sel"]), V(x["out"]), V(x["lse"]),
                                                   V(ws_a), ws_a.numel(), sp))
        x["layer"] = (lib.ksa_paged_vote_layer_decode, (pp, pg, V(x["q"]), V(x["kp"]), V(x["vp"]), N,
                                                        W, V(x["out"]), V(x["lse"]), V(x["idx"]),
                                                        None, V(ws_l), ws_l.numel(), sp))
        x["dense"] = (lib.ksa_paged_dense_decode, (pp, pg, V(x["q"]), V(x["kp"]), V(x["vp"]),
                                                   V(x["out"]), V(x["lse"]), V(ws_d), ws_d.numel(),
                                                   sp))
    run = lambda key: (lambda i: R.run(L[i % layers][key]))

    def sel_step(i):
        R.run(L[i % layers]["vote"])
        R.run(L[i % layers]["attn"])

    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        warm(torch, sel_step, args.warmup, args.warm_seconds)
        ms_step = timed(torch, stream, args.steps, sel_step)
        pct = per_step(torch, stream, args.steps, sel_step)
        ms_sparse = timed(torch, stream, args.steps, run("attn"))
        warm(torch, run("layer"), 1, args.warm_seconds)
        ms_layer = timed(torch, stream, max(3, args.dense_steps), run("layer"))
        warm(torch, run("dense"), 1, args.warm_seconds)
        ms_dense = timed(torch, stream, args.dense_steps, run("dense"))
    tl = np.array(lens)
    hist = np.where(tl > N, tl - W, 0)
    sel = np.minimum(tl, N)
    q_bytes, out_bytes = B * Hq * D * elt, B * Hq * (D + 1) * 4
    sparse_bytes = int(sel.sum()) * Hkv * D * elt * 2 + q_bytes + out_bytes + B * n_out * 4
    step_bytes = int(hist.sum()) * Hkv * D * elt + q_bytes + sparse_bytes
    dense_bytes = int(tl.sum()) * Hkv * D * elt * 2 + q_bytes + out_bytes
    gbps = lambda n, ms: round(n / (ms * 1e-3) / 1e9, 1)
    cfg = {"workload": "%s: %s" % (w.name, w.description), "batch": B, "q_heads": Hq,
           "kv_heads": Hkv, "head_dim": D, "context": T, "layers_cycled": layers,
           "token_budget": N, "recent_window": W, "page_size": Bs, "paged": args.paged,
           "seq_len_mean": round(float(tl.mean()), 1), "seq_len_min": int(tl.min()),
           "pages_per_layer": int(L[0]["kp"].shape[0])}
    sparse_gbps = gbps(sparse_bytes, ms_sparse)
    line = {
        "metric": "sparse decode seqs*steps/s per layer, with achieved HBM GB/s (% of peak) vs dense",
        "value": round(B / (ms_step * 1e-3), 1), "unit": "seqs*steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "step_ms_percentiles": pct,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if elt == 2 else "f32",
        "data": "synthetic (seeded N(0,1) K/V/q with planted tokens), paged in a random page order",
        "config": cfg, "step_bytes": step_bytes, "step_gbps": gbps(step_bytes, ms_step),
        "sparse_layer_step": {"ms": round(ms_sparse, 5), "value": round(B / (ms_sparse * 1e-3), 1),
                              "gbps": sparse_gbps, "speedup_vs_dense": round(ms_dense / ms_sparse, 3)},
        "selection_layer": {"ms": round(ms_layer, 5), "call": "ksa_paged_vote_layer_decode"},
        "dense": {"ms_per_step": round(ms_dense, 5), "value": round(B / (ms_dense * 1e-3), 1),
                  "gbps": gbps(dense_bytes, ms_dense)},
        "speedup_vs_dense": round(ms_dense / ms_step, 3),
        "roofline": {"kernel": "ksa_paged_sparse_decode over the shared set (sparse layer)",
                     "bound": "hbm", "achieved": sparse_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(sparse_gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "avg_launch_ms": round(ms_sparse, 5), "bytes_per_launch": sparse_bytes},
        "cpu_baseline": None,
        "input_gen_s": round(gen_s, 2),
    }
    print(json.dumps(line), flush=True)


def schedule_main(args):
    """One decode step of a whole LessIsMore model at the c4 shape: layers 0
    and 1 attend densely, layer 2 and every --select-every-th layer after it
    is a selection layer (dense attention plus the vote, one K read:
    ksa_vote_layer_decode), and every other layer attends the set chosen by
    the last selection layer (ksa_sparse_decode, TOKENS).  Each layer has
    its own KV cache (distinct caches are cycled so no layer reads bytes the
    previous ones left in the caches).  Compared with every layer dense."""
    import torch

    import sparse_attention_decode_ksa_amd as ksa
    from sparse_attention_decode_ksa_amd.inputs import WORKLOADS, make_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    lib = ksa.load_library()
    R = Runner(lib, ksa)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOADS["c4"]
    B, Hq, Hkv, D, T, N, W = w.B, w.Hq, w.Hkv, w.D, w.T, w.token_budget, w.recent_window
    nL, every = args.schedule_layers, args.select_every
    kinds = []
    for l in range(nL):
        if l < 2:
            kinds.append("dense")
        elif (l - 2) % every == 0:
            kinds.append("select")
        else:
            kinds.append("sparse")
    ncache = args.layers or 8
    t0 = time.time()
    C = [make_inputs(w, device=dev, seed=w.seed * 1000 + c) for c in range(ncache)]
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    prob = ksa.Problem(B, Hq, Hkv, D, T, w.cap, 1, ksa.KSA_BF16, 0.0)
    pp = ctypes.byref(prob)
    stream = torch.cuda.Stream(device=dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    V = lambda t: ctypes.c_void_p(t.data_ptr())
    n_sel = min(N, T)
    ws_layer = ksa.new_workspace(ksa.ksa_workspace_bytes(prob, ksa.KSA_OP_VOTE_LAYER, N), dev)
    ws_attn = ksa.new_workspace(max(ksa.ksa_workspace_bytes(prob, ksa.KSA_OP_SPARSE_TOKENS, n_sel),
                                    ksa.ksa_workspace_bytes(prob, ksa.KSA_OP_DENSE, 0)), dev)
    idx = torch.empty((B, n_sel), dtype=torch.int32, device=dev)
    sel = ksa.Selection(ksa.KSA_SEL_TOKENS, V(idx).value, n_sel)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    calls, dense_calls = [], []
    for l, kind in enumerate(kinds):
        x = C[l % ncache]
        dense = (lib.ksa_dense_decode, (pp, V(x["q"]), V(x["k"]), V(x["v"]), V(out), V(lse),
                                        V(ws_attn), ws_attn.numel(), sp))
        dense_calls.append(dense)
        if kind == "dense":
            calls.append(dense)
        elif kind == "select":
            calls.append((lib.ksa_vote_layer_decode,
                          (pp, V(x["q"]), V(x["k"]), V(x["v"]), N, W, V(out), V(lse), V(idx), None,
                           V(ws_layer), ws_layer.numel(), sp)))
        else:
            calls.append((lib.ksa_sparse_decode,
                          (pp, V(x["q"]), V(x["k"]), V(x["v"]), ctypes.byref(sel), V(out), V(lse),
                           V(ws_attn), ws_attn.numel(), sp)))

    def model_step(i):
        for c in calls:
            R.run(c)

    def dense_step(i):
        for c in dense_calls:
            R.run(c)

    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        warm(torch, model_step, max(1, args.warmup // 4), args.warm_seconds)
        steps = max(2, args.steps // 10)
        ms_model = timed(torch, stream, steps, model_step)
        warm(torch, dense_step, 1, args.warm_seconds)
        ms_dense = timed(torch, stream, max(2, args.dense_steps // 4), dense_step)
    per_layer = ms_model / nL
    cfg = {"workload": "c4 shape, LessIsMore schedule: %d layers, 2 dense, a selection layer every "
                       "%d from layer 2, sparse layers between" % (nL, every),
           "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "context": T,
           "token_budget": N, "recent_window": W, "layers": nL,
           "selection_layers": kinds.count("select"), "sparse_layers": kinds.count("sparse"),
           "kv_caches_cycled": ncache}
    line = {
        "metric": "decode seqs*steps/s per layer, amortized over the layer schedule, vs every "
                  "layer dense",
        "value": round(B / (per_layer * 1e-3), 1), "unit": "seqs*steps/s", "n_gpus": 1,
        "steps": steps, "warmup": max(1, args.warmup // 4), "ms_per_step": round(ms_model, 5),
        "ms_per_layer": round(per_layer, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) K/V/q with planted tokens)", "config": cfg,
        "dense": {"ms_per_step": round(ms_dense, 5), "ms_per_layer": round(ms_dense / nL, 5)},
        "speedup_vs_dense": round(ms_dense / ms_model, 3),
        "roofline": None, "cpu_baseline": None, "input_gen_s": round(gen_s, 2),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
