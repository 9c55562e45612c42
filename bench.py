"""Benchmark of one DSA sparse decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c1_l32k]

A step is the whole hot path for one batch: fp8 indexer scores over every
cached token (the bf16 indexer queries quantized in the kernel), exact
top-2048 (per split, then merged), split-K sparse absorbed-MLA attention over
the selected paged fp8 rows (QK on bf16 matrix cores with the bf16 query as it
is), and the LSE merge.  Inputs are seeded synthetic tensors already resident
in HBM.  Prints ONE JSON line (rank 0).

The default workload is bulk decode at the metric's point: 64 requests, one
query row each, 32768 cached tokens each, 256-token pages shuffled in the
pool, 64 x 128 fp8 indexer, 32 MLA heads over 576-wide fp8 rows, top-2048.

Timing: W untimed steps, then K steps between two device synchronisations,
replayed from HIP graphs (``--eager`` launches the kernels directly instead).
Consecutive steps cycle through ``--rotate`` independent input sets (default
3), so that no step re-reads bytes the one before left in the chip's 256 MB
memory-side cache: every step reads its inputs from HBM, as the layers of a
real decode step do.  Then every kernel is replayed back to back from a graph
of 20 launches (cycling through the input sets) between two HIP events on the
stream it runs on, for per-kernel durations and the roofline of the dominant
kernel.  The cache write (the step before the path: one new token per request
into the paged caches) and the merge fused with the W_UV value projection (the
step after it) are timed the same way and reported on their own; they are
not part of the step.  The oracle (fp64, CPU) is timed on a bounded sample of
the same workload as a reported baseline.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DSA decode steps/s (index+top-k+sparse MLA) at B=64 L=32k; % peak HBM BW"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 MFMA, vendor figure (no sparsity)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c1_l32k")
    ap.add_argument("--index-splits", type=int, default=None)
    ap.add_argument("--attn-splits", type=int, default=None)
    ap.add_argument("--eager", action="store_true", help="launch kernels directly, no HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle sample")
    ap.add_argument("--cpu-seconds-1t", type=float, default=4.0, help="budget of the one-thread oracle sample")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the bandwidth kernels and the MTP-verify indexer measurement")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--rotate", type=int, default=3,
                    help="independent input sets that consecutive steps and launches cycle through, "
                         "so that no launch re-reads what the one before left in the memory-side cache")
    return ap.parse_args()


CACHE_WRITE_BYTES_PER_TOKEN = 1024 + 128 + 256 + 256 + 12 + 580 + 132


def merge_project_bytes(inp, n_splits: int) -> int:
    """Per (row, head): S bf16 partials of 512 and S lse read, 128 bf16 and
    one lse written; the bf16 weights [H, 128, 512] once."""
    r, h = inp.n_rows, inp.mla_heads
    return r * h * (n_splits * (512 * 2 + 4) + 128 * 2 + 4) + h * 128 * 512 * 2


def algorithmic_bytes(inp) -> dict:
    """Bytes the method must move per step, from the actual geometry.

    Per row with V visible slots: 132 B per slot of index key + scale and
    4 B per page-table entry, the bf16 indexer query (64 x 128 x 2) and head
    weights (64 x 4), 580 B per selected MLA row + scale, the bf16 MLA query
    (H x 576 x 2), the bf16 output (H x 512 x 2) and its lse (H x 4).  Rows
    scored together (a group of query rows of one request: MTP verify,
    prefill) share their keys, which count once, at the group's longest span.
    Intermediates (scores, top-k lists, split partials) are not counted.
    The indexer kernel's share is the first part; its fp8 contraction does
    2 x 64 x 128 flops per visible slot of a row.
    """
    vis = inp.row_vis.cpu().tolist()
    p, k, h, g = inp.page_size, inp.top_k, inp.mla_heads, inp.cfg.group_rows
    c = inp.cfg.index_share
    if c > 1:
        # MTP IndexShare: only each chain's first row is scored, and the
        # chain's rows attend one list, whose rows count once per chain.
        lead = vis[::c]
        keys = sum(132 * m + 4 * math.ceil(m / p) for m in lead)
        idx = keys + len(lead) * (64 * 128 * 2 + 64 * 4)
        mla = sum(580 * min(v, k) for v in lead) + len(vis) * (h * 576 * 2 + h * 512 * 2 + h * 4)
        return {"step": idx + mla, "index_kernel": idx, "index_flops": sum(2 * 64 * 128 * v for v in lead)}
    keys = sum(132 * m + 4 * math.ceil(m / p) for m in (max(vis[i:i + g]) for i in range(0, len(vis), g)))
    idx = keys + len(vis) * (64 * 128 * 2 + 64 * 4)
    mla = sum(580 * min(v, k) + h * 576 * 2 + h * 512 * 2 + h * 4 for v in vis)
    return {"step": idx + mla, "index_kernel": idx, "index_flops": sum(2 * 64 * 128 * v for v in vis)}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _time_oracle_rows(inps, seconds: float):
    """The oracle on one row at a time of the workload (every 8th row first,
    then the rest, input set after input set) until `seconds` of CPU work are
    done; returns (rows, seconds)."""
    from oracle import dsa_oracle as O
    from sparse_attention_decode_dsa_amd import workload as W

    n_rows = inps[0].n_rows
    rows = list(range(n_rows))
    order = rows[::8] + [r for r in rows if r % 8]
    done, t_total = 0, 0.0
    for inp in inps:
        for r in order:
            sub = W.as_numpy(W.subset(inp, [r]))
            t0 = time.perf_counter()
            O.decode_step(sub, inp.cfg.index_splits, inp.cfg.attn_splits)
            t_total += time.perf_counter() - t0
            done += 1
            if t_total >= seconds:
                return done, t_total
    return done, t_total


def cpu_baseline(inps, seconds: float, one_thread_seconds: float) -> dict:
    """The oracle, as it stands, on rows of the same workload (the rotated
    input sets in turn) until the time budget is spent, with its BLAS pool
    pinned to every core this process may run on; then again with one
    thread.  Scaled to steps/s of the full batch."""
    from threadpoolctl import threadpool_limits

    n_rows = inps[0].n_rows
    affinity = len(os.sched_getaffinity(0))
    # The host's share of cores: OMP_NUM_THREADS where the environment sets
    # one (the GPU machines do), else every core the process may run on.
    cores = min(affinity, int(os.environ.get("OMP_NUM_THREADS", affinity) or affinity))
    with threadpool_limits(limits=cores):
        done, t_total = _time_oracle_rows(inps, seconds)
    with threadpool_limits(limits=1):
        done1, t1 = _time_oracle_rows(inps, one_thread_seconds)
    return {"value": done / t_total / n_rows, "unit": "steps/s", "cores": cores,
            "affinity_cores": affinity, "cpu_model": _cpu_model(), "kind": "oracle",
            "sample": f"{done} rows ({done / n_rows:.2f} steps of {n_rows} rows, over "
                      f"{len(inps)} input sets), timed one row at a time ({t_total:.1f} s) with "
                      f"{cores} BLAS threads, scaled to whole steps",
            "one_thread": {"value": done1 / t1 / n_rows, "unit": "steps/s",
                           "sample": f"{done1} rows timed one at a time ({t1:.1f} s), 1 thread"}}


def measure_bandwidth(dev, nbytes: int, reps: int = 20) -> dict:
    """Plain streaming-read and copy kernels (libdsa_bw.so) over `nbytes`,
    cycling through four buffers (more than the chip's 256 MB memory-side
    cache holds in total), timed like the step's kernels: a graph of `reps`
    launches replayed between two HIP events on the launch stream.  Copy
    counts the bytes read plus the bytes written."""
    import ctypes

    import torch

    from sparse_attention_decode_dsa_amd import build as B

    L = ctypes.CDLL(B.BW_LIB)
    L.dsa_bw_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p,
                                     ctypes.c_void_p]
    L.dsa_bw_stream_read_nt.argtypes = L.dsa_bw_stream_read.argtypes
    L.dsa_bw_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p]
    nbytes = nbytes // 16 * 16
    bufs = [torch.ones(nbytes // 4, dtype=torch.float32, device=dev) for _ in range(4)]
    sink = torch.empty(4096 * 256, dtype=torch.int32, device=dev)

    def timed(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for j in range(4):
                fn(j, side.cuda_stream)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st = torch.cuda.current_stream().cuda_stream
            for j in range(reps):
                fn(j % 4, st)
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        stream = torch.cuda.current_stream()
        e0.record(stream)
        for _ in range(3):
            g.replay()
        e1.record(stream)
        e1.synchronize()
        return 1e3 * e0.elapsed_time(e1) / (3 * reps)

    best_read, best_nt, best_copy = 0.0, 0.0, 0.0
    for wgs in (512, 1024, 2048):
        us = timed(lambda j, st: L.dsa_bw_stream_read(bufs[j].data_ptr(), nbytes, wgs, sink.data_ptr(), st))
        best_read = max(best_read, nbytes / us / 1e3)
        us = timed(lambda j, st: L.dsa_bw_stream_read_nt(bufs[j].data_ptr(), nbytes, wgs, sink.data_ptr(), st))
        best_nt = max(best_nt, nbytes / us / 1e3)
        us = timed(lambda j, st: L.dsa_bw_copy(bufs[j].data_ptr(), bufs[(j + 1) % 4].data_ptr(), nbytes, wgs, st))
        best_copy = max(best_copy, 2 * nbytes / us / 1e3)
    del bufs, sink
    torch.cuda.synchronize()
    return {"stream_read_GBps": round(max(best_read, best_nt), 1), "stream_read_plain_GBps": round(best_read, 1),
            "stream_read_nt_GBps": round(best_nt, 1), "copy_GBps": round(best_copy, 1), "bytes": nbytes,
            "how": "libdsa_bw.so kernels, 256-thread workgroups, best of 512/1024/2048 workgroups, "
                   "four buffers in turn; stream_read is the faster of plain and non-temporal loads; "
                   "copy counts bytes read + written"}


def c3_indexer(dev, seed: int, reps: int = 20) -> dict:
    """The multi-row indexer at the MTP-verify workload (32 requests x 6
    causal rows, kv_len U[16384, 65536], groups of 6 rows), timed like the
    step's kernels over two input sets, against the dense fp8 MFMA peak."""
    import torch

    from sparse_attention_decode_dsa_amd import dsa
    from sparse_attention_decode_dsa_amd import workload as W

    inps = [W.make("c3", seed=seed + k, device=dev) for k in range(2)]
    steps = [dsa.DecodeStep(x) for x in inps]
    fns = [lambda i=i, st=st: dsa.index_scores(
        i.q_idx, i.head_w, i.k_code, i.k_scale, i.page_table, i.kv_lens, i.row_req, i.row_vis,
        group_rows=st.group_rows, score_stride=st.score_stride, scores=st.scores, status=st.status)
        for i, st in zip(inps, steps)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for fn in fns:
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for j in range(reps):
            fns[j % 2]()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        g.replay()
    e1.record(stream)
    e1.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / (3 * reps)
    for st in steps:
        dsa.check_status(st.status)
    flops = sum(algorithmic_bytes(x)["index_flops"] for x in inps) / 2
    tflops = flops / (us * 1e-6) / 1e12
    out = {"workload": "c3: 32 requests x 6 causal MTP rows, kv_len U[16384, 65536], rows scored in groups of 6",
           "us_per_launch": round(us, 2), "fp8_flops_per_launch": flops, "achieved_TFLOPs": round(tflops, 1),
           "peak_TFLOPs": FP8_PEAK_TFLOPS, "frac": round(tflops / FP8_PEAK_TFLOPS, 4)}
    del inps, steps
    torch.cuda.synchronize()
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only (one process, one MI355X); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_attention_decode_dsa_amd import dsa
    from sparse_attention_decode_dsa_amd import workload as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n_sets = max(1, args.rotate)
    base_seed = args.seed if args.seed is not None else sum(map(ord, args.config))
    inps = [W.make(args.config, seed=base_seed + k, device=dev) for k in range(n_sets)]
    steps = [dsa.DecodeStep(x, args.index_splits, args.attn_splits) for x in inps]
    inp, step = inps[0], steps[0]
    stream = torch.cuda.current_stream()

    # Correctness gate before timing: one eager step per input set, no device faults.
    for st in steps:
        st.run()
    torch.cuda.synchronize()
    for st in steps:
        dsa.check_status(st.status)

    if args.calib_copy_mb:
        n = args.calib_copy_mb * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # A graph of one step per input set (a round), and one graph per single
    # step for the remainder, so that exactly K steps run.
    round_graph, single = None, []
    if not args.eager:
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            for _ in range(2):
                for st in steps:
                    st.run()
        stream.wait_stream(s)
        torch.cuda.synchronize()
        round_graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(round_graph):
            for st in steps:
                st.run()
        for st in steps:
            g1 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g1):
                st.run()
            single.append(g1)
        torch.cuda.synchronize()

    def run_steps(k):
        if round_graph is not None:
            for _ in range(k // n_sets):
                round_graph.replay()
            for j in range(k % n_sets):
                single[j].replay()
        else:
            for j in range(k):
                steps[j % n_sets].run()

    run_steps(args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(args.steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed * 1e3 / args.steps
    for st in steps:
        dsa.check_status(st.status)

    # Per-kernel durations: each kernel launched 20 times back to back from a
    # HIP graph, the launches cycling through the input sets (each set's
    # launch reads that set's inputs and rewrites its outputs), the graph
    # replayed K/4 times on the launch stream between two HIP events,
    # averaged per launch.
    def kernel_launches(i, st):
        if st.index_topk:
            # The step's own two kernels: the indexer with its candidate
            # epilogue, then the merge (dsa_index_topk's two phases).
            def fused(phases):
                return lambda: dsa.index_topk(
                    st.lead_q, st.lead_w, i.k_code, i.k_scale, i.page_table, i.kv_lens, st.lead_req,
                    st.lead_vis, i.top_k, score_stride=st.score_stride, scores=st.scores,
                    workspace=st.workspace, topk_idx=st.topk_idx, topk_count=st.topk_count,
                    status=st.status, phases=phases)
            fns = {"index_scores": fused(dsa.PHASE_SCORE), "topk": fused(dsa.PHASE_SELECT)}
        else:
            fns = {
                "index_scores": lambda: dsa.index_scores(
                    st.lead_q, st.lead_w, i.k_code, i.k_scale, i.page_table, i.kv_lens,
                    st.lead_req, st.lead_vis, group_rows=st.group_rows, score_stride=st.score_stride,
                    scores=st.scores, status=st.status, whole_rows=st.whole_rows),
                "topk": lambda: dsa.topk(st.scores, st.lead_vis, i.top_k, st.index_splits,
                                         workspace=st.workspace, topk_idx=st.topk_idx,
                                         topk_count=st.topk_count, status=st.status),
            }
        if st.row_list is not None:
            s_ = st.attn_splits
            fns["sparse_mla"] = lambda: dsa.sparse_mla_decode_shared(
                i.q_mla, i.kv_cache, i.page_table, i.row_req, i.row_vis, st.row_list, st.topk_idx,
                st.topk_count, s_, i.sm_scale, part_o=st.part_o, part_lse=st.part_lse, out=st.out,
                out_lse=st.out_lse, status=st.status)
            if s_ > 1:
                fns["lse_merge"] = lambda: dsa.lse_merge(st.part_o, st.part_lse, out=st.out, out_lse=st.out_lse)
        elif st.attn_splits == 1:
            fns["sparse_mla"] = lambda: dsa.sparse_mla_decode(
                i.q_mla, i.kv_cache, i.page_table, i.row_req, i.row_vis,
                st.topk_idx, st.topk_count, 1, i.sm_scale, out=st.out, out_lse=st.out_lse,
                status=st.status)
        else:
            fns["sparse_mla"] = lambda: dsa.sparse_mla_decode(
                i.q_mla, i.kv_cache, i.page_table, i.row_req, i.row_vis,
                st.topk_idx, st.topk_count, st.attn_splits, i.sm_scale, part_o=st.part_o,
                part_lse=st.part_lse, status=st.status)
            fns["lse_merge"] = lambda: dsa.lse_merge(st.part_o, st.part_lse, out=st.out,
                                                     out_lse=st.out_lse)
        # The step before the path, timed on its own: one new token per
        # request, written at its last slot (kv_len - 1) with the rope part
        # rotated.  It runs after the timed steps, so they never see it.
        if st.attn_splits > 1:
            # The step after the path, timed on its own: the merge fused with
            # the W_UV value projection (it would replace lse_merge).
            fns["lse_merge_project"] = lambda: dsa.lse_merge_project(
                st.part_o, st.part_lse, w_uv[id(i)], out=proj_out[id(i)], out_lse=st.out_lse)
        nt = new_tokens[id(i)]
        fns["cache_write"] = lambda: dsa.cache_write(
            nt.latent, nt.rope, nt.index_k, nt.tok_req, nt.tok_slot, i.page_table, i.kv_cache,
            i.k_code, i.k_scale, rope_cos=nt.rope_cos, rope_sin=nt.rope_sin, status=st.status)
        return fns

    new_tokens, w_uv, proj_out = {}, {}, {}
    for k, x in enumerate(inps):
        w_uv[id(x)] = W.make_w_uv(x.mla_heads, seed=base_seed + k, device=dev)
        proj_out[id(x)] = torch.empty((x.n_rows, x.mla_heads, W.D_V), dtype=torch.bfloat16, device=dev)
        live = torch.nonzero(x.kv_lens > 0).flatten().cpu()
        new_tokens[id(x)] = W.make_new_tokens(x, live, (x.kv_lens[live] - 1).cpu(), seed=base_seed + k)
    n_new = int(new_tokens[id(inps[0])].tok_req.shape[0])
    per_set = [kernel_launches(x, st) for x, st in zip(inps, steps)]
    kern_us = {}
    reps = 20
    for n in per_set[0]:
        fns = [d[n] for d in per_set]
        g = None
        if not args.eager:
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                for fn in fns:
                    fn()
            stream.wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for j in range(reps):
                    fns[j % n_sets]()
            torch.cuda.synchronize()
        n_iter = max(1, args.steps // 4)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n_iter):
            if g is not None:
                g.replay()
            else:
                for j in range(reps):
                    fns[j % n_sets]()
        e1.record(stream)
        e1.synchronize()
        kern_us[n] = 1e3 * e0.elapsed_time(e1) / (n_iter * reps)
    torch.cuda.synchronize()
    for st in steps:
        dsa.check_status(st.status)

    ab = algorithmic_bytes(inp)
    idx_us = kern_us["index_scores"]
    achieved = ab["index_kernel"] / (idx_us * 1e-6) / 1e9
    # Several query rows per key (MTP verify, prefill): the indexer is a dense
    # fp8 contraction, and its roofline is the MFMA peak.
    multi = step.group_rows > 1
    tflops = ab["index_flops"] / (idx_us * 1e-6) / 1e12
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "index_scores_c1_l32k_traffic.json")
    if os.path.exists(tfile) and args.config == "c1_l32k":
        with open(tfile) as f:
            t = json.load(f)
        if t.get("kernel_source_sha") == _kernel_sha():
            traffic = t.get("bytes_per_launch")

    line = {
        "metric": METRIC,
        "value": 1e3 / ms,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {
            "workload": f"{args.config}: {inp.n_rows} query rows, kv_len "
                        f"{int(inp.row_vis.min())}..{int(inp.row_vis.max())}, top-{inp.top_k}, "
                        f"indexer 64x128 fp8, MLA {inp.mla_heads} heads x 576 fp8, page {inp.page_size}",
            "batch": inp.n_rows, "kv_len_max": int(inp.row_vis.max()), "top_k": inp.top_k,
            "page_size": inp.page_size, "mla_heads": inp.mla_heads,
            "index_splits": "in the indexer's chunks" if step.index_topk else step.index_splits,
            "attn_splits": step.attn_splits,
            "launch": "eager" if round_graph is None else "hipgraph",
            "input_sets": n_sets,
        },
        "roofline": ({
            "kernel": "index_scores",
            "bound": "mfma",
            "achieved": tflops,
            "peak": FP8_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / FP8_PEAK_TFLOPS,
            "traffic": None,
            "hbm_GBps": achieved,
        } if multi else {
            "kernel": "index_scores",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
        }),
        "step_algorithmic_bytes": ab["step"],
        "step_hbm_frac": ab["step"] / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "kernels_us": {n: round(v, 2) for n, v in kern_us.items()},
        # The step before the path (not in the step above): per new token it
        # reads 1024 + 128 + 256 B of bf16 rows, a 256 B cos/sin row, 12 B of
        # request, slot and page id, and writes 580 + 132 B of codes and scales.
        "lse_merge_project": (None if "lse_merge_project" not in kern_us else {
            "us_per_launch": round(kern_us["lse_merge_project"], 2),
            "algorithmic_bytes": merge_project_bytes(inp, steps[0].attn_splits),
            "achieved_GBps": round(merge_project_bytes(inp, steps[0].attn_splits)
                                   / (kern_us["lse_merge_project"] * 1e3), 1),
            "bound": "hbm",
        }),
        "cache_write": {
            "tokens": n_new,
            "us_per_launch": round(kern_us["cache_write"], 2),
            "algorithmic_bytes": CACHE_WRITE_BYTES_PER_TOKEN * n_new,
            "achieved_GBps": round(CACHE_WRITE_BYTES_PER_TOKEN * n_new / (kern_us["cache_write"] * 1e3), 1),
            "bound": "latency",
        },
    }
    if not args.no_extras:
        bw = measure_bandwidth(dev, ab["index_kernel"])
        line["roofline"]["measured"] = bw
        if line["roofline"]["unit"] == "GB/s":
            line["roofline"]["frac_of_measured_read"] = round(achieved / bw["stream_read_GBps"], 4)
        line["step_frac_of_measured_read"] = round(ab["step"] / (ms * 1e-3) / (bw["stream_read_GBps"] * 1e9), 4)
        if args.config != "c3":
            line["c3_indexer_mfma"] = c3_indexer(dev, base_seed + 100)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inps, args.cpu_seconds, args.cpu_seconds_1t)
    print(json.dumps(line), flush=True)


def _kernel_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ("index_scores.hip", "device_common.h"):
        with open(os.path.join(ROOT, "sparse_attention_decode_dsa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
