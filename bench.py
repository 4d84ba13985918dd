"""Throughput of the sparse-attention hot path on one MI355X.

    python bench.py [--workload decode64k|decode1m|batched|prefill128k]
                    [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

A step is one pass of the whole path over one batch of synthetic input
(inputs already resident in GPU memory):
  decode64k : indexer scores + top-p(0.9) select (+4 sink, +512 window) +
              split-KV sparse decode; B=1, 32/4 heads, d=128, L=65536, bf16
  decode1m  : Taylor page scores + top-32 pages + sparse decode; L=2^20
  batched   : as decode64k for 32 sequences of 16K-128K tokens, 32/8 heads
  prefill128k: block top-k(2048) selection + block-sparse causal prefill
Prints one JSON line.  The value is the algorithmic HBM bytes of the step
(indexer keys or page statistics, plus the selected K/V rows) per second for
the decode workloads, and selected-block FLOP/s for prefill.
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

METRIC = ("sparse decode µs/step + HBM GB/s at 64K/1M; sparse prefill TFLOP/s at 128K")
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode64k",
                    choices=["decode64k", "decode1m", "batched", "prefill128k",
                             "prefill32k_query"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--warm", action="store_true",
                    help="reuse one input replica every step (cache-warm)")
    ap.add_argument("--rla", action="store_true",
                    help="decode workloads: the step also forms the residual linear attention "
                         "over the unselected tokens (sa_decode_step_rla; state built first)")
    ap.add_argument("--policy", default="indexer", choices=["indexer", "oracle"],
                    help="token-level decode workloads: take the support from the low-rank "
                         "indexer (default) or from the dense head-averaged attention mass "
                         "(the attention-mass oracle: sa_attention_mass + sa_select_topp)")
    ap.add_argument("--selection", default="indexer", choices=["indexer", "pbs", "oracle"],
                    help="prefill128k: block supports from the low-rank indexer (default) or from "
                         "the segment-permuted mean-pooled blocks (sa_pbs_*; segments of 2048, "
                         "importance from the last 64 queries, top-32 blocks); prefill32k_query: "
                         "oracle = per-query supports from the dense attention mass "
                         "(sa_select_prefill_oracle)")
    ap.add_argument("--coverage", action="store_true",
                    help="prefill128k: also report the dense attention mass the supports keep on "
                         "8 sampled (query block, group) items (float64 on the host, untimed)")
    ap.add_argument("--aggregate", default="logits", choices=["logits", "probs"],
                    help="prefill32k_query: rank by the head-collapsed logits or by the mean of "
                         "the heads' probabilities (sa_select_prefill_topk_probs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device copy (5 dispatches): the reference "
                         "for scaling FETCH_SIZE / WRITE_SIZE counter readings to bytes")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_loop(fn, n, warmup=3, reps=1):
    """Average device milliseconds per call of fn(i).

    At least 16 calls fn(i % reps) (rotating over the input replicas) are
    captured once into a HIP graph on a side stream (every library call
    launches on the current stream), and the graph is replayed until n calls
    have run, timed with HIP events on that stream: the figure excludes Python
    and graph-launch overhead between calls, not the gaps between kernels."""
    import torch
    per_graph = max(reps, 16)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(max(warmup, 1)):
            fn(i % reps)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(per_graph):
            fn(i % reps)
    torch.cuda.synchronize()
    n_rep = max(1, math.ceil(n / per_graph))
    with torch.cuda.stream(s):
        for _ in range(max(1, warmup // per_graph)):
            g.replay()
        a, b = _events()
        a.record(s)
        for _ in range(n_rep):
            g.replay()
        b.record(s)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (n_rep * per_graph)


# Kernel -> the sources its code comes from (a counter reading is only used
# while these are unchanged).
KERNEL_SOURCES = {
    "decode_step (single fused launch)": ["fused.hip"],
    "decode_step_pages (single fused launch)": ["fused.hip"],
    "page_scores": ["index.hip"],
    "index_scores": ["index.hip"],
    "sparse_decode": ["decode.hip"],
    "sparse_decode_rla": ["decode.hip"],
    "sparse_prefill": ["prefill.hip"],
    "attention_mass": ["mass.hip"],
    "sparse_prefill_query": ["decode.hip", "prefill.hip"],
    "pbs_select": ["pbs.hip", "mass.hip", "select.hip"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def source_digest(files):
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dynamic_sparse_attention_02_amd", "csrc")
    for f in sorted(files) + ["sa_internal.h"]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter record (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's
    reading), or None if there is none or the kernel's sources changed."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel") != kernel:
        return None
    if rec.get("source_digest") != source_digest(KERNEL_SOURCES.get(kernel, [])):
        return None
    return rec.get("traffic_bytes")


def calibrate_copy():
    """A plain device-to-device copy of 1 GiB, 5 dispatches."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"calibration": "device copy", "bytes_read": n, "bytes_written": n, "dispatches": 5}


def fill_kidx(ops, shape, inp, kidx_pool):
    """Indexer keys of every pool row through sa_index_append (cache
    maintenance, outside the timed region)."""
    import torch
    P, Hkv, page, d = inp.k_pool.shape
    step = max(1, (1 << 26) // (page * Hkv * d))
    for p0 in range(0, P, step):
        p1 = min(P, p0 + step)
        k_pre = inp.k_pool[p0:p1].permute(0, 2, 1, 3).reshape(-1, Hkv, d).contiguous()
        slot = torch.arange(p0 * page, p1 * page, device=k_pre.device, dtype=torch.int64)
        ops.sa_index_append(shape, k_pre, inp.w_k, slot, kidx_pool)


def cpu_threads_info():
    return len(os.sched_getaffinity(0))


def blas_threads():
    """Threads numpy's BLAS runs with (its default: the oracle is timed as it
    stands); the rest of the oracle (sorts, Python loops) is single-threaded."""
    from threadpoolctl import threadpool_info
    n = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    return max(n) if n else 1


# ---------------------------------------------------------------------------
# decode workloads
# ---------------------------------------------------------------------------


def bench_decode(args, name):
    import numpy as np
    import torch

    import synth
    from dynamic_sparse_attention_02_amd import _lib as L
    from dynamic_sparse_attention_02_amd import ops

    dev = "cuda"
    if name == "decode64k":
        inp = synth.make_decode64k(device="cpu").to(dev)  # CPU draw keeps the budget fixed
    elif name == "batched":
        inp = synth.make_batched_decode(device=dev)
    else:
        inp = synth.make_decode1m(device=dev)
    B, Hq, Hkv, d = inp.B, inp.H_q, inp.H_kv, inp.d
    rows = B * Hkv
    Lmax = max(inp.seq_lens)
    shape = ops.make_shape(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                           max_pages=inp.max_pages, max_len=Lmax, n_pool_pages=inp.n_pages)
    lens = inp.seq_lens_tensor()
    pages = ops.make_pages(inp.page_table, lens)
    page_mode = name == "decode1m"
    oracle_policy = args.policy == "oracle"
    if oracle_policy and page_mode:
        raise SystemExit("--policy oracle takes a token-level workload (decode64k or batched)")
    sel = inp.select
    n_sink, n_window = sel.get("n_sink", 0), sel.get("n_window", 0)

    if page_mode:
        stats = torch.empty((inp.n_pages, Hkv, 2, d), dtype=inp.dtype, device=dev)
        pid = torch.arange(inp.n_pages, dtype=torch.int32, device=dev)
        nval = torch.full((inp.n_pages,), 64, dtype=torch.int32, device=dev)
        ops.sa_page_stats(shape, inp.k_pool, pid, nval, stats)
        cache_a = stats
        k_pages = sel["k_pages"]
        cap = k_pages * 64
        n_cand = inp.max_pages
        x = torch.empty((rows, n_cand), dtype=torch.float32, device=dev)
        per_row_index_bytes = [math.ceil(L / 64) * 2 * d * 2 for L in inp.seq_lens]
    else:
        kidx = torch.zeros((inp.n_pages, Hkv, 64, 16), dtype=inp.dtype, device=dev)
        fill_kidx(ops, shape, inp, kidx)
        cache_a = kidx
        cap = Lmax
        x = torch.empty((rows, Lmax), dtype=torch.float32, device=dev)
        # indexer: the 32 B K~ row of every token; oracle: the full K row
        per_row_index_bytes = [L * (d * 2 if oracle_policy else 16 * 2) for L in inp.seq_lens]
    idx = torch.empty((rows, cap), dtype=torch.int32, device=dev)
    count = torch.empty((rows,), dtype=torch.int32, device=dev)
    out = torch.empty((B, Hq, d), dtype=inp.dtype, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws_sel = ops.alloc_workspace(ops.workspace_size(L.SA_OP_SELECT, shape, x.shape[1]))
    ws_dec = ops.alloc_workspace(ops.workspace_size(L.SA_OP_SPARSE_DECODE, shape, cap))
    ws_idx = ops.alloc_workspace(ops.workspace_size(L.SA_OP_INDEX_SCORES, shape, 0))
    ws_mass = (ops.alloc_workspace(ops.workspace_size(L.SA_OP_ATTENTION_MASS, shape, 0))
               if not page_mode else None)

    # bytes a step must touch (index part: all of it; K/V: the selected rows)
    def run_select(rep):
        a, kp, vp = rep
        if page_mode:
            ops.sa_page_scores(shape, pages, inp.q, a, inp.s_att, x)
            ops.sa_select_topk(shape, pages, x, k_pages, 64, 0, 0, idx, count, ws_sel)
        elif oracle_policy:
            ops.sa_attention_mass(shape, pages, inp.q, kp, inp.s_att, x, ws_mass)
            ops.sa_select_topp(shape, pages, x, sel["p"], n_sink, n_window, idx, count, ws_sel)
        else:
            ops.sa_index_scores(shape, pages, inp.q, inp.w_q, a, inp.s_idx, x, ws_idx)
            ops.sa_select_topp(shape, pages, x, sel["p"], n_sink, n_window, idx, count, ws_sel)

    # the whole-step call (token-level indexer or page-level Taylor scores)
    use_step = not oracle_policy and not (args.rla and page_mode)
    if args.rla:  # state of every sequence's cache (maintenance, outside the timed steps)
        rla_state = torch.zeros((B, Hkv, d + 1, d), dtype=torch.float32, device=dev)
        ops.sa_rla_state(shape, pages, inp.k_pool, inp.v_pool, 0, rla_state)
        rla_num = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        rla_den = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        ws_dec = ops.alloc_workspace(ops.workspace_size(L.SA_OP_SPARSE_DECODE_RLA, shape, cap))
        state_bytes = rla_state.numel() * 4
    if use_step:
        ws_step = ops.alloc_workspace(ops.workspace_size(
            L.SA_OP_DECODE_STEP_PAGES if page_mode else
            (L.SA_OP_DECODE_STEP_RLA if args.rla else L.SA_OP_DECODE_STEP), shape, cap))
    fused = use_step and rows <= 16 and inp.G >= 4
    if page_mode:
        fused = fused and k_pages <= 32 and inp.dtype == torch.bfloat16
    if args.rla:
        fused = fused and inp.dtype == torch.bfloat16

    def run_step(rep):
        if use_step and page_mode:
            ops.sa_decode_step_pages(shape, pages, inp.q, rep[0], rep[1], rep[2], inp.s_att,
                                     k_pages, x, idx, count, out, lse, ws_step)
            return
        if use_step and args.rla:
            ops.sa_decode_step_rla(shape, pages, inp.q, inp.w_q, rep[0], rep[1], rep[2],
                                   inp.s_idx, inp.s_att, sel.get("p", 0.0), 0, n_sink, n_window,
                                   x, idx, count, out, lse, rla_state, rla_num, rla_den, ws_step)
            return
        if use_step:
            ops.sa_decode_step(shape, pages, inp.q, inp.w_q, rep[0], rep[1], rep[2], inp.s_idx,
                               inp.s_att, sel.get("p", 0.0), 0, n_sink, n_window, x, idx, count,
                               out, lse, ws_step)
            return
        run_select(rep)
        decode_call(rep)

    def decode_call(rep):
        if args.rla:
            ops.sa_sparse_decode_rla(shape, pages, inp.q, rep[1], rep[2], idx, count, inp.s_att, out,
                                     lse, rla_state, rla_num, rla_den, ws_dec)
        else:
            ops.sa_sparse_decode(shape, pages, inp.q, rep[1], rep[2], idx, count, inp.s_att, out,
                                 lse, ws_dec)

    base = (cache_a, inp.k_pool, inp.v_pool)
    run_step(base)
    torch.cuda.synchronize()
    counts = count.cpu().numpy().astype(np.int64)
    kv_bytes = int(counts.sum()) * 2 * d * 2
    if args.rla:
        kv_bytes += state_bytes  # the decode call also reads each group's state
    index_bytes = int(sum(per_row_index_bytes[b] for b in range(B) for _ in range(Hkv)))
    step_bytes = index_bytes + kv_bytes

    # input replicas so that a step does not find the previous step's rows in
    # the 256 MB last-level cache
    R = 1 if args.warm else max(1, min(32, math.ceil(4 * MALL_BYTES / step_bytes)))
    reps = [base] + [tuple(t.clone() for t in base) for _ in range(R - 1)]
    torch.cuda.synchronize()

    ms = time_loop(lambda i: run_step(reps[i]), args.steps, warmup=args.warmup, reps=R)
    # the graph replays must reproduce an eager step bit for bit
    torch.cuda.synchronize()
    g_out, g_idx, g_cnt = out.clone(), idx.clone(), count.clone()
    g_rla = (rla_num.clone(), rla_den.clone()) if args.rla else None
    run_step(reps[R - 1])
    torch.cuda.synchronize()
    assert torch.equal(g_cnt, count) and torch.equal(g_idx, idx) and torch.equal(g_out, out), \
        "graph replay differs from the eager step"
    if args.rla:
        assert torch.equal(g_rla[0], rla_num) and torch.equal(g_rla[1], rla_den), \
            "graph replay differs from the eager step (residual terms)"
    # per-component times (same rotation), for the breakdown and the roofline
    if page_mode:
        t_index = time_loop(lambda i: ops.sa_page_scores(shape, pages, inp.q, reps[i][0],
                                                         inp.s_att, x), args.steps, reps=R)
    elif oracle_policy:
        t_index = time_loop(lambda i: ops.sa_attention_mass(shape, pages, inp.q, reps[i][1],
                                                            inp.s_att, x, ws_mass),
                            args.steps, reps=R)
    else:
        t_index = time_loop(lambda i: ops.sa_index_scores(shape, pages, inp.q, inp.w_q,
                                                          reps[i][0], inp.s_idx, x, ws_idx),
                            args.steps, reps=R)
    run_select(base)
    t_select = time_loop(lambda i: (ops.sa_select_topk(shape, pages, x, k_pages, 64, 0, 0, idx,
                                                       count, ws_sel) if page_mode else
                                    ops.sa_select_topp(shape, pages, x, sel["p"], n_sink,
                                                       n_window, idx, count, ws_sel)), args.steps)
    t_decode = time_loop(lambda i: decode_call(reps[i]), args.steps, reps=R)
    first = "page_scores" if page_mode else ("attention_mass" if oracle_policy else "index_scores")
    comp = {first: (t_index, index_bytes),
            "select": (t_select, 0),
            ("sparse_decode_rla" if args.rla else "sparse_decode"): (t_decode, kv_bytes)}
    if fused:
        # the whole step is one kernel: its bytes are the step's
        dom = "decode_step%s (single fused launch)" % ("_pages" if page_mode else "")
        dom_ms, dom_bytes = ms, step_bytes
    else:
        dom = max((k for k in comp if comp[k][1] > 0), key=lambda k: comp[k][0])
        dom_ms, dom_bytes = comp[dom]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    gbs = step_bytes / (ms * 1e-3) / 1e9
    res_workload = name + ("+rla" if args.rla else "") + ("+oracle" if oracle_policy else "")
    res = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": res_workload, "batch": B,
                   "context": (Lmax if B == 1 else
                                                              [min(inp.seq_lens), Lmax]),
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "selection": ("top-%d pages (Taylor page score)" % sel["k_pages"]
                                 if page_mode else
                                 ("dense attention mass " if oracle_policy else "") +
                                 f"top-p {sel['p']} + sink {n_sink} + window {n_window}"),
                   "input_replicas": R},
        "step_bytes": step_bytes,
        "index_bytes": index_bytes,
        "kv_bytes": kv_bytes,
        "budget_fraction": round(float(counts.sum()) / float(sum(inp.seq_lens) * Hkv), 5),
        "step_call": (("sa_decode_step_pages" if page_mode else
                       ("sa_decode_step_rla" if args.rla else "sa_decode_step")) +
                      (" (fused)" if fused else "")) if use_step else
                     ((("sa_page_scores + sa_select_topk") if page_mode else
                       ("sa_attention_mass" if oracle_policy else "sa_index_scores") +
                       " + sa_select_topp") +
                      (" + sa_sparse_decode_rla" if args.rla else " + sa_sparse_decode")),
        "separate_calls_ms": {k: round(v[0], 5) for k, v in comp.items()},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(res_workload, dom),
                     "bytes_per_launch": dom_bytes, "avg_launch_ms": round(dom_ms, 5)},
    }
    # the cold protocol: every step after a 1 GiB scrub, timed alone
    c_med, c_min, c_max, c_n = time_cold(lambda: run_step(base), min(args.steps, 20))
    res["cold"] = {"us_per_step_median": round(c_med * 1e3, 2), "us_min": round(c_min * 1e3, 2),
                   "us_max": round(c_max * 1e3, 2), "steps": c_n,
                   "gb_s_median": round(step_bytes / (c_med * 1e-3) / 1e9, 2),
                   "protocol": "1 GiB written then read before each step; HIP events around the step"}
    if not page_mode:
        res["coverage"] = support_coverage(ops, shape, pages, inp, base, x.shape[1], idx, count,
                                           sel["p"], ws_mass, ws_sel, run_step)
    if not args.no_cpu_baseline and not oracle_policy:
        res["cpu_baseline"] = cpu_baseline_decode(inp, cache_a if not page_mode else None,
                                                  step_bytes, args.cpu_seconds, page_mode,
                                                  stats if page_mode else None)
    return res


def support_coverage(ops, shape, pages, inp, base, ldx, idx, count, p, ws_mass, ws_sel, run_step):
    """Dense attention mass the step's supports keep (outside the timed
    region): the head-averaged dense distribution of every row, the mass of
    the step's support under it, and the attention-mass oracle's own top-p
    support (without sink/window) for comparison."""
    import torch
    rows = count.numel()
    xm = torch.empty((rows, ldx), dtype=torch.float32, device="cuda")
    run_step(base)
    ops.sa_attention_mass(shape, pages, inp.q, base[1], inp.s_att, xm, ws_mass)
    idx_o, count_o = torch.empty_like(idx), torch.empty_like(count)
    ops.sa_select_topp(shape, pages, xm, p, 0, 0, idx_o, count_o, ws_sel)
    mass = torch.empty((rows,), dtype=torch.float32, device="cuda")
    ov = torch.empty((rows,), dtype=torch.int32, device="cuda")
    ops.sa_support_coverage(shape, pages, xm, idx, count, mass, idx_o, count_o, ov)
    torch.cuda.synchronize()
    lens = inp.seq_lens_tensor().repeat_interleave(inp.H_kv).double()
    m = mass.double()
    return {"dense_mass_kept_mean": round(float(m.mean()), 4),
            "dense_mass_kept_min": round(float(m.min()), 4),
            "budget_fraction": round(float(count.double().sum() / lens.sum()), 5),
            "oracle_topp_budget_fraction": round(float(count_o.double().sum() / lens.sum()), 5),
            "support_in_oracle_topp": round(float(ov.double().sum() / count.double().sum()), 4),
            "p": p}


def cpu_baseline_decode(inp, kidx, step_bytes, seconds, page_mode, stats):
    """The float64 oracle on the host cores, on a bounded sample of the same
    step: whole (b, g) rows, repeated until ~seconds of CPU work."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle as O

    rows = [(b, g) for b in range(inp.B) for g in range(inp.H_kv)]
    data = []
    for b, g in rows[: min(len(rows), 8)]:
        hs = inp.heads(g)
        q = inp.q[b, hs].double().cpu().numpy()
        K = inp.seq_keys(b, g).double().cpu().numpy()
        V = inp.seq_values(b, g).double().cpu().numpy()
        if page_mode:
            L = inp.seq_lens[b]
            npg = (L + 63) // 64
            st = stats[inp.page_table[b, :npg].long(), g].reshape(npg, -1)
            st = st.double().cpu().numpy()
            n = np.array([min(64, L - 64 * p) for p in range(st.shape[0])])
            data.append((q, st[:, :inp.d], st[:, inp.d:], n, K, V))
        else:
            kt = inp.seq_rows(kidx, b, g).double().cpu().numpy()
            data.append((q, inp.w_q[hs].double().cpu().numpy(), kt, K, V, inp.seq_lens[b]))
    sel = inp.select
    done_bytes = 0.0
    t0 = time.perf_counter()
    n_rows = 0
    with threadpool_limits() as tl:
        threads = blas_threads()
        while True:
            for item in data:
                if page_mode:
                    q, mu, var, n, K, V = item
                    r = O.decode_row_pages(q, mu, var, n, K, V, s_att=inp.s_att,
                                           k_pages=sel["k_pages"])
                    done_bytes += mu.shape[0] * 2 * inp.d * 2 + len(r["S"]) * 2 * inp.d * 2
                else:
                    q, wq, kt, K, V, L = item
                    r = O.decode_row(q, wq, kt, K, V, s_idx=inp.s_idx, s_att=inp.s_att,
                                     p=float(np.float32(sel["p"])), n_sink=sel["n_sink"],
                                     n_window=sel["n_window"])
                    done_bytes += L * 16 * 2 + len(r["S"]) * 2 * inp.d * 2
                n_rows += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"value": round(done_bytes / el / 1e9, 5), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n_rows} (sequence, group) rows of the same step, float64 numpy, "
                      f"{el:.1f} s", "host_threads_available": cpu_threads_info()}


def bench_prefill(args):
    """Block selection (top-k 2048 per 64-query block) + block-sparse causal
    attention over the 128K prefill.  FLOPs = 4 * d * (query, key) pairs
    attended per head, counted from the actual supports (diagonal pairs
    causal only)."""
    import numpy as np
    import torch

    import synth
    from dynamic_sparse_attention_02_amd import _lib as L
    from dynamic_sparse_attention_02_amd import ops

    inp = synth.make_prefill128k(device="cuda")
    N, Hq, Hkv, d = inp.N, inp.H_q, inp.H_kv, inp.d
    G = Hq // Hkv
    pbs = args.selection == "pbs"
    seg, k_blocks = 2048, inp.top_k // 64
    shape = ops.make_shape(batch=1, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                           max_pages=inp.page_table.shape[1], max_len=N,
                           n_pool_pages=inp.k_pool.shape[0])
    pages = ops.make_pages(inp.page_table, None)
    kidx = torch.zeros((inp.k_pool.shape[0], Hkv, 64, 16), dtype=inp.dtype, device="cuda")
    fill_kidx(ops, shape, inp, kidx)
    nblk = inp.n_blocks
    k = inp.top_k
    cap = min(k, N)
    idx = torch.empty((nblk * Hkv, cap), dtype=torch.int32, device="cuda")
    count = torch.empty((nblk * Hkv,), dtype=torch.int32, device="cuda")
    out = torch.empty((N, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((N, Hq), dtype=torch.float32, device="cuda")
    if pbs:
        imp = torch.empty((Hkv, N), dtype=torch.float32, device="cuda")
        perm = torch.empty((Hkv, N), dtype=torch.int32, device="cuda")
        ws_imp = ops.alloc_workspace(ops.workspace_size(L.SA_OP_PBS_IMPORTANCE, shape, 64))
        ws = ops.alloc_workspace(ops.workspace_size(L.SA_OP_PBS_SELECT, shape, k_blocks))
    else:
        ws = ops.alloc_workspace(ops.workspace_size(L.SA_OP_PREFILL_SELECT, shape, N))

    def select():
        if pbs:
            ops.sa_pbs_importance(shape, pages, N, inp.q, inp.k_pool, inp.s_att, 64, imp, ws_imp)
            ops.sa_pbs_permutation(shape, imp, N, seg, perm)
            ops.sa_pbs_select(shape, pages, N, inp.q, inp.k_pool, perm, seg, 64, k_blocks, idx,
                              count, ws)
            return
        ops.sa_select_prefill_topk(shape, pages, N, inp.q, inp.w_q, kidx, inp.s_idx, 64, k, idx,
                                   count, ws)

    def attend():
        ops.sa_sparse_prefill(shape, pages, N, inp.q, inp.k_pool, inp.v_pool, idx, count, 64,
                              inp.s_att, out, lse)

    select()
    attend()
    torch.cuda.synchronize()
    cnt = count.cpu().numpy().astype(np.int64).reshape(nblk, Hkv)
    nq = np.minimum(64, N - 64 * np.arange(nblk))
    pairs = (cnt * nq[:, None]).sum() + Hkv * (nq * (nq + 1) // 2).sum()
    flops = 4.0 * d * G * float(pairs)
    steps = args.steps
    for _ in range(args.warmup):
        select()
        attend()
    t_sel = time_events(select, steps)
    t_att = time_events(attend, steps)
    ms = t_sel + t_att
    tflops = flops / (ms * 1e-3) / 1e12
    att_tflops = flops / (t_att * 1e-3) / 1e12
    res = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill128k" + ("+pbs" if pbs else ""), "tokens": N,
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "b_sel": 64, "top_k": k,
                   "selection": ("segment-permuted mean-pooled blocks (segment %d, top-%d blocks)"
                                 % (seg, k_blocks)) if pbs else "low-rank indexer, top-k keys"},
        "algorithmic_flops": flops,
        "breakdown_ms": {"select": round(t_sel, 4), "attention": round(t_att, 4)},
        "attention_tflops": round(att_tflops, 2),
        "roofline": {"kernel": "sparse_prefill", "bound": "mfma", "achieved": round(att_tflops, 2),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(att_tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": recorded_traffic("prefill128k" + ("+pbs" if pbs else ""),
                                                 "sparse_prefill"),
                     "flops_per_launch": flops, "avg_launch_ms": round(t_att, 4)},
    }
    if pbs:
        res["breakdown_ms"]["pbs_select_parts"] = "importance + permutation + block selection"
    if args.coverage:
        res["coverage"] = prefill_coverage(inp, idx, count)
    if not args.no_cpu_baseline and not pbs:
        res["cpu_baseline"] = cpu_baseline_prefill(inp, kidx, args.cpu_seconds)
    return res


def bench_prefill_query(args):
    """Per-query (b_sel = 1) prefill at 32K: a top-2048 support per (query,
    group) plus the own token, and each query's attention over its list
    (split-KV kernels).  Bytes = 512 B of K/V per listed key per group (what
    the per-query gather needs); FLOPs = 4 * d per listed key per head."""
    import numpy as np
    import torch

    import synth
    from dynamic_sparse_attention_02_amd import _lib as L
    from dynamic_sparse_attention_02_amd import ops

    inp = synth.make_prefill_query32k(device="cuda")
    N, Hq, Hkv, d = inp.N, inp.H_q, inp.H_kv, inp.d
    G = Hq // Hkv
    probs = args.aggregate == "probs"
    oracle_sel = args.selection == "oracle"
    shape = ops.make_shape(batch=1, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d,
                           max_pages=inp.page_table.shape[1], max_len=N,
                           n_pool_pages=inp.k_pool.shape[0])
    pages = ops.make_pages(inp.page_table, None)
    kidx = torch.zeros((inp.k_pool.shape[0], Hkv, 64, 16), dtype=inp.dtype, device="cuda")
    fill_kidx(ops, shape, inp, kidx)
    k = inp.top_k
    cap = min(k + 1, N)
    idx = torch.empty((N * Hkv, cap), dtype=torch.int32, device="cuda")
    count = torch.empty((N * Hkv,), dtype=torch.int32, device="cuda")
    out = torch.empty((N, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((N, Hq), dtype=torch.float32, device="cuda")
    ws = ops.alloc_workspace(ops.workspace_size(
        L.SA_OP_PREFILL_ORACLE if oracle_sel else L.SA_OP_PREFILL_SELECT, shape, N))
    ws_a = ops.alloc_workspace(ops.workspace_size(L.SA_OP_PREFILL_QUERY, shape, cap))
    sel_fn = ops.sa_select_prefill_topk_probs if probs else ops.sa_select_prefill_topk

    def select():
        if oracle_sel:
            ops.sa_select_prefill_oracle(shape, pages, N, inp.q, inp.k_pool, inp.s_att, 1, k, idx,
                                         count, ws)
            return
        sel_fn(shape, pages, N, inp.q, inp.w_q, kidx, inp.s_idx, 1, k, idx, count, ws)

    def attend():
        ops.sa_sparse_prefill_query(shape, pages, N, inp.q, inp.k_pool, inp.v_pool, idx, count,
                                    inp.s_att, out, lse, ws_a)

    select()
    attend()
    torch.cuda.synchronize()
    listed = int(count.cpu().numpy().astype(np.int64).sum())
    flops = 4.0 * d * G * float(listed)
    kv_bytes = listed * 2 * d * 2
    for _ in range(args.warmup):
        select()
        attend()
    t_sel = time_events(select, args.steps)
    t_att = time_events(attend, args.steps)
    ms = t_sel + t_att
    gbs = kv_bytes / (t_att * 1e-3) / 1e9
    name = "prefill32k_query" + ("+probs" if probs else "") + ("+oracle" if oracle_sel else "")
    res = {
        "metric": METRIC, "value": round(flops / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "tokens": N, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "b_sel": 1, "top_k": k,
                   "aggregate": ("dense attention mass (oracle)" if oracle_sel else
                                 "mean of head probabilities" if probs else "head-collapsed logits")},
        "algorithmic_flops": flops, "kv_bytes": kv_bytes,
        "budget_fraction": round(listed / (Hkv * N * (N + 1) / 2), 5),
        "breakdown_ms": {"select": round(t_sel, 4), "attention": round(t_att, 4)},
        "attention_tflops": round(flops / (t_att * 1e-3) / 1e12, 3),
        "roofline": {"kernel": "sparse_prefill_query", "bound": "hbm", "achieved": round(gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(name, "sparse_prefill_query"),
                     "bytes_per_launch": kv_bytes, "avg_launch_ms": round(t_att, 4),
                     "note": "gathered K/V rows per listed key; the 134 MB cache of this "
                             "workload fits the last-level cache, so rows repeat from it"},
    }
    if not args.no_cpu_baseline and not oracle_sel:
        res["cpu_baseline"] = cpu_baseline_prefill_query(inp, kidx, args.cpu_seconds, probs)
    return res


def cpu_baseline_prefill_query(inp, kidx, seconds, probs):
    """The float64 oracle on a bounded sample of the per-query prefill: whole
    (query, group) rows (scores, support, attention), last queries first."""
    import oracle as O
    from threadpoolctl import threadpool_limits

    g = 0
    hs = inp.heads(g)
    K = inp.keys(g).double().cpu().numpy()
    V = inp.values(g).double().cpu().numpy()
    kt = inp.rows(kidx, g).double().cpu().numpy()
    wq = inp.w_q[hs].double().cpu().numpy()
    flops = 0.0
    n_rows = 0
    t0 = time.perf_counter()
    with threadpool_limits():
        threads = blas_threads()
        for i in range(inp.N - 1, -1, -1):
            qi = inp.q[i, hs].double().cpu().numpy()
            x = O.prefill_query_scores(qi, wq, kt, i, inp.s_idx, "probs" if probs else "logits")
            S_ = O.prefill_query_support(x, i, inp.top_k)
            O.prefill_query_attend(qi, K, V, S_, inp.s_att)
            flops += 4.0 * inp.d * len(hs) * len(S_)
            n_rows += 1
            if time.perf_counter() - t0 >= seconds:
                break
    el = time.perf_counter() - t0
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n_rows} (query, group) rows of the last queries (scores + support + "
                      f"attention), float64 numpy, {el:.1f} s",
            "host_threads_available": cpu_threads_info()}


def prefill_coverage(inp, idx, count):
    """Dense attention mass (head mean of each query row's causal softmax)
    that the block supports plus the causal diagonal keep, on sampled
    (query block, group) items; float64 on the host, outside the timed
    region."""
    import numpy as np

    import oracle as O

    nblk = inp.n_blocks
    kept = []
    for g in (0, inp.H_kv - 1):
        hs = inp.heads(g)
        K = inp.keys(g).double().cpu().numpy()
        for blk in (nblk // 4, nblk // 2, 3 * nblk // 4, nblk - 1):
            n = int(count[blk * inp.H_kv + g])
            sup = idx[blk * inp.H_kv + g, :n].cpu().numpy().astype(np.int64)
            for i in range(blk * 64, min(inp.N, blk * 64 + 64), 8):
                P = O.head_mean_attention(inp.q[i, hs].double().cpu().numpy(), K[:i + 1], inp.s_att)
                kept.append(P[sup].sum() + P[blk * 64:i + 1].sum())
    kept = np.array(kept)
    return {"dense_mass_kept_mean": round(float(kept.mean()), 4),
            "dense_mass_kept_min": round(float(kept.min()), 4),
            "sample": "8 query rows of each of 4 query blocks x 2 groups"}


def time_cold(fn, n, scrub_bytes=1 << 30):
    """Per-step milliseconds of fn() with the caches cold: before each step a
    scrub writes and then reads scrub_bytes (four times the 256 MB last-level
    cache), and HIP events on the current stream bracket the step alone.  The
    scrub is still running on the GPU while the host enqueues the step, so
    the events see no host launch gap.  Returns (median, min, max, n)."""
    import torch
    scrub = torch.empty(scrub_bytes, dtype=torch.uint8, device="cuda")
    fn()
    torch.cuda.synchronize()
    times = []
    for i in range(n):
        scrub.fill_(i & 0xFF)
        scrub.view(torch.int64).sum()
        a, b = _events()
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    del scrub
    times.sort()
    return times[len(times) // 2], times[0], times[-1], n


def time_events(fn, n):
    """Average milliseconds of fn() over n calls (HIP events, current stream)."""
    import torch
    fn()
    torch.cuda.synchronize()
    a, b = _events()
    a.record()
    for _ in range(n):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def cpu_baseline_prefill(inp, kidx, seconds):
    """The float64 oracle on a bounded sample of the prefill: whole (query
    block, group) items (selection + attention), late blocks first."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle as O

    g = 0
    hs = inp.heads(g)
    K = inp.keys(g).double().cpu().numpy()
    V = inp.values(g).double().cpu().numpy()
    kt = inp.rows(kidx, g).double().cpu().numpy()
    wq = inp.w_q[hs].double().cpu().numpy()
    nblk = inp.n_blocks
    flops = 0.0
    n_items = 0
    t0 = time.perf_counter()
    with threadpool_limits() as tl:
        threads = blas_threads()
        for blk in range(nblk - 1, -1, -1):
            rows = O.prefill_block_rows(blk, 64, inp.N)
            Qb = inp.q[rows.start:rows.stop][:, hs].double().cpu().numpy()
            qc = O.prefill_block_query(Qb, wq, inp.s_idx)
            S_ = O.prefill_block_support(qc, kt, blk, 64, inp.top_k)
            O.prefill_block_attend(Qb, K, V, S_, blk, 64, inp.s_att)
            nq = rows.stop - rows.start
            flops += 4.0 * inp.d * len(hs) * (nq * len(S_) + nq * (nq + 1) / 2)
            n_items += 1
            if time.perf_counter() - t0 >= seconds:
                break
    el = time.perf_counter() - t0
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_items} (query block, group) items of the last blocks (selection + "
                      f"attention), float64 numpy, {el:.1f} s",
            "host_threads_available": cpu_threads_info()}


# ---------------------------------------------------------------------------


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only (one GPU's share of the work); --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    if args.calibrate_copy:
        print(json.dumps(calibrate_copy()))
        return
    import dynamic_sparse_attention_02_amd as pkg
    pkg.load_library()
    if args.workload == "prefill128k":
        res = bench_prefill(args)
    elif args.workload == "prefill32k_query":
        res = bench_prefill_query(args)
    else:
        res = bench_decode(args, args.workload)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
