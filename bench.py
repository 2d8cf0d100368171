"""Benchmark of the sparse-verification step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
  dustin_score (draft + target-subset scoring)
  -> dustin_topk (global verification set per sequence)
  -> L x dustin_sparse_verify_attn (one call per target layer, each layer its
     own K/V buffers, the same index set).
Default workload: Qwen2.5-72B-shaped target (64 query / 8 KV heads, head_dim
128, 80 layers), 0.5B-shaped draft (24 layers x 14 heads, 2 KV heads,
head_dim 64), batch 16, context 32768, w = Gamma = 4, k = 2048, bf16.

Prints ONE JSON line (rank 0).  `value` is microseconds per step (lower is
better), timed with HIP events around K steps replayed from a HIP graph
(eager timing reported alongside).  The dominant kernel (the gathered
attention) is also timed per launch with HIP events on its stream, and the
whole step is related to the 8 TB/s HBM peak through its algorithmic bytes.
The CPU oracle is timed on a bounded sample (whole step for one sequence
with one attention layer) and scaled to a full step.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--attn-timeline-child", action="store_true", help=argparse.SUPPRESS)
    p.add_argument("--timeline-v-offset", type=int, default=0,
                   help="attention timeline with every V buffer placed this many bytes (multiple of 256) past an "
                        "allocation boundary, K left aligned")
    p.add_argument("--no-lse", action="store_true",
                   help="skip the labelled step with caller-supplied draft row normalisers")
    p.add_argument("--no-timeline", action="store_true",
                   help="skip the attention phase timeline (phase-trace build of the library, in a child process)")
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", default="c4")
    p.add_argument("--k", type=int, default=None)
    p.add_argument("--layers", type=int, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-dense", action="store_true")
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--no-window", action="store_true",
                   help="skip the verification-window step (append + causal verify attention + commit)")
    p.add_argument("--no-sweep", action="store_true", help="skip the policy sweep (ARR of the compared policies)")
    p.add_argument("--no-ksweep", action="store_true", help="skip the step at the other budgets k (512, 1024)")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the one-layer steps of the other workloads (tiny f32, 7B, 32B, ragged paged)")
    p.add_argument("--no-search", action="store_true",
                   help="skip the offline configuration search (SRH matrix, greedy target/draft, m search)")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the achievable-rate probes (streaming read, K/V row gather, last-level-cache re-read)")
    p.add_argument("--no-srh", action="store_true",
                   help="skip the step restricted to the searched draft layers and target heads (Dustin-H, blog Fig. 6)")
    p.add_argument("--no-curve", action="store_true",
                   help="skip the estimator-overhead curve (dense, naive, Quest-16, Dustin-T/D/H over context length)")
    p.add_argument("--pmc-probe", action="store_true",
                   help="for counter collection: one warm step, a 1 GiB float32 copy (the calibration "
                        "kernel of known size), then one more step and one window attention of w = 4 and of "
                        "w = 8 on layer 0; prints no JSON")
    p.add_argument("--no-evaluator", action="store_true",
                   help="skip the window-attention timings of the evaluator (w = 4 and w = 8 on the c4 cache)")
    return p.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_kernel_c4_k2048_traffic.txt")
TRAFFIC_SOURCES = ["sparse_kv_verification_amd/csrc/attn.hip", "sparse_kv_verification_amd/csrc/common.h",
                   "sparse_kv_verification_amd/csrc/attn.h"]


def attn_source_digest():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per sparse-attention launch from the committed counter
    summary, or None when the kernel sources changed after it was taken."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if "=" in line and not line.startswith("#"):
                    a, b = line.split("=", 1)
                    kv[a.strip()] = b.strip()
        if kv.get("source_sha256") != attn_source_digest():
            return None
        return {"bytes_per_launch": int(kv["hbm_bytes_per_launch"]),
                "fetch_bytes": int(kv["fetch_bytes_per_launch"]), "write_bytes": int(kv["write_bytes_per_launch"])}
    except (OSError, KeyError, ValueError):
        return None


def algorithmic_bytes(sh, x, k_eff, counts, sub_heads):
    """Bytes the method must move (no second passes, no partials)."""
    import torch
    esz = 4 if sh.dtype == "f32" else 2
    n_tot = int(x.seq_lens.sum())
    U = len({(l, h // sh.G) for (l, h) in sub_heads})
    draft = sh.L_d * n_tot * sh.Hkv_d * sh.d_d * esz + x.q_draft.numel() * esz
    target = n_tot * U * sh.d * esz + x.q_hist.numel() * esz
    scores_out = 2 * sh.B * sh.n * 4
    select = 2 * sh.B * sh.n * 4 + sh.B * k_eff * (4 + 1) + sh.B * 4
    sel_rows = int(counts.sum())
    per_layer = sel_rows * sh.Hkv * sh.d * esz * 2 + 2 * x.q.numel() * esz + sh.B * k_eff * 4 + sh.B * 4
    return {
        "score": draft + target + scores_out,
        "select": select,
        "attn_per_layer": per_layer,
        "step": draft + target + scores_out + select + sh.layers * per_layer,
        "dense_per_layer": n_tot * sh.Hkv * sh.d * esz * 2 + 2 * x.q.numel() * esz,
    }


def cpu_baseline(sh, x, k, m, n_sink, n_window, budget_s=20.0):
    """Time the oracle (as it stands) on whole sequences of the step: draft
    and target scoring, selection and every attention layer of the sequence
    (the layers hold identical copies, so one host copy serves all of them),
    until about `budget_s` seconds of oracle time; scale to all B sequences."""
    import numpy as np
    import oracle
    f = lambda t: t.detach().float().cpu().numpy().astype(np.float64)
    done, total = 0, {"score": 0.0, "select": 0.0, "attention": 0.0}
    for b in range(sh.B):
        n = int(x.seq_lens[b])
        K, V = f(x.logical("K", b)), f(x.logical("V", b))
        Kd = f(x.logical("Kd", b))
        qd, qh, q = f(x.q_draft[b]), f(x.q_hist[b]), f(x.q[b])
        t0 = time.perf_counter()
        sd = oracle.score_draft(qd, Kd)
        st = oracle.score_target(qh, {0: K}, x.sub_heads, sh.Hq)
        t1 = time.perf_counter()
        I, _ = oracle.select_verify_set(sd, st, n, k, m, n_sink, n_window)
        t2 = time.perf_counter()
        for _ in range(sh.layers):
            oracle.sparse_attention(q, K, V, I)
        t3 = time.perf_counter()
        total["score"] += t1 - t0
        total["select"] += t2 - t1
        total["attention"] += t3 - t2
        done += 1
        del K, V, Kd
        if sum(total.values()) >= budget_s:
            break
    threads = None
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max((i.get("num_threads", 1) for i in info), default=1)
    except Exception:
        threadpoolctl = None
        threads = os.cpu_count()
    measured = sum(total.values())
    # sequence 0: score + select + one attention layer with all threads and with one thread, and one
    # dense (full-cache) layer, stated x layers as an extrapolation
    n = int(x.seq_lens[0])
    K, V, Kd = f(x.logical("K", 0)), f(x.logical("V", 0)), f(x.logical("Kd", 0))
    qd, qh, q = f(x.q_draft[0]), f(x.q_hist[0]), f(x.q[0])

    def one_layer():
        sd = oracle.score_draft(qd, Kd)
        st = oracle.score_target(qh, {0: K}, x.sub_heads, sh.Hq)
        I, _ = oracle.select_verify_set(sd, st, n, k, m, n_sink, n_window)
        oracle.sparse_attention(q, K, V, I)

    t0 = time.perf_counter()
    one_layer()
    t_all = time.perf_counter() - t0
    t_one = None
    if threadpoolctl is not None:
        with threadpoolctl.threadpool_limits(1):
            t0 = time.perf_counter()
            one_layer()
            t_one = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.dense_attention(q, K, V)
    t_dense = time.perf_counter() - t0
    return {
        "value": measured / done * sh.B * 1e6,
        "unit": "us/step",
        "cores": int(threads or 1),
        "kind": "oracle",
        "sample": (f"sequences 0..{done - 1} of {sh.B} (n={sh.n}), each: score_draft + score_target + select + "
                   f"all {sh.layers} attention layers, fp64 NumPy; {measured:.1f} s measured, scaled x{sh.B / done:g}"),
        "measured_s": {a: round(b, 3) for a, b in total.items()},
        "host_cpu": platform.processor() or platform.machine(),
        "host_cpu_count": os.cpu_count(),
        "one_sequence_one_layer_s": {"all_threads": round(t_all, 3), "threads": int(threads or 1),
                                     "one_thread": None if t_one is None else round(t_one, 3)},
        "dense_layer_one_sequence_s": round(t_dense, 3),
        "dense_step_extrapolated_s": round(t_dense * sh.layers * sh.B, 1),
    }


TRACE_LIB = os.path.join(ROOT, "sparse_kv_verification_amd", "libdustin_trace.so")
TIMELINE_PHASES = ["entry", "rows_ready", "first_tile", "loop_end", "partial_stored", "handshake", "exit"]


def attn_timeline_child(args):
    """Run in a child process with DUSTIN_LIBRARY = the phase-trace build:
    the step's score and select on the generated inputs, then 80 attention
    launches over 16 distinct layer buffers replayed from a HIP graph, and
    the per-work-group phase stamps of the last replay, summarised.  Prints
    one JSON line."""
    import ctypes
    import numpy as np
    import torch
    import synth
    import sparse_kv_verification_amd as dk
    dev = torch.device("cuda:0")
    sh = synth.preset(args.config)
    x = synth.make(sh, device=dev)
    NL, L = 16, 80
    Ks = [x.K] + [x.K.clone() for _ in range(NL - 1)]
    off = args.timeline_v_offset
    assert off >= 0 and off % 256 == 0, "--timeline-v-offset takes a multiple of 256 bytes"
    if off:
        Vs = []
        for _ in range(NL):
            flat = torch.empty(x.V.numel() + off // 2, dtype=x.V.dtype, device=dev)
            v = flat[off // 2:].view(x.V.shape)
            v.copy_(x.V)
            Vs.append(v)
    else:
        Vs = [x.V] + [x.V.clone() for _ in range(NL - 1)]
    kvs = [dk.KV(Ks[l], Vs[l], x.seq_lens, x.page_table) for l in range(NL)]
    dkv = [dk.KV(x.Kd[l], None, x.seq_lens, x.page_table) for l in range(sh.L_d)]
    n_sink, n_window, m = synth.tier_defaults(sh.k)
    s_d, s_t = dk.dustin_score(dkv, x.q_draft, [kvs[0]], x.q_hist, x.sub_heads, sh.Hq)
    idx, cnt, _ = dk.dustin_topk(s_d, s_t, x.seq_lens, sh.k, m, n_sink, n_window, want_tier=False)
    out = torch.empty_like(x.q)
    ws = dk.Workspace()
    lib = dk.lib()
    lib.dustin_trace_attn_restart.restype = None
    lib.dustin_trace_attn_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]

    def layers():
        for l in range(L):
            dk.dustin_sparse_verify_attn(x.q, kvs[l % NL], idx, cnt, out=out, ws=ws)

    layers()
    torch.cuda.synchronize()
    lib.dustin_trace_attn_restart()            # the captured launches take rows 0..79
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            layers()
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    e1.synchronize()
    buf = np.zeros((80, 1024, 8), dtype=np.uint64)
    rc = lib.dustin_trace_attn_read(buf.ctypes.data_as(ctypes.c_void_p), buf.nbytes)
    assert rc == 0, f"dustin_trace_attn_read: hipError {rc}"
    nwg = int((buf[0, :, 0] > 0).sum())        # the array starts zeroed: recorded groups are nonzero
    st = buf[:, :nwg, :].astype(np.int64)
    start = st[:, :, 0].min(axis=1)
    rel = (st[:, :, :7] - start[:, None, None]) / 100.0      # us since the launch's first work-group began
    ok = st[:, :, :7] > 0
    res = {"workload": f"{sh.name}: B={sh.B} n={sh.n} Hq={sh.Hq} Hkv={sh.Hkv} d={sh.d} w={sh.w} k={sh.k}, "
                       f"{L} launches over {NL} layer buffers, graph replay",
           "v_offset_bytes": off,
           "work_groups_per_launch": nwg, "us_per_launch": round(e0.elapsed_time(e1) * 1e3 / L, 2),
           "launch_span_us_p50": round(float(np.median((st[:, :, 6].max(axis=1) - start) / 100.0)), 2),
           "gap_between_launches_us_p50": round(float(np.median((start[1:] - st[:-1, :, 6].max(axis=1)) / 100.0)), 2),
           "phases_us_since_launch_start_p0_p50_p90_p100": {}}
    for i, nm in enumerate(TIMELINE_PHASES):
        v = rel[:, :, i][ok[:, :, i]]
        if v.size:
            res["phases_us_since_launch_start_p0_p50_p90_p100"][nm] = [
                round(float(np.percentile(v, q)), 2) for q in (0, 50, 90, 100)]
    loop = np.where(ok[:, :, 2] & ok[:, :, 3], rel[:, :, 3] - rel[:, :, 2], np.nan)   # a split with no tile: none
    wg = np.arange(nwg)
    splits = nwg // (sh.B * sh.Hkv)
    head = (wg // splits) % sh.Hkv
    xcc = (st[:, :, 7] >> 8) & 0xF
    res["token_loop_us_by_kv_head"] = {int(h): round(float(np.nanmean(loop[:, head == h])), 2)
                                       for h in range(sh.Hkv)}
    res["token_loop_us_by_xcd"] = {int(c): round(float(np.nanmean(loop[xcc == c])), 2)
                                   for c in range(8) if (xcc == c).any()}
    res["paths"] = {["one split", "merged at once", "merged after arriving last", "published only"][int(p)]:
                    int(((st[:, :, 7] & 0xFF) == p).sum()) for p in np.unique(st[:, :, 7] & 0xFF)}
    print(json.dumps(res), flush=True)


def attn_timeline(args):
    """The attention phase timeline from the phase-trace build, in a child
    process (the trace build exports the same entry points)."""
    import subprocess
    if not os.path.exists(TRACE_LIB):
        log("attention timeline skipped: no phase-trace build (python -m sparse_kv_verification_amd.build --trace)")
        return None
    env = dict(os.environ, DUSTIN_LIBRARY=TRACE_LIB)
    r = subprocess.run([sys.executable, "-u", os.path.abspath(__file__), "--attn-timeline-child", "--config",
                        args.config], capture_output=True, text=True, env=env, timeout=600)
    if r.returncode != 0:
        log("attention timeline failed: " + (r.stderr or "")[-2000:])
        return None
    res = json.loads(r.stdout.strip().splitlines()[-1])
    ph = res["phases_us_since_launch_start_p0_p50_p90_p100"]
    log(f"attention timeline (phase-trace build, {res['us_per_launch']} us/launch): " +
        ", ".join(f"{k} p50 {v[1]} max {v[3]}" for k, v in ph.items()) +
        f"; token loop by KV head {res['token_loop_us_by_kv_head']}")
    return res


def main():
    args = parse()
    if args.attn_timeline_child:
        return attn_timeline_child(args)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import sparse_kv_verification_amd as dk

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    over = {}
    if args.k:
        over["k"] = args.k
    if args.layers:
        over["layers"] = args.layers
    sh = synth.preset(args.config).replace(**over)
    k = sh.k
    n_sink, n_window, m = synth.tier_defaults(k)
    log(f"config {sh.name} B={sh.B} n={sh.n} Hq={sh.Hq} Hkv={sh.Hkv} d={sh.d} w={sh.w} k={k} "
        f"layers={sh.layers} draft {sh.L_d}x{sh.H_d} (kv {sh.Hkv_d}, d {sh.d_d}); m={m} sink={n_sink} window={n_window}")
    t = time.time()
    x = synth.make(sh, device=dev)
    torch.cuda.synchronize()
    log(f"inputs generated in {time.time() - t:.1f}s")

    # per-layer K/V buffers: layer 0 is the generated cache, the others are
    # copies in distinct allocations (so no layer is served from cache)
    Ks, Vs = [x.K], [x.V]
    for _ in range(1, sh.layers):
        Ks.append(x.K.clone())
        Vs.append(x.V.clone())
    torch.cuda.synchronize()
    log(f"{sh.layers} layers resident ({sh.layers * 2 * x.K.numel() * x.K.element_size() / 1e9:.1f} GB)")
    kvs = [dk.KV(Ks[l], Vs[l], x.seq_lens, x.page_table) for l in range(sh.layers)]
    dkv = [dk.KV(x.Kd[l], None, x.seq_lens, x.page_table) for l in range(sh.L_d)]
    s_d = torch.empty((sh.B, sh.n), dtype=torch.float32, device=dev)
    s_t = torch.empty_like(s_d)
    idx = torch.empty((sh.B, k), dtype=torch.int32, device=dev)
    cnt = torch.empty((sh.B,), dtype=torch.int32, device=dev)
    out = torch.empty_like(x.q)
    ws_s, ws_k, ws_a = dk.Workspace(), dk.Workspace(), dk.Workspace()

    def score():
        dk.dustin_score(dkv, x.q_draft, [kvs[0]], x.q_hist, x.sub_heads, sh.Hq, s_draft=s_d, s_target=s_t, ws=ws_s)

    def select():
        dk.dustin_topk(s_d, s_t, x.seq_lens, k, m, n_sink, n_window, idx=idx, count=cnt, want_tier=False, ws=ws_k)

    def attn(l):
        dk.dustin_sparse_verify_attn(x.q, kvs[l], idx, cnt, out=out, ws=ws_a)

    def step():
        score()
        select()
        for l in range(sh.layers):
            attn(l)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    if args.pmc_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)    # 1 GiB
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        log("pmc probe: calibration copy of 1073741824 bytes (read + write)")
        dst.copy_(src)
        torch.cuda.synchronize()
        log("pmc probe: one step")
        step()
        torch.cuda.synchronize()
        log("pmc probe: window attention, w = 4 and w = 8")
        q8 = torch.cat([x.q, x.q.flip(1)], dim=1).contiguous()
        dk.dustin_window_attn(x.q, kvs[0])
        dk.dustin_window_attn(q8, kvs[0])
        torch.cuda.synchronize()
        log("pmc probe done")
        return
    bytes_ = algorithmic_bytes(sh, x, k, cnt, x.sub_heads)
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3   # us

    eager_us = timed(step, args.steps)
    log(f"eager step {eager_us:.1f} us")

    graph_us = None
    cap = torch.cuda.Stream()
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            step()                       # warm the capture stream's workspaces
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=cap):
                step()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        graph_us = timed(g.replay, args.steps)
        log(f"graph step {graph_us:.1f} us")
    step_us = graph_us if graph_us is not None else eager_us
    # per-step distribution: one event pair around each replay (or eager step)
    pairs = []
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        (g.replay if graph_us is not None else step)()
        e1.record(stream)
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    ts = sorted(a_.elapsed_time(b_) * 1e3 for a_, b_ in pairs)
    pick = lambda q: ts[min(len(ts) - 1, int(round(q * (len(ts) - 1))))]
    step_pct = {"p10": round(pick(0.1), 1), "p50": round(pick(0.5), 1), "p90": round(pick(0.9), 1)}
    log(f"step distribution over {len(ts)} single-step timings: p10 {step_pct['p10']} p50 {step_pct['p50']} "
        f"p90 {step_pct['p90']} us")
    # a device-to-device copy of 1 GiB (read + write) as the measured bandwidth reference
    csrc = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    copy_us = timed(lambda: cdst.copy_(csrc), 5)
    copy_gbps = 2 * csrc.numel() * 4 / copy_us / 1e3
    del csrc, cdst
    log(f"device copy of 1 GiB: {copy_us:.0f} us, {copy_gbps:.0f} GB/s (read + write)")

    # component timings (eager, events on the launch stream)
    score_us = timed(score, args.steps)
    select_us = timed(select, args.steps)
    # dominant kernel: the L attention launches of a step, replayed from a
    # HIP graph and timed with events on the launch stream; divided by L this
    # is the average launch duration (inter-kernel gaps inside the graph
    # included).  One event pair per eager launch is reported alongside.
    attn_graph_us = None
    if not args.no_graph:
        ga = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(ga, stream=cap):
                for l in range(sh.layers):
                    attn(l)
        torch.cuda.synchronize()
        ga.replay()
        attn_graph_us = timed(ga.replay, args.steps) / sh.layers
    durs = []
    for _ in range(args.steps):
        for l in range(sh.layers):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            attn(l)
            e1.record(stream)
            durs.append((e0, e1))
    torch.cuda.synchronize()
    attn_event_us = sum(a.elapsed_time(b) for a, b in durs) / len(durs) * 1e3
    attn_loop_us = timed(lambda: [attn(l) for l in range(sh.layers)], args.steps) / sh.layers
    attn_launch_us = attn_graph_us if attn_graph_us is not None else attn_loop_us
    log(f"score {score_us:.1f} us, select {select_us:.1f} us, attention {attn_launch_us:.2f} us/launch "
        f"(graph replay; eager loop {attn_loop_us:.2f}, single event-bracketed launch {attn_event_us:.2f})")

    dense = None
    if not args.no_dense:
        dout = torch.empty_like(x.q)
        ws_d = dk.Workspace()
        def dense_layers():
            for l in range(sh.layers):
                dk.dustin_sparse_verify_attn(x.q, kvs[l], None, None, out=dout, ws=ws_d)
        dense_layers()
        dense_us = timed(dense_layers, 2)
        dense = {
            "us_per_step_attention": dense_us,
            "GBps": bytes_["dense_per_layer"] * sh.layers / dense_us / 1e3,
            "speedup_sparse_step_vs_dense_attention": dense_us / step_us,
            # the attention alone: the same L layers over the selected rows only
            "speedup_sparse_attention_vs_dense_attention": dense_us / (attn_launch_us * sh.layers),
        }
        dense["frac"] = dense["GBps"] / HBM_PEAK_GBPS
        log(f"dense attention {dense_us:.1f} us/step ({dense['GBps']:.0f} GB/s), "
            f"sparse step is {dense['speedup_sparse_step_vs_dense_attention']:.2f}x faster, "
            f"sparse attention alone {dense['speedup_sparse_attention_vs_dense_attention']:.2f}x")

    ceil = None if args.no_ceilings else ceilings(args, sh, x, Ks, Vs, idx, cnt, cap, timed)
    traffic = measured_traffic()
    step_gbps = bytes_["step"] / step_us / 1e3
    attn_gbps = bytes_["attn_per_layer"] / attn_launch_us / 1e3
    res = {
        "metric": "sparse-verify us/step + HBM GB/s (% roofline), 32k ctx, b=16, k=2048, w=4",
        "value": round(step_us, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_us / 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if sh.dtype == "bf16" else "f32",
        "data": "synthetic (seeded heavy-hitter Gaussian K/V/Q, projected draft)",
        "config": {
            "workload": f"{sh.name}: B={sh.B} n={sh.n} Hq={sh.Hq} Hkv={sh.Hkv} d={sh.d} w={sh.w} k={k} "
                        f"layers={sh.layers} draft={sh.L_d}x{sh.H_d}/{sh.Hkv_d}x{sh.d_d}",
            "global_batch": sh.B, "seq_len": sh.n, "k": k, "m": m, "n_sink": n_sink, "n_window": n_window,
            "scored_target_heads": len(x.sub_heads), "parallelism": "single-gpu",
        },
        "step_GBps": round(step_gbps, 1),
        "step_frac_of_hbm_peak": round(step_gbps / HBM_PEAK_GBPS, 4),
        "step_us_distribution": step_pct,
        "d2d_copy_GBps": round(copy_gbps, 1),
        "step_frac_of_d2d_copy": round(step_gbps / copy_gbps, 4),
        "step_algorithmic_bytes": bytes_["step"],
        "eager_us_per_step": round(eager_us, 2),
        "graph_us_per_step": None if graph_us is None else round(graph_us, 2),
        "components_us": {"score": round(score_us, 2), "select": round(select_us, 2),
                          "attention_per_launch": round(attn_launch_us, 3),
                          "attention_per_launch_eager_loop": round(attn_loop_us, 3),
                          "attention_single_launch_event_bracketed": round(attn_event_us, 3)},
        "roofline": {
            "kernel": "attn_bf16_kernel<128, 2, 8, false, false> (dustin_sparse_verify_attn)",
            "launch_us": round(attn_launch_us, 3),
            "bound": "hbm",
            "achieved": round(attn_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(attn_gbps / HBM_PEAK_GBPS, 4),
            "traffic": None if traffic is None else traffic["bytes_per_launch"],
            "algorithmic_bytes_per_launch": bytes_["attn_per_layer"],
            # the same bytes gathered by a kernel that does nothing else
            # (dustin_probe_gather_rows): the rate this access pattern reaches
            "achievable_GBps": None if ceil is None else ceil["gather_kv_rows_GBps"],
            "frac_of_achievable": None if ceil is None else round(attn_gbps / ceil["gather_kv_rows_GBps"], 4),
        },
        "ceilings": ceil,
        "dense_baseline": dense,
    }
    if not args.no_lse:
        res["supplied_draft_normalisers"] = supplied_lse_step(args, sh, x, kvs, dkv, k, m, n_sink, n_window, cap,
                                                              timed, bytes_)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline(sh, x, k, m, n_sink, n_window)
    if not args.no_evaluator:
        res["evaluator"] = evaluator(args, sh, x, kvs[0], cap, timed)
    if not args.no_sweep:
        res["policy_sweep"] = policy_sweep(args, sh, x, kvs[0], s_d, s_t, n_sink, n_window, timed)
    if not args.no_ksweep:
        res["k_sweep"] = k_sweep(args, sh, x, kvs, dkv, s_d, s_t, cap, timed)
    if not args.no_curve:
        res["estimator_curve"] = estimator_curve(args, sh, x, cap, timed)
    search = None
    if not args.no_search:
        res["config_search"] = search = config_search(args, sh)
    if not args.no_srh:
        res["srh_restricted_step"] = srh_step(args, sh, x, kvs, dkv, cap, timed, search)
    if not args.no_window:
        # Last of the c4 legs, because it writes the window rows into every layer's cache.
        res["verification_window"] = window_step(args, sh, x, Ks, Vs, k, m, n_sink, n_window, cap, timed)
    if not args.no_configs:
        res["other_configs"] = other_configs(args, cap, timed)
    if not args.no_timeline and args.config == "c4":
        res["attention_timeline"] = attn_timeline(args)
    print(json.dumps(res), flush=True)


def supplied_lse_step(args, sh, x, kvs, dkv, k, m, n_sink, n_window, cap, timed, bytes_):
    """Labelled extra line, never the headline: the step when the caller
    supplies the draft softmaxes' row normalisers (the draft model's own
    attention over the history computes them while drafting), so S_Draft
    reads the draft keys once.  The normalisers come from
    dustin_draft_row_lse, untimed here (it stands in for the draft model's
    attention output); its own time is reported beside."""
    import torch
    import sparse_kv_verification_amd as dk
    dev = x.q.device
    lse = dk.dustin_draft_row_lse(dkv, x.q_draft)
    s_d = torch.empty((sh.B, kvs[0].desc.N_max), dtype=torch.float32, device=dev)
    s_t = torch.empty_like(s_d)
    idx = torch.empty((sh.B, k), dtype=torch.int32, device=dev)
    cnt = torch.empty((sh.B,), dtype=torch.int32, device=dev)
    out = torch.empty_like(x.q)
    ws_s, ws_k, ws_a, ws_l = dk.Workspace(), dk.Workspace(), dk.Workspace(), dk.Workspace()

    def score():
        dk.dustin_score(dkv, x.q_draft, [kvs[0]], x.q_hist, x.sub_heads, sh.Hq, s_draft=s_d, s_target=s_t, ws=ws_s,
                        draft_lse=lse)

    def step():
        score()
        dk.dustin_topk(s_d, s_t, x.seq_lens, k, m, n_sink, n_window, idx=idx, count=cnt, want_tier=False, ws=ws_k)
        for l in range(sh.layers):
            dk.dustin_sparse_verify_attn(x.q, kvs[l], idx, cnt, out=out, ws=ws_a)

    reps = max(3, args.steps // 2)
    step_us = graph_time(args, step, cap, timed, reps)
    score_us = graph_time(args, score, cap, timed, reps)
    lse_us = graph_time(args, lambda: dk.dustin_draft_row_lse(dkv, x.q_draft, out=lse, ws=ws_l), cap, timed, reps)
    by = bytes_["step"]
    res = {"label": "not the headline: draft row normalisers supplied by the caller",
           "us_per_step": round(step_us, 1), "score_us": round(score_us, 1),
           "step_GBps": round(by / step_us / 1e3, 1), "step_frac_of_hbm_peak": round(by / step_us / 1e3 / HBM_PEAK_GBPS, 4),
           "draft_row_lse_query_us": round(lse_us, 1)}
    log(f"supplied draft normalisers (labelled line): step {step_us:.1f} us, score {score_us:.1f} us "
        f"(the normaliser query itself {lse_us:.1f} us)")
    return res


SWEEP_DELTAS = (1, 4, 16, 64)
SWEEP_KS = (128, 256, 512, 1024, 2048)


def ceilings(args, sh, x, Ks, Vs, idx, cnt, cap, timed):
    """Achievable HBM rates on this part, measured with the library's
    measurement kernels (dustin_probe_*): a streaming read of 4 GiB with the
    nontemporal and the default cache policy (each after 4 GiB of other
    reads, so nothing is cached), the gather of the step's K/V rows (the
    rows the attention reads for the current index set: 256-byte head rows
    of K and V, the attention's work split), timed like the attention (one
    launch per layer buffer, L launches replayed from a HIP graph), and a
    128 MiB re-read that the 256 MiB last-level cache (MALL) could serve,
    cold and warm, with either policy."""
    import torch
    import sparse_kv_verification_amd as dk
    dev = x.q.device
    out = {}
    big = torch.empty(1 << 30, dtype=torch.int32, device=dev)           # 4 GiB
    other = torch.empty_like(big)
    big.fill_(1)
    other.fill_(2)
    sink = torch.zeros(2048, dtype=torch.int32, device=dev)
    reps = 3

    def once(fn, flush=True):
        ts = []
        for _ in range(reps):
            if flush:
                dk.dustin_probe_stream_read(other, True, sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return sorted(ts)[reps // 2]

    nb = big.numel() * 4
    for nt in (True, False):
        us = once(lambda: dk.dustin_probe_stream_read(big, nt, sink))
        out["stream_read_" + ("nontemporal" if nt else "default") + "_GBps"] = round(nb / us / 1e3, 1)
    # the attention's gather: row (b, j, g) of K (and V) for every selected j
    B, N, Hkv = sh.B, x.K.shape[1], sh.Hkv
    sel = idx.long()
    valid = torch.arange(idx.shape[1], device=dev)[None, :] < cnt[:, None].long()
    jj = torch.where(valid, sel, torch.zeros_like(sel))
    rows = ((torch.arange(B, device=dev)[:, None, None] * N + jj[:, None, :]) * Hkv
            + torch.arange(Hkv, device=dev)[None, :, None])                # [B][Hkv][k]
    rows = rows.to(torch.int32).reshape(-1).contiguous()
    def gather_layers():
        for l in range(len(Ks)):
            dk.dustin_probe_gather_rows(Ks[l], rows, 256, 256, base2=Vs[l])

    us = graph_time(args, gather_layers, cap, timed, max(2, args.steps // 4)) / len(Ks)
    gb = rows.numel() * 256 * 2
    out["gather_kv_rows_GBps"] = round(gb / us / 1e3, 1)
    out["gather_kv_rows_us"] = round(us, 2)
    out["gather_kv_rows_bytes"] = gb
    # MALL: 128 MiB reads, four back-to-back under one pair of events: cold
    # = four distinct 128 MiB regions after 4 GiB of other reads; warm = one
    # region read four times after an untimed read of it
    mb = 128 << 20
    regions = [big[i * (mb // 4):(i + 1) * (mb // 4)] for i in range(4)]
    for nt in (True, False):
        cold, warm = [], []
        for _ in range(reps):
            for lst, bufs in ((cold, regions), (warm, [regions[0]] * 4)):
                dk.dustin_probe_stream_read(other, True, sink)
                if lst is warm:
                    dk.dustin_probe_stream_read(regions[0], nt, sink)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for r in bufs:
                    dk.dustin_probe_stream_read(r, nt, sink)
                e1.record()
                e1.synchronize()
                lst.append(e0.elapsed_time(e1) * 1e3)
        pol = "nontemporal" if nt else "default"
        out[f"mall_128MiB_cold_{pol}_GBps"] = round(4 * mb / sorted(cold)[reps // 2] / 1e3, 1)
        out[f"mall_128MiB_warm_{pol}_GBps"] = round(4 * mb / sorted(warm)[reps // 2] / 1e3, 1)
    del big, other
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log("ceilings: " + ", ".join(f"{k} {v}" for k, v in out.items()))
    return out


def evaluator(args, sh, x, kv, cap, timed):
    """Window attention A (Eq. 1) of one layer, as the evaluator, the policy
    sweep and the configuration search call it: w = 4 (the window's queries)
    and w = 8 (the window and its reverse, two slices of four steps), graph
    replayed.  Two passes read K (row normalisers, then probabilities), so
    the rate is given on twice the K bytes."""
    import torch
    import sparse_kv_verification_amd as dk
    q8 = torch.cat([x.q, x.q.flip(1)], dim=1).contiguous()
    kbytes = int(x.seq_lens.sum()) * sh.Hkv * sh.d * x.K.element_size()
    out = {}
    for w, q in ((sh.w, x.q), (2 * sh.w, q8)):
        A = torch.empty((sh.B, w, kv.desc.N_max), dtype=torch.float32, device=x.q.device)
        ws = dk.Workspace()
        fn = lambda: dk.dustin_window_attn(q, kv, A=A, ws=ws)
        us = graph_time(args, fn, cap, timed, max(3, args.steps // 2))
        out[f"w{w}"] = {"us": round(us, 1), "k_reads": 2 * ((w + 3) // 4),
                        "GBps_on_k_reads": round(2 * ((w + 3) // 4) * kbytes / us / 1e3, 1)}
    log("evaluator window attention: " + ", ".join(f"{k_} {v['us']:.0f} us ({v['GBps_on_k_reads']:.0f} GB/s over "
                                                   f"{v['k_reads']} K reads)" for k_, v in out.items()))
    return out


def policy_sweep(args, sh, x, kv, s_d, s_t, n_sink, n_window, timed):
    """Windowed ARR (Eq. 2) of the compared selection policies on the step's
    own scores and window queries, at several budgets: the SD oracle, the
    history policy at look-back distances 1/4/16/64, the draft lookahead and
    Dustin-T/D/H (mean over the batch), with the sweep's time and the
    oracle's time for the same sweep of one sequence."""
    import numpy as np
    import synth
    import sparse_kv_verification_amd as dk
    qpast = synth.history_trajectory(x, SWEEP_DELTAS)
    ks = [kk for kk in SWEEP_KS if kk >= n_sink + n_window]
    ms = [synth.tier_defaults(kk)[2] for kk in ks]
    ws = dk.Workspace()
    arr = dk.dustin_policy_sweep(x.q, qpast, kv, s_d, s_t, ks, ms, n_sink, n_window, ws=ws)
    us = timed(lambda: dk.dustin_policy_sweep(x.q, qpast, kv, s_d, s_t, ks, ms, n_sink, n_window, arr=arr, ws=ws),
               max(2, args.steps // 4))
    mean = arr.mean(dim=2).cpu().numpy()          # [policies][ks]
    names = ["oracle"] + [f"history_delta{dd}" for dd in SWEEP_DELTAS] + ["draft", "dustin_T", "dustin_D", "dustin_H"]
    table = {nm: {str(kk): round(float(mean[r, i]), 4) for i, kk in enumerate(ks)} for r, nm in enumerate(names)}
    log(f"policy sweep {us:.0f} us ({len(names)} policies x {len(ks)} budgets); windowed ARR at k={ks[-1]}: " +
        ", ".join(f"{nm} {mean[r, -1]:.3f}" for r, nm in enumerate(names)))
    out = {"us_per_sweep": round(us, 1), "deltas": list(SWEEP_DELTAS), "ks": ks, "m_hybrid": ms,
           "mean_windowed_arr": table}
    if not args.no_cpu_baseline:
        import oracle
        f = lambda t: t.detach().float().cpu().numpy().astype(np.float64)
        n = int(x.seq_lens[0])
        K = f(x.logical("K", 0))
        t0 = time.perf_counter()
        oracle.policy_sweep(f(x.q[0]), f(qpast[:, 0]), K, f(s_d[0, :n]), f(s_t[0, :n]), ks, ms, n_sink, n_window)
        dt = time.perf_counter() - t0
        out["cpu_oracle_one_sequence_s"] = round(dt, 2)
        out["cpu_oracle_scaled_us"] = round(dt * sh.B * 1e6, 0)
    return out


def graph_time(args, fn, cap, timed, reps):
    """HIP-graph replay time of fn (eager with --no-graph)."""
    import torch
    fn()
    torch.cuda.synchronize()
    if args.no_graph:
        return timed(fn, reps)
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(gr, stream=cap):
            fn()
    torch.cuda.synchronize()
    gr.replay()
    return timed(gr.replay, reps)


def k_sweep(args, sh, x, kvs, dkv, s_d, s_t, cap, timed):
    """The same 80-layer step at the other budgets of the 72B workload."""
    import torch
    import synth
    import sparse_kv_verification_amd as dk
    out = {}
    ws_s, ws_k, ws_a = dk.Workspace(), dk.Workspace(), dk.Workspace()
    for kk in sh.k_sweep:
        if kk == sh.k:
            continue
        ns, nw, mm = synth.tier_defaults(kk)
        idx = torch.empty((sh.B, kk), dtype=torch.int32, device=x.q.device)
        cnt = torch.empty((sh.B,), dtype=torch.int32, device=x.q.device)
        o = torch.empty_like(x.q)

        def step():
            dk.dustin_score(dkv, x.q_draft, [kvs[0]], x.q_hist, x.sub_heads, sh.Hq, s_draft=s_d, s_target=s_t, ws=ws_s)
            dk.dustin_topk(s_d, s_t, x.seq_lens, kk, mm, ns, nw, idx=idx, count=cnt, want_tier=False, ws=ws_k)
            for l in range(sh.layers):
                dk.dustin_sparse_verify_attn(x.q, kvs[l], idx, cnt, out=o, ws=ws_a)

        def attn_layers():
            for l in range(sh.layers):
                dk.dustin_sparse_verify_attn(x.q, kvs[l], idx, cnt, out=o, ws=ws_a)

        us = graph_time(args, step, cap, timed, max(2, args.steps // 4))
        a_us = graph_time(args, attn_layers, cap, timed, max(2, args.steps // 4)) / sh.layers
        bys = algorithmic_bytes(sh, x, kk, cnt, x.sub_heads)
        by, ab = bys["step"], bys["attn_per_layer"]
        out[str(kk)] = {"us_per_step": round(us, 1), "GBps": round(by / us / 1e3, 1),
                        "frac_of_hbm_peak": round(by / us / 1e3 / HBM_PEAK_GBPS, 4), "algorithmic_bytes": by,
                        "attention_us_per_launch": round(a_us, 2),
                        "attention_GBps": round(ab / a_us / 1e3, 1),
                        "attention_frac_of_hbm_peak": round(ab / a_us / 1e3 / HBM_PEAK_GBPS, 4),
                        "attention_algorithmic_bytes_per_launch": ab}
        log(f"k={kk}: step {us:.1f} us, {by / us / 1e3:.0f} GB/s; attention {a_us:.2f} us/launch "
            f"({ab / a_us / 1e3:.0f} GB/s, {ab / a_us / 1e3 / HBM_PEAK_GBPS:.3f} of peak)")
    return out


# The configuration the offline search picks on the synthetic profiling
# batch (its last measured result), used when the search leg is skipped.
SRH_DEFAULT = {"draft_layers": [0, 6, 12, 18, 23], "target_heads": [(10 * g, 8 * g) for g in range(8)]}


def srh_step(args, sh, x, kvs, dkv, cap, timed, search):
    """Dustin-H restricted to a searched configuration (blog section 2.4,
    Fig. 6: only the searched target heads and draft layers are scored; the
    efficiency figures of blog section 3, Fig. 8, are for that restricted
    estimator): the step with S_Draft over the searched draft layers and
    S_Target over the searched target heads (in their own layers), then the
    same select and L attention layers.  The headline step scores every
    draft layer and head, as the task defines S_Draft; this is an extra,
    labelled measurement.  Also the restricted score alone against dense
    full-cache attention of every layer (one point of the estimator curve)."""
    import torch
    import synth
    import sparse_kv_verification_amd as dk
    cfg = SRH_DEFAULT if not search else {"draft_layers": search["draft_layers"],
                                          "target_heads": [tuple(p) for p in search["target_heads"]]}
    dl = [int(l) for l in cfg["draft_layers"]]
    th = [(int(l), int(h)) for l, h in cfg["target_heads"]]
    t_layers = sorted({l for l, _ in th})
    sub = [(t_layers.index(l), h) for l, h in th]
    tk = [kvs[l] for l in t_layers]
    qd = x.q_draft[:, dl].contiguous() if dl else None
    dsub = [dkv[l] for l in dl]
    qh = x.q[:, -1][:, [h for _, h in th]].contiguous()      # the scored heads' most recent queries
    k = sh.k
    ns, nw, mm = synth.tier_defaults(k)
    s_d = torch.empty((sh.B, sh.n), dtype=torch.float32, device=x.q.device)
    s_t = torch.empty_like(s_d)
    idx = torch.empty((sh.B, k), dtype=torch.int32, device=x.q.device)
    cnt = torch.empty((sh.B,), dtype=torch.int32, device=x.q.device)
    o = torch.empty_like(x.q)
    ws_s, ws_k, ws_a, ws_d = dk.Workspace(), dk.Workspace(), dk.Workspace(), dk.Workspace()

    def score():
        dk.dustin_score(dsub, qd, tk, qh, sub, sh.Hq, s_draft=s_d if dl else None, s_target=s_t, ws=ws_s,
                        want_draft=bool(dl))

    def step():
        score()
        dk.dustin_topk(s_d if dl else None, s_t, x.seq_lens, k, mm, ns, nw, idx=idx, count=cnt, want_tier=False,
                       ws=ws_k)
        for l in range(sh.layers):
            dk.dustin_sparse_verify_attn(x.q, kvs[l], idx, cnt, out=o, ws=ws_a)

    def dense():
        for l in range(sh.layers):
            dk.dustin_sparse_verify_attn(x.q, kvs[l], None, None, out=o, ws=ws_d)

    reps = max(2, args.steps // 4)
    us = graph_time(args, step, cap, timed, reps)
    score_us = graph_time(args, score, cap, timed, reps)
    dense_us = None if args.no_dense else graph_time(args, dense, cap, timed, 2)
    # global layer ids for the byte count (U = distinct (layer, KV head) pairs)
    by = algorithmic_bytes(sh.replace(L_d=len(dl)), x, k, cnt, th)
    out = {"source": "config_search leg" if search else "default (search leg skipped)",
           "draft_layers": dl, "target_heads": [list(p) for p in th], "m": mm,
           "us_per_step": round(us, 1), "score_us": round(score_us, 1),
           "step_GBps": round(by["step"] / us / 1e3, 1),
           "step_frac_of_hbm_peak": round(by["step"] / us / 1e3 / HBM_PEAK_GBPS, 4),
           "algorithmic_bytes": by["step"]}
    if dense_us is not None:
        out["dense_attention_us"] = round(dense_us, 1)
        out["speedup_vs_dense_attention"] = round(dense_us / us, 2)
        out["score_normalized_by_dense"] = round(score_us / dense_us, 5)
    log(f"SRH-restricted Dustin-H ({len(dl)} draft layers, {len(th)} target heads over {len(t_layers)} layers): "
        f"step {us:.1f} us ({out['step_frac_of_hbm_peak']:.3f} of peak), score {score_us:.1f} us" +
        ("" if dense_us is None else f", {out['speedup_vs_dense_attention']:.2f}x faster than dense, score = "
                                      f"1/{1 / out['score_normalized_by_dense']:.0f} of dense"))
    return out


def other_configs(args, cap, timed):
    """One-layer steps (score, select, one attention layer) of the other
    workloads: tiny float32, 7B-shaped 16k, 32B-shaped 32k, ragged paged."""
    import torch
    import synth
    import sparse_kv_verification_amd as dk
    out = {}
    for name in ("c1", "c2", "c3", "c5"):
        sh = synth.preset(name).replace(layers=1)
        x = synth.make(sh, device="cuda")
        k = sh.k
        ns, nw, mm = synth.tier_defaults(k)
        kv = dk.KV(x.K, x.V, x.seq_lens, x.page_table)
        dkv = [dk.KV(x.Kd[l], None, x.seq_lens, x.page_table) for l in range(sh.L_d)]
        N = kv.desc.N_max
        s_d = torch.empty((sh.B, N), dtype=torch.float32, device="cuda")
        s_t = torch.empty_like(s_d)
        idx = torch.empty((sh.B, k), dtype=torch.int32, device="cuda")
        cnt = torch.empty((sh.B,), dtype=torch.int32, device="cuda")
        o = torch.empty_like(x.q)
        ws_s, ws_k, ws_a = dk.Workspace(), dk.Workspace(), dk.Workspace()

        def score():
            dk.dustin_score(dkv, x.q_draft, [kv], x.q_hist, x.sub_heads, sh.Hq, s_draft=s_d, s_target=s_t, ws=ws_s)

        def select():
            dk.dustin_topk(s_d, s_t, x.seq_lens, k, mm, ns, nw, idx=idx, count=cnt, want_tier=False, ws=ws_k)

        def attn():
            dk.dustin_sparse_verify_attn(x.q, kv, idx, cnt, out=o, ws=ws_a)

        def step():
            score()
            select()
            attn()

        reps = max(3, args.steps // 2)
        us = graph_time(args, step, cap, timed, reps)
        parts = {nm: round(graph_time(args, fn, cap, timed, reps), 1)
                 for nm, fn in (("score", score), ("select", select), ("attention", attn))}
        by = algorithmic_bytes(sh, x, k, cnt, x.sub_heads)["step"]
        out[name] = {"workload": f"{sh.name}: B={sh.B} n={sh.n}{' (ragged, paged)' if sh.n_lo else ''} "
                                 f"Hq={sh.Hq} Hkv={sh.Hkv} d={sh.d} w={sh.w} k={k} {sh.dtype}, one layer",
                     "us_per_step": round(us, 1), "GBps": round(by / us / 1e3, 1),
                     "frac_of_hbm_peak": round(by / us / 1e3 / HBM_PEAK_GBPS, 4), "algorithmic_bytes": by,
                     "components_us": parts}
        if not args.no_lse and sh.dtype == "bf16":
            # labelled, not the line above: the same step with the draft row
            # normalisers supplied (one read of draft K)
            lse = dk.dustin_draft_row_lse(dkv, x.q_draft)

            def step_lse():
                dk.dustin_score(dkv, x.q_draft, [kv], x.q_hist, x.sub_heads, sh.Hq, s_draft=s_d, s_target=s_t,
                                ws=ws_s, draft_lse=lse)
                select()
                attn()

            us_l = graph_time(args, step_lse, cap, timed, reps)
            out[name]["supplied_draft_normalisers"] = {
                "us_per_step": round(us_l, 1), "frac_of_hbm_peak": round(by / us_l / 1e3 / HBM_PEAK_GBPS, 4)}
        log(f"{name}: one-layer step {us:.1f} us, {by / us / 1e3:.0f} GB/s; parts {parts}"
            + (f"; with supplied draft normalisers {out[name]['supplied_draft_normalisers']['us_per_step']} us"
               if "supplied_draft_normalisers" in out[name] else ""))
        del x, kv, dkv, s_d, s_t
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


SEARCH = dict(B=8, n=8192, k=512, T=64, S=8, max_draft=24)


def config_search(args, sh):
    """The offline configuration search (blog section 2.4, Fig. 6) on a
    synthetic multi-layer profiling batch with the target's full depth
    (sh.layers layers x H_q heads, every head a candidate) and the draft's
    layers: per-layer window attention for the objective, per-head S_Target
    rows, the SRH score matrix and its head TopK (T), greedy target heads
    (at most S), greedy draft layers, and the m search.  Each phase is timed
    with a device synchronisation around it (the greedy steps read their
    objectives back every round)."""
    import numpy as np
    import torch
    import synth
    import sparse_kv_verification_amd as dk
    P = SEARCH
    ssh = sh.replace(B=P["B"], n=P["n"], L_d=sh.L_d)
    k = P["k"]
    n_sink, n_window, m0 = synth.tier_defaults(k)
    ms = list(range(0, k - n_sink - n_window + 1, 8))
    L, B, N, Hq = sh.layers, ssh.B, ssh.n, sh.Hq
    t0 = time.perf_counter()
    x = synth.make_search(ssh, L, device="cuda")
    torch.cuda.synchronize()
    log(f"config search: profiling batch generated in {time.perf_counter() - t0:.1f}s "
        f"({L} target layers x {Hq} heads, {ssh.L_d} draft layers, B={B}, n={N}, k={k})")
    dev = x.K.device
    abar_l = torch.empty((L, B, N), dtype=torch.float32, device=dev)
    units = torch.empty((L * Hq, B, N), dtype=torch.float32, device=dev)
    d_units = torch.empty((ssh.L_d, B, N), dtype=torch.float32, device=dev)
    heads = [(0, h) for h in range(Hq)]
    kvs = [dk.KV(x.K[l], None, x.seq_lens, None) for l in range(L)]
    dkvs = [dk.KV(x.Kd[l], None, x.seq_lens, None) for l in range(ssh.L_d)]
    qd = [x.q_draft[:, l:l + 1].contiguous() for l in range(ssh.L_d)]
    A = torch.empty((B, ssh.w, N), dtype=torch.float32, device=dev)
    us = {}

    def phase(name, fn):
        torch.cuda.synchronize()
        t = time.perf_counter()
        out = fn()
        torch.cuda.synchronize()
        us[name] = round((time.perf_counter() - t) * 1e6, 1)
        return out

    def objective_rows():
        for l in range(L):
            dk.dustin_window_attn(x.q[l], kvs[l], A=A)
            dk.dustin_window_mean(A, Abar=abar_l[l])
        return dk.dustin_window_mean(abar_l.reshape(1, L, B * N)).reshape(B, N)

    def head_rows():
        for l in range(L):
            dk.dustin_head_scores([kvs[l]], x.q_prev[l], heads, Hq, out=units[l * Hq:(l + 1) * Hq])

    def draft_rows():
        for l in range(ssh.L_d):
            dk.dustin_score([dkvs[l]], qd[l], [dkvs[l]], None, None, Hq, s_draft=d_units[l], want_target=False)

    for _ in range(2):                     # the second pass is timed (workspaces allocated, code loaded)
        us = {}
        abar = phase("objective_attention", objective_rows)
        phase("head_rows", head_rows)
        _, M = phase("srh_matrix", lambda: dk.dustin_candidate_arr(x.seq_lens, abar, k, 0, n_sink, n_window,
                                                                     target_units=units))
        nM = torch.full((1,), L * Hq, dtype=torch.int32, device=dev)
        idx, cnt, _ = phase("srh_topk", lambda: dk.dustin_topk(None, M[None].contiguous(), nM, P["T"], 0, 0, 0,
                                                               want_tier=False))
        cand = [int(i) for i in idx[0, :int(cnt[0])].cpu()]
        ch_t, curve_t, s_t = phase("greedy_target", lambda: dk.dustin_greedy_select(
            units, x.seq_lens, abar, k, 0, n_sink, n_window, P["S"], 0, unit_ids=cand))
        phase("draft_rows", draft_rows)
        ch_d, curve_d, s_d = phase("greedy_draft", lambda: dk.dustin_greedy_select(
            d_units, x.seq_lens, abar, k, m0, n_sink, n_window, P["max_draft"], 1, s_target_fixed=s_t))
        vals = None
        if ch_d:
            _, vals = phase("m_search", lambda: dk.dustin_candidate_arr(x.seq_lens, abar, k, 0, n_sink, n_window,
                                                                        s_draft=s_d, s_target=s_t, m_cand=ms))
    us["total"] = round(sum(us.values()), 1)
    vals = None if vals is None else vals.cpu().numpy()
    m_best = ms[int(np.argmax(vals))] if vals is not None else 0
    rho = x.rho.numpy()
    target_heads = [(cand[c] // Hq, cand[c] % Hq) for c in ch_t]
    out = {
        "workload": f"{L} target layers x {Hq} heads (head_dim {sh.d}), {ssh.L_d} draft layers x {ssh.H_d} heads, "
                    f"profiling batch B={B}, n={N}, k={k}, T={P['T']}, S<={P['S']}, w={ssh.w}",
        "us": us,
        "srh_matrix_rho_corr": round(float(np.corrcoef(M.cpu().numpy(), rho.ravel())[0, 1]), 3),
        "target_heads": target_heads, "target_curve": [round(v, 4) for v in curve_t],
        "draft_layers": ch_d, "draft_curve": [round(v, 4) for v in curve_d],
        "m": m_best, "objective": round(float(vals.max()), 4) if vals is not None else None,
    }
    log(f"config search {us['total'] / 1e3:.1f} ms ({', '.join(f'{kk} {v / 1e3:.2f}' for kk, v in us.items() if kk != 'total')} ms); "
        f"heads {target_heads} curve {out['target_curve']}; draft {ch_d} curve {out['draft_curve']}; m {m_best}, "
        f"objective {out['objective']}")
    if not args.no_cpu_baseline:
        import oracle
        f = lambda t: t.detach().float().cpu().numpy().astype(np.float64)
        t = time.perf_counter()
        Ao = [[oracle.window_attention(f(x.q[l, 0]), f(x.K[l, 0])) for l in range(L)]]
        hp = np.stack([oracle.head_probs(f(x.q_prev[l, 0])[None], f(x.K[l, 0]))[:, 0] for l in range(L)])[None]
        du = np.stack([oracle.score_draft(f(x.q_draft[0, l:l + 1]), f(x.Kd[l:l + 1, 0]))[None]
                       for l in range(ssh.L_d)])
        oracle.config_search(Ao, hp, du, k, m0, ms, n_sink, n_window, P["T"], P["S"], P["max_draft"])
        dt = time.perf_counter() - t
        out["cpu_oracle_one_sequence_s"] = round(dt, 1)
        out["cpu_oracle_note"] = "the same search on sequence 0 alone (B = 1), fp64 NumPy"
        log(f"config search: oracle on one sequence {dt:.1f}s")
    del x, units, d_units, abar_l, kvs, dkvs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


CURVE_NS = (4096, 8192, 16384, 32768)
CURVE_DISTINCT_LAYERS = 8


def estimator_curve(args, sh, x, cap, timed):
    """Criticality-estimation cost against context length, normalised by
    full-cache attention (the comparison of the blog's Fig. 8), per
    verification step of the whole target model (sh.layers layers):
      dense     full-cache attention of the w window queries, every layer
      naive     every head of every layer scored: the draft side over all
                draft layers and heads plus all H_q target heads of every
                target layer (S_Target materialised per layer)
      quest16   page scores of every layer from 16-position min/max key
                bounds (bounds built outside the timed region: they are kept
                up to date as pages fill)
      dustin_T  the scored target-head subset (S heads of one layer)
      dustin_D  the draft side as configured
      dustin_H  both sides (the step's score call)
    normalized_byte_floor is the same ratio for the bytes each estimator has
    to read (K of the scored layers, draft K, page bounds), which a faster
    kernel cannot go below.
    The n-position inputs are the first n positions of the generated cache.
    Per-layer work cycles over 8 distinct layer buffers, each far larger
    than the last-level cache, so no launch is served from cache.  Every
    estimator is replayed from a HIP graph and timed with events."""
    import torch
    import sparse_kv_verification_amd as dk
    if x.page_table is not None:
        return None
    dev = x.q.device
    NL = CURVE_DISTINCT_LAYERS
    reps = max(2, args.steps // 4)
    all_heads = [(0, h) for h in range(sh.Hq)]
    q_all = x.q[:, -1].contiguous()                     # [B][H_q][d]: one target query per head
    rows = []

    def graph_us(fn):
        fn()
        torch.cuda.synchronize()
        if args.no_graph:
            return timed(fn, reps)
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            fn()
            torch.cuda.synchronize()
            with torch.cuda.graph(gr, stream=cap):
                fn()
        torch.cuda.synchronize()
        gr.replay()
        return timed(gr.replay, reps)

    for n in CURVE_NS:
        if n > sh.n:
            continue
        lens = torch.full((sh.B,), n, dtype=torch.int32, device=dev)
        Kn = [x.K[:, :n].clone() for _ in range(NL)]
        Vn = [x.V[:, :n].clone() for _ in range(NL)]
        kv = [dk.KV(Kn[i], Vn[i], lens, None) for i in range(NL)]
        Kd = [x.Kd[l][:, :n].contiguous() for l in range(sh.L_d)]
        dkv = [dk.KV(Kd[l], None, lens, None) for l in range(sh.L_d)]
        s_d = torch.empty((sh.B, n), dtype=torch.float32, device=dev)
        s_t = torch.empty_like(s_d)
        out = torch.empty_like(x.q)
        ws = {nm: dk.Workspace() for nm in ("dense", "naive_t", "naive_d", "t", "d", "h")}
        bounds = [dk.dustin_page_bounds(kv[i]) for i in range(NL)]
        pscores = torch.empty((sh.B, (n + 15) // 16), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

        def dense():
            for l in range(sh.layers):
                dk.dustin_sparse_verify_attn(x.q, kv[l % NL], None, None, out=out, ws=ws["dense"])

        def naive():
            dk.dustin_score(dkv, x.q_draft, [kv[0]], None, None, sh.Hq, s_draft=s_d, ws=ws["naive_d"],
                            want_target=False)
            for l in range(sh.layers):
                dk.dustin_score([], None, [kv[l % NL]], q_all, all_heads, sh.Hq, s_target=s_t, ws=ws["naive_t"],
                                want_draft=False)

        def quest():
            for l in range(sh.layers):
                dk.dustin_page_scores(x.q, kv[l % NL], bounds[l % NL][0], bounds[l % NL][1], scores=pscores)

        def quest_bounds():
            for i in range(NL):
                dk.dustin_page_bounds(kv[i], bounds[i][0], bounds[i][1])

        def dustin_t():
            dk.dustin_score([], None, [kv[0]], x.q_hist, x.sub_heads, sh.Hq, s_target=s_t, ws=ws["t"],
                            want_draft=False)

        def dustin_d():
            dk.dustin_score(dkv, x.q_draft, [kv[0]], None, None, sh.Hq, s_draft=s_d, ws=ws["d"], want_target=False)

        def dustin_h():
            dk.dustin_score(dkv, x.q_draft, [kv[0]], x.q_hist, x.sub_heads, sh.Hq, s_draft=s_d, s_target=s_t,
                            ws=ws["h"])

        us = {nm: graph_us(fn) for nm, fn in (("dense", dense), ("naive", naive), ("quest16", quest),
                                               ("dustin_T", dustin_t), ("dustin_D", dustin_d),
                                               ("dustin_H", dustin_h))}
        bounds_us = timed(quest_bounds, reps) / NL
        # page scores per launch against the HBM peak: both bounds tensors, q and the scores
        eb = x.K.element_size()
        pbytes = (2 * sh.B * ((n + 15) // 16) * sh.Hkv * sh.d * eb + sh.B * sh.w * sh.Hq * sh.d * eb
                  + sh.B * ((n + 15) // 16) * 4)
        p_us = us["quest16"] / sh.layers
        # bytes every estimator must read at least, against dense attention's K + V of every layer
        kbytes = sh.B * n * sh.Hkv * sh.d * eb
        dbytes = sh.L_d * sh.B * n * sh.Hkv_d * sh.d_d * x.Kd[0].element_size()
        floors = {"naive": (kbytes * sh.layers + dbytes) / (2 * kbytes * sh.layers),
                  "quest16": (2 * kbytes / 16 * sh.layers) / (2 * kbytes * sh.layers),
                  "dustin_T": kbytes / (2 * kbytes * sh.layers),
                  "dustin_D": dbytes / (2 * kbytes * sh.layers),
                  "dustin_H": (kbytes + dbytes) / (2 * kbytes * sh.layers)}
        row = {"n": n, "us": {k_: round(v, 1) for k_, v in us.items()},
               "normalized": {k_: round(v / us["dense"], 5) for k_, v in us.items() if k_ != "dense"},
               "normalized_byte_floor": {k_: round(v, 5) for k_, v in floors.items()},
               "quest16_page_scores_per_launch_us": round(p_us, 2),
               "quest16_page_scores_GBps": round(pbytes / p_us / 1e3, 1),
               "quest16_page_scores_frac": round(pbytes / p_us / 1e3 / HBM_PEAK_GBPS, 4),
               "quest16_page_bounds_per_layer_us": round(bounds_us, 1)}
        log(f"estimator curve n={n}: dense {us['dense']:.0f} us; normalized " +
            ", ".join(f"{k_} {v:.4f} (1/{1 / v:.0f})" for k_, v in row["normalized"].items()) +
            f"; page scores {p_us:.2f} us/launch ({row['quest16_page_scores_GBps']:.0f} GB/s)")
        rows.append(row)
        del Kn, Vn, kv, Kd, dkv, bounds, ws
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return {"layers": sh.layers, "distinct_layer_buffers": NL, "draft_layers": sh.L_d, "draft_heads": sh.H_d,
            "target_heads_scored": len(x.sub_heads), "rows": rows}


def window_step(args, sh, x, Ks, Vs, k, m, n_sink, n_window, cap, timed):
    """The step with the draft window in the cache: score, select, L causal
    verification attentions over the set plus the window, each appending its
    layer's window rows to the cache in the same launch
    (dustin_verify_attn_append), and the commit.  The same step with the
    appends as separate launches (dustin_append_window_kv for every layer,
    then dustin_verify_attn) is timed beside it.  The histories are w shorter
    than the generated ones so the window fits behind them; the commit
    accepts 0 tokens so the timed step repeats on the same lengths."""
    import torch
    import sparse_kv_verification_amd as dk
    dev = x.q.device
    lens_w = (x.seq_lens - sh.w).clamp_min(0).to(torch.int32)
    kvw = [dk.KV(Ks[l], Vs[l], lens_w, x.page_table) for l in range(sh.layers)]
    dkw = [dk.KV(x.Kd[l], None, lens_w, x.page_table) for l in range(sh.L_d)]
    g = torch.Generator(device=dev)
    g.manual_seed(1000 + sh.seed)
    shp = (sh.B, sh.w, sh.Hkv, sh.d)
    k_win = torch.randn(shp, generator=g, device=dev).to(x.K.dtype)
    v_win = torch.randn(shp, generator=g, device=dev).to(x.K.dtype)
    accepted = torch.zeros((sh.B,), dtype=torch.int32, device=dev)
    s_d = torch.empty((sh.B, sh.n), dtype=torch.float32, device=dev)
    s_t = torch.empty_like(s_d)
    idx = torch.empty((sh.B, k), dtype=torch.int32, device=dev)
    cnt = torch.empty((sh.B,), dtype=torch.int32, device=dev)
    out = torch.empty_like(x.q)
    ws_s, ws_k, ws_v = dk.Workspace(), dk.Workspace(), dk.Workspace()

    def append():
        for l in range(sh.layers):
            dk.dustin_append_window_kv(kvw[l], k_win, v_win)

    def verify():
        for l in range(sh.layers):
            dk.dustin_verify_attn(x.q, kvw[l], idx, cnt, out=out, ws=ws_v)

    def verify_fused():
        for l in range(sh.layers):
            dk.dustin_verify_attn_append(x.q, kvw[l], k_win, v_win, idx, cnt, out=out, ws=ws_v)

    def select():
        dk.dustin_score(dkw, x.q_draft, [kvw[0]], x.q_hist, x.sub_heads, sh.Hq, s_draft=s_d, s_target=s_t, ws=ws_s)
        dk.dustin_topk(s_d, s_t, lens_w, k, m, n_sink, n_window, idx=idx, count=cnt, want_tier=False, ws=ws_k)

    def step():
        select()
        verify_fused()
        dk.dustin_commit_window(lens_w, accepted, sh.w)

    def step_separate():
        append()
        select()
        verify()
        dk.dustin_commit_window(lens_w, accepted, sh.w)

    for _ in range(max(1, args.warmup)):
        step_separate()
        step()
    torch.cuda.synchronize()
    fns = (step, verify_fused, step_separate, verify)
    runs = list(fns)
    graphs = []
    if not args.no_graph:
        for fn in fns:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.stream(cap):
                with torch.cuda.graph(gr, stream=cap):
                    fn()
            torch.cuda.synchronize()
            gr.replay()
            graphs.append(gr)
        runs = [gr.replay for gr in graphs]
    step_us = timed(runs[0], args.steps)
    fused_us = timed(runs[1], args.steps) / sh.layers
    step_sep_us = timed(runs[2], args.steps)
    verify_us = timed(runs[3], args.steps) / sh.layers
    append_us = timed(append, args.steps) / sh.layers
    commit_us = timed(lambda: dk.dustin_commit_window(lens_w, accepted, sh.w), args.steps)
    esz = x.K.element_size()
    rows = int(cnt.sum()) + sh.B * sh.w
    per_layer = rows * sh.Hkv * sh.d * esz * 2 + 2 * x.q.numel() * esz + sh.B * k * 4 + sh.B * 4
    log(f"window step {step_us:.1f} us (appends fused into the attention; {step_sep_us:.1f} us with separate "
        f"appends); verify attention + append {fused_us:.2f} us/launch, verify attention alone {verify_us:.2f} "
        f"us/launch ({per_layer / verify_us / 1e3:.0f} GB/s), separate append {append_us:.2f} us/layer, "
        f"commit {commit_us:.2f} us")
    return {
        "step_us": round(step_us, 2),
        "step_us_separate_appends": round(step_sep_us, 2),
        "verify_attn_append_per_launch_us": round(fused_us, 3),
        "verify_attn_per_launch_us": round(verify_us, 3),
        "verify_attn_GBps": round(per_layer / verify_us / 1e3, 1),
        "verify_attn_algorithmic_bytes_per_launch": per_layer,
        "append_per_layer_us_eager": round(append_us, 3),
        "commit_us_eager": round(commit_us, 3),
        "timing": "graph replay" if graphs else "eager",
        "histories": "generated lengths minus w (room for the window)",
    }


if __name__ == "__main__":
    main()
