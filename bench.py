"""Benchmark: verified tree-nodes/s for one verification pass of a drafted token tree.

One step = the whole hot path on one batch: ancestor-mask build, tree attention over
the KV prefix + ancestors, acceptance (rejection sampling for the Llama-3-70B-shaped
layer), and KV compaction of the accepted path.  Inputs are seeded synthetic arrays
already resident in HBM; several buffer sets rotate so that the timed footprint is at
least 512 MB (twice the 256 MB Infinity Cache) and no step reads a cache-warm copy.
The steps of one rotation through the sets are captured into one HIP graph
(torch.cuda.CUDAGraph) and replayed, so the timed loop measures the GPU rather than Python
marshalling or per-step graph launches.

Printed: one JSON line with the metric, per-kernel timings, the attention kernel's
roofline fraction (HIP events around that kernel's launches on its own stream) and the
CPU oracle's throughput on the same workload as a reported baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import tree_attention_verification_ev_amd as ev  # noqa: E402
from synth import CONFIGS, config_by_name, draft_tree_logits, generate, sampled_drafts  # noqa: E402
from synth.device import to_device  # noqa: E402

METRIC = "verified tree-nodes/s + KV HBM GB/s (% roofline), GQA 64/8 d128 L=4096 T=64"
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
FOOTPRINT_BYTES = 512 << 20
ATTN_SRC = os.path.join(ROOT, "tree_attention_verification_ev_amd", "csrc", "tree_attention.hip")


def algorithmic_work(inp):
    """Bytes and flops of one attention launch by the definitions of the method."""
    cfg = inp.cfg
    e = 2 if cfg.dtype == "bf16" else 4
    anc_depth = []
    for p in inp.parent:
        depth = np.zeros(cfg.T, np.int64)
        for i in range(1, cfg.T):
            depth[i] = depth[p[i]] + 1
        anc_depth.append(int((depth + 1).sum()))
    L = inp.prefix_len.astype(np.int64)
    kv_bytes = int(sum(2 * cfg.Hkv * (L[b] + cfg.T) * cfg.d * e for b in range(cfg.B)))
    qo_bytes = 2 * cfg.B * cfg.T * cfg.Hq * cfg.d * e + 4 * cfg.B * cfg.T * cfg.Hq
    table = 0
    if inp.layout == "paged":
        table = int(sum(4 * math.ceil((L[b] + cfg.T) / cfg.block_size) for b in range(cfg.B)))
    flops = int(sum(4 * cfg.Hq * cfg.d * (cfg.T * L[b] + anc_depth[b]) for b in range(cfg.B)))
    return {"bytes": kv_bytes + qo_bytes + table, "kv_bytes": kv_bytes, "flops": flops,
            "logit_bytes": 4 * cfg.B * cfg.T * cfg.V}


# Calls timed one by one; the step runs STEP_PARTS (the four steps in two calls).
ALL_PARTS = ("mask", "attention", "mask_attention", "accept", "compact", "accept_compact")
STEP_PARTS = ("mask_attention", "accept_compact")
ATTN_PART = "mask_attention"          # the attention call the step makes (roofline, rates)


class BufferSet:
    """Device inputs, preallocated outputs and the per-call graphs of one batch copy."""

    def __init__(self, inp, dev, ws_attn, ws_acc):
        cfg = inp.cfg
        self.cfg, self.d = cfg, dev
        self.kv = ev.KvCache(dev.k, dev.v, dev.block_table)
        B, T = cfg.B, cfg.T
        z = lambda *s, dt=torch.int32: torch.zeros(s, dtype=dt, device="cuda")
        self.anc, self.depth = z(B, T, dt=torch.int64), z(B, T)
        self.out = torch.empty_like(dev.q)
        self.lse = z(B, T, cfg.Hq, dt=torch.float32)
        self.acc, self.path, self.tok, self.new_len = z(B), z(B, T), z(B, T), z(B)
        self.status = z(1)
        self.ws_attn, self.ws_acc = ws_attn, ws_acc
        self.scale = float(np.float32(1.0 / math.sqrt(cfg.d)))
        self.max_prefix = int(inp.prefix_len.max())
        self.mode = "rejection" if "rejection" in cfg.accept else "greedy"

    def mask(self):
        ev.ev_tree_mask_build(self.d.parent, self.anc, self.depth, self.status)

    def mask_attention(self):
        ev.ev_tree_mask_attention(self.d.q, self.kv, self.d.prefix_len, self.d.parent, self.scale,
                                  self.out, self.lse, self.anc, self.depth, self.ws_attn,
                                  self.status, max_prefix_len=self.max_prefix)

    def attention(self):
        ev.ev_tree_attention(self.d.q, self.kv, self.d.prefix_len, self.anc, self.scale, self.out,
                             self.lse, self.ws_attn, self.status, max_prefix_len=self.max_prefix)

    def accept(self):
        if self.mode == "rejection":
            ev.ev_accept_rejection(self.d.logits, self.d.tokens, self.d.parent, self.d.tau,
                                   self.d.uniforms, self.acc, self.path, self.tok, self.ws_acc,
                                   self.status)
        else:
            ev.ev_accept_greedy(self.d.logits, self.d.tokens, self.d.parent, self.acc, self.path,
                                self.tok, self.ws_acc, self.status)

    def compact(self):
        ev.ev_kv_compact(self.kv, self.d.prefix_len, self.path, self.acc, self.new_len, self.status)

    def accept_compact(self):
        if self.mode == "rejection":
            ev.ev_accept_rejection_compact(self.d.logits, self.d.tokens, self.d.parent, self.d.tau,
                                           self.d.uniforms, self.kv, self.d.prefix_len, self.acc,
                                           self.path, self.tok, self.new_len, self.ws_acc,
                                           self.status)
        else:
            ev.ev_accept_greedy_compact(self.d.logits, self.d.tokens, self.d.parent, self.kv,
                                        self.d.prefix_len, self.acc, self.path, self.tok,
                                        self.new_len, self.ws_acc, self.status)

    def step(self):
        # mask build with attention, and acceptance with compaction: two calls (three
        # launches with the split merge) for the four steps of the pass
        self.mask_attention()
        self.accept_compact()


def capture(fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def prime_gpu(ms: float = 20.0):
    """Queue a few ms of unrelated GPU work so that the host enqueues ahead of the device."""
    a = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(4):
        a = a @ a
        a = a / (a.abs().amax() + 1)
    torch.cuda.synchronize()
    per = (time.perf_counter() - t0) / 4
    for _ in range(max(1, int(ms / 1e3 / max(per, 1e-6)))):
        a = a @ a
    return a


def kernel_times(sets, reps):
    """Average device time of one call of each part of the step, from HIP events on the
    launch stream around a graph of back-to-back calls that cycles through the buffer
    sets (so each call reads cache-cold inputs and graph-launch overhead is amortised)."""
    out = {}
    n_calls = len(sets) * max(1, math.ceil(32 / len(sets)))
    for name in ALL_PARTS:
        calls = [getattr(sets[i % len(sets)], name) for i in range(n_calls)]
        g = capture(lambda: [c() for c in calls])
        g.replay()
        torch.cuda.synchronize()
        keep = prime_gpu()
        pairs = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        del keep
        ts = [a.elapsed_time(b) * 1e3 / n_calls for a, b in pairs]
        out[name] = {"mean_us": statistics.fmean(ts), "median_us": statistics.median(ts),
                     "p10_us": float(np.percentile(ts, 10)), "p90_us": float(np.percentile(ts, 90)),
                     "calls_per_graph": n_calls}
    return out


def box_peaks(reps: int = 3):
    """What this GPU sustains, for rooflines against the box as well as the published peaks:
    the bf16 matrix-core rate of a register-operand MFMA loop (four independent
    32x32x16 products per wavefront, 4 wavefronts per CU-slot) and the bandwidths of a
    16-byte grid-stride copy and read of 2 GiB; each is the best of `reps` timed launches."""
    n_wg, iters = 1024, 20000
    flops = n_wg * 4 * iters * 4 * 32768
    sink = torch.empty(n_wg, dtype=torch.float32, device="cuda")
    ev.ev_peak_mfma_bf16(n_wg, 200, sink)
    mfma = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ev.ev_peak_mfma_bf16(n_wg, iters, sink)
        e1.record()
        torch.cuda.synchronize()
        mfma = max(mfma, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    src = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    ev.ev_peak_copy(src, dst)
    copy = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ev.ev_peak_copy(src, dst)
        e1.record()
        torch.cuda.synchronize()
        copy = max(copy, 2 * src.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    sink_r = torch.empty(64 * 256, dtype=torch.int32, device="cuda")
    read = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ev.ev_peak_read(src, sink_r)
        e1.record()
        torch.cuda.synchronize()
        read = max(read, src.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, dst
    return {"mfma_bf16_tflops": mfma, "copy_gbps": copy, "read_gbps": read,
            "method": "ev_peak_mfma_bf16 (1024 workgroups x 20000 rounds), ev_peak_copy "
                      "(2 GiB, read + write counted) and ev_peak_read (2 GiB, 16384 workgroups), "
                      "best of 3 each"}


def _counter_values(csv_path, counter):
    """Per-dispatch values of one counter in a rocprofv3 counter_collection.csv, by kernel."""
    import csv
    acc = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return acc


TRAFFIC_PARTS = {
    # part: (kernel-name keys, source file, record file stem)
    "attention": (("tree_attn_", "attn_merge_kernel"), ATTN_SRC, "tree_attention"),
    "accept": (("accept_kernel",), os.path.join(ROOT, "tree_attention_verification_ev_amd", "csrc",
                                                "accept.hip"), "accept"),
}


def traffic_path(part, workload):
    return os.path.join(ROOT, "profiles", f"{TRAFFIC_PARTS[part][2]}_{workload}_traffic.json")


def write_traffic(fetch_csv, write_csv, command, part="attention", workload="llama3_70b_layer"):
    """HBM bytes per call of one part of the step (attention: main + split merge kernels;
    accept: the acceptance kernel) from two rocprofv3 --pmc runs of `bench.py --calibrate`,
    each counter scaled by what it reads for the 256 MiB device copy of the same run."""
    fetch, write = _counter_values(fetch_csv, "FETCH_SIZE"), _counter_values(write_csv, "WRITE_SIZE")
    copy_kib = (256 << 20) / 1024
    keys, src, _ = TRAFFIC_PARTS[part]

    def pick(table, key):
        hits = [(k, v) for k, v in table.items() if key in k]
        return max(hits, key=lambda kv: len(kv[1])) if hits else None

    # the calibration copy is the largest device copy of the run
    cal_f = copy_kib / max(max(v) for k, v in fetch.items() if "copyBuffer" in k)
    cal_w = copy_kib / max(max(v) for k, v in write.items() if "copyBuffer" in k)
    kernels = {}
    total = 0.0
    for key in keys:
        pf, pw = pick(fetch, key), pick(write, key)
        if pf is None or pw is None:
            continue                     # e.g. no split merge at a one-split plan
        (kf, vf), (kw, vw) = pf, pw
        f_kib, nf, w_kib, nw = statistics.fmean(vf), len(vf), statistics.fmean(vw), len(vw)
        b = f_kib * 1024 * cal_f + w_kib * 1024 * cal_w
        kernels[kf] = {"fetch_kib": f_kib, "write_kib": w_kib, "dispatches": [nf, nw],
                       "hbm_bytes": b}
        total += b
    if not kernels:
        raise SystemExit(f"no kernel matching {keys} in the counter files")
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    inp = generate(config_by_name(workload), with_kv=False, with_logits=False)
    work = algorithmic_work(inp)
    algo = work["bytes"] if part == "attention" else work["logit_bytes"]
    rec = {"workload": workload, "part": part, "hbm_bytes_per_launch": total,
           "algorithmic_bytes": algo, "ratio_to_algorithmic": total / algo,
           "fetch_calibration": cal_f, "write_calibration": cal_w, "kernels": kernels,
           "source_sha256": sha, "command": command}
    with open(traffic_path(part, workload), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def traffic_entry(workload):
    """HBM bytes per attention launch from committed rocprofv3 counter runs of this
    workload, if they were taken on the current kernel source."""
    try:
        with open(traffic_path("attention", workload)) as f:
            t = json.load(f)
        with open(ATTN_SRC, "rb") as f:
            h = hashlib.sha256(f.read()).hexdigest()
        if t.get("source_sha256") != h:
            return None
        return t["hbm_bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def cpu_description():
    """CPU model and the BLAS library numpy runs on (as threadpoolctl reports them)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    from threadpoolctl import threadpool_info
    blas = [{"api": p.get("internal_api"), "version": p.get("version"),
             "threads": p.get("num_threads"), "library": os.path.basename(p.get("filepath", ""))}
            for p in threadpool_info() if p.get("user_api") == "blas"]
    return model, blas


def cpu_baseline(inp, budget_s: float):
    """The oracle, untouched, on the host: whole verification steps for about budget_s
    seconds (the reported value), then the median of 3 timings of each part, attention
    also with one BLAS thread."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    cfg = inp.cfg
    scale = float(np.float32(1.0 / math.sqrt(cfg.d)))
    rej = "rejection" in cfg.accept

    def mask():
        return oracle.tree_mask_batch(inp.parent)[0]

    def attention(anc):
        return oracle.tree_attention_batch(inp.q, inp.k, inp.v, inp.prefix_len, anc, inp.layout,
                                           inp.block_table, cfg.block_size, scale)

    def accept():
        if rej:
            return oracle.rejection_batch(inp.logits, inp.tokens, inp.parent, inp.tau, inp.uniforms)
        return oracle.greedy_batch(inp.logits, inp.tokens, inp.parent)

    def compact(r):
        return oracle.kv_compact(inp.k, inp.v, inp.prefix_len, r[1], r[0], inp.layout,
                                 inp.block_table, cfg.block_size)

    steps = 0
    t0 = time.perf_counter()
    while True:
        anc = mask()
        attention(anc)
        r = accept()
        compact(r)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break

    def med(fn, *a):
        ts = []
        for _ in range(3):
            t = time.perf_counter()
            out = fn(*a)
            ts.append(time.perf_counter() - t)
        return statistics.median(ts), out

    t_mask, anc = med(mask)
    t_attn, _ = med(attention, anc)
    with threadpool_limits(limits=1):
        t_attn1, _ = med(attention, anc)
    t_acc, r = med(accept)
    t_cmp, _ = med(compact, r)
    work = algorithmic_work(inp)
    model, blas = cpu_description()
    return {"value": cfg.B * cfg.T * steps / el, "unit": "tree-nodes/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{steps} full verification step(s) of the {cfg.name} workload (B={cfg.B}, "
                      f"T={cfg.T}): float64 mask + explicit-mask attention + "
                      f"{'rejection' if rej else 'greedy'} walk + compaction, "
                      f"{el:.1f} s on the host; then 3 timings of each part",
            "cpu_model": model, "blas": blas,
            "parts_s": {"mask": t_mask, "attention": t_attn, "attention_1_thread": t_attn1,
                        "accept": t_acc, "compact": t_cmp},
            "attention_nodes_per_s": cfg.B * cfg.T / t_attn,
            "attention_bytes_per_s": work["bytes"] / t_attn,
            "attention_bytes_per_s_1_thread": work["bytes"] / t_attn1}


def timed_rotation(step_fns, steps, warmup):
    """Wall time of exactly `steps` steps replayed from graphs (one per step function, plus
    one of a whole rotation), after `warmup` untimed steps."""
    graphs = [capture(f) for f in step_fns]
    rotation = capture(lambda: [f() for f in step_fns])

    def run(n):
        done = 0
        while n - done >= len(step_fns):
            rotation.replay()
            done += len(step_fns)
        for i in range(n - done):
            graphs[i].replay()

    run(warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def call_time_us(step_fns, reps=10):
    """Mean device time of one step from HIP events around a graph of about 32 steps."""
    n = len(step_fns) * max(1, math.ceil(32 / len(step_fns)))
    g = capture(lambda: [step_fns[i % len(step_fns)]() for i in range(n)])
    g.replay()
    torch.cuda.synchronize()
    keep = prime_gpu()
    pairs = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    del keep
    return statistics.fmean(a.elapsed_time(b) * 1e3 / n for a, b in pairs)


def bench_sampled(args, cfg):
    """Acceptance with sampled drafts (target and draft logit rows of every node)."""
    inp = generate(cfg, with_kv=False)
    draft, tokens = sampled_drafts(inp)
    mc = max(int((p == a).sum()) for p in inp.parent for a in range(cfg.T))
    to = lambda x, dt: torch.from_numpy(np.ascontiguousarray(x)).to("cuda", dt)
    tk, pa, un = to(tokens, torch.int32), to(inp.parent, torch.int32), to(inp.uniforms, torch.float64)
    per_set = 2 * inp.logits.nbytes
    n_sets = max(1, math.ceil(FOOTPRINT_BYTES / per_set))
    lg = [to(inp.logits, torch.float32) for _ in range(n_sets)]
    dr = [to(draft, torch.float32) for _ in range(n_sets)]
    B, T, V = cfg.B, cfg.T, cfg.V
    ws = torch.zeros(ev.ev_accept_sampled_workspace(B, T, V), dtype=torch.uint8, device="cuda")
    z = lambda *sh: torch.zeros(sh, dtype=torch.int32, device="cuda")
    acc, path, out, st = z(B), z(B, T), z(B, T), z(1)
    fns = [lambda i=i: ev.ev_accept_sampled(lg[i], dr[i], tk, pa, inp.tau, 0.8, un, mc, acc, path,
                                            out, ws, st) for i in range(n_sets)]
    fns[0]()
    torch.cuda.synchronize()
    if int(st.item()) != 0:
        raise ev.EvError(int(st.item()), "bench eager step")
    elapsed = timed_rotation(fns, args.steps, args.warmup)
    t_call = call_time_us(fns) * 1e-6
    useful = 8 * B * T * V                     # both logit rows of every node, read once
    achieved = useful / t_call / 1e9
    result = {
        "metric": "verified tree-nodes/s, acceptance with sampled drafts (target + draft logits)",
        "value": B * T * args.steps / elapsed, "unit": "tree-nodes/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": cfg.workload + ", sampled drafts", "B": B, "T": T, "V": V,
                   "tau": cfg.tau, "draft_tau": 0.8, "max_children": mc, "buffer_sets": n_sets},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": None,
                     "kernel": "ev_accept_sampled (statistics launch + rounds)",
                     "algorithmic_bytes": useful},
        "call_us": t_call * 1e6,
    }
    if not args.no_cpu_baseline:
        import oracle
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_budget:
            oracle.stochastic_batch(inp.logits, draft, tokens, inp.parent, inp.tau, 0.8, inp.uniforms)
            n += 1
        el = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": B * T * n / el, "unit": "tree-nodes/s", "cores": 1,
                                  "kind": "oracle",
                                  "sample": f"{n} full call(s) of the oracle's sampled-draft walk "
                                            f"(B={B}, T={T}, V={V}) in {el:.1f} s"}
    print(json.dumps(result), flush=True)


def bench_draft_tree(args, cfg, depths=6, beam=8, k_max=8, n_nodes=64):
    """Dynamic draft-tree construction: `depths` beam expansions over the drafter's logit
    rows (a synthetic stand-in) and the final rerank, for the configuration's batch and
    vocabulary."""
    B, V = cfg.B, cfg.V
    host = draft_tree_logits(B, V, depths=depths, beam=beam)
    per_set = sum(x.nbytes for x in host)
    n_sets = max(1, math.ceil(FOOTPRINT_BYTES / per_set))
    sets = [[torch.from_numpy(x).cuda() for x in host] for _ in range(n_sets)]
    ws = torch.zeros(ev.ev_draft_tree_workspace(B, beam, V), dtype=torch.uint8, device="cuda")
    z = lambda *sh: torch.zeros(sh, dtype=torch.int32, device="cuda")
    ft = [z(B, beam) for _ in range(depths)]
    fs = [z(B, beam) for _ in range(depths)]
    fc = [z(B) for _ in range(depths)]
    root, par, tok, size, st = z(B), z(B, n_nodes), z(B, n_nodes), z(B), z(1)

    def build(i):
        for d in range(depths):
            ev.ev_draft_tree_expand(sets[i][d], d, 1.0, k_max, ws, ft[d], fs[d], fc[d], st)
        ev.ev_draft_tree_finalize(root, beam, V, n_nodes, ws, par, tok, size)

    fns = [lambda i=i: build(i) for i in range(n_sets)]
    fns[0]()
    torch.cuda.synchronize()
    if int(st.item()) != 0:
        raise ev.EvError(int(st.item()), "bench eager tree")
    rows = sum(int(c.sum().item()) for c in fc[:-1]) + B     # live frontier rows, all depths
    elapsed = timed_rotation(fns, args.steps, args.warmup)
    t_call = call_time_us(fns) * 1e-6
    useful = 4 * V * rows                      # each live frontier row's logits, read once
    achieved = useful / t_call / 1e9
    result = {
        "metric": "draft trees/s (entropy-guided beam expansion + rerank to <= 64 nodes)",
        "value": B * args.steps / elapsed, "unit": "trees/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": f"draft-tree construction, {cfg.workload} batch and vocabulary",
                   "B": B, "V": V, "depths": depths, "beam": beam, "k_max": k_max,
                   "n_nodes": n_nodes, "frontier_rows": rows, "buffer_sets": n_sets,
                   "mean_tree_size": float(size.float().mean().item())},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": None,
                     "kernel": "ev_draft_tree_expand x depths + ev_draft_tree_finalize",
                     "algorithmic_bytes": useful},
        "tree_us": t_call * 1e6,
    }
    if not args.no_cpu_baseline:
        import oracle
        sample = [x[:1] for x in host]
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_budget:
            oracle.build_batch(sample, beam, k_max, 1.0, n_nodes, [0])
            n += 1
        el = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": n / el, "unit": "trees/s", "cores": 1, "kind": "oracle",
                                  "sample": f"{n} tree(s) of sequence 0 built by the oracle "
                                            f"({depths} depths, V={V}) in {el:.1f} s"}
    print(json.dumps(result), flush=True)


def bench_compact_remap(args, cfg, n_layers=80):
    """Pruning after acceptance on the configuration's batch with one-token pages across a
    whole model's layers: block-table remapping (ev_kv_compact_remap) against row copies
    (ev_kv_compact).  Each step first restores the block table (a device copy), so both
    variants do their full work every step; the restore alone is timed too."""
    rng = np.random.default_rng(11)
    B, T, bs = cfg.B, cfg.T, 1
    lo, hi = cfg.prefix_range()
    L = rng.integers(lo, hi + 1, size=B).astype(np.int32) if lo != hi else np.full(B, lo, np.int32)
    max_blocks = int(L.max()) + T
    n_blocks = int((L + T).sum())
    perm = rng.permutation(n_blocks).astype(np.int32)
    table = np.full((B, max_blocks), -1, np.int32)
    at = 0
    for b in range(B):
        n = int(L[b]) + T
        table[b, :n] = perm[at:at + n]
        at += n
    paths = np.full((B, T), -1, np.int32)
    acc = np.zeros(B, np.int32)
    for b in range(B):                          # 2..6 accepted nodes, as the gauges report
        kb = int(rng.integers(2, 7))
        paths[b, :kb + 1] = [0] + sorted(rng.choice(np.arange(1, T), size=kb, replace=False).tolist())
        acc[b] = kb
    shape = (n_layers, n_blocks, cfg.Hkv, bs, cfg.d)
    k = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    v = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    t0 = torch.from_numpy(table).cuda()
    td = t0.clone()
    kv = ev.KvCache(k, v, td, layered=True)
    c = lambda x: torch.from_numpy(x).cuda()
    Ld, pd, ad = c(L), c(paths), c(acc)
    z = lambda *sh: torch.zeros(sh, dtype=torch.int32, device="cuda")
    nl, fr, fc, cp, st = z(B), z(B, max_blocks), z(B), z(B), z(1)
    ws = torch.empty(ev.ev_kv_compact_remap_workspace(B), dtype=torch.uint8, device="cuda")

    def restore():
        td.copy_(t0)

    def remap():
        restore()
        ev.ev_kv_compact_remap(kv, Ld, pd, ad, nl, fr, fc, cp, ws, st)

    def copy():
        restore()
        ev.ev_kv_compact(kv, Ld, pd, ad, nl, st)

    remap()
    torch.cuda.synchronize()
    if int(st.item()) != 0:
        raise ev.EvError(int(st.item()), "bench eager remap")
    copied = int(cp.sum().item())
    elapsed = timed_rotation([remap], args.steps, args.warmup)
    t_remap, t_copy, t_restore = (call_time_us([f]) for f in (remap, copy, restore))
    row = cfg.d * 2
    moved = int(acc.sum()) * n_layers * cfg.Hkv * 2 * row * 2     # K and V, read + write
    table_bytes = 2 * 4 * int((L + T).sum() - L.sum())           # tree entries read + written
    achieved = table_bytes / ((t_remap - t_restore) * 1e-6) / 1e9
    result = {
        "metric": "pruned sequences/s, zero-copy block-table remapping (one-token pages, 80 layers)",
        "value": B * args.steps / elapsed, "unit": "sequences/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": f"pruning after acceptance, {cfg.workload} batch, one-token pages",
                   "B": B, "T": T, "n_layers": n_layers, "Hkv": cfg.Hkv, "d": cfg.d,
                   "accepted_nodes": int(acc.sum())},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": None,
                     "kernel": "ev_kv_compact_remap (plan + commit; no rows copied)",
                     "algorithmic_bytes": table_bytes},
        "remap_us": t_remap - t_restore, "copy_compaction_us": t_copy - t_restore,
        "table_restore_us": t_restore, "slots_copied_by_remap": copied,
        "bytes_moved_by_copy_compaction": moved,
    }
    print(json.dumps(result), flush=True)


def bench_int4(args, cfg):
    """Tree attention over an INT4-quantised KV cache (4-bit values, one float32 scale per
    row) against the bfloat16 cache of the same workload."""
    from synth import quantize_int4
    inp = generate(cfg, with_logits=False)
    kq, ks = quantize_int4(inp.k)
    vq, vs = quantize_int4(inp.v)
    c = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    per_set = kq.nbytes + vq.nbytes + ks.nbytes + vs.nbytes
    n_sets = max(1, math.ceil(FOOTPRINT_BYTES / per_set))
    bt = c(inp.block_table) if inp.block_table is not None else None
    caches = [ev.KvCache(c(kq), c(vq), bt, k_scale=c(ks), v_scale=c(vs)) for _ in range(n_sets)]
    dev = to_device(inp)
    bf_sets = max(1, math.ceil(FOOTPRINT_BYTES / (dev.k.numel() * 4)))
    bf = [ev.KvCache(dev.k.clone(), dev.v.clone(), dev.block_table) for _ in range(bf_sets)]
    q = dev.q
    anc, _ = ev.ev_tree_mask_build(dev.parent, check=True)
    scale = float(np.float32(1.0 / math.sqrt(cfg.d)))
    B, T, Hq = cfg.B, cfg.T, cfg.Hq
    out = torch.empty_like(q)
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    mpl = int(inp.prefix_len.max())
    ws = torch.zeros(max(1, ev.ev_tree_attention_workspace(caches[0], B, T, Hq, mpl)),
                     dtype=torch.uint8, device="cuda")
    wsb = torch.zeros(max(1, ev.ev_tree_attention_workspace(bf[0], B, T, Hq, mpl)),
                      dtype=torch.uint8, device="cuda")
    f4 = [lambda kv=kv: ev.ev_tree_attention(q, kv, dev.prefix_len, anc, scale, out, lse, ws, st,
                                             max_prefix_len=mpl) for kv in caches]
    fb = [lambda kv=kv: ev.ev_tree_attention(q, kv, dev.prefix_len, anc, scale, out, lse, wsb, st,
                                             max_prefix_len=mpl) for kv in bf]
    f4[0]()
    torch.cuda.synchronize()
    if int(st.item()) != 0:
        raise ev.EvError(int(st.item()), "bench eager int4 attention")
    elapsed = timed_rotation(f4, args.steps, args.warmup)
    t4, tb = call_time_us(f4) * 1e-6, call_time_us(fb) * 1e-6
    work = algorithmic_work(inp)
    L = inp.prefix_len.astype(np.int64)
    rows = int(sum(cfg.Hkv * (L[b] + T) for b in range(B)))
    kv4 = 2 * rows * (cfg.d // 2 + 4)                    # packed values + scales, K and V
    useful = kv4 + work["bytes"] - work["kv_bytes"]      # plus Q, O and LSE
    achieved = useful / t4 / 1e9
    result = {
        "metric": "verified tree-nodes/s, tree attention over an INT4 KV cache",
        "value": B * T * args.steps / elapsed, "unit": "tree-nodes/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int4 KV, bf16 Q/O", "data": "synthetic",
        "config": {"workload": cfg.workload + ", INT4 cache", "B": B, "Hq": Hq, "Hkv": cfg.Hkv,
                   "d": cfg.d, "L": cfg.L, "T": T, "kv_layout": inp.layout, "buffer_sets": n_sets},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": None,
                     "kernel": "ev_tree_attention (INT4 cache; register-staged)",
                     "algorithmic_bytes": useful},
        "attention_int4_us": t4 * 1e6, "attention_bf16_us": tb * 1e6,
        "kv_bytes_int4": kv4, "kv_bytes_bf16": work["kv_bytes"],
        "attention_tflops_int4": work["flops"] / t4 / 1e12,
    }
    print(json.dumps(result), flush=True)


MAX_SETS = 64                      # buffer sets of a tiny workload (launch-bound anyway)
ROOF_RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)   # flop per byte


def build_sets(inp):
    """Buffer sets of one workload: enough copies that the rotation touches >= 512 MB."""
    cfg = inp.cfg
    dev0 = to_device(inp)
    per_set = sum(t.numel() * t.element_size() for t in (dev0.q, dev0.k, dev0.v, dev0.logits))
    n_sets = min(MAX_SETS, max(1, math.ceil(FOOTPRINT_BYTES / per_set)))
    kv_tmp = ev.KvCache(dev0.k, dev0.v, dev0.block_table)
    mpl = int(inp.prefix_len.max())
    ws_attn = torch.empty(max(1, ev.ev_tree_attention_workspace(kv_tmp, cfg.B, cfg.T, cfg.Hq, mpl)),
                          dtype=torch.uint8, device="cuda")
    ws_acc = torch.zeros(max(1, ev.ev_accept_workspace(cfg.B, cfg.T, cfg.V)), dtype=torch.uint8,
                         device="cuda")
    return [BufferSet(inp, dev0 if i == 0 else to_device(inp), ws_attn, ws_acc)
            for i in range(n_sets)]


def rooflines(inp, kt):
    """Rates and roofline fractions of one workload's attention call and step."""
    cfg = inp.cfg
    work = algorithmic_work(inp)
    t_attn = kt[ATTN_PART]["mean_us"] * 1e-6
    t_acc = kt["accept"]["mean_us"] * 1e-6
    tflops = work["flops"] / t_attn / 1e12
    gbps = work["bytes"] / t_attn / 1e9
    if cfg.dtype == "f32":
        bound, frac = "latency", None
    elif work["flops"] / work["bytes"] > ROOF_RIDGE:
        bound, frac = "mfma", tflops / PEAK_BF16_TFLOPS
    else:
        bound, frac = "hbm", gbps / PEAK_HBM_GBPS
    return {"workload": cfg.workload, "kv_layout": inp.layout,
            "acceptance": "rejection" if "rejection" in cfg.accept else "greedy",
            "kernels_us": {k: round(v["mean_us"], 3) for k, v in kt.items()},
            "step_us": round(sum(kt[k]["mean_us"] for k in STEP_PARTS), 3),
            "tree_nodes_per_s_step": cfg.B * cfg.T / (sum(kt[k]["mean_us"] for k in STEP_PARTS) * 1e-6),
            "attention_tree_nodes_per_s": cfg.B * cfg.T / t_attn,
            "attention_tflops": tflops, "attention_mfma_frac": tflops / PEAK_BF16_TFLOPS,
            "attention_gbps": gbps, "attention_hbm_frac": gbps / PEAK_HBM_GBPS,
            "attention_bound": bound, "attention_frac_of_bound": frac,
            "algorithmic_flops": work["flops"], "algorithmic_bytes": work["bytes"],
            "accept_logit_gbps": work["logit_bytes"] / t_acc / 1e9,
            "accept_hbm_frac": work["logit_bytes"] / t_acc / 1e9 / PEAK_HBM_GBPS}


def config_entry(cfg, reps):
    """Per-call times of every part of the step for one workload (parity configs)."""
    inp = generate(cfg)
    sets = build_sets(inp)
    sets[0].step()
    torch.cuda.synchronize()
    if int(sets[0].status.item()) != 0:
        raise ev.EvError(int(sets[0].status.item()), f"bench eager step ({cfg.name})")
    e = rooflines(inp, kernel_times(sets, reps))
    e["buffer_sets"] = len(sets)
    del sets
    torch.cuda.empty_cache()
    return e


def capacity_entry(inp, sets, caps):
    """Attention per call over caches sized for longer contexts (same contents, NaN beyond),
    split plan from the real longest prefix: the time should not depend on the capacity."""
    cfg = inp.cfg
    out = {}
    for cap in caps:
        kvs = []
        for st in sets:
            k = torch.full((cfg.B, cfg.Hkv, cap, cfg.d), float("nan"), dtype=torch.bfloat16,
                           device="cuda")
            v = torch.full_like(k, float("nan"))
            k[:, :, :inp.cap] = st.d.k
            v[:, :, :inp.cap] = st.d.v
            kvs.append(ev.KvCache(k, v))
        mpl = int(inp.prefix_len.max())
        ws = torch.empty(max(1, ev.ev_tree_attention_workspace(kvs[0], cfg.B, cfg.T, cfg.Hq, mpl)),
                         dtype=torch.uint8, device="cuda")

        def call(i, kv):
            st = sets[i]
            ev.ev_tree_attention(st.d.q, kv, st.d.prefix_len, st.anc, st.scale, st.out, st.lse, ws,
                                 st.status, max_prefix_len=mpl)

        fns = [lambda i=i, kv=kv: call(i, kv) for i, kv in enumerate(kvs)]
        out[str(cap)] = round(call_time_us(fns), 3)
        del kvs, ws
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="llama3_70b_layer")
    ap.add_argument("--path", default="verify",
                    choices=("verify", "sampled", "draft_tree", "compact_remap", "int4"),
                    help="verify: the verification step (default); sampled: acceptance with "
                         "sampled drafts; draft_tree: dynamic draft-tree construction; "
                         "compact_remap: zero-copy pruning against row copies; int4: "
                         "attention over an INT4 cache against the bf16 cache")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-call timings of the other workloads and cache capacities")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the attention traffic record from two rocprofv3 --pmc "
                         "counter files (FETCH_SIZE, WRITE_SIZE) and exit (no GPU needed)")
    ap.add_argument("--traffic-command", default="", help="command recorded with --traffic-from")
    ap.add_argument("--traffic-part", default="attention", choices=tuple(TRAFFIC_PARTS),
                    help="which part of the step the --traffic-from record covers")
    ap.add_argument("--no-box-peaks", action="store_true",
                    help="skip the calibration kernels (counter runs)")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic(*args.traffic_from, args.traffic_command, args.traffic_part, args.config)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the per-GPU share of a sharded verification is the single-GPU workload).",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    ev.lib()
    cfg = config_by_name(args.config)
    if args.path == "sampled":
        return bench_sampled(args, cfg)
    if args.path == "draft_tree":
        return bench_draft_tree(args, cfg)
    if args.path == "compact_remap":
        return bench_compact_remap(args, cfg)
    if args.path == "int4":
        return bench_int4(args, cfg)
    inp = generate(cfg)
    sets = build_sets(inp)
    n_sets = len(sets)
    mode = sets[0].mode
    if args.calibrate:          # counter runs profile the main workload's kernels only
        args.no_configs = True

    # eager reference of the acceptance result, then capture
    sets[0].step()
    torch.cuda.synchronize()
    if int(sets[0].status.item()) != 0:
        raise ev.EvError(int(sets[0].status.item()), "bench eager step")
    ref = (sets[0].acc.clone(), sets[0].path.clone(), sets[0].tok.clone())
    # One graph per buffer set (one step each) and one graph of a whole rotation (one step
    # per set, in order), so that graph launch is paid once per rotation, not per step.
    graphs = [capture(s.step) for s in sets]
    rotation = capture(lambda: [s.step() for s in sets])
    for g in (graphs[0], rotation, graphs[0], rotation):  # replays agree with the eager run
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (sets[0].acc, sets[0].path, sets[0].tok)):
            if not torch.equal(a, b):
                raise RuntimeError("graph replay disagrees with the eager step")

    def run_steps(n):
        """Exactly n steps: whole rotations, then single steps."""
        done = 0
        while n - done >= n_sets:
            rotation.replay()
            done += n_sets
        for i in range(n - done):
            graphs[i].replay()

    run_steps(args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(args.steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if any(int(s.status.item()) != 0 for s in sets):
        raise RuntimeError("device status reported an error during the timed steps")

    if args.calibrate:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    kt = kernel_times(sets, 10)
    work = algorithmic_work(inp)
    t_attn = kt[ATTN_PART]["mean_us"] * 1e-6
    ms_per_step = elapsed * 1e3 / args.steps
    nodes = cfg.B * cfg.T
    if cfg.dtype == "bf16":
        bound, peak, unit = "mfma", PEAK_BF16_TFLOPS, "TFLOP/s"
        achieved = work["flops"] / t_attn / 1e12
    else:
        bound, peak, unit = "alu", PEAK_F32_TFLOPS, "TFLOP/s"
        achieved = work["flops"] / t_attn / 1e12
    kv_gbps = work["bytes"] / t_attn / 1e9
    this = rooflines(inp, kt)
    this["buffer_sets"] = n_sets
    capacity = (capacity_entry(inp, sets, (32848, 131152))
                if not inp.cfg.paged and cfg.B == 1 and not args.no_configs else None)
    del sets, graphs, rotation
    torch.cuda.empty_cache()
    configs = {}
    if not args.no_configs:
        for c in CONFIGS:
            configs[c.name] = this if c.name == cfg.name else config_entry(c, 5)
    box = None if args.no_box_peaks else box_peaks()
    result = {
        "metric": METRIC,
        "value": nodes / (ms_per_step * 1e-3),
        "unit": "tree-nodes/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.workload, "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "d": cfg.d,
                   "L": cfg.L, "T": cfg.T, "V": cfg.V, "kv_layout": inp.layout,
                   "acceptance": mode, "tau": cfg.tau, "buffer_sets": n_sets},
        "roofline": {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": traffic_entry(cfg.name),
                     "kernel": "ev_tree_mask_attention", "algorithmic_flops": work["flops"],
                     "algorithmic_bytes": work["bytes"],
                     "frac_of_box_peak": (achieved / (box["mfma_bf16_tflops"] if bound == "mfma"
                                                      else peak)) if box else None},
        "kv_hbm_gbps": kv_gbps,
        "kv_hbm_frac": kv_gbps / PEAK_HBM_GBPS,
        "kv_hbm_frac_of_box_read": kv_gbps / box["read_gbps"] if box else None,
        "box_peaks": box,
        "attention_nodes_per_s": nodes / t_attn,
        "kernels_us": {k: round(v["mean_us"], 3) for k, v in kt.items()},
        "kernels_us_p10_p90": {k: [round(v["p10_us"], 3), round(v["p90_us"], 3)] for k, v in kt.items()},
        "accept_len": int(ref[0].float().mean().item()),
        "tokens_per_step": float(ref[0].float().mean().item()) + 1.0,
        "attention_us_by_cache_capacity": (dict({str(inp.cap): round(kt["attention"]["mean_us"], 3)},
                                                **capacity) if capacity else None),
        "configs": configs or None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
