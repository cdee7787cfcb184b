"""Decode-step throughput of the QSA select + sparse-attention path on one
MI355X.

Workloads (``--workload``):

* long_context (default): the long-context decode batch -- R=128 query rows,
  each of a 131072-token request (32768 compressed blocks), a 32768-page
  fp16 N(0,1) compressed-key cache (1 GiB) behind random permuted block
  tables, and full-width [128,2051] sparse attention over a 131072-token
  packed fp16 KV cache (128 MiB).
* long_context_fp8: the long-context batch with its compressed keys
  absmax-quantized to an e4m3 cache (128 B of codes + one fp32 scale per
  key, 528 MiB), timed through qsa_decode_step_fp8.
* long_context_two_pass: the long-context batch with per-head weights
  (uniform in [-0.5, 1.5]), selected in two passes -- qsa_paged_logits
  writes the [128, 32768] fp32 logits matrix, qsa_topk_per_row reduces it --
  then attention; the fused weighted selection (qsa_select_weighted) is
  timed on the same inputs for comparison.
* multi_token_metadata: the multi_token batch with its per-row request ids
  and positions built on the device each step by qsa_build_metadata (from
  the cumulative query starts and sequence lengths, k work items included)
  and fed to qsa_decode_step with no host synchronisation.
* multi_token: several query rows per request -- 48 speculative-decode
  requests with 4 draft positions each and 4 chunked-prefill requests with
  16 positions each (R=256), lengths uniform in [8192, 65536], an 8192-page
  N(0,1) compressed-key cache (256 MiB).  The selection queries go in as
  runs of 4 rows ([64, 4, 4, 128], --rows-per-run), so each run's keys are
  read once; the row-by-row selection is timed beside it.

Inputs are seeded synthetic data, resident in HBM before timing starts.

One step = one qsa_decode_step call (selection then attention on one
stream, no host sync); K steps (200 by default) are timed with HIP events at
both ends.  The
steps rotate over distinct KV caches, as consecutive layers would.  A second
pass runs the two stages through qsa_select and qsa_sparse_attn with events
between them for the per-stage times and the roofline.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "select+sparse-attn decode rows/sec and achieved HBM GB/s (% of peak), 1 GPU"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
KERNEL_SOURCES = [os.path.join(ROOT, "paged_top_indexer_amd", "csrc", f)
                  for f in ("qsa_select.hip", "qsa_device.h", "qsa_launch.h", "qsa_select_plan.cpp")]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def select_algorithmic_bytes(seq_lens, query_pos, token_to_req, key_bytes: int = 256) -> int:
    """Bytes the selection must move per launch.  Per request, its compressed
    keys once (key_bytes per block visible to its furthest row: 256 for fp16
    keys, 132 for e4m3 codes + scale) and the 4 B block-table entries that
    map them: rows of one request read the same pages.  Per row, the 1 KiB
    query, 16 B of row metadata and the 8204 B output row."""
    furthest = {}
    total = 0
    for r in range(len(token_to_req)):
        req = int(token_to_req[r])
        L = int(seq_lens[req])
        qp = int(query_pos[r])
        v = max(0, min((qp + 1) // 4, L // 4))
        furthest[req] = max(furthest.get(req, 0), v)
        total += 1024 + 16 + 8204
    for v in furthest.values():
        total += key_bytes * v + 4 * (-(-v // 128))
    return total


def logits_algorithmic_bytes(seq_lens, query_pos, token_to_req, width: int) -> int:
    """Bytes the paged-logits pass must move per launch: the keys and
    table entries as for the selection, per row the 1 KiB query, 16 B of
    weights, 16 B of row metadata and its 4 B x width logits row."""
    furthest = {}
    total = 0
    for r in range(len(token_to_req)):
        req = int(token_to_req[r])
        L = int(seq_lens[req])
        qp = int(query_pos[r])
        v = max(0, min((qp + 1) // 4, L // 4))
        furthest[req] = max(furthest.get(req, 0), v)
        total += 1024 + 16 + 16 + 4 * width
    for v in furthest.values():
        total += 256 * v + 4 * (-(-v // 128))
    return total


def attn_algorithmic_bytes(indices: np.ndarray) -> int:
    """Per row: 1 KiB per distinct valid token (K and V halves), the 8204 B
    index row, the 1.5 KiB query and the 1.5 KiB output."""
    total = 0
    for row in indices:
        total += 1024 * len(np.unique(row[row >= 0])) + 8204 + 1536 + 1536
    return total


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str):
    """HBM bytes per select launch from the committed counter summary of this
    workload (profiles/select_<workload>_counters.json), if it was taken on
    the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"select_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash() or rec.get("workload") != workload:
        return None
    return rec.get("hbm_bytes_per_launch")


def read_ceiling(torch, qsa, dev, gib: int = 2, reps: int = 5) -> float:
    """The box's practical HBM read ceiling (GB/s): qsa_read_probe streaming
    `gib` GiB with nontemporal loads, `reps` times between HIP events."""
    buf = torch.empty(gib << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    qsa.qsa_read_probe(buf, sink)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    stream = torch.cuda.current_stream(dev)
    ev[0].record(stream)
    for _ in range(reps):
        qsa.qsa_read_probe(buf, sink)
    ev[1].record(stream)
    torch.cuda.synchronize()
    gbs = (gib << 30) * reps / (ev[0].elapsed_time(ev[1]) / 1e3) / 1e9
    del buf
    return gbs


def r1_latencies(torch, qsa, wl, dev, calls: int = 64) -> dict:
    """Mean single-row latencies of the pages' own cases (their figures are
    for an Intel XPU; context only): selection of the 519-token row (129
    blocks) and of the saturated 9215-token row (2303 blocks), and
    attention over the saturated row's 2051 indices.  `*_ms`: calls back to
    back from Python (host marshalling and launch included); `graph_*_ms`:
    the same calls captured once in a HIP graph and replayed (device time
    per call; the replayed outputs are checked against the eager ones)."""
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    stream = torch.cuda.current_stream(dev)

    def mean_ms(fn):
        for _ in range(5):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(calls):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / calls

    def graph_ms(fn, result):
        fn()
        torch.cuda.synchronize()
        eager = result.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(calls):
                fn()
        result.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(result, eager), "graph replay differs from the eager call"
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        g.replay()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / calls

    out = {}
    tiny_w = wl.tiny_integer(0)
    tiny = [d(a) for a in tiny_w.select_inputs()]
    idx1 = torch.empty((1, 2051), dtype=torch.int32, device=dev)
    ws_t = torch.zeros(max(1, qsa.select_workspace_bytes(1, tiny_w.block_table.shape[1])),
                       dtype=torch.uint8, device=dev)
    sel_tiny = lambda: qsa.qsa_select(*tiny, out=idx1, workspace=ws_t)  # noqa: E731
    out["select_519_tokens_ms"] = round(mean_ms(sel_tiny), 5)
    out["graph_select_519_tokens_ms"] = round(graph_ms(sel_tiny, idx1), 5)
    sat = wl.saturated_row(0)
    satd = [d(a) for a in sat.select_inputs()]
    ws_s = torch.zeros(max(1, qsa.select_workspace_bytes(1, sat.block_table.shape[1])),
                       dtype=torch.uint8, device=dev)
    sel_sat = lambda: qsa.qsa_select(*satd, out=idx1, workspace=ws_s)  # noqa: E731
    out["select_2303_blocks_ms"] = round(mean_ms(sel_sat), 5)
    out["graph_select_2303_blocks_ms"] = round(graph_ms(sel_sat, idx1), 5)
    kvd = d(sat.kv)
    k, v = qsa.kv_views(kvd)
    q = d(sat.q_attn)
    sel_sat()
    o = torch.empty((1, 3, 256), dtype=torch.float16, device=dev)
    ws_a = torch.zeros(max(1, qsa.sparse_attn_workspace_bytes(1)), dtype=torch.uint8, device=dev)
    attn = lambda: qsa.qsa_sparse_attn(q, k, v, idx1, wl.SOFTMAX_SCALE, out=o,  # noqa: E731
                                       workspace=ws_a)
    out["attention_width_2051_ms"] = round(mean_ms(attn), 5)
    out["graph_attention_width_2051_ms"] = round(graph_ms(attn, o), 5)
    out["pages_intel_xpu_ms"] = {"select_519_tokens": 0.053155, "select_2303_blocks": 0.319464,
                                 "attention_width_2051": 0.710274}
    return out


def units_protocol(torch, stream, decode_call, attn_call, warmup_units: int = 5,
                   samples: int = 10) -> dict:
    """The pages' own timing protocol: warmup_units excluded units, then
    `samples` timed units of 64 decode-step calls and of 128 attention calls
    (events around each unit); mean, median and min of the per-call time."""
    def stats(call, per_unit):
        for u in range(warmup_units):
            for i in range(per_unit):
                call(u * per_unit + i)
        times = []
        for u in range(samples):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            for i in range(per_unit):
                call(u * per_unit + i)
            ev[1].record(stream)
            torch.cuda.synchronize()
            times.append(ev[0].elapsed_time(ev[1]) / per_unit)
        return {"mean": round(float(np.mean(times)), 4), "median": round(float(np.median(times)), 4),
                "min": round(float(np.min(times)), 4)}

    return {"warmup_units": warmup_units, "samples": samples,
            "decode_step_ms_per_call": {"calls_per_unit": 64, **stats(decode_call, 64)},
            "attention_ms_per_call": {"calls_per_unit": 128, **stats(attn_call, 128)}}


def batched_step(torch, qsa, wl, dev, steps: int = 20) -> dict:
    """The batched configuration (64 rows, lengths uniform in [512, 32768],
    requests 2i and 2i+1 sharing their first pages): mean decode-step time
    and the selection stage's algorithmic rate; context only."""
    w = wl.batched_shared(0)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    sel = [d(a) for a in w.select_inputs()]
    kvd = d(w.kv)
    k, v = qsa.kv_views(kvd)
    q = d(w.q_attn)
    idx = torch.empty((w.rows, 2051), dtype=torch.int32, device=dev)
    out = torch.empty((w.rows, 3, 256), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def mean_ms(fn):
        for _ in range(5):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(steps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / steps

    step = mean_ms(lambda: qsa.qsa_decode_step(*sel, q, k, v, wl.SOFTMAX_SCALE, indices=idx,
                                               out=out))
    select = mean_ms(lambda: qsa.qsa_select(*sel, out=idx))
    sel_bytes = select_algorithmic_bytes(w.seq_lens, w.query_pos, w.token_to_req)
    return {"workload": w.name, "rows": int(w.rows), "step_ms": round(step, 4),
            "rows_per_s": round(w.rows / step * 1e3, 1), "select_ms": round(select, 4),
            "select_algorithmic_gbs": round(sel_bytes / select / 1e6, 1)}


def host_cpu() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    """The CPU threads this process may run on, at most 16 (the host share of
    one GPU on a shared node, whatever the machine's own count)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(w, scale: float, fp8: bool = False, weights=None,
                 max_seconds: float = 20.0, threaded_seconds: float = 8.0) -> dict:
    """The CPU oracle (plain C, unmodified) on the host cores: the whole decode
    step of the first rows of the same workload, single-threaded until all
    rows are done or max_seconds of work have been spent; then the same
    per-row calls with the rows dealt to host_threads() threads (the C calls
    release the interpreter lock and keep no shared state) for about
    threaded_seconds, cycling over the rows."""
    import itertools
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    orc = oracle.default()
    q, kc, bt, t2r, sl, qp = w.select_inputs()

    def one_row(i: int):
        r = np.array([i])
        if fp8:
            sel = orc.select_fp8(q[r], w.kcodes, w.kscale, bt, t2r[r], sl, qp[r])
        elif weights is not None:
            lg = orc.paged_logits(q[r], weights[r], bt, t2r[r], sl, qp[r], bt.shape[1] * 128,
                                  kcache=kc)
            sel = orc.topk_per_row(lg, t2r[r], sl, qp[r])
        else:
            sel = orc.select(q[r], kc, bt, t2r[r], sl, qp[r])
        return sel, orc.sparse_attn(w.q_attn[r], w.kv, sel, scale)

    done = 0
    t0 = time.perf_counter()
    outs = []
    while done < w.rows and time.perf_counter() - t0 < max_seconds:
        outs.append(one_row(done))
        done += 1
    dt = time.perf_counter() - t0

    threads = host_threads()
    ticket = itertools.count()  # next() on a count is atomic under the interpreter lock
    t1 = time.perf_counter()
    stop = t1 + threaded_seconds

    def worker(_):
        n = 0
        while time.perf_counter() < stop:
            one_row(next(ticket) % w.rows)
            n += 1
        return n

    with ThreadPoolExecutor(threads) as ex:
        done_t = sum(ex.map(worker, range(threads)))
    dt_t = time.perf_counter() - t1
    return {"value": done / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"first {done} of {w.rows} rows of the same workload, select + attention "
                      f"per row, {dt:.1f} s single-threaded",
            "host_cpu": host_cpu(), "host_threads": threads,
            "threaded": {"value": done_t / dt_t, "unit": "rows/s", "cores": threads,
                         "sample": f"{done_t} rows (row i mod {w.rows}) dealt to {threads} "
                                   f"threads, {dt_t:.1f} s"},
            "_outs": outs}


def gpu_clocks():
    """GPU clocks and power as rocm-smi reports them right after the timed
    region (None if it cannot be read); the bench does not pin clocks."""
    import subprocess

    try:
        p = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--json"],
                           capture_output=True, text=True, timeout=30)
        rec = json.loads(p.stdout)
    except (OSError, subprocess.SubprocessError, ValueError):
        return None
    if not isinstance(rec, dict):
        return None
    keep = {}
    for card, fields in rec.items():
        if isinstance(fields, dict):
            keep[card] = {k: v for k, v in fields.items()
                          if any(t in k.lower() for t in ("sclk", "mclk", "fclk", "power"))}
    return keep or None


def workload_config(w, kv_copies: int) -> dict:
    lens = w.seq_lens[w.token_to_req].astype(np.int64)
    cfg = {"workload": w.name, "rows": int(w.rows), "requests": int(len(np.unique(w.token_to_req))),
           "cache_pages": int(w.kcache.shape[0]), "kv_tokens": int(w.kv.shape[0] * w.kv.shape[1]),
           "top_blocks": 512, "index_width": 2051, "kv_caches_rotated": kv_copies}
    if np.all(lens == lens[0]):
        cfg["seq_len"] = int(lens[0])
    else:
        cfg["seq_len_range"] = [int(lens.min()), int(lens.max())]
    return cfg


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 200 by default: a timed region carries a fixed ~0.14 ms start cost
    # (measured: 0.2382 / 0.2340 / 0.2321 ms per step at K = 20 / 64 / 200),
    # which a short region would spread over its few steps
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the read-ceiling probe and the single-row latencies")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", choices=["long_context", "long_context_fp8",
                                           "long_context_two_pass", "multi_token",
                                           "multi_token_metadata"],
                    default="long_context")
    ap.add_argument("--rows-per-run", type=int, default=0,
                    help="pass the selection queries as [R/n, n, 4, 128] (runs of n rows of "
                         "one request); default 4 for the multi_token workloads, else 1")
    ap.add_argument("--kv-copies", type=int, default=8,
                    help="distinct KV caches the steps rotate over (one per simulated layer)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the bench, run a plain device copy of MIB MiB three "
                         "times (reference for the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(rows shard across GPUs with no exchange; see the design notes)", file=sys.stderr)
        return 2

    import torch
    import paged_top_indexer_amd as qsa
    from paged_top_indexer_amd import workloads as wl

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 2, dtype=torch.float16, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)  # one elementwise kernel: reads n bytes, writes n bytes
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))
        return 0

    t0 = time.perf_counter()
    fp8 = args.workload == "long_context_fp8"
    two_pass = args.workload == "long_context_two_pass"
    meta = args.workload == "multi_token_metadata"
    head_w = None
    if args.workload in ("multi_token", "multi_token_metadata"):
        w = wl.multi_token_rows(args.seed)
        if meta:
            w.name = w.name + "_metadata"
    else:
        w = wl.long_context(args.seed)
        if fp8:
            w = wl.with_fp8_keys(w, integer=False)
        if two_pass:
            head_w = wl.head_weights(np.random.default_rng(args.seed + 555), w.rows)
            w.name = w.name + "_two_pass"
    log(f"generated {w.name} in {time.perf_counter() - t0:.1f} s")
    dev = torch.device("cuda:0")
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    if fp8:
        sel_in = [d(a) for a in w.select_inputs_fp8()]
        sel_in[1] = sel_in[1].view(torch.float8_e4m3fn)
        select_fn, decode_fn = qsa.qsa_select_fp8, qsa.qsa_decode_step_fp8
    else:
        sel_in = [d(a) for a in w.select_inputs()]
        select_fn, decode_fn = qsa.qsa_select, qsa.qsa_decode_step
    multi = args.workload in ("multi_token", "multi_token_metadata")
    run = args.rows_per_run or (4 if multi else 1)
    q_rows = sel_in[0]
    if run > 1:
        assert w.rows % run == 0, "rows must split into whole runs"
        sel_in[0] = q_rows.view(w.rows // run, run, 4, 128)
    # Consecutive decode steps of a model read different layers' caches.  The
    # steps here rotate over distinct KV caches (8 x 128 MiB by default, four
    # times the 256 MB Infinity Cache) so that no step finds its KV in the
    # last-level cache because an earlier step read it.
    kv_sets = [d(w.kv)]
    for i in range(1, args.kv_copies):
        kv_sets.append(d(wl.normal_f16(np.random.default_rng(args.seed + 1000 + i), w.kv.shape)))
    kv_views = [qsa.kv_views(t) for t in kv_sets]
    q_attn = d(w.q_attn)
    R = w.rows
    idx = torch.empty((R, 2051), dtype=torch.int32, device=dev)
    out = torch.empty((R, 3, 256), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream(dev)
    sel_ws = torch.zeros(max(1, qsa.select_workspace_bytes(R, w.block_table.shape[1])),
                         dtype=torch.uint8, device=dev)
    att_ws = torch.zeros(max(1, qsa.sparse_attn_workspace_bytes(R)), dtype=torch.uint8, device=dev)
    scale = wl.SOFTMAX_SCALE
    torch.cuda.synchronize()

    ws_all = torch.zeros(max(1, qsa.decode_step_workspace_bytes(R, w.block_table.shape[1])),
                         dtype=torch.uint8, device=dev)

    if meta:
        # the per-row request ids and positions come from the builder
        qsl = d(wl.query_start_loc(w))
        meta_ws = torch.zeros(max(1, qsa.build_metadata_workspace_bytes(len(w.seq_lens))),
                              dtype=torch.uint8, device=dev)
        meta_out = qsa.qsa_build_metadata(qsl, sel_in[4], sel_in[2], R, max_num_work=R,
                                          workspace=meta_ws)
        built_in = [sel_in[0], sel_in[1], sel_in[2], meta_out["token_to_req"], sel_in[4],
                    meta_out["logical_positions"]]

        def build_metadata():
            qsa.qsa_build_metadata(qsl, sel_in[4], sel_in[2], R, max_num_work=R, out=meta_out,
                                   workspace=meta_ws)

        def select_stage(mark=None):
            build_metadata()
            if mark is not None:
                mark.record(stream)
            select_fn(*built_in, out=idx, workspace=sel_ws)

        def step(i):
            k, v = kv_views[i % len(kv_views)]
            build_metadata()
            decode_fn(*built_in, q_attn, k, v, scale, indices=idx, out=out, workspace=ws_all)
    elif two_pass:
        wt = d(head_w)
        logits_width = w.block_table.shape[1] * 128
        logits = torch.empty((R, logits_width), dtype=torch.float32, device=dev)
        topk_ws = torch.zeros(max(1, qsa.topk_per_row_workspace_bytes(R, logits_width)),
                              dtype=torch.uint8, device=dev)

        def select_stage(mark=None):
            qsa.qsa_paged_logits(*sel_in, weights=wt, logits=logits)
            if mark is not None:
                mark.record(stream)
            qsa.qsa_topk_per_row(logits, sel_in[3], sel_in[4], sel_in[5], out=idx,
                                 workspace=topk_ws)

        def step(i):
            k, v = kv_views[i % len(kv_views)]
            select_stage()
            qsa.qsa_sparse_attn(q_attn, k, v, idx, scale, out=out, workspace=att_ws)
    else:
        def select_stage(mark=None):
            select_fn(*sel_in, out=idx, workspace=sel_ws)

        def step(i):
            k, v = kv_views[i % len(kv_views)]
            decode_fn(*sel_in, q_attn, k, v, scale, indices=idx, out=out, workspace=ws_all)

    # warm-up, then exactly K timed decode steps (events only at the ends)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t_start = time.perf_counter()
    t_ev[0].record(stream)
    for i in range(args.steps):
        step(i)
    t_ev[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = t_ev[0].elapsed_time(t_ev[1]) / args.steps
    clocks = None if args.no_context else gpu_clocks()

    # Per-stage times for the roofline: the same two stages through their own
    # entry points, with events recorded on the launch stream around each.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        k, v = kv_views[i % len(kv_views)]
        events[i][0].record(stream)
        select_stage(mark=events[i][3] if (two_pass or meta) else None)
        events[i][1].record(stream)
        qsa.qsa_sparse_attn(q_attn, k, v, idx, scale, out=out, workspace=att_ws)
        events[i][2].record(stream)
    torch.cuda.synchronize()
    sel_ms = [e[0].elapsed_time(e[1]) for e in events]
    att_ms = [e[1].elapsed_time(e[2]) for e in events]
    extra = {}
    if meta:
        meta_ms = [e[0].elapsed_time(e[3]) for e in events]
        sel_only_ms = [e[3].elapsed_time(e[1]) for e in events]
        extra = {"metadata_ms": round(float(np.mean(meta_ms)), 4),
                 "select_only_ms": round(float(np.mean(sel_only_ms)), 4)}
        log(f"metadata build {extra['metadata_ms']:.4f} ms, select {extra['select_only_ms']:.4f} ms")
    if two_pass:
        logits_ms = [e[0].elapsed_time(e[3]) for e in events]
        topk_ms = [e[3].elapsed_time(e[1]) for e in events]
        # the fused weighted selection on the same inputs, for comparison
        fused_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        fused_idx = torch.empty_like(idx)
        qsa.qsa_select_weighted(sel_in[0], wt, *sel_in[1:], out=fused_idx, workspace=sel_ws)
        fused_ev[0].record(stream)
        for _ in range(args.steps):
            qsa.qsa_select_weighted(sel_in[0], wt, *sel_in[1:], out=fused_idx, workspace=sel_ws)
        fused_ev[1].record(stream)
        torch.cuda.synchronize()
        extra = {"logits_ms": round(float(np.mean(logits_ms)), 4),
                 "topk_ms": round(float(np.mean(topk_ms)), 4),
                 "fused_weighted_select_ms": round(fused_ev[0].elapsed_time(fused_ev[1]) / args.steps, 4)}
        log(f"two-pass: logits {extra['logits_ms']:.4f} ms + top-k {extra['topk_ms']:.4f} ms; "
            f"fused weighted select {extra['fused_weighted_select_ms']:.4f} ms")
    if run > 1 and not meta:
        # the same selection with the queries passed row by row, for comparison
        flat_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        flat_idx = torch.empty_like(idx)
        flat_in = [q_rows] + sel_in[1:]
        select_fn(*flat_in, out=flat_idx, workspace=sel_ws)
        flat_ev[0].record(stream)
        for _ in range(args.steps):
            select_fn(*flat_in, out=flat_idx, workspace=sel_ws)
        flat_ev[1].record(stream)
        torch.cuda.synchronize()
        extra["select_row_by_row_ms"] = round(flat_ev[0].elapsed_time(flat_ev[1]) / args.steps, 4)
        log(f"selection row by row {extra['select_row_by_row_ms']:.4f} ms")
    log(f"step {ms_per_step:.4f} ms (wall {wall * 1e3 / args.steps:.4f} ms); stages: select "
        f"{np.mean(sel_ms):.4f} ms (min {np.min(sel_ms):.4f}), attention {np.mean(att_ms):.4f} ms")

    # one more step on the first KV cache (the oracle's) for the parity check
    step(0)
    torch.cuda.synchronize()

    got_idx = idx.cpu().numpy()
    got_out = out.cpu().numpy()
    sel_bytes = select_algorithmic_bytes(w.seq_lens, w.query_pos, w.token_to_req,
                                         key_bytes=132 if fp8 else 256)
    att_bytes = attn_algorithmic_bytes(got_idx)
    # kernel launches of one timed step at these shapes (the committed kernel
    # traces show one call of each per step)
    kernels_per_step = (["qsa_metadata_kernel"] if meta else []) + (
        ["qsa_select_chunk_kernel (paged logits)", "qsa_select_chunk_kernel (top-k per row)"]
        if two_pass else ["qsa_select_chunk_kernel"]) + [
        "qsa_select_merge_kernel", "qsa_attn_kernel", "qsa_attn_combine_kernel"]
    sel_avg_s = float(np.mean(sel_ms)) / 1e3
    att_avg_s = float(np.mean(att_ms)) / 1e3

    def back_to_back_ms(fn) -> float:
        """Average duration of fn's launches: K calls back to back on the
        launch stream between two events (no events between the kernels)."""
        fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(args.steps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / args.steps

    if two_pass:
        # the dominant kernel of the two-pass step is the paged-logits pass
        roof_bytes = logits_algorithmic_bytes(w.seq_lens, w.query_pos, w.token_to_req,
                                              logits_width)
        roof_ms = back_to_back_ms(lambda: qsa.qsa_paged_logits(*sel_in, weights=wt, logits=logits))
        roof_kernel = "qsa_paged_logits (qsa_select_chunk_kernel, logits out)"
    else:
        roof_bytes = sel_bytes
        roof_ms = back_to_back_ms(lambda: select_fn(*(built_in if meta else sel_in), out=idx,
                                                    workspace=sel_ws))
        roof_kernel = (("qsa_select_fp8" if fp8 else "qsa_select") +
                       " (qsa_select_chunk_kernel + qsa_select_merge_kernel)")
    roof_s = roof_ms / 1e3
    log(f"roofline launches back to back: {roof_ms:.4f} ms each")
    achieved = roof_bytes / roof_s / 1e9
    traffic = stored_traffic(w.name)
    ceiling = None if args.no_context else read_ceiling(torch, qsa, dev)
    context = None if args.no_context else r1_latencies(torch, qsa, wl, dev)
    units = None if args.no_context else units_protocol(
        torch, stream, step,
        lambda i: qsa.qsa_sparse_attn(q_attn, *kv_views[i % len(kv_views)], idx, scale, out=out,
                                      workspace=att_ws))
    batched = None if args.no_context else batched_step(torch, qsa, wl, dev)
    if ceiling:
        log(f"read ceiling {ceiling:.0f} GB/s; single-row latencies {context}")
    rows_per_s = R / (ms_per_step / 1e3)
    step_bytes = sel_bytes + att_bytes + (R * logits_width * 8 if two_pass else 0)
    step_gbs = step_bytes / (ms_per_step / 1e3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(rows_per_s, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 keys x f16 queries, f16 attention" if fp8 else "f16",
        "data": ("synthetic (seeded N(0,1) keys absmax-quantized to e4m3 with one fp32 scale per "
                 "key; N(0,1) fp16 queries/KV; random permuted block tables)" if fp8 else
                 "synthetic (seeded N(0,1) fp16 keys/queries/KV, per-head weights U[-0.5, 1.5], "
                 "random permuted block tables)" if two_pass else
                 "synthetic (seeded N(0,1) fp16 keys/queries/KV, random permuted block tables)"),
        "config": {**workload_config(w, len(kv_sets)), "rows_per_run": run},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": roof_kernel,
                     "ceiling": None if ceiling is None else round(ceiling, 1),
                     "frac_of_ceiling": None if ceiling is None else round(achieved / ceiling, 4),
                     "bytes_per_launch": roof_bytes, "avg_launch_ms": round(roof_s * 1e3, 4)},
        "stages": {"select_ms": round(sel_avg_s * 1e3, 4), "attention_ms": round(att_avg_s * 1e3, 4),
                   # per-step event times of the instrumented pass (K samples each)
                   "select_ms_median": round(float(np.median(sel_ms)), 4),
                   "select_ms_min": round(float(np.min(sel_ms)), 4),
                   "attention_ms_median": round(float(np.median(att_ms)), 4),
                   "attention_ms_min": round(float(np.min(att_ms)), 4),
                   "kernels_per_step": kernels_per_step,
                   "attention_bytes": att_bytes,
                   "attention_gbs": round(att_bytes / att_avg_s / 1e9, 1),
                   "step_gbs": round(step_gbs, 1),
                   "step_frac_of_peak": round(step_gbs / HBM_PEAK_GBS, 4),
                   "step_frac_of_ceiling": round(step_gbs / ceiling, 4) if ceiling else None,
                   "timed_entry_point": ("qsa_paged_logits + qsa_topk_per_row + qsa_sparse_attn"
                                         if two_pass else
                                         "qsa_build_metadata + qsa_decode_step" if meta else
                                         "qsa_decode_step_fp8" if fp8 else "qsa_decode_step"),
                   **extra,
                   "stage_timing": "separate pass: qsa_select and qsa_sparse_attn with events "
                                   "between them (the records add a few us per stage); "
                                   "roofline.avg_launch_ms: the roofline call K times back "
                                   "to back between two events"},
    }
    if context is not None:
        result["single_row_latency"] = context
        result["batched_64_rows"] = batched
        result["units_protocol"] = units
        result["gpu_clocks_after_timing"] = clocks
    if not args.no_cpu_baseline:
        base = cpu_baseline(w, scale, fp8=fp8, weights=head_w)
        outs = base.pop("_outs")
        # the timed configuration's output on the rows the oracle finished
        same = sum(np.array_equal(sel[0], got_idx[i]) for i, (sel, _) in enumerate(outs))
        errs = [float(np.max(np.abs(got_out[i].astype(np.float64) - a)))
                for i, (sel, a) in enumerate(outs) if np.array_equal(sel[0], got_idx[i])]
        result["cpu_baseline"] = base
        result["parity"] = {"rows_checked": len(outs), "selection_identical": int(same),
                            "attention_max_abs_err": max(errs) if errs else None}
        log(f"oracle: {base['value']:.2f} rows/s, {base['threaded']['value']:.2f} rows/s on "
            f"{base['host_threads']} threads; identical selections {same}/{len(outs)}")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
