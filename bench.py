"""Decode-step throughput of the QSA select + sparse-attention path on one
MI355X.

Workloads (``--workload``), one per configuration of the decode batch:

* tiny: one decode row of 519 tokens (129 visible blocks, a 3-token tail)
  over an 8-page cache of integer-valued keys with forced exact ties.
* saturated: one decode row of 9215 tokens (2303 blocks) over an 8192-page
  N(0,1) cache: the top-512 fills the 2051-wide output.
* batched: 64 decode rows, lengths uniform in [512, 32768], requests 2i and
  2i+1 sharing their first pages, a 16384-page N(0,1) cache.
* ties_edges: 32 rows over edge lengths (0, 1-3, one page, page crossings,
  65536) with keys from a 64-vector integer palette (massive ties).
* long_context (default): R=128 query rows, each of a 131072-token request
  (32768 compressed blocks), a 32768-page fp16 N(0,1) compressed-key cache
  (1 GiB) behind random permuted block tables, and full-width [128,2051]
  sparse attention over a 131072-token packed fp16 KV cache (128 MiB).
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
stream, no host sync); after ~25 ms of plain HBM reads (the device's ramp-up
under load) and W warm-up steps, K steps (200 by default) are timed with HIP
events at both ends, the last warm-up step queued right before the start
event (so the region opens on a busy GPU, one step behind another).  The
steps rotate over distinct KV caches and over block tables that map the
rows through distinct page permutations of the key cache, as consecutive
layers would read distinct caches (no step finds its data in the last-level
cache because an earlier step read it).  The same K steps replayed from a
HIP graph give the device's time per step without the host's launches
(stages.ms_per_step_graph: a small batch's calls from Python are bound by
their argument marshalling).  A second pass runs the two stages through
qsa_select and qsa_sparse_attn with events between them for the per-stage
times; each stage's K calls back to back, replayed from a HIP graph, give
the roofline.  Prints one JSON line.
The oracle then checks every row of the timed configuration's output (the
band rule on N(0,1) inputs, bit-exact selection on integer inputs, attention
within 2e-3 and one fp16 ulp); the exit status is 1 when any row fails.

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
# the sources that fix the kernels' memory traffic (a counter summary is
# used only while their hash matches the one it was taken on)
KERNEL_SOURCES = [os.path.join(ROOT, "paged_top_indexer_amd", "csrc", f)
                  for f in ("qsa_select.hip", "qsa_attn.hip", "qsa_device.h", "qsa_launch.h",
                            "qsa_topk.h", "qsa_plan.cpp")]

# --workload name -> (builder, integer inputs: the selection is checked
# bit-exact; else by the band rule)
WORKLOADS = {
    "tiny": ("tiny_integer", True),
    "saturated": ("saturated_row", False),
    "batched": ("batched_shared", False),
    "ties_edges": ("ties_and_edges", True),
    "long_context": ("long_context", False),
    "long_context_fp8": ("long_context", False),
    "long_context_two_pass": ("long_context", False),
    "multi_token": ("multi_token_rows", False),
    "multi_token_metadata": ("multi_token_rows", False),
}


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


def attn_algorithmic_bytes(indices: np.ndarray) -> tuple[int, int]:
    """(HBM bytes, gather bytes) the attention must move per launch.  Every
    row of a launch indexes the same packed KV cache, so HBM must supply each
    distinct valid token of the launch once: 1 KiB (K and V halves) per
    token of the union over all rows.  Gather bytes count 1 KiB per distinct
    valid token of each row, i.e. what the rows read, repeats across rows
    included (those come from the caches when they hit).  Both add, per row,
    the 8204 B index row, the 1.5 KiB query and the 1.5 KiB output."""
    per_row = (8204 + 1536 + 1536) * indices.shape[0]
    union = 1024 * len(np.unique(indices[indices >= 0]))
    gather = sum(1024 * len(np.unique(row[row >= 0])) for row in indices)
    return union + per_row, gather + per_row


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_counters(workload: str):
    """The committed counter summary of this workload
    (profiles/select_<workload>_counters.json) if it was taken on the
    current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"select_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash() or rec.get("workload") != workload:
        return None
    return rec


def read_probe(torch, dev, gib: int = 2):
    """A callable that streams a `gib` GiB device buffer once with
    nontemporal loads: qsa_read_probe of libqsa_probe.so (include/qsa_probe.h,
    a measurement aid built apart from the method's library), on the current
    stream.  Returns (probe, buffer bytes)."""
    import ctypes

    from paged_top_indexer_amd import build

    lib = ctypes.CDLL(build.PROBE_LIBRARY)
    lib.qsa_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_size_t, ctypes.c_void_p]
    lib.qsa_read_probe.restype = ctypes.c_int
    buf = torch.empty(gib << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def probe():
        rc = lib.qsa_read_probe(buf.data_ptr(), buf.numel(), sink.data_ptr(), 4,
                                stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"qsa_read_probe failed with status {rc}")

    return probe, buf.numel()


def read_ceiling(torch, probe, nbytes: int, reps: int = 5) -> float:
    """The box's practical HBM read ceiling (GB/s): the read probe over its
    `nbytes` buffer, `reps` times between HIP events."""
    stream = torch.cuda.current_stream()
    probe()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        probe()
    ev[1].record(stream)
    torch.cuda.synchronize()
    return nbytes * reps / (ev[0].elapsed_time(ev[1]) / 1e3) / 1e9


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
    """Threads for the oracle: the CPUs this process may run on, at most 16
    (the host share of one GPU on a shared node, whatever the machine's own
    count)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _pin(cpu: int):
    """Pin the calling thread to one CPU; returns the previous set."""
    before = os.sched_getaffinity(0)
    os.sched_setaffinity(0, {cpu})
    return before


def oracle_rows_fn(w, scale: float, kind: str, weights=None, batch: int = 4):
    """(per-batch inputs prepared up front, fn(batch inputs) running the whole
    decode step of those rows through the oracle).  Slicing and copying the
    rows' inputs happens here, outside any timed region; a call then only
    hands the arrays to the C oracle (a few microseconds against ~50 ms per
    row at the long-context shape)."""
    import oracle

    orc = oracle.default()
    q, kc, bt, t2r, sl, qp = w.select_inputs()
    R = w.rows
    batches = []
    for i in range(0, R, batch):
        rs = np.arange(i, min(R, i + batch))
        batches.append(dict(q=np.ascontiguousarray(q[rs]), t2r=np.ascontiguousarray(t2r[rs]),
                            qp=np.ascontiguousarray(qp[rs]),
                            qa=np.ascontiguousarray(w.q_attn[rs]),
                            wt=None if weights is None else np.ascontiguousarray(weights[rs]),
                            rows=len(rs)))

    def run(b):
        if kind == "fp8":
            sel = orc.select_fp8(b["q"], w.kcodes, w.kscale, bt, b["t2r"], sl, b["qp"])
        elif kind == "two_pass":
            lg = orc.paged_logits(b["q"], b["wt"], bt, b["t2r"], sl, b["qp"], bt.shape[1] * 128,
                                  kcache=kc)
            sel = orc.topk_per_row(lg, b["t2r"], sl, b["qp"])
        else:
            sel = orc.select(b["q"], kc, bt, b["t2r"], sl, b["qp"])
        orc.sparse_attn(b["qa"], w.kv, sel, scale)
        return b["rows"]

    return batches, run


def cpu_baseline(w, scale: float, kind: str, weights=None, min_seconds: float = 10.0,
                 max_seconds: float = 25.0, threaded_seconds: float = 6.0) -> dict:
    """The CPU oracle (plain C, unmodified) on the host cores, over the same
    workload: the whole decode step (selection then attention) of batches of
    4 rows, cycling over the rows.  Single-threaded leg: the calling thread
    pinned to one CPU, until every row is done once and at least min_seconds
    have passed (at most max_seconds).  Threaded leg: host_threads() threads,
    each pinned to its own CPU, taking batches from a shared counter for
    about threaded_seconds (the C calls release the interpreter lock and
    keep no shared state)."""
    import itertools
    from concurrent.futures import ThreadPoolExecutor

    batches, run = oracle_rows_fn(w, scale, kind, weights)
    cpus = sorted(os.sched_getaffinity(0))
    before = _pin(cpus[0])
    try:
        run(batches[0])  # warm-up (page-in of the oracle and the inputs)
        done, k = 0, 0
        t0 = time.perf_counter()
        while True:
            dt = time.perf_counter() - t0
            if dt >= max_seconds or (dt >= min_seconds and done >= w.rows):
                break
            done += run(batches[k % len(batches)])
            k += 1
        dt = time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, before)

    threads = host_threads()
    ticket = itertools.count()  # next() on a count is atomic under the interpreter lock
    t1 = time.perf_counter()
    stop = t1 + threaded_seconds

    def worker(i):
        os.sched_setaffinity(0, {cpus[i % len(cpus)]})
        n = 0
        while time.perf_counter() < stop:
            n += run(batches[next(ticket) % len(batches)])
        return n

    with ThreadPoolExecutor(threads) as ex:
        done_t = sum(ex.map(worker, range(threads)))
    dt_t = time.perf_counter() - t1
    return {"value": done / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} rows ({w.rows} distinct, batches of 4 cycled) of the same "
                      f"workload, selection + attention per row, {dt:.1f} s on one pinned CPU "
                      f"(inputs sliced before the clock starts)",
            "host_cpu": host_cpu(), "nproc": os.cpu_count(), "affinity_cpus": len(cpus),
            "threaded": {"value": done_t / dt_t, "unit": "rows/s", "cores": threads,
                         "sample": f"{done_t} rows dealt in batches of 4 to {threads} threads "
                                   f"pinned to distinct CPUs, {dt_t:.1f} s"}}


def parity_all_rows(w, kind: str, exact: bool, got_idx, got_out, scale: float,
                    weights=None) -> dict:
    """The timed configuration's output against the oracle on every row:
    the selection bit-exact (integer inputs) or within the band rule
    (N(0,1) inputs), and the attention over the GPU's own index rows within
    2e-3 and one fp16 ulp of the float64 oracle.  Rows are dealt to host
    threads."""
    import oracle
    from oracle import acceptance as acc

    orc = oracle.default()
    t0 = time.perf_counter()
    inputs = w.select_inputs()
    row_scores = None
    if kind == "fp8":
        inputs = w.select_inputs_fp8()
        ref = acc.oracle_select(orc, inputs)
    elif kind == "two_pass":
        q, kc, bt, t2r, sl, qp = inputs
        width = bt.shape[1] * 128
        ref = acc.map_rows(lambda rs: orc.select_weighted(q[rs], weights[rs], bt, t2r[rs], sl,
                                                          qp[rs], kcache=kc), range(w.rows))

        def row_scores(r):
            return orc.paged_logits(q[r:r + 1], weights[r:r + 1], bt, t2r[r:r + 1], sl,
                                    qp[r:r + 1], width, kcache=kc)[0]
    else:
        ref = acc.oracle_select(orc, inputs)
    identical = int(np.all(got_idx == ref, axis=1).sum())
    if exact:
        problems = {int(r): "differs" for r in np.flatnonzero(~np.all(got_idx == ref, axis=1))}
    else:
        problems = acc.band_problems(orc, got_idx, ref, inputs, row_scores=row_scores)
    want = acc.oracle_attn(orc, w.q_attn, w.kv, got_idx, scale)
    err, over = acc.attn_error(got_out, want)
    ok = not problems and err <= acc.ATTN_TOL and over == 0
    return {"rows_checked": int(w.rows),
            "selection_rule": "bit-exact" if exact else "band 1e-3 * max(|s_n|, 1)",
            "selection_identical": identical,
            "selection_within_rule": int(w.rows - len(problems)),
            "selection_failures": {str(k): v for k, v in list(problems.items())[:5]},
            "attention_rows_checked": int(w.rows), "attention_index_rows": "the GPU's own",
            "attention_max_abs_err": err, "attention_over_1ulp": over,
            "attention_tol": acc.ATTN_TOL, "ok": bool(ok),
            "check_s": round(time.perf_counter() - t0, 1)}


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


def workload_config(w, kv_copies: int, key_tables: int) -> dict:
    lens = w.seq_lens[w.token_to_req].astype(np.int64)
    cfg = {"workload": w.name, "rows": int(w.rows), "requests": int(len(np.unique(w.token_to_req))),
           "cache_pages": int(w.kcache.shape[0]), "kv_tokens": int(w.kv.shape[0] * w.kv.shape[1]),
           "top_blocks": 512, "index_width": 2051, "kv_caches_rotated": kv_copies,
           "key_tables_rotated": key_tables}
    if np.all(lens == lens[0]):
        cfg["seq_len"] = int(lens[0])
    else:
        cfg["seq_len_range"] = [int(lens.min()), int(lens.max())]
    return cfg


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 200 by default: a region opened on an idle GPU carries a fixed ~0.14 ms
    # start cost (measured: 0.2382 / 0.2340 / 0.2321 ms per step at K = 20 /
    # 64 / 200), which the lead-in below takes out of the timed region
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle: no CPU baseline and no parity check")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the read-ceiling probe, the single-row latencies and the pages' "
                         "unit protocol")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="long_context")
    ap.add_argument("--rows-per-run", type=int, default=0,
                    help="pass the selection queries as [R/n, n, 4, 128] (runs of n rows of "
                         "one request); default 4 for the multi_token workloads, else 1")
    ap.add_argument("--kv-copies", type=int, default=8,
                    help="distinct KV caches the steps rotate over (one per simulated layer)")
    ap.add_argument("--key-tables", type=int, default=8,
                    help="block tables (page permutations of the key cache) the steps' "
                         "selections rotate over (one per simulated layer)")
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
    builder, exact = WORKLOADS[args.workload]
    fp8 = args.workload == "long_context_fp8"
    two_pass = args.workload == "long_context_two_pass"
    meta = args.workload == "multi_token_metadata"
    multi = args.workload in ("multi_token", "multi_token_metadata")
    kind = "fp8" if fp8 else "two_pass" if two_pass else "f16"
    head_w = None
    w = getattr(wl, builder)(args.seed)
    if fp8:
        w = wl.with_fp8_keys(w, integer=False)
    if two_pass:
        head_w = wl.head_weights(np.random.default_rng(args.seed + 555), w.rows)
        w.name = w.name + "_two_pass"
    if meta:
        w.name = w.name + "_metadata"
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
    run = args.rows_per_run or (4 if multi else 1)
    q_rows = sel_in[0]
    if run > 1:
        assert w.rows % run == 0, "rows must split into whole runs"
        sel_in[0] = q_rows.view(w.rows // run, run, 4, 128)
    # Consecutive decode steps of a model read different layers' caches.  The
    # steps here rotate over distinct KV caches (8 x 128 MiB by default at the
    # long-context shape, four times the 256 MB Infinity Cache) so that no
    # step finds its KV in the last-level cache because an earlier step read
    # it.
    kv_sets = [d(w.kv)]
    for i in range(1, args.kv_copies):
        kv_sets.append(d(wl.normal_f16(np.random.default_rng(args.seed + 1000 + i), w.kv.shape)))
    kv_views = [qsa.kv_views(t) for t in kv_sets]
    # Likewise the selection: a layer's compressed keys are read once per
    # step, so the steps rotate over block tables that map the rows through
    # distinct page permutations of the cache (table 0 is the workload's own;
    # same rows, lengths and sharing, other physical pages).  No step then
    # finds its keys in the last-level cache because an earlier step read
    # them.
    sel_sets = [sel_in]
    perm_rng = np.random.default_rng(args.seed + 2000)
    bt_at = 3 if fp8 else 2  # (e4m3 inputs carry the key scales before the table)
    for i in range(1, args.key_tables):
        perm = perm_rng.permutation(w.kcache.shape[0]).astype(np.int32)
        bt = np.asarray(w.block_table).copy()
        bt[bt >= 0] = perm[bt[bt >= 0]]
        sel_sets.append(sel_in[:bt_at] + [d(bt)] + sel_in[bt_at + 1:])
    sel_at = lambda i: sel_sets[i % len(sel_sets)]  # noqa: E731
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
        built_at = lambda i: [sel_at(i)[0], sel_at(i)[1], sel_at(i)[2]] + built_in[3:]  # noqa: E731

        def build_metadata():
            qsa.qsa_build_metadata(qsl, sel_in[4], sel_in[2], R, max_num_work=R, out=meta_out,
                                   workspace=meta_ws)

        def select_stage(i, mark=None):
            build_metadata()
            if mark is not None:
                mark.record(stream)
            select_fn(*built_at(i), out=idx, workspace=sel_ws)

        def step(i):
            k, v = kv_views[i % len(kv_views)]
            build_metadata()
            decode_fn(*built_at(i), q_attn, k, v, scale, indices=idx, out=out, workspace=ws_all)
    elif two_pass:
        wt = d(head_w)
        logits_width = w.block_table.shape[1] * 128
        logits = torch.empty((R, logits_width), dtype=torch.float32, device=dev)
        topk_ws = torch.zeros(max(1, qsa.topk_per_row_workspace_bytes(R, logits_width)),
                              dtype=torch.uint8, device=dev)

        def select_stage(i, mark=None):
            qsa.qsa_paged_logits(*sel_at(i), weights=wt, logits=logits)
            if mark is not None:
                mark.record(stream)
            qsa.qsa_topk_per_row(logits, sel_in[3], sel_in[4], sel_in[5], out=idx,
                                 workspace=topk_ws)

        def step(i):
            k, v = kv_views[i % len(kv_views)]
            select_stage(i)
            qsa.qsa_sparse_attn(q_attn, k, v, idx, scale, out=out, workspace=att_ws)
    else:
        def select_stage(i, mark=None):
            select_fn(*sel_at(i), out=idx, workspace=sel_ws)

        def step(i):
            k, v = kv_views[i % len(kv_views)]
            decode_fn(*sel_at(i), q_attn, k, v, scale, indices=idx, out=out, workspace=ws_all)

    # The device runs the first ~10 ms of memory load after an idle spell
    # slower while it ramps up (measured at the long-context shape:
    # consecutive regions of 20 decode steps from the process's start read
    # 0.2305, 0.2258, then 0.2230-0.2239 ms per step; after ~10-25 ms of
    # plain HBM reads the first region already reads 0.2235-0.2240 ms, while
    # a 25 ms device sleep does not help; in one process, K = 20 selections
    # timed after a graph capture read 4% slower than the same a pass
    # later).  device_warmup queues
    # `reps` streams of the read probe's 2 GiB buffer (none of the
    # workload's; ~0.3 ms each) before a timed measurement, so that a short
    # timed region does not measure that ramp.
    probe, probe_bytes = read_probe(torch, dev)

    def device_warmup(reps: int) -> None:
        for _ in range(reps):
            probe()

    def graph_ms(fn) -> float:
        """ms per call of fn(0..K-1) captured once in a HIP graph and replayed
        between two events on the launch stream (fn(0) runs once outside the
        capture first).  After the capture ~10 ms of plain reads and an
        eager fn(4) (another cache and table than the graph's first call)
        are queued before the start event: the device is up to speed and
        busy while the host launches the graph."""
        fn(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(args.steps):
                fn(i)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        device_warmup(32)
        fn(4)
        ev[0].record(stream)
        g.replay()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / args.steps

    def timed_steps(lead_in) -> float:
        """ms per step over exactly K decode steps between two events, after a
        synchronisation.  lead_in: work queued between the synchronisation
        and the start event, so that the timed region opens with the GPU
        busy and the first timed step already queued -- otherwise it also
        holds the host's first launch (marshalling, the launch path) on an
        idle GPU, a fixed cost that a short region spreads over its few
        steps.  None opens the region on an idle GPU."""
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        if lead_in is not None:
            lead_in()
        ev[0].record(stream)
        for i in range(args.steps):
            step(i)
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / args.steps

    # ~25 ms of plain HBM reads (device_warmup), W untimed warm-up steps,
    # then exactly K timed decode steps (events only at the ends).  The last warm-up step is the lead-in: it is queued after
    # the synchronisation, right before the start event, so the region opens
    # as a serving loop runs, one step behind another (a ~0.2 ms device sleep
    # there instead, on an idle-but-for-one-wave GPU, read ~1 us per step more
    # at K = 20 on one box).  Without warm-up the sleep is the lead-in.
    device_warmup(80)
    torch.cuda.synchronize()
    for i in range(args.warmup - 1):
        step(i)
    if args.warmup > 0:
        lead = lambda: step(args.warmup - 1)  # noqa: E731
    else:
        lead = lambda: torch.cuda._sleep(500_000)  # noqa: E731  (GPU clock cycles, ~0.2 ms)
    t_start = time.perf_counter()
    ms_per_step = timed_steps(lead)
    wall = time.perf_counter() - t_start
    # the same K steps with the region opening on an idle GPU, for reference
    ms_per_step_cold = timed_steps(None)
    # and captured once in a HIP graph, replayed between two events: the
    # device's time per step without the host's launches (a small batch's
    # steps from Python are bound by their ~12 us of argument marshalling)
    ms_per_step_graph = graph_ms(step)
    clocks = None if args.no_context else gpu_clocks()

    # Per-stage times: the same two stages through their own entry points,
    # with events recorded on the launch stream around each.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        k, v = kv_views[i % len(kv_views)]
        events[i][0].record(stream)
        select_stage(i, mark=events[i][3] if (two_pass or meta) else None)
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
        for i in range(args.steps):
            qsa.qsa_select_weighted(sel_in[0], wt, *sel_at(i)[1:], out=fused_idx,
                                    workspace=sel_ws)
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
        select_fn(q_rows, *sel_in[1:], out=flat_idx, workspace=sel_ws)
        flat_ev[0].record(stream)
        for i in range(args.steps):
            select_fn(q_rows, *sel_at(i)[1:], out=flat_idx, workspace=sel_ws)
        flat_ev[1].record(stream)
        torch.cuda.synchronize()
        extra["select_row_by_row_ms"] = round(flat_ev[0].elapsed_time(flat_ev[1]) / args.steps, 4)
        log(f"selection row by row {extra['select_row_by_row_ms']:.4f} ms")
    log(f"step {ms_per_step:.4f} ms (cold start {ms_per_step_cold:.4f} ms, graph-replayed "
        f"{ms_per_step_graph:.4f} ms; wall {wall * 1e3 / args.steps:.4f} ms with the lead-in); "
        f"stages: select "
        f"{np.mean(sel_ms):.4f} ms (min {np.min(sel_ms):.4f}), attention {np.mean(att_ms):.4f} ms")

    # one more step on the first KV cache (the oracle's) for the parity check
    step(0)
    torch.cuda.synchronize()

    got_idx = idx.cpu().numpy()
    got_out = out.cpu().numpy()
    sel_bytes = select_algorithmic_bytes(w.seq_lens, w.query_pos, w.token_to_req,
                                         key_bytes=132 if fp8 else 256)
    att_bytes, att_gather = attn_algorithmic_bytes(got_idx)
    # kernel launches of one timed step at these shapes (the committed kernel
    # traces show one call of each per step).  This mirrors the library's
    # plans: rows of several chunks need a merge (a selection workspace),
    # except in a decode step whose attention takes 12-wave workgroups (up
    # to 256 rows), which selects them itself (every workload here keeps a
    # row's candidates within the 8192 the attention workgroup holds); a
    # top-k per row over at most 32768 columns is one kernel; several splits
    # per row need a combine (an attention workspace).
    plan_chunks = qsa.select_workspace_bytes(R, w.block_table.shape[1]) > 0
    row_waves = 0 < R <= 256
    combine = ["qsa_attn_combine_kernel"] if qsa.sparse_attn_workspace_bytes(R) > 0 else []
    if two_pass:
        topk = (["qsa_topk_row_kernel"] if logits_width <= 32768 else
                ["qsa_select_chunk_kernel (top-k per row)", "qsa_select_merge_kernel"])
        kernels_per_step = ["qsa_select_chunk_kernel (paged logits)"] + topk + ["qsa_attn_kernel"]
    else:
        fused = plan_chunks and row_waves
        kernels_per_step = (["qsa_metadata_kernel"] if meta else []) + ["qsa_select_chunk_kernel"] + (
            ["qsa_select_merge_kernel"] if plan_chunks and not fused else []) + (
            ["qsa_attn_kernel (selecting multi-chunk rows)"] if fused else ["qsa_attn_kernel"])
    kernels_per_step += combine
    sel_avg_s = float(np.mean(sel_ms)) / 1e3
    att_avg_s = float(np.mean(att_ms)) / 1e3

    def back_to_back_ms(fn) -> float:
        """Average duration of fn's launches: K calls back to back on the
        launch stream between two events (no events between the kernels),
        replayed from a HIP graph so that no host launch gap sits between
        them."""
        return graph_ms(fn)

    # Roofline of each stage: algorithmic bytes per launch / the launch's
    # average duration back to back; the stage that takes longer is the
    # dominant one (the selection at every shape with long rows).
    if two_pass:
        sel_roof_bytes = logits_algorithmic_bytes(w.seq_lens, w.query_pos, w.token_to_req,
                                                  logits_width)
        sel_roof_ms = back_to_back_ms(
            lambda i: qsa.qsa_paged_logits(*sel_at(i), weights=wt, logits=logits))
        sel_kernel = "qsa_paged_logits (qsa_select_chunk_kernel, logits out)"
    else:
        sel_roof_bytes = sel_bytes
        sel_roof_ms = back_to_back_ms(lambda i: select_fn(*(built_at(i) if meta else sel_at(i)),
                                                          out=idx, workspace=sel_ws))
        sel_kernel = (("qsa_select_fp8" if fp8 else "qsa_select") + " (qsa_select_chunk_kernel" +
                      (" + qsa_select_merge_kernel)" if plan_chunks else ")"))
    att_roof_ms = back_to_back_ms(
        lambda i: qsa.qsa_sparse_attn(q_attn, *kv_views[i % len(kv_views)], idx, scale, out=out,
                                      workspace=att_ws))
    att_kernel = "qsa_sparse_attn (qsa_attn_kernel" + (
        " + qsa_attn_combine_kernel)" if qsa.sparse_attn_workspace_bytes(R) > 0 else ")")
    log(f"back to back: selection {sel_roof_ms:.4f} ms, attention {att_roof_ms:.4f} ms per launch")
    counters = stored_counters(w.name)
    ceiling = None if args.no_context else read_ceiling(torch, probe, probe_bytes)

    def roof(nbytes, ms, kernel, traffic):
        gbs = nbytes / (ms / 1e3) / 1e9
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
                "ceiling": None if ceiling is None else round(ceiling, 1),
                "frac_of_ceiling": None if ceiling is None else round(gbs / ceiling, 4),
                "bytes_per_launch": int(nbytes), "avg_launch_ms": round(ms, 4)}

    sel_roof = roof(sel_roof_bytes, sel_roof_ms, sel_kernel,
                    counters.get("hbm_bytes_per_launch") if counters else None)
    att_roof = roof(att_bytes, att_roof_ms, att_kernel,
                    counters.get("attn_hbm_bytes_per_launch") if counters else None)
    dominant, other = (sel_roof, att_roof) if sel_roof_ms >= att_roof_ms else (att_roof, sel_roof)
    context = None if args.no_context else r1_latencies(torch, qsa, wl, dev)
    units = None if args.no_context else units_protocol(
        torch, stream, step,
        lambda i: qsa.qsa_sparse_attn(q_attn, *kv_views[i % len(kv_views)], idx, scale, out=out,
                                      workspace=att_ws))
    if ceiling:
        log(f"read ceiling {ceiling:.0f} GB/s; single-row latencies {context}")
    rows_per_s = R / (ms_per_step / 1e3)
    step_bytes = sel_bytes + att_bytes + (R * logits_width * 8 if two_pass else 0)
    step_gbs = step_bytes / (ms_per_step / 1e3) / 1e9
    data = ("synthetic (seeded N(0,1) keys absmax-quantized to e4m3 with one fp32 scale per "
            "key; N(0,1) fp16 queries/KV; random permuted block tables)" if fp8 else
            "synthetic (seeded N(0,1) fp16 keys/queries/KV, per-head weights U[-0.5, 1.5], "
            "random permuted block tables)" if two_pass else
            "synthetic (seeded integer-valued fp16 keys/queries with exact ties; N(0,1) fp16 KV)"
            if exact else
            "synthetic (seeded N(0,1) fp16 keys/queries/KV, random block tables)")

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
        "data": data,
        "config": {**workload_config(w, len(kv_sets), len(sel_sets)), "rows_per_run": run},
        "roofline": dominant,
        "stages": {"select_ms": round(sel_avg_s * 1e3, 4), "attention_ms": round(att_avg_s * 1e3, 4),
                   # per-step event times of the instrumented pass (K samples each)
                   "select_ms_median": round(float(np.median(sel_ms)), 4),
                   "select_ms_min": round(float(np.min(sel_ms)), 4),
                   "attention_ms_median": round(float(np.median(att_ms)), 4),
                   "attention_ms_min": round(float(np.min(att_ms)), 4),
                   "kernels_per_step": kernels_per_step,
                   "other_stage_roofline": other,
                   "attention_bytes": att_bytes,
                   "attention_gather_bytes": att_gather,
                   "attention_gbs": round(att_bytes / (att_roof_ms / 1e3) / 1e9, 1),
                   "attention_gather_gbs": round(att_gather / (att_roof_ms / 1e3) / 1e9, 1),
                   "attention_fetch_bytes_measured": (counters.get("attn_fetch_bytes_per_launch")
                                                      if counters else None),
                   "select_bytes": sel_bytes,
                   "step_bytes": step_bytes,
                   "step_gbs": round(step_gbs, 1),
                   "step_frac_of_peak": round(step_gbs / HBM_PEAK_GBS, 4),
                   "step_frac_of_ceiling": round(step_gbs / ceiling, 4) if ceiling else None,
                   "ms_per_step_cold_start": round(ms_per_step_cold, 4),
                   "ms_per_step_graph": round(ms_per_step_graph, 4),
                   "timed_entry_point": ("qsa_paged_logits + qsa_topk_per_row + qsa_sparse_attn"
                                         if two_pass else
                                         "qsa_build_metadata + qsa_decode_step" if meta else
                                         "qsa_decode_step_fp8" if fp8 else "qsa_decode_step"),
                   **extra,
                   "stage_timing": "select_ms / attention_ms: a separate pass through "
                                   "qsa_select and qsa_sparse_attn with events between them "
                                   "(the records add a few us per stage); roofline "
                                   "avg_launch_ms: each stage's call K times back to back "
                                   "between two events (attention rotating the KV caches), "
                                   "replayed from a HIP graph; ms_per_step_graph: the K "
                                   "decode steps likewise"},
    }
    if context is not None:
        result["single_row_latency"] = context
        result["units_protocol"] = units
        result["gpu_clocks_after_timing"] = clocks
    status = 0
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, scale, kind, weights=head_w)
        base = result["cpu_baseline"]
        log(f"oracle: {base['value']:.2f} rows/s on one pinned CPU, "
            f"{base['threaded']['value']:.2f} rows/s on {base['threaded']['cores']} threads")
        par = parity_all_rows(w, kind, exact, got_idx, got_out, scale, weights=head_w)
        result["parity"] = par
        log(f"parity: selection {par['selection_within_rule']}/{par['rows_checked']} within "
            f"the rule ({par['selection_identical']} identical), attention max abs err "
            f"{par['attention_max_abs_err']:.2e} over {par['attention_rows_checked']} rows, "
            f"{par['attention_over_1ulp']} elements over 1 ulp")
        if not par["ok"]:
            status = 1
    print(json.dumps(result), flush=True)
    return status


if __name__ == "__main__":
    sys.exit(main())
