"""Baseline/candidate/baseline (B/C/B) comparison of two builds of the
library on one workload, in the protocol of the page "vLLM: integrate FP16
packed QSA extension" (section "Validation"): excluded warm-up units, then
units alternating baseline and candidate -- B0 C0 B1 C1 ... B(n-1) C(n-1) Bn
-- each unit a fixed number of calls between two HIP events.  Candidate
unit i wins when it is faster than the mean of the baseline units around it
(Bi, Bi+1); the baseline's drift is (Bn - B0) / B0.  Both builds then run
once more on the same inputs and their outputs are compared.

    python bench_ab.py --baseline OLD.so [--candidate NEW.so] [--workload NAME]
                       [--op decode_step|select|attention] [--pairs 10] [--rows R]
                       [--graph]

With --graph each build's unit of calls is captured once in a HIP graph and
every unit is one replay: device time only, for calls shorter than the
host's ~12 us of argument marshalling per call from Python (a single
row's attention), which eager units would time instead.

The candidate defaults to the tree's libqsa_amd.so; a baseline of an
earlier revision is built with `python -m paged_top_indexer_amd.build --rev
REV --out OLD.so`.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BUILDERS = {"tiny": "tiny_integer", "saturated": "saturated_row", "batched": "batched_shared",
            "ties_edges": "ties_and_edges", "long_context": "long_context",
            "multi_token": "multi_token_rows"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--baseline", required=True, help="the baseline build (a .so path)")
    ap.add_argument("--candidate", default=None, help="the candidate build (default: the tree's)")
    ap.add_argument("--workload", choices=sorted(BUILDERS), default="long_context")
    ap.add_argument("--op", choices=["decode_step", "select", "attention"], default="decode_step")
    ap.add_argument("--calls", type=int, default=0,
                    help="calls per unit (default 64; 128 for attention)")
    ap.add_argument("--warmup-units", type=int, default=5)
    ap.add_argument("--pairs", type=int, default=10)
    ap.add_argument("--rows-per-run", type=int, default=0,
                    help="queries as [R/n, n, 4, 128]; default 4 for multi_token, else 1")
    ap.add_argument("--rows", type=int, default=0,
                    help="long_context: its batch size (<= 128); multi_token: its "
                         "rows (4 prefill requests x 16 rows plus decode requests "
                         "x 4 rows; default 256)")
    ap.add_argument("--kv-copies", type=int, default=8)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--graph", action="store_true",
                    help="time each unit as one replay of a HIP graph of its calls")
    args = ap.parse_args()

    import torch
    import paged_top_indexer_amd as qsa
    from paged_top_indexer_amd import _binding
    from paged_top_indexer_amd import workloads as wl

    libs = {"baseline": os.path.abspath(args.baseline),
            "candidate": os.path.abspath(args.candidate or _binding.LIBRARY)}
    for name, path in libs.items():
        if not os.path.exists(path):
            print(f"{name} library {path} is missing", file=sys.stderr)
            return 2
    calls = args.calls or (128 if args.op == "attention" else 64)
    if args.rows and args.workload not in ("long_context", "multi_token"):
        print("--rows applies to long_context and multi_token only", file=sys.stderr)
        return 2
    if args.rows and args.workload == "long_context":
        w = wl.long_context(args.seed, rows=args.rows)
    elif args.rows:
        if args.rows < 64 or args.rows % 4:
            print("multi_token --rows: a multiple of 4, at least 64", file=sys.stderr)
            return 2
        w = wl.multi_token_rows(args.seed, decode_requests=(args.rows - 64) // 4)
    else:
        w = getattr(wl, BUILDERS[args.workload])(args.seed)
    dev = torch.device("cuda:0")
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    sel = [d(a) for a in w.select_inputs()]
    run = args.rows_per_run or (4 if args.workload == "multi_token" else 1)
    if run > 1:
        sel[0] = sel[0].view(w.rows // run, run, 4, 128)
    kv_sets = [d(w.kv)] + [d(wl.normal_f16(np.random.default_rng(args.seed + 1000 + i), w.kv.shape))
                           for i in range(1, args.kv_copies)]
    kv_views = [qsa.kv_views(t) for t in kv_sets]
    q_attn = d(w.q_attn)
    R, W = w.rows, w.block_table.shape[1]
    scale = wl.SOFTMAX_SCALE
    # each build gets buffers of its own (workspace sizes may differ)
    bufs = {}
    for name, path in libs.items():
        _binding.use_library(path)
        bufs[name] = dict(
            idx=torch.empty((R, 2051), dtype=torch.int32, device=dev),
            out=torch.empty((R, 3, 256), dtype=torch.float16, device=dev),
            ws=torch.zeros(max(1, qsa.decode_step_workspace_bytes(R, W),
                               qsa.select_workspace_bytes(R, W),
                               qsa.sparse_attn_workspace_bytes(R)), dtype=torch.uint8,
                           device=dev))
    # attention units read the index rows the baseline selects
    _binding.use_library(libs["baseline"])
    ref_idx = qsa.qsa_select(*sel)
    torch.cuda.synchronize()

    def call(name, i):
        b = bufs[name]
        k, v = kv_views[i % len(kv_views)]
        if args.op == "decode_step":
            qsa.qsa_decode_step(*sel, q_attn, k, v, scale, indices=b["idx"], out=b["out"],
                                workspace=b["ws"])
        elif args.op == "select":
            qsa.qsa_select(*sel, out=b["idx"], workspace=b["ws"])
        else:
            qsa.qsa_sparse_attn(q_attn, k, v, ref_idx, scale, out=b["out"], workspace=b["ws"])

    stream = torch.cuda.current_stream(dev)
    counter = [0]
    graphs = {}
    if args.graph:
        for name in libs:
            _binding.use_library(libs[name])
            call(name, 0)  # outside the capture first
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(calls):
                    call(name, i)
            graphs[name] = g
        torch.cuda.synchronize()

    def unit(name) -> float:
        _binding.use_library(libs[name])
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        if args.graph:
            graphs[name].replay()
        else:
            for _ in range(calls):
                call(name, counter[0])
                counter[0] += 1
        ev[1].record(stream)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / calls

    for u in range(args.warmup_units):
        unit("baseline" if u % 2 == 0 else "candidate")
    base, cand = [unit("baseline")], []
    for _ in range(args.pairs):
        cand.append(unit("candidate"))
        base.append(unit("baseline"))
    wins = sum(c < 0.5 * (base[i] + base[i + 1]) for i, c in enumerate(cand))

    # outputs of the two builds on the same inputs (first KV cache)
    outs = {}
    for name in libs:
        b = bufs[name]
        b["idx"].fill_(-7)
        b["out"].fill_(0)
        _binding.use_library(libs[name])
        if args.op == "attention":
            qsa.qsa_sparse_attn(q_attn, *kv_views[0], ref_idx, scale, out=b["out"], workspace=b["ws"])
        else:
            qsa.qsa_decode_step(*sel, q_attn, *kv_views[0], scale, indices=b["idx"], out=b["out"],
                                workspace=b["ws"])
        torch.cuda.synchronize()
        outs[name] = (b["idx"].cpu().numpy(), b["out"].cpu().numpy())
    _binding.use_library(None)
    same_idx = bool(np.array_equal(outs["baseline"][0], outs["candidate"][0]))
    diff_out = float(np.max(np.abs(outs["baseline"][1].astype(np.float64) -
                                   outs["candidate"][1].astype(np.float64))))
    res = {"workload": w.name, "rows": w.rows, "op": args.op, "calls_per_unit": calls,
           "warmup_units": args.warmup_units, "pairs": args.pairs, "graph": args.graph,
           "baseline": {"lib": libs["baseline"], "mean_ms": round(float(np.mean(base)), 5),
                        "median_ms": round(float(np.median(base)), 5)},
           "candidate": {"lib": libs["candidate"], "mean_ms": round(float(np.mean(cand)), 5),
                         "median_ms": round(float(np.median(cand)), 5)},
           "speedup": round(float(np.mean(base) / np.mean(cand)), 4),
           "wins": f"{wins}/{args.pairs}",
           "baseline_drift_pct": round(100.0 * (base[-1] - base[0]) / base[0], 3),
           "units_ms": {"baseline": [round(x, 5) for x in base],
                        "candidate": [round(x, 5) for x in cand]},
           "indices_identical": same_idx if args.op != "attention" else None,
           "out_max_abs_diff": diff_out}
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
