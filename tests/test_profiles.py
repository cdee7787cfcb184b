"""The committed rocprofv3 summaries agree with the code they describe: the
stored HBM counters were taken on the current kernel sources (otherwise the
bench reports no traffic), and every kernel trace shows one dispatch of each
kernel per selection and per decode step."""

import json
import os
import re

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
WORKLOADS = ["long_context_R128_L131072", "long_context_R128_L131072_fp8",
             "long_context_R128_L131072_two_pass", "multi_token_R256_next4_prefill16",
             "multi_token_R256_next4_prefill16_metadata", "batched_R64_shared_pages",
             "tiny_integer_R1_L519", "saturated_R1_L9215_P8192", "ties_edges_R32_palette64"]


def trace_calls(workload: str) -> tuple[dict, int, int, int, int]:
    """Kernel name -> calls from the summary table, the number of steps the
    run made (the sum of the counts in its 'Calls = ...' line), the
    back-to-back selection and attention calls after them, and how many of
    the steps were decode-step calls (warm-up, timed and parity)."""
    with open(os.path.join(PROFILES, f"kernel_trace_decode_step_{workload}.md")) as f:
        text = f.read()
    calls = {}
    for m in re.finditer(r"^\| (qsa\S.*?) \| (\d+) \|", text, re.M):
        calls[m.group(1)] = int(m.group(2))
    protocol = re.search(r"Calls = (\d+) warm-up \+ (\d+) timed .*? \+ (\d+) instrumented "
                         r"steps .*?\+ (\d+) parity step", text, re.S)
    assert protocol, f"{workload}: no call protocol line"
    roof = re.search(r"plus (\d+) back-to-back roofline calls \(selection\) and (\d+) "
                     r"back-to-back attention calls", text)
    assert roof, f"{workload}: no back-to-back calls in the protocol line"
    g = [int(x) for x in protocol.groups()]
    return calls, sum(g), int(roof.group(1)), int(roof.group(2)), g[0] + g[1] + g[3]


@pytest.mark.parametrize("workload", WORKLOADS)
def test_counters_taken_on_current_sources(workload):
    with open(os.path.join(PROFILES, f"select_{workload}_counters.json")) as f:
        rec = json.load(f)
    assert rec["workload"] == workload
    assert rec["source_hash"] == bench.kernel_source_hash(), \
        "kernel sources changed since the counters were taken: profile again"
    got = bench.stored_counters(workload)
    assert got is not None and got["hbm_bytes_per_launch"] == rec["hbm_bytes_per_launch"] > 0
    assert rec["attn_fetch_bytes_per_launch"] > 0
    cal = rec["copy_calibration"]
    assert abs(cal["fetch_factor"] - 2.0) < 0.01 and abs(cal["write_factor"] - 1.0) < 0.01


@pytest.mark.parametrize("workload", WORKLOADS)
def test_one_dispatch_per_step(workload):
    calls, steps, roof, attn_b2b, decode_steps = trace_calls(workload)
    # one attention launch per step and per back-to-back call (<4> or <12>
    # waves; <12, true> is the decode step's fused selection + attention)
    attn = sum(v for k, v in calls.items() if k.startswith("qsa_attn_kernel<"))
    assert attn == steps + attn_b2b
    fused = calls.get("qsa_attn_kernel<12, true>", 0)
    assert fused in (0, decode_steps)
    if "qsa_attn_combine_kernel" in calls:
        assert calls["qsa_attn_combine_kernel"] == steps + attn_b2b
    chunk = {k: v for k, v in calls.items() if k.startswith("qsa_select_chunk_kernel<")}
    # a selection over several chunks per row is one chunk launch and one
    # merge launch; the paged-logits form (second template argument true)
    # writes the matrix and has no merge
    selecting = sum(v for k, v in chunk.items() if k.split(",")[1].strip() == "false")
    if "qsa_select_merge_kernel" in calls:
        # the fused decode steps launch no merge: their attention selects
        assert calls["qsa_select_merge_kernel"] == selecting - (decode_steps if fused else 0)
    if workload.endswith("_two_pass"):
        assert chunk["qsa_select_chunk_kernel<0, true, 1, 256>"] == steps + roof
        # the top-k per row of 32768-column logits: one workgroup per row
        assert calls["qsa_topk_row_kernel"] == steps
        assert not any(k.startswith("qsa_select_chunk_kernel<2,") for k in chunk)
    elif workload.endswith("_metadata"):
        builder = [v for k, v in calls.items() if "qsa_metadata_kernel" in k]
        assert builder and builder[0] >= steps
        assert sum(chunk.values()) == steps + roof
    else:
        # the timed instantiation runs once per step and per roofline call
        # (the multi-token run adds a row-by-row comparison through the
        # one-row instantiation)
        assert steps + roof in chunk.values()
