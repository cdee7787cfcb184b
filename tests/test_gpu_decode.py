"""GPU parity of qsa_decode_step: selection then attention on one stream."""

import numpy as np
import pytest
import torch

from paged_top_indexer_amd import workloads as wl
import paged_top_indexer_amd as qsa
from gpu_util import banner, check_attn, check_select_band, dev, orc, subset_rows

pytestmark = pytest.mark.gpu
SCALE = wl.SOFTMAX_SCALE


def decode_gpu(w):
    kvd = dev(w.kv)
    k, v = qsa.kv_views(kvd)
    sel = [dev(a) for a in w.select_inputs()]
    idx, out = qsa.qsa_decode_step(*sel, dev(w.q_attn), k, v, SCALE)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), out.cpu().numpy()


@pytest.mark.parametrize("make", [wl.tiny_integer, wl.ties_and_edges], ids=["tiny", "edges"])
def test_integer_workloads_exact_selection(make):
    w = make(0)
    banner(f"decode {w.name}")
    idx, out = decode_gpu(w)
    want_idx = orc().select(*w.select_inputs())
    assert np.array_equal(idx, want_idx)
    check_attn(out, orc().sparse_attn(w.q_attn, w.kv, want_idx, SCALE), w.name)


def test_batched_shared():
    w = wl.batched_shared(0)
    banner("decode batched_shared R=64")
    idx, out = decode_gpu(w)
    inputs = w.select_inputs()
    want_idx = orc().select(*inputs)
    check_select_band(idx, want_idx, orc(), inputs, range(w.rows))
    same = np.all(idx == want_idx, axis=1)
    assert same.mean() > 0.5
    rows = np.flatnonzero(same)
    want = orc().sparse_attn(w.q_attn[rows], w.kv, want_idx[rows], SCALE)
    check_attn(out[rows], want, "batched rows with identical selection")


def test_long_context_full_size():
    """The bench's workload and launch configuration, checked on sampled rows."""
    w = wl.long_context(0)
    banner("decode long_context R=128 L=131072 (full size)")
    idx, out = decode_gpu(w)
    rows = [0, 5, 63, 127]
    inputs = w.select_inputs()
    sub = subset_rows(inputs, rows)
    want_idx = orc().select(*sub)
    check_select_band(idx[rows], want_idx, orc(), sub, range(len(rows)))
    same = [i for i, r in enumerate(rows) if np.array_equal(idx[r], want_idx[i])]
    assert same, "no sampled row matched the oracle selection exactly"
    rs = [rows[i] for i in same]
    want = orc().sparse_attn(w.q_attn[rs], w.kv, want_idx[same], SCALE)
    check_attn(out[rs], want, "long rows with identical selection")
    # the decode step's attention equals the standalone attention on its indices
    kvd = dev(w.kv)
    k, v = qsa.kv_views(kvd)
    alone = qsa.qsa_sparse_attn(dev(w.q_attn), k, v, dev(idx), SCALE).cpu().numpy()
    assert np.array_equal(alone, out)


def test_multi_token_rows():
    w = wl.multi_token_rows(0)
    banner(f"decode {w.name}")
    idx, out = decode_gpu(w)
    inputs = w.select_inputs()
    want_idx = orc().select(*inputs)
    check_select_band(idx, want_idx, orc(), inputs, range(w.rows))
    same = np.flatnonzero(np.all(idx == want_idx, axis=1))
    assert same.size > w.rows // 2
    want = orc().sparse_attn(w.q_attn[same], w.kv, want_idx[same], SCALE)
    check_attn(out[same], want, "multi-token rows with identical selection")
