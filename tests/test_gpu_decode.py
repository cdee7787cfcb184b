"""GPU parity of qsa_decode_step: selection then attention on one stream."""

import numpy as np
import pytest
import torch

from paged_top_indexer_amd import workloads as wl
import paged_top_indexer_amd as qsa
from gpu_util import (banner, check_attn, check_select_band, dev, oracle_attn, oracle_select,
                      orc)

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
    """Every row: the selection against the oracle's (band rule), the
    attention against the oracle over the decode step's own index rows."""
    w = wl.batched_shared(0)
    banner("decode batched_shared R=64")
    idx, out = decode_gpu(w)
    inputs = w.select_inputs()
    want_idx = orc().select(*inputs)
    check_select_band(idx, want_idx, orc(), inputs, range(w.rows))
    check_attn(out, oracle_attn(orc(), w.q_attn, w.kv, idx, SCALE), "batched, every row")


def test_long_context_full_size():
    """The bench's workload and launch configuration, every row: the
    selection against the oracle's (band rule) and the attention against
    the oracle over the decode step's own index rows."""
    w = wl.long_context(0)
    banner("decode long_context R=128 L=131072 (full size)")
    idx, out = decode_gpu(w)
    inputs = w.select_inputs()
    want_idx = oracle_select(orc(), inputs)
    check_select_band(idx, want_idx, orc(), inputs, range(w.rows))
    banner(f"rows identical to the oracle: {int(np.all(idx == want_idx, axis=1).sum())}/{w.rows}")
    err = check_attn(out, oracle_attn(orc(), w.q_attn, w.kv, idx, SCALE), "long rows, every row")
    banner(f"attention max abs error {err:.2e} over {w.rows} rows")
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
    want_idx = oracle_select(orc(), inputs)
    check_select_band(idx, want_idx, orc(), inputs, range(w.rows))
    check_attn(out, oracle_attn(orc(), w.q_attn, w.kv, idx, SCALE), "multi-token, every row")


@pytest.mark.parametrize("rows", [1, 2, 23, 24, 40])
def test_small_and_uneven_batches(rows):
    """The first rows of the long-context batch (128K-token rows, N(0,1)),
    each row's selection folded into whole-CU attention workgroups: one row
    (all its workgroups on one XCD, 11 splits of 192 positions), 2 to 23
    rows dealt over the XCDs (11 splits each), 24 and 40 rows (6 splits of
    384; 40 rows do not fill whole groups of 4 rows per XCD).  Every row's
    selection within the band, every row's attention against the oracle
    over the GPU's own index row."""
    w = wl.long_context(0, rows=rows)
    inputs = w.select_inputs()
    banner(f"decode long_context rows={rows}")
    idx, out = decode_gpu(w)
    want_idx = oracle_select(orc(), inputs)
    check_select_band(idx, want_idx, orc(), inputs, range(rows))
    check_attn(out, oracle_attn(orc(), w.q_attn, w.kv, idx, SCALE), f"rows={rows}, every row")


def test_small_batch_over_fused_candidates():
    """Three rows of 262,656 tokens (513 pages each): 17 chunks of 32 pages
    leave 8704 candidates per row, more than an attention workgroup holds,
    so the merge launch selects (two batches of candidates) and 4-wave
    attention workgroups follow, all dealt over the XCDs.  N(0,1) keys of
    the long-context cache behind a seeded page permutation; every row's
    selection within the band, the attention against the oracle."""
    base = wl.long_context(0, rows=3)
    rng = np.random.default_rng(11)
    L, W = 262656, 513
    bt = rng.permutation(base.kcache.shape[0])[:3 * W].astype(np.int32).reshape(3, W)
    t2r, sl, qp = wl.decode_rows([L] * 3)
    kv = wl.normal_f16(rng, (W, wl.TOKENS_PER_PAGE, wl.KV_ROW))
    w = wl.Workload("long_rows_R3_L262656", 0, base.q_sel, base.kcache, bt, t2r, sl, qp,
                    base.q_attn, kv)
    inputs = w.select_inputs()
    banner("decode 3 rows of 262656 tokens (8704 candidates per row)")
    idx, out = decode_gpu(w)
    want_idx = oracle_select(orc(), inputs)
    check_select_band(idx, want_idx, orc(), inputs, range(3))
    check_attn(out, oracle_attn(orc(), w.q_attn, w.kv, idx, SCALE), "long rows, every row")


@pytest.mark.parametrize("rows,lo,hi", [(4096, 0, 1500), (800, 4000, 12000)],
                         ids=["R4096_short", "R800_mid"])
def test_large_batches(rows, lo, hi):
    """Large batches: 4096 short rows (tables of <= 3 pages: one chunk per
    row, no merge) and 800 rows of 4000-12000 tokens (16-page chunks, so the
    rows past 8192 tokens take two and a merge; attention at one split per
    row, no combine).  Integer keys and queries over a shared 2048-page
    cache: the selection bit-exact on every row; the decode step's attention
    against the oracle on sampled rows."""
    rng = np.random.default_rng(rows + lo)
    lengths = rng.integers(lo, hi + 1, size=rows)
    width = max(wl.pages_needed(int(L)) for L in lengths)
    P = 2048
    # integers in [-4, 4] drawn as int8 (a fraction of the int64 draw's time)
    kcache = rng.integers(-4, 5, size=(P, 128, 1, 128), dtype=np.int8).astype(np.float16)
    bt = wl.block_table_per_row(rng, lengths, P, width=width)
    q = wl.int_f16(rng, -4, 4, (rows, 4, 128))
    t2r, sl, qp = wl.decode_rows(lengths)
    kv_pages = -(-int(lengths.max()) // 512) + 1
    kv = wl.normal_f16(rng, (kv_pages, 512, 512))
    q_attn = wl.normal_f16(rng, (rows, 3, 256))
    assert width <= 4 if hi <= 1500 else qsa.select_workspace_bytes(rows, width) > 0
    banner(f"decode large batch R={rows} L=[{lo},{hi}] W={width} "
           f"select ws={qsa.select_workspace_bytes(rows, width)} "
           f"attn ws={qsa.sparse_attn_workspace_bytes(rows)}")
    k, v = qsa.kv_views(dev(kv))
    idx, out = qsa.qsa_decode_step(dev(q), dev(kcache), dev(bt), dev(t2r), dev(sl), dev(qp),
                                   dev(q_attn), k, v, SCALE)
    torch.cuda.synchronize()
    got, out = idx.cpu().numpy(), out.cpu().numpy()
    want = orc().select(q, kcache, bt, t2r, sl, qp)
    bad = np.flatnonzero(~np.all(got == want, axis=1))
    assert bad.size == 0, f"rows differ: {bad[:10]}"
    rows_s = sorted(set(rng.choice(rows, size=12, replace=False).tolist()) | {0, rows - 1})
    check_attn(out[rows_s], orc().sparse_attn(q_attn[rows_s], kv, want[rows_s], SCALE),
               "large batch")
