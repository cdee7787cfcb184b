"""GPU parity of qsa_sparse_attn (through the C ABI) against the float64
CPU oracle: max abs error <= 2e-3 and <= 1 fp16 ulp."""

import numpy as np
import pytest
import torch

from paged_top_indexer_amd import workloads as wl
import paged_top_indexer_amd as qsa
from gpu_util import attn_gpu, banner, check_attn, dev, orc

pytestmark = pytest.mark.gpu
SCALE = wl.SOFTMAX_SCALE


def test_tiny_integer_on_oracle_selection():
    w = wl.tiny_integer(0)
    idx = orc().select(*w.select_inputs())
    banner("attn tiny_integer width 519")
    got = attn_gpu(w.q_attn, w.kv, idx, SCALE)
    check_attn(got, orc().sparse_attn(w.q_attn, w.kv, idx, SCALE), "tiny")


def test_saturated_row_holes_duplicates():
    w = wl.saturated_row(0)
    sel = orc().select(*w.select_inputs())
    pert = w.notes["attn_perturb"]
    idx = wl.inject_holes_and_duplicates(np.random.default_rng(pert["seed"]), sel,
                                         pert["hole_frac"], pert["dup_frac"])
    assert (idx == -1).sum() > 100
    banner("attn saturated_row with 5% holes / 5% duplicates")
    got = attn_gpu(w.q_attn, w.kv, idx, SCALE)
    check_attn(got, orc().sparse_attn(w.q_attn, w.kv, idx, SCALE), "saturated")


def test_ties_and_edges_rows():
    w = wl.ties_and_edges(0)
    sel = orc().select(*w.select_inputs())
    pert = w.notes["attn_perturb"]
    idx = wl.inject_holes_and_duplicates(np.random.default_rng(pert["seed"]), sel,
                                         pert["hole_frac"], pert["dup_frac"])
    idx = np.concatenate([idx, w.notes["attn_extra_rows"]])
    banner("attn ties_and_edges (35 rows incl. empty / single / repeated)")
    got = attn_gpu(w.attn_q, w.kv, idx, SCALE)
    want = orc().sparse_attn(w.attn_q, w.kv, idx, SCALE)
    check_attn(got, want, "edges")
    assert np.all(got[32] == 0)  # all holes -> zeros
    v_single = w.kv.reshape(-1, 512)[idx[33][idx[33] >= 0][0], 256:]
    assert np.array_equal(got[33], np.broadcast_to(v_single, (3, 256)))
    v_rep = w.kv.reshape(-1, 512)[idx[34, 0], 256:]
    assert np.array_equal(got[34], np.broadcast_to(v_rep, (3, 256)))


NAMED = ["empty", "holes_dups_crosspage", "width32", "width2051"]


@pytest.mark.parametrize("rows", [1, 2])
@pytest.mark.parametrize("case", NAMED)
def test_named_cases(rows, case):
    """The attention cases the page lists for R in {1, 2}."""
    rng = np.random.default_rng(100 * rows + NAMED.index(case))
    pages = 6
    kv = wl.normal_f16(rng, (pages, 512, 512))
    q = wl.normal_f16(rng, (rows, 3, 256))
    NT = pages * 512
    if case == "empty":
        idx = np.full((rows, 2051), -1, np.int32)
    elif case == "holes_dups_crosspage":
        idx = wl.random_index_rows(rng, rows, NT, valid=2051, distinct=False)
        idx = wl.inject_holes_and_duplicates(rng, idx, 0.2, 0.2)
    elif case == "width32":
        idx = wl.random_index_rows(rng, rows, NT, valid=32)
    else:
        idx = wl.random_index_rows(rng, rows, NT, valid=2051)
    banner(f"attn R={rows} {case}")
    got = attn_gpu(q, kv, idx, SCALE)
    check_attn(got, orc().sparse_attn(q, kv, idx, SCALE), case)
    if case == "empty":
        assert np.all(got == 0)


def test_sharp_softmax_and_large_scale():
    """A large scale makes the softmax nearly one-hot: the online max/rescale
    path across tiles, waves and splits must keep it exact."""
    rng = np.random.default_rng(31)
    kv = wl.normal_f16(rng, (8, 512, 512))
    q = wl.normal_f16(rng, (4, 3, 256))
    idx = wl.random_index_rows(rng, 4, 8 * 512, valid=2051)
    banner("attn sharp softmax (scale 0.5)")
    got = attn_gpu(q, kv, idx, 0.5)
    check_attn(got, orc().sparse_attn(q, kv, idx, 0.5), "sharp")


def test_long_context_full_size_standalone():
    """All 128 rows of the R=128 batch with 2051 distinct valid indices each."""
    w = wl.long_context(0)
    banner("attn long_context R=128 full width 2051")
    got = attn_gpu(w.attn_q, w.kv, w.attn_indices, SCALE)
    check_attn(got, orc().sparse_attn(w.attn_q, w.kv, w.attn_indices, SCALE), "long")


def test_out_of_range_index_is_a_hole():
    rng = np.random.default_rng(33)
    kv = wl.normal_f16(rng, (2, 512, 512))
    q = wl.normal_f16(rng, (1, 3, 256))
    idx = wl.random_index_rows(rng, 1, 1024, valid=100)
    bad = idx.copy()
    bad[0, 100:110] = 1024 + np.arange(10)  # beyond the cache: must read nothing
    bad[0, 110] = -5
    got = attn_gpu(q, kv, bad, SCALE)
    check_attn(got, orc().sparse_attn(q, kv, idx, SCALE), "oob-as-hole")


def test_inputs_unchanged_and_fail_closed():
    rng = np.random.default_rng(34)
    kv = dev(wl.normal_f16(rng, (2, 512, 512)))
    q = dev(wl.normal_f16(rng, (2, 3, 256)))
    idx = dev(wl.random_index_rows(rng, 2, 1024, valid=500))
    before = [t.clone() for t in (kv, q, idx)]
    k, v = qsa.kv_views(kv)
    qsa.qsa_sparse_attn(q, k, v, idx, SCALE)
    torch.cuda.synchronize()
    for a, b in zip((kv, q, idx), before):
        assert torch.equal(a, b)
    out = torch.full((2, 3, 256), 7.0, dtype=torch.float16, device=q.device)
    with pytest.raises(RuntimeError, match="QSA_ERR_LAYOUT"):
        qsa.qsa_sparse_attn(q, k, k, idx, SCALE, out=out)  # V not at +256
    with pytest.raises(RuntimeError, match="QSA_ERR_ARG"):
        qsa.qsa_sparse_attn(q, k, v, idx, 0.0, out=out)
    with pytest.raises(RuntimeError, match="QSA_ERR_DTYPE"):
        qsa.qsa_sparse_attn(q.float(), k, v, idx, SCALE, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


# Batch sizes across the split plans and workgroup placements: 4-wave
# workgroups below 8 rows (33 splits of 64 positions, fewer and longer as
# rows grow) and from 257 rows up (one split per row, no combine, from 768
# rows); 12-wave workgroups from 8 to 256 rows (11 splits of 192 positions
# up to 23 rows, 6 of 384 at 24 rows, 4 at 64, one per row at 256).  One row
# sits on one XCD; larger batches are dealt over the XCDs row by row.
SPLIT_BATCHES = [1, 2, 3, 5, 7, 8, 16, 23, 24, 33, 64, 100, 256, 300, 767, 768, 900]


@pytest.mark.parametrize("rows", SPLIT_BATCHES)
def test_split_plans(rows):
    """Random index rows (valid widths from 0 to 2051, holes, repeats, a few
    out-of-range entries treated as holes) over a 64-page cache."""
    rng = np.random.default_rng(77 + rows)
    pages = 64
    kv = wl.normal_f16(rng, (pages, 512, 512))
    q = wl.normal_f16(rng, (rows, 3, 256))
    idx = np.full((rows, 2051), -1, dtype=np.int32)
    widths = rng.integers(0, 2052, size=rows)
    widths[rng.random(rows) < 0.3] = 2051
    for r in range(rows):
        idx[r, :widths[r]] = rng.integers(0, pages * 512, size=widths[r])
    holes = rng.random(idx.shape) < 0.05
    idx[holes] = -1
    repeat = (rng.random(idx.shape) < 0.05) & (idx >= 0)
    idx[repeat] = idx[repeat][::-1]  # repeats of other valid entries
    oob = rng.random(idx.shape) < 0.002
    idx[oob] = pages * 512 + 7  # past the cache: a hole
    banner(f"attn split plan rows={rows} workspace={qsa.sparse_attn_workspace_bytes(rows)}")
    got = attn_gpu(q, kv, idx, SCALE)
    ref_idx = np.where(idx < pages * 512, idx, -1).astype(np.int32)
    check_attn(got, orc().sparse_attn(q, kv, ref_idx, SCALE), f"rows={rows}")
