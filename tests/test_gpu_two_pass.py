"""GPU parity of the per-head-weight and two-pass entry points
(qsa_select_weighted, qsa_paged_logits, qsa_topk_per_row) against the CPU
oracle, and of the two passes composed against the fused selection."""

import numpy as np
import pytest
import torch

from paged_top_indexer_amd import workloads as wl
import paged_top_indexer_amd as qsa
from gpu_util import banner, check_select_band, dev, dev_e4m3, orc, subset_rows
from oracle.acceptance import map_rows
from test_gpu_select import PLAN_CASES, integer_inputs

pytestmark = pytest.mark.gpu


def weighted_gpu(q, w, bt, t2r, sl, qp, kcache=None, codes=None, scales=None):
    if codes is not None:
        out = qsa.qsa_select_weighted(dev(q), dev(w), dev_e4m3(codes), dev(bt), dev(t2r), dev(sl),
                                      dev(qp), kscale=dev(scales))
    else:
        out = qsa.qsa_select_weighted(dev(q), dev(w), dev(kcache), dev(bt), dev(t2r), dev(sl),
                                      dev(qp))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def logits_gpu(q, bt, t2r, sl, qp, w=None, kcache=None, codes=None, scales=None, width=None):
    kc = dev_e4m3(codes) if codes is not None else dev(kcache)
    lg = qsa.qsa_paged_logits(dev(q), kc, dev(bt), dev(t2r), dev(sl), dev(qp),
                              weights=None if w is None else dev(w),
                              kscale=None if scales is None else dev(scales), width=width)
    torch.cuda.synchronize()
    return lg.cpu().numpy()


@pytest.mark.parametrize("rows,width,lengths", PLAN_CASES,
                         ids=[f"R{c[0]}_W{c[1]}" for c in PLAN_CASES])
def test_weighted_integer_bit_exact(rows, width, lengths):
    """Integer keys, queries and head weights in [-3, 3]: every fp32 sum is
    exact, so the weighted selection is the oracle's exactly (fp16 and e4m3
    caches)."""
    pages = max(64, sum(wl.pages_needed(L) for L in lengths) // 4 + 8)
    q, kcache, bt, t2r, sl, qp = integer_inputs(rows * 11 + width, lengths, width, pages,
                                                palette=5, q_range=2)
    rng = np.random.default_rng(rows + 3 * width)
    w = wl.head_weights(rng, rows, integer=True)
    banner(f"select_weighted integer R={rows} W={width}")
    want = orc().select_weighted(q, w, bt, t2r, sl, qp, kcache=kcache)
    got = weighted_gpu(q, w, bt, t2r, sl, qp, kcache=kcache)
    bad = np.flatnonzero(~np.all(got == want, axis=1))
    assert bad.size == 0, f"rows differ: {bad[:10]}"
    codes, scales = wl.fp8_integer_keys(rng, kcache)
    got8 = weighted_gpu(q, w, bt, t2r, sl, qp, codes=codes, scales=scales)
    assert np.array_equal(got8, want)


def test_weighted_normal_band():
    w_ = wl.batched_shared(0)
    q, kcache, bt, t2r, sl, qp = w_.select_inputs()
    w = wl.head_weights(np.random.default_rng(7), w_.rows)
    banner("select_weighted batched_shared R=64")
    got = weighted_gpu(q, w, bt, t2r, sl, qp, kcache=kcache)
    want = orc().select_weighted(q, w, bt, t2r, sl, qp, kcache=kcache)
    width = bt.shape[1] * 128
    lg = orc().paged_logits(q, w, bt, t2r, sl, qp, width, kcache=kcache)
    V = [orc().row_extent(int(sl[t2r[r]]), int(qp[r]))[0] for r in range(w_.rows)]
    check_select_band(got, want, orc(), w_.select_inputs(), range(w_.rows),
                      row_scores=lambda r: lg[r, :V[r]])


def test_paged_logits_integer_exact():
    """Exact fp32 logits on integer inputs, -inf past V, a logits width
    beyond the table's and rows of a strided (wider) buffer."""
    lengths = [70001, 131072, 0, 3, 4096, 2051, 1027, 513]
    q, kcache, bt, t2r, sl, qp = integer_inputs(9, lengths, 256, 900, palette=None, q_range=2)
    w = wl.head_weights(np.random.default_rng(9), len(lengths), integer=True)
    width = 256 * 128 + 300
    banner("paged_logits integer R=8")
    for weights in (None, w):
        want = orc().paged_logits(q, weights, bt, t2r, sl, qp, width, kcache=kcache)
        got = logits_gpu(q, bt, t2r, sl, qp, w=weights, kcache=kcache, width=width)
        assert np.array_equal(got, want)
    # the same through an e4m3 cache holding the same keys
    codes, scales = wl.fp8_integer_keys(np.random.default_rng(10), kcache)
    got8 = logits_gpu(q, bt, t2r, sl, qp, w=w, codes=codes, scales=scales, width=width)
    assert np.array_equal(got8, want)
    # rows of a wider buffer (row stride > width): the gap stays untouched
    buf = torch.full((len(lengths), width + 64), 7.0, dtype=torch.float32, device="cuda:0")
    view = buf[:, :width]
    qsa.qsa_paged_logits(dev(q), dev(kcache), dev(bt), dev(t2r), dev(sl), dev(qp),
                         weights=dev(w), logits=view)
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert np.array_equal(b[:, :width], want)
    assert np.all(b[:, width:] == 7.0)


def test_paged_logits_normal_close():
    w_ = wl.saturated_row(0)
    q, kcache, bt, t2r, sl, qp = w_.select_inputs()
    w = wl.head_weights(np.random.default_rng(11), 1)
    width = bt.shape[1] * 128
    banner("paged_logits saturated_row")
    want = orc().paged_logits(q, w, bt, t2r, sl, qp, width, kcache=kcache)
    got = logits_gpu(q, bt, t2r, sl, qp, w=w, kcache=kcache)
    V = 2303
    assert np.all(np.isneginf(got[0, V:]))
    assert np.allclose(got[0, :V], want[0, :V], rtol=1e-4, atol=1e-3)


def random_logits(seed, rows, width):
    """Coarse-grid normal logits (many exact ties), signed zeros, some -inf."""
    rng = np.random.default_rng(seed)
    lg = (np.round(rng.normal(size=(rows, width)) * 8) / 8).astype(np.float32)
    z = rng.random(lg.shape) < 0.05
    lg[z] = np.where(rng.random(z.sum()) < 0.5, 0.0, -0.0)
    lg[rng.random(lg.shape) < 0.01] = -np.inf
    return lg


@pytest.mark.parametrize("rows,width", [(1, 600), (7, 5000), (3, 32768), (2, 32769),
                                        (64, 33000), (130, 9000)])
def test_topk_per_row_exact(rows, width):
    """Given logits, the selection is exact (no arithmetic): ties, signed
    zeros, -inf, junk past each row's visible blocks, rows shorter and longer
    than 512 blocks, multi-row requests.  Up to 32768 columns one workgroup
    selects a whole row; wider rows go through chunks and a merge."""
    rng = np.random.default_rng(rows + width)
    lg = random_logits(rows * 3 + width, rows, width)
    nreq = max(1, rows // 2)
    t2r = rng.integers(0, nreq, size=rows).astype(np.int32)
    sl = rng.integers(0, 4 * width + 1, size=nreq).astype(np.int32)
    qp = np.array([rng.integers(-1, max(0, int(sl[t])) + 1) for t in t2r], np.int64)
    qp = np.minimum(qp, 4 * width - 1)
    for r in range(rows):
        V, _ = orc().row_extent(int(sl[t2r[r]]), int(qp[r]))
        lg[r, V:] = 1e30
    banner(f"topk_per_row R={rows} Wl={width}")
    want = orc().topk_per_row(lg, t2r, sl, qp)
    got = qsa.qsa_topk_per_row(dev(lg), dev(t2r), dev(sl), dev(qp))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), want)


def test_two_pass_equals_fused_full_size():
    """At the long-context shape (R=128, 32768 blocks per row) with head
    weights: paged logits then top-k per row give exactly the fused
    weighted selection (the same scorer computes the same fp32 values), and
    every row satisfies the band rule against the oracle's weighted
    selection."""
    w_ = wl.long_context(0)
    inputs = w_.select_inputs()
    q, kcache, bt, t2r, sl, qp = inputs
    w = wl.head_weights(np.random.default_rng(12), w_.rows)
    d = [dev(a) for a in inputs]
    wd = dev(w)
    banner("two-pass vs fused, long_context R=128 L=131072 with weights")
    fused = qsa.qsa_select_weighted(d[0], wd, *d[1:])
    lg = qsa.qsa_paged_logits(*d, weights=wd)
    two = qsa.qsa_topk_per_row(lg, d[3], d[4], d[5])
    torch.cuda.synchronize()
    fused, two, lgh = fused.cpu().numpy(), two.cpu().numpy(), lg.cpu().numpy()
    assert np.array_equal(fused, two)
    R = w_.rows

    def sub(rs):
        return subset_rows(inputs, rs)

    want = map_rows(lambda rs: orc().select_weighted(sub(rs)[0], w[rs], *sub(rs)[2:],
                                                     kcache=kcache), range(R))
    wl_or = map_rows(lambda rs: orc().paged_logits(sub(rs)[0], w[rs], *sub(rs)[2:], 32768,
                                                   kcache=kcache), range(R))
    check_select_band(two, want, orc(), inputs, range(R), row_scores=lambda i: wl_or[i])
    assert np.allclose(lgh, wl_or, rtol=1e-4, atol=1e-3)
    # the top-k of the oracle's own logits is the oracle's weighted selection
    rows = [0, 77, 127]
    assert np.array_equal(orc().topk_per_row(wl_or[rows], *sub(rows)[3:]), want[rows])


def test_fail_closed_through_binding():
    w_ = wl.tiny_integer(0)
    q, kcache, bt, t2r, sl, qp = [dev(a) for a in w_.select_inputs()]
    with pytest.raises(RuntimeError, match="QSA_ERR_SHAPE"):
        qsa.qsa_paged_logits(q, kcache, bt, t2r, sl, qp, width=100)
    with pytest.raises(RuntimeError, match="QSA_ERR_DTYPE"):
        qsa.qsa_select_weighted(q, torch.ones((1, 4), dtype=torch.float16, device=q.device),
                                kcache, bt, t2r, sl, qp)
    with pytest.raises(RuntimeError, match="QSA_ERR_DTYPE"):
        qsa.qsa_topk_per_row(torch.zeros((1, 600), dtype=torch.float16, device=q.device), t2r, sl, qp)
