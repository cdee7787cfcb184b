"""GPU parity of qsa_select (through the C ABI) against the CPU oracle."""

import numpy as np
import pytest
import torch

from paged_top_indexer_amd import workloads as wl
import paged_top_indexer_amd as qsa
from gpu_util import (banner, check_select_band, dev, oracle_select, orc, select_gpu,
                      select_gpu_fp8, subset_rows)

pytestmark = pytest.mark.gpu


def integer_inputs(seed, lengths, width, num_pages, palette=None, q_range=4):
    rng = np.random.default_rng(seed)
    if palette:
        pal = wl.int_f16(rng, -4, 4, (palette, 128))
        kcache = pal[rng.integers(0, palette, size=(num_pages, 128))].reshape(num_pages, 128, 1, 128)
    else:
        kcache = wl.int_f16(rng, -4, 4, (num_pages, 128, 1, 128))
    bt = wl.block_table_per_row(rng, lengths, num_pages, width=width)
    q = wl.int_f16(rng, -q_range, q_range, (len(lengths), 4, 128))
    t2r, sl, qp = wl.decode_rows(lengths)
    return q, kcache, bt, t2r, sl, qp


def test_tiny_integer_bit_exact():
    w = wl.tiny_integer(0)
    banner("select tiny_integer R=1 L=519")
    got = select_gpu(*w.select_inputs())
    want = orc().select(*w.select_inputs())
    assert int((want[0] >= 0).sum()) == 519
    assert np.array_equal(got, want)


def test_ties_and_edges_bit_exact():
    w = wl.ties_and_edges(0)
    banner("select ties_and_edges R=32 palette 64")
    got = select_gpu(*w.select_inputs())
    want = orc().select(*w.select_inputs())
    assert np.array_equal(got, want)


# Plans: (rows, table width) pick the chunk size (1..32 pages, or the whole
# table up to 4 pages); these cover chunks below and above 512 blocks,
# one-chunk rows, multi-chunk merges with ragged last chunks, and few rows
# of a long table (chunks grown until a row's candidates fit one merge
# batch: 16 pages for 5 rows of 256).
PLAN_CASES = [
    (5, 4, [0, 1, 515, 2048, 2047]),  # tables of <= 4 pages: one chunk per row
    (3, 3, [1536, 9, 1100]),
    (1, 20, [9215]),
    (3, 40, [0, 20000, 517]),
    (8, 64, [1, 2, 3, 512, 515, 516, 2049, 32768]),
    (5, 256, [131072, 131071, 70001, 131072, 99999]),
    (64, 256, [70001, 131072, 0, 3, 4096, 2051, 1027, 513] * 8),
    (130, 256, [131071, 65539, 9999, 600, 131072] * 26),
]


@pytest.mark.parametrize("rows,width,lengths", PLAN_CASES,
                         ids=[f"R{c[0]}_W{c[1]}" for c in PLAN_CASES])
@pytest.mark.parametrize("palette", [None, 5], ids=["int4", "palette5"])
def test_integer_plans_bit_exact(rows, width, lengths, palette):
    assert len(lengths) == rows
    pages = max(64, sum(wl.pages_needed(L) for L in lengths) // 4 + 8)
    inputs = integer_inputs(rows * 7 + width, lengths, width, pages, palette=palette,
                            q_range=4 if palette is None else 1)
    banner(f"select integer R={rows} W={width} palette={palette} "
           f"ws={qsa.select_workspace_bytes(rows, width)}")
    got = select_gpu(*inputs)
    want = orc().select(*inputs)
    bad = np.flatnonzero(~np.all(got == want, axis=1))
    assert bad.size == 0, f"rows differ: {bad[:10]}"


@pytest.mark.parametrize("palette", [None, 3], ids=["int4", "palette3"])
def test_very_long_rows_bit_exact(palette):
    """Rows of 2^20 and 1000003 tokens (262144 and 250000 blocks, 2048 table
    entries): two rows get 4-page chunks, 512 per row, so each row's merge
    takes up to 262144 candidates in 32 batches; with a 3-key palette almost
    every score ties and block order decides.  The same rows also through
    the e4m3 cache and with signed integer head weights."""
    lengths = [1 << 20, 1000003]
    inputs = integer_inputs(77 if palette is None else 78, lengths, 2048, 2048, palette=palette,
                            q_range=4 if palette is None else 1)
    banner(f"select very long rows L={lengths} palette={palette}")
    got = select_gpu(*inputs)
    want = orc().select(*inputs)
    assert np.array_equal(got, want)
    # the same rows through the e4m3 cache (integer keys re-encoded exactly)
    # and with signed integer head weights
    q, kcache, bt, t2r, sl, qp = inputs
    rng = np.random.default_rng(79)
    codes, scales = wl.fp8_integer_keys(rng, kcache)
    assert np.array_equal(select_gpu_fp8(q, codes, scales, bt, t2r, sl, qp), want)
    w = wl.head_weights(rng, len(lengths), integer=True)
    got_w = qsa.qsa_select_weighted(dev(q), dev(w), dev(kcache), dev(bt), dev(t2r), dev(sl),
                                    dev(qp))
    torch.cuda.synchronize()
    want_w = orc().select_weighted(q, w, bt, t2r, sl, qp, kcache=kcache)
    assert np.array_equal(got_w.cpu().numpy(), want_w)


def test_invalid_page_ids_read_as_zero_keys():
    """Table entries outside [0, P) for visible blocks (an unmet device-side
    precondition): the kernels stay in bounds and read such a page as
    all-zero keys (score 0), so the result equals the oracle's with those
    entries pointed at an appended all-zero page -- fp16 and e4m3 caches."""
    rng = np.random.default_rng(31)
    P = 48
    kcache = wl.int_f16(rng, -4, 4, (P, 128, 1, 128))
    lengths = [9000, 20000, 3000]
    bt = wl.block_table_per_row(rng, lengths, P, width=40)
    bad = [(0, 3, -1), (1, 0, P), (1, 17, P + 1000), (2, 5, -7)]
    bt_gpu, bt_orc = bt.copy(), bt.copy()
    for i, j, val in bad:
        assert bt[i, j] >= 0  # a visible block's entry
        bt_gpu[i, j] = val
        bt_orc[i, j] = P
    q = wl.int_f16(rng, -4, 4, (3, 4, 128))
    t2r, sl, qp = wl.decode_rows(lengths)
    banner("select with table entries outside [0, P)")
    got = select_gpu(q, kcache, bt_gpu, t2r, sl, qp)
    kz = np.concatenate([kcache, np.zeros((1, 128, 1, 128), np.float16)])
    want = orc().select(q, kz, bt_orc, t2r, sl, qp)
    assert np.array_equal(got, want)
    codes, scales = wl.fp8_integer_keys(rng, kcache)
    got8 = select_gpu_fp8(q, codes, scales, bt_gpu, t2r, sl, qp)
    cz = np.concatenate([codes, np.zeros((1, 128, 1, 128), np.uint8)])
    sz = np.concatenate([scales, np.ones((1, 128), np.float32)])
    assert np.array_equal(got8, orc().select_fp8(q, cz, sz, bt_orc, t2r, sl, qp))


def test_multirow_requests_and_padding():
    """Several query rows of one request (prefill-style positions), a padded
    row (position -1), an out-of-range request id (treated as empty)."""
    rng = np.random.default_rng(21)
    kcache = wl.int_f16(rng, -4, 4, (64, 128, 1, 128))
    lengths = [9000, 700]
    bt = wl.block_table_per_row(rng, lengths, 64, width=24)
    t2r = np.array([0, 0, 0, 1, 1, 0], dtype=np.int32)
    qp = np.array([8999, 2050, 13, 699, 515, -1], dtype=np.int64)
    sl = np.array(lengths, dtype=np.int32)
    q = wl.int_f16(rng, -3, 3, (6, 4, 128))
    banner("select multi-row requests")
    got = select_gpu(q, kcache, bt, t2r, sl, qp)
    want = orc().select(q, kcache, bt, t2r, sl, qp)
    assert np.array_equal(got, want)


def test_shared_physical_pages():
    """Two requests whose tables map the same physical pages: same keys,
    same scores, same selection."""
    rng = np.random.default_rng(22)
    kcache = wl.int_f16(rng, -4, 4, (32, 128, 1, 128))
    pages = rng.permutation(32)[:10].astype(np.int32)
    bt = np.stack([pages, pages])
    t2r, sl, qp = wl.decode_rows([5000, 5000])
    q = wl.int_f16(rng, -4, 4, (1, 4, 128)).repeat(2, axis=0)
    banner("select shared physical pages")
    got = select_gpu(q, kcache, bt, t2r, sl, qp)
    assert np.array_equal(got[0], got[1])
    assert np.array_equal(got, orc().select(q, kcache, bt, t2r, sl, qp))


def test_saturated_row_band():
    w = wl.saturated_row(0)
    banner("select saturated_row R=1 L=9215 P=8192")
    inputs = w.select_inputs()
    got = select_gpu(*inputs)
    want = orc().select(*inputs)
    assert int((got[0] >= 0).sum()) == 2051
    check_select_band(got, want, orc(), inputs, [0])


def test_batched_shared_band():
    w = wl.batched_shared(0)
    banner("select batched_shared R=64")
    inputs = w.select_inputs()
    got = select_gpu(*inputs)
    want = orc().select(*inputs)
    check_select_band(got, want, orc(), inputs, range(w.rows))
    exact = np.mean(np.all(got == want, axis=1))
    banner(f"rows identical to the oracle: {exact:.3f}")


@pytest.fixture(scope="module")
def long_context():
    return wl.long_context(0)


def test_long_context_full_size(long_context):
    """The full R=128, L=131072 batch in the bench's launch configuration:
    every row against the oracle (band rule), plus the structure of every
    row."""
    w = long_context
    inputs = w.select_inputs()
    banner("select long_context R=128 L=131072 (full size)")
    got = select_gpu(*inputs)
    want = oracle_select(orc(), inputs)
    check_select_band(got, want, orc(), inputs, range(w.rows))
    banner(f"rows identical to the oracle: {int(np.all(got == want, axis=1).sum())}/{w.rows}")
    for r in range(w.rows):
        g = got[r]
        assert np.all(g[2048:] == -1)  # L % 4 == 0: no tail
        b = g[:2048:4] // 4
        assert len(np.unique(b)) == 512 and b.min() >= 0 and b.max() < 32768
        assert np.array_equal(g[:2048].reshape(512, 4), (4 * b)[:, None] + np.arange(4))


def test_deterministic_repeats():
    """Merges race-free: repeated launches give identical bytes."""
    lengths = [70001, 131072, 0, 3, 4096, 2051, 1027, 513] * 8
    inputs = integer_inputs(5, lengths, 256, 1200, palette=3, q_range=1)
    d = [dev(a) for a in inputs]
    out = torch.empty((len(lengths), 2051), dtype=torch.int32, device=d[0].device)
    banner("select determinism x100")
    ref = None
    for i in range(100):
        out.fill_(-7)
        qsa.qsa_select(*d, out=out)
        got = out.cpu().numpy()
        if ref is None:
            ref = got
        assert np.array_equal(got, ref), f"repeat {i} differs"
    assert np.array_equal(ref, orc().select(*inputs))


def test_inputs_unchanged_and_zero_rows():
    w = wl.tiny_integer(0)
    d = [dev(a) for a in w.select_inputs()]
    before = [t.clone() for t in d]
    qsa.qsa_select(*d)
    torch.cuda.synchronize()
    for a, b in zip(d, before):
        assert torch.equal(a, b)
    empty = qsa.qsa_select(d[0][:0], d[1], d[2], d[3][:0], d[4], d[5][:0])
    assert empty.shape == (0, 2051)


def test_fail_closed_leaves_output_untouched():
    w = wl.tiny_integer(0)
    d = [dev(a) for a in w.select_inputs()]
    out = torch.full((1, 2051), 12345, dtype=torch.int32, device=d[0].device)
    with pytest.raises(RuntimeError, match="QSA_ERR_DTYPE"):
        qsa.qsa_select(d[0].float(), *d[1:], out=out)
    with pytest.raises(RuntimeError, match="QSA_ERR_SHAPE"):
        qsa.qsa_select(*d, out=torch.empty((1, 2048), dtype=torch.int32, device=d[0].device))
    torch.cuda.synchronize()
    assert torch.all(out == 12345)


@pytest.mark.parametrize("integer", [True, False], ids=["int", "normal"])
def test_multi_token_rows(integer):
    """Speculative-decode (4 draft positions per request) and chunked-prefill
    (16 positions) rows: each row's visible blocks and tail follow its own
    query position."""
    w = wl.multi_token_rows(0, integer=integer)
    inputs = w.select_inputs()
    banner(f"select {w.name}")
    got = select_gpu(*inputs)
    want = orc().select(*inputs)
    if integer:
        bad = np.flatnonzero(~np.all(got == want, axis=1))
        assert bad.size == 0, f"rows differ: {bad[:10]}"
    else:
        check_select_band(got, want, orc(), inputs, range(w.rows))
    # rows of one request differ only through their positions: tails shift
    widths = (got >= 0).sum(axis=1)
    for r in range(w.rows):
        V, T = orc().row_extent(int(w.seq_lens[w.token_to_req[r]]), int(w.query_pos[r]))
        assert widths[r] == min(2048, 4 * V) + T
