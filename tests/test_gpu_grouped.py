"""GPU parity of the selection family when the queries come in runs of
next_n rows of one request (q given as [B, n, 4, 128]): up to four rows are
scored against one read of their request's keys.  The grouping changes the
work, never the result: integer inputs must match the oracle bit for bit,
N(0,1) inputs follow the band rule, also when a run spans several requests,
holds padded or empty rows, or ends in a partial group."""

import numpy as np
import pytest
import torch

from paged_top_indexer_amd import workloads as wl
import paged_top_indexer_amd as qsa
from gpu_util import (banner, check_attn, check_select_band, dev, dev_e4m3, oracle_attn,
                      orc)

pytestmark = pytest.mark.gpu

SCALE = 1.0 / 16.0


def runs(q: np.ndarray, n: int) -> torch.Tensor:
    """q [R,4,128] on the device as [R/n, n, 4, 128]."""
    assert q.shape[0] % n == 0
    return dev(q).view(q.shape[0] // n, n, 4, 128)


def request_rows(seed, rows_per_req, lengths, num_pages, width=None, palette=None):
    """Integer inputs whose requests own consecutive rows (the last
    rows_per_req[i] positions of request i), as speculative-decode and
    chunked-prefill batches lay them out."""
    rng = np.random.default_rng(seed)
    if palette:
        pal = wl.int_f16(rng, -4, 4, (palette, 128))
        kcache = pal[rng.integers(0, palette, size=(num_pages, 128))].reshape(num_pages, 128, 1, 128)
    else:
        kcache = wl.int_f16(rng, -4, 4, (num_pages, 128, 1, 128))
    bt = wl.block_table_per_row(rng, lengths, num_pages, width=width)
    t2r = np.concatenate([np.full(c, i, np.int32) for i, c in enumerate(rows_per_req)])
    qp = np.concatenate([int(L) - c + np.arange(c) for L, c in zip(lengths, rows_per_req)])
    q = wl.int_f16(rng, -4 if palette is None else -1, 4 if palette is None else 1,
                   (t2r.size, 4, 128))
    return q, kcache, bt, t2r, np.asarray(lengths, np.int32), qp.astype(np.int64)


def select_runs(inputs, n):
    q, kcache, bt, t2r, sl, qp = inputs
    out = qsa.qsa_select(runs(q, n), dev(kcache), dev(bt), dev(t2r), dev(sl), dev(qp))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def assert_rows_equal(got, want):
    bad = np.flatnonzero(~np.all(got == want, axis=1))
    assert bad.size == 0, f"rows differ: {bad[:10]}"


# (rows per request, lengths, run lengths n to try).  Aligned runs of 4;
# runs that straddle requests; R not a multiple of 4 (a partial last
# group); rows of 1..1024 visible blocks (one chunk, sorted in the chunk
# kernel) next to rows of many chunks.
RUN_CASES = [
    ([4] * 12, [600, 2051, 4100, 9000, 17000, 33000, 40000, 5, 1, 0, 70001, 131072], [4, 2]),
    ([3, 5, 1, 7, 4, 2, 6], [9215, 5000, 130000, 2049, 519, 65536, 30001], [4, 7, 2, 14]),
    ([16, 16], [20000, 4096], [4, 16, 8]),
    ([5, 3, 7], [3000, 100000, 12345], [3, 5]),
]


@pytest.mark.parametrize("case", range(len(RUN_CASES)))
@pytest.mark.parametrize("palette", [None, 5], ids=["int4", "palette5"])
def test_runs_integer_bit_exact(case, palette):
    rows_per_req, lengths, ns = RUN_CASES[case]
    pages = max(64, sum(wl.pages_needed(L) for L in lengths) + 8)
    inputs = request_rows(case * 31 + 7, rows_per_req, lengths, pages, palette=palette)
    want = orc().select(*inputs)
    for n in ns:
        banner(f"select runs case={case} n={n} R={inputs[0].shape[0]} palette={palette}")
        assert_rows_equal(select_runs(inputs, n), want)


def test_runs_with_padded_and_empty_rows():
    """Padded rows (position -1) and rows of an out-of-range request inside
    runs: they come out all -1 and do not disturb their neighbours."""
    q, kcache, bt, t2r, sl, qp = request_rows(5, [4, 4, 4, 4], [9000, 600, 70000, 2000], 256)
    qp[[1, 2, 6, 9, 15]] = -1
    want = orc().select(q, kcache, bt, t2r, sl, qp)
    assert np.all(want[[1, 2, 6, 9, 15]] == -1)
    # the kernels treat a request id outside [0, N) as an empty row (the
    # oracle refuses it, so it is asked about the equivalent padded row)
    t2r_bad = t2r.copy()
    t2r_bad[[2, 9]] = 57
    banner("select runs with padded and empty rows")
    assert_rows_equal(select_runs((q, kcache, bt, t2r_bad, sl, qp), 4), want)


def test_runs_fp8_and_weighted_integer():
    """e4m3 keys (integer-valued dequantized keys) and integer per-head
    weights through the grouped scorers."""
    rows_per_req, lengths, _ = RUN_CASES[1]
    pages = sum(wl.pages_needed(L) for L in lengths) + 8
    q, kcache, bt, t2r, sl, qp = request_rows(99, rows_per_req, lengths, pages, palette=5)
    rng = np.random.default_rng(4)
    codes, scales = wl.fp8_integer_keys(rng, kcache)
    want = orc().select(q, kcache, bt, t2r, sl, qp)
    banner("select_fp8 runs n=4")
    got = qsa.qsa_select_fp8(runs(q, 4), dev_e4m3(codes), dev(scales), dev(bt), dev(t2r),
                             dev(sl), dev(qp))
    torch.cuda.synchronize()
    assert_rows_equal(got.cpu().numpy(), want)
    w = wl.head_weights(rng, q.shape[0], integer=True)
    want_w = orc().select_weighted(q, w, bt, t2r, sl, qp, kcache=kcache)
    for n, kc, ks in [(4, dev(kcache), None), (2, dev_e4m3(codes), dev(scales))]:
        banner(f"select_weighted runs n={n} e4m3={ks is not None}")
        got = qsa.qsa_select_weighted(runs(q, n), dev(w), kc, dev(bt), dev(t2r), dev(sl), dev(qp),
                                      kscale=ks)
        torch.cuda.synchronize()
        assert_rows_equal(got.cpu().numpy(), want_w)


def test_runs_paged_logits():
    """Grouped paged logits: the same matrix as row by row (exact on
    integer inputs), -inf past each row's visible blocks."""
    rows_per_req, lengths, _ = RUN_CASES[0]
    pages = sum(wl.pages_needed(L) for L in lengths) + 8
    q, kcache, bt, t2r, sl, qp = request_rows(3, rows_per_req, lengths, pages)
    banner("paged_logits runs n=4")
    flat = qsa.qsa_paged_logits(dev(q), dev(kcache), dev(bt), dev(t2r), dev(sl), dev(qp))
    grouped = qsa.qsa_paged_logits(runs(q, 4), dev(kcache), dev(bt), dev(t2r), dev(sl), dev(qp))
    torch.cuda.synchronize()
    flat, grouped = flat.cpu().numpy(), grouped.cpu().numpy()
    assert np.array_equal(flat, grouped)
    width = flat.shape[1]
    want = orc().paged_logits(q, None, bt, t2r, sl, qp, width, kcache=kcache)
    assert np.array_equal(grouped, want.astype(np.float32))


@pytest.fixture(scope="module")
def multi_token():
    return wl.multi_token_rows(0)


def test_multi_token_normal_band(multi_token):
    """The multi-token workload (48 speculative-decode requests x 4 rows,
    4 chunked-prefill requests x 16 rows) grouped in runs of 4."""
    w = multi_token
    inputs = w.select_inputs()
    banner(f"select runs {w.name}")
    got = select_runs(inputs, 4)
    want = orc().select(*inputs)
    check_select_band(got, want, orc(), inputs, range(w.rows))
    flat = qsa.qsa_select(*[dev(x) for x in inputs])
    torch.cuda.synchronize()
    same = int(np.all(got == flat.cpu().numpy(), axis=1).sum())
    print(f"[gpu] grouped == row-by-row on {same}/{w.rows} rows", flush=True)


def test_multi_token_decode_step(multi_token):
    """qsa_decode_step with grouped queries: selection within the band,
    attention against the oracle over the step's own index rows."""
    w = multi_token
    inputs = w.select_inputs()
    kvd = dev(w.kv)
    k, v = qsa.kv_views(kvd)
    q, kcache, bt, t2r, sl, qp = inputs
    banner(f"decode runs {w.name}")
    idx, out = qsa.qsa_decode_step(runs(q, 4), dev(kcache), dev(bt), dev(t2r), dev(sl), dev(qp),
                                   dev(w.q_attn), k, v, SCALE)
    torch.cuda.synchronize()
    idx, out = idx.cpu().numpy(), out.cpu().numpy()
    want_idx = orc().select(*inputs)
    check_select_band(idx, want_idx, orc(), inputs, range(w.rows))
    check_attn(out, oracle_attn(orc(), w.q_attn, w.kv, idx, SCALE),
               "grouped multi-token rows, every row")


def test_runs_full_size_chunks_integer():
    """A batch large enough for the grouped plan's full chunks (8 pages =
    1024 blocks): 64 groups of 4 rows.  One prefill run crosses the chunk
    boundary (V = 1023..1027), so a group mixes rows finished in the chunk
    kernel with rows merged later; fp16 keys, e4m3 keys and per-head
    weights, bit-exact."""
    rng = np.random.default_rng(123)
    rows_per_req = [16] + [4] * 60
    lengths = [4108] + list(rng.integers(4000, 65536, size=59)) + [65536]
    pages = sum(wl.pages_needed(L) for L in lengths) + 8
    q, kcache, bt, t2r, sl, qp = request_rows(17, rows_per_req, lengths, pages, palette=5)
    V = np.maximum(0, np.minimum((qp + 1) // 4, sl[t2r] // 4))
    assert V[:16].min() <= 1024 < V[:16].max()
    assert qsa.select_workspace_bytes(len(t2r), bt.shape[1]) > 0
    want = orc().select(q, kcache, bt, t2r, sl, qp)
    banner("select runs full-size chunks R=256")
    assert_rows_equal(select_runs((q, kcache, bt, t2r, sl, qp), 4), want)
    codes, scales = wl.fp8_integer_keys(rng, kcache)
    banner("select_fp8 runs full-size chunks R=256")
    got = qsa.qsa_select_fp8(runs(q, 4), dev_e4m3(codes), dev(scales), dev(bt), dev(t2r), dev(sl),
                             dev(qp))
    torch.cuda.synchronize()
    assert_rows_equal(got.cpu().numpy(), want)
    w = wl.head_weights(rng, q.shape[0], integer=True)
    want_w = orc().select_weighted(q, w, bt, t2r, sl, qp, kcache=kcache)
    banner("select_weighted runs full-size chunks R=256")
    got = qsa.qsa_select_weighted(runs(q, 4), dev(w), dev(kcache), dev(bt), dev(t2r), dev(sl),
                                  dev(qp))
    torch.cuda.synchronize()
    assert_rows_equal(got.cpu().numpy(), want_w)
    banner("paged_logits runs full-size chunks R=256")
    grouped = qsa.qsa_paged_logits(runs(q, 4), dev(kcache), dev(bt), dev(t2r), dev(sl), dev(qp),
                                   weights=dev(w))
    flat = qsa.qsa_paged_logits(dev(q), dev(kcache), dev(bt), dev(t2r), dev(sl), dev(qp),
                                weights=dev(w))
    torch.cuda.synchronize()
    grouped = grouped.cpu().numpy()
    assert np.array_equal(grouped, flat.cpu().numpy())
    want_l = orc().paged_logits(q, w, bt, t2r, sl, qp, grouped.shape[1], kcache=kcache)
    assert np.array_equal(grouped, want_l.astype(np.float32))


def test_decode_step_deterministic(multi_token):
    """The decode step (grouped queries, several chunks per row, split
    attention) gives identical bytes on 100 repeated calls."""
    w = multi_token
    q, kcache, bt, t2r, sl, qp = w.select_inputs()
    kvd = dev(w.kv)
    k, v = qsa.kv_views(kvd)
    args = [runs(q, 4), dev(kcache), dev(bt), dev(t2r), dev(sl), dev(qp), dev(w.q_attn), k, v]
    idx = torch.empty((w.rows, 2051), dtype=torch.int32, device=kvd.device)
    out = torch.empty((w.rows, 3, 256), dtype=torch.float16, device=kvd.device)
    banner(f"decode determinism x100 {w.name}")
    ref = None
    for i in range(100):
        idx.fill_(-7)
        out.fill_(7)
        qsa.qsa_decode_step(*args, SCALE, indices=idx, out=out)
        got = (idx.cpu().numpy(), out.view(torch.int16).cpu().numpy())
        if ref is None:
            ref = got
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), f"repeat {i} differs"


def test_multi_token_decode_step_fp8():
    """qsa_decode_step_fp8 with grouped queries over the multi-token batch's
    keys absmax-quantized to e4m3: selection within the band of the oracle's
    e4m3 scores, attention against the oracle over the step's own index
    rows."""
    w = wl.with_fp8_keys(wl.multi_token_rows(0), integer=False)
    inputs = w.select_inputs_fp8()
    q, codes, scales, bt, t2r, sl, qp = inputs
    kvd = dev(w.kv)
    k, v = qsa.kv_views(kvd)
    banner(f"decode_fp8 runs {w.name}")
    idx, out = qsa.qsa_decode_step_fp8(runs(q, 4), dev_e4m3(codes), dev(scales), dev(bt), dev(t2r),
                                       dev(sl), dev(qp), dev(w.q_attn), k, v, SCALE)
    torch.cuda.synchronize()
    idx, out = idx.cpu().numpy(), out.cpu().numpy()
    want_idx = orc().select_fp8(*inputs)
    check_select_band(idx, want_idx, orc(), inputs, range(w.rows))
    check_attn(out, oracle_attn(orc(), w.q_attn, w.kv, idx, SCALE),
               "grouped e4m3 multi-token rows, every row")
