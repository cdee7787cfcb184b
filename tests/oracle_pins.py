"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees with:

* the worked examples printed on the pages (``golden/pages_worked_examples.txt``),
* an independent brute force on small integer-valued inputs (exact int64
  scores, visible blocks counted token by token, selection by counting how
  many blocks outrank each block -- no sort),
* numpy's float64 gather and library sort on N(0,1) inputs,
* closed-form special cases of selection and of attention,
* torch's float64 softmax on gathered rows,
* numpy's binary16 decoder, for every bit pattern,
* torch's float8_e4m3fn decoder, for every code; the fp16 selection
  (pinned above) on integer keys re-encoded as e4m3 codes with power-of-two
  scales, which dequantize to exactly the same keys.

The same functions run against the trusted oracle (they must all pass) and
against builds with one planted mistake (at least one must fail).
"""

from __future__ import annotations

import os

import numpy as np

from paged_top_indexer_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "pages_worked_examples.txt")
WIDTH, TOPK, RATIO = 2051, 512, 4


def read_golden():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, L, qp, vis, valid = line.split()
            rows.append((name, int(L), int(qp), int(vis), int(valid)))
    return rows


# ---------------------------------------------------------------------------
# independent brute force for selection

def brute_visible(seq_len: int, query_pos: int) -> tuple[int, int]:
    """Count, token by token, the tokens the query can see, the complete
    groups of four among them and the leftover tail."""
    seen = [t for t in range(max(0, seq_len)) if t <= query_pos]
    blocks = [b for b in range(len(seen)) if 4 * b + 3 < len(seen)]
    tail = [t for t in range(4 * len(blocks), len(seen))]
    return len(blocks), len(tail)


def brute_select_integer(q, kcache, bt, t2r, sl, qp, weights=None) -> np.ndarray:
    """Selection from exact integer scores and rank counting (inputs must be
    integer-valued fp16; weights, when given, integer-valued [R,4])."""
    R = q.shape[0]
    out = np.full((R, WIDTH), -1, dtype=np.int32)
    qi = q.astype(np.int64)
    for r in range(R):
        req = int(t2r[r])
        V, T = brute_visible(int(sl[req]), int(qp[r]))
        b = np.arange(V)
        keys = kcache[bt[req, b // 128], b % 128, 0, :].astype(np.int64)  # [V,128]
        dots = keys @ qi[r].T                                               # [V,4]
        wr = np.ones(4, np.int64) if weights is None else weights[r].astype(np.int64)
        s = (np.maximum(dots, 0) * wr).sum(axis=1)                          # [V]
        # rank = blocks with a larger score + earlier blocks with an equal score
        better = (s[None, :] > s[:, None]) | ((s[None, :] == s[:, None]) & (b[None, :] < b[:, None]))
        rank = better.sum(axis=1)
        n = min(TOPK, V)
        for blk in range(V):
            if rank[blk] < n:
                out[r, 4 * rank[blk]:4 * rank[blk] + 4] = 4 * blk + np.arange(4)
        out[r, 4 * n:4 * n + T] = 4 * V + np.arange(T)
    return out


def integer_problem(seed: int, lengths, palette: int | None, q_range: int,
                    num_pages: int = 96):
    rng = np.random.default_rng(seed)
    if palette:
        pal = wl.int_f16(rng, -4, 4, (palette, 128))
        kcache = pal[rng.integers(0, palette, size=(num_pages, 128))].reshape(num_pages, 128, 1, 128)
    else:
        kcache = wl.int_f16(rng, -4, 4, (num_pages, 128, 1, 128))
    bt = wl.block_table_per_row(rng, lengths, num_pages)
    q = wl.int_f16(rng, -q_range, q_range, (len(lengths), 4, 128))
    t2r, sl, qp = wl.decode_rows(lengths)
    return q, kcache, bt, t2r, sl, qp


PIN_LENGTHS = [0, 1, 3, 4, 7, 512, 515, 516, 2044, 2047, 2048, 2049, 2052, 2055, 4099, 6001]


def pin_select_brute_force_integer(orc):
    """Bit-exact against the brute force, with and without massive ties."""
    for seed, palette, qr in [(0, None, 4), (1, 8, 2), (2, 3, 1), (3, None, 1)]:
        args = integer_problem(seed, PIN_LENGTHS, palette, qr)
        got = orc.select(*args)
        want = brute_select_integer(*args)
        assert np.array_equal(got, want), f"brute force mismatch (seed {seed})"


def pin_select_multirow_requests(orc):
    """Several query rows per request (chunked-prefill style positions) and a
    padded row with query position -1: V and T follow each row's position."""
    rng = np.random.default_rng(11)
    kcache = wl.int_f16(rng, -4, 4, (40, 128, 1, 128))
    lengths = [3000, 700]
    bt = wl.block_table_per_row(rng, lengths, 40)
    t2r = np.array([0, 0, 0, 1, 1, 0], dtype=np.int32)
    qp = np.array([2999, 2050, 13, 699, 515, -1], dtype=np.int64)
    sl = np.array(lengths, dtype=np.int32)
    q = wl.int_f16(rng, -3, 3, (6, 4, 128))
    got = orc.select(q, kcache, bt, t2r, sl, qp)
    want = brute_select_integer(q, kcache, bt, t2r, sl, qp)
    assert np.array_equal(got, want)
    assert np.all(got[5] == -1)


def pin_select_worked_examples(orc):
    """The pages' printed visible blocks and valid widths."""
    for name, L, qp, vis, valid in read_golden():
        V, T = orc.row_extent(L, qp)
        assert V == vis, (name, V, vis)
        rng = np.random.default_rng(5)
        pages = wl.pages_needed(L)
        kcache = wl.int_f16(rng, -4, 4, (pages + 3, 128, 1, 128))
        bt = rng.permutation(pages + 3)[:pages].astype(np.int32).reshape(1, pages)
        q = wl.int_f16(rng, -4, 4, (1, 4, 128))
        out = orc.select(q, kcache, bt, np.array([0], np.int32), np.array([L], np.int32),
                         np.array([qp], np.int64))
        width = int((out[0] >= 0).sum())
        assert width == valid, (name, width, valid)
        assert np.all(out[0, width:] == -1)
        # the tail is appended right after the expanded blocks
        assert np.array_equal(out[0, width - T:width], 4 * V + np.arange(T))


def pin_select_closed_forms(orc):
    """Equal scores everywhere -> blocks in ascending order; one dominant
    block -> first; zero query -> ascending; a key that only matches head 3
    still scores."""
    rng = np.random.default_rng(7)
    L = 2600
    pages = wl.pages_needed(L)
    one = np.ones((pages, 128, 1, 128), np.float16)
    bt = np.arange(pages, dtype=np.int32).reshape(1, pages)
    t2r, sl, qp = wl.decode_rows([L])
    V = L // 4
    ascending = np.concatenate([np.arange(2048), 4 * V + np.arange(L % 4)])
    for q in [wl.int_f16(rng, -4, 4, (1, 4, 128)), np.zeros((1, 4, 128), np.float16)]:
        out = orc.select(q, one, bt, t2r, sl, qp)
        assert np.array_equal(out[0, :ascending.size], ascending)
    # a dominant block, visible only through head 3, at the last visible slot
    kc = np.zeros((pages, 128, 1, 128), np.float16)
    last = V - 1
    kc[last // 128, last % 128, 0, 5] = 2.0
    q = np.zeros((1, 4, 128), np.float16)
    q[0, 3, 5] = 1.0
    q[0, 0, 5] = -1.0  # head 0 sees it negatively: ReLU must drop that
    out = orc.select(q, kc, bt, t2r, sl, qp)
    assert np.array_equal(out[0, :4], 4 * last + np.arange(4))
    assert np.array_equal(out[0, 4:8], np.arange(4))


def pin_select_gather_and_sort_normal(orc):
    """N(0,1) inputs: scores against a numpy float64 gather, selection
    against numpy's lexsort of the float32-rounded scores."""
    rng = np.random.default_rng(3)
    lengths = [2900, 517, 64]
    P = 64
    kcache = wl.normal_f16(rng, (P, 128, 1, 128))
    bt = wl.block_table_per_row(rng, lengths, P)
    q = wl.normal_f16(rng, (3, 4, 128))
    t2r, sl, qp = wl.decode_rows(lengths)
    out = orc.select(q, kcache, bt, t2r, sl, qp)
    for r, L in enumerate(lengths):
        V = L // 4
        b = np.arange(V)
        keys = kcache[bt[r, b // 128], b % 128, 0, :].astype(np.float64)
        s64 = np.maximum(keys @ q[r].astype(np.float64).T, 0.0).sum(axis=1)
        s32 = s64.astype(np.float32)
        got_scores = orc.row_scores(r, q, kcache, bt, t2r, sl, qp)
        assert np.allclose(got_scores, s64, rtol=1e-6, atol=1e-6)
        order = np.lexsort((b, -s32.astype(np.float64)))
        n = min(TOPK, V)
        want = (4 * order[:n, None] + np.arange(4)).reshape(-1)
        assert np.array_equal(out[r, :4 * n], want)
        assert np.array_equal(out[r, 4 * n:4 * n + L % 4], 4 * V + np.arange(L % 4))
        assert np.all(out[r, 4 * n + L % 4:] == -1)


# ---------------------------------------------------------------------------
# attention

def _exact_dot(a16, b16) -> float:
    return float(np.dot(a16.astype(np.float64), b16.astype(np.float64)))


def pin_attn_closed_forms(orc):
    rng = np.random.default_rng(9)
    NT = 64
    kv = wl.normal_f16(rng, (NT, 512))
    q = wl.normal_f16(rng, (5, 3, 256))
    idx = np.full((5, WIDTH), -1, np.int32)
    idx[1, 700] = 17                       # one valid index
    idx[2, ::7] = 23                        # one index repeated, holes between
    idx[3, :] = 41                          # one index over the full width
    idx[4, 0] = 0                           # token 0 present...
    idx[4, 0] = -1                          # ...then removed: all holes again
    out = orc.sparse_attn(q, kv, idx, 1.0 / 16)
    V = kv[:, 256:].astype(np.float64)
    assert np.all(out[0] == 0.0) and np.all(out[4] == 0.0)
    for r, t in [(1, 17), (2, 23), (3, 41)]:
        assert np.allclose(out[r], np.broadcast_to(V[t], (3, 256)), rtol=0, atol=1e-12)


def pin_attn_equal_logits_mean(orc):
    """Identical K rows -> every logit equal -> output = mean of V over the
    multiset of valid positions (duplicates weighted by multiplicity)."""
    rng = np.random.default_rng(10)
    NT = 32
    kv = wl.normal_f16(rng, (NT, 512))
    kv[:, :256] = kv[0, :256]
    q = wl.normal_f16(rng, (1, 3, 256))
    idx = np.full((1, WIDTH), -1, np.int32)
    members = [3, 3, 3, 9, 30, 30, 0]
    idx[0, [5, 100, 2000, 7, 8, 2050, 1]] = members
    out = orc.sparse_attn(q, kv, idx, 0.0625)
    want = kv[members, 256:].astype(np.float64).mean(axis=0)
    assert np.allclose(out[0], np.broadcast_to(want, (3, 256)), rtol=0, atol=1e-12)


def pin_attn_two_token_logistic(orc):
    """Tokens a (once) and b (twice): weight of b is 2e^{l_b}/(e^{l_a}+2e^{l_b})
    with l = scale * q.k from exact integer dot products."""
    rng = np.random.default_rng(12)
    kv = np.zeros((8, 512), np.float16)
    kv[:, :256] = wl.int_f16(rng, -2, 2, (8, 256))
    kv[:, 256:] = wl.normal_f16(rng, (8, 256))
    q = wl.int_f16(rng, -1, 1, (1, 3, 256))
    idx = np.full((1, WIDTH), -1, np.int32)
    idx[0, 10], idx[0, 11], idx[0, 1500] = 2, 5, 5
    scale = 0.03125
    out = orc.sparse_attn(q, kv, idx, scale)
    for h in range(3):
        la = scale * _exact_dot(q[0, h], kv[2, :256])
        lb = scale * _exact_dot(q[0, h], kv[5, :256])
        wb = 1.0 / (1.0 + 0.5 * np.exp(la - lb))
        want = (1 - wb) * kv[2, 256:].astype(np.float64) + wb * kv[5, 256:].astype(np.float64)
        assert np.allclose(out[0, h], want, rtol=0, atol=1e-12)


def pin_attn_torch_float64(orc):
    """Random rows with holes and duplicates against torch's float64 softmax
    over the gathered rows."""
    import torch
    rng = np.random.default_rng(13)
    NT = 1024
    kv = wl.normal_f16(rng, (NT, 512))
    q = wl.normal_f16(rng, (4, 3, 256))
    idx = wl.random_index_rows(rng, 4, NT, valid=WIDTH, distinct=False)
    idx = wl.inject_holes_and_duplicates(rng, idx, 0.1, 0.1)
    idx[3, 100:] = -1
    scale = 1.0 / 16
    out = orc.sparse_attn(q, kv, idx, scale)
    kvt = torch.from_numpy(kv.astype(np.float64))
    for r in range(4):
        sel = torch.from_numpy(idx[r][idx[r] >= 0].astype(np.int64))
        K, Vr = kvt[sel, :256], kvt[sel, 256:]
        qt = torch.from_numpy(q[r].astype(np.float64))
        p = torch.softmax(qt @ K.T * scale, dim=-1)
        want = (p @ Vr).numpy()
        assert np.allclose(out[r], want, rtol=0, atol=1e-12)


def pin_half_to_double(orc):
    """Every binary16 bit pattern against numpy's decoder."""
    bits = np.arange(65536, dtype=np.uint32)
    want = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(int(b)) for b in bits[::1]])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


# ---------------------------------------------------------------------------
# e4m3 key cache

def torch_e4m3_table() -> np.ndarray:
    """float64 value of every e4m3fn code, decoded by torch."""
    import torch

    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def pin_e4m3_to_double(orc):
    """Every e4m3 code against torch's float8_e4m3fn decoder."""
    want = torch_e4m3_table()
    got = np.array([orc.e4m3_to_double(c) for c in range(256)])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def pin_select_fp8_integer_equivalence(orc):
    """Integer keys re-encoded as e4m3 codes with per-key power-of-two
    scales dequantize to the same keys: the fp8 selection equals the brute
    force on the integer keys, ties included."""
    for seed, palette, qr in [(0, None, 4), (1, 8, 2), (2, 3, 1)]:
        args = integer_problem(seed, PIN_LENGTHS, palette, qr)
        q, kcache, bt, t2r, sl, qp = args
        codes, scales = wl.fp8_integer_keys(np.random.default_rng(100 + seed), kcache)
        assert len(np.unique(scales)) == 5
        got = orc.select_fp8(q, codes, scales, bt, t2r, sl, qp)
        want = brute_select_integer(*args)
        assert np.array_equal(got, want), f"fp8 integer mismatch (seed {seed})"


def pin_row_scores_fp8_one_hot(orc):
    """One-hot queries read a single code back: with head 0 = +1 and head
    1 = -1 on dimension 7, block i scores exactly float32(s_i * |e4m3(c_i)|)
    (one of the two ReLUs passes it), for every finite code and arbitrary
    float32 scales."""
    table = torch_e4m3_table()
    finite = np.flatnonzero(~np.isnan(table))
    n = finite.size                       # 254 codes -> 254 blocks
    pages = -(-n // 128)
    rng = np.random.default_rng(17)
    codes = np.zeros((pages, 128, 1, 128), np.uint8)
    scales = rng.uniform(0.01, 3.0, size=(pages, 128)).astype(np.float32)
    b = np.arange(n)
    codes[b // 128, b % 128, 0, 7] = finite
    q = np.zeros((1, 4, 128), np.float16)
    q[0, 0, 7], q[0, 1, 7] = 1.0, -1.0
    bt = np.arange(pages, dtype=np.int32).reshape(1, pages)
    t2r, sl, qp = wl.decode_rows([4 * n])
    got = orc.row_scores_fp8(0, q, codes, scales, bt, t2r, sl, qp)
    want = (scales[b // 128, b % 128].astype(np.float64) * np.abs(table[finite])).astype(np.float32)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


def pin_select_fp8_gather_and_sort_normal(orc):
    """Absmax-quantized N(0,1) keys: scores against a numpy float64 gather of
    the dequantized keys (torch's decoder x scale), selection against
    lexsort of the float32-rounded scores."""
    rng = np.random.default_rng(23)
    lengths = [2900, 517]
    P = 48
    kcache = wl.normal_f16(rng, (P, 128, 1, 128))
    codes, scales = wl.fp8_normal_keys(kcache)
    bt = wl.block_table_per_row(rng, lengths, P)
    q = wl.normal_f16(rng, (2, 4, 128))
    t2r, sl, qp = wl.decode_rows(lengths)
    table = torch_e4m3_table()
    out = orc.select_fp8(q, codes, scales, bt, t2r, sl, qp)
    for r, L in enumerate(lengths):
        V = L // 4
        b = np.arange(V)
        pg, sl_ = bt[r, b // 128], b % 128
        keys = table[codes[pg, sl_, 0, :]] * scales[pg, sl_][:, None].astype(np.float64)
        s64 = np.maximum(keys @ q[r].astype(np.float64).T, 0.0).sum(axis=1)
        got_scores = orc.row_scores_fp8(r, q, codes, scales, bt, t2r, sl, qp)
        assert np.allclose(got_scores, s64, rtol=1e-6, atol=1e-6)
        order = np.lexsort((b, -s64.astype(np.float32).astype(np.float64)))
        n = min(TOPK, V)
        want = (4 * order[:n, None] + np.arange(4)).reshape(-1)
        assert np.array_equal(out[r, :4 * n], want)
        assert np.array_equal(out[r, 4 * n:4 * n + L % 4], 4 * V + np.arange(L % 4))


# ---------------------------------------------------------------------------
# per-head weights and the two-pass form

def pin_select_weighted_brute_force(orc):
    """Integer head weights in [-3, 3] (zero and negative included): exact
    int64 scores and rank counting, fp16 and e4m3 caches."""
    for seed, palette, qr in [(4, None, 3), (5, 6, 2)]:
        args = integer_problem(seed, PIN_LENGTHS, palette, qr)
        q, kcache, bt, t2r, sl, qp = args
        rng = np.random.default_rng(50 + seed)
        w = rng.integers(-3, 4, size=(q.shape[0], 4)).astype(np.float32)
        w[0] = [0, 0, 0, 0]                       # every score 0: ascending blocks
        w[1] = [-1, -2, -1, -3]                   # every score <= 0
        want = brute_select_integer(*args, weights=w)
        got = orc.select_weighted(q, w, bt, t2r, sl, qp, kcache=kcache)
        assert np.array_equal(got, want), f"weighted brute force (seed {seed})"
        codes, scales = wl.fp8_integer_keys(np.random.default_rng(60 + seed), kcache)
        got8 = orc.select_weighted(q, w, bt, t2r, sl, qp, codes=codes, scales=scales)
        assert np.array_equal(got8, want), f"weighted e4m3 brute force (seed {seed})"


def pin_weights_of_one(orc):
    """Weights of one give the unweighted selection; the paged logits with no
    weights are the exact row scores followed by -inf; top-k per row over
    them is the brute-force selection."""
    args = integer_problem(6, PIN_LENGTHS[:10], 5, 2)
    q, kcache, bt, t2r, sl, qp = args
    ones = np.ones((q.shape[0], 4), np.float32)
    assert np.array_equal(orc.select_weighted(q, ones, bt, t2r, sl, qp, kcache=kcache),
                          brute_select_integer(*args))
    width = bt.shape[1] * 128 + 7
    lg = orc.paged_logits(q, None, bt, t2r, sl, qp, width, kcache=kcache)
    for r in range(q.shape[0]):
        V, _ = brute_visible(int(sl[t2r[r]]), int(qp[r]))
        b = np.arange(V)
        keys = kcache[bt[t2r[r], b // 128], b % 128, 0, :].astype(np.int64)
        want = np.maximum(keys @ q[r].astype(np.int64).T, 0).sum(axis=1)
        assert np.array_equal(lg[r, :V], want.astype(np.float32))
        assert np.all(np.isneginf(lg[r, V:]))
    # the two passes compose to the brute-force selection (rows with V < 512
    # would pick up -inf entries if the top-k read past V)
    assert np.array_equal(orc.topk_per_row(lg, t2r, sl, qp), brute_select_integer(*args))


def pin_paged_logits_gather_normal(orc):
    """N(0,1) keys and real weights of both signs: the logits against a numpy
    float64 gather, -inf past the visible blocks."""
    rng = np.random.default_rng(31)
    lengths = [2900, 517, 0]
    P = 40
    kcache = wl.normal_f16(rng, (P, 128, 1, 128))
    bt = wl.block_table_per_row(rng, lengths, P)
    q = wl.normal_f16(rng, (3, 4, 128))
    t2r, sl, qp = wl.decode_rows(lengths)
    w = rng.normal(size=(3, 4)).astype(np.float32)
    width = bt.shape[1] * 128
    lg = orc.paged_logits(q, w, bt, t2r, sl, qp, width, kcache=kcache)
    for r, L in enumerate(lengths):
        V = L // 4
        b = np.arange(V)
        keys = kcache[bt[r, b // 128], b % 128, 0, :].astype(np.float64)
        dots = keys @ q[r].astype(np.float64).T
        want = (np.maximum(dots, 0.0) * w[r].astype(np.float64)).sum(axis=1)
        assert np.allclose(lg[r, :V], want, rtol=1e-6, atol=1e-6)
        assert np.all(np.isneginf(lg[r, V:]))


def pin_topk_per_row_lexsort(orc):
    """Top-k per row over arbitrary logits -- negative values, +0 and -0
    (equal), many exact repeats, huge junk past each row's visible blocks --
    against numpy's lexsort of the first V entries."""
    rng = np.random.default_rng(41)
    lengths = [2900, 1337, 519, 4, 0, 6001]
    qpos = [2899, 1000, 518, 3, -1, 6000]
    width = 1600
    lg = np.round(rng.normal(size=(len(lengths), width)) * 4) / 4   # coarse grid: ties
    lg = lg.astype(np.float32)
    zeros = rng.random(lg.shape) < 0.1
    lg[zeros] = np.where(rng.random(zeros.sum()) < 0.5, 0.0, -0.0)
    t2r = np.arange(len(lengths), dtype=np.int32)
    sl = np.array(lengths, np.int32)
    qp = np.array(qpos, np.int64)
    for r in range(len(lengths)):
        V, _ = brute_visible(lengths[r], qpos[r])
        lg[r, V:] = 1e30                                             # never read
    got = orc.topk_per_row(lg, t2r, sl, qp)
    for r in range(len(lengths)):
        V, T = brute_visible(lengths[r], qpos[r])
        b = np.arange(V)
        order = np.lexsort((b, -lg[r, :V].astype(np.float64)))
        n = min(TOPK, V)
        want = np.full(WIDTH, -1, np.int32)
        want[:4 * n] = (4 * order[:n, None] + np.arange(4)).reshape(-1)
        want[4 * n:4 * n + T] = 4 * V + np.arange(T)
        assert np.array_equal(got[r], want), f"row {r}"


# ---------------------------------------------------------------------------
# metadata builder

def metadata_batch(seed: int, kinds, pad: int, width: int):
    """A batch built request by request; returns the builder's inputs and the
    expected outputs known by construction (no request search anywhere).
    kinds: per request (seq_len, query_len)."""
    rng = np.random.default_rng(seed)
    N = len(kinds)
    qsl = np.zeros(N + 1, np.int32)
    for r, (L, q) in enumerate(kinds):
        qsl[r + 1] = qsl[r] + q
    mapped = int(qsl[-1])
    T = mapped + pad
    sl = np.array([L for L, _ in kinds], np.int32)
    bt = rng.integers(0, 5000, size=(N, width)).astype(np.int32)
    bt[rng.random(bt.shape) < 0.1] = -1                      # holes in the table
    csm = rng.integers(0, 1 << 20, size=T).astype(np.int64)
    csm[rng.random(T) < 0.05] = -1                           # tokens the main cache skips
    want = {"token_to_req": np.zeros(T, np.int32), "logical_positions": np.full(T, -1, np.int64),
            "visible_blocks": np.zeros(T, np.int32), "slot_mapping": np.full(T, -1, np.int64),
            "ring": np.full(T, -1, np.int64), "work": []}
    for r, (L, q) in enumerate(kinds):
        for i in range(q):
            t = int(qsl[r]) + i
            pos = L - q + i
            want["token_to_req"][t] = r
            want["logical_positions"][t] = pos
            V, _ = brute_visible(L, pos)
            want["visible_blocks"][t] = V
            if (pos + 1) % RATIO == 0:                       # token closing a group
                group = (pos + 1) // RATIO - 1
                blk = group // 128
                if blk < width and bt[r, blk] >= 0 and csm[t] >= 0:
                    want["slot_mapping"][t] = int(bt[r, blk]) * 128 + group % 128
            if i >= q - 8 and bt[r, 0] >= 0:                  # last 8 tokens: the ring
                want["ring"][t] = int(bt[r, 0]) * 8 + pos % 8
        if q > 0:
            groups = [g for g in range(L // RATIO) if g * RATIO + RATIO - 1 >= L - q]
            want["work"] += [(r, i) for i in range(max(len(groups), 1))]
    return qsl, sl, bt, csm, T, want


METADATA_KINDS = [(519, 1), (1004, 4), (0, 0), (20, 3), (9215, 16), (3, 3), (777, 0),
                  (131072, 1), (40000, 37), (4, 4), (5, 1), (100, 100)]


def pin_metadata_by_construction(orc):
    """Per-token request, position, visible blocks, compressed and ring
    slots, and the k work items of a batch built request by request: decode,
    speculative and prefill rows, empty queries, a query as long as its
    sequence, padding tokens, holes in the table, skipped main-cache slots."""
    for seed, width in [(0, 400), (1, 3)]:
        qsl, sl, bt, csm, T, want = metadata_batch(seed, METADATA_KINDS, pad=5, width=width)
        for M in (len(want["work"]) + 7, max(1, len(want["work"]) - 5)):
            got = orc.build_metadata(qsl, sl, bt, T, common_slot_mapping=csm, max_num_work=M)
            for k in ("token_to_req", "logical_positions", "visible_blocks", "slot_mapping"):
                assert np.array_equal(got[k], want[k]), (seed, k)
            w = np.full((M, 2), -1, np.int32)
            n = min(M, len(want["work"]))
            w[:n] = np.array(want["work"][:n], np.int32).reshape(-1, 2)
            assert np.array_equal(got["k_work"], w), (seed, "k_work")
        ring = orc.build_metadata(qsl, sl, bt, T, circular_buffer_size=8)
        assert np.array_equal(ring["slot_mapping"], want["ring"]), (seed, "ring")
        plain = orc.build_metadata(qsl, sl, bt, T, compress_ratio=1, common_slot_mapping=csm)
        assert np.array_equal(plain["slot_mapping"], csm)


def pin_metadata_searchsorted(orc):
    """Request search on random batches (many empty queries) against numpy's
    searchsorted; positions and visible blocks from their closed forms."""
    rng = np.random.default_rng(71)
    for N in (1, 2, 37, 500):
        q = rng.integers(0, 6, size=N)
        q[rng.random(N) < 0.3] = 0
        L = q + rng.integers(0, 3000, size=N)
        qsl = np.concatenate([[0], np.cumsum(q)]).astype(np.int32)
        T = int(qsl[-1]) + 3
        bt = np.zeros((N, 30), np.int32)
        got = orc.build_metadata(qsl, L.astype(np.int32), bt, T, with_slots=False)
        t = np.arange(int(qsl[-1]))
        r = np.searchsorted(qsl[1:], t, side="right")
        assert np.array_equal(got["token_to_req"][:t.size], r)
        assert np.all(got["token_to_req"][t.size:] == 0)
        lp = L[r] - q[r] + (t - qsl[r])
        assert np.array_equal(got["logical_positions"][:t.size], lp)
        assert np.all(got["logical_positions"][t.size:] == -1)
        vis = np.maximum(0, np.minimum((lp + 1) // 4, L[r] // 4))
        assert np.array_equal(got["visible_blocks"][:t.size], vis)


def pin_metadata_closed_forms(orc):
    """A prefill from position 0 through an identity table writes compressed
    slot g exactly at token 4g + 3; a decode row owns exactly one k work item
    whether or not its token completes a group, and a prefill of n tokens
    from position s owns floor((s+n)/4) - floor(s/4) items (at least one)."""
    L = 2000
    qsl = np.array([0, L], np.int32)
    bt = np.arange(16, dtype=np.int32).reshape(1, 16)
    got = orc.build_metadata(qsl, np.array([L], np.int32), bt, L, max_num_work=600)
    t = np.arange(L)
    want = np.where((t + 1) % 4 == 0, (t + 1) // 4 - 1, -1)
    assert np.array_equal(got["slot_mapping"], want)
    assert np.array_equal(got["k_work"][:500], np.stack([np.zeros(500), np.arange(500)], 1))
    assert np.all(got["k_work"][500:] == -1)
    lens = np.array([517, 518, 519, 520, 4, 1], np.int32)          # decode rows
    qsl = np.arange(len(lens) + 1, dtype=np.int32)
    got = orc.build_metadata(qsl, lens, np.zeros((len(lens), 8), np.int32), len(lens),
                             max_num_work=len(lens) + 2)
    assert np.array_equal(got["k_work"][:len(lens)],
                          np.stack([np.arange(len(lens)), np.zeros(len(lens))], 1))
    assert np.all(got["k_work"][len(lens):] == -1)
    for s0, n in [(0, 3), (1, 9), (6, 2), (7, 1), (8, 16)]:
        got = orc.build_metadata(np.array([0, n], np.int32), np.array([s0 + n], np.int32),
                                 np.zeros((1, 8), np.int32), n, max_num_work=40)
        count = max((s0 + n) // 4 - s0 // 4, 1)
        assert np.array_equal(got["k_work"][:count, 1], np.arange(count))
        assert np.all(got["k_work"][count:] == -1)


ALL_PINS = [
    pin_half_to_double,
    pin_e4m3_to_double,
    pin_select_fp8_integer_equivalence,
    pin_row_scores_fp8_one_hot,
    pin_select_fp8_gather_and_sort_normal,
    pin_select_weighted_brute_force,
    pin_weights_of_one,
    pin_paged_logits_gather_normal,
    pin_topk_per_row_lexsort,
    pin_metadata_by_construction,
    pin_metadata_searchsorted,
    pin_metadata_closed_forms,
    pin_select_worked_examples,
    pin_select_brute_force_integer,
    pin_select_multirow_requests,
    pin_select_closed_forms,
    pin_select_gather_and_sort_normal,
    pin_attn_closed_forms,
    pin_attn_equal_logits_mean,
    pin_attn_two_token_logistic,
    pin_attn_torch_float64,
]
