"""The seeded generator: determinism and the structure each workload promises."""

import numpy as np

from paged_top_indexer_amd import workloads as wl


def _same(a, b):
    for name in ["q_sel", "kcache", "block_table", "token_to_req", "seq_lens", "query_pos",
                 "q_attn", "kv"]:
        assert np.array_equal(getattr(a, name), getattr(b, name)), name


def test_deterministic_small():
    _same(wl.tiny_integer(0), wl.tiny_integer(0))
    _same(wl.ties_and_edges(0), wl.ties_and_edges(0))
    a, b = wl.tiny_integer(0), wl.tiny_integer(1)
    assert not np.array_equal(a.kcache, b.kcache)


def test_tiny_integer_structure():
    w = wl.tiny_integer(0)
    assert w.q_sel.shape == (1, 4, 128) and w.kcache.shape == (8, 128, 1, 128)
    assert w.block_table.shape == (1, 2) and len(set(w.block_table[0])) == 2
    assert int(w.seq_lens[0]) == 519 and int(w.query_pos[0]) == 518
    assert w.query_pos.dtype == np.int64
    vals = np.unique(w.kcache.astype(np.float32))
    assert set(vals) <= set(range(-4, 5))
    # slot 15 of every 16-slot group duplicates another slot of its group
    k = w.kcache[:, :, 0, :].reshape(8, 8, 16, 128)
    for p in range(8):
        for g in range(8):
            assert any(np.array_equal(k[p, g, 15], k[p, g, s]) for s in range(15))
    assert w.kv.shape == (2, 512, 512)


def test_ties_and_edges_structure():
    w = wl.ties_and_edges(0)
    assert w.rows == 32
    assert set(w.seq_lens.tolist()) == set(wl.EDGE_LENGTHS)
    flat = w.kcache.reshape(-1, 128)
    assert len(np.unique(flat, axis=0)) <= 64
    assert np.all(np.abs(w.q_sel.astype(np.float32)) <= 2)
    for r, L in enumerate(w.seq_lens):
        n = wl.pages_needed(int(L))
        assert np.all(w.block_table[r, :n] >= 0) and np.all(w.block_table[r, n:] == -1)
    extra = w.notes["attn_extra_rows"]
    assert np.all(extra[0] == -1) and (extra[1] >= 0).sum() == 1
    assert len(np.unique(extra[2])) == 1 and extra[2, 0] >= 0


def test_inject_holes_and_duplicates():
    rng = np.random.default_rng(0)
    idx = wl.random_index_rows(rng, 3, 10000)
    out = wl.inject_holes_and_duplicates(np.random.default_rng(1), idx, 0.05, 0.05)
    for r in range(3):
        holes = (out[r] == -1).sum()
        assert holes == round(0.05 * 2051)
        valid = out[r][out[r] >= 0]
        assert len(valid) - len(np.unique(valid)) == round(0.05 * 2051)
        assert set(valid.tolist()) <= set(idx[r].tolist())


def test_shared_pages_batched_table_only():
    # the batched workload's table logic, at a reduced page count
    rng = np.random.default_rng(0)
    lengths = [600, 5000, 33000, 20000]
    bt = wl.block_table_distinct(rng, lengths, 1000)
    used = bt[bt >= 0]
    assert len(np.unique(used)) == used.size
    assert [int((row >= 0).sum()) for row in bt] == [wl.pages_needed(L) for L in lengths]


def test_multi_token_rows_structure():
    w = wl.multi_token_rows(0, decode_requests=6, next_n=3, prefill_requests=2, prefill_chunk=5)
    assert w.rows == 6 * 3 + 2 * 5
    # rows of a request are adjacent and end at the request's last position
    for req in range(8):
        rows = np.flatnonzero(w.token_to_req == req)
        assert np.all(np.diff(rows) == 1)
        pos = w.query_pos[rows]
        assert pos[-1] == w.seq_lens[req] - 1 and np.all(np.diff(pos) == 1)
    assert w.query_pos.dtype == np.int64 and w.token_to_req.dtype == np.int32


def test_fp8_key_caches():
    """e4m3 caches: no NaN codes; the integer re-encoding dequantizes to the
    same keys exactly; absmax scaling puts each key's largest code at 448."""
    import torch

    table = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    w = wl.with_fp8_keys(wl.ties_and_edges(0), integer=True)
    assert w.name.endswith("_fp8") and w.kcodes.dtype == np.uint8 and w.kscale.dtype == np.float32
    assert not np.isnan(table[w.kcodes]).any()
    deq = table[w.kcodes] * w.kscale[:, :, None, None]
    assert np.array_equal(deq, w.kcache.astype(np.float64))
    rng = np.random.default_rng(1)
    k = wl.normal_f16(rng, (4, 128, 1, 128))
    codes, scales = wl.fp8_normal_keys(k)
    vals = np.abs(table[codes])
    assert not np.isnan(vals).any()
    assert np.all(vals.max(axis=(2, 3)) == 448.0)
    # round to nearest: within half a step, 2^-4 relative for normals and
    # 2^-10 x scale absolute in the subnormal range
    err = np.abs(table[codes] * scales[:, :, None, None] - k.astype(np.float64))
    bound = np.maximum(np.abs(k.astype(np.float64)) * 2.0 ** -4, scales[:, :, None, None] * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-6))
