"""GPU parity of qsa_build_metadata against the CPU oracle (integers:
exact), and the builder feeding the selection."""

import numpy as np
import pytest
import torch

from paged_top_indexer_amd import workloads as wl
import paged_top_indexer_amd as qsa
from gpu_util import banner, dev, orc
from oracle_pins import METADATA_KINDS, metadata_batch

pytestmark = pytest.mark.gpu
KEYS = ("token_to_req", "logical_positions", "visible_blocks", "slot_mapping")


def build_gpu(qsl, sl, bt, T, **kw):
    csm = kw.pop("common_slot_mapping", None)
    o = qsa.qsa_build_metadata(dev(qsl), dev(sl), dev(bt), T,
                               common_slot_mapping=None if csm is None else dev(csm), **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in o.items()}


def compare(got, want, what):
    for k in KEYS:
        if want.get(k) is not None:
            assert np.array_equal(got[k], want[k]), f"{what}: {k}"
    if want.get("k_work") is not None:
        assert np.array_equal(got["k_work"], want["k_work"]), f"{what}: k_work"


@pytest.mark.parametrize("seed,width", [(0, 400), (1, 3)])
def test_constructed_batches(seed, width):
    qsl, sl, bt, csm, T, _ = metadata_batch(seed, METADATA_KINDS, pad=5, width=width)
    banner(f"build_metadata constructed seed={seed} width={width}")
    for M in (0, 40, 700):
        want = orc().build_metadata(qsl, sl, bt, T, common_slot_mapping=csm, max_num_work=M)
        got = build_gpu(qsl, sl, bt, T, common_slot_mapping=csm, max_num_work=M)
        compare(got, want, f"compressed M={M}")
    for kw in (dict(circular_buffer_size=8), dict(compress_ratio=1, common_slot_mapping=csm),
               dict(storage_block_size=64, compress_ratio=2), dict(common_slot_mapping=None)):
        want = orc().build_metadata(qsl, sl, bt, T, max_num_work=9, **kw)
        got = build_gpu(qsl, sl, bt, T, max_num_work=9, **kw)
        compare(got, want, str(kw))


@pytest.mark.parametrize("N", [1, 37, 500, 5000])
def test_random_batches(N):
    """Many empty queries, padding tokens; 5000 requests exceed the LDS
    staging of the searches (global-memory binary search)."""
    rng = np.random.default_rng(N)
    q = rng.integers(0, 40, size=N)
    q[rng.random(N) < 0.3] = 0
    L = (q + rng.integers(0, 70000, size=N)).astype(np.int32)
    qsl = np.concatenate([[0], np.cumsum(q)]).astype(np.int32)
    T = int(qsl[-1]) + 17
    bt = rng.integers(-1, 1 << 16, size=(N, 140)).astype(np.int32)
    csm = rng.integers(-1, 1 << 30, size=T).astype(np.int64)
    M = int(rng.integers(1, 3 * N + 2))
    banner(f"build_metadata random N={N} T={T} M={M}")
    want = orc().build_metadata(qsl, L, bt, T, common_slot_mapping=csm, max_num_work=M)
    got = build_gpu(qsl, L, bt, T, common_slot_mapping=csm, max_num_work=M)
    compare(got, want, f"N={N}")


def test_serving_batch_and_repeat():
    qsl, sl, bt, csm, T = wl.serving_batch(0)
    M = 4096
    banner(f"build_metadata serving batch N={len(sl)} T={T}")
    want = orc().build_metadata(qsl, sl, bt, T, common_slot_mapping=csm, max_num_work=M)
    d = [dev(a) for a in (qsl, sl, bt, csm)]
    out = None
    for _ in range(3):  # preallocated outputs reused: every call rewrites them
        out = qsa.qsa_build_metadata(d[0], d[1], d[2], T, common_slot_mapping=d[3],
                                     max_num_work=M, out=out)
        torch.cuda.synchronize()
        compare({k: v.cpu().numpy() for k, v in out.items()}, want, "serving")
        for v in out.values():
            v.fill_(-7)


def test_builder_feeds_selection():
    """The builder's requests and positions of the multi-token batch are the
    selection's inputs: identical to the workload's own, and the selection
    over them equals the oracle's."""
    w = wl.multi_token_rows(0, integer=True)
    qsl = wl.query_start_loc(w)
    banner(f"build_metadata -> select, {w.name}")
    d_q, d_kc, d_bt, d_sl = dev(w.q_sel), dev(w.kcache), dev(w.block_table), dev(w.seq_lens)
    m = qsa.qsa_build_metadata(dev(qsl), d_sl, d_bt, w.rows)
    idx = qsa.qsa_select(d_q, d_kc, d_bt, m["token_to_req"], d_sl, m["logical_positions"])
    # the same rows passed as runs of 4 (the batch's requests own 4 or 16 rows)
    idx4 = qsa.qsa_select(d_q.view(w.rows // 4, 4, 4, 128), d_kc, d_bt, m["token_to_req"], d_sl,
                          m["logical_positions"])
    torch.cuda.synchronize()
    assert np.array_equal(m["token_to_req"].cpu().numpy(), w.token_to_req)
    assert np.array_equal(m["logical_positions"].cpu().numpy(), w.query_pos)
    V = np.array([orc().row_extent(int(w.seq_lens[w.token_to_req[r]]), int(w.query_pos[r]))[0]
                  for r in range(w.rows)])
    assert np.array_equal(m["visible_blocks"].cpu().numpy(), V)
    want = orc().select(*w.select_inputs())
    assert np.array_equal(idx.cpu().numpy(), want)
    assert np.array_equal(idx4.cpu().numpy(), want)
