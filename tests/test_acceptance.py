"""The acceptance rules of oracle.acceptance on the CPU: the oracle's own
output passes, planted mistakes (a block swapped for one far below the
boundary, a broken quadruple, a wrong tail, an attention output off by
more than the bounds) fail."""

import numpy as np

import oracle
from oracle import acceptance
from paged_top_indexer_amd import workloads as wl


def _setup():
    w = wl.saturated_row(0)
    orc = oracle.default()
    inputs = w.select_inputs()
    ref = acceptance.oracle_select(orc, inputs)
    return w, orc, inputs, ref


def test_oracle_passes_its_own_rule_and_threads_agree():
    w, orc, inputs, ref = _setup()
    assert np.array_equal(ref, orc.select(*inputs))
    assert acceptance.band_problems(orc, ref, ref, inputs) == {}
    multi = wl.multi_token_rows(0)
    mi = multi.select_inputs()
    rows = [0, 5, 17, 100, 255]
    threaded = acceptance.oracle_select(orc, mi, rows, threads=4)
    assert np.array_equal(threaded, orc.select(*acceptance.subset_rows(mi, rows)))


def test_planted_selection_mistakes_fail():
    w, orc, inputs, ref = _setup()
    scores = orc.row_scores(0, *inputs)
    V, T = orc.row_extent(int(w.seq_lens[0]), int(w.query_pos[0]))
    assert (V, T) == (2303, 3)
    chosen = set((ref[0, :2048:4] // 4).tolist())
    worst = int(np.argmin(np.where([b in chosen for b in range(V)], np.inf, scores)))
    bad = ref.copy()
    bad[0, 0:4] = 4 * worst + np.arange(4)  # the best block swapped for the worst
    assert "outside the band" in acceptance.band_problems(orc, bad, ref, inputs)[0]
    quad = ref.copy()
    quad[0, 1] += 1
    assert acceptance.band_problems(orc, quad, ref, inputs)[0] == "quadruple"
    tail = ref.copy()
    tail[0, 2049] = -1
    assert acceptance.band_problems(orc, tail, ref, inputs)[0] == "tail"
    # two neighbours swapped inside the band (equal within 1e-3) still pass
    s_sel = scores[ref[0, :2048:4] // 4]
    i = int(np.argmin(np.abs(np.diff(s_sel))))
    if abs(s_sel[i] - s_sel[i + 1]) <= 1e-3 * max(abs(s_sel[i + 1]), 1.0):
        sw = ref.copy()
        sw[0, 4 * i:4 * i + 4], sw[0, 4 * i + 4:4 * i + 8] = (ref[0, 4 * i + 4:4 * i + 8].copy(),
                                                              ref[0, 4 * i:4 * i + 4].copy())
        assert acceptance.band_problems(orc, sw, ref, inputs) == {}


def test_attention_bounds():
    want = np.array([[[0.5, 1e-4, -3.0]]])
    got = want.astype(np.float16)
    assert acceptance.attn_error(got, want) == (float(np.max(np.abs(got - want))), 0)
    off = got.copy()
    off[0, 0, 0] = np.float16(0.5 + 3 * 2.0 ** -11)  # 3 half-ulps of 0.5 away
    err, over = acceptance.attn_error(off, want)
    assert over == 1 and err < acceptance.ATTN_TOL
