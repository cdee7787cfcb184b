"""Acceptance rules the GPU path is held to against the oracle.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: used by the GPU
tests and by the parity leg of the bench, never by the product package.

Rules (the page "vLLM: integrate FP16 packed QSA extension", "Exact
contracts", gives the selection order and tie rule and the attention's
treatment of holes and duplicates; the tolerances are the build's own):

* selection on integer-valued inputs: bit-exact (every fp32 sum is exact);
* selection on N(0,1) inputs: width, tail and -1 padding exact, every block
  expanded to its exact token quadruple, distinct blocks, and the selected
  set may differ from the oracle's only by blocks whose oracle score lies
  within 1e-3 * max(|s_n|, 1) of the oracle's n-th score s_n; consecutive
  selected blocks must not be out of order by more than that band;
* attention: max |gpu - oracle| <= 2e-3 against the float64 oracle, and at
  most one fp16 ulp from the oracle rounded to fp16, the ulp of values below
  2^-10 taken as that of 2^-10 (9.5e-7): near zero an fp16 ulp is smaller
  than the fp32 rounding of the softmax weights, whose absolute error scales
  with the weighted magnitudes summed (~1), not with the result.

The oracle's C calls release the interpreter lock and keep no shared state,
so rows can be dealt to threads (``map_rows``).
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ATTN_TOL = 2e-3
BAND = 1e-3


def host_threads() -> int:
    """Threads for the oracle: the CPUs this process may run on, at most 16
    (the host share of one GPU on a shared node)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def map_rows(fn, rows, threads: int | None = None, per_call: int = 4):
    """fn(list_of_rows) -> array with one leading entry per row, applied to
    consecutive slices of `rows` in a thread pool; results concatenated in
    row order."""
    rows = [int(r) for r in rows]
    if not rows:
        return []
    slices = [rows[i:i + per_call] for i in range(0, len(rows), per_call)]
    n = threads or host_threads()
    if n == 1 or len(slices) == 1:
        parts = [fn(s) for s in slices]
    else:
        with ThreadPoolExecutor(min(n, len(slices))) as ex:
            parts = list(ex.map(fn, slices))
    return np.concatenate(parts, axis=0)


def subset_rows(inputs, rows):
    """Selection inputs restricted to some query rows (requests unchanged);
    six (fp16 cache: q, kcache, table, token_to_req, seq_lens, query_pos) or
    seven (e4m3: q, codes, scales, ...) inputs."""
    rows = np.asarray(rows)
    q, *cache, bt, t2r, sl, qp = inputs
    return (q[rows], *cache, bt, t2r[rows], sl, qp[rows])


def oracle_select(orc, inputs, rows=None, threads: int | None = None) -> np.ndarray:
    """The oracle's [len(rows), 2051] selection of the listed rows (all by
    default), rows dealt to threads."""
    R = len(inputs[-1])
    rows = range(R) if rows is None else rows
    fn = orc.select_fp8 if len(inputs) == 7 else orc.select
    return map_rows(lambda rs: fn(*subset_rows(inputs, rs)), rows, threads)


def oracle_attn(orc, q_attn, kv, indices, scale: float, rows=None,
                threads: int | None = None) -> np.ndarray:
    """The oracle's float64 attention of the listed rows over the given index
    rows ([R, 2051], one per row of q_attn)."""
    R = q_attn.shape[0]
    rows = range(R) if rows is None else rows
    return map_rows(lambda rs: orc.sparse_attn(q_attn[rs], kv, indices[rs], scale), rows, threads)


def row_scores_fn(orc, inputs):
    """r -> the oracle's float32 scores of every visible block of row r."""
    if len(inputs) == 7:
        return lambda r: orc.row_scores_fp8(r, *inputs)
    return lambda r: orc.row_scores(r, *inputs)


def band_problem(g: np.ndarray, o: np.ndarray, V: int, T: int, scores) -> str | None:
    """None when GPU row g passes the N(0,1) selection rule against oracle
    row o (V visible blocks, T tail tokens); else what fails.  `scores` is
    the oracle's float32 score array of the row, or a callable returning it
    (only called when the two rows differ: an identical row passes)."""
    n = min(512, V)
    width = 4 * n + T
    if not np.all(g[width:] == -1):
        return "padding"
    if not np.array_equal(g[4 * n:width], 4 * V + np.arange(T)):
        return "tail"
    if np.array_equal(g, o):
        return None
    quads = g[:4 * n].reshape(n, 4)
    if not np.all(quads[:, 0] % 4 == 0):
        return "block start"
    if not np.array_equal(quads, quads[:, :1] + np.arange(4)):
        return "quadruple"
    bg = quads[:, 0] // 4
    bo = o[:4 * n].reshape(n, 4)[:, 0] // 4
    if len(np.unique(bg)) != n or np.any(bg >= V) or np.any(bg < 0):
        return "blocks"
    if n == 0:
        return None
    sc = (scores() if callable(scores) else scores).astype(np.float64)
    s_n = sc[bo[-1]]
    band = BAND * max(abs(s_n), 1.0)
    diff = np.setxor1d(bg, bo)
    bad = diff[np.abs(sc[diff] - s_n) > band]
    if bad.size:
        return f"{bad.size} blocks differ outside the band"
    sg = sc[bg]
    tol = BAND * np.maximum(np.abs(sg[1:]), 1.0)
    if not np.all(sg[:-1] >= sg[1:] - tol):
        return "order"
    return None


def band_problems(orc, gpu: np.ndarray, ref: np.ndarray, inputs, rows=None, row_scores=None,
                  threads: int | None = None) -> dict:
    """{row: problem} over the listed rows (all by default) of a GPU
    selection `gpu` against the oracle's `ref` (both indexed by row);
    row_scores(r) overrides the oracle's unweighted scores (e.g. weighted
    ones).  Rows are checked in a thread pool."""
    *_, bt, t2r, sl, qp = inputs
    rows = list(range(len(t2r))) if rows is None else [int(r) for r in rows]
    scores_of = row_scores or row_scores_fn(orc, inputs)

    def one(r):
        V, T = orc.row_extent(int(sl[t2r[r]]), int(qp[r]))
        return band_problem(gpu[r], ref[r], V, T, lambda: scores_of(r))

    n = threads or host_threads()
    if n == 1 or len(rows) < 2:
        res = [one(r) for r in rows]
    else:
        with ThreadPoolExecutor(min(n, len(rows))) as ex:
            res = list(ex.map(one, rows))
    return {r: p for r, p in zip(rows, res) if p is not None}


def attn_error(got16: np.ndarray, want64: np.ndarray) -> tuple[float, int]:
    """(max |gpu - oracle|, elements more than one fp16 ulp from the oracle
    rounded to fp16, the ulp floored at that of 2^-10)."""
    got = got16.astype(np.float64)
    err = float(np.max(np.abs(got - want64))) if got.size else 0.0
    ref16 = want64.astype(np.float16)
    ulp = np.maximum(np.abs(np.spacing(ref16)), np.spacing(np.float16(2.0 ** -10))).astype(np.float64)
    over = int(np.count_nonzero(np.abs(got - ref16.astype(np.float64)) > ulp + 1e-12))
    return err, over
