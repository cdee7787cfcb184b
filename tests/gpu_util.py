"""Helpers shared by the GPU parity tests: device copies, calls through the
C ABI (via the binding) and the comparison rules.

Comparison rules
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
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
import paged_top_indexer_amd as qsa

DEV = "cuda:0"
ATTN_TOL = 2e-3
BAND = 1e-3


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def banner(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)


def select_gpu(q, kcache, bt, t2r, sl, qp) -> np.ndarray:
    out = qsa.qsa_select(dev(q), dev(kcache), dev(bt), dev(t2r), dev(sl), dev(qp))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def dev_e4m3(codes: np.ndarray) -> torch.Tensor:
    """uint8 e4m3 codes as a float8_e4m3fn device tensor (same bytes)."""
    return dev(codes.astype(np.uint8)).view(torch.float8_e4m3fn)


def select_gpu_fp8(q, codes, scales, bt, t2r, sl, qp) -> np.ndarray:
    out = qsa.qsa_select_fp8(dev(q), dev_e4m3(codes), dev(scales), dev(bt), dev(t2r), dev(sl),
                             dev(qp))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def attn_gpu(q, kv, idx, scale) -> np.ndarray:
    kvd = dev(kv.reshape(-1, 512, 512))
    k, v = qsa.kv_views(kvd)
    out = qsa.qsa_sparse_attn(dev(q), k, v, dev(idx), scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_attn(got16: np.ndarray, want64: np.ndarray, what: str = "") -> float:
    got = got16.astype(np.float64)
    err = float(np.max(np.abs(got - want64))) if got.size else 0.0
    assert err <= ATTN_TOL, f"{what}: max abs error {err:.3e} > {ATTN_TOL}"
    # at most one fp16 ulp from the float64 oracle rounded to fp16 (the ulp
    # floored at that of 2^-10)
    ref16 = want64.astype(np.float16)
    ulp = np.maximum(np.abs(np.spacing(ref16)), np.spacing(np.float16(2.0 ** -10))).astype(np.float64)
    assert np.all(np.abs(got - ref16.astype(np.float64)) <= ulp + 1e-12), f"{what}: > 1 ulp"
    return err


def check_select_band(gpu: np.ndarray, ref: np.ndarray, orc, inputs, rows,
                      row_scores=None) -> None:
    """The N(0,1) acceptance rule on the listed rows (inputs as passed to the
    oracle -- six for an fp16 cache, seven with codes and scales for an e4m3
    cache -- and rows as indices into them).  row_scores(r), when given,
    returns the oracle's scores of row r (e.g. weighted ones)."""
    if row_scores is not None:
        q, *_, bt, t2r, sl, qp = inputs
    elif len(inputs) == 7:
        q, codes, scales, bt, t2r, sl, qp = inputs
        row_scores = lambda r: orc.row_scores_fp8(r, *inputs)  # noqa: E731
    else:
        q, kcache, bt, t2r, sl, qp = inputs
        row_scores = lambda r: orc.row_scores(r, *inputs)  # noqa: E731
    for r in rows:
        g, o = gpu[r], ref[r]
        V, T = orc.row_extent(int(sl[t2r[r]]), int(qp[r]))
        n = min(512, V)
        width = 4 * n + T
        assert np.all(g[width:] == -1), f"row {r}: padding"
        assert np.array_equal(g[4 * n:width], 4 * V + np.arange(T)), f"row {r}: tail"
        quads = g[:4 * n].reshape(n, 4)
        assert np.all(quads[:, 0] % 4 == 0), f"row {r}: block start"
        assert np.array_equal(quads, quads[:, :1] + np.arange(4)), f"row {r}: quadruple"
        bg = quads[:, 0] // 4
        bo = o[:4 * n].reshape(n, 4)[:, 0] // 4
        assert len(np.unique(bg)) == n and np.all(bg < V) and np.all(bg >= 0), f"row {r}: blocks"
        if n == 0:
            continue
        scores = row_scores(r).astype(np.float64)
        s_n = scores[bo[-1]]
        band = BAND * max(abs(s_n), 1.0)
        diff = np.setxor1d(bg, bo)
        bad = diff[np.abs(scores[diff] - s_n) > band]
        assert bad.size == 0, f"row {r}: {bad.size} blocks differ outside the band"
        sg = scores[bg]
        tol = BAND * np.maximum(np.abs(sg[1:]), 1.0)
        assert np.all(sg[:-1] >= sg[1:] - tol), f"row {r}: order"


def subset_rows(inputs, rows):
    """Selection inputs restricted to some query rows (requests unchanged);
    six (fp16 cache) or seven (e4m3 codes + scales) inputs."""
    rows = np.asarray(rows)
    q, *cache, bt, t2r, sl, qp = inputs
    return (q[rows], *cache, bt, t2r[rows], sl, qp[rows])


def orc():
    return oracle.default()
