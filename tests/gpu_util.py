"""Helpers shared by the GPU parity tests: device copies, calls through the
C ABI (via the binding) and the comparison rules of ``oracle.acceptance``
(selection bit-exact on integer inputs, the band rule on N(0,1) inputs,
attention within 2e-3 and one fp16 ulp of the float64 oracle).
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
from oracle import acceptance
from oracle.acceptance import ATTN_TOL, oracle_attn, oracle_select, subset_rows  # noqa: F401
import paged_top_indexer_amd as qsa

DEV = "cuda:0"


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
    err, over = acceptance.attn_error(got16, want64)
    assert err <= ATTN_TOL, f"{what}: max abs error {err:.3e} > {ATTN_TOL}"
    assert over == 0, f"{what}: {over} elements more than one fp16 ulp from the oracle"
    return err


def check_select_band(gpu: np.ndarray, ref: np.ndarray, orc, inputs, rows,
                      row_scores=None) -> None:
    """The N(0,1) acceptance rule on the listed rows (inputs as passed to the
    oracle -- six for an fp16 cache, seven with codes and scales for an e4m3
    cache -- and rows as indices into them and into gpu/ref).
    row_scores(r), when given, returns the oracle's scores of row r (e.g.
    weighted ones).  Rows are checked in a thread pool."""
    bad = acceptance.band_problems(orc, gpu, ref, inputs, rows, row_scores=row_scores)
    assert not bad, f"{len(bad)} rows fail the band rule: {dict(list(bad.items())[:5])}"


def orc():
    return oracle.default()
