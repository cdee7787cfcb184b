"""Seeded random sweep of selection configurations against the oracle,
bit-exact on integer inputs: batch sizes, row lengths and table widths that
pick every chunk size of both plans, shared physical pages, palettes that
force exact ties, padded rows, queries passed row by row or as runs of n
rows, fp16 or e4m3 keys, with or without per-head weights.  Each case is
drawn from its own seed, so a failure names a reproducible configuration."""

import numpy as np
import pytest
import torch

from paged_top_indexer_amd import workloads as wl
import paged_top_indexer_amd as qsa
from gpu_util import banner, check_attn, dev, dev_e4m3, orc

pytestmark = pytest.mark.gpu

CASES = 24


def random_case(seed: int, n_req: int | None = None, run: int | None = None,
                fixed_hint: int | None = None, fp8_keys: bool | None = None):
    """A random configuration; n_req, run, the runs hint and the key cache's
    format may be fixed instead (the draws are made either way, so the
    other choices stay those of the seed)."""
    rng = np.random.default_rng(1000 + seed)
    n_draw = int(rng.integers(1, 40))
    n_req = n_draw if n_req is None else n_req
    run_draw = int(rng.choice([1, 1, 2, 3, 4, 5, 8]))  # rows per request (and the runs hint)
    run = run_draw if run is None else run
    long_tail = rng.random() < 0.5
    hi = 131072 if long_tail else 20000
    lengths = rng.integers(0, hi, size=n_req)
    tiny = rng.random(n_req) < 0.1  # empty and shorter-than-a-block requests
    lengths[tiny] = rng.integers(0, 8, size=int(tiny.sum()))
    need = [wl.pages_needed(int(L)) for L in lengths]
    width = max(need + [1]) + int(rng.integers(0, 3))
    P = max(16, sum(need) // int(rng.choice([1, 2, 4])) + 4)  # pages may be shared by chance
    palette = int(rng.choice([0, 3, 16]))
    if palette:
        pal = wl.int_f16(rng, -4, 4, (palette, 128))
        kcache = pal[rng.integers(0, palette, size=(P, 128))].reshape(P, 128, 1, 128)
    else:
        kcache = wl.int_f16(rng, -4, 4, (P, 128, 1, 128))
    bt = np.full((n_req, width), -1, dtype=np.int32)
    for i, n in enumerate(need):
        if n:
            bt[i, :n] = rng.choice(P, size=n, replace=n > P)
    t2r = np.repeat(np.arange(n_req, dtype=np.int32), run)
    qp = np.concatenate([int(L) - run + np.arange(run) for L in lengths]).astype(np.int64)
    pad = rng.random(t2r.size) < 0.05
    qp[pad] = -1
    q = wl.int_f16(rng, -2 if palette else -4, 2 if palette else 4, (t2r.size, 4, 128))
    fp8 = rng.random() < 0.3
    fp8 = fp8 if fp8_keys is None else fp8_keys
    weights = wl.head_weights(rng, t2r.size, integer=True) if rng.random() < 0.3 else None
    hint = run if rng.random() < 0.7 else 1
    hint = hint if fixed_hint is None else fixed_hint
    return dict(q=q, kcache=kcache, bt=bt, t2r=t2r, sl=lengths.astype(np.int32), qp=qp, fp8=fp8,
                weights=weights, hint=hint, rng=rng, desc=f"seed={seed} reqs={n_req} run={run} "
                f"hint={hint} W={width} P={P} palette={palette} fp8={fp8} weights={weights is not None}")


@pytest.mark.parametrize("seed", range(CASES))
def test_random_selection_bit_exact(seed):
    c = random_case(seed)
    q, kcache, bt, t2r, sl, qp = c["q"], c["kcache"], c["bt"], c["t2r"], c["sl"], c["qp"]
    R = q.shape[0]
    banner(f"random selection R={R} {c['desc']}")
    if c["weights"] is not None:
        want = orc().select_weighted(q, c["weights"], bt, t2r, sl, qp, kcache=kcache)
    else:
        want = orc().select(q, kcache, bt, t2r, sl, qp)
    qd = dev(q)
    if c["hint"] > 1:
        qd = qd.view(R // c["hint"], c["hint"], 4, 128)
    args = [dev(bt), dev(t2r), dev(sl), dev(qp)]
    if c["fp8"]:
        codes, scales = wl.fp8_integer_keys(c["rng"], kcache)
        kc, ks = dev_e4m3(codes), dev(scales)
    else:
        kc, ks = dev(kcache), None
    if c["weights"] is not None:
        got = qsa.qsa_select_weighted(qd, dev(c["weights"]), kc, *args, kscale=ks)
    elif c["fp8"]:
        got = qsa.qsa_select_fp8(qd, kc, ks, *args)
    else:
        got = qsa.qsa_select(qd, kc, *args)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    bad = np.flatnonzero(~np.all(got == want, axis=1))
    assert bad.size == 0, f"{c['desc']}: rows differ: {bad[:10]}"


DECODE_CASES = 8


def run_decode_case(c, seed):
    """The decode step on configuration c: index rows bit-exact against the
    oracle, attention against the oracle over those index rows."""
    q, kcache, bt, t2r, sl, qp = c["q"], c["kcache"], c["bt"], c["t2r"], c["sl"], c["qp"]
    R = q.shape[0]
    rng = np.random.default_rng(5000 + seed)
    kv_pages = -(-int(max(int(sl.max()), 1)) // 512) + 1
    kv = wl.normal_f16(rng, (kv_pages, 512, 512))
    q_attn = wl.normal_f16(rng, (R, 3, 256))
    scale = wl.SOFTMAX_SCALE
    banner(f"random decode step R={R} {c['desc']} kv_pages={kv_pages}")
    want = orc().select(q, kcache, bt, t2r, sl, qp)
    qd = dev(q)
    if c["hint"] > 1:
        qd = qd.view(R // c["hint"], c["hint"], 4, 128)
    k, v = qsa.kv_views(dev(kv))
    args = [dev(bt), dev(t2r), dev(sl), dev(qp), dev(q_attn), k, v, scale]
    if c["fp8"]:
        codes, scales = wl.fp8_integer_keys(c["rng"], kcache)
        idx, out = qsa.qsa_decode_step_fp8(qd, dev_e4m3(codes), dev(scales), *args)
    else:
        idx, out = qsa.qsa_decode_step(qd, dev(kcache), *args)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    bad = np.flatnonzero(~np.all(idx == want, axis=1))
    assert bad.size == 0, f"{c['desc']}: rows differ: {bad[:10]}"
    check_attn(out.cpu().numpy(), orc().sparse_attn(q_attn, kv, idx, scale), c["desc"])


@pytest.mark.parametrize("seed", range(DECODE_CASES))
def test_random_decode_step(seed):
    """The decode step over the same kind of random configurations (no head
    weights: the decode step has none): its index rows bit-exact against the
    oracle, its attention against the oracle's over those index rows.  Batch
    sizes from 1 to ~300 rows cover both attention plans, and with them the
    decode steps that select inside the attention launch and those that
    launch a merge."""
    run_decode_case(random_case(100 + seed), seed)


# (requests, rows per request) at the row counts where the grid placement
# changes -- one row on one XCD; single rows dealt over the XCDs (chunks in
# cells of 4 rows, attention splits row by row) except the attention's XCD
# groups at multiples of 32 rows; runs of 4 rows dealt below 32 runs and in
# XCD groups from 32 -- and where the attention plan changes (8 rows).
PLACEMENT_CASES = [(1, 1), (7, 1), (8, 1), (31, 1), (32, 1), (33, 1), (65, 1), (96, 1),
                   (31, 4), (32, 4), (33, 4)]


@pytest.mark.parametrize("n_req,run", PLACEMENT_CASES,
                         ids=[f"R{n * r}_run{r}" for n, r in PLACEMENT_CASES])
def test_decode_step_placement_boundaries(n_req, run):
    """Random integer configurations (fp16 keys) with the batch size fixed
    at a placement or plan boundary; runs of 4 rows passed as runs."""
    seed = 300 + n_req * run
    run_decode_case(random_case(seed, n_req=n_req, run=run, fixed_hint=run, fp8_keys=False),
                    seed)
