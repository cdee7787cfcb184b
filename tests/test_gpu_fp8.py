"""GPU parity of the e4m3 key-cache entry points (qsa_select_fp8,
qsa_decode_step_fp8) against the CPU oracle.

Integer-valued keys re-encoded as e4m3 codes with power-of-two scales
dequantize to exactly the fp16 keys, and every fp32 sum stays exact, so the
selection is bit-exact (and equal to the fp16 path's); absmax-quantized
N(0,1) keys follow the band rule."""

import numpy as np
import pytest
import torch

from paged_top_indexer_amd import workloads as wl
import paged_top_indexer_amd as qsa
from gpu_util import (banner, check_attn, check_select_band, dev, dev_e4m3, oracle_attn,
                      oracle_select, orc, select_gpu, select_gpu_fp8)
from test_gpu_select import PLAN_CASES, integer_inputs

pytestmark = pytest.mark.gpu
SCALE = wl.SOFTMAX_SCALE


@pytest.mark.parametrize("make", [wl.tiny_integer, wl.ties_and_edges,
                                  lambda s: wl.multi_token_rows(s, integer=True)],
                         ids=["tiny", "edges", "multi_token"])
def test_integer_workloads_bit_exact(make):
    w = wl.with_fp8_keys(make(0), integer=True)
    banner(f"select_fp8 {w.name}")
    got = select_gpu_fp8(*w.select_inputs_fp8())
    want = orc().select_fp8(*w.select_inputs_fp8())
    bad = np.flatnonzero(~np.all(got == want, axis=1))
    assert bad.size == 0, f"rows differ: {bad[:10]}"
    # the same keys through the fp16 path
    assert np.array_equal(got, select_gpu(*w.select_inputs()))


@pytest.mark.parametrize("rows,width,lengths", PLAN_CASES,
                         ids=[f"R{c[0]}_W{c[1]}" for c in PLAN_CASES])
def test_integer_plans_bit_exact(rows, width, lengths):
    pages = max(64, sum(wl.pages_needed(L) for L in lengths) // 4 + 8)
    q, kcache, bt, t2r, sl, qp = integer_inputs(rows * 7 + width + 1, lengths, width, pages,
                                                palette=5, q_range=1)
    codes, scales = wl.fp8_integer_keys(np.random.default_rng(rows + width), kcache)
    banner(f"select_fp8 integer R={rows} W={width}")
    got = select_gpu_fp8(q, codes, scales, bt, t2r, sl, qp)
    want = orc().select_fp8(q, codes, scales, bt, t2r, sl, qp)
    bad = np.flatnonzero(~np.all(got == want, axis=1))
    assert bad.size == 0, f"rows differ: {bad[:10]}"


def test_every_code_and_scale():
    """One-hot queries read every finite code back through the kernel's
    decoding: block i holds code c_i at dim 7 (zeros elsewhere) with scale
    2^j; head 0 = +1 and head 1 = -1 on dim 7, so block i scores
    2^j * |e4m3(c_i)| exactly, with many exact ties across codes and scales,
    and the selection is the oracle's exactly."""
    rng = np.random.default_rng(4)
    codes_all = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    n = 3 * codes_all.size  # every code three times, with different scales (> 512 blocks)
    pages = -(-n // 128)
    codes = np.zeros((pages, 128, 1, 128), np.uint8)
    b = np.arange(n)
    codes[b // 128, b % 128, 0, 7] = np.concatenate(
        [codes_all, rng.permutation(codes_all), rng.permutation(codes_all)])
    scales = np.ldexp(np.float32(1), rng.integers(-6, 7, size=(pages, 128))).astype(np.float32)
    q = np.zeros((1, 4, 128), np.float16)
    q[0, 0, 7], q[0, 1, 7] = 1.0, -1.0
    bt = np.arange(pages, dtype=np.int32).reshape(1, pages)
    t2r, sl, qp = wl.decode_rows([4 * n + 2])
    banner("select_fp8 every code")
    got = select_gpu_fp8(q, codes, scales, bt, t2r, sl, qp)
    want = orc().select_fp8(q, codes, scales, bt, t2r, sl, qp)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("make", [wl.saturated_row, wl.batched_shared], ids=["saturated", "batched"])
def test_normal_band(make):
    w = wl.with_fp8_keys(make(0), integer=False)
    inputs = w.select_inputs_fp8()
    banner(f"select_fp8 {w.name}")
    got = select_gpu_fp8(*inputs)
    want = orc().select_fp8(*inputs)
    check_select_band(got, want, orc(), inputs, range(w.rows))
    banner(f"rows identical to the oracle: {np.mean(np.all(got == want, axis=1)):.3f}")


def test_long_context_full_size():
    """The bench's e4m3 workload and launch configuration, every row: the
    selection against the oracle's (band rule) and the decode step's
    attention against the oracle over its own index rows."""
    w = wl.with_fp8_keys(wl.long_context(0), integer=False)
    inputs = w.select_inputs_fp8()
    banner("decode_step_fp8 long_context R=128 L=131072 (full size)")
    kvd = dev(w.kv)
    k, v = qsa.kv_views(kvd)
    q, codes, scales, bt, t2r, sl, qp = inputs
    idx, out = qsa.qsa_decode_step_fp8(dev(q), dev_e4m3(codes), dev(scales), dev(bt), dev(t2r),
                                       dev(sl), dev(qp), dev(w.q_attn), k, v, SCALE)
    torch.cuda.synchronize()
    got, out = idx.cpu().numpy(), out.cpu().numpy()
    want = oracle_select(orc(), inputs)
    check_select_band(got, want, orc(), inputs, range(w.rows))
    banner(f"rows identical to the oracle: {int(np.all(got == want, axis=1).sum())}/{w.rows}")
    for r in range(w.rows):
        b = got[r, :2048:4] // 4
        assert np.all(got[r, 2048:] == -1)
        assert len(np.unique(b)) == 512 and b.min() >= 0 and b.max() < 32768
    check_attn(out, oracle_attn(orc(), w.q_attn, w.kv, got, SCALE), "fp8 decode, every row")
    # the selection stage alone gives the same indices
    alone = select_gpu_fp8(*inputs)
    assert np.array_equal(alone, got)


def test_fail_closed_through_binding():
    w = wl.with_fp8_keys(wl.tiny_integer(0), integer=True)
    q, codes, scales, bt, t2r, sl, qp = [dev(a) for a in w.select_inputs_fp8()]
    codes8 = codes.view(torch.float8_e4m3fn)
    out = torch.full((1, 2051), 77, dtype=torch.int32, device=q.device)
    with pytest.raises(RuntimeError, match="QSA_ERR_DTYPE"):
        qsa.qsa_select_fp8(q, codes, scales, bt, t2r, sl, qp, out=out)  # uint8, not e4m3
    with pytest.raises(RuntimeError, match="QSA_ERR_SHAPE"):
        qsa.qsa_select_fp8(q, codes8, scales[:, :64].contiguous(), bt, t2r, sl, qp, out=out)
    with pytest.raises(RuntimeError, match="QSA_ERR_DTYPE"):
        qsa.qsa_select(q, codes8, bt, t2r, sl, qp, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 77)


def e4m3_value(c: int) -> float:
    """The value of an OCP e4m3 code from its bit fields: sign bit 7,
    exponent bits 6..3 with bias 7, fraction bits 2..0; exponent 0 is
    subnormal (fraction/8 * 2^-6)."""
    sign = -1.0 if c & 0x80 else 1.0
    e, m = (c >> 3) & 0xF, c & 7
    return sign * (m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))


def test_every_code_logits():
    """Sign and magnitude of every finite code, read back as scores: key i
    holds code c_i at dim 7 with scale 2^j; head 0 = +1 and head 1 = -1/2 on
    dim 7, so the key scores 2^j * v for v = e4m3(c_i) >= 0 and
    2^j * |v| / 2 for v < 0, exactly (a sign error or a wrong exponent bias
    changes the value)."""
    rng = np.random.default_rng(5)
    codes_all = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    n = 2 * codes_all.size
    pages = -(-n // 128)
    codes = np.zeros((pages, 128, 1, 128), np.uint8)
    b = np.arange(n)
    per_key = np.concatenate([codes_all, rng.permutation(codes_all)])
    codes[b // 128, b % 128, 0, 7] = per_key
    exps = rng.integers(-6, 7, size=(pages, 128))
    scales = np.ldexp(np.float32(1), exps).astype(np.float32)
    q = np.zeros((1, 4, 128), np.float16)
    q[0, 0, 7], q[0, 1, 7] = 1.0, -0.5
    bt = np.arange(pages, dtype=np.int32).reshape(1, pages)
    t2r, sl, qp = wl.decode_rows([4 * n + 1])
    banner("paged_logits e4m3 every code, signed")
    lg = qsa.qsa_paged_logits(dev(q), dev_e4m3(codes), dev(bt), dev(t2r), dev(sl), dev(qp),
                              kscale=dev(scales))
    torch.cuda.synchronize()
    lg = lg.cpu().numpy()[0]
    v = np.array([e4m3_value(int(c)) for c in per_key])
    want = np.where(v >= 0, v, -v / 2) * np.ldexp(1.0, exps.reshape(-1)[:n])
    assert np.array_equal(lg[:n], want.astype(np.float32))
    assert np.all(np.isneginf(lg[n:]))
