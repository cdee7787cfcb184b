"""qsa_decode_step_noalloc (the decode step over the library's fixed
per-GPU scratch, for callers that cannot allocate) through the C ABI,
against qsa_decode_step with a workspace on the same inputs: identical
indices and outputs on consecutive calls, each smaller than the one before
(the scratch keeps the previous call's bytes), and a call too large for the
scratch refused before anything is launched."""

import numpy as np
import pytest
import torch

from paged_top_indexer_amd import workloads as wl
import paged_top_indexer_amd as qsa
from gpu_util import banner, check_attn, dev, orc

pytestmark = pytest.mark.gpu
SCALE = wl.SOFTMAX_SCALE


def both_ways(w, runs: int = 1):
    sel = [dev(a) for a in w.select_inputs()]
    if runs > 1:
        sel[0] = sel[0].view(w.rows // runs, runs, 4, 128)
    k, v = qsa.kv_views(dev(w.kv))
    q = dev(w.q_attn)
    ref_idx, ref_out = qsa.qsa_decode_step(*sel, q, k, v, SCALE)
    idx = torch.full((w.rows, 2051), -7, dtype=torch.int32, device=q.device)
    out = torch.full((w.rows, 3, 256), 1.5, dtype=torch.float16, device=q.device)
    qsa.qsa_decode_step_noalloc(*sel, q, k, v, SCALE, idx, out)
    torch.cuda.synchronize()
    return ref_idx.cpu().numpy(), ref_out.cpu().numpy(), idx.cpu().numpy(), out.cpu().numpy()


def test_noalloc_equals_decode_step_on_consecutive_calls():
    # 1: 256 multi-token rows as runs of 4 (grouped chunks, merge, attention
    #    splits and combine: the most scratch of the three)
    # 2: 64 batched rows (row-by-row chunks, merge, splits)
    # 3: one 519-token row (a single chunk, 33 attention splits)
    cases = [(wl.multi_token_rows(0), 4), (wl.batched_shared(0), 1), (wl.tiny_integer(0), 1)]
    sizes = []
    for w, runs in cases:
        need = qsa.decode_step_workspace_bytes(w.rows, w.block_table.shape[1])
        sizes.append(need)
        banner(f"noalloc decode {w.name} R={w.rows} runs={runs} (workspace query {need} B)")
        ref_idx, ref_out, idx, out = both_ways(w, runs)
        assert np.array_equal(idx, ref_idx), f"{w.name}: indices differ"
        assert np.array_equal(out.view(np.uint16), ref_out.view(np.uint16)), f"{w.name}: out differs"
    assert sizes[0] > sizes[1] > sizes[2] >= 0
    # the last call's integer selection is the oracle's, its attention within the bounds
    w = cases[2][0]
    want = orc().select(*w.select_inputs())
    assert np.array_equal(idx, want)
    check_attn(out, orc().sparse_attn(w.q_attn, w.kv, want, SCALE), "noalloc tiny")


def test_noalloc_refuses_a_call_too_large_for_the_scratch():
    # 4096 rows over a 256-page table: ~64 MiB of candidates > 32 MiB
    R, W = 4096, 256
    d = "cuda:0"
    q = torch.zeros((R, 4, 128), dtype=torch.float16, device=d)
    kcache = torch.zeros((1, 128, 1, 128), dtype=torch.float16, device=d)
    bt = torch.zeros((R, W), dtype=torch.int32, device=d)
    t2r = torch.arange(R, dtype=torch.int32, device=d)
    sl = torch.full((R,), 128 * W * 4, dtype=torch.int32, device=d)
    qp = (sl.to(torch.int64) - 1)
    q_attn = torch.zeros((R, 3, 256), dtype=torch.float16, device=d)
    k, v = qsa.kv_views(torch.zeros((1, 512, 512), dtype=torch.float16, device=d))
    idx = torch.full((R, 2051), 5, dtype=torch.int32, device=d)
    out = torch.full((R, 3, 256), 2.0, dtype=torch.float16, device=d)
    assert qsa.decode_step_workspace_bytes(R, W) > 32 << 20
    with pytest.raises(RuntimeError, match="QSA_ERR_WORKSPACE"):
        qsa.qsa_decode_step_noalloc(q, kcache, bt, t2r, sl, qp, q_attn, k, v, SCALE, idx, out)
    torch.cuda.synchronize()
    assert torch.all(idx == 5) and torch.all(out == 2.0)
