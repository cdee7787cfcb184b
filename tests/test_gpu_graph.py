"""The decode step captured in a HIP graph (torch.cuda.CUDAGraph).  A call
of the library only launches kernels -- no allocation, no memset, no host
sync -- so a capture of qsa_decode_step replays the whole path.  Each replay
is checked against an eager call on the same inputs (the kernels are
deterministic: identical bits), with the queries changed and eager work run
between replays; the integer batch's first replay is also checked against
the oracle."""

import numpy as np
import pytest
import torch

from paged_top_indexer_amd import workloads as wl
import paged_top_indexer_amd as qsa
from gpu_util import DEV, banner, check_attn, dev, dev_e4m3, orc

pytestmark = pytest.mark.gpu
SCALE = wl.SOFTMAX_SCALE


@pytest.mark.parametrize("case", ["multi_token_runs_integer", "batched_normal", "batched_e4m3"])
def test_decode_step_graph_replays(case):
    integer = case.endswith("integer")
    fp8 = case.endswith("e4m3")
    w = wl.multi_token_rows(0, integer=True) if integer else wl.batched_shared(0)
    if fp8:
        w = wl.with_fp8_keys(w, integer=False)
    run = 4 if integer else 1
    R = w.rows
    banner(f"decode step graph replays: {w.name} R={R} rows_per_run={run} e4m3={fp8}")
    qd = dev(w.q_sel)
    qv = qd.view(R // run, run, 4, 128) if run > 1 else qd
    bt, t2r, sl, qp = (dev(a) for a in (w.block_table, w.token_to_req, w.seq_lens, w.query_pos))
    if fp8:
        keys = (dev_e4m3(w.kcodes), dev(w.kscale))
        decode = qsa.qsa_decode_step_fp8
    else:
        keys = (dev(w.kcache),)
        decode = qsa.qsa_decode_step
    k, v = qsa.kv_views(dev(w.kv))
    qa = dev(w.q_attn)
    ws_bytes = max(1, qsa.decode_step_workspace_bytes(R, w.block_table.shape[1]))
    ws_g = torch.zeros(ws_bytes, dtype=torch.uint8, device=DEV)
    ws_e = torch.zeros(ws_bytes, dtype=torch.uint8, device=DEV)
    idx_g = torch.empty((R, 2051), dtype=torch.int32, device=DEV)
    out_g = torch.empty((R, 3, 256), dtype=torch.float16, device=DEV)

    def step():
        decode(qv, *keys, bt, t2r, sl, qp, qa, k, v, SCALE, indices=idx_g, out=out_g,
               workspace=ws_g)

    step()  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    rng = np.random.default_rng(8)
    for rep in range(3):
        if rep:
            q_new = (wl.int_f16(rng, -4, 4, w.q_sel.shape) if integer
                     else wl.normal_f16(rng, w.q_sel.shape))
            qd.copy_(dev(q_new))
        idx_g.fill_(-7)
        out_g.fill_(7)
        g.replay()
        torch.cuda.synchronize()
        gi, go = idx_g.cpu().numpy(), out_g.cpu().numpy()
        # eager: the same inputs into buffers of its own
        ei, eo = decode(qv, *keys, bt, t2r, sl, qp, qa, k, v, SCALE, workspace=ws_e)
        torch.cuda.synchronize()
        assert np.array_equal(gi, ei.cpu().numpy()), f"replay {rep}: indices differ from eager"
        assert np.array_equal(go, eo.cpu().numpy()), f"replay {rep}: output differs from eager"
        if integer and rep == 0:
            q_host = qd.cpu().numpy()
            want = orc().select(q_host, w.kcache, w.block_table, w.token_to_req, w.seq_lens,
                                w.query_pos)
            assert np.array_equal(gi, want)
            rows = [0, 5, R - 1]
            check_attn(go[rows], orc().sparse_attn(w.q_attn[rows], w.kv, want[rows], SCALE),
                       "graph replay")
