"""The C-ABI library on the host: it loads, exports every declared symbol,
reports the contract constants and rejects bad arguments before launching
anything (descriptors point at fake device addresses; no call here reaches
a kernel launch)."""

import ctypes
import os
import re

import pytest

from paged_top_indexer_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")

OK, NULL, DTYPE, SHAPE, LAYOUT, ALIAS, WORKSPACE, ARG = 0, 1, 2, 3, 4, 5, 6, 7


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"QSA_API\s+[\w\s\*]+?\b(qsa_\w+)\s*\(", text)


def test_exports_every_declared_symbol():
    lib = B.library()
    names = declared_symbols()
    assert {"qsa_select", "qsa_sparse_attn", "qsa_decode_step"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_constants_and_status_strings():
    assert B.constants() == (2048, 4, 2051, 512)
    lib = B.library()
    assert lib.qsa_status_string(0) == b"QSA_OK"
    assert lib.qsa_status_string(4) == b"QSA_ERR_LAYOUT"


def test_workspace_sizes():
    assert B.select_workspace_bytes(0, 256) == 0
    assert B.sparse_attn_workspace_bytes(0) == 0
    # one chunk per row needs no workspace: a table of at most 4 pages (512
    # blocks, no top-k) is one chunk whatever the batch
    assert B.select_workspace_bytes(1, 1) == 0
    assert B.select_workspace_bytes(1, 4) == 0 and B.select_workspace_bytes(4096, 3) == 0
    assert B.select_workspace_bytes(1, 5) > 0
    big = B.select_workspace_bytes(128, 256)
    # 32-page chunks: 8 chunks per row, 512 candidates (key + block) each
    assert big >= 128 * 8 * 512 * 8
    assert B.decode_step_workspace_bytes(128, 256) >= big + B.sparse_attn_workspace_bytes(128)
    assert B.sparse_attn_workspace_bytes(128) > 0
    # few rows of a long table: 1024 workgroups would mean 1-page chunks
    # (256 chunks x 128 candidates per row, 4 merge batches); the chunks grow
    # until a row's candidates fit one merge batch of 8192 where the largest
    # chunk allows -- 16 x 512 for single rows, and for row groups (largest
    # chunk 8 pages) 32 x 512, which sizes the workspace: two uint32 arrays
    assert B.select_workspace_bytes(4, 256) == 2 * (4 * 32 * 512 * 4)
    # a row that fits one batch already keeps its 1024-workgroup chunks
    assert B.select_workspace_bytes(4, 64) == 2 * (4 * 64 * 128 * 4)
    # 2 rows: 4-wave attention workgroups, 33 splits of 64 positions --
    # partials, then (max, sum) rounded up to 256 bytes
    assert B.sparse_attn_workspace_bytes(2) == 2 * 33 * 3 * 256 * 4 + 1792
    # the decode step of a 40-page table: 40 one-page chunks of 128
    # candidates per row (5120 <= 8192), selected inside whole-CU attention
    # workgroups, 11 splits of 192 positions
    assert B.decode_step_workspace_bytes(2, 40) == 2 * (2 * 40 * 128 * 4) + (
        2 * 11 * 3 * 256 * 4 + 768)
    # 8 rows: whole-CU attention workgroups, 11 splits
    assert B.sparse_attn_workspace_bytes(8) == 8 * 11 * 3 * 256 * 4 + 2304
    # 300 rows: 4-wave workgroups, 3 splits of 704 positions
    assert B.sparse_attn_workspace_bytes(300) == 300 * 3 * 3 * 256 * 4 + 21760


# ---------------------------------------------------------------------------
# fake device memory: disjoint, 256-aligned address ranges

class Fake:
    next = 1 << 40  # shared by every instance: no two fake buffers overlap

    def alloc(self, nbytes):
        p = Fake.next
        Fake.next += ((nbytes + 4095) // 4096 + 1) * 4096
        return p


def contig(shape):
    st, acc = [], 1
    for s in reversed(shape):
        st.append(acc)
        acc *= s
    return tuple(reversed(st))


def mk(fake, dtype, shape, esize, stride=None, ptr=None):
    stride = stride or contig(shape)
    n = 1
    for s in shape:
        n *= s
    p = ptr if ptr is not None else fake.alloc(n * esize)
    return B.descriptor(p, dtype, shape, stride)


def select_args(R=4, P=8, N=4, W=3):
    f = Fake()
    a = dict(
        q=mk(f, B.F16, (R, 4, 128), 2),
        kcache=mk(f, B.F16, (P, 128, 1, 128), 2),
        bt=mk(f, B.I32, (N, W), 4),
        t2r=mk(f, B.I32, (R,), 4),
        sl=mk(f, B.I32, (N,), 4),
        qp=mk(f, B.I64, (R,), 8),
        out=mk(f, B.I32, (R, 2051), 4),
    )
    ws_bytes = B.select_workspace_bytes(R, W)
    return f, a, f.alloc(ws_bytes), ws_bytes


def call_select(a, ws, ws_bytes):
    lib = B.library()
    order = ["q", "kcache", "bt", "t2r", "sl", "qp", "out"]
    ptrs = [ctypes.byref(a[k]) if a[k] is not None else None for k in order]
    return lib.qsa_select(*ptrs, ctypes.c_void_p(ws), ws_bytes, None)


def attn_args(R=2, NP=4):
    f = Fake()
    base = f.alloc(NP * 512 * 512 * 2)
    k = B.descriptor(base, B.F16, (NP, 512, 1, 256), (262144, 512, 256, 1))
    v = B.descriptor(base + 512, B.F16, (NP, 512, 1, 256), (262144, 512, 256, 1))
    a = dict(q=mk(f, B.F16, (R, 3, 256), 2), k=k, v=v,
             idx=mk(f, B.I32, (R, 2051), 4), out=mk(f, B.F16, (R, 3, 256), 2))
    ws_bytes = B.sparse_attn_workspace_bytes(R)
    return f, a, f.alloc(ws_bytes), ws_bytes, base


def call_attn(a, ws, ws_bytes, scale=0.0625):
    lib = B.library()
    return lib.qsa_sparse_attn(ctypes.byref(a["q"]), ctypes.byref(a["k"]), ctypes.byref(a["v"]),
                               ctypes.byref(a["idx"]), ctypes.c_float(scale),
                               ctypes.byref(a["out"]), ctypes.c_void_p(ws), ws_bytes, None)


def test_descriptor_bytes():
    """The packed descriptor matches qsa_tensor field by field; more than 4
    dims keep ndim with the first 4 extents (the library rejects them)."""
    d = B.descriptor(0x1234560, B.I64, (3, 5), (5, 1))
    assert (d.data, d.dtype, d.ndim) == (0x1234560, B.I64, 2)
    assert list(d.shape) == [3, 5, 0, 0] and list(d.stride) == [5, 1, 0, 0]
    d5 = B.descriptor(256, B.F16, (1, 2, 3, 4, 5), (120, 60, 20, 5, 1))
    assert d5.ndim == 5 and list(d5.shape) == [1, 2, 3, 4] and list(d5.stride) == [120, 60, 20, 5]


def test_select_zero_rows_is_noop():
    f, a, ws, wsb = select_args(R=0)
    assert call_select(a, 0, 0) == OK


SELECT_CASES = {
    "q_dtype": (lambda f, a: a.__setitem__("q", mk(f, 0, (4, 4, 128), 4)), DTYPE),
    "q_heads": (lambda f, a: a.__setitem__("q", mk(f, B.F16, (4, 3, 128), 2)), SHAPE),
    "q_rank": (lambda f, a: a.__setitem__("q", mk(f, B.F16, (4, 512), 2)), SHAPE),
    "q_rank5": (lambda f, a: a.__setitem__("q", mk(f, B.F16, (1, 2, 2, 4, 128), 2)), SHAPE),
    "q_strided": (lambda f, a: a.__setitem__("q", mk(f, B.F16, (4, 4, 128), 2, stride=(1024, 256, 1))), LAYOUT),
    "q_misaligned": (lambda f, a: a.__setitem__("q", mk(f, B.F16, (4, 4, 128), 2, ptr=f.alloc(8192) + 2)), LAYOUT),
    "kcache_bf16": (lambda f, a: a.__setitem__("kcache", mk(f, 0, (8, 128, 1, 128), 2)), DTYPE),
    "kcache_slots": (lambda f, a: a.__setitem__("kcache", mk(f, B.F16, (8, 64, 1, 128), 2)), SHAPE),
    "kcache_heads": (lambda f, a: a.__setitem__("kcache", mk(f, B.F16, (8, 128, 2, 128), 2)), SHAPE),
    "kcache_empty": (lambda f, a: a.__setitem__("kcache", mk(f, B.F16, (0, 128, 1, 128), 2)), SHAPE),
    "table_i64": (lambda f, a: a.__setitem__("bt", mk(f, B.I64, (4, 3), 8)), DTYPE),
    "table_col_stride": (lambda f, a: a.__setitem__("bt", mk(f, B.I32, (4, 3), 4, stride=(6, 2))), LAYOUT),
    "t2r_rows": (lambda f, a: a.__setitem__("t2r", mk(f, B.I32, (5,), 4)), SHAPE),
    "seq_lens_i64": (lambda f, a: a.__setitem__("sl", mk(f, B.I64, (4,), 8)), DTYPE),
    "seq_lens_count": (lambda f, a: a.__setitem__("sl", mk(f, B.I32, (3,), 4)), SHAPE),
    "qpos_i32": (lambda f, a: a.__setitem__("qp", mk(f, B.I32, (4,), 4)), DTYPE),
    "out_width": (lambda f, a: a.__setitem__("out", mk(f, B.I32, (4, 2048), 4)), SHAPE),
    "out_i64": (lambda f, a: a.__setitem__("out", mk(f, B.I64, (4, 2051), 8)), DTYPE),
    "out_strided": (lambda f, a: a.__setitem__("out", mk(f, B.I32, (4, 2051), 4, stride=(4096, 1))), LAYOUT),
    "out_aliases_kcache": (lambda f, a: a.__setitem__("out", mk(f, B.I32, (4, 2051), 4, ptr=a["kcache"].data)), ALIAS),
    "out_aliases_q": (lambda f, a: a.__setitem__("out", mk(f, B.I32, (4, 2051), 4, ptr=a["q"].data + 64)), ALIAS),
    "null_table": (lambda f, a: a.__setitem__("bt", None), NULL),
    # q as runs [B, n, 4, 128]: R = B * n must match the per-row inputs
    "runs_heads": (lambda f, a: a.__setitem__("q", mk(f, B.F16, (2, 2, 3, 128), 2)), SHAPE),
    "runs_rows": (lambda f, a: a.__setitem__("q", mk(f, B.F16, (2, 3, 4, 128), 2)), SHAPE),
    "runs_dtype": (lambda f, a: a.__setitem__("q", mk(f, B.F32, (2, 2, 4, 128), 4)), DTYPE),
    "runs_strided": (lambda f, a: a.__setitem__("q", mk(f, B.F16, (2, 2, 4, 128), 2, stride=(2048, 512, 128, 1))), LAYOUT),
}


@pytest.mark.parametrize("case", sorted(SELECT_CASES))
def test_select_fail_closed(case):
    mutate, want = SELECT_CASES[case]
    f, a, ws, wsb = select_args(R=4, W=40)
    mutate(f, a)
    rc = call_select(a, ws, wsb)
    assert rc == want, (rc, B.library().qsa_last_error())
    assert B.library().qsa_last_error() != b""


def test_select_workspace_checks():
    f, a, ws, wsb = select_args(R=4, W=40)
    assert wsb > 0
    assert call_select(a, 0, wsb) == WORKSPACE
    assert call_select(a, ws, wsb - 1) == WORKSPACE
    assert call_select(a, ws + 16, wsb) == WORKSPACE
    assert call_select(a, a["out"].data, wsb) == ALIAS


ATTN_CASES = {
    "q_heads": (lambda f, a, base: a.__setitem__("q", mk(f, B.F16, (2, 4, 256), 2)), SHAPE),
    "q_dtype": (lambda f, a, base: a.__setitem__("q", mk(f, B.I32, (2, 3, 256), 4)), DTYPE),
    "k_strides": (lambda f, a, base: a.__setitem__("k", B.descriptor(base, B.F16, (4, 512, 1, 256), (131072, 256, 256, 1))), LAYOUT),
    "v_strides": (lambda f, a, base: a.__setitem__("v", B.descriptor(base + 512, B.F16, (4, 512, 1, 256), (262144, 512, 512, 1))), LAYOUT),
    "v_offset": (lambda f, a, base: a.__setitem__("v", B.descriptor(base + 256, B.F16, (4, 512, 1, 256), (262144, 512, 256, 1))), LAYOUT),
    "v_pages": (lambda f, a, base: a.__setitem__("v", B.descriptor(base + 512, B.F16, (3, 512, 1, 256), (262144, 512, 256, 1))), SHAPE),
    "k_page_rows": (lambda f, a, base: a.__setitem__("k", B.descriptor(base, B.F16, (4, 256, 1, 256), (262144, 512, 256, 1))), SHAPE),
    "indices_i64": (lambda f, a, base: a.__setitem__("idx", mk(f, B.I64, (2, 2051), 8)), DTYPE),
    "indices_width": (lambda f, a, base: a.__setitem__("idx", mk(f, B.I32, (2, 2048), 4)), SHAPE),
    "out_bf16": (lambda f, a, base: a.__setitem__("out", mk(f, 0, (2, 3, 256), 2)), DTYPE),
    "out_rows": (lambda f, a, base: a.__setitem__("out", mk(f, B.F16, (3, 3, 256), 2)), SHAPE),
    "out_aliases_kv": (lambda f, a, base: a.__setitem__("out", mk(f, B.F16, (2, 3, 256), 2, ptr=base + 4096)), ALIAS),
    "out_aliases_indices": (lambda f, a, base: a.__setitem__("out", mk(f, B.F16, (2, 3, 256), 2, ptr=a["idx"].data)), ALIAS),
}


@pytest.mark.parametrize("case", sorted(ATTN_CASES))
def test_attn_fail_closed(case):
    mutate, want = ATTN_CASES[case]
    f, a, ws, wsb, base = attn_args()
    mutate(f, a, base)
    rc = call_attn(a, ws, wsb)
    assert rc == want, (rc, B.library().qsa_last_error())


@pytest.mark.parametrize("scale", [0.0, -1.0, float("nan"), float("inf")])
def test_attn_scale_checked(scale):
    f, a, ws, wsb, base = attn_args()
    assert call_attn(a, ws, wsb, scale) == ARG


def test_decode_step_checks():
    lib = B.library()
    f, s, sws, swsb = select_args(R=2, W=40)
    g, a, aws, awsb, base = attn_args(R=2)
    wsb = B.decode_step_workspace_bytes(2, 40)
    ws = f.alloc(wsb)

    def call(q_attn=None, idx=None):
        qa = q_attn or a["q"]
        ix = idx or s["out"]
        return lib.qsa_decode_step(
            ctypes.byref(s["q"]), ctypes.byref(s["kcache"]), ctypes.byref(s["bt"]),
            ctypes.byref(s["t2r"]), ctypes.byref(s["sl"]), ctypes.byref(s["qp"]),
            ctypes.byref(qa), ctypes.byref(a["k"]), ctypes.byref(a["v"]), ctypes.c_float(0.0625),
            ctypes.byref(ix), ctypes.byref(a["out"]), ctypes.c_void_p(ws), wsb, None)

    assert call(q_attn=mk(g, B.F16, (3, 3, 256), 2)) == SHAPE
    assert call(idx=mk(g, B.I32, (2, 2051), 4, ptr=base)) == ALIAS
    assert call(idx=mk(g, B.I32, (2, 2051), 4, ptr=s["q"].data)) == ALIAS
    # a too-small workspace is rejected before anything is launched
    assert lib.qsa_decode_step(
        ctypes.byref(s["q"]), ctypes.byref(s["kcache"]), ctypes.byref(s["bt"]),
        ctypes.byref(s["t2r"]), ctypes.byref(s["sl"]), ctypes.byref(s["qp"]),
        ctypes.byref(a["q"]), ctypes.byref(a["k"]), ctypes.byref(a["v"]), ctypes.c_float(0.0625),
        ctypes.byref(s["out"]), ctypes.byref(a["out"]), ctypes.c_void_p(ws), wsb - 256, None) == WORKSPACE


def test_decode_step_noalloc_checks():
    """The no-allocation decode step validates like qsa_decode_step and
    refuses a call whose workspace would exceed the fixed scratch, before it
    looks the scratch up or launches anything (no GPU needed to see that)."""
    lib = B.library()
    f, s, _, _ = select_args(R=2, W=40)
    g, a, _, _, base = attn_args(R=2)

    def call(sel, att, idx=None):
        return lib.qsa_decode_step_noalloc(
            ctypes.byref(sel["q"]), ctypes.byref(sel["kcache"]), ctypes.byref(sel["bt"]),
            ctypes.byref(sel["t2r"]), ctypes.byref(sel["sl"]), ctypes.byref(sel["qp"]),
            ctypes.byref(att["q"]), ctypes.byref(att["k"]), ctypes.byref(att["v"]),
            ctypes.c_float(0.0625), ctypes.byref(idx or sel["out"]), ctypes.byref(att["out"]),
            None)

    assert call(s, a, idx=mk(g, B.I32, (2, 2051), 4, ptr=base)) == ALIAS
    assert call(s, a, idx=mk(g, B.I32, (3, 2051), 4)) == SHAPE
    # 4096 rows over a 256-page table: ~64 MiB of candidates > the 32 MiB scratch
    R, W = 4096, 256
    f2, big, _, _ = select_args(R=R, N=R, W=W)
    g2, att2, _, _, _ = attn_args(R=R)
    assert B.decode_step_workspace_bytes(R, W) > 32 << 20
    assert call(big, att2) == WORKSPACE
    assert b"fixed scratch holds 33554432" in lib.qsa_last_error()


def test_torch_descriptor_dtype_refused():
    """A float32 query is refused by the library; the binding turns the
    status into RuntimeError."""
    import torch
    q = torch.zeros((1, 4, 128), dtype=torch.float32)
    f, a, ws, wsb = select_args(R=1)
    a["q"] = B.tensor_desc(q)
    with pytest.raises(RuntimeError, match="QSA_ERR_DTYPE"):
        B.check(call_select(a, ws, wsb))


# ---------------------------------------------------------------------------
# e4m3 key cache entry points

def fp8_args(R=4, P=8, N=4, W=40):
    f, a, ws, wsb = select_args(R=R, P=P, N=N, W=W)
    a["kcache"] = mk(f, B.E4M3, (P, 128, 1, 128), 1)
    a["kscale"] = mk(f, B.F32, (P, 128), 4)
    return f, a, ws, wsb


def call_select_fp8(a, ws, ws_bytes):
    lib = B.library()
    order = ["q", "kcache", "kscale", "bt", "t2r", "sl", "qp", "out"]
    ptrs = [ctypes.byref(a[k]) if a[k] is not None else None for k in order]
    return lib.qsa_select_fp8(*ptrs, ctypes.c_void_p(ws), ws_bytes, None)


FP8_CASES = {
    "kcache_f16": (lambda f, a: a.__setitem__("kcache", mk(f, B.F16, (8, 128, 1, 128), 2)), DTYPE),
    "kcache_misaligned": (lambda f, a: a.__setitem__("kcache", mk(f, B.E4M3, (8, 128, 1, 128), 1, ptr=f.alloc(1 << 17) + 8)), LAYOUT),
    "kcache_strided": (lambda f, a: a.__setitem__("kcache", mk(f, B.E4M3, (8, 128, 1, 128), 1, stride=(32768, 256, 128, 1))), LAYOUT),
    "kscale_f16": (lambda f, a: a.__setitem__("kscale", mk(f, B.F16, (8, 128), 2)), DTYPE),
    "kscale_pages": (lambda f, a: a.__setitem__("kscale", mk(f, B.F32, (7, 128), 4)), SHAPE),
    "kscale_slots": (lambda f, a: a.__setitem__("kscale", mk(f, B.F32, (8, 64), 4)), SHAPE),
    "kscale_rank": (lambda f, a: a.__setitem__("kscale", mk(f, B.F32, (8 * 128,), 4)), SHAPE),
    "kscale_strided": (lambda f, a: a.__setitem__("kscale", mk(f, B.F32, (8, 128), 4, stride=(256, 1))), LAYOUT),
    "kscale_misaligned": (lambda f, a: a.__setitem__("kscale", mk(f, B.F32, (8, 128), 4, ptr=f.alloc(8192) + 2)), LAYOUT),
    "kscale_null": (lambda f, a: a.__setitem__("kscale", None), NULL),
    "out_aliases_kscale": (lambda f, a: a.__setitem__("out", mk(f, B.I32, (4, 2051), 4, ptr=a["kscale"].data)), ALIAS),
}


@pytest.mark.parametrize("case", sorted(FP8_CASES))
def test_select_fp8_fail_closed(case):
    mutate, want = FP8_CASES[case]
    f, a, ws, wsb = fp8_args()
    mutate(f, a)
    rc = call_select_fp8(a, ws, wsb)
    assert rc == want, (rc, B.library().qsa_last_error())
    assert B.library().qsa_last_error() != b""


def test_select_fp8_zero_rows_and_workspace():
    f, a, ws, wsb = fp8_args(R=0)
    assert call_select_fp8(a, 0, 0) == OK
    f, a, ws, wsb = fp8_args()
    assert wsb > 0
    assert call_select_fp8(a, ws, wsb - 1) == WORKSPACE
    assert call_select_fp8(a, a["kscale"].data, wsb) == ALIAS


def test_fp16_entry_refuses_e4m3_cache():
    f, a, ws, wsb = fp8_args()
    assert call_select(a, ws, wsb) == DTYPE


def test_decode_step_fp8_checks():
    lib = B.library()
    f, s, sws, swsb = fp8_args(R=2)
    g, a, aws, awsb, base = attn_args(R=2)
    wsb = B.decode_step_workspace_bytes(2, 40)
    ws = f.alloc(wsb)

    def call(out=None, ws_bytes=wsb, kscale=None):
        return lib.qsa_decode_step_fp8(
            ctypes.byref(s["q"]), ctypes.byref(s["kcache"]), ctypes.byref(kscale or s["kscale"]),
            ctypes.byref(s["bt"]), ctypes.byref(s["t2r"]), ctypes.byref(s["sl"]),
            ctypes.byref(s["qp"]), ctypes.byref(a["q"]), ctypes.byref(a["k"]),
            ctypes.byref(a["v"]), ctypes.c_float(0.0625), ctypes.byref(s["out"]),
            ctypes.byref(out or a["out"]), ctypes.c_void_p(ws), ws_bytes, None)

    assert call(out=mk(g, B.F16, (2, 3, 256), 2, ptr=s["kscale"].data)) == ALIAS
    assert call(ws_bytes=wsb - 256) == WORKSPACE
    assert call(kscale=mk(g, B.F32, (8, 127), 4)) == SHAPE


# ---------------------------------------------------------------------------
# per-head weights, paged logits, top-k per row

def call_weighted(a, ws, ws_bytes, weights, kscale=None):
    lib = B.library()
    opt = lambda t: ctypes.byref(t) if t is not None else None  # noqa: E731
    return lib.qsa_select_weighted(ctypes.byref(a["q"]), opt(weights), ctypes.byref(a["kcache"]),
                                   opt(kscale), *[ctypes.byref(a[k]) for k in
                                                  ("bt", "t2r", "sl", "qp", "out")],
                                   ctypes.c_void_p(ws), ws_bytes, None)


def test_select_weighted_checks():
    f, a, ws, wsb = select_args(R=4, W=40)
    w = mk(f, B.F32, (4, 4), 4)
    assert call_weighted(a, ws, wsb, None) == NULL
    assert call_weighted(a, ws, wsb, mk(f, B.F16, (4, 4), 2)) == DTYPE
    assert call_weighted(a, ws, wsb, mk(f, B.F32, (4, 3), 4)) == SHAPE
    assert call_weighted(a, ws, wsb, mk(f, B.F32, (5, 4), 4)) == SHAPE
    assert call_weighted(a, ws, wsb, mk(f, B.F32, (4, 4), 4, ptr=f.alloc(4096) + 4)) == LAYOUT
    a2 = dict(a, out=mk(f, B.I32, (4, 2051), 4, ptr=w.data))
    assert call_weighted(a2, ws, wsb, w) == ALIAS
    assert call_weighted(a, ws, wsb - 1, w) == WORKSPACE
    assert call_weighted(a, w.data, wsb, w) == ALIAS
    # an e4m3 cache needs its scales, an fp16 cache must not get them
    f8, a8, ws8, wsb8 = fp8_args()
    assert call_weighted(a8, ws8, wsb8, mk(f8, B.F32, (4, 4), 4)) == DTYPE
    assert call_weighted(a, ws, wsb, w, kscale=mk(f, B.F32, (8, 128), 4)) == DTYPE


def call_logits(a, logits, weights=None, kscale=None):
    lib = B.library()
    opt = lambda t: ctypes.byref(t) if t is not None else None  # noqa: E731
    return lib.qsa_paged_logits(ctypes.byref(a["q"]), opt(weights), ctypes.byref(a["kcache"]),
                                opt(kscale), *[ctypes.byref(a[k]) for k in
                                               ("bt", "t2r", "sl", "qp")],
                                opt(logits), None)


def test_paged_logits_checks():
    f, a, ws, wsb = select_args(R=4, W=40)
    assert call_logits(a, None) == NULL
    assert call_logits(a, mk(f, B.F16, (4, 5120), 2)) == DTYPE
    assert call_logits(a, mk(f, B.F32, (4, 5119), 4)) == SHAPE
    assert call_logits(a, mk(f, B.F32, (3, 5120), 4)) == SHAPE
    assert call_logits(a, mk(f, B.F32, (4, 5120), 4, stride=(10240, 2))) == LAYOUT
    assert call_logits(a, mk(f, B.F32, (4, 5120), 4, stride=(5000, 1))) == LAYOUT
    assert call_logits(a, mk(f, B.F32, (4, 5120), 4, ptr=a["q"].data)) == ALIAS
    assert call_logits(a, mk(f, B.F32, (4, 5120), 4), weights=mk(f, B.F32, (4, 2), 4)) == SHAPE


def test_paged_logits_zero_rows():
    f, a, ws, wsb = select_args(R=0, W=40)
    assert call_logits(a, mk(f, B.F32, (0, 5120), 4)) == OK


def call_topk(lg, t2r, sl, qp, out, ws, ws_bytes):
    lib = B.library()
    return lib.qsa_topk_per_row(*[ctypes.byref(x) for x in (lg, t2r, sl, qp, out)],
                                ctypes.c_void_p(ws), ws_bytes, None)


def test_topk_per_row_checks():
    f = Fake()
    # rows of at most 32768 columns are selected one workgroup per row,
    # without workspace; wider rows go through chunks and a merge
    assert B.topk_per_row_workspace_bytes(4, 32768) == 0
    assert B.topk_per_row_workspace_bytes(4, 32769) > 0
    R, Wl = 4, 40000
    lg = mk(f, B.F32, (R, Wl), 4)
    t2r, sl, qp = mk(f, B.I32, (R,), 4), mk(f, B.I32, (2,), 4), mk(f, B.I64, (R,), 8)
    out = mk(f, B.I32, (R, 2051), 4)
    wsb = B.topk_per_row_workspace_bytes(R, Wl)
    assert wsb > 0 and B.topk_per_row_workspace_bytes(0, Wl) == 0
    ws = f.alloc(wsb)
    assert call_topk(mk(f, B.F16, (R, Wl), 2), t2r, sl, qp, out, ws, wsb) == DTYPE
    assert call_topk(mk(f, B.F32, (R, 0), 4), t2r, sl, qp, out, ws, wsb) == SHAPE
    assert call_topk(mk(f, B.F32, (R, Wl), 4, stride=(2 * Wl, 2)), t2r, sl, qp, out, ws, wsb) == LAYOUT
    assert call_topk(lg, mk(f, B.I32, (R + 1,), 4), sl, qp, out, ws, wsb) == SHAPE
    assert call_topk(lg, t2r, mk(f, B.I32, (0,), 4), qp, out, ws, wsb) == SHAPE
    assert call_topk(lg, t2r, sl, mk(f, B.I32, (R,), 4), out, ws, wsb) == DTYPE
    assert call_topk(lg, t2r, sl, qp, mk(f, B.I32, (R, 2048), 4), ws, wsb) == SHAPE
    assert call_topk(lg, t2r, sl, qp, mk(f, B.I32, (R, 2051), 4, ptr=lg.data), ws, wsb) == ALIAS
    assert call_topk(lg, t2r, sl, qp, out, ws, wsb - 1) == WORKSPACE
    assert call_topk(lg, t2r, sl, qp, out, lg.data, wsb) == ALIAS
    assert call_topk(mk(f, B.F32, (0, Wl), 4), mk(f, B.I32, (0,), 4), sl, mk(f, B.I64, (0,), 8),
                     mk(f, B.I32, (0, 2051), 4), 0, 0) == OK


# ---------------------------------------------------------------------------
# metadata builder

def meta_args(N=3, T=10, W=4, M=8):
    f = Fake()
    a = dict(qsl=mk(f, B.I32, (N + 1,), 4), sl=mk(f, B.I32, (N,), 4), bt=mk(f, B.I32, (N, W), 4),
             csm=mk(f, B.I64, (T,), 8), t2r=mk(f, B.I32, (T,), 4), lp=mk(f, B.I64, (T,), 8),
             vis=mk(f, B.I32, (T,), 4), slots=mk(f, B.I64, (T,), 8),
             work=mk(f, B.I32, (M, 2), 4) if M else None)
    wsb = B.build_metadata_workspace_bytes(N) if M else 0
    return f, a, (f.alloc(wsb) if wsb else 0), wsb


def call_meta(a, ws, wsb, block=128, ratio=4, ring=0):
    lib = B.library()
    opt = lambda t: ctypes.byref(t) if t is not None else None  # noqa: E731
    return lib.qsa_build_metadata(opt(a["qsl"]), opt(a["sl"]), opt(a["bt"]), opt(a["csm"]),
                                  block, ratio, ring, opt(a["t2r"]), opt(a["lp"]), opt(a["vis"]),
                                  opt(a["slots"]), opt(a["work"]), ctypes.c_void_p(ws), wsb, None)


META_CASES = {
    "qsl_len": (lambda f, a: a.__setitem__("qsl", mk(f, B.I32, (3,), 4)), SHAPE),
    "qsl_i64": (lambda f, a: a.__setitem__("qsl", mk(f, B.I64, (4,), 8)), DTYPE),
    "seq_lens_null": (lambda f, a: a.__setitem__("sl", None), NULL),
    "table_rows": (lambda f, a: a.__setitem__("bt", mk(f, B.I32, (2, 4), 4)), SHAPE),
    "table_col_stride": (lambda f, a: a.__setitem__("bt", mk(f, B.I32, (3, 4), 4, stride=(8, 2))), LAYOUT),
    "positions_i32": (lambda f, a: a.__setitem__("lp", mk(f, B.I32, (10,), 4)), DTYPE),
    "visible_len": (lambda f, a: a.__setitem__("vis", mk(f, B.I32, (9,), 4)), SHAPE),
    "csm_i32": (lambda f, a: a.__setitem__("csm", mk(f, B.I32, (10,), 4)), DTYPE),
    "slots_len": (lambda f, a: a.__setitem__("slots", mk(f, B.I64, (11,), 8)), SHAPE),
    "work_cols": (lambda f, a: a.__setitem__("work", mk(f, B.I32, (8, 3), 4)), SHAPE),
    "out_overlap": (lambda f, a: a.__setitem__("vis", mk(f, B.I32, (10,), 4, ptr=a["t2r"].data)), ALIAS),
    "out_on_input": (lambda f, a: a.__setitem__("lp", mk(f, B.I64, (10,), 8, ptr=a["qsl"].data)), ALIAS),
}


@pytest.mark.parametrize("case", sorted(META_CASES))
def test_metadata_fail_closed(case):
    mutate, want = META_CASES[case]
    f, a, ws, wsb = meta_args()
    mutate(f, a)
    rc = call_meta(a, ws, wsb)
    assert rc == want, (rc, B.library().qsa_last_error())


def test_metadata_scalar_and_workspace_checks():
    f, a, ws, wsb = meta_args()
    assert call_meta(a, ws, wsb, block=0) == ARG
    assert call_meta(a, ws, wsb, ratio=0) == ARG
    assert call_meta(a, ws, wsb, ring=-1) == ARG
    assert wsb > 0 and B.build_metadata_workspace_bytes(0) == 0
    assert call_meta(a, ws, wsb - 1) == WORKSPACE
    assert call_meta(a, 0, wsb) == WORKSPACE
    assert call_meta(a, a["t2r"].data, wsb) == ALIAS
    # no tokens and no work items: nothing to do
    f, a, ws, wsb = meta_args(T=0, M=0)
    assert call_meta(a, 0, 0) == OK


def test_select_runs_zero_rows_and_workspace():
    """q given as runs [B, n, 4, 128]: zero rows either way is a no-op; the
    grouped plan cuts rows into smaller chunks (more candidates) and the
    workspace query covers it."""
    for shape in [(0, 4, 4, 128), (3, 0, 4, 128)]:
        f, a, ws, wsb = select_args(R=0)
        a["q"] = mk(f, B.F16, shape, 2)
        assert call_select(a, 0, 0) == OK
    R, W = 128, 256
    f, a, ws, wsb = select_args(R=R, W=W)
    # 4-row groups: 32 groups x 32 chunks of 8 pages, 512 candidates each
    assert wsb >= R * 32 * 512 * 8
    a["q"] = mk(f, B.F16, (R // 4, 4, 4, 128), 2)
    assert call_select(a, ws, R * 8 * 512 * 8) == WORKSPACE  # sized for rows one by one
    f, a, ws, wsb = select_args(R=R, W=W)
    a["q"] = mk(f, B.F16, (R // 4, 4, 4, 128), 2)
    a["t2r"] = mk(f, B.I32, (R + 1,), 4)
    assert call_select(a, ws, wsb) == SHAPE


def test_launch_size_limits():
    """Shapes whose grid would not fit one launch are refused before
    anything is launched (grid sizes are never truncated)."""
    f, a, ws, wsb = select_args(R=(1 << 30), W=(1 << 22))
    assert call_select(a, ws, 1 << 62) == SHAPE
    assert b"exceed one launch" in B.library().qsa_last_error()
    # 2^22 rows x 8 chunks of 256 threads = 2^33 work-items: more than one
    # dispatch holds, although far fewer than 2^31 workgroups
    f, a, ws, wsb = select_args(R=(1 << 22), W=256)
    assert call_select(a, ws, 1 << 62) == SHAPE
    assert b"exceed one launch" in B.library().qsa_last_error()
    f, a, ws, wsb = select_args(R=(1 << 20), W=256)
    assert call_select(a, 0, 0) == WORKSPACE  # fits one launch; only the workspace is missing
    # attention at one split per row: 2^25 rows x 256 threads = 2^33 work-items
    g, at, aws, awsb, _ = attn_args(R=(1 << 25))
    assert call_attn(at, 0, 0) == SHAPE
    assert b"exceed one launch" in B.library().qsa_last_error()
    # top-k per row, one 1024-thread workgroup per row of <= 32768 columns:
    # 2^22 rows x 1024 threads = 2^32 work-items, one more than a launch holds
    f = Fake()
    R, Wl = 1 << 22, 100
    lg = mk(f, B.F32, (R, Wl), 4)
    t2r, sl, qp = mk(f, B.I32, (R,), 4), mk(f, B.I32, (2,), 4), mk(f, B.I64, (R,), 8)
    out = mk(f, B.I32, (R, 2051), 4)
    assert call_topk(lg, t2r, sl, qp, out, 0, 0) == SHAPE
    assert b"exceed one launch" in B.library().qsa_last_error()
    # attention: a batch this large runs one split per row (no partials, so
    # no workspace), whose grid of padded rows always fits one launch
    assert B.sparse_attn_workspace_bytes(1 << 30) == 0
    assert B.sparse_attn_workspace_bytes(767) > 0 and B.sparse_attn_workspace_bytes(768) == 0


def probe_library():
    from paged_top_indexer_amd import build

    lib = ctypes.CDLL(build.PROBE_LIBRARY)
    lib.qsa_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                   ctypes.c_size_t, ctypes.c_void_p]
    lib.qsa_read_probe.restype = ctypes.c_int
    return lib


def test_read_probe_is_apart_from_the_method():
    """The read-ceiling probe is a measurement aid: exported by
    libqsa_probe.so as include/qsa_probe.h declares, absent from the method's
    library and header."""
    assert not hasattr(B.library(), "qsa_read_probe")
    assert "qsa_read_probe" not in declared_symbols()
    text = open(os.path.join(ROOT, "include", "qsa_probe.h")).read()
    assert re.findall(r"QSA_API\s+[\w\s\*]+?\b(qsa_\w+)\s*\(", text) == ["qsa_read_probe"]
    assert hasattr(probe_library(), "qsa_read_probe")


def test_read_probe_checks():
    lib = probe_library()
    f = Fake()
    d, k = f.alloc(1 << 20), f.alloc(64)
    assert lib.qsa_read_probe(None, 1 << 20, ctypes.c_void_p(k), 4, None) == NULL
    assert lib.qsa_read_probe(ctypes.c_void_p(d + 8), 1 << 20, ctypes.c_void_p(k), 4, None) == LAYOUT
    assert lib.qsa_read_probe(ctypes.c_void_p(d), (1 << 20) + 4, ctypes.c_void_p(k), 4, None) == LAYOUT
    assert lib.qsa_read_probe(ctypes.c_void_p(d), 1 << 20, ctypes.c_void_p(k), 2, None) == WORKSPACE
    assert lib.qsa_read_probe(ctypes.c_void_p(d), 1 << 20, ctypes.c_void_p(d + 64), 4, None) == ALIAS
    assert lib.qsa_read_probe(ctypes.c_void_p(d), 0, ctypes.c_void_p(k), 4, None) == OK


@pytest.mark.parametrize("lang", ["c99", "c++17"])
def test_header_compiles_standalone(lang, tmp_path):
    """include/qsa.h (and the probe's qsa_probe.h) need no HIP header and
    compile on their own as C99 and as C++17 (a C caller includes them as
    they are)."""
    import shutil
    import subprocess

    compiler = "gcc" if lang == "c99" else "g++"
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not found")
    src = tmp_path / ("use.c" if lang == "c99" else "use.cpp")
    src.write_text('#include "qsa.h"\n#include "qsa_probe.h"\n'
                   'int main(void) { int32_t w; qsa_constants(0, 0, &w, 0); '
                   'int (*probe)(const void*, size_t, void*, size_t, qsa_stream) = qsa_read_probe; '
                   '(void)probe; return w == QSA_OUT_WIDTH ? 0 : 1; }\n')
    res = subprocess.run([compiler, f"-std={lang}", "-Wall", "-Wextra", "-Werror", "-pedantic",
                          "-fsyntax-only", f"-I{os.path.join(ROOT, 'include')}", str(src)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
