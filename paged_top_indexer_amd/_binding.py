"""ctypes binding of libqsa_amd.so (include/qsa.h).

Argument marshalling only: torch tensors become qsa_tensor descriptors,
the stream is torch's current HIP stream, and workspaces are zero-filled
device buffers cached per (device, stream).  Every step of the path runs in
the library's HIP kernels; there is no fallback -- if the library is missing
or refuses the arguments, these functions raise.
"""

from __future__ import annotations

import ctypes
import os
import struct
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libqsa_amd.so")

F16, I32, I64, F32, E4M3 = 1, 2, 3, 4, 5
TOKEN_TOPK, COMPRESS_RATIO, OUT_WIDTH, TOPK_BLOCKS = 2048, 4, 2051, 512
STATUS = {0: "QSA_OK", 1: "QSA_ERR_NULL", 2: "QSA_ERR_DTYPE", 3: "QSA_ERR_SHAPE",
          4: "QSA_ERR_LAYOUT", 5: "QSA_ERR_ALIAS", 6: "QSA_ERR_WORKSPACE",
          7: "QSA_ERR_ARG", 8: "QSA_ERR_LAUNCH"}


class QsaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


# qsa_tensor's bytes: data, dtype, ndim, shape[4], stride[4] (packed in one
# call: filling the ctypes fields one by one costs several us per call)
_DESC = struct.Struct("<Qii4q4q")
assert _DESC.size == ctypes.sizeof(QsaTensor)
_PAD = ((), (0,), (0, 0), (0, 0, 0), (0, 0, 0, 0))


def descriptor(data_ptr: int, dtype: int, shape, stride) -> QsaTensor:
    """A qsa_tensor; more than 4 dims keep ndim (the library rejects them)
    with the first 4 extents and strides."""
    n = len(shape)
    if n <= 4:
        pad = _PAD[4 - n]
        raw = _DESC.pack(data_ptr, dtype, n, *shape, *pad, *stride, *pad)
    else:
        raw = _DESC.pack(data_ptr, dtype, n, *shape[:4], *stride[:4])
    return QsaTensor.from_buffer_copy(raw)


_libs: dict = {}
_current = LIBRARY
_lock = threading.Lock()

_P = ctypes.POINTER(QsaTensor)


def _configure(lib: ctypes.CDLL) -> None:
    """Argument and result types of every entry point the library exports
    (a library built from an older revision may lack some)."""
    sz, i64, vp, f32, i = ctypes.c_size_t, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    sigs = {
        "qsa_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "qsa_last_error": ([], ctypes.c_char_p),
        "qsa_constants": ([ctypes.POINTER(ctypes.c_int32)] * 4, None),
        "qsa_select_workspace_bytes": ([i64, i64], sz),
        "qsa_sparse_attn_workspace_bytes": ([i64], sz),
        "qsa_decode_step_workspace_bytes": ([i64, i64], sz),
        "qsa_select": ([_P] * 7 + [vp, sz, vp], i),
        "qsa_sparse_attn": ([_P] * 4 + [f32, _P, vp, sz, vp], i),
        "qsa_decode_step": ([_P] * 9 + [f32, _P, _P, vp, sz, vp], i),
        "qsa_select_fp8": ([_P] * 8 + [vp, sz, vp], i),
        "qsa_decode_step_fp8": ([_P] * 10 + [f32, _P, _P, vp, sz, vp], i),
        "qsa_decode_step_noalloc": ([_P] * 9 + [f32, _P, _P, vp], i),
        "qsa_select_weighted": ([_P] * 9 + [vp, sz, vp], i),
        "qsa_paged_logits": ([_P] * 9 + [vp], i),
        "qsa_topk_per_row_workspace_bytes": ([i64, i64], sz),
        "qsa_topk_per_row": ([_P] * 5 + [vp, sz, vp], i),
        "qsa_build_metadata_workspace_bytes": ([i64], sz),
        "qsa_build_metadata": ([_P] * 4 + [i64, i64, i64] + [_P] * 5 + [vp, sz, vp], i),
    }
    for name, (args, res) in sigs.items():
        fn = getattr(lib, name, None)
        if fn is not None:
            fn.argtypes = args
            fn.restype = res


def library() -> ctypes.CDLL:
    """The library the entry points call: libqsa_amd.so (built by
    paged_top_indexer_amd.build), or the one use_library() selected."""
    with _lock:
        lib = _libs.get(_current)
        if lib is None:
            if not os.path.exists(_current):
                raise RuntimeError(
                    f"{_current} is missing: build it with `python -m paged_top_indexer_amd.build` "
                    "(there is no fallback implementation)")
            lib = ctypes.CDLL(_current)
            _configure(lib)
            _libs[_current] = lib
        return lib


def use_library(path: str | None = None) -> str:
    """Route the entry points to another build of the library (e.g. the
    baseline of an A/B comparison; None: back to libqsa_amd.so).  Returns
    the previous path."""
    global _current
    prev = _current
    _current = os.path.abspath(path) if path else LIBRARY
    library()
    return prev


def check(status: int) -> None:
    if status != 0:
        detail = library().qsa_last_error().decode()
        raise RuntimeError(f"{STATUS.get(status, status)}: {detail}")


def constants() -> tuple[int, int, int, int]:
    vals = [ctypes.c_int32() for _ in range(4)]
    library().qsa_constants(*[ctypes.byref(v) for v in vals])
    return tuple(v.value for v in vals)


def select_workspace_bytes(rows: int, table_width: int) -> int:
    return int(library().qsa_select_workspace_bytes(int(rows), int(table_width)))


def sparse_attn_workspace_bytes(rows: int) -> int:
    return int(library().qsa_sparse_attn_workspace_bytes(int(rows)))


def decode_step_workspace_bytes(rows: int, table_width: int) -> int:
    return int(library().qsa_decode_step_workspace_bytes(int(rows), int(table_width)))


# ---------------------------------------------------------------------------
# torch marshalling

def _torch():
    import torch
    return torch


_CODES: dict = {}


def _dtype_code(t) -> int:
    if not _CODES:
        torch = _torch()
        _CODES.update({torch.float16: F16, torch.int32: I32, torch.int64: I64,
                       torch.float32: F32, torch.float8_e4m3fn: E4M3})
    return _CODES.get(t.dtype, 0)


def tensor_desc(t) -> QsaTensor:
    """Descriptor of a torch tensor (the element pointer includes the storage
    offset).  Unsupported dtypes get code 0, which the library rejects."""
    return descriptor(t.data_ptr(), _dtype_code(t), t.shape, t.stride())


def kv_views(kv):
    """K and V views of a packed [NP, 512, 512] fp16 cache: shape
    [NP,512,1,256], strides [262144,512,256,1], V at storage offset +256."""
    pages = kv.shape[0]
    split = kv.view(pages, 512, 2, 256)
    return split[:, :, 0:1, :], split[:, :, 1:2, :]


_workspaces: dict = {}


def workspace(nbytes: int, device, stream_handle: int, kind: str):
    """A device buffer of at least nbytes, cached per (device, stream, entry
    point).  The library keeps no state in a workspace between calls, so
    consecutive calls on one stream may share it."""
    torch = _torch()
    if nbytes == 0:
        return None
    key = (str(device), int(stream_handle), kind)
    buf = _workspaces.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = buf
    return buf


def _stream(stream, device):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def _ws_args(nbytes, device, stream_handle, ws, kind):
    if ws is None:
        ws = workspace(nbytes, device, stream_handle, kind)
    if ws is None:
        return None, 0
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


def _rows(q):
    """Query rows of a selection query: [R,4,128], or [B,n,4,128] for R = B*n
    rows in runs of n rows of one request (scored up to 4 at a time)."""
    return q.shape[0] * q.shape[1] if q.dim() == 4 else q.shape[0]


def qsa_select(q, kcache, block_table, token_to_req, seq_lens, query_pos, out=None,
               workspace=None, stream=None):
    """Paged top-512 selection; returns out ([R,2051] int32).  q is
    [R,4,128], or [B,n,4,128] when rows come in runs of n rows of one
    request (speculative-decode positions): the runs share key reads."""
    torch = _torch()
    lib = library()
    R = _rows(q)
    if out is None:
        out = torch.empty((R, OUT_WIDTH), dtype=torch.int32, device=q.device)
    sh = _stream(stream, q.device)
    need = select_workspace_bytes(R, block_table.shape[1]) if block_table.dim() == 2 else 0
    ws, ws_bytes = _ws_args(need, q.device, sh, workspace, "select")
    descs = [tensor_desc(t) for t in (q, kcache, block_table, token_to_req, seq_lens, query_pos, out)]
    check(lib.qsa_select(*[ctypes.byref(d) for d in descs], ws, ws_bytes, ctypes.c_void_p(sh)))
    return out


def qsa_select_fp8(q, kcache, kscale, block_table, token_to_req, seq_lens, query_pos, out=None,
                   workspace=None, stream=None):
    """Selection over an e4m3 key cache (kcache torch.float8_e4m3fn
    [P,128,1,128], kscale float32 [P,128]); returns out ([R,2051] int32)."""
    torch = _torch()
    lib = library()
    R = _rows(q)
    if out is None:
        out = torch.empty((R, OUT_WIDTH), dtype=torch.int32, device=q.device)
    sh = _stream(stream, q.device)
    need = select_workspace_bytes(R, block_table.shape[1]) if block_table.dim() == 2 else 0
    ws, ws_bytes = _ws_args(need, q.device, sh, workspace, "select")
    descs = [tensor_desc(t) for t in (q, kcache, kscale, block_table, token_to_req, seq_lens,
                                      query_pos, out)]
    check(lib.qsa_select_fp8(*[ctypes.byref(d) for d in descs], ws, ws_bytes, ctypes.c_void_p(sh)))
    return out


def _opt(t):
    """Descriptor pointer of an optional tensor (None -> NULL)."""
    return None if t is None else ctypes.byref(tensor_desc(t))


def qsa_select_weighted(q, weights, kcache, block_table, token_to_req, seq_lens, query_pos,
                        kscale=None, out=None, workspace=None, stream=None):
    """Selection with per-head weights [R,4] float32 (fp16 cache, or e4m3
    codes with kscale); returns out ([R,2051] int32)."""
    torch = _torch()
    lib = library()
    R = _rows(q)
    if out is None:
        out = torch.empty((R, OUT_WIDTH), dtype=torch.int32, device=q.device)
    sh = _stream(stream, q.device)
    need = select_workspace_bytes(R, block_table.shape[1]) if block_table.dim() == 2 else 0
    ws, ws_bytes = _ws_args(need, q.device, sh, workspace, "select")
    d = [tensor_desc(t) for t in (q, weights, kcache)]
    rest = [tensor_desc(t) for t in (block_table, token_to_req, seq_lens, query_pos, out)]
    check(lib.qsa_select_weighted(*[ctypes.byref(x) for x in d], _opt(kscale),
                                  *[ctypes.byref(x) for x in rest], ws, ws_bytes,
                                  ctypes.c_void_p(sh)))
    return out


def qsa_paged_logits(q, kcache, block_table, token_to_req, seq_lens, query_pos, weights=None,
                     kscale=None, logits=None, width=None, stream=None):
    """Block scores as an fp32 logits matrix [R, width] (width defaults to
    the block table's width x 128; -inf past each row's visible blocks)."""
    torch = _torch()
    lib = library()
    R = _rows(q)
    if logits is None:
        W = block_table.shape[1] * 128 if width is None else int(width)
        logits = torch.empty((R, W), dtype=torch.float32, device=q.device)
    sh = _stream(stream, q.device)
    rest = [tensor_desc(t) for t in (block_table, token_to_req, seq_lens, query_pos, logits)]
    check(lib.qsa_paged_logits(ctypes.byref(tensor_desc(q)), _opt(weights),
                               ctypes.byref(tensor_desc(kcache)), _opt(kscale),
                               *[ctypes.byref(x) for x in rest], ctypes.c_void_p(sh)))
    return logits


def topk_per_row_workspace_bytes(rows: int, logits_width: int) -> int:
    return int(library().qsa_topk_per_row_workspace_bytes(int(rows), int(logits_width)))


def qsa_topk_per_row(logits, token_to_req, seq_lens, query_pos, out=None, workspace=None,
                     stream=None):
    """Top-512 blocks per row of a logits matrix, expanded as by qsa_select;
    returns out ([R,2051] int32)."""
    torch = _torch()
    lib = library()
    R = logits.shape[0]
    if out is None:
        out = torch.empty((R, OUT_WIDTH), dtype=torch.int32, device=logits.device)
    sh = _stream(stream, logits.device)
    need = topk_per_row_workspace_bytes(R, logits.shape[1]) if logits.dim() == 2 else 0
    ws, ws_bytes = _ws_args(need, logits.device, sh, workspace, "topk")
    d = [tensor_desc(t) for t in (logits, token_to_req, seq_lens, query_pos, out)]
    check(lib.qsa_topk_per_row(*[ctypes.byref(x) for x in d], ws, ws_bytes, ctypes.c_void_p(sh)))
    return out


def qsa_sparse_attn(q, k, v, indices, softmax_scale: float, out=None, workspace=None, stream=None):
    """Sparse attention over index rows; returns out ([R,3,256] fp16)."""
    torch = _torch()
    lib = library()
    R = _rows(q)
    if out is None:
        out = torch.empty((R, 3, 256), dtype=torch.float16, device=q.device)
    sh = _stream(stream, q.device)
    ws, ws_bytes = _ws_args(sparse_attn_workspace_bytes(R), q.device, sh, workspace, "attn")
    descs = [tensor_desc(t) for t in (q, k, v, indices)]
    od = tensor_desc(out)
    check(lib.qsa_sparse_attn(*[ctypes.byref(d) for d in descs], ctypes.c_float(softmax_scale),
                              ctypes.byref(od), ws, ws_bytes, ctypes.c_void_p(sh)))
    return out


def qsa_decode_step(q_sel, kcache, block_table, token_to_req, seq_lens, query_pos, q_attn, k, v,
                    softmax_scale: float, indices=None, out=None, workspace=None, stream=None):
    """Selection then attention on one stream; returns (indices, out)."""
    torch = _torch()
    lib = library()
    R = _rows(q_sel)
    if indices is None:
        indices = torch.empty((R, OUT_WIDTH), dtype=torch.int32, device=q_sel.device)
    if out is None:
        out = torch.empty((R, 3, 256), dtype=torch.float16, device=q_sel.device)
    sh = _stream(stream, q_sel.device)
    need = decode_step_workspace_bytes(R, block_table.shape[1]) if block_table.dim() == 2 else 0
    ws, ws_bytes = _ws_args(need, q_sel.device, sh, workspace, "decode")
    first = [tensor_desc(t) for t in (q_sel, kcache, block_table, token_to_req, seq_lens,
                                      query_pos, q_attn, k, v)]
    idd, od = tensor_desc(indices), tensor_desc(out)
    check(lib.qsa_decode_step(*[ctypes.byref(d) for d in first], ctypes.c_float(softmax_scale),
                              ctypes.byref(idd), ctypes.byref(od), ws, ws_bytes,
                              ctypes.c_void_p(sh)))
    return indices, out


def qsa_decode_step_fp8(q_sel, kcache, kscale, block_table, token_to_req, seq_lens, query_pos,
                        q_attn, k, v, softmax_scale: float, indices=None, out=None,
                        workspace=None, stream=None):
    """qsa_decode_step with the e4m3 key cache of qsa_select_fp8; returns
    (indices, out)."""
    torch = _torch()
    lib = library()
    R = _rows(q_sel)
    if indices is None:
        indices = torch.empty((R, OUT_WIDTH), dtype=torch.int32, device=q_sel.device)
    if out is None:
        out = torch.empty((R, 3, 256), dtype=torch.float16, device=q_sel.device)
    sh = _stream(stream, q_sel.device)
    need = decode_step_workspace_bytes(R, block_table.shape[1]) if block_table.dim() == 2 else 0
    ws, ws_bytes = _ws_args(need, q_sel.device, sh, workspace, "decode")
    first = [tensor_desc(t) for t in (q_sel, kcache, kscale, block_table, token_to_req, seq_lens,
                                      query_pos, q_attn, k, v)]
    idd, od = tensor_desc(indices), tensor_desc(out)
    check(lib.qsa_decode_step_fp8(*[ctypes.byref(d) for d in first], ctypes.c_float(softmax_scale),
                                  ctypes.byref(idd), ctypes.byref(od), ws, ws_bytes,
                                  ctypes.c_void_p(sh)))
    return indices, out


def qsa_decode_step_noalloc(q_sel, kcache, block_table, token_to_req, seq_lens, query_pos, q_attn,
                            k, v, softmax_scale: float, indices, out, stream=None):
    """qsa_decode_step without a workspace: the library's fixed per-GPU
    scratch stands in (for callers that cannot allocate; calls that overlap
    on one GPU race).  indices ([R,2051] int32) and out ([R,3,256] fp16) are
    the caller's; returns (indices, out)."""
    lib = library()
    sh = _stream(stream, q_sel.device)
    first = [tensor_desc(t) for t in (q_sel, kcache, block_table, token_to_req, seq_lens,
                                      query_pos, q_attn, k, v)]
    idd, od = tensor_desc(indices), tensor_desc(out)
    check(lib.qsa_decode_step_noalloc(*[ctypes.byref(d) for d in first],
                                      ctypes.c_float(softmax_scale), ctypes.byref(idd),
                                      ctypes.byref(od), ctypes.c_void_p(sh)))
    return indices, out


def build_metadata_workspace_bytes(num_reqs: int) -> int:
    return int(library().qsa_build_metadata_workspace_bytes(int(num_reqs)))


def qsa_build_metadata(query_start_loc, seq_lens, block_table, num_tokens: int,
                       storage_block_size: int = 128, compress_ratio: int = 4,
                       circular_buffer_size: int = 0, common_slot_mapping=None,
                       max_num_work: int = 0, with_slots: bool = True, out=None,
                       workspace=None, stream=None) -> dict:
    """Per-token metadata (token_to_req int32, logical_positions int64,
    visible_blocks int32, slot_mapping int64) and k work items
    [max_num_work, 2] int32, as device tensors in a dict (``out`` may hold
    preallocated ones under the same keys)."""
    torch = _torch()
    lib = library()
    dev = seq_lens.device
    T = int(num_tokens)
    o = dict(out or {})
    o.setdefault("token_to_req", torch.empty(T, dtype=torch.int32, device=dev))
    o.setdefault("logical_positions", torch.empty(T, dtype=torch.int64, device=dev))
    o.setdefault("visible_blocks", torch.empty(T, dtype=torch.int32, device=dev))
    if with_slots:
        o.setdefault("slot_mapping", torch.empty(T, dtype=torch.int64, device=dev))
    if max_num_work > 0:
        o.setdefault("k_work", torch.empty((int(max_num_work), 2), dtype=torch.int32, device=dev))
    sh = _stream(stream, dev)
    need = build_metadata_workspace_bytes(seq_lens.shape[0]) if max_num_work > 0 else 0
    ws, ws_bytes = _ws_args(need, dev, sh, workspace, "metadata")
    ins = [ctypes.byref(tensor_desc(t)) for t in (query_start_loc, seq_lens, block_table)]
    outs = [ctypes.byref(tensor_desc(o[k])) for k in ("token_to_req", "logical_positions",
                                                      "visible_blocks")]
    check(lib.qsa_build_metadata(*ins, _opt(common_slot_mapping), int(storage_block_size),
                                 int(compress_ratio), int(circular_buffer_size), *outs,
                                 _opt(o.get("slot_mapping")), _opt(o.get("k_work")), ws, ws_bytes,
                                 ctypes.c_void_p(sh)))
    return o
