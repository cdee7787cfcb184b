"""CPU oracle for the QSA selection + sparse-attention decode path.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the CPU-baseline leg of the bench, never by the product package.  It loads
``libqsa_oracle.so`` (plain single-threaded C, built with gcc from
``qsa_oracle.c``) through ctypes and hands it numpy arrays.  Nothing here
touches the HIP library.

Parity status of each function (the pins live in ``tests/oracle_pins.py``):

* ``row_extent``   pinned: the pages' worked examples, closed forms.
* ``select``       pinned: brute force over exact integer scores with a
  rank-counting selector, library-sort cross-check, invariants, special
  cases with closed-form answers.
* ``row_scores``   pinned: exact integer dot products; numpy float64 gather.
* ``sparse_attn``  pinned: single-index/duplicate/hole closed forms, equal
  logits -> mean, two-token logistic form, torch float64 library softmax.
* ``half_to_double`` pinned: every binary16 bit pattern against numpy.
* ``e4m3_to_double`` pinned: every e4m3 code against torch.float8_e4m3fn.
* ``select_fp8`` / ``row_scores_fp8`` pinned: integer keys re-encoded as
  e4m3 codes with power-of-two scales give the fp16 selection (itself
  pinned by brute force) exactly; one-hot queries read back scale * code for
  every code; numpy float64 gather of the dequantized keys + lexsort.
* ``select_weighted`` / ``paged_logits`` / ``topk_per_row`` pinned: integer
  brute force with integer (also negative) head weights; weights of one give
  the unweighted selection; numpy float64 gather + weights; top-k per row
  against numpy's lexsort on arbitrary logits (negative values, signed zeros,
  repeats, junk past the visible blocks).
* ``build_metadata`` pinned: batches built request by request (decode,
  speculative, prefill chunks, empty queries, padding tokens, holes in the
  block table, invalid common slots) whose per-token request, position,
  visible blocks, slots and k work items are known by construction; numpy's
  searchsorted for the request search on random batches.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "qsa_oracle.c")
LIBRARY = os.path.join(HERE, "libqsa_oracle.so")

WIDTH = 2051
TOPK_BLOCKS = 512
RATIO = 4

ERRORS = {
    -1: "token_to_req outside [0, N)",
    -2: "a visible block lies beyond the block table",
    -3: "a needed page id outside [0, P)",
    -4: "an attention index outside [-1, NT)",
    -5: "out of memory",
    -6: "bad argument",
}


def build(out_path: str = LIBRARY, mutant: int = 0) -> str:
    """Compile the oracle with gcc (no fast-math, no threads).

    ``mutant`` > 0 plants one known mistake (see the source header); only the
    pin tests' self-check asks for that.
    """
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
           f"-DQSA_ORACLE_MUTANT={int(mutant)}", "-o", out_path, SOURCE, "-lm"]
    subprocess.run(cmd, check=True)
    return out_path


class Oracle:
    """ctypes view of one build of the oracle library."""

    def __init__(self, path: str = LIBRARY):
        if not os.path.exists(path):
            build(path)
        self.path = path
        lib = ctypes.CDLL(path)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.qsa_oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.qsa_oracle_half_to_double.restype = ctypes.c_double
        lib.qsa_oracle_row_extent.argtypes = [i64, i64, p, p]
        lib.qsa_oracle_row_extent.restype = None
        lib.qsa_oracle_row_scores.argtypes = [i64, i64, i64, i64, p, p, p, p, p, p, p, i64, p]
        lib.qsa_oracle_row_scores.restype = ctypes.c_int
        lib.qsa_oracle_select.argtypes = [i64, i64, i64, i64, p, p, p, p, p, p, p]
        lib.qsa_oracle_select.restype = ctypes.c_int
        lib.qsa_oracle_sparse_attn.argtypes = [i64, i64, p, p, p, ctypes.c_double, p]
        lib.qsa_oracle_sparse_attn.restype = ctypes.c_int
        lib.qsa_oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        lib.qsa_oracle_e4m3_to_double.restype = ctypes.c_double
        lib.qsa_oracle_row_scores_fp8.argtypes = [i64, i64, i64, i64, p, p, p, p, p, p, p, p, i64, p]
        lib.qsa_oracle_row_scores_fp8.restype = ctypes.c_int
        lib.qsa_oracle_select_fp8.argtypes = [i64, i64, i64, i64, p, p, p, p, p, p, p, p]
        lib.qsa_oracle_select_fp8.restype = ctypes.c_int
        lib.qsa_oracle_select_weighted.argtypes = [i64, i64, i64, i64] + [p] * 10
        lib.qsa_oracle_select_weighted.restype = ctypes.c_int
        lib.qsa_oracle_paged_logits.argtypes = [i64, i64, i64, i64] + [p] * 10 + [i64, i64]
        lib.qsa_oracle_paged_logits.restype = ctypes.c_int
        lib.qsa_oracle_topk_per_row.argtypes = [i64, i64, p, i64, i64, p, p, p, p]
        lib.qsa_oracle_topk_per_row.restype = ctypes.c_int
        lib.qsa_oracle_build_metadata.argtypes = [i64, i64, p, p, p, p, i64, i64, i64, i64, i64,
                                                   p, p, p, p, p, i64]
        lib.qsa_oracle_build_metadata.restype = ctypes.c_int
        lib.qsa_oracle_mutant.argtypes = []
        lib.qsa_oracle_mutant.restype = ctypes.c_int
        self.lib = lib
        self.mutant = lib.qsa_oracle_mutant()

    # -- helpers -----------------------------------------------------------
    @staticmethod
    def _c(a: np.ndarray, dtype) -> np.ndarray:
        return np.ascontiguousarray(a, dtype=dtype)

    @staticmethod
    def _ptr(a: np.ndarray):
        return ctypes.c_void_p(a.ctypes.data)

    @staticmethod
    def _check(rc: int) -> None:
        if rc != 0:
            raise ValueError(f"oracle precondition violated: {ERRORS.get(rc, rc)}")

    # -- API ---------------------------------------------------------------
    def half_to_double(self, bits: int) -> float:
        return self.lib.qsa_oracle_half_to_double(int(bits) & 0xFFFF)

    def e4m3_to_double(self, code: int) -> float:
        return self.lib.qsa_oracle_e4m3_to_double(int(code) & 0xFF)

    def row_extent(self, seq_len: int, query_pos: int) -> tuple[int, int]:
        """(visible blocks V, tail length T) of one query row."""
        v, t = ctypes.c_int64(), ctypes.c_int64()
        self.lib.qsa_oracle_row_extent(int(seq_len), int(query_pos),
                                       ctypes.byref(v), ctypes.byref(t))
        return v.value, t.value

    def _select_args(self, q, kcache, block_table, token_to_req, seq_lens, query_pos):
        q = self._c(q, np.float16)
        kcache = self._c(kcache, np.float16)
        bt = self._c(block_table, np.int32)
        t2r = self._c(token_to_req, np.int32)
        sl = self._c(seq_lens, np.int32)
        qp = self._c(query_pos, np.int64)
        assert q.ndim == 3 and q.shape[1:] == (4, 128)
        assert kcache.shape[1:] == (128, 1, 128)
        assert bt.ndim == 2
        return q, kcache, bt, t2r, sl, qp

    def select(self, q, kcache, block_table, token_to_req, seq_lens, query_pos) -> np.ndarray:
        """[R,2051] int32 selected token indices (see qsa_oracle.c)."""
        q, kcache, bt, t2r, sl, qp = self._select_args(
            q, kcache, block_table, token_to_req, seq_lens, query_pos)
        R = q.shape[0]
        out = np.empty((R, WIDTH), dtype=np.int32)
        rc = self.lib.qsa_oracle_select(
            R, kcache.shape[0], sl.shape[0], bt.shape[1], self._ptr(q), self._ptr(kcache),
            self._ptr(bt), self._ptr(t2r), self._ptr(sl), self._ptr(qp), self._ptr(out))
        self._check(rc)
        return out

    def row_scores(self, r, q, kcache, block_table, token_to_req, seq_lens, query_pos) -> np.ndarray:
        """float32 scores of every visible block of row r, in block order."""
        q, kcache, bt, t2r, sl, qp = self._select_args(
            q, kcache, block_table, token_to_req, seq_lens, query_pos)
        max_blocks = bt.shape[1] * 128
        scores = np.zeros(max_blocks, dtype=np.float32)
        v = ctypes.c_int64()
        rc = self.lib.qsa_oracle_row_scores(
            int(r), kcache.shape[0], sl.shape[0], bt.shape[1], self._ptr(q), self._ptr(kcache),
            self._ptr(bt), self._ptr(t2r), self._ptr(sl), self._ptr(qp), self._ptr(scores),
            max_blocks, ctypes.byref(v))
        self._check(rc)
        return scores[: v.value].copy()

    def _fp8_cache(self, codes, scales):
        codes = self._c(codes, np.uint8)
        scales = self._c(scales, np.float32)
        assert codes.shape[1:] == (128, 1, 128)
        assert scales.shape == codes.shape[:2]
        return codes, scales

    def select_fp8(self, q, codes, scales, block_table, token_to_req, seq_lens,
                   query_pos) -> np.ndarray:
        """[R,2051] int32 selection over an e4m3 key cache: codes
        [P,128,1,128] uint8, scales [P,128] float32."""
        q, _, bt, t2r, sl, qp = self._select_args(
            q, np.zeros((1, 128, 1, 128), np.float16), block_table, token_to_req, seq_lens,
            query_pos)
        codes, scales = self._fp8_cache(codes, scales)
        R = q.shape[0]
        out = np.empty((R, WIDTH), dtype=np.int32)
        rc = self.lib.qsa_oracle_select_fp8(
            R, codes.shape[0], sl.shape[0], bt.shape[1], self._ptr(q), self._ptr(codes),
            self._ptr(scales), self._ptr(bt), self._ptr(t2r), self._ptr(sl), self._ptr(qp),
            self._ptr(out))
        self._check(rc)
        return out

    def row_scores_fp8(self, r, q, codes, scales, block_table, token_to_req, seq_lens,
                       query_pos) -> np.ndarray:
        """float32 scores of every visible block of row r over an e4m3 cache."""
        q, _, bt, t2r, sl, qp = self._select_args(
            q, np.zeros((1, 128, 1, 128), np.float16), block_table, token_to_req, seq_lens,
            query_pos)
        codes, scales = self._fp8_cache(codes, scales)
        max_blocks = bt.shape[1] * 128
        out = np.zeros(max_blocks, dtype=np.float32)
        v = ctypes.c_int64()
        rc = self.lib.qsa_oracle_row_scores_fp8(
            int(r), codes.shape[0], sl.shape[0], bt.shape[1], self._ptr(q), self._ptr(codes),
            self._ptr(scales), self._ptr(bt), self._ptr(t2r), self._ptr(sl), self._ptr(qp),
            self._ptr(out), max_blocks, ctypes.byref(v))
        self._check(rc)
        return out[: v.value].copy()

    def _cache_ptrs(self, kcache, codes, scales):
        """(kcache, codes, scales) arrays and pointers for the entry points
        that take either an fp16 cache or e4m3 codes + scales."""
        if codes is not None:
            codes, scales = self._fp8_cache(codes, scales)
            return codes.shape[0], None, self._ptr(codes), self._ptr(scales), (codes, scales)
        kcache = self._c(kcache, np.float16)
        assert kcache.shape[1:] == (128, 1, 128)
        return kcache.shape[0], self._ptr(kcache), None, None, (kcache,)

    def _weights(self, weights, R):
        if weights is None:
            return None, None
        w = self._c(weights, np.float32)
        assert w.shape == (R, 4)
        return w, self._ptr(w)

    def select_weighted(self, q, weights, block_table, token_to_req, seq_lens, query_pos,
                        kcache=None, codes=None, scales=None) -> np.ndarray:
        """[R,2051] selection with per-head weights [R,4] (fp16 cache, or
        e4m3 codes + scales)."""
        q, _, bt, t2r, sl, qp = self._select_args(
            q, np.zeros((1, 128, 1, 128), np.float16), block_table, token_to_req, seq_lens,
            query_pos)
        R = q.shape[0]
        P, kp, cp, sp, keep = self._cache_ptrs(kcache, codes, scales)
        w, wp = self._weights(weights, R)
        out = np.empty((R, WIDTH), dtype=np.int32)
        rc = self.lib.qsa_oracle_select_weighted(
            R, P, sl.shape[0], bt.shape[1], self._ptr(q), wp, kp, cp, sp, self._ptr(bt),
            self._ptr(t2r), self._ptr(sl), self._ptr(qp), self._ptr(out))
        self._check(rc)
        return out

    def paged_logits(self, q, weights, block_table, token_to_req, seq_lens, query_pos, width,
                     kcache=None, codes=None, scales=None) -> np.ndarray:
        """[R,width] float32: block scores for b < V, -inf past V."""
        q, _, bt, t2r, sl, qp = self._select_args(
            q, np.zeros((1, 128, 1, 128), np.float16), block_table, token_to_req, seq_lens,
            query_pos)
        R = q.shape[0]
        P, kp, cp, sp, keep = self._cache_ptrs(kcache, codes, scales)
        w, wp = self._weights(weights, R)
        out = np.empty((R, int(width)), dtype=np.float32)
        rc = self.lib.qsa_oracle_paged_logits(
            R, P, sl.shape[0], bt.shape[1], self._ptr(q), wp, kp, cp, sp, self._ptr(bt),
            self._ptr(t2r), self._ptr(sl), self._ptr(qp), self._ptr(out), int(width), int(width))
        self._check(rc)
        return out

    def topk_per_row(self, logits, token_to_req, seq_lens, query_pos) -> np.ndarray:
        """[R,2051] selection from a given [R, width] float32 logits matrix."""
        lg = self._c(logits, np.float32)
        t2r = self._c(token_to_req, np.int32)
        sl = self._c(seq_lens, np.int32)
        qp = self._c(query_pos, np.int64)
        R = lg.shape[0]
        out = np.empty((R, WIDTH), dtype=np.int32)
        rc = self.lib.qsa_oracle_topk_per_row(
            R, sl.shape[0], self._ptr(lg), lg.shape[1], lg.shape[1], self._ptr(t2r),
            self._ptr(sl), self._ptr(qp), self._ptr(out))
        self._check(rc)
        return out

    def build_metadata(self, query_start_loc, seq_lens, block_table, num_tokens: int,
                       storage_block_size: int = 128, compress_ratio: int = 4,
                       circular_buffer_size: int = 0, common_slot_mapping=None,
                       max_num_work: int = 0, with_slots: bool = True) -> dict:
        """Per-token metadata (token_to_req, logical_positions,
        visible_blocks, slot_mapping) and the k work items [max_num_work, 2]."""
        qsl = self._c(query_start_loc, np.int32)
        sl = self._c(seq_lens, np.int32)
        bt = self._c(block_table, np.int32)
        N = sl.shape[0]
        assert qsl.shape == (N + 1,) and bt.ndim == 2 and bt.shape[0] == N
        T = int(num_tokens)
        csm = None if common_slot_mapping is None else self._c(common_slot_mapping, np.int64)
        if csm is not None:
            assert csm.shape == (T,)
        t2r = np.empty(T, np.int32)
        lp = np.empty(T, np.int64)
        vis = np.empty(T, np.int32)
        slots = np.empty(T, np.int64) if with_slots else None
        work = np.empty((int(max_num_work), 2), np.int32) if max_num_work > 0 else None
        rc = self.lib.qsa_oracle_build_metadata(
            N, T, self._ptr(qsl), self._ptr(sl), None if csm is None else self._ptr(csm),
            self._ptr(bt), bt.shape[1], bt.shape[1], int(storage_block_size), int(compress_ratio),
            int(circular_buffer_size), self._ptr(t2r), self._ptr(lp), self._ptr(vis),
            None if slots is None else self._ptr(slots), None if work is None else self._ptr(work),
            int(max_num_work))
        self._check(rc)
        return {"token_to_req": t2r, "logical_positions": lp, "visible_blocks": vis,
                "slot_mapping": slots, "k_work": work}

    def sparse_attn(self, q, kv, indices, scale: float) -> np.ndarray:
        """[R,3,256] float64 attention output.  kv is [..., 512] fp16 with
        token t at flat row t (K = [:256], V = [256:])."""
        q = self._c(q, np.float16)
        kv = self._c(kv, np.float16).reshape(-1, 512)
        idx = self._c(indices, np.int32)
        assert q.ndim == 3 and q.shape[1:] == (3, 256)
        assert idx.shape == (q.shape[0], WIDTH)
        out = np.empty((q.shape[0], 3, 256), dtype=np.float64)
        rc = self.lib.qsa_oracle_sparse_attn(
            q.shape[0], kv.shape[0], self._ptr(q), self._ptr(kv), self._ptr(idx),
            float(scale), self._ptr(out))
        self._check(rc)
        return out


_DEFAULT: Oracle | None = None


def default() -> Oracle:
    """The trusted (mutant-free) oracle build, compiled on first use."""
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle(LIBRARY)
        assert _DEFAULT.mutant == 0
    return _DEFAULT
