"""Seeded synthetic workloads for the QSA decode path.

This module only draws inputs.  It holds none of the method's arithmetic
(no visible-block rule, no scores, no selection); the same arrays feed the
HIP path and the CPU oracle.  Everything is drawn on the CPU with
``numpy.random.default_rng(seed)`` in the fixed order listed for each
workload, so a seed names the bytes exactly.

Layouts (fp16 unless stated):

* ``q_sel``        [R, 4, 128]        four indexer heads per query row
* ``kcache``       [P, 128, 1, 128]   compressed keys, 128 slots per page
* ``block_table``  [N, W] int32       physical page of logical page j, -1 unused
* ``token_to_req`` [R] int32, ``seq_lens`` [N] int32, ``query_pos`` [R] int64
* ``q_attn``       [R, 3, 256]        three query heads sharing one K/V head
* ``kv``           [NP, 512, 512]     packed token rows: K = [..., :256],
                                      V = [..., 256:]; token t is flat row t
* ``indices``      [R, 2051] int32    attention index rows, -1 = hole
* ``kcodes``       [P, 128, 1, 128] uint8, ``kscale`` [P, 128] float32: the
                   same keys as an e4m3 cache (codes plus one scale per key),
                   for the workloads that carry one

A page of the compressed cache covers 128 compressed keys, i.e. 512 tokens
at four tokens per key, so a request of L tokens holds ceil(L / 512) pages.
Normal draws are float32 N(0,1) rounded to fp16.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

WIDTH = 2051
TOKENS_PER_PAGE = 512  # 128 compressed slots x 4 tokens
SLOTS = 128
SEL_HEADS, SEL_DIM = 4, 128
ATT_HEADS, ATT_DIM = 3, 256
KV_ROW = 512
SOFTMAX_SCALE = 1.0 / 16.0  # 1/sqrt(256)

_CHUNK = 1 << 24


@dataclass
class Workload:
    name: str
    seed: int
    q_sel: np.ndarray
    kcache: np.ndarray
    block_table: np.ndarray
    token_to_req: np.ndarray
    seq_lens: np.ndarray
    query_pos: np.ndarray
    q_attn: np.ndarray
    kv: np.ndarray
    scale: float = SOFTMAX_SCALE
    # standalone attention rows, when the workload defines them
    attn_indices: np.ndarray | None = None
    attn_q: np.ndarray | None = None
    notes: dict = field(default_factory=dict)
    # e4m3 form of the compressed-key cache (with_fp8_keys)
    kcodes: np.ndarray | None = None
    kscale: np.ndarray | None = None

    @property
    def rows(self) -> int:
        return int(self.q_sel.shape[0])

    def select_inputs(self) -> tuple:
        return (self.q_sel, self.kcache, self.block_table, self.token_to_req,
                self.seq_lens, self.query_pos)

    def select_inputs_fp8(self) -> tuple:
        assert self.kcodes is not None, "workload has no e4m3 key cache"
        return (self.q_sel, self.kcodes, self.kscale, self.block_table, self.token_to_req,
                self.seq_lens, self.query_pos)


# ---------------------------------------------------------------------------
# primitive draws

def normal_f16(rng: np.random.Generator, shape) -> np.ndarray:
    """float32 N(0,1) rounded to fp16, drawn in fixed-size chunks (so large
    caches do not need a float32 copy of the whole tensor)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float16)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    return out.reshape(shape)


def int_f16(rng: np.random.Generator, lo: int, hi: int, shape) -> np.ndarray:
    """Integer values uniform in [lo, hi] as fp16."""
    return rng.integers(lo, hi + 1, size=shape).astype(np.float16)


E4M3_MAX = 448.0


def e4m3_codes(values: np.ndarray) -> np.ndarray:
    """uint8 e4m3 ("e4m3fn") codes of float32 values, rounded to nearest even
    by torch's float8 cast after clipping to the format's range."""
    import torch

    v = np.clip(np.ascontiguousarray(values, dtype=np.float32), -E4M3_MAX, E4M3_MAX)
    return torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def fp8_integer_keys(rng: np.random.Generator, kcache: np.ndarray):
    """An e4m3 cache holding exactly the same integer-valued keys: each key
    gets a scale 2^j, j uniform in {-2..2}, and codes key / 2^j (integers in
    [-4, 4] scaled by 2^-j have at most two significant bits, so every code
    is exact and scale * code == key)."""
    P = kcache.shape[0]
    scales = np.ldexp(np.float32(1.0), rng.integers(-2, 3, size=(P, SLOTS))).astype(np.float32)
    vals = kcache.astype(np.float32) / scales[:, :, None, None]
    codes = e4m3_codes(vals)
    return codes, scales


def fp8_normal_keys(kcache: np.ndarray, slab: int = 1024):
    """Per-key absmax quantization of fp16 keys: scale = max|k| / 448 (1 for
    an all-zero key), codes = e4m3(k / scale).  Done in slabs of pages."""
    P = kcache.shape[0]
    codes = np.empty(kcache.shape, dtype=np.uint8)
    scales = np.empty((P, SLOTS), dtype=np.float32)
    for s0 in range(0, P, slab):
        k = kcache[s0:s0 + slab].astype(np.float32)
        amax = np.abs(k).max(axis=(2, 3))
        sc = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        scales[s0:s0 + slab] = sc
        codes[s0:s0 + slab] = e4m3_codes(k / sc[:, :, None, None])
    return codes, scales


def with_fp8_keys(w: "Workload", integer: bool) -> "Workload":
    """The workload with an e4m3 copy of its compressed-key cache attached:
    the same integer keys exactly (``integer``; scale exponents drawn from
    default_rng(seed + 7777)), or the absmax quantization of its keys."""
    if integer:
        w.kcodes, w.kscale = fp8_integer_keys(np.random.default_rng(w.seed + 7777), w.kcache)
    else:
        w.kcodes, w.kscale = fp8_normal_keys(w.kcache)
    w.name = w.name + "_fp8"
    return w


def head_weights(rng: np.random.Generator, rows: int, integer: bool = False) -> np.ndarray:
    """Per-head weights [rows, 4] float32: integers in [-3, 3] (exact sums
    on integer inputs), or uniform in [-0.5, 1.5] (mostly positive, some
    negative)."""
    if integer:
        return rng.integers(-3, 4, size=(rows, SEL_HEADS)).astype(np.float32)
    return rng.uniform(-0.5, 1.5, size=(rows, SEL_HEADS)).astype(np.float32)


def pages_needed(seq_len: int) -> int:
    """Pages a request of seq_len tokens occupies in the compressed cache."""
    return -(-int(seq_len) // TOKENS_PER_PAGE)


def block_table_distinct(rng: np.random.Generator, lengths, num_pages: int,
                         width: int | None = None) -> np.ndarray:
    """One row per request; pages drawn without replacement over the whole
    batch (no sharing); unused entries -1."""
    need = [pages_needed(L) for L in lengths]
    w = max(need + [1]) if width is None else width
    total = sum(need)
    assert total <= num_pages, "not enough pages for distinct tables"
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.full((len(lengths), w), -1, dtype=np.int32)
    pos = 0
    for i, n in enumerate(need):
        bt[i, :n] = perm[pos:pos + n]
        pos += n
    return bt


def block_table_per_row(rng: np.random.Generator, lengths, num_pages: int,
                        width: int | None = None) -> np.ndarray:
    """Distinct pages within each row, drawn independently per row (rows may
    share pages by chance); unused entries -1."""
    need = [pages_needed(L) for L in lengths]
    w = max(need + [1]) if width is None else width
    bt = np.full((len(lengths), w), -1, dtype=np.int32)
    for i, n in enumerate(need):
        if n:
            bt[i, :n] = rng.permutation(num_pages)[:n]
    return bt


def inject_holes_and_duplicates(rng: np.random.Generator, indices: np.ndarray,
                                hole_frac: float, dup_frac: float) -> np.ndarray:
    """Copy of ``indices`` in which, per row, round(hole_frac * 2051) columns
    holding a valid index become -1 and round(dup_frac * 2051) other valid
    columns are overwritten with a copy of another valid entry of the row."""
    out = np.array(indices, dtype=np.int32, copy=True)
    n_holes = int(round(hole_frac * WIDTH))
    n_dups = int(round(dup_frac * WIDTH))
    for r in range(out.shape[0]):
        valid = np.flatnonzero(out[r] >= 0)
        if valid.size < 2:
            continue
        pick = rng.permutation(valid)
        holes = pick[:min(n_holes, valid.size // 3)]
        dups = pick[holes.size:holes.size + min(n_dups, valid.size // 3)]
        keep = pick[holes.size + dups.size:]
        if dups.size and keep.size:
            out[r, dups] = out[r, rng.choice(keep, size=dups.size)]
        out[r, holes] = -1
    return out


def random_index_rows(rng: np.random.Generator, rows: int, num_tokens: int,
                      valid: int = WIDTH, distinct: bool = True) -> np.ndarray:
    """[rows, 2051] rows whose first ``valid`` columns are random token slots
    (distinct within a row when asked), the rest -1."""
    out = np.full((rows, WIDTH), -1, dtype=np.int32)
    for r in range(rows):
        if distinct:
            out[r, :valid] = rng.choice(num_tokens, size=valid, replace=False)
        else:
            out[r, :valid] = rng.integers(0, num_tokens, size=valid)
    return out


def decode_rows(lengths) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One decode query per request: token_to_req = r, query_pos = L - 1."""
    lengths = np.asarray(lengths, dtype=np.int64)
    R = lengths.size
    return (np.arange(R, dtype=np.int32), lengths.astype(np.int32),
            (lengths - 1).astype(np.int64))


# ---------------------------------------------------------------------------
# the named workloads

def tiny_integer(seed: int = 0) -> Workload:
    """R=1, L=519 (a cross-page tail), integer-valued keys and queries.

    Draw order: q_sel int [-4,4]; kcache int [-4,4] [8,128,1,128]; for every
    page and every group of 16 slots, slot 15 of the group is overwritten
    with a copy of a random slot 0..14 of the same group (1 key in 16 is a
    duplicate, forcing exact score ties); block table = 2 distinct pages of
    8; q_attn N(0,1) [1,3,256]; kv N(0,1) [2,512,512].
    """
    rng = np.random.default_rng(seed)
    q_sel = int_f16(rng, -4, 4, (1, SEL_HEADS, SEL_DIM))
    kcache = int_f16(rng, -4, 4, (8, SLOTS, 1, SEL_DIM))
    for p in range(8):
        for g in range(SLOTS // 16):
            src = int(rng.integers(0, 15))
            kcache[p, 16 * g + 15] = kcache[p, 16 * g + src]
    bt = rng.permutation(8)[:2].astype(np.int32).reshape(1, 2)
    t2r, sl, qp = decode_rows([519])
    q_attn = normal_f16(rng, (1, ATT_HEADS, ATT_DIM))
    kv = normal_f16(rng, (2, TOKENS_PER_PAGE, KV_ROW))
    return Workload("tiny_integer_R1_L519", seed, q_sel, kcache, bt, t2r, sl, qp, q_attn, kv)


def saturated_row(seed: int = 0) -> Workload:
    """R=1, L=9215 over an 8192-page N(0,1) cache: 2303 visible blocks, the
    top-512 saturates the 2051-wide output.

    Draw order: kcache N(0,1) [8192,128,1,128]; block table = 18 distinct
    pages; q_sel N(0,1); q_attn N(0,1); kv N(0,1) [32,512,512].
    Attention index rows are the selection output with 5% holes and 5%
    duplicates injected by ``inject_holes_and_duplicates`` (seed + 1).
    """
    rng = np.random.default_rng(seed)
    kcache = normal_f16(rng, (8192, SLOTS, 1, SEL_DIM))
    bt = rng.permutation(8192)[:18].astype(np.int32).reshape(1, 18)
    t2r, sl, qp = decode_rows([9215])
    q_sel = normal_f16(rng, (1, SEL_HEADS, SEL_DIM))
    q_attn = normal_f16(rng, (1, ATT_HEADS, ATT_DIM))
    kv = normal_f16(rng, (32, TOKENS_PER_PAGE, KV_ROW))
    w = Workload("saturated_R1_L9215_P8192", seed, q_sel, kcache, bt, t2r, sl, qp, q_attn, kv)
    w.notes["attn_perturb"] = dict(hole_frac=0.05, dup_frac=0.05, seed=seed + 1)
    return w


def batched_shared(seed: int = 0) -> Workload:
    """R=64 decode rows, L uniform in [512, 32768], 16384 N(0,1) pages; the
    block tables of requests 2i and 2i+1 map their first
    floor(min(n_2i, n_2i+1) / 2) logical pages to the same physical pages.

    Draw order: lengths; distinct block tables; kcache N(0,1); q_sel N(0,1);
    q_attn N(0,1); kv N(0,1) sized to the longest request.
    """
    rng = np.random.default_rng(seed)
    R, P = 64, 16384
    lengths = rng.integers(512, 32768 + 1, size=R)
    bt = block_table_distinct(rng, lengths, P)
    for i in range(0, R, 2):
        share = min(pages_needed(lengths[i]), pages_needed(lengths[i + 1])) // 2
        bt[i + 1, :share] = bt[i, :share]
    kcache = normal_f16(rng, (P, SLOTS, 1, SEL_DIM))
    q_sel = normal_f16(rng, (R, SEL_HEADS, SEL_DIM))
    q_attn = normal_f16(rng, (R, ATT_HEADS, ATT_DIM))
    kv_pages = pages_needed(int(lengths.max()))
    kv = normal_f16(rng, (kv_pages, TOKENS_PER_PAGE, KV_ROW))
    t2r, sl, qp = decode_rows(lengths)
    return Workload("batched_R64_shared_pages", seed, q_sel, kcache, bt, t2r, sl, qp, q_attn, kv)


EDGE_LENGTHS = [0, 1, 2, 3, 512, 513, 516, 1027, 2049, 4100, 65535, 65536]


def ties_and_edges(seed: int = 0) -> Workload:
    """R=32 rows cycling over EDGE_LENGTHS (empty, tail only, exactly one page
    of blocks, page crossings, 65536).  Keys come from a palette of 64
    integer vectors in [-4,4], so scores tie massively; queries are integers
    in [-2,2].

    Draw order: palette int [-4,4] [64,128]; palette choice per cache slot
    (P=4096); per-row block tables (distinct within a row); q_sel int
    [-2,2]; q_attn N(0,1) [35,3,256]; kv N(0,1) [128,512,512]; then the
    standalone attention rows: 32 selection-shaped rows are made by the
    caller, plus three explicit rows appended here (all -1; one index; one
    index repeated 2051 times) whose token ids are drawn last.
    """
    rng = np.random.default_rng(seed)
    R, P = 32, 4096
    lengths = [EDGE_LENGTHS[i % len(EDGE_LENGTHS)] for i in range(R)]
    palette = int_f16(rng, -4, 4, (64, SEL_DIM))
    choice = rng.integers(0, 64, size=(P, SLOTS))
    kcache = palette[choice].reshape(P, SLOTS, 1, SEL_DIM)
    bt = block_table_per_row(rng, lengths, P, width=128)
    q_sel = int_f16(rng, -2, 2, (R, SEL_HEADS, SEL_DIM))
    q_attn = normal_f16(rng, (R + 3, ATT_HEADS, ATT_DIM))
    kv = normal_f16(rng, (128, TOKENS_PER_PAGE, KV_ROW))
    extra = np.full((3, WIDTH), -1, dtype=np.int32)
    extra[1, 0] = rng.integers(0, 128 * TOKENS_PER_PAGE)
    extra[2, :] = rng.integers(0, 128 * TOKENS_PER_PAGE)
    t2r, sl, qp = decode_rows(lengths)
    w = Workload("ties_edges_R32_palette64", seed, q_sel, kcache, bt, t2r, sl, qp,
                 q_attn[:R], kv)
    w.attn_q = q_attn
    w.notes["attn_extra_rows"] = extra
    w.notes["attn_perturb"] = dict(hole_frac=0.05, dup_frac=0.05, seed=seed + 1)
    return w


def long_context(seed: int = 0, rows: int = 128) -> Workload:
    """R=128 decode rows of L=131072 (32768 blocks each) over a 32768-page
    N(0,1) cache (1 GiB) behind a random permutation of the pages; packed
    KV of 131072 tokens (128 MiB).

    Draw order: kcache N(0,1) [32768,128,1,128]; block table =
    permutation(32768) reshaped [128,256]; q_sel N(0,1); q_attn N(0,1);
    kv N(0,1) [256,512,512]; standalone attention rows = 2051 distinct
    random token slots per row.  ``rows`` < 128 keeps the first rows of the
    same draw (for bounded checks).
    """
    rng = np.random.default_rng(seed)
    R, P = 128, 32768
    kcache = normal_f16(rng, (P, SLOTS, 1, SEL_DIM))
    bt = rng.permutation(P).astype(np.int32).reshape(R, P // R)
    q_sel = normal_f16(rng, (R, SEL_HEADS, SEL_DIM))
    q_attn = normal_f16(rng, (R, ATT_HEADS, ATT_DIM))
    kv = normal_f16(rng, (256, TOKENS_PER_PAGE, KV_ROW))
    attn_idx = random_index_rows(rng, R, 256 * TOKENS_PER_PAGE)
    t2r, sl, qp = decode_rows([131072] * R)
    w = Workload("long_context_R128_L131072", seed, q_sel[:rows], kcache, bt[:rows],
                 t2r[:rows], sl[:rows], qp[:rows], q_attn[:rows], kv)
    w.attn_indices = attn_idx[:rows]
    w.attn_q = q_attn[:rows]
    return w


def multi_token_rows(seed: int = 0, decode_requests: int = 48, next_n: int = 4,
                     prefill_requests: int = 4, prefill_chunk: int = 16,
                     integer: bool = False) -> Workload:
    """Several query rows per request: speculative-decode requests score
    next_n draft positions each (query positions L - next_n .. L - 1) and
    chunked-prefill requests score a chunk of prefill_chunk positions
    (L - prefill_chunk .. L - 1); one row per position, rows of a request
    adjacent.  L is uniform in [8192, 65536]; 8192 N(0,1) pages (or integer
    keys in [-4,4] with integer queries in [-2,2] when ``integer``).

    Draw order: lengths (decode requests, then prefill requests); per-row
    distinct block tables; kcache; q_sel; q_attn; kv (N(0,1), sized to the
    longest request).
    """
    rng = np.random.default_rng(seed)
    N = decode_requests + prefill_requests
    lengths = rng.integers(8192, 65536 + 1, size=N)
    per_req = [next_n] * decode_requests + [prefill_chunk] * prefill_requests
    P = 8192
    bt = block_table_per_row(rng, lengths, P)
    if integer:
        kcache = int_f16(rng, -4, 4, (P, SLOTS, 1, SEL_DIM))
    else:
        kcache = normal_f16(rng, (P, SLOTS, 1, SEL_DIM))
    t2r = np.concatenate([np.full(c, i, np.int32) for i, c in enumerate(per_req)])
    qp = np.concatenate([int(L) - c + np.arange(c) for L, c in zip(lengths, per_req)]).astype(np.int64)
    R = t2r.size
    q_sel = int_f16(rng, -2, 2, (R, SEL_HEADS, SEL_DIM)) if integer else normal_f16(rng, (R, SEL_HEADS, SEL_DIM))
    q_attn = normal_f16(rng, (R, ATT_HEADS, ATT_DIM))
    kv = normal_f16(rng, (pages_needed(int(lengths.max())), TOKENS_PER_PAGE, KV_ROW))
    name = f"multi_token_R{R}_next{next_n}_prefill{prefill_chunk}" + ("_int" if integer else "")
    return Workload(name, seed, q_sel, kcache, bt, t2r, lengths.astype(np.int32), qp, q_attn, kv)


def query_start_loc(w: Workload) -> np.ndarray:
    """Cumulative query starts [N+1] int32 of a workload whose rows are
    grouped request by request (the metadata builder's input)."""
    t2r = np.asarray(w.token_to_req)
    assert np.all(np.diff(t2r) >= 0), "rows must be grouped by request"
    counts = np.bincount(t2r, minlength=len(w.seq_lens))
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


def serving_batch(seed: int = 0, decode: int = 160, spec: int = 48, next_n: int = 4,
                  prefill: int = 8, chunk: int = 512, empty: int = 16, pad: int = 64):
    """Builder inputs for a mixed serving step: decode rows (1 token),
    speculative rows (next_n tokens), chunked-prefill rows (chunk tokens),
    requests with an empty query, interleaved at random, L ~ U[1024, 131072];
    a block table of random block ids with 5% holes; a common slot mapping
    with 2% skipped tokens; pad padding tokens.

    Draw order: request kinds permutation; lengths; block table; holes;
    common slots; skipped-slot mask.
    Returns (query_start_loc, seq_lens, block_table, common_slot_mapping,
    num_tokens)."""
    rng = np.random.default_rng(seed)
    kinds = np.array([1] * decode + [next_n] * spec + [chunk] * prefill + [0] * empty)
    kinds = kinds[rng.permutation(kinds.size)]
    N = kinds.size
    L = rng.integers(1024, 131072 + 1, size=N)
    qsl = np.concatenate([[0], np.cumsum(kinds)]).astype(np.int32)
    W = pages_needed(131072)
    bt = rng.integers(0, 1 << 20, size=(N, W)).astype(np.int32)
    bt[rng.random(bt.shape) < 0.05] = -1
    T = int(qsl[-1]) + pad
    csm = rng.integers(0, 1 << 30, size=T).astype(np.int64)
    csm[rng.random(T) < 0.02] = -1
    return qsl, L.astype(np.int32), bt, csm, T


NAMED = {
    1: tiny_integer,
    2: saturated_row,
    3: batched_shared,
    4: ties_and_edges,
    5: long_context,
    6: multi_token_rows,
}


def make(config: int, seed: int = 0) -> Workload:
    return NAMED[int(config)](seed)
