/*
 * qsa.h -- C ABI of the MI355X (gfx950) QSA sparse-attention decode library.
 *
 * Two stages of one decode step, as the page "vLLM: integrate FP16 packed QSA
 * extension" (intel/llm-scaler PR #651) defines them in its sections
 * "Summary" and "Exact contracts":
 *
 *   qsa_select       paged top-512 block selection -> [R,2051] token indices
 *   qsa_sparse_attn  fp16 attention over exactly those indices
 *   qsa_decode_step  both, back to back on one stream, indices stay on device
 *
 * and the same selection over an fp8 e4m3 compressed-key cache
 * (qsa_select_fp8, qsa_decode_step_fp8), with per-head weights
 * (qsa_select_weighted), and in two passes: scores materialised as a logits
 * matrix (qsa_paged_logits), then a top-k per row over it
 * (qsa_topk_per_row); and the metadata step before them
 * (qsa_build_metadata: per-token request, position, visible blocks, cache
 * slots and k work items).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are passed as qsa_tensor descriptors: a DEVICE pointer to the
 *   first element (any storage offset already applied), a dtype code, and
 *   shape/strides in elements.  The descriptors themselves are host memory
 *   read during the call only.  The library never keeps a pointer.
 * - Every call is asynchronous on `stream` (a hipStream_t; NULL = the legacy
 *   default stream of the current device).  The library never allocates,
 *   never synchronises and never prints.  Pointers must belong to the
 *   current HIP device.
 * - Fail-closed: all arguments are validated on the host before anything is
 *   launched ("fail-closed dtype/layout checks" and "fail-closed
 *   dtype/output checks" in the page's "Validation" section).  On a
 *   validation status (anything but QSA_OK and QSA_ERR_LAUNCH) nothing is
 *   launched and no output or workspace byte is written; qsa_last_error()
 *   then describes the first failed check.  QSA_ERR_LAUNCH means the HIP
 *   runtime rejected a kernel launch (qsa_decode_step: the selection may
 *   already be enqueued when the attention launch is rejected).
 * - Outputs are caller-owned and must not overlap any input or the
 *   workspace; inputs are never written ("caller-owned output; inputs remain
 *   unchanged", "Exact contracts").
 * - R = 0 rows is a valid no-op returning QSA_OK.
 * - Device-side preconditions that cannot be checked without a sync:
 *   token_to_req[r] in [0, N); the block-table entries of every visible
 *   block in [0, P); every attention index is -1 or in [0, NT); fp16 inputs
 *   finite.  The kernels stay memory-safe when these fail (a row with an
 *   out-of-range request is treated as empty, a page id outside [0,P) as an
 *   all-zero key, visible blocks beyond the block table's width are not
 *   read, an index outside [-1, NT) as a hole) but the result is then
 *   unspecified.
 * - Workspaces: device memory of at least the queried size, 256-byte
 *   aligned, with any content (the library keeps no state in it between
 *   calls: every byte it reads there was written earlier in the same call).
 *   Calls that may run concurrently (different streams) must not share a
 *   workspace; consecutive calls on one stream may.
 * - Thread safety: any host thread may call; qsa_last_error() is per thread.
 */
#ifndef QSA_H_
#define QSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_API __attribute__((visibility("default")))

/* Fixed contract constants ("Exact contracts", selection: token_topk=2048,
 * compress_ratio=4, output [R,2051]). */
#define QSA_TOKEN_TOPK 2048
#define QSA_COMPRESS_RATIO 4
#define QSA_TOPK_BLOCKS 512  /* token_topk / compress_ratio */
#define QSA_OUT_WIDTH 2051   /* 2048 selected tokens + at most 3 tail tokens */
#define QSA_PAGE_SLOTS 128   /* compressed keys per cache page */
#define QSA_SEL_HEADS 4
#define QSA_SEL_DIM 128
#define QSA_ATT_HEADS 3
#define QSA_ATT_DIM 256
#define QSA_KV_PAGE_TOKENS 512

typedef enum {
  QSA_DTYPE_F16 = 1,
  QSA_DTYPE_I32 = 2,
  QSA_DTYPE_I64 = 3,
  QSA_DTYPE_F32 = 4,
  QSA_DTYPE_E4M3 = 5 /* one byte per element: OCP e4m3 without infinities ("e4m3fn") */
} qsa_dtype;

typedef enum {
  QSA_OK = 0,
  QSA_ERR_NULL = 1,      /* a required pointer or descriptor is NULL */
  QSA_ERR_DTYPE = 2,     /* wrong dtype code */
  QSA_ERR_SHAPE = 3,     /* wrong rank or extent */
  QSA_ERR_LAYOUT = 4,    /* wrong strides, V offset or alignment */
  QSA_ERR_ALIAS = 5,     /* an output overlaps an input or the workspace */
  QSA_ERR_WORKSPACE = 6, /* workspace missing, too small or misaligned */
  QSA_ERR_ARG = 7,       /* a scalar argument out of range */
  QSA_ERR_LAUNCH = 8     /* the HIP runtime rejected a launch */
} qsa_status;

typedef struct qsa_tensor {
  void* data;        /* device address of element [0,...,0] */
  int32_t dtype;     /* qsa_dtype */
  int32_t ndim;      /* 1..4 */
  int64_t shape[4];  /* extents; entries >= ndim ignored */
  int64_t stride[4]; /* strides in elements; entries >= ndim ignored */
} qsa_tensor;

/* hipStream_t, passed opaquely so this header needs no HIP header. */
typedef void* qsa_stream;

/* Name of a status code (static string). */
QSA_API const char* qsa_status_string(int status);

/* Detail of the last non-OK status returned to the calling thread (static
 * per-thread buffer; "" when there is none). */
QSA_API const char* qsa_last_error(void);

/* The fixed contract constants: 2048, 4, 2051, 512.  NULL outputs skipped. */
QSA_API void qsa_constants(int32_t* token_topk, int32_t* compress_ratio,
                           int32_t* out_width, int32_t* topk_blocks);

/* Workspace bytes qsa_select needs for `rows` query rows and a block table
 * of `table_width` columns, with q given either way ([R,4,128] or
 * [B,n,4,128], see qsa_select).  0 when rows == 0. */
QSA_API size_t qsa_select_workspace_bytes(int64_t rows, int64_t table_width);

/* Workspace bytes qsa_sparse_attn needs for `rows` rows. */
QSA_API size_t qsa_sparse_attn_workspace_bytes(int64_t rows);

/* Workspace bytes qsa_decode_step needs (both stages, one buffer). */
QSA_API size_t qsa_decode_step_workspace_bytes(int64_t rows, int64_t table_width);

/*
 * qsa_select -- fused paged top-512 selection ("Summary": reads paged
 * compressed keys, computes four-head ReLU(Q*K) scores, performs streaming
 * top-512 selection, expands blocks to 2,048 tokens, appends the tail and
 * writes caller-owned [R,2051] int32 output; "Exact contracts", selection).
 *
 *   q            F16 [R,4,128] contiguous: 4 indexer heads per query row;
 *                or F16 [B,n,4,128] contiguous for R = B*n rows that come
 *                in runs of n consecutive rows of one request, as the
 *                paged MQA logits call on the page "[XPU] Enable multiple
 *                key kernels for sparse attention" takes its queries with
 *                next_n positions per request (speculative decode).  Then
 *                up to 4 rows of a run are scored against one read of the
 *                request's keys.  The shape only groups the work: each
 *                row's request and position still come from token_to_req
 *                and query_pos, and a run that spans several requests is
 *                still correct (its requests' keys are read one by one).
 *   kcache       F16 [P,128,1,128] contiguous, P >= 1: compressed keys, 128
 *                per page (vllm qsa_cache.py page: the compressed cache's
 *                block table and slot mapping).
 *   block_table  I32 [N,W], stride[1] == 1, stride[0] >= W: physical page
 *                of logical page j of request n.  Only the first
 *                ceil(V/128) entries of a row are read.
 *   token_to_req I32 [R] (stride 1): request of each query row.
 *   seq_lens     I32 [N] (stride 1): tokens of each request.
 *   query_pos    I64 [R] (stride 1): logical position of each query row
 *                (a decode row has L-1; -1 marks a padded row).
 *   out          I32 [R,2051] contiguous, written.
 *
 * Per row r: V = max(0, min(floor((qp+1)/4), floor(L/4))) visible blocks
 * (qsa_cache.py page, the visible-block rule of _build_qsa_metadata_kernel),
 * T = max(0, min(qp+1, L) - 4V) tail tokens.  Block b's key is
 * kcache[block_table[req][b/128]][b%128][0]; its score is the fp32 sum over
 * the 4 heads of ReLU(q_h . key) with fp32 accumulation.  The first
 * min(512, V) blocks in (score descending, block index ascending) order are
 * written as tokens 4b..4b+3, then the T tail tokens 4V..4V+T-1, then -1.
 */
QSA_API int qsa_select(const qsa_tensor* q, const qsa_tensor* kcache,
                       const qsa_tensor* block_table, const qsa_tensor* token_to_req,
                       const qsa_tensor* seq_lens, const qsa_tensor* query_pos,
                       const qsa_tensor* out, void* workspace, size_t workspace_bytes,
                       qsa_stream stream);

/*
 * qsa_select_fp8 -- qsa_select over an fp8 e4m3 compressed-key cache.  The
 * page "qsa_cache.py" (vllm qwen4_exp, QSAStateBackend) lists fp8 / fp8_e4m3
 * among the compressed indexer cache's dtypes, and the fp8 logits calls on
 * the page "[XPU] Enable multiple key kernels for sparse attention" take the
 * keys as k_quant with a k_scale; neither fixes the scale layout.  Here
 * every compressed key carries one fp32 scale:
 *
 *   kcache   E4M3 [P,128,1,128] contiguous, 16-byte aligned: the codes.
 *   kscale   F32 [P,128] contiguous (same P): the scale of each key.
 *
 * The key scored for block b is the dequantized vector
 * kscale[page][slot] * e4m3(kcache[page][slot][0][d]); everything else --
 * the other arguments, V and T, the order, the output, the workspace
 * (qsa_select_workspace_bytes) and the error behaviour -- is as for
 * qsa_select.  Device-side preconditions in addition: scales finite and
 * >= 0, codes not NaN (0x7F, 0xFF).
 */
QSA_API int qsa_select_fp8(const qsa_tensor* q, const qsa_tensor* kcache,
                           const qsa_tensor* kscale, const qsa_tensor* block_table,
                           const qsa_tensor* token_to_req, const qsa_tensor* seq_lens,
                           const qsa_tensor* query_pos, const qsa_tensor* out, void* workspace,
                           size_t workspace_bytes, qsa_stream stream);

/*
 * qsa_select_weighted -- qsa_select with per-head weights.  The page "[XPU]
 * Enable multiple key kernels for sparse attention" shows the paged MQA
 * logits call taking per-head `weights`; here block b scores
 *
 *   s_b = sum_h weights[r][h] * ReLU(q[r][h] . key_b)
 *
 * (weights of 1 give qsa_select's score).  Weighted scores may be negative;
 * the order is still (score descending, block ascending) with -0 == +0.
 *
 *   weights  F32 [R,4] contiguous, 16-byte aligned, finite.
 *   kscale   NULL: kcache is an F16 cache as for qsa_select; otherwise
 *            kcache is an E4M3 cache and kscale its F32 [P,128] scales, as
 *            for qsa_select_fp8.
 *
 * Everything else (arguments, output, workspace = qsa_select_workspace_bytes,
 * errors) as for qsa_select.
 */
QSA_API int qsa_select_weighted(const qsa_tensor* q, const qsa_tensor* weights,
                                const qsa_tensor* kcache, const qsa_tensor* kscale,
                                const qsa_tensor* block_table, const qsa_tensor* token_to_req,
                                const qsa_tensor* seq_lens, const qsa_tensor* query_pos,
                                const qsa_tensor* out, void* workspace, size_t workspace_bytes,
                                qsa_stream stream);

/*
 * qsa_paged_logits -- the first of the two passes of the same page (paged
 * MQA logits with per-head weights, returned as a logits matrix): the score
 * of every visible block, written as fp32 logits.
 *
 *   q, kcache, block_table, token_to_req, seq_lens, query_pos  as for
 *            qsa_select; weights F32 [R,4] or NULL (all 1); kscale NULL (F16
 *            cache) or the scales of an E4M3 cache, as for
 *            qsa_select_weighted.
 *   logits   F32 [R, Wl], stride[1] == 1, stride[0] >= Wl, 4-byte aligned,
 *            written: logits[r][b] = s_b for b < V, -inf for V <= b < Wl.
 *            Wl >= W * 128 (W = block_table columns), so every visible block
 *            has its column.  Must not overlap any input.
 *
 * No workspace.  Errors as for qsa_select.
 */
QSA_API int qsa_paged_logits(const qsa_tensor* q, const qsa_tensor* weights,
                             const qsa_tensor* kcache, const qsa_tensor* kscale,
                             const qsa_tensor* block_table, const qsa_tensor* token_to_req,
                             const qsa_tensor* seq_lens, const qsa_tensor* query_pos,
                             const qsa_tensor* logits, qsa_stream stream);

/* Workspace bytes qsa_topk_per_row needs for `rows` rows of `logits_width`
 * columns.  0 when rows == 0 or logits_width <= 32768 (such rows are
 * selected one workgroup per row). */
QSA_API size_t qsa_topk_per_row_workspace_bytes(int64_t rows, int64_t logits_width);

/*
 * qsa_topk_per_row -- the second pass (the page's top_k_per_row_decode
 * step): the selection of qsa_select applied to given block scores.
 *
 *   logits       F32 [R, Wl], stride[1] == 1, stride[0] >= Wl, 4-byte
 *                aligned: logits[r][b] is the score of block b of row r.
 *   token_to_req I32 [R], seq_lens I32 [N], query_pos I64 [R]: as for
 *                qsa_select; they give each row's V and T.
 *   out          I32 [R,2051] contiguous, written as by qsa_select.
 *
 * Only the first V logits of a row are read (V <= Wl is a precondition; the
 * kernel reads at most Wl); values must not be NaN.  Workspace:
 * qsa_topk_per_row_workspace_bytes(R, Wl).  Errors as for qsa_select.
 */
QSA_API int qsa_topk_per_row(const qsa_tensor* logits, const qsa_tensor* token_to_req,
                             const qsa_tensor* seq_lens, const qsa_tensor* query_pos,
                             const qsa_tensor* out, void* workspace, size_t workspace_bytes,
                             qsa_stream stream);

/*
 * qsa_sparse_attn -- fp16 sparse decode attention over logical indices with
 * holes and duplicates ("Exact contracts", attention).
 *
 *   q        F16 [R,3,256] contiguous: 3 query heads sharing one K/V head.
 *   k        F16 [NP,512,1,256], strides exactly [262144,512,256,1]: the K
 *            half of a packed KV cache whose token rows are 512 elements,
 *            K = row[0:256].
 *   v        F16, same shape and strides as k, and v->data == k->data + 256
 *            elements (the page's "V storage_offset=256").
 *   indices  I32 [R,2051] contiguous: token t addresses flat row t of the
 *            packed cache (page t/512, row t%512); -1 is a hole.
 *   softmax_scale  finite, > 0 (logits are scale * q.k).
 *   out      F16 [R,3,256] contiguous, written.
 *
 * out[r][h] = sum_j p_j V[idx_j] with p = softmax over the valid positions
 * j of row r of scale * q[r][h].K[idx_j]; every position counts, so a
 * repeated index weighs once per repetition; a row with no valid index
 * yields zeros.  fp32 accumulation, fp16 round-to-nearest-even output.
 */
QSA_API int qsa_sparse_attn(const qsa_tensor* q, const qsa_tensor* k, const qsa_tensor* v,
                            const qsa_tensor* indices, float softmax_scale,
                            const qsa_tensor* out, void* workspace, size_t workspace_bytes,
                            qsa_stream stream);

/*
 * qsa_decode_step -- qsa_select then qsa_sparse_attn on one stream, with the
 * selection output fed to the attention without any host synchronisation
 * ("Summary": no per-row .item()/CPU synchronisation).
 *
 * The selection arguments are as for qsa_select; q_attn, k, v,
 * softmax_scale and out are as for qsa_sparse_attn with the same R.
 * `indices` (I32 [R,2051] contiguous, caller-owned) receives the selection
 * and is read back by the attention.  It is an output and must not overlap
 * any input, `out` or the workspace.
 */
QSA_API int qsa_decode_step(const qsa_tensor* q_sel, const qsa_tensor* kcache,
                            const qsa_tensor* block_table, const qsa_tensor* token_to_req,
                            const qsa_tensor* seq_lens, const qsa_tensor* query_pos,
                            const qsa_tensor* q_attn, const qsa_tensor* k,
                            const qsa_tensor* v, float softmax_scale,
                            const qsa_tensor* indices, const qsa_tensor* out,
                            void* workspace, size_t workspace_bytes, qsa_stream stream);

/*
 * qsa_decode_step_fp8 -- qsa_decode_step with the selection of
 * qsa_select_fp8 (kcache E4M3 codes plus kscale F32 [P,128]).  Workspace:
 * qsa_decode_step_workspace_bytes.
 */
QSA_API int qsa_decode_step_fp8(const qsa_tensor* q_sel, const qsa_tensor* kcache,
                                const qsa_tensor* kscale, const qsa_tensor* block_table,
                                const qsa_tensor* token_to_req, const qsa_tensor* seq_lens,
                                const qsa_tensor* query_pos, const qsa_tensor* q_attn,
                                const qsa_tensor* k, const qsa_tensor* v, float softmax_scale,
                                const qsa_tensor* indices, const qsa_tensor* out, void* workspace,
                                size_t workspace_bytes, qsa_stream stream);

/*
 * qsa_decode_step_noalloc -- qsa_decode_step for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments and results as
 * qsa_decode_step (the caller still passes every input and output), but no
 * workspace: the kernels use a fixed scratch array inside the library,
 * QSA_STATIC_SCRATCH_BYTES (32 MiB) per GPU, which each GPU the library runs
 * on holds from the first call until the process ends.  The call allocates
 * nothing (no hipMalloc, no hipFree, no allocating library routine).
 *
 * Limit: a call whose decode-step workspace (qsa_decode_step_workspace_bytes
 * for the grouping q implies) exceeds QSA_STATIC_SCRATCH_BYTES fails with
 * QSA_ERR_WORKSPACE before anything is launched -- e.g. 128 rows over a
 * 256-page block table need about 6.6 MB and fit.  Every call on one GPU
 * shares that GPU's scratch: calls that may overlap on one GPU (different
 * streams, no ordering between them) race and must not be made; calls in
 * order on one stream are fine (nothing in the scratch needs clearing:
 * every byte read was written earlier in the same call).
 */
#define QSA_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
QSA_API int qsa_decode_step_noalloc(const qsa_tensor* q_sel, const qsa_tensor* kcache,
                                    const qsa_tensor* block_table, const qsa_tensor* token_to_req,
                                    const qsa_tensor* seq_lens, const qsa_tensor* query_pos,
                                    const qsa_tensor* q_attn, const qsa_tensor* k,
                                    const qsa_tensor* v, float softmax_scale,
                                    const qsa_tensor* indices, const qsa_tensor* out,
                                    qsa_stream stream);

/* Workspace bytes qsa_build_metadata needs for num_reqs requests when
 * k_work_metadata is given (0 otherwise). */
QSA_API size_t qsa_build_metadata_workspace_bytes(int64_t num_reqs);

/*
 * qsa_build_metadata -- the per-step metadata of the QSA side caches, as the
 * vllm qsa_cache.py page builds it (_build_qsa_metadata_kernel and its torch
 * fallback), on the device with no host synchronisation.  Its token_to_req
 * and logical_positions are the token_to_req and query_pos inputs of the
 * selection entry points.
 *
 *   query_start_loc   I32 [N+1], N >= 1: query tokens of request r are
 *                     [query_start_loc[r], query_start_loc[r+1]); tokens at
 *                     or past query_start_loc[N] are padding.
 *   seq_lens          I32 [N]: tokens of each request (>= its query length).
 *   block_table       I32 [N, W], stride[1] == 1: the side cache's blocks.
 *   common_slot_mapping  I64 [T] or NULL: the main cache's slots (< 0: the
 *                     token writes no slot; NULL: every token writes one).
 *   storage_block_size   compressed slots per block (>= 1).
 *   compress_ratio    tokens per compressed key (>= 1).
 *   circular_buffer_size 0, or the raw-key ring size (> 0 selects the ring
 *                     owner's slots).
 *   token_to_req      I32 [T] (T >= 0 tokens), written: the last request
 *                     whose query starts at or before the token; 0 for
 *                     padding.
 *   logical_positions I64 [T], written: seq_len - query_len + offset inside
 *                     the query; -1 for padding.
 *   visible_blocks    I32 [T], written: max(0, min(floor((pos+1)/ratio),
 *                     floor(seq_len/ratio))).
 *   slot_mapping      I64 [T] or NULL, written: with a ring, a request's
 *                     last ring-size tokens write block_table[r][0] * ring +
 *                     pos mod ring; else with ratio > 1 the token that
 *                     completes a group writes block_table[r][c / B] * B +
 *                     c mod B for compressed position c = pos / ratio (if
 *                     that column exists, holds a block >= 0 and the common
 *                     slot is >= 0); else the common slot.  -1 elsewhere.
 *   k_work_metadata   I32 [M, 2] or NULL, written: per request with a
 *                     nonempty query max(floor(L/ratio) - floor((L-q)/ratio),
 *                     1) items, laid out request after request as (request,
 *                     index inside the request); (-1, -1) past the last item.
 *
 * Outputs must not overlap each other, any input or the workspace
 * (qsa_build_metadata_workspace_bytes(N) bytes when k_work_metadata is
 * given).  Device-side preconditions: query_start_loc[0] = 0 and
 * nondecreasing; seq_lens >= query lengths.  Errors as for qsa_select
 * (QSA_ERR_ARG for a size or ratio out of range).
 */
QSA_API int qsa_build_metadata(const qsa_tensor* query_start_loc, const qsa_tensor* seq_lens,
                               const qsa_tensor* block_table,
                               const qsa_tensor* common_slot_mapping,
                               int64_t storage_block_size, int64_t compress_ratio,
                               int64_t circular_buffer_size, const qsa_tensor* token_to_req,
                               const qsa_tensor* logical_positions,
                               const qsa_tensor* visible_blocks, const qsa_tensor* slot_mapping,
                               const qsa_tensor* k_work_metadata, void* workspace,
                               size_t workspace_bytes, qsa_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H_ */
