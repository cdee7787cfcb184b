/*
 * qsa_oracle.c -- plain, slow, single-threaded CPU oracle for the QSA
 * sparse-attention decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * bench's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP path and never calls into it.
 *
 * What it computes (intel/llm-scaler PR #651, "vLLM: integrate FP16 packed
 * QSA extension", sections "Summary" and "Exact contracts"):
 *
 *   selection, per query row r
 *     req  = token_to_req[r], L = seq_lens[req], qp = query_pos[r]
 *     V    = max(0, min(floor((qp+1)/4), floor(L/4)))       visible blocks
 *            (vllm qsa_cache.py page, _build_qsa_metadata_kernel and its
 *             torch fallback: the visible-block rule)
 *     T    = max(0, min(qp+1, L) - 4V)                       tail tokens
 *     key of block b = kcache[bt[req][b / 128]][b % 128][0][:]
 *            (qsa_cache.py page, compressed_qsa_slot_mapping: the
 *             compressed position b lives in logical page b / 128 at slot
 *             b % 128)
 *     score s_b = sum over the 4 indexer heads h of ReLU(q[r][h] . key_b)
 *     order all V blocks by score descending, ties by ascending block
 *     index; keep the first n = min(512, V)
 *     out[r][4i+j] = 4*b_i + j (i < n, j < 4), then the tail tokens
 *     4V .. 4V+T-1, then -1 up to width 2051.
 *
 *   attention, per row r and query head h in {0,1,2}
 *     J = positions j of indices[r] with indices[r][j] >= 0 (a multiset:
 *         a repeated index is a separate member)
 *     l_j = scale * sum_d q[r][h][d] * K[idx_j][d]      (K = kv[t][0:256])
 *     o[r][h][:] = sum_j softmax(l)_j * V[idx_j][:]      (V = kv[t][256:512])
 *     an empty J gives o = 0.
 *
 *   fp8 key cache (the vllm qsa_cache.py page lists fp8 / fp8_e4m3 among
 *   the compressed indexer cache's dtypes; the "[XPU] Enable multiple key
 *   kernels for sparse attention" page's fp8 logits calls take the keys as
 *   k_quant with a k_scale): each compressed key is 128 e4m3 codes plus one
 *   binary32 scale, and the key used for scoring is the dequantized vector
 *   scale * e4m3(code[d]); everything else is as above.
 *
 *   per-head weights and the two-pass form (the "[XPU] Enable multiple key
 *   kernels for sparse attention" page: the paged MQA logits call takes
 *   per-head weights and returns a logits matrix, which top_k_per_row_decode
 *   then reduces): score s_b = sum_h w[r][h] * ReLU(q[r][h] . key_b) with
 *   fp32 weights (w = 1 is the unweighted score above); paged logits =
 *   the matrix of s_b for b < V and -inf for V <= b < width; top-k per row
 *   = the selection above applied to a given logits row, reading its first V
 *   entries only.
 *
 *   metadata (the vllm qsa_cache.py page, _build_qsa_metadata_kernel and
 *   its torch fallback): from cumulative query starts and sequence lengths,
 *   per token its request (the last request whose query starts at or
 *   before it), its logical position, its visible blocks, its slot in the
 *   compressed cache (or in the raw-key ring), and the per-request k work
 *   items, laid out request after request.
 *
 * Precision: fp16 inputs are widened to double with a conversion written
 * from the IEEE 754 binary16 definition; every dot product and softmax is
 * evaluated in double.  A selection score is rounded once to binary32 at
 * the end, so that both sides of a comparison decide ties in binary32.
 *
 * Sorting uses the C library's qsort as the one library primitive.
 *
 * Compile-time switch QSA_ORACLE_MUTANT (default 0) plants a single known
 * mistake; it exists only so that the pin tests can show they would catch
 * that mistake.  The oracle the tests trust is built without it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef QSA_ORACLE_MUTANT
#define QSA_ORACLE_MUTANT 0
#endif

/* Fixed contract of the pages ("Exact contracts", selection): 2048 tokens
 * from 512 blocks of 4, plus up to three tail tokens. */
#define OR_TOKEN_TOPK 2048
#define OR_RATIO 4
#define OR_TOPK_BLOCKS (OR_TOKEN_TOPK / OR_RATIO)
#define OR_WIDTH 2051
#define OR_PAGE_SLOTS 128
#define OR_SEL_HEADS 4
#define OR_SEL_DIM 128
#define OR_ATT_HEADS 3
#define OR_ATT_DIM 256
#define OR_KV_ROW 512

enum {
  OR_OK = 0,
  OR_ERR_REQ = -1,      /* token_to_req outside [0, N) */
  OR_ERR_TABLE = -2,    /* a visible block lies beyond the block table */
  OR_ERR_PAGE = -3,     /* a needed page id outside [0, P) */
  OR_ERR_INDEX = -4,    /* an attention index outside [-1, NT) */
  OR_ERR_NOMEM = -5,
  OR_ERR_ARG = -6
};

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Exponent 0 encodes subnormals (fraction * 2^-24); exponent 31
 * encodes infinities and NaNs. */
double qsa_oracle_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 31;
  int frac = h & 1023;
  double v;
  if (expo == 0) {
    v = ldexp((double)frac, -24);
  } else if (expo == 31) {
    v = frac ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + frac), expo - 25);
  }
  return sign ? -v : v;
}

/* OCP 8-bit floating point, E4M3 variant without infinities ("e4m3fn"):
 * 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits.  Exponent 0
 * encodes subnormals (fraction * 2^-9); the all-ones pattern S.1111.111 is
 * NaN and every other pattern is finite (largest 448). */
double qsa_oracle_e4m3_to_double(uint8_t c) {
  int sign = (c >> 7) & 1;
  int expo = (c >> 3) & 15;
  int frac = c & 7;
  double v;
  if (expo == 15 && frac == 7) {
    v = NAN;
  } else if (expo == 0) {
#if QSA_ORACLE_MUTANT == 13
    v = ldexp((double)(8 + frac), -9); /* planted: subnormal read as normal */
#else
    v = ldexp((double)frac, -9);
#endif
  } else {
#if QSA_ORACLE_MUTANT == 12
    v = ldexp((double)(8 + frac), expo - 11); /* planted: exponent bias 8 */
#else
    v = ldexp((double)(8 + frac), expo - 10);
#endif
  }
  return sign ? -v : v;
}

/* Visible blocks and tail length of one query row. */
void qsa_oracle_row_extent(int64_t seq_len, int64_t query_pos, int64_t* visible,
                           int64_t* tail) {
  int64_t upto = query_pos + 1; /* tokens up to and including the query */
#if QSA_ORACLE_MUTANT == 8
  upto = query_pos; /* planted: off by one in the visible-block rule */
#endif
  int64_t a = upto >= 0 ? upto / OR_RATIO : -1;
  int64_t b = seq_len >= 0 ? seq_len / OR_RATIO : -1;
  int64_t v = a < b ? a : b;
  if (v < 0) v = 0;
  int64_t end = upto < seq_len ? upto : seq_len;
  int64_t t = end - OR_RATIO * v;
  if (t < 0) t = 0;
#if QSA_ORACLE_MUTANT == 4
  t = 0; /* planted: tail omitted */
#endif
  *visible = v;
  *tail = t;
}

typedef struct {
  float score;
  int64_t block;
} scored_block;

/* Score descending; equal scores by ascending block index. */
static int by_score_then_index(const void* pa, const void* pb) {
  const scored_block* a = (const scored_block*)pa;
  const scored_block* b = (const scored_block*)pb;
#if QSA_ORACLE_MUTANT == 10
  if (a->score < b->score) return -1; /* planted: ascending score */
  if (a->score > b->score) return 1;
#else
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
#endif
#if QSA_ORACLE_MUTANT == 1
  if (a->block > b->block) return -1; /* planted: ties by descending index */
  if (a->block < b->block) return 1;
#else
  if (a->block < b->block) return -1;
  if (a->block > b->block) return 1;
#endif
  return 0;
}

/* The row's four query heads widened to double. */
static void widen_query(const uint16_t* q_row, double* qd) {
  for (int i = 0; i < OR_SEL_HEADS * OR_SEL_DIM; ++i) qd[i] = qsa_oracle_half_to_double(q_row[i]);
}

/* The compressed key cache: binary16 keys, or e4m3 codes with one binary32
 * scale per key.  Both are [P,128,1,128] in elements; scales are [P,128]. */
typedef struct {
  const uint16_t* f16;
  const uint8_t* codes;
  const float* scales;
} key_cache;

/* Key number `slot_index` (= page * 128 + slot) widened to double: the
 * binary16 values, or scale * e4m3(code) per element. */
static void widen_key(const key_cache* kc, int64_t slot_index, double* kd) {
  if (kc->f16) {
    const uint16_t* key = kc->f16 + slot_index * OR_SEL_DIM;
    for (int d = 0; d < OR_SEL_DIM; ++d) kd[d] = qsa_oracle_half_to_double(key[d]);
    return;
  }
  const uint8_t* code = kc->codes + slot_index * OR_SEL_DIM;
  double scale = (double)kc->scales[slot_index];
#if QSA_ORACLE_MUTANT == 11
  scale = 1.0; /* planted: per-key scale ignored */
#endif
  for (int d = 0; d < OR_SEL_DIM; ++d) kd[d] = scale * qsa_oracle_e4m3_to_double(code[d]);
}

/* Score of one compressed key (kd, widened) against the row's four indexer
 * heads (qd: the row's query widened to double, [4][128]), each head's ReLU
 * term weighted by w[h] (w NULL: every weight 1). */
static float block_score(const double* qd, const double* kd, const float* w) {
  double total = 0.0;
  int heads = OR_SEL_HEADS;
#if QSA_ORACLE_MUTANT == 5
  heads = 3; /* planted: one head dropped */
#endif
  for (int h = 0; h < heads; ++h) {
    double dot = 0.0;
    for (int d = 0; d < OR_SEL_DIM; ++d) {
      dot += qd[h * OR_SEL_DIM + d] * kd[d];
    }
    double wh = w ? (double)w[h] : 1.0;
#if QSA_ORACLE_MUTANT == 14
    wh = 1.0; /* planted: head weights ignored */
#endif
#if QSA_ORACLE_MUTANT == 2
    total += wh * dot; /* planted: ReLU dropped */
#elif QSA_ORACLE_MUTANT == 15
    total += wh * dot > 0.0 ? wh * dot : 0.0; /* planted: ReLU after the weight */
#else
    total += wh * (dot > 0.0 ? dot : 0.0);
#endif
  }
  return (float)total;
}

/* Cache slot (page * 128 + slot) of compressed key b of a request, or -1
 * with *err set when the block table or the page id cannot serve it. */
static int64_t key_slot(int64_t num_pages, const int32_t* table_row, int64_t table_width,
                        int64_t b, int* err) {
  int64_t logical_page = b / OR_PAGE_SLOTS;
  int64_t slot = b % OR_PAGE_SLOTS;
#if QSA_ORACLE_MUTANT == 3
  logical_page = b % OR_PAGE_SLOTS; /* planted: page and slot transposed */
  slot = b / OR_PAGE_SLOTS;
  if (logical_page >= table_width) logical_page = table_width - 1;
#endif
  if (logical_page >= table_width) {
    *err = OR_ERR_TABLE;
    return -1;
  }
  int64_t page = table_row[logical_page];
  if (page < 0 || page >= num_pages) {
    *err = OR_ERR_PAGE;
    return -1;
  }
  return page * OR_PAGE_SLOTS + slot;
}

static int row_scores(int64_t r, int64_t num_pages, int64_t num_reqs, int64_t table_width,
                      const uint16_t* q, const float* weights, const key_cache* kc,
                      const int32_t* block_table, const int32_t* token_to_req,
                      const int32_t* seq_lens, const int64_t* query_pos, float* scores,
                      int64_t max_blocks, int64_t* visible) {
  int64_t req = token_to_req[r];
  if (req < 0 || req >= num_reqs) return OR_ERR_REQ;
  int64_t v, t;
  qsa_oracle_row_extent(seq_lens[req], query_pos[r], &v, &t);
  *visible = v;
  if (v > max_blocks) return OR_ERR_ARG;
  double qd[OR_SEL_HEADS * OR_SEL_DIM];
  widen_query(q + r * OR_SEL_HEADS * OR_SEL_DIM, qd);
  const int32_t* table_row = block_table + req * table_width;
  double kd[OR_SEL_DIM];
  for (int64_t b = 0; b < v; ++b) {
    int err = OR_OK;
    int64_t at = key_slot(num_pages, table_row, table_width, b, &err);
    if (at < 0) return err;
    widen_key(kc, at, kd);
    scores[b] = block_score(qd, kd, weights ? weights + r * OR_SEL_HEADS : NULL);
  }
  return OR_OK;
}

/*
 * Scores of every visible block of one row, in block order.  scores must
 * hold max_blocks floats; *visible receives V.  Returns OR_OK or an error.
 */
int qsa_oracle_row_scores(int64_t r, int64_t num_pages, int64_t num_reqs,
                          int64_t table_width, const uint16_t* q,
                          const uint16_t* kcache, const int32_t* block_table,
                          const int32_t* token_to_req, const int32_t* seq_lens,
                          const int64_t* query_pos, float* scores,
                          int64_t max_blocks, int64_t* visible) {
  key_cache kc = {kcache, NULL, NULL};
  return row_scores(r, num_pages, num_reqs, table_width, q, NULL, &kc, block_table, token_to_req,
                    seq_lens, query_pos, scores, max_blocks, visible);
}

/* As qsa_oracle_row_scores, for an e4m3 cache: codes [P,128,1,128] bytes,
 * scales [P,128] binary32. */
int qsa_oracle_row_scores_fp8(int64_t r, int64_t num_pages, int64_t num_reqs,
                              int64_t table_width, const uint16_t* q, const uint8_t* codes,
                              const float* scales, const int32_t* block_table,
                              const int32_t* token_to_req, const int32_t* seq_lens,
                              const int64_t* query_pos, float* scores, int64_t max_blocks,
                              int64_t* visible) {
  key_cache kc = {NULL, codes, scales};
  return row_scores(r, num_pages, num_reqs, table_width, q, NULL, &kc, block_table, token_to_req,
                    seq_lens, query_pos, scores, max_blocks, visible);
}

/* Fill one output row from its V blocks already sorted by (score desc,
 * block asc): the first min(512, V) blocks expanded to 4 tokens each, then
 * the T tail tokens, then -1. */
static void write_row(int32_t* out_row, const scored_block* sorted, int64_t v, int64_t t) {
  for (int i = 0; i < OR_WIDTH; ++i) out_row[i] = -1;
  int64_t n = v < OR_TOPK_BLOCKS ? v : OR_TOPK_BLOCKS;
  for (int64_t i = 0; i < n; ++i) {
    for (int j = 0; j < OR_RATIO; ++j) {
      out_row[OR_RATIO * i + j] = (int32_t)(OR_RATIO * sorted[i].block + j);
    }
  }
  for (int64_t k = 0; k < t; ++k) out_row[OR_RATIO * n + k] = (int32_t)(OR_RATIO * v + k);
}

static int select_rows(int64_t R, int64_t num_pages, int64_t num_reqs, int64_t table_width,
                       const uint16_t* q, const float* weights, const key_cache* kc,
                       const int32_t* block_table, const int32_t* token_to_req,
                       const int32_t* seq_lens, const int64_t* query_pos, int32_t* out) {
  for (int64_t r = 0; r < R; ++r) {
    int32_t* out_row = out + r * OR_WIDTH;
    for (int i = 0; i < OR_WIDTH; ++i) out_row[i] = -1;
    int64_t req = token_to_req[r];
    if (req < 0 || req >= num_reqs) return OR_ERR_REQ;
    int64_t v, t;
    qsa_oracle_row_extent(seq_lens[req], query_pos[r], &v, &t);
    scored_block* all = NULL;
    if (v > 0) {
      all = (scored_block*)malloc((size_t)v * sizeof(scored_block));
      if (!all) return OR_ERR_NOMEM;
    }
    double qd[OR_SEL_HEADS * OR_SEL_DIM];
    widen_query(q + r * OR_SEL_HEADS * OR_SEL_DIM, qd);
    const int32_t* table_row = block_table + req * table_width;
    double kd[OR_SEL_DIM];
    for (int64_t b = 0; b < v; ++b) {
      int err = OR_OK;
      int64_t at = key_slot(num_pages, table_row, table_width, b, &err);
      if (at < 0) {
        free(all);
        return err;
      }
      widen_key(kc, at, kd);
      all[b].score = block_score(qd, kd, weights ? weights + r * OR_SEL_HEADS : NULL);
      all[b].block = b;
    }
    if (v > 1) qsort(all, (size_t)v, sizeof(scored_block), by_score_then_index);
    write_row(out_row, all, v, t);
    free(all);
  }
  return OR_OK;
}

/*
 * Selection for rows [0, R).  Shapes: q [R,4,128] fp16 bits,
 * kcache [P,128,1,128] fp16 bits, block_table [N,W] int32,
 * token_to_req [R] int32, seq_lens [N] int32, query_pos [R] int64,
 * out [R,2051] int32 (written).  Returns OR_OK or the first error.
 */
int qsa_oracle_select(int64_t R, int64_t num_pages, int64_t num_reqs,
                      int64_t table_width, const uint16_t* q, const uint16_t* kcache,
                      const int32_t* block_table, const int32_t* token_to_req,
                      const int32_t* seq_lens, const int64_t* query_pos,
                      int32_t* out) {
  key_cache kc = {kcache, NULL, NULL};
  return select_rows(R, num_pages, num_reqs, table_width, q, NULL, &kc, block_table,
                     token_to_req, seq_lens, query_pos, out);
}

/* As qsa_oracle_select, for an e4m3 cache: codes [P,128,1,128] bytes,
 * scales [P,128] binary32. */
int qsa_oracle_select_fp8(int64_t R, int64_t num_pages, int64_t num_reqs,
                          int64_t table_width, const uint16_t* q, const uint8_t* codes,
                          const float* scales, const int32_t* block_table,
                          const int32_t* token_to_req, const int32_t* seq_lens,
                          const int64_t* query_pos, int32_t* out) {
  key_cache kc = {NULL, codes, scales};
  return select_rows(R, num_pages, num_reqs, table_width, q, NULL, &kc, block_table,
                     token_to_req, seq_lens, query_pos, out);
}

/* Weighted selection: weights [R,4] binary32; the key cache is binary16
 * (kcache) when codes is NULL, else e4m3 codes with scales. */
int qsa_oracle_select_weighted(int64_t R, int64_t num_pages, int64_t num_reqs,
                               int64_t table_width, const uint16_t* q, const float* weights,
                               const uint16_t* kcache, const uint8_t* codes,
                               const float* scales, const int32_t* block_table,
                               const int32_t* token_to_req, const int32_t* seq_lens,
                               const int64_t* query_pos, int32_t* out) {
  key_cache kc = {codes ? NULL : kcache, codes, scales};
  return select_rows(R, num_pages, num_reqs, table_width, q, weights, &kc, block_table,
                     token_to_req, seq_lens, query_pos, out);
}

/*
 * Paged logits: logits[r][b] (row stride `stride` floats) = the score of
 * block b for b < V, -inf for V <= b < width.  weights may be NULL (all 1);
 * key cache as for qsa_oracle_select_weighted.  V > width is an error.
 */
int qsa_oracle_paged_logits(int64_t R, int64_t num_pages, int64_t num_reqs, int64_t table_width,
                            const uint16_t* q, const float* weights, const uint16_t* kcache,
                            const uint8_t* codes, const float* scales,
                            const int32_t* block_table, const int32_t* token_to_req,
                            const int32_t* seq_lens, const int64_t* query_pos, float* logits,
                            int64_t width, int64_t stride) {
  key_cache kc = {codes ? NULL : kcache, codes, scales};
  for (int64_t r = 0; r < R; ++r) {
    float* row = logits + r * stride;
    int64_t v = 0;
    int rc = row_scores(r, num_pages, num_reqs, table_width, q, weights, &kc, block_table,
                        token_to_req, seq_lens, query_pos, row, width, &v);
    if (rc != OR_OK) return rc;
    for (int64_t b = v; b < width; ++b) row[b] = -INFINITY;
  }
  return OR_OK;
}

/*
 * Top-k per row over given logits (row stride `stride` floats, `width`
 * columns): for each query row, V and T from its request and position as in
 * the selection; the first V logits are the block scores; they are ordered
 * by (score descending, block ascending) and written exactly as the
 * selection writes its output.  Entries at or past V are never read.
 */
int qsa_oracle_topk_per_row(int64_t R, int64_t num_reqs, const float* logits, int64_t width,
                            int64_t stride, const int32_t* token_to_req,
                            const int32_t* seq_lens, const int64_t* query_pos, int32_t* out) {
  for (int64_t r = 0; r < R; ++r) {
    int64_t req = token_to_req[r];
    if (req < 0 || req >= num_reqs) return OR_ERR_REQ;
    int64_t v, t;
    qsa_oracle_row_extent(seq_lens[req], query_pos[r], &v, &t);
#if QSA_ORACLE_MUTANT == 16
    v = width; /* planted: the whole logits row read */
#endif
    if (v > width) return OR_ERR_ARG;
    scored_block* all = NULL;
    if (v > 0) {
      all = (scored_block*)malloc((size_t)v * sizeof(scored_block));
      if (!all) return OR_ERR_NOMEM;
    }
    for (int64_t b = 0; b < v; ++b) {
      all[b].score = logits[r * stride + b];
      all[b].block = b;
    }
    if (v > 1) qsort(all, (size_t)v, sizeof(scored_block), by_score_then_index);
    write_row(out + r * OR_WIDTH, all, v, t);
    free(all);
  }
  return OR_OK;
}

/*
 * Sparse attention for rows [0, R).  q [R,3,256] fp16 bits, kv [NT,512]
 * fp16 bits (token t: K = kv[t][0:256], V = kv[t][256:512]),
 * indices [R,2051] int32, out [R,3,256] double (written).
 */
int qsa_oracle_sparse_attn(int64_t R, int64_t num_tokens, const uint16_t* q,
                           const uint16_t* kv, const int32_t* indices, double scale,
                           double* out) {
  double* logit = (double*)malloc(OR_WIDTH * sizeof(double));
  double* kq = (double*)malloc(OR_ATT_DIM * sizeof(double));
  if (!logit || !kq) {
    free(logit);
    free(kq);
    return OR_ERR_NOMEM;
  }
  int rc = OR_OK;
  for (int64_t r = 0; r < R && rc == OR_OK; ++r) {
    const int32_t* idx = indices + r * OR_WIDTH;
    for (int j = 0; j < OR_WIDTH; ++j) {
      if (idx[j] < -1 || idx[j] >= num_tokens) rc = OR_ERR_INDEX;
    }
    if (rc != OR_OK) break;
    for (int h = 0; h < OR_ATT_HEADS; ++h) {
      const uint16_t* qh = q + (r * OR_ATT_HEADS + h) * OR_ATT_DIM;
      double* o = out + (r * OR_ATT_HEADS + h) * OR_ATT_DIM;
      for (int d = 0; d < OR_ATT_DIM; ++d) {
        kq[d] = qsa_oracle_half_to_double(qh[d]);
        o[d] = 0.0;
      }
      /* logits of the members of J, and their maximum */
      int members = 0;
      double m = -INFINITY;
      for (int j = 0; j < OR_WIDTH; ++j) {
        int64_t t = idx[j];
#if QSA_ORACLE_MUTANT == 9
        if (t < 0) t = 0; /* planted: a hole read as token 0 */
#endif
        if (t < 0) continue;
#if QSA_ORACLE_MUTANT == 7
        int seen = 0; /* planted: a repeated index counted once */
        for (int j2 = 0; j2 < j; ++j2) seen |= (idx[j2] == idx[j]);
        if (seen) {
          logit[j] = -INFINITY;
          continue;
        }
#endif
        const uint16_t* krow = kv + t * OR_KV_ROW;
        double dot = 0.0;
        for (int d = 0; d < OR_ATT_DIM; ++d) {
          dot += kq[d] * qsa_oracle_half_to_double(krow[d]);
        }
#if QSA_ORACLE_MUTANT == 6
        logit[j] = dot; /* planted: softmax scale dropped */
        (void)scale;
#else
        logit[j] = scale * dot;
#endif
        if (logit[j] > m) m = logit[j];
        ++members;
      }
      if (members == 0) continue; /* empty J: output stays zero */
      /* softmax weights relative to the maximum, then the weighted V sum */
      double z = 0.0;
      for (int j = 0; j < OR_WIDTH; ++j) {
        int64_t t = idx[j];
#if QSA_ORACLE_MUTANT == 9
        if (t < 0) t = 0;
#endif
        if (t < 0 || logit[j] == -INFINITY) continue;
        double w = exp(logit[j] - m);
        z += w;
        const uint16_t* vrow = kv + t * OR_KV_ROW + OR_ATT_DIM;
        for (int e = 0; e < OR_ATT_DIM; ++e) {
          o[e] += w * qsa_oracle_half_to_double(vrow[e]);
        }
      }
      for (int e = 0; e < OR_ATT_DIM; ++e) o[e] /= z;
    }
  }
  free(logit);
  free(kq);
  return rc;
}

/* floor(a / b) for b > 0 (C division truncates toward zero). */
static int64_t floor_div(int64_t a, int64_t b) {
  int64_t q = a / b;
  if ((a % b != 0) && (a < 0)) q -= 1;
  return q;
}

/*
 * QSA metadata for num_tokens tokens of num_reqs requests.
 *
 *   query_start_loc [N+1] int32: query tokens of request r are
 *       [query_start_loc[r], query_start_loc[r+1]); mapped tokens are those
 *       below query_start_loc[N], the rest are padding.
 *   seq_lens [N] int32; block_table [N][table_width] int32 with row stride
 *   table_stride; common_slot_mapping [num_tokens] int64 or NULL (all >= 0).
 *   storage_block_size: compressed slots per cache block; compress_ratio;
 *   circular_buffer_size: > 0 selects the raw-key ring owner.
 *
 * Outputs per token: token_to_req (0 for padding), logical_positions (-1
 * for padding), visible_blocks, slot_mapping (NULL: not written; -1 where
 * the token writes no slot); k_work [max_num_work][2] (NULL: not written):
 * (request, index of the item inside the request), -1 past the last item.
 */
int qsa_oracle_build_metadata(int64_t num_reqs, int64_t num_tokens,
                              const int32_t* query_start_loc, const int32_t* seq_lens,
                              const int64_t* common_slot_mapping, const int32_t* block_table,
                              int64_t table_width, int64_t table_stride,
                              int64_t storage_block_size, int64_t compress_ratio,
                              int64_t circular_buffer_size, int32_t* token_to_req,
                              int64_t* logical_positions, int32_t* visible_blocks,
                              int64_t* slot_mapping, int32_t* k_work, int64_t max_num_work) {
  if (num_reqs < 1 || storage_block_size < 1 || compress_ratio < 1 || circular_buffer_size < 0) {
    return OR_ERR_ARG;
  }
  const int64_t num_mapped = query_start_loc[num_reqs];
  for (int64_t t = 0; t < num_tokens; ++t) {
    const int mapped = t < num_mapped;
    int64_t r = 0;
    int64_t lp = -1;
    int64_t seq = 0;
    if (mapped) {
      /* the last request whose query starts at or before t */
      for (int64_t c = 0; c < num_reqs; ++c) {
#if QSA_ORACLE_MUTANT == 17
        if (query_start_loc[c] < t) r = c; /* planted: a request's first token given to the one before */
#else
        if (query_start_loc[c] <= t) r = c;
#endif
      }
      const int64_t start = query_start_loc[r];
      const int64_t qlen = (int64_t)query_start_loc[r + 1] - start;
      seq = seq_lens[r];
      lp = seq - qlen + (t - start);
#if QSA_ORACLE_MUTANT == 18
      lp = seq + (t - start) - 1; /* planted: positions counted from the end of the sequence */
#endif
    }
    token_to_req[t] = (int32_t)r;
    logical_positions[t] = lp;
    int64_t v = floor_div(lp + 1, compress_ratio);
    const int64_t cap = floor_div(seq, compress_ratio);
    if (cap < v) v = cap;
    if (v < 0) v = 0;
    visible_blocks[t] = (int32_t)v;
    if (!slot_mapping) continue;
    int64_t slot = -1;
    if (circular_buffer_size > 0) {
      /* raw-key ring: a request's last circular_buffer_size query tokens
       * write slot (position mod ring size) of its first block */
      if (mapped && lp >= 0 && t + circular_buffer_size >= query_start_loc[r + 1] &&
          table_width > 0) {
        const int64_t phys = block_table[r * table_stride];
        if (phys >= 0) slot = phys * circular_buffer_size + lp % circular_buffer_size;
      }
    } else if (compress_ratio != 1) {
      /* compressed cache: the token that completes a group of compress_ratio
       * tokens writes compressed position lp / compress_ratio */
      const int64_t cp = (lp > 0 ? lp : 0) / compress_ratio;
      const int64_t lb = cp / storage_block_size;
#if QSA_ORACLE_MUTANT == 19
      int ok = mapped && lp >= 0 && lp % compress_ratio == 0 && lb < table_width; /* planted: group start */
#else
      int ok = mapped && lp >= 0 && (lp + 1) % compress_ratio == 0 && lb < table_width;
#endif
      if (ok) {
        const int64_t phys = block_table[r * table_stride + lb];
        ok = phys >= 0 && (!common_slot_mapping || common_slot_mapping[t] >= 0);
        if (ok) slot = phys * storage_block_size + cp % storage_block_size;
      }
    } else {
      /* no compression and no ring: the main cache's own slots */
      slot = common_slot_mapping ? common_slot_mapping[t] : -1;
    }
    slot_mapping[t] = slot;
  }
  if (k_work) {
    int64_t w = 0;
    for (int64_t r = 0; r < num_reqs; ++r) {
      const int64_t qlen = (int64_t)query_start_loc[r + 1] - query_start_loc[r];
      const int64_t chunk_start = (int64_t)seq_lens[r] - qlen;
      int64_t groups = floor_div(seq_lens[r], compress_ratio) - floor_div(chunk_start, compress_ratio);
#if QSA_ORACLE_MUTANT != 20
      if (groups < 1) groups = 1; /* the first item also commits the raw suffix */
#else
      if (groups < 0) groups = 0; /* planted: no item without a completed group */
#endif
      const int64_t count = qlen > 0 ? groups : 0;
      for (int64_t i = 0; i < count && w < max_num_work; ++i, ++w) {
        k_work[2 * w] = (int32_t)r;
        k_work[2 * w + 1] = (int32_t)i;
      }
    }
    for (; w < max_num_work; ++w) {
      k_work[2 * w] = -1;
      k_work[2 * w + 1] = -1;
    }
  }
  return OR_OK;
}

/* Which mistake this build carries (0 = none). */
int qsa_oracle_mutant(void) { return QSA_ORACLE_MUTANT; }
