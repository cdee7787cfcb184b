// qsa_capi.cpp -- the C ABI declared in include/qsa.h: fail-closed argument
// validation, launch planning and dispatch.  Plain host C++: no HIP header,
// no device code; every check runs before anything is enqueued.
//
// The checks follow the contracts of the page "vLLM: integrate FP16 packed
// QSA extension" ("Exact contracts": dtypes, shapes, the exact-packed K/V
// strides [262144,512,256,1] and V storage offset 256, caller-owned
// outputs, unchanged inputs; "Validation": fail-closed dtype/layout/output
// checks).
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/qsa.h"
#include "qsa_launch.h"

static_assert(QSA_STATIC_SCRATCH_BYTES == qsa::kStaticScratchBytes,
              "the header states the fixed scratch's size");

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int64_t elem_size(int32_t dtype) {
  switch (dtype) {
    case QSA_DTYPE_F16: return 2;
    case QSA_DTYPE_I32: return 4;
    case QSA_DTYPE_I64: return 8;
    case QSA_DTYPE_F32: return 4;
    case QSA_DTYPE_E4M3: return 1;
    default: return 0;
  }
}

const char* dtype_name(int32_t dtype) {
  switch (dtype) {
    case QSA_DTYPE_F16: return "f16";
    case QSA_DTYPE_I32: return "i32";
    case QSA_DTYPE_I64: return "i64";
    case QSA_DTYPE_F32: return "f32";
    case QSA_DTYPE_E4M3: return "e4m3";
    default: return "unknown";
  }
}

// Byte range [lo, hi) a tensor can touch (empty when any extent is 0).
struct Span {
  uintptr_t lo = 0, hi = 0;
};

Span span_of(const qsa_tensor* t) {
  Span s;
  int64_t last = 0;
  for (int d = 0; d < t->ndim; ++d) {
    if (t->shape[d] == 0) return s;
    last += (t->shape[d] - 1) * t->stride[d];
  }
  s.lo = reinterpret_cast<uintptr_t>(t->data);
  s.hi = s.lo + static_cast<uintptr_t>((last + 1) * elem_size(t->dtype));
  return s;
}

bool overlaps(Span a, Span b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

// Checks dtype, rank and (when want[d] >= 0) each extent.
int check_tensor(const char* name, const qsa_tensor* t, int32_t dtype, int ndim,
                 const int64_t* want) {
  if (!t) return fail(QSA_ERR_NULL, "%s: descriptor is NULL", name);
  if (t->dtype != dtype) {
    return fail(QSA_ERR_DTYPE, "%s: dtype %s (code %d), expected %s", name, dtype_name(t->dtype),
                (int)t->dtype, dtype_name(dtype));
  }
  if (t->ndim != ndim) return fail(QSA_ERR_SHAPE, "%s: rank %d, expected %d", name, (int)t->ndim, ndim);
  for (int d = 0; d < ndim; ++d) {
    if (t->shape[d] < 0) return fail(QSA_ERR_SHAPE, "%s: negative extent in dim %d", name, d);
    if (want[d] >= 0 && t->shape[d] != want[d]) {
      return fail(QSA_ERR_SHAPE, "%s: dim %d is %lld, expected %lld", name, d,
                  (long long)t->shape[d], (long long)want[d]);
    }
  }
  int64_t numel = 1;
  for (int d = 0; d < ndim; ++d) numel *= t->shape[d];
  if (numel > 0 && !t->data) return fail(QSA_ERR_NULL, "%s: data pointer is NULL", name);
  return QSA_OK;
}

int check_contiguous(const char* name, const qsa_tensor* t) {
  int64_t expect = 1;
  for (int d = t->ndim - 1; d >= 0; --d) {
    if (t->shape[d] > 1 && t->stride[d] != expect) {
      return fail(QSA_ERR_LAYOUT, "%s: not contiguous (dim %d stride %lld, expected %lld)", name, d,
                  (long long)t->stride[d], (long long)expect);
    }
    expect *= t->shape[d];
  }
  return QSA_OK;
}

int check_aligned(const char* name, const qsa_tensor* t, uintptr_t align) {
  if (reinterpret_cast<uintptr_t>(t->data) % align) {
    return fail(QSA_ERR_LAYOUT, "%s: data pointer not %zu-byte aligned", name, (size_t)align);
  }
  return QSA_OK;
}

#define QSA_TRY(expr)              \
  do {                             \
    int rc_ = (expr);              \
    if (rc_ != QSA_OK) return rc_; \
  } while (0)

struct SelectView {
  int64_t rows = 0, pages = 0, reqs = 0, width = 0, bt_stride = 0;
  int group = 1;  // rows scored per key stream (q given as [B, n, 4, 128]: min(n, 4))
};

// The selection family's inputs.  e4m3 false: an fp16 key cache (kscale
// unused); true: e4m3 codes with per-key scales.  weights may be NULL.
int validate_select_inputs(const qsa_tensor* q, const qsa_tensor* weights,
                           const qsa_tensor* kcache, const qsa_tensor* kscale, bool e4m3,
                           const qsa_tensor* bt, const qsa_tensor* t2r, const qsa_tensor* sl,
                           const qsa_tensor* qp, SelectView* v) {
  // q is [R, 4, 128], or [B, n, 4, 128] for R = B * n rows in runs of n
  // consecutive rows (next_n draft positions of one request): then rows are
  // scored min(n, 4) at a time against one read of their keys.  Each row's
  // request and position still come from token_to_req and query_pos; the
  // run length only groups the work.
  const bool runs = q && q->ndim == 4;
  const int64_t any3[3] = {-1, QSA_SEL_HEADS, QSA_SEL_DIM};
  const int64_t any4[4] = {-1, -1, QSA_SEL_HEADS, QSA_SEL_DIM};
  QSA_TRY(runs ? check_tensor("q", q, QSA_DTYPE_F16, 4, any4)
               : check_tensor("q", q, QSA_DTYPE_F16, 3, any3));
  QSA_TRY(check_contiguous("q", q));
  QSA_TRY(check_aligned("q", q, 16));
  if (runs && (q->shape[0] > ((int64_t)1 << 30) || q->shape[1] > ((int64_t)1 << 30))) {
    return fail(QSA_ERR_SHAPE, "q: too many rows");
  }
  const int64_t R = runs ? q->shape[0] * q->shape[1] : q->shape[0];
  v->group = runs ? (int)std::max<int64_t>(1, std::min<int64_t>(q->shape[1], qsa::kMaxGroup)) : 1;
  const int64_t kshape[4] = {-1, QSA_PAGE_SLOTS, 1, QSA_SEL_DIM};
  QSA_TRY(check_tensor("kcache", kcache, e4m3 ? QSA_DTYPE_E4M3 : QSA_DTYPE_F16, 4, kshape));
  QSA_TRY(check_contiguous("kcache", kcache));
  QSA_TRY(check_aligned("kcache", kcache, 16));
  if (kcache->shape[0] < 1) return fail(QSA_ERR_SHAPE, "kcache: needs at least one page");
  if (e4m3) {
    const int64_t sshape[2] = {kcache->shape[0], QSA_PAGE_SLOTS};
    QSA_TRY(check_tensor("kscale", kscale, QSA_DTYPE_F32, 2, sshape));
    QSA_TRY(check_contiguous("kscale", kscale));
    QSA_TRY(check_aligned("kscale", kscale, 4));
  }
  const int64_t bshape[2] = {-1, -1};
  QSA_TRY(check_tensor("block_table", bt, QSA_DTYPE_I32, 2, bshape));
  const int64_t N = bt->shape[0], W = bt->shape[1];
  if (W > 1 && bt->stride[1] != 1) return fail(QSA_ERR_LAYOUT, "block_table: stride[1] must be 1");
  if (N > 1 && bt->stride[0] < W) return fail(QSA_ERR_LAYOUT, "block_table: stride[0] < width");
  const int64_t rshape[1] = {R};
  QSA_TRY(check_tensor("token_to_req", t2r, QSA_DTYPE_I32, 1, rshape));
  QSA_TRY(check_contiguous("token_to_req", t2r));
  const int64_t nshape[1] = {N};
  QSA_TRY(check_tensor("seq_lens", sl, QSA_DTYPE_I32, 1, nshape));
  QSA_TRY(check_contiguous("seq_lens", sl));
  QSA_TRY(check_tensor("query_pos", qp, QSA_DTYPE_I64, 1, rshape));
  QSA_TRY(check_contiguous("query_pos", qp));
  if (weights) {
    const int64_t wshape[2] = {R, QSA_SEL_HEADS};
    QSA_TRY(check_tensor("weights", weights, QSA_DTYPE_F32, 2, wshape));
    QSA_TRY(check_contiguous("weights", weights));
    QSA_TRY(check_aligned("weights", weights, 16));
  }
  if (R > 0 && N < 1) return fail(QSA_ERR_SHAPE, "seq_lens/block_table: no requests for %lld rows", (long long)R);
  if (R > (int64_t)1 << 30) return fail(QSA_ERR_SHAPE, "q: too many rows");
  if (W > ((int64_t)1 << 22)) return fail(QSA_ERR_SHAPE, "block_table: too wide");
  v->rows = R;
  v->pages = kcache->shape[0];
  v->reqs = N;
  v->width = W;
  v->bt_stride = N > 1 ? bt->stride[0] : W;
  return QSA_OK;
}

// An output of the selection family must not overlap any of its inputs.
int check_select_output(const char* what, const qsa_tensor* out, const qsa_tensor* q,
                        const qsa_tensor* weights, const qsa_tensor* kcache,
                        const qsa_tensor* kscale, bool e4m3, const qsa_tensor* bt,
                        const qsa_tensor* t2r, const qsa_tensor* sl, const qsa_tensor* qp) {
  const Span so = span_of(out);
  const qsa_tensor* ins[8] = {q, kcache, bt, t2r, sl, qp, e4m3 ? kscale : nullptr, weights};
  const char* names[8] = {"q", "kcache", "block_table", "token_to_req", "seq_lens", "query_pos",
                          "kscale", "weights"};
  for (int i = 0; i < 8; ++i) {
    if (ins[i] && overlaps(so, span_of(ins[i]))) {
      return fail(QSA_ERR_ALIAS, "%s overlaps %s", what, names[i]);
    }
  }
  return QSA_OK;
}

int check_index_rows(const char* name, const qsa_tensor* out, int64_t rows) {
  const int64_t oshape[2] = {rows, QSA_OUT_WIDTH};
  QSA_TRY(check_tensor(name, out, QSA_DTYPE_I32, 2, oshape));
  return check_contiguous(name, out);
}

// A logits matrix: F32 [R, width], unit column stride, row stride >= width.
int check_logits(const char* name, const qsa_tensor* t, int64_t rows) {
  const int64_t shape[2] = {rows, -1};
  QSA_TRY(check_tensor(name, t, QSA_DTYPE_F32, 2, shape));
  const int64_t width = t->shape[1];
  if (width < 1) return fail(QSA_ERR_SHAPE, "%s: width must be >= 1", name);
  if (width > ((int64_t)1 << 29)) return fail(QSA_ERR_SHAPE, "%s: too wide", name);
  if (width > 1 && t->stride[1] != 1) return fail(QSA_ERR_LAYOUT, "%s: stride[1] must be 1", name);
  if (rows > 1 && t->stride[0] < width) return fail(QSA_ERR_LAYOUT, "%s: stride[0] < width", name);
  return check_aligned(name, t, 4);
}

int64_t logits_stride(const qsa_tensor* t) { return t->shape[0] > 1 ? t->stride[0] : t->shape[1]; }

struct AttnView {
  int64_t rows = 0, tokens = 0;
};

int validate_attn(const qsa_tensor* q, const qsa_tensor* k, const qsa_tensor* v,
                  const qsa_tensor* idx, float scale, const qsa_tensor* out, bool idx_is_output,
                  AttnView* view) {
  const int64_t qshape[3] = {-1, QSA_ATT_HEADS, QSA_ATT_DIM};
  QSA_TRY(check_tensor("q", q, QSA_DTYPE_F16, 3, qshape));
  QSA_TRY(check_contiguous("q", q));
  QSA_TRY(check_aligned("q", q, 16));
  const int64_t R = q->shape[0];
  const int64_t kshape[4] = {-1, QSA_KV_PAGE_TOKENS, 1, QSA_ATT_DIM};
  QSA_TRY(check_tensor("k", k, QSA_DTYPE_F16, 4, kshape));
  QSA_TRY(check_tensor("v", v, QSA_DTYPE_F16, 4, kshape));
  static const int64_t packed[4] = {262144, 512, 256, 1};
  for (int d = 0; d < 4; ++d) {
    if (k->stride[d] != packed[d]) {
      return fail(QSA_ERR_LAYOUT, "k: strides must be exactly [262144,512,256,1] (dim %d is %lld)",
                  d, (long long)k->stride[d]);
    }
    if (v->stride[d] != packed[d]) {
      return fail(QSA_ERR_LAYOUT, "v: strides must be exactly [262144,512,256,1] (dim %d is %lld)",
                  d, (long long)v->stride[d]);
    }
  }
  if (v->shape[0] != k->shape[0]) return fail(QSA_ERR_SHAPE, "v: page count differs from k");
  if (k->shape[0] < 1) return fail(QSA_ERR_SHAPE, "k: needs at least one page");
  if (static_cast<char*>(v->data) != static_cast<char*>(k->data) + 2 * QSA_ATT_DIM) {
    return fail(QSA_ERR_LAYOUT, "v: must start 256 elements after k (packed K|V rows)");
  }
  QSA_TRY(check_aligned("k", k, 16));
  if (k->shape[0] > ((int64_t)1 << 31) / QSA_KV_PAGE_TOKENS - 1) {
    return fail(QSA_ERR_SHAPE, "k: too many tokens for int32 indices");
  }
  const int64_t ishape[2] = {R, QSA_OUT_WIDTH};
  QSA_TRY(check_tensor("indices", idx, QSA_DTYPE_I32, 2, ishape));
  QSA_TRY(check_contiguous("indices", idx));
  QSA_TRY(check_tensor("out", out, QSA_DTYPE_F16, 3, qshape));
  if (out->shape[0] != R) return fail(QSA_ERR_SHAPE, "out: rows differ from q");
  QSA_TRY(check_contiguous("out", out));
  if (!std::isfinite(scale) || !(scale > 0.f)) {
    return fail(QSA_ERR_ARG, "softmax_scale must be finite and > 0");
  }
  if (R > (int64_t)1 << 30) return fail(QSA_ERR_SHAPE, "q: too many rows");
  // the packed cache as one span: pages x 512 rows x 512 elements
  qsa_tensor whole = *k;
  whole.ndim = 2;
  whole.shape[0] = k->shape[0] * QSA_KV_PAGE_TOKENS;
  whole.shape[1] = 2 * QSA_ATT_DIM;
  whole.stride[0] = 2 * QSA_ATT_DIM;
  whole.stride[1] = 1;
  const Span so = span_of(out);
  if (overlaps(so, span_of(q))) return fail(QSA_ERR_ALIAS, "out overlaps q");
  if (overlaps(so, span_of(&whole))) return fail(QSA_ERR_ALIAS, "out overlaps k/v");
  if (overlaps(so, span_of(idx))) return fail(QSA_ERR_ALIAS, "out overlaps indices");
  if (idx_is_output) {
    const Span si = span_of(idx);
    if (overlaps(si, span_of(q))) return fail(QSA_ERR_ALIAS, "indices overlap q_attn");
    if (overlaps(si, span_of(&whole))) return fail(QSA_ERR_ALIAS, "indices overlap k/v");
  }
  view->rows = R;
  view->tokens = k->shape[0] * QSA_KV_PAGE_TOKENS;
  return QSA_OK;
}

int check_workspace(void* ws, size_t have, size_t need, Span guarded[], int nguarded) {
  if (need == 0) return QSA_OK;
  if (!ws) return fail(QSA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(QSA_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (have < need) return fail(QSA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  Span w;
  w.lo = reinterpret_cast<uintptr_t>(ws);
  w.hi = w.lo + need;
  for (int i = 0; i < nguarded; ++i) {
    if (overlaps(w, guarded[i])) return fail(QSA_ERR_ALIAS, "workspace overlaps a tensor argument");
  }
  return QSA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// A launch of `cols` workgroups of `threads` threads per row over `rows`
// rows must stay under 2^32 work-items, the limit of one dispatch; checked
// for rows padded to whole XCD groups, which no placement's grid exceeds
// (grid_blocks).
int check_grid(const char* what, int64_t rows, int64_t cols, int threads) {
  const int64_t per_row = (cols > 0 ? cols : 1) * (int64_t)threads;
  if (qsa::padded_rows(rows) > qsa::kMaxWorkItems / per_row) {
    return fail(QSA_ERR_SHAPE, "%s: %lld rows x %lld workgroups per row exceed one launch", what,
                (long long)rows, (long long)cols);
  }
  return QSA_OK;
}

// Both kernels of the selection (chunks over the row groups; the merge,
// one workgroup per row of the padded groups).
int check_select_grid(const char* what, const qsa::SelectPlan& plan, int64_t groups) {
  QSA_TRY(check_grid(what, groups, plan.chunks_per_row,
                     plan.big ? qsa::kChunkBigThreads : qsa::kChunkThreads));
  return check_grid(what, qsa::padded_rows(groups) * plan.group, 1, qsa::kMergeThreads);
}

// Both kernels of the attention (splits of plan.waves waves; combine, one
// workgroup per head).
int check_attn_grid(int64_t rows, const qsa::AttnPlan& plan) {
  QSA_TRY(check_grid("attention", rows, plan.splits, 64 * plan.waves));
  return check_grid("attention", rows, qsa::kAttHeads, qsa::kCombineThreads);
}

// Grid rows of the chunk kernel: one per group of plan.group query rows.
int64_t plan_groups(const qsa::SelectPlan& plan, int64_t rows) {
  return (rows + plan.group - 1) / plan.group;
}

}  // namespace


namespace {

void fill_select_args(qsa::SelectArgs& a, const qsa_tensor* q, const qsa_tensor* weights,
                      const qsa_tensor* kcache, const qsa_tensor* kscale, bool e4m3,
                      const qsa_tensor* block_table, const qsa_tensor* token_to_req,
                      const qsa_tensor* seq_lens, const qsa_tensor* query_pos,
                      const qsa_tensor* out, void* workspace, const SelectView& v) {
  a.q = static_cast<const uint16_t*>(q->data);
  a.weights = weights ? static_cast<const float*>(weights->data) : nullptr;
  a.kcache = e4m3 ? nullptr : static_cast<const uint16_t*>(kcache->data);
  a.kcodes = e4m3 ? static_cast<const uint8_t*>(kcache->data) : nullptr;
  a.kscale = e4m3 ? static_cast<const float*>(kscale->data) : nullptr;
  a.block_table = static_cast<const int32_t*>(block_table->data);
  a.token_to_req = static_cast<const int32_t*>(token_to_req->data);
  a.seq_lens = static_cast<const int32_t*>(seq_lens->data);
  a.query_pos = static_cast<const int64_t*>(query_pos->data);
  a.out = out ? static_cast<int32_t*>(out->data) : nullptr;  // NULL: paged logits
  a.workspace = workspace;
  a.rows = v.rows;
  a.num_pages = v.pages;
  a.num_reqs = v.reqs;
  a.table_width = v.width;
  a.bt_stride = v.bt_stride;
  a.max_visible = v.width * QSA_PAGE_SLOTS;
}

int select_impl(const qsa_tensor* q, const qsa_tensor* weights, const qsa_tensor* kcache,
                const qsa_tensor* kscale, bool e4m3, const qsa_tensor* block_table,
                const qsa_tensor* token_to_req, const qsa_tensor* seq_lens,
                const qsa_tensor* query_pos, const qsa_tensor* out, void* workspace,
                size_t workspace_bytes, qsa_stream stream) {
  g_last_error[0] = '\0';
  SelectView v;
  QSA_TRY(validate_select_inputs(q, weights, kcache, kscale, e4m3, block_table, token_to_req,
                                 seq_lens, query_pos, &v));
  QSA_TRY(check_index_rows("out", out, v.rows));
  QSA_TRY(check_select_output("out", out, q, weights, kcache, kscale, e4m3, block_table,
                              token_to_req, seq_lens, query_pos));
  if (v.rows == 0) return QSA_OK;
  const qsa::SelectPlan plan = qsa::plan_select(v.rows, v.width, v.group, true);
  QSA_TRY(check_select_grid("selection", plan, plan_groups(plan, v.rows)));
  Span guarded[9] = {span_of(q),        span_of(kcache),   span_of(block_table),
                     span_of(token_to_req), span_of(seq_lens), span_of(query_pos),
                     span_of(out),      e4m3 ? span_of(kscale) : Span(),
                     weights ? span_of(weights) : Span()};
  QSA_TRY(check_workspace(workspace, workspace_bytes, plan.bytes, guarded, 9));
  qsa::SelectArgs a;
  fill_select_args(a, q, weights, kcache, kscale, e4m3, block_table, token_to_req, seq_lens,
                   query_pos, out, workspace, v);
  const int err = qsa::launch_select(a, plan, stream);
  if (err) return fail(QSA_ERR_LAUNCH, "selection launch failed (hipError %d)", err);
  return QSA_OK;
}

// static_ws: the workspace is the library's fixed device scratch (the
// no-allocation entry point; `workspace` is ignored), looked up only after
// every check has passed, including that the call fits in it.
int decode_impl(const qsa_tensor* q_sel, const qsa_tensor* kcache, const qsa_tensor* kscale,
                bool e4m3, const qsa_tensor* block_table, const qsa_tensor* token_to_req,
                const qsa_tensor* seq_lens, const qsa_tensor* query_pos, const qsa_tensor* q_attn,
                const qsa_tensor* k, const qsa_tensor* v, float softmax_scale,
                const qsa_tensor* indices, const qsa_tensor* out, void* workspace,
                size_t workspace_bytes, qsa_stream stream, bool static_ws = false) {
  g_last_error[0] = '\0';
  SelectView sv;
  QSA_TRY(validate_select_inputs(q_sel, nullptr, kcache, kscale, e4m3, block_table,
                                 token_to_req, seq_lens, query_pos, &sv));
  QSA_TRY(check_index_rows("indices", indices, sv.rows));
  QSA_TRY(check_select_output("indices", indices, q_sel, nullptr, kcache, kscale, e4m3,
                              block_table, token_to_req, seq_lens, query_pos));
  AttnView av;
  QSA_TRY(validate_attn(q_attn, k, v, indices, softmax_scale, out, true, &av));
  if (av.rows != sv.rows) return fail(QSA_ERR_SHAPE, "q_attn rows differ from q_sel rows");
  // the attention output must not overlap any selection input either
  const qsa_tensor* sel_in[7] = {q_sel, kcache, block_table, token_to_req, seq_lens, query_pos,
                                 kscale};
  for (int i = 0; i < (e4m3 ? 7 : 6); ++i) {
    if (overlaps(span_of(out), span_of(sel_in[i]))) {
      return fail(QSA_ERR_ALIAS, "out overlaps a selection input");
    }
  }
  if (sv.rows == 0) return QSA_OK;
  const qsa::DecodePlan plan = qsa::plan_decode(sv.rows, sv.width, sv.group);
  const qsa::SelectPlan& splan = plan.select;
  const qsa::AttnPlan& aplan = plan.attn;
  QSA_TRY(check_select_grid("selection", splan, plan_groups(splan, sv.rows)));
  QSA_TRY(check_attn_grid(av.rows, aplan));
  const size_t need = plan.bytes;
  if (static_ws) {
    if (need > qsa::kStaticScratchBytes) {
      return fail(QSA_ERR_WORKSPACE,
                  "%lld rows with a %lld-page block table need %zu bytes of scratch; the fixed "
                  "scratch holds %zu (use qsa_decode_step with a workspace)",
                  (long long)sv.rows, (long long)sv.width, need, qsa::kStaticScratchBytes);
    }
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0) {
      const int err = qsa::static_scratch(&workspace);
      if (err) return fail(QSA_ERR_LAUNCH, "fixed scratch lookup failed (hipError %d)", err);
      workspace_bytes = qsa::kStaticScratchBytes;
    }
  }
  qsa_tensor whole = *k;
  whole.ndim = 1;
  whole.shape[0] = av.tokens * 2 * QSA_ATT_DIM;
  whole.stride[0] = 1;
  Span guarded[11] = {span_of(q_sel),        span_of(kcache),   span_of(block_table),
                      span_of(token_to_req), span_of(seq_lens), span_of(query_pos),
                      span_of(q_attn),       span_of(&whole),   span_of(indices),
                      span_of(out),          e4m3 ? span_of(kscale) : Span()};
  QSA_TRY(check_workspace(workspace, workspace_bytes, need, guarded, 11));

  qsa::SelectArgs s;
  fill_select_args(s, q_sel, nullptr, kcache, kscale, e4m3, block_table, token_to_req, seq_lens,
                   query_pos, indices, workspace, sv);
  // Fused path: with whole-CU attention workgroups and rows whose
  // candidates fit in LDS, the attention kernel selects each multi-chunk
  // row itself instead of a merge launch.
  const bool fused = plan.fused;
  qsa::FusedSelect fs;
  if (fused) {
    char* ws = static_cast<char*>(workspace);
    fs.cand_keys = reinterpret_cast<const uint32_t*>(ws + splan.keys_off);
    fs.cand_blocks = reinterpret_cast<const uint32_t*>(ws + splan.blocks_off);
    fs.token_to_req = s.token_to_req;
    fs.seq_lens = s.seq_lens;
    fs.query_pos = s.query_pos;
    fs.num_reqs = s.num_reqs;
    fs.max_visible = s.max_visible;
    fs.chunks_per_row = splan.chunks_per_row;
    fs.chunk_blocks = splan.chunk_pages * QSA_PAGE_SLOTS;
    fs.cand_cap = (int)splan.cand_cap;
  }
  int err = qsa::launch_select(s, splan, stream, !fused);
  if (err) return fail(QSA_ERR_LAUNCH, "selection launch failed (hipError %d)", err);

  qsa::AttnArgs a;
  a.q = static_cast<const uint16_t*>(q_attn->data);
  a.kv = static_cast<const uint16_t*>(k->data);
  a.indices = static_cast<const int32_t*>(indices->data);
  a.out = static_cast<uint16_t*>(out->data);
  a.workspace = aplan.bytes ? static_cast<char*>(workspace) + plan.attn_off : nullptr;
  a.rows = av.rows;
  a.num_tokens = av.tokens;
  a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
  a.fused = fused ? &fs : nullptr;
  err = qsa::launch_attn(a, aplan, stream);
  if (err) return fail(QSA_ERR_LAUNCH, "attention launch failed (hipError %d)", err);
  return QSA_OK;
}

}  // namespace

extern "C" {

QSA_API const char* qsa_status_string(int status) {
  switch (status) {
    case QSA_OK: return "QSA_OK";
    case QSA_ERR_NULL: return "QSA_ERR_NULL";
    case QSA_ERR_DTYPE: return "QSA_ERR_DTYPE";
    case QSA_ERR_SHAPE: return "QSA_ERR_SHAPE";
    case QSA_ERR_LAYOUT: return "QSA_ERR_LAYOUT";
    case QSA_ERR_ALIAS: return "QSA_ERR_ALIAS";
    case QSA_ERR_WORKSPACE: return "QSA_ERR_WORKSPACE";
    case QSA_ERR_ARG: return "QSA_ERR_ARG";
    case QSA_ERR_LAUNCH: return "QSA_ERR_LAUNCH";
    default: return "QSA_ERR_UNKNOWN";
  }
}

QSA_API const char* qsa_last_error(void) { return g_last_error; }

QSA_API void qsa_constants(int32_t* token_topk, int32_t* compress_ratio, int32_t* out_width,
                           int32_t* topk_blocks) {
  if (token_topk) *token_topk = QSA_TOKEN_TOPK;
  if (compress_ratio) *compress_ratio = QSA_COMPRESS_RATIO;
  if (out_width) *out_width = QSA_OUT_WIDTH;
  if (topk_blocks) *topk_blocks = QSA_TOPK_BLOCKS;
}

QSA_API size_t qsa_select_workspace_bytes(int64_t rows, int64_t table_width) {
  if (rows <= 0) return 0;
  // enough for every row grouping (q as [R, 4, 128] or [B, n, 4, 128])
  size_t bytes = 0;
  for (int group = 1; group <= qsa::kMaxGroup; ++group) {
    bytes = std::max(bytes, qsa::plan_select(rows, table_width, group, true).bytes);
  }
  return bytes;
}

QSA_API size_t qsa_sparse_attn_workspace_bytes(int64_t rows) {
  if (rows <= 0) return 0;
  return qsa::plan_attn(rows).bytes;
}

QSA_API size_t qsa_decode_step_workspace_bytes(int64_t rows, int64_t table_width) {
  if (rows <= 0) return 0;
  // enough for every row grouping
  size_t bytes = 0;
  for (int group = 1; group <= qsa::kMaxGroup; ++group) {
    bytes = std::max(bytes, qsa::plan_decode(rows, table_width, group).bytes);
  }
  return bytes;
}

QSA_API int qsa_select(const qsa_tensor* q, const qsa_tensor* kcache, const qsa_tensor* block_table,
                       const qsa_tensor* token_to_req, const qsa_tensor* seq_lens,
                       const qsa_tensor* query_pos, const qsa_tensor* out, void* workspace,
                       size_t workspace_bytes, qsa_stream stream) {
  return select_impl(q, nullptr, kcache, nullptr, false, block_table, token_to_req, seq_lens,
                     query_pos, out, workspace, workspace_bytes, stream);
}

QSA_API int qsa_select_fp8(const qsa_tensor* q, const qsa_tensor* kcache,
                           const qsa_tensor* kscale, const qsa_tensor* block_table,
                           const qsa_tensor* token_to_req, const qsa_tensor* seq_lens,
                           const qsa_tensor* query_pos, const qsa_tensor* out, void* workspace,
                           size_t workspace_bytes, qsa_stream stream) {
  return select_impl(q, nullptr, kcache, kscale, true, block_table, token_to_req, seq_lens,
                     query_pos, out, workspace, workspace_bytes, stream);
}

QSA_API int qsa_select_weighted(const qsa_tensor* q, const qsa_tensor* weights,
                                const qsa_tensor* kcache, const qsa_tensor* kscale,
                                const qsa_tensor* block_table, const qsa_tensor* token_to_req,
                                const qsa_tensor* seq_lens, const qsa_tensor* query_pos,
                                const qsa_tensor* out, void* workspace, size_t workspace_bytes,
                                qsa_stream stream) {
  g_last_error[0] = '\0';
  if (!weights) return fail(QSA_ERR_NULL, "weights: descriptor is NULL");
  return select_impl(q, weights, kcache, kscale, kscale != nullptr, block_table, token_to_req,
                     seq_lens, query_pos, out, workspace, workspace_bytes, stream);
}

QSA_API int qsa_paged_logits(const qsa_tensor* q, const qsa_tensor* weights,
                             const qsa_tensor* kcache, const qsa_tensor* kscale,
                             const qsa_tensor* block_table, const qsa_tensor* token_to_req,
                             const qsa_tensor* seq_lens, const qsa_tensor* query_pos,
                             const qsa_tensor* logits, qsa_stream stream) {
  g_last_error[0] = '\0';
  const bool e4m3 = kscale != nullptr;
  SelectView v;
  QSA_TRY(validate_select_inputs(q, weights, kcache, kscale, e4m3, block_table, token_to_req,
                                 seq_lens, query_pos, &v));
  QSA_TRY(check_logits("logits", logits, v.rows));
  if (logits->shape[1] < v.width * QSA_PAGE_SLOTS) {
    return fail(QSA_ERR_SHAPE, "logits: width %lld < block_table width x 128 = %lld",
                (long long)logits->shape[1], (long long)(v.width * QSA_PAGE_SLOTS));
  }
  QSA_TRY(check_select_output("logits", logits, q, weights, kcache, kscale, e4m3, block_table,
                              token_to_req, seq_lens, query_pos));
  if (v.rows == 0) return QSA_OK;
  const qsa::SelectPlan plan = qsa::plan_select(v.rows, v.width, v.group);
  QSA_TRY(check_grid("paged logits", plan_groups(plan, v.rows), plan.chunks_per_row,
                     qsa::kChunkThreads));
  qsa::SelectArgs a;
  fill_select_args(a, q, weights, kcache, kscale, e4m3, block_table, token_to_req, seq_lens,
                   query_pos, nullptr, nullptr, v);
  a.logits_out = static_cast<float*>(logits->data);
  a.logits_stride = logits_stride(logits);
  a.logits_width = logits->shape[1];
  const int err = qsa::launch_paged_logits(a, plan, stream);
  if (err) return fail(QSA_ERR_LAUNCH, "paged logits launch failed (hipError %d)", err);
  return QSA_OK;
}

QSA_API size_t qsa_topk_per_row_workspace_bytes(int64_t rows, int64_t logits_width) {
  // rows of at most kRowTopkMaxWidth columns: one workgroup per row, none
  if (rows <= 0 || logits_width <= qsa::kRowTopkMaxWidth) return 0;
  return qsa::plan_select(rows, (logits_width + QSA_PAGE_SLOTS - 1) / QSA_PAGE_SLOTS).bytes;
}

QSA_API int qsa_topk_per_row(const qsa_tensor* logits, const qsa_tensor* token_to_req,
                             const qsa_tensor* seq_lens, const qsa_tensor* query_pos,
                             const qsa_tensor* out, void* workspace, size_t workspace_bytes,
                             qsa_stream stream) {
  g_last_error[0] = '\0';
  if (!logits) return fail(QSA_ERR_NULL, "logits: descriptor is NULL");
  const int64_t R = logits->shape[0];
  QSA_TRY(check_logits("logits", logits, logits->ndim == 2 ? R : -1));
  const int64_t rshape[1] = {R};
  QSA_TRY(check_tensor("token_to_req", token_to_req, QSA_DTYPE_I32, 1, rshape));
  QSA_TRY(check_contiguous("token_to_req", token_to_req));
  const int64_t any1[1] = {-1};
  QSA_TRY(check_tensor("seq_lens", seq_lens, QSA_DTYPE_I32, 1, any1));
  QSA_TRY(check_contiguous("seq_lens", seq_lens));
  QSA_TRY(check_tensor("query_pos", query_pos, QSA_DTYPE_I64, 1, rshape));
  QSA_TRY(check_contiguous("query_pos", query_pos));
  QSA_TRY(check_index_rows("out", out, R));
  const int64_t N = seq_lens->shape[0];
  if (R > 0 && N < 1) return fail(QSA_ERR_SHAPE, "seq_lens: no requests for %lld rows", (long long)R);
  if (R > (int64_t)1 << 30) return fail(QSA_ERR_SHAPE, "logits: too many rows");
  const qsa_tensor* ins[4] = {logits, token_to_req, seq_lens, query_pos};
  const char* names[4] = {"logits", "token_to_req", "seq_lens", "query_pos"};
  for (int i = 0; i < 4; ++i) {
    if (overlaps(span_of(out), span_of(ins[i]))) return fail(QSA_ERR_ALIAS, "out overlaps %s", names[i]);
  }
  if (R == 0) return QSA_OK;
  const int64_t width = logits->shape[1];
  const int64_t pages = (width + QSA_PAGE_SLOTS - 1) / QSA_PAGE_SLOTS;
  // rows of at most kRowTopkMaxWidth columns: one workgroup per row holds
  // the whole row; wider ones go through chunks and a merge
  const bool whole_rows = width <= qsa::kRowTopkMaxWidth;
  const qsa::SelectPlan plan = whole_rows ? qsa::SelectPlan{} : qsa::plan_select(R, pages);
  if (whole_rows) {
    QSA_TRY(check_grid("top-k", R, 1, qsa::kRowTopkThreads));
  } else {
    QSA_TRY(check_select_grid("top-k", plan, R));
  }
  Span guarded[5] = {span_of(logits), span_of(token_to_req), span_of(seq_lens),
                     span_of(query_pos), span_of(out)};
  QSA_TRY(check_workspace(workspace, workspace_bytes, plan.bytes, guarded, 5));
  qsa::SelectArgs a;
  a.logits_in = static_cast<const float*>(logits->data);
  a.logits_stride = logits_stride(logits);
  a.logits_width = width;
  a.max_visible = width;
  a.token_to_req = static_cast<const int32_t*>(token_to_req->data);
  a.seq_lens = static_cast<const int32_t*>(seq_lens->data);
  a.query_pos = static_cast<const int64_t*>(query_pos->data);
  a.out = static_cast<int32_t*>(out->data);
  a.workspace = workspace;
  a.rows = R;
  a.num_reqs = N;
  a.table_width = pages;
  const int err = whole_rows ? qsa::launch_topk_rows(a, stream) : qsa::launch_select(a, plan, stream);
  if (err) return fail(QSA_ERR_LAUNCH, "top-k launch failed (hipError %d)", err);
  return QSA_OK;
}

QSA_API int qsa_sparse_attn(const qsa_tensor* q, const qsa_tensor* k, const qsa_tensor* v,
                            const qsa_tensor* indices, float softmax_scale, const qsa_tensor* out,
                            void* workspace, size_t workspace_bytes, qsa_stream stream) {
  g_last_error[0] = '\0';
  AttnView view;
  QSA_TRY(validate_attn(q, k, v, indices, softmax_scale, out, false, &view));
  if (view.rows == 0) return QSA_OK;
  const qsa::AttnPlan plan = qsa::plan_attn(view.rows);
  QSA_TRY(check_attn_grid(view.rows, plan));
  qsa_tensor whole = *k;
  whole.ndim = 1;
  whole.shape[0] = view.tokens * 2 * QSA_ATT_DIM;
  whole.stride[0] = 1;
  Span guarded[4] = {span_of(q), span_of(&whole), span_of(indices), span_of(out)};
  QSA_TRY(check_workspace(workspace, workspace_bytes, plan.bytes, guarded, 4));
  qsa::AttnArgs a;
  a.q = static_cast<const uint16_t*>(q->data);
  a.kv = static_cast<const uint16_t*>(k->data);
  a.indices = static_cast<const int32_t*>(indices->data);
  a.out = static_cast<uint16_t*>(out->data);
  a.workspace = workspace;
  a.rows = view.rows;
  a.num_tokens = view.tokens;
  a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
  const int err = qsa::launch_attn(a, plan, stream);
  if (err) return fail(QSA_ERR_LAUNCH, "attention launch failed (hipError %d)", err);
  return QSA_OK;
}

QSA_API int qsa_decode_step(const qsa_tensor* q_sel, const qsa_tensor* kcache,
                            const qsa_tensor* block_table, const qsa_tensor* token_to_req,
                            const qsa_tensor* seq_lens, const qsa_tensor* query_pos,
                            const qsa_tensor* q_attn, const qsa_tensor* k, const qsa_tensor* v,
                            float softmax_scale, const qsa_tensor* indices, const qsa_tensor* out,
                            void* workspace, size_t workspace_bytes, qsa_stream stream) {
  return decode_impl(q_sel, kcache, nullptr, false, block_table, token_to_req, seq_lens,
                     query_pos, q_attn, k, v, softmax_scale, indices, out, workspace,
                     workspace_bytes, stream);
}

QSA_API int qsa_decode_step_fp8(const qsa_tensor* q_sel, const qsa_tensor* kcache,
                                const qsa_tensor* kscale, const qsa_tensor* block_table,
                                const qsa_tensor* token_to_req, const qsa_tensor* seq_lens,
                                const qsa_tensor* query_pos, const qsa_tensor* q_attn,
                                const qsa_tensor* k, const qsa_tensor* v, float softmax_scale,
                                const qsa_tensor* indices, const qsa_tensor* out, void* workspace,
                                size_t workspace_bytes, qsa_stream stream) {
  return decode_impl(q_sel, kcache, kscale, true, block_table, token_to_req, seq_lens, query_pos,
                     q_attn, k, v, softmax_scale, indices, out, workspace, workspace_bytes, stream);
}

QSA_API int qsa_decode_step_noalloc(const qsa_tensor* q_sel, const qsa_tensor* kcache,
                                    const qsa_tensor* block_table, const qsa_tensor* token_to_req,
                                    const qsa_tensor* seq_lens, const qsa_tensor* query_pos,
                                    const qsa_tensor* q_attn, const qsa_tensor* k,
                                    const qsa_tensor* v, float softmax_scale,
                                    const qsa_tensor* indices, const qsa_tensor* out,
                                    qsa_stream stream) {
  return decode_impl(q_sel, kcache, nullptr, false, block_table, token_to_req, seq_lens,
                     query_pos, q_attn, k, v, softmax_scale, indices, out, nullptr, 0, stream,
                     true);
}

QSA_API size_t qsa_build_metadata_workspace_bytes(int64_t num_reqs) {
  if (num_reqs <= 0) return 0;
  return align256((size_t)num_reqs * sizeof(int32_t));
}

QSA_API int qsa_build_metadata(const qsa_tensor* query_start_loc, const qsa_tensor* seq_lens,
                               const qsa_tensor* block_table,
                               const qsa_tensor* common_slot_mapping,
                               int64_t storage_block_size, int64_t compress_ratio,
                               int64_t circular_buffer_size, const qsa_tensor* token_to_req,
                               const qsa_tensor* logical_positions,
                               const qsa_tensor* visible_blocks, const qsa_tensor* slot_mapping,
                               const qsa_tensor* k_work_metadata, void* workspace,
                               size_t workspace_bytes, qsa_stream stream) {
  g_last_error[0] = '\0';
  if (storage_block_size < 1 || storage_block_size > ((int64_t)1 << 30)) {
    return fail(QSA_ERR_ARG, "storage_block_size must be in [1, 2^30]");
  }
  if (compress_ratio < 1 || compress_ratio > ((int64_t)1 << 30)) {
    return fail(QSA_ERR_ARG, "compress_ratio must be in [1, 2^30]");
  }
  if (circular_buffer_size < 0 || circular_buffer_size > ((int64_t)1 << 30)) {
    return fail(QSA_ERR_ARG, "circular_buffer_size must be in [0, 2^30]");
  }
  const int64_t any1[1] = {-1};
  QSA_TRY(check_tensor("seq_lens", seq_lens, QSA_DTYPE_I32, 1, any1));
  QSA_TRY(check_contiguous("seq_lens", seq_lens));
  const int64_t N = seq_lens->shape[0];
  if (N < 1) return fail(QSA_ERR_SHAPE, "seq_lens: needs at least one request");
  if (N > ((int64_t)1 << 24)) return fail(QSA_ERR_SHAPE, "seq_lens: too many requests");
  const int64_t qshape[1] = {N + 1};
  QSA_TRY(check_tensor("query_start_loc", query_start_loc, QSA_DTYPE_I32, 1, qshape));
  QSA_TRY(check_contiguous("query_start_loc", query_start_loc));
  const int64_t bshape[2] = {N, -1};
  QSA_TRY(check_tensor("block_table", block_table, QSA_DTYPE_I32, 2, bshape));
  const int64_t W = block_table->shape[1];
  if (W > 1 && block_table->stride[1] != 1) return fail(QSA_ERR_LAYOUT, "block_table: stride[1] must be 1");
  if (N > 1 && block_table->stride[0] < W) return fail(QSA_ERR_LAYOUT, "block_table: stride[0] < width");
  QSA_TRY(check_tensor("token_to_req", token_to_req, QSA_DTYPE_I32, 1, any1));
  QSA_TRY(check_contiguous("token_to_req", token_to_req));
  const int64_t T = token_to_req->shape[0];
  if (T > ((int64_t)1 << 31) - 1) return fail(QSA_ERR_SHAPE, "token_to_req: too many tokens");
  const int64_t tshape[1] = {T};
  QSA_TRY(check_tensor("logical_positions", logical_positions, QSA_DTYPE_I64, 1, tshape));
  QSA_TRY(check_contiguous("logical_positions", logical_positions));
  QSA_TRY(check_tensor("visible_blocks", visible_blocks, QSA_DTYPE_I32, 1, tshape));
  QSA_TRY(check_contiguous("visible_blocks", visible_blocks));
  if (common_slot_mapping) {
    QSA_TRY(check_tensor("common_slot_mapping", common_slot_mapping, QSA_DTYPE_I64, 1, tshape));
    QSA_TRY(check_contiguous("common_slot_mapping", common_slot_mapping));
  }
  if (slot_mapping) {
    QSA_TRY(check_tensor("slot_mapping", slot_mapping, QSA_DTYPE_I64, 1, tshape));
    QSA_TRY(check_contiguous("slot_mapping", slot_mapping));
  }
  int64_t M = 0;
  if (k_work_metadata) {
    const int64_t kshape[2] = {-1, 2};
    QSA_TRY(check_tensor("k_work_metadata", k_work_metadata, QSA_DTYPE_I32, 2, kshape));
    QSA_TRY(check_contiguous("k_work_metadata", k_work_metadata));
    M = k_work_metadata->shape[0];
    if (M > ((int64_t)1 << 31) - 1) return fail(QSA_ERR_SHAPE, "k_work_metadata: too many items");
  }
  // outputs must not overlap each other or any input
  const qsa_tensor* outs[5] = {token_to_req, logical_positions, visible_blocks, slot_mapping,
                               k_work_metadata};
  const char* onames[5] = {"token_to_req", "logical_positions", "visible_blocks", "slot_mapping",
                           "k_work_metadata"};
  const qsa_tensor* ins[4] = {query_start_loc, seq_lens, block_table, common_slot_mapping};
  const char* inames[4] = {"query_start_loc", "seq_lens", "block_table", "common_slot_mapping"};
  for (int o = 0; o < 5; ++o) {
    if (!outs[o]) continue;
    for (int i = 0; i < 4; ++i) {
      if (ins[i] && overlaps(span_of(outs[o]), span_of(ins[i]))) {
        return fail(QSA_ERR_ALIAS, "%s overlaps %s", onames[o], inames[i]);
      }
    }
    for (int o2 = o + 1; o2 < 5; ++o2) {
      if (outs[o2] && overlaps(span_of(outs[o]), span_of(outs[o2]))) {
        return fail(QSA_ERR_ALIAS, "%s overlaps %s", onames[o], onames[o2]);
      }
    }
  }
  const size_t need = M > 0 ? qsa_build_metadata_workspace_bytes(N) : 0;
  Span guarded[9];
  int ng = 0;
  for (int o = 0; o < 5; ++o) if (outs[o]) guarded[ng++] = span_of(outs[o]);
  for (int i = 0; i < 4; ++i) if (ins[i]) guarded[ng++] = span_of(ins[i]);
  QSA_TRY(check_workspace(workspace, workspace_bytes, need, guarded, ng));
  if (T == 0 && M == 0) return QSA_OK;
  qsa::MetaArgs a;
  a.query_start_loc = static_cast<const int32_t*>(query_start_loc->data);
  a.seq_lens = static_cast<const int32_t*>(seq_lens->data);
  a.block_table = static_cast<const int32_t*>(block_table->data);
  a.common_slot_mapping =
      common_slot_mapping ? static_cast<const int64_t*>(common_slot_mapping->data) : nullptr;
  a.token_to_req = static_cast<int32_t*>(token_to_req->data);
  a.logical_positions = static_cast<int64_t*>(logical_positions->data);
  a.visible_blocks = static_cast<int32_t*>(visible_blocks->data);
  a.slot_mapping = slot_mapping ? static_cast<int64_t*>(slot_mapping->data) : nullptr;
  a.k_work = M > 0 ? static_cast<int32_t*>(k_work_metadata->data) : nullptr;
  a.work_ends = M > 0 ? static_cast<int32_t*>(workspace) : nullptr;
  a.num_reqs = N;
  a.num_tokens = T;
  a.max_num_work = M;
  a.table_width = W;
  a.bt_stride = N > 1 ? block_table->stride[0] : W;
  a.storage_block_size = storage_block_size;
  a.compress_ratio = compress_ratio;
  a.circular_buffer_size = circular_buffer_size;
  const int err = qsa::launch_metadata(a, stream);
  if (err) return fail(QSA_ERR_LAUNCH, "metadata launch failed (hipError %d)", err);
  return QSA_OK;
}

}  // extern "C"
