/*
 * A plain C caller of the library: no Python, no torch.  Device buffers come
 * from hipMalloc, qsa_tensor descriptors are filled by hand, and one
 * qsa_decode_step call runs on the null stream; the result is checked
 * against the CPU oracle's C entry points (test infrastructure: this
 * program may link the oracle, the library never does).  Also checks that a
 * call with a wrong dtype fails closed with a message.  Exit status 0 when
 * everything matches.
 *
 * Inputs are exact in binary16: selection keys and queries are integers in
 * [-4, 4] (every fp32 sum exact, so the selection must match bit for bit),
 * attention queries and K/V are multiples of 1/8 in [-1, 1].
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qsa.h"

/* the oracle's C entry points (oracle/qsa_oracle.c) */
int qsa_oracle_select(int64_t R, int64_t num_pages, int64_t num_reqs, int64_t table_width,
                      const uint16_t* q, const uint16_t* kcache, const int32_t* block_table,
                      const int32_t* token_to_req, const int32_t* seq_lens,
                      const int64_t* query_pos, int32_t* out);
int qsa_oracle_sparse_attn(int64_t R, int64_t num_tokens, const uint16_t* q, const uint16_t* kv,
                           const int32_t* indices, double scale, double* out);
double qsa_oracle_half_to_double(uint16_t h);

#define R 3
#define NREQ 3
#define P 16
#define W 5
#define NP 5 /* KV pages of 512 tokens: covers the longest row */

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) { /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static int uniform_int(int lo, int hi) { return lo + (int)(next_u32() % (uint32_t)(hi - lo + 1)); }

/* binary16 bits of x, which must be 0 or a normal binary16 value exactly
 * (true for every input made here) */
static uint16_t half_bits(double x) {
  if (x == 0.0) return 0;
  uint16_t sign = x < 0 ? 0x8000u : 0u;
  double a = fabs(x);
  int e = 0;
  while (a >= 2.0) { a /= 2.0; ++e; }
  while (a < 1.0) { a *= 2.0; --e; }
  return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)((a - 1.0) * 1024.0));
}

static qsa_tensor desc(void* data, int dtype, int ndim, const int64_t* shape) {
  qsa_tensor t;
  memset(&t, 0, sizeof t);
  t.data = data;
  t.dtype = dtype;
  t.ndim = ndim;
  int64_t stride = 1;
  for (int d = ndim - 1; d >= 0; --d) {
    t.shape[d] = shape[d];
    t.stride[d] = stride;
    stride *= shape[d];
  }
  return t;
}

#define HIP_OK(call)                                                   \
  do {                                                                 \
    hipError_t e_ = (call);                                            \
    if (e_ != hipSuccess) {                                            \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_)); \
      return 2;                                                        \
    }                                                                  \
  } while (0)

static void* upload(const void* host, size_t bytes, int* bad) {
  void* dev = NULL;
  if (hipMalloc(&dev, bytes) != hipSuccess || hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice) != hipSuccess) *bad = 1;
  return dev;
}

int main(void) {
  const int32_t lengths[NREQ] = {519, 2200, 0}; /* 129 blocks + 3 tail; 550 blocks; empty */
  static uint16_t q_sel[R * 4 * 128], kcache[P * 128 * 128], q_attn[R * 3 * 256];
  static uint16_t kv[NP * 512 * 512];
  int32_t bt[NREQ * W], t2r[R], sl[NREQ];
  int64_t qp[R];
  for (size_t i = 0; i < sizeof q_sel / 2; ++i) q_sel[i] = half_bits(uniform_int(-4, 4));
  for (size_t i = 0; i < sizeof kcache / 2; ++i) kcache[i] = half_bits(uniform_int(-4, 4));
  for (size_t i = 0; i < sizeof q_attn / 2; ++i) q_attn[i] = half_bits(uniform_int(-8, 8) / 8.0);
  for (size_t i = 0; i < sizeof kv / 2; ++i) kv[i] = half_bits(uniform_int(-8, 8) / 8.0);
  for (int r = 0; r < NREQ; ++r) {
    /* distinct pages per row: a rotation of 0..P-1 */
    int start = uniform_int(0, P - 1);
    for (int j = 0; j < W; ++j) bt[r * W + j] = (start + 3 * j) % P;
    t2r[r] = r;
    sl[r] = lengths[r];
    qp[r] = (int64_t)lengths[r] - 1;
  }

  int bad = 0;
  void* d_q = upload(q_sel, sizeof q_sel, &bad);
  void* d_kc = upload(kcache, sizeof kcache, &bad);
  void* d_bt = upload(bt, sizeof bt, &bad);
  void* d_t2r = upload(t2r, sizeof t2r, &bad);
  void* d_sl = upload(sl, sizeof sl, &bad);
  void* d_qp = upload(qp, sizeof qp, &bad);
  void* d_qa = upload(q_attn, sizeof q_attn, &bad);
  void* d_kv = upload(kv, sizeof kv, &bad);
  void *d_idx = NULL, *d_out = NULL, *d_ws = NULL;
  size_t ws_bytes = qsa_decode_step_workspace_bytes(R, W);
  if (bad) { fprintf(stderr, "upload failed\n"); return 2; }
  HIP_OK(hipMalloc(&d_idx, (size_t)R * QSA_OUT_WIDTH * sizeof(int32_t)));
  HIP_OK(hipMalloc(&d_out, (size_t)R * 3 * 256 * sizeof(uint16_t)));
  if (ws_bytes) HIP_OK(hipMalloc(&d_ws, ws_bytes));

  const int64_t s_q[3] = {R, 4, 128}, s_kc[4] = {P, 128, 1, 128}, s_bt[2] = {NREQ, W};
  const int64_t s_r[1] = {R}, s_n[1] = {NREQ}, s_qa[3] = {R, 3, 256}, s_idx[2] = {R, QSA_OUT_WIDTH};
  qsa_tensor tq = desc(d_q, QSA_DTYPE_F16, 3, s_q), tkc = desc(d_kc, QSA_DTYPE_F16, 4, s_kc);
  qsa_tensor tbt = desc(d_bt, QSA_DTYPE_I32, 2, s_bt), tt2r = desc(d_t2r, QSA_DTYPE_I32, 1, s_r);
  qsa_tensor tsl = desc(d_sl, QSA_DTYPE_I32, 1, s_n), tqp = desc(d_qp, QSA_DTYPE_I64, 1, s_r);
  qsa_tensor tqa = desc(d_qa, QSA_DTYPE_F16, 3, s_qa), tidx = desc(d_idx, QSA_DTYPE_I32, 2, s_idx);
  qsa_tensor tout = desc(d_out, QSA_DTYPE_F16, 3, s_qa);
  /* K and V: [NP,512,1,256] views of the packed cache, V at element +256 */
  qsa_tensor tk, tv;
  memset(&tk, 0, sizeof tk);
  tk.data = d_kv;
  tk.dtype = QSA_DTYPE_F16;
  tk.ndim = 4;
  const int64_t kshape[4] = {NP, 512, 1, 256}, kstride[4] = {262144, 512, 256, 1};
  memcpy(tk.shape, kshape, sizeof kshape);
  memcpy(tk.stride, kstride, sizeof kstride);
  tv = tk;
  tv.data = (uint16_t*)d_kv + 256;
  const float scale = 0.0625f;

  /* fail-closed: an int32 query is rejected before anything is launched */
  qsa_tensor wrong = tq;
  wrong.dtype = QSA_DTYPE_I32;
  int st = qsa_decode_step(&wrong, &tkc, &tbt, &tt2r, &tsl, &tqp, &tqa, &tk, &tv, scale, &tidx,
                           &tout, d_ws, ws_bytes, NULL);
  if (st != QSA_ERR_DTYPE || qsa_last_error()[0] == '\0') {
    fprintf(stderr, "wrong dtype: status %d (%s)\n", st, qsa_status_string(st));
    return 1;
  }

  st = qsa_decode_step(&tq, &tkc, &tbt, &tt2r, &tsl, &tqp, &tqa, &tk, &tv, scale, &tidx, &tout,
                       d_ws, ws_bytes, NULL);
  if (st != QSA_OK) {
    fprintf(stderr, "qsa_decode_step: %s: %s\n", qsa_status_string(st), qsa_last_error());
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());
  static int32_t got_idx[R * QSA_OUT_WIDTH], want_idx[R * QSA_OUT_WIDTH];
  static uint16_t got_out[R * 3 * 256];
  static double want_out[R * 3 * 256];
  HIP_OK(hipMemcpy(got_idx, d_idx, sizeof got_idx, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(got_out, d_out, sizeof got_out, hipMemcpyDeviceToHost));

  if (qsa_oracle_select(R, P, NREQ, W, q_sel, kcache, bt, t2r, sl, qp, want_idx) != 0 ||
      qsa_oracle_sparse_attn(R, NP * 512, q_attn, kv, want_idx, scale, want_out) != 0) {
    fprintf(stderr, "oracle failed\n");
    return 2;
  }
  for (int i = 0; i < R * QSA_OUT_WIDTH; ++i) {
    if (got_idx[i] != want_idx[i]) {
      fprintf(stderr, "index %d: %d, oracle %d\n", i, got_idx[i], want_idx[i]);
      return 1;
    }
  }
  double max_err = 0.0;
  for (int i = 0; i < R * 3 * 256; ++i) {
    double e = fabs(qsa_oracle_half_to_double(got_out[i]) - want_out[i]);
    if (e > max_err) max_err = e;
  }
  if (max_err > 2e-3) {
    fprintf(stderr, "attention max abs error %.3e\n", max_err);
    return 1;
  }
  int valid = 0;
  for (int j = 0; j < QSA_OUT_WIDTH; ++j) valid += got_idx[j] >= 0;
  printf("c caller ok: row 0 width %d, row 2 empty, attention max err %.2e\n", valid, max_err);
  hipFree(d_q); hipFree(d_kc); hipFree(d_bt); hipFree(d_t2r); hipFree(d_sl); hipFree(d_qp);
  hipFree(d_qa); hipFree(d_kv); hipFree(d_idx); hipFree(d_out);
  if (d_ws) hipFree(d_ws);
  return 0;
}
