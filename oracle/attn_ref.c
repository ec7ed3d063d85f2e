/*
 * TEST INFRASTRUCTURE ONLY.  Reference attention for the verification-step
 * oracle.  Only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark load this file's library; the product library never links it.
 *
 * Source: "Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV
 * Hierarchy" (arXiv 2610.13708).
 *   - §2.1, eq. (1): u_t = Attn(h_t, {c_s : s in S_t}).  The pages only name
 *     Attn; the reading used here is per-head scaled dot-product softmax
 *     attention, K = row[0:d_qk], V = row[v_off : v_off+d_v].
 *   - §2.1 (text after eq. 1): S_t is kept as the ordered list the top-k
 *     returns; §3.5, eqs. (11)-(12): every list entry receives its own
 *     location, so every entry is one softmax term (a repeated entry counts
 *     twice).
 *
 * Plain definition, no tiling, no online rescaling: for each head,
 *   s_e = scale * sum_c q[c] * K_e[c]
 *   m   = max_e s_e
 *   w_e = exp(s_e - m),  Z = sum_e w_e
 *   out[c] = sum_e w_e * V_e[c] / Z
 * in double, from exact bf16 inputs (a bf16 value is the top half of an
 * IEEE float).  Queries are split over POSIX threads.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_to_double(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

typedef struct {
  int n_q, n_heads, d_qk, v_off, d_v, row_elems;
  double scale;
  const uint64_t *q_ptrs;
  const int64_t *row_begin;
  const uint64_t *row_ptrs;
  double *out;
  int tid, n_threads;
  int status;
} job_t;

/* one query: rows row_ptrs[row_begin[qi] .. row_begin[qi+1]) */
static int attend_one(const job_t *jb, int qi) {
  const int H = jb->n_heads, dqk = jb->d_qk, dv = jb->d_v, re = jb->row_elems;
  const int64_t b = jb->row_begin[qi], n = jb->row_begin[qi + 1] - b;
  double *out = jb->out + (int64_t)qi * H * dv;
  memset(out, 0, sizeof(double) * (size_t)H * dv);
  if (n <= 0) return 0;
  const uint16_t *q = (const uint16_t *)(uintptr_t)jb->q_ptrs[qi];
  double *rows = (double *)malloc(sizeof(double) * (size_t)n * re);
  double *s = (double *)malloc(sizeof(double) * (size_t)n);
  double *qd = (double *)malloc(sizeof(double) * (size_t)dqk);
  if (!rows || !s || !qd) { free(rows); free(s); free(qd); return -1; }
  for (int64_t e = 0; e < n; ++e) {
    const uint16_t *src = (const uint16_t *)(uintptr_t)jb->row_ptrs[b + e];
    for (int c = 0; c < re; ++c) rows[e * re + c] = bf16_to_double(src[c]);
  }
  for (int h = 0; h < H; ++h) {
    for (int c = 0; c < dqk; ++c) qd[c] = bf16_to_double(q[(int64_t)h * dqk + c]);
    double m = -INFINITY;
    for (int64_t e = 0; e < n; ++e) {
      double acc = 0.0;
      for (int c = 0; c < dqk; ++c) acc += qd[c] * rows[e * re + c];
      s[e] = jb->scale * acc;
      if (s[e] > m) m = s[e];
    }
    double z = 0.0;
    for (int64_t e = 0; e < n; ++e) { s[e] = exp(s[e] - m); z += s[e]; }
    double *o = out + (int64_t)h * dv;
    for (int64_t e = 0; e < n; ++e) {
      const double w = s[e] / z;
      const double *v = rows + e * re + jb->v_off;
      for (int c = 0; c < dv; ++c) o[c] += w * v[c];
    }
  }
  free(rows); free(s); free(qd);
  return 0;
}

static void *worker(void *arg) {
  job_t *jb = (job_t *)arg;
  for (int qi = jb->tid; qi < jb->n_q; qi += jb->n_threads)
    if (attend_one(jb, qi) != 0) { jb->status = -1; break; }
  return NULL;
}

/* Returns 0 on success, -1 on allocation failure or bad arguments.
 * q_ptrs[qi]  : address of bf16 [n_heads][d_qk] for query qi
 * row_begin   : n_q+1 offsets into row_ptrs
 * row_ptrs[e] : address of a bf16 row of row_elems elements
 * out         : double [n_q][n_heads][d_v]                                  */
int oracle_attend_batch(int n_q, int n_heads, int d_qk, int v_off, int d_v, int row_elems,
                        double scale, const uint64_t *q_ptrs, const int64_t *row_begin,
                        const uint64_t *row_ptrs, double *out, int n_threads) {
  if (n_q < 0 || n_heads <= 0 || d_qk <= 0 || d_v <= 0 || v_off < 0 ||
      d_qk > row_elems || v_off + d_v > row_elems)
    return -1;
  if (n_threads < 1) n_threads = 1;
  if (n_threads > n_q) n_threads = n_q > 0 ? n_q : 1;
  job_t *jobs = (job_t *)calloc((size_t)n_threads, sizeof(job_t));
  pthread_t *th = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
  if (!jobs || !th) { free(jobs); free(th); return -1; }
  int rc = 0;
  for (int t = 0; t < n_threads; ++t) {
    jobs[t] = (job_t){n_q, n_heads, d_qk, v_off, d_v, row_elems, scale, q_ptrs, row_begin,
                      row_ptrs, out, t, n_threads, 0};
    if (t > 0 && pthread_create(&th[t], NULL, worker, &jobs[t]) != 0) { jobs[t].status = -2; }
  }
  worker(&jobs[0]);
  for (int t = 1; t < n_threads; ++t) {
    if (jobs[t].status == -2) { rc = -1; continue; }
    pthread_join(th[t], NULL);
  }
  for (int t = 0; t < n_threads; ++t) if (jobs[t].status != 0) rc = -1;
  free(jobs); free(th);
  return rc;
}
