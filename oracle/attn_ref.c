/*
 * Oracle: exact (naive, materialised) attention forward in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header or table with the GPU library.
 *
 * What it computes (the plain definition the pages start from):
 *   - "15-operators-attention" (TileLang tutorial), section 1.1: per
 *     (batch, head) S = Q K^T * s, P = row-softmax(S), O = P V.
 *   - same page, section 2.1: the safe softmax subtracts the row maximum.
 *   - same page, section 5.1 (2): a row that sees no key gets O = 0; its
 *     log-sum-exp is taken as -inf (the page leaves it open).
 *   - same page, section 3.4 (2) and 5.3: causal masking is aligned to the
 *     bottom right, key j visible to query i iff j <= i + (Skv - Sq); varlen
 *     sequences use the same rule inside each sequence.
 *   - same page, section 4.8 (1): query head h reads KV head h / (H / Hkv).
 *   - "learn-cuda-from-scratch" ch.12, FA3 skeleton: the log-sum-exp output is
 *     m + log(l) in the natural base, of the scaled scores.
 *   - sliding window (TileLang tutorial section 5.2; the CUDA course ch.12,
 *     section 12.9.5): with window W > 0 key j is visible to query i iff
 *     i + (Skv - Sq) - W < j <= i + (Skv - Sq), the causal bound included.
 *   - attention sink (TileLang tutorial sections 4.6 and 4.7): a per-head
 *     logit that joins the softmax denominator only, exp(sink - m) added to
 *     l, with m taken as max(row max, sink) so that a large sink cannot
 *     overflow; the log-sum-exp then includes the sink.  A row that sees no
 *     key but has a sink gets O = 0 and LSE = sink.
 *
 * For each row the scores of every visible key are materialised in an fp64
 * buffer, the maximum m is taken, p_j = exp(s_j - m), l = sum p_j,
 * O = sum (p_j / l) v_j, LSE = m + ln l.  Inputs arrive as fp32 arrays; bf16
 * and fp32 sources are represented exactly.  All arithmetic is fp64, the sums
 * run in index order.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  const float *q, *k, *v;
  int B, H, Hkv, Sq, Skv, d, causal;
  int window;            /* > 0: sliding window of this many keys (causal implied) */
  const double* sinks;   /* NULL, or one logit per query head */
  double scale;
  const int32_t* cu;  /* NULL: dense batch */
  const int64_t* rows; /* NULL: every row */
  int64_t nrows;
  double *o, *lse;
  int tid, nthreads;
  int status;
} job_t;

/* Row number r -> (b, h, i).  Without an explicit row list the rows are
 * enumerated in output order: dense [B,H,Sq], varlen [H,T]. */
static void row_coords(const job_t* J, int64_t r, int* b, int* h, int* i) {
  if (J->rows) {
    *b = (int)J->rows[3 * r + 0];
    *h = (int)J->rows[3 * r + 1];
    *i = (int)J->rows[3 * r + 2];
    return;
  }
  if (J->cu) {
    int64_t T = J->cu[J->B];
    int hh = (int)(r / T);
    int t = (int)(r % T);
    int bb = 0;
    while (bb + 1 < J->B && J->cu[bb + 1] <= t) bb++;
    *b = bb;
    *h = hh;
    *i = t - J->cu[bb];
    return;
  }
  *i = (int)(r % J->Sq);
  *h = (int)((r / J->Sq) % J->H);
  *b = (int)(r / ((int64_t)J->Sq * J->H));
}

static void* worker(void* arg) {
  job_t* J = (job_t*)arg;
  const int d = J->d;
  const int group = J->H / J->Hkv;
  int64_t total = J->nrows;
  int maxk = J->Skv;
  if (J->cu) {
    maxk = 0;
    for (int b = 0; b < J->B; ++b) {
      int L = J->cu[b + 1] - J->cu[b];
      if (L > maxk) maxk = L;
    }
  }
  double* s = (double*)malloc(sizeof(double) * (size_t)(maxk > 0 ? maxk : 1));
  double* acc = (double*)malloc(sizeof(double) * (size_t)d);
  if (!s || !acc) {
    J->status = 3;
    free(s);
    free(acc);
    return NULL;
  }
  for (int64_t r0 = (int64_t)J->tid * 64; r0 < total; r0 += (int64_t)J->nthreads * 64) {
    int64_t r1 = r0 + 64 < total ? r0 + 64 : total;
    for (int64_t r = r0; r < r1; ++r) {
      int b, h, i;
      row_coords(J, r, &b, &h, &i);
      int hk = h / group;
      int sq, skv;
      const float *qrow, *kbase, *vbase;
      int64_t orow; /* element offset of this row in the full output */
      if (J->cu) {
        int64_t T = J->cu[J->B];
        int start = J->cu[b];
        sq = skv = J->cu[b + 1] - start;
        qrow = J->q + ((int64_t)h * T + start + i) * d;
        kbase = J->k + ((int64_t)hk * T + start) * d;
        vbase = J->v + ((int64_t)hk * T + start) * d;
        orow = (int64_t)h * T + start + i;
      } else {
        sq = J->Sq;
        skv = J->Skv;
        qrow = J->q + (((int64_t)b * J->H + h) * sq + i) * d;
        kbase = J->k + ((int64_t)b * J->Hkv + hk) * (int64_t)skv * d;
        vbase = J->v + ((int64_t)b * J->Hkv + hk) * (int64_t)skv * d;
        orow = ((int64_t)b * J->H + h) * sq + i;
      }
      double* out = J->o + (J->rows ? r : orow) * d;
      double* lout = J->lse ? J->lse + (J->rows ? r : orow) : NULL;

      /* visible keys: jlo <= j < nvis; j < skv, j <= i + (skv - sq) when
         causal (or windowed), j > i + (skv - sq) - window with a window */
      int64_t nvis = skv;
      if (J->causal || J->window > 0) {
        int64_t lim = (int64_t)i + (skv - sq) + 1;
        if (lim < nvis) nvis = lim;
        if (nvis < 0) nvis = 0;
      }
      int64_t jlo = 0;
      if (J->window > 0) {
        jlo = (int64_t)i + (skv - sq) - J->window + 1;
        if (jlo < 0) jlo = 0;
      }
      const double sink = J->sinks ? J->sinks[h] : -INFINITY;
      if (nvis <= jlo) {
        for (int t = 0; t < d; ++t) out[t] = 0.0;
        if (lout) *lout = -INFINITY;
        if (lout && J->sinks) *lout = sink; /* l = exp(sink - sink) = 1 */
        continue;
      }
      const int64_t n = nvis - jlo;
      /* materialise the scaled scores of the row (s[j] is key jlo + j) */
      double m = -INFINITY;
      for (int64_t j = 0; j < n; ++j) {
        const float* krow = kbase + (jlo + j) * d;
        double dot = 0.0;
        for (int t = 0; t < d; ++t) dot += (double)qrow[t] * (double)krow[t];
        s[j] = J->scale * dot;
        if (s[j] > m) m = s[j];
      }
      if (J->sinks && sink > m) m = sink; /* m* = max(row max, sink) */
      /* safe softmax: p_j = exp(s_j - m), l = sum p_j (+ the sink's term) */
      double l = 0.0;
      for (int64_t j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
      }
      if (J->sinks) l += exp(sink - m);
      /* O = sum_j (p_j / l) v_j */
      for (int t = 0; t < d; ++t) acc[t] = 0.0;
      for (int64_t j = 0; j < n; ++j) {
        const double w = s[j] / l;
        const float* vrow = vbase + (jlo + j) * d;
        for (int t = 0; t < d; ++t) acc[t] += w * (double)vrow[t];
      }
      for (int t = 0; t < d; ++t) out[t] = acc[t];
      if (lout) *lout = m + log(l);
    }
  }
  free(s);
  free(acc);
  return NULL;
}

/*
 * q: [B,H,Sq,d]; k, v: [B,Hkv,Skv,d]; o: [B,H,Sq,d]; lse: [B,H,Sq] (may be NULL).
 * With cu_seqlens (B+1 int32 prefix sums, host memory) the tensors are packed:
 * q, o: [H,T,d]; k, v: [Hkv,T,d]; lse: [H,T], T = cu_seqlens[B]; each
 * sequence attends to itself (Sq_b = Skv_b); Sq, Skv are ignored.
 * rows: optional list of nrows (b, h, i) triples (i is the row inside its
 * sequence); then o is [nrows,d] and lse [nrows].
 * window: 0, or a sliding window of that many keys (the causal bound is
 * implied); sinks: NULL, or H per-query-head logits.
 * Returns 0 on success, 1 on invalid arguments, 3 when memory runs out.
 */
int oracle_attn_f64(const float* q, const float* k, const float* v, int B, int H, int Hkv,
                    int Sq, int Skv, int d, double scale, int causal,
                    const int32_t* cu_seqlens, const int64_t* rows, int64_t nrows, double* o,
                    double* lse, int nthreads, int window, const double* sinks) {
  if (B < 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0 || d <= 0 || !q || !k || !v || !o) return 1;
  if (window < 0) return 1;
  if (!cu_seqlens && (Sq < 0 || Skv < 0)) return 1;
  if (cu_seqlens) {
    if (cu_seqlens[0] != 0) return 1;
    for (int b = 0; b < B; ++b)
      if (cu_seqlens[b + 1] < cu_seqlens[b]) return 1;
  }
  int64_t all = cu_seqlens ? (int64_t)H * cu_seqlens[B] : (int64_t)B * H * Sq;
  if (!rows) nrows = all;
  if (rows) {
    for (int64_t r = 0; r < nrows; ++r) {
      int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
      int64_t lim = cu_seqlens ? (b >= 0 && b < B ? cu_seqlens[b + 1] - cu_seqlens[b] : 0) : Sq;
      if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= lim) return 1;
    }
  }
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  job_t* jobs = (job_t*)calloc((size_t)nthreads, sizeof(job_t));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !th) {
    free(jobs);
    free(th);
    return 3;
  }
  for (int t = 0; t < nthreads; ++t) {
    job_t* J = &jobs[t];
    J->q = q; J->k = k; J->v = v;
    J->B = B; J->H = H; J->Hkv = Hkv; J->Sq = Sq; J->Skv = Skv; J->d = d;
    J->causal = causal; J->scale = scale; J->cu = cu_seqlens;
    J->window = window; J->sinks = sinks;
    J->rows = rows; J->nrows = nrows; J->o = o; J->lse = lse;
    J->tid = t; J->nthreads = nthreads; J->status = 0;
  }
  int status = 0;
  int started = 0;
  for (int t = 1; t < nthreads; ++t) {
    if (pthread_create(&th[t], NULL, worker, &jobs[t]) != 0) break;
    started = t;
  }
  /* rows owned by threads that failed to start are done here, in order */
  for (int t = started + 1; t < nthreads; ++t) worker(&jobs[t]);
  worker(&jobs[0]);
  for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
  for (int t = 0; t < nthreads; ++t)
    if (jobs[t].status) status = jobs[t].status;
  free(jobs);
  free(th);
  return status;
}
