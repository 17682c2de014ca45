/*
 * smla_ref.c -- fp64 CPU oracle for sparse MLA decode with split-K over the
 * top-k list.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * bench's CPU-baseline leg are the only callers.  It shares no code, header,
 * table or constant with the HIP library, and the HIP library never calls it.
 *
 * Sources (web pages; cited by title and section):
 *   [SPLITK] "The Moment of Truth: Validating Split-K Parallelization for
 *            Blackwell MLA Decode", section "The Split-K Imperative": the
 *            top-k candidate set of a query token is partitioned across
 *            blocks, each block produces a partial attention output, and a
 *            log-sum-exp combine merges the partials.
 *   [NSPLIT] "The Occupancy Hypothesis: How One Kernel Parameter Unlocked
 *            1.8x Decode Speedup on Blackwell", sections "The Occupancy
 *            Insight" (tokens per split = context / NSPLIT: 2875 at 46K with
 *            16 splits, 719 with 64) and "The Broader Context" (flash-decode
 *            partial + reduce).
 *
 * The operation itself (the pages give no formula; this is the plain
 * definition of softmax attention restricted to the selected rows):
 *   row width 576 bf16 = 512 latent columns followed by 64 rope columns;
 *   the value vector of a row is its first 512 columns;
 *   for token t, head h, with J = list entries j whose row r_j satisfies
 *   0 <= r_j < kv_rows (entries -1 or out of range carry zero weight; each
 *   remaining entry, duplicates included, is its own softmax term):
 *     s_j   = scale * sum_{d<576} q[t,h,d] * kv[r_j,d]
 *     O[c]  = sum_j exp(s_j - m) kv[r_j,c] / sum_j exp(s_j - m),  c < 512
 *     LSE   = m + ln sum_j exp(s_j - m),    m = max_j s_j
 *   and J empty gives O = 0, LSE = -inf.
 * All arithmetic is fp64 on the exact values of the bf16 inputs.  It is the
 * two-pass definition, not the online (streaming) softmax the kernel uses.
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdatomic.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define REF_D 576  /* q and cache row width */
#define REF_DV 512 /* value width: the first 512 columns of a row */

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static int row_valid(int32_t r, int64_t kv_rows) { return r >= 0 && (int64_t)r < kv_rows; }

/*
 * Softmax weights of one (token, head) over list entries [lo, hi) of idx_row.
 * w[j - lo] = exp(s_j - m) / Z for valid entries, 0 for masked ones.
 * Returns the number of valid entries; *lse_out = m + ln Z (or -inf).
 * Scratch: s must hold hi - lo doubles.
 */
static int weights_range(const uint16_t *q_row, const uint16_t *kv, int64_t kv_rows,
                         const int32_t *idx_row, int lo, int hi, double scale,
                         double *s, double *w, double *lse_out) {
  int nvalid = 0;
  double m = -INFINITY;
  for (int j = lo; j < hi; ++j) {
    int32_t r = idx_row[j];
    if (!row_valid(r, kv_rows)) {
      s[j - lo] = -INFINITY;
      continue;
    }
    const uint16_t *k = kv + (int64_t)r * REF_D;
    double dot = 0.0;
    for (int d = 0; d < REF_D; ++d) dot += bf16_to_double(q_row[d]) * bf16_to_double(k[d]);
    s[j - lo] = scale * dot;
    if (s[j - lo] > m) m = s[j - lo];
    ++nvalid;
  }
  if (nvalid == 0) {
    for (int j = lo; j < hi; ++j) w[j - lo] = 0.0;
    *lse_out = -INFINITY;
    return 0;
  }
  double z = 0.0;
  for (int j = lo; j < hi; ++j) {
    double e = row_valid(idx_row[j], kv_rows) ? exp(s[j - lo] - m) : 0.0;
    w[j - lo] = e;
    z += e;
  }
  for (int j = lo; j < hi; ++j) w[j - lo] /= z;
  *lse_out = m + log(z);
  return nvalid;
}

/* Attention of one (token, head) over list entries [lo, hi): o[512], *lse. */
static void attend_range(const uint16_t *q_row, const uint16_t *kv, int64_t kv_rows,
                         const int32_t *idx_row, int lo, int hi, double scale, double *s,
                         double *w, double *o, double *lse) {
  int nvalid = weights_range(q_row, kv, kv_rows, idx_row, lo, hi, scale, s, w, lse);
  for (int c = 0; c < REF_DV; ++c) o[c] = 0.0;
  if (nvalid == 0) return;
  for (int j = lo; j < hi; ++j) {
    if (!row_valid(idx_row[j], kv_rows)) continue;
    const uint16_t *v = kv + (int64_t)idx_row[j] * REF_D;
    double wj = w[j - lo];
    for (int c = 0; c < REF_DV; ++c) o[c] += wj * bf16_to_double(v[c]);
  }
}

/* Entries of split `split` out of `nsplit`: contiguous slices of
 * ceil(topk / nsplit) entries, the last one possibly short or empty
 * ([NSPLIT] "The Occupancy Insight": 46K tokens in 16 splits are 2875 per
 * split, in 64 splits 719, i.e. the ceiling of the quotient). */
static void split_range(int topk, int nsplit, int split, int *lo, int *hi) {
  int per = (topk + nsplit - 1) / nsplit;
  long a = (long)split * per, b = a + per;
  if (a > topk) a = topk;
  if (b > topk) b = topk;
  *lo = (int)a;
  *hi = (int)b;
}

/* ---------------------------------------------------------------- threads */

typedef struct {
  const uint16_t *q, *kv;
  int64_t kv_rows;
  const int32_t *idx;
  int64_t tokens;
  int heads, topk, nsplit; /* nsplit == 0: unsplit decode */
  double scale;
  double *out, *lse;
  atomic_long next;
  atomic_int oom;
} job_t;

static void *worker(void *arg) {
  job_t *jb = (job_t *)arg;
  int cap = jb->topk > 0 ? jb->topk : 1;
  double *s = (double *)malloc(sizeof(double) * cap);
  double *w = (double *)malloc(sizeof(double) * cap);
  if (!s || !w) {
    atomic_store(&jb->oom, 1);
    free(s);
    free(w);
    return NULL;
  }
  int ns = jb->nsplit > 0 ? jb->nsplit : 1;
  long units = (long)jb->tokens * jb->heads;
  for (;;) {
    long u = atomic_fetch_add(&jb->next, 1);
    if (u >= units) break;
    long t = u / jb->heads;
    int h = (int)(u % jb->heads);
    const uint16_t *q_row = jb->q + ((int64_t)t * jb->heads + h) * REF_D;
    const int32_t *idx_row = jb->idx + (int64_t)t * jb->topk;
    for (int sp = 0; sp < ns; ++sp) {
      int lo = 0, hi = jb->topk;
      if (jb->nsplit > 0) split_range(jb->topk, jb->nsplit, sp, &lo, &hi);
      /* unsplit: out [T,H,512], lse [T,H]; split: out [T,S,H,512], lse [T,S,H] */
      int64_t slot = ((int64_t)t * ns + sp) * jb->heads + h;
      attend_range(q_row, jb->kv, jb->kv_rows, idx_row, lo, hi, jb->scale, s, w,
                   jb->out + slot * REF_DV, jb->lse + slot);
    }
  }
  free(s);
  free(w);
  return NULL;
}

static int host_threads(void) {
  cpu_set_t set;
  if (sched_getaffinity(0, sizeof set, &set) == 0) {
    int n = CPU_COUNT(&set);
    if (n > 0) return n;
  }
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

static int run_job(job_t *jb, int nthreads) {
  if (nthreads <= 0) nthreads = host_threads();
  long units = (long)jb->tokens * jb->heads;
  if (units < nthreads) nthreads = units > 0 ? (int)units : 1;
  atomic_init(&jb->next, 0);
  atomic_init(&jb->oom, 0);
  pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
  if (!th) return -3;
  int started = 0;
  for (int i = 0; i < nthreads; ++i) {
    if (pthread_create(&th[i], NULL, worker, jb) != 0) break;
    ++started;
  }
  if (started == 0) worker(jb); /* no thread could start: run inline */
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  return atomic_load(&jb->oom) ? -3 : 0;
}

/* ------------------------------------------------------------- public API */

/* Number of threads the oracle uses when asked for 0 (the affinity mask). */
int smla_ref_threads(void) { return host_threads(); }

/*
 * Unsplit decode.  q [tokens, heads, 576] bf16 bits, kv [kv_rows, 576] bf16
 * bits, idx [tokens, topk] int32; out [tokens, heads, 512] fp64,
 * lse [tokens, heads] fp64.  nthreads 0 = every core in the affinity mask.
 * Returns 0, or -1 for a null pointer, -2 for a negative size, -3 for OOM.
 */
int smla_ref_decode(const uint16_t *q, const uint16_t *kv, int64_t kv_rows,
                    const int32_t *idx, int64_t tokens, int heads, int topk, float scale,
                    double *out, double *lse, int nthreads) {
  if (tokens < 0 || heads < 0 || topk < 0 || kv_rows < 0) return -2;
  if (tokens == 0 || heads == 0) return 0;
  if (!q || !out || !lse || (topk > 0 && !idx) || (kv_rows > 0 && !kv)) return -1;
  job_t jb = {.q = q, .kv = kv, .kv_rows = kv_rows, .idx = idx, .tokens = tokens,
              .heads = heads, .topk = topk, .nsplit = 0, .scale = (double)scale,
              .out = out, .lse = lse};
  return run_job(&jb, nthreads);
}

/*
 * Split partials ([SPLITK] "The Split-K Imperative"): split s covers list
 * entries [s*c, min(topk, (s+1)*c)), c = ceil(topk / nsplit); each split is
 * attention over its own entries alone (an empty split gives O = 0,
 * LSE = -inf).  part_o [tokens, nsplit, heads, 512], part_lse
 * [tokens, nsplit, heads], both fp64.
 */
int smla_ref_partial(const uint16_t *q, const uint16_t *kv, int64_t kv_rows,
                     const int32_t *idx, int64_t tokens, int heads, int topk, float scale,
                     int nsplit, double *part_o, double *part_lse, int nthreads) {
  if (tokens < 0 || heads < 0 || topk < 0 || kv_rows < 0) return -2;
  if (nsplit < 1) return -2;
  if (tokens == 0 || heads == 0) return 0;
  if (!q || !part_o || !part_lse || (topk > 0 && !idx) || (kv_rows > 0 && !kv)) return -1;
  job_t jb = {.q = q, .kv = kv, .kv_rows = kv_rows, .idx = idx, .tokens = tokens,
              .heads = heads, .topk = topk, .nsplit = nsplit, .scale = (double)scale,
              .out = part_o, .lse = part_lse};
  return run_job(&jb, nthreads);
}

/*
 * Log-sum-exp combine of split partials ([SPLITK] "The Split-K Imperative"):
 * per (token, head), M = max_s LSE_s; M = -inf gives O = 0, LSE = -inf;
 * otherwise w_s = exp(LSE_s - M), O = sum_s w_s O_s / sum_s w_s and
 * LSE = M + ln sum_s w_s.  Inputs as written by smla_ref_partial.
 */
int smla_ref_combine(const double *part_o, const double *part_lse, int64_t tokens, int heads,
                     int nsplit, double *out, double *lse) {
  if (tokens < 0 || heads < 0 || nsplit < 1) return -2;
  if (tokens == 0 || heads == 0) return 0;
  if (!part_o || !part_lse || !out || !lse) return -1;
  for (int64_t t = 0; t < tokens; ++t) {
    for (int h = 0; h < heads; ++h) {
      double mx = -INFINITY;
      for (int s = 0; s < nsplit; ++s) {
        double l = part_lse[(t * nsplit + s) * heads + h];
        if (l > mx) mx = l;
      }
      double *o = out + (t * heads + h) * REF_DV;
      for (int c = 0; c < REF_DV; ++c) o[c] = 0.0;
      if (mx == -INFINITY) {
        lse[t * heads + h] = -INFINITY;
        continue;
      }
      double wsum = 0.0;
      for (int s = 0; s < nsplit; ++s) {
        int64_t slot = (t * nsplit + s) * heads + h;
        double l = part_lse[slot];
        if (l == -INFINITY) continue;
        double w = exp(l - mx);
        wsum += w;
        const double *os = part_o + slot * REF_DV;
        for (int c = 0; c < REF_DV; ++c) o[c] += w * os[c];
      }
      for (int c = 0; c < REF_DV; ++c) o[c] /= wsum;
      lse[t * heads + h] = mx + log(wsum);
    }
  }
  return 0;
}

/*
 * Softmax weights of one (token, head): w[j] for every list entry j < topk
 * (0 for masked entries).  Returns the number of valid entries or a negative
 * status; *lse receives LSE.
 */
int smla_ref_weights(const uint16_t *q_row, const uint16_t *kv, int64_t kv_rows,
                     const int32_t *idx_row, int topk, float scale, double *w, double *lse) {
  if (topk < 0 || kv_rows < 0) return -2;
  if (!q_row || !lse || (topk > 0 && (!idx_row || !w)) || (kv_rows > 0 && !kv)) return -1;
  double *s = (double *)malloc(sizeof(double) * (topk > 0 ? topk : 1));
  if (!s) return -3;
  int n = weights_range(q_row, kv, kv_rows, idx_row, 0, topk, (double)scale, s, w, lse);
  free(s);
  return n;
}
