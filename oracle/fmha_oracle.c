/*
 * fmha_oracle.c -- plain CPU reference for exact scaled-dot-product attention
 * forward with per-row log-sum-exp, split-KV partials and their LSE-weighted
 * combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path never
 * calls it, and it shares no code, header or table with the HIP library.
 *
 * What it computes (the plain definition, in fp64, one output row at a time):
 *
 *   s_j   = scale * q_descale * k_descale * sum_d q[i,h,d] * k[j,hk,d]
 *   A     = keys j in [0, sk) allowed by the mask of row i
 *   m     = max_{j in A} s_j,   l = sum_{j in A} exp(s_j - m)
 *   O     = sum_{j in A} exp(s_j - m) / l * v_descale * v[j,hk,:]
 *   LSE   = m + ln(l)          (natural log of the sum of exp of scaled scores)
 *
 * Sources (the web pages on split-KV flash attention):
 *  - "Adds variable sequence lengths to the Hopper CuTe DSL FMHA example"
 *    (CUTLASS), section Interface: cumulative int32 sequence lengths
 *    [0, s0, s0+s1, ...], None for a fixed-length side, tensors packed along
 *    the sequence dimension; section Implementation: query rows of a sequence
 *    with no keys are not written; section Tests: output and LSE compared per
 *    sequence, bottom-right causal for different q/k lengths, window (128, 0),
 *    GQA 8:8 / 8:2 / 8:1.
 *  - "[FlyDSL] Enable FP8 FMHA split-K for short cached-prefix queries"
 *    (aiter), description and measurement: split-K partials followed by a split
 *    combine, FP8 e4m3 inputs with per-tensor scales, return_lse.
 *  - "[Cute,Fwd,Sm100] Support q_stage=1 for inference" (flash-attention),
 *    description: split KV across CTAs for inference-sized query counts.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *  - LSE is the natural log of sum_j exp(s_j) over allowed keys, s_j already
 *    scaled.
 *  - Bottom-right causal: key j is allowed for query i iff j <= i + sk - sq.
 *  - Window (wl, wr) is relative to that same diagonal d0 = i + sk - sq and
 *    inclusive: d0 - wl <= j <= d0 + wr; a negative bound is unbounded.
 *    Causal together with a window clamps wr to min(wr, 0) (0 if unbounded).
 *  - A row of a sequence with sk > 0 whose allowed set is empty gets O = 0 and
 *    LSE = -inf (the empty sum).
 *  - Rows of a sequence with sk == 0 are left untouched.
 *  - GQA: query head h reads kv head h / (Hq / Hkv).
 *  - FP8 is OCP e4m3fn (bias 7, no infinities, 0x7f / 0xff are NaN); the real
 *    value of a stored element is its decoded value times its tensor's descale.
 *  - Split s of sequence b covers keys [s*chunk, min((s+1)*chunk, sk_b));
 *    sequence b has ceil(sk_b / chunk) splits.  A split whose range is empty
 *    or fully masked for a row gives (O, LSE) = (0, -inf) for that row.
 *  - Combine of partials: L = max_s lse_s; if L = -inf then O = 0, LSE = -inf;
 *    otherwise LSE = L + ln sum_s exp(lse_s - L) and
 *    O = sum_s exp(lse_s - LSE) * O_s.
 *
 * Layouts (all contiguous, element strides implied):
 *   q   [Tq][Hq][Dqk]    k [Tk][Hkv][Dqk]    v [Tk][Hkv][Dv]
 *   out [Tq][Hq][Dv]  (double)                lse [Hq][Tq] (double)
 * where Tq = total query tokens (fixed length: batch * seqlen_q, sequence b
 * starting at token b * seqlen_q) and likewise for Tk.
 *
 * Parity pins for every function here live in tests/test_oracle_pins.py
 * (brute force in 50-digit arithmetic, torch fp64 SDPA, closed forms,
 * invariants, and planted-mistake checks).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_FP8_E4M3 = 3 };

/* ---- element decoding (format definitions, written out) ---------------- */

static double dec_f16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24); /* subnormal: m / 2^10 * 2^-14 */
  } else if (e == 31) {
    v = (m == 0) ? INFINITY : NAN;
  } else {
    v = ldexp(1.0 + (double)m / 1024.0, e - 15);
  }
  return sign ? -v : v;
}

static double dec_bf16(uint16_t b) {
  /* bf16 is the upper half of an IEEE binary32 */
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double dec_e4m3(uint8_t x) {
  int sign = (x >> 7) & 1;
  int e = (x >> 3) & 0xf;
  int m = x & 7;
  double v;
  if (e == 15 && m == 7) return NAN; /* e4m3fn has NaN only, no infinity */
  if (e == 0) {
    v = ldexp((double)m, -9); /* subnormal: m / 8 * 2^-6 */
  } else {
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  }
  return sign ? -v : v;
}

static double elem(const void* base, int dtype, int64_t idx) {
  switch (dtype) {
    case OR_F32: return (double)((const float*)base)[idx];
    case OR_F16: return dec_f16(((const uint16_t*)base)[idx]);
    case OR_BF16: return dec_bf16(((const uint16_t*)base)[idx]);
    case OR_FP8_E4M3: return dec_e4m3(((const uint8_t*)base)[idx]);
    default: return NAN;
  }
}

/* Decode n elements of a buffer to doubles (exported for the decoder pins). */
void oracle_decode(const void* base, int dtype, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = elem(base, dtype, i);
}

/* ---- sequence bookkeeping ----------------------------------------------- */

static int seq_start(const int32_t* cu, int fixed_len, int b) {
  return cu ? cu[b] : b * fixed_len;
}
static int seq_len(const int32_t* cu, int fixed_len, int b) {
  return cu ? cu[b + 1] - cu[b] : fixed_len;
}

/* Mask predicate for query i of a sequence with sq queries and sk keys.
 * wl, wr < 0 mean unbounded; causal has already been folded into wr. */
static int allowed(int i, int j, int sq, int sk, int wl, int wr) {
  int d0 = i + sk - sq; /* bottom-right aligned diagonal */
  if (j < 0 || j >= sk) return 0;
  if (wl >= 0 && j < d0 - wl) return 0;
  if (wr >= 0 && j > d0 + wr) return 0;
  return 1;
}

typedef struct {
  const void *q, *k, *v;
  int dtype;
  const int32_t *cu_q, *cu_k;
  int batch, seqlen_q, seqlen_k;
  int hq, hkv, dqk, dv;
  double scale, qs, ks, vs;
  int wl, wr;
} problem;

/* One output row: keys restricted to [klo, khi) on top of the mask.
 * An empty allowed set gives the row O = 0 and LSE = -inf. */
static void attend_row(const problem* P, int b, int h, int i, int klo, int khi,
                       double* scores, double* o_row, double* lse_out) {
  int qs0 = seq_start(P->cu_q, P->seqlen_q, b);
  int ks0 = seq_start(P->cu_k, P->seqlen_k, b);
  int sq = seq_len(P->cu_q, P->seqlen_q, b);
  int sk = seq_len(P->cu_k, P->seqlen_k, b);
  int hk = h / (P->hq / P->hkv);
  int64_t qrow = ((int64_t)(qs0 + i) * P->hq + h) * P->dqk;
  double m = -INFINITY;
  int any = 0;
  for (int j = klo; j < khi; ++j) {
    if (!allowed(i, j, sq, sk, P->wl, P->wr)) {
      scores[j - klo] = -INFINITY;
      continue;
    }
    int64_t krow = ((int64_t)(ks0 + j) * P->hkv + hk) * P->dqk;
    double dot = 0.0;
    for (int d = 0; d < P->dqk; ++d)
      dot += elem(P->q, P->dtype, qrow + d) * elem(P->k, P->dtype, krow + d);
    double s = P->scale * P->qs * P->ks * dot;
    scores[j - klo] = s;
    if (s > m) m = s;
    any = 1;
  }
  for (int e = 0; e < P->dv; ++e) o_row[e] = 0.0;
  if (!any) {
    *lse_out = -INFINITY;
    return;
  }
  double l = 0.0;
  for (int j = klo; j < khi; ++j) {
    if (scores[j - klo] == -INFINITY) continue;
    l += exp(scores[j - klo] - m);
  }
  for (int j = klo; j < khi; ++j) {
    if (scores[j - klo] == -INFINITY) continue;
    double p = exp(scores[j - klo] - m) / l;
    int64_t vrow = ((int64_t)(ks0 + j) * P->hkv + hk) * P->dv;
    for (int e = 0; e < P->dv; ++e)
      o_row[e] += p * P->vs * elem(P->v, P->dtype, vrow + e);
  }
  *lse_out = m + log(l);
}

/* Causal is the window's right bound clamped to the diagonal: min(wr, 0),
 * and 0 when the right bound is unbounded -- i.e. always 0. */
static int fold_causal(int causal, int wr) { return causal ? 0 : wr; }

static int check_problem(const problem* P) {
  if (!P->q || !P->k || !P->v) return -1;
  if (P->hq <= 0 || P->hkv <= 0 || P->hq % P->hkv) return -1;
  if (P->dqk <= 0 || P->dv <= 0 || P->batch < 0) return -1;
  if (P->dtype < OR_F32 || P->dtype > OR_FP8_E4M3) return -1;
  return 0;
}

static int total_tokens(const int32_t* cu, int fixed_len, int batch) {
  return cu ? cu[batch] : batch * fixed_len;
}

/* Core driver: every (b, h, i) row, keys limited by split (chunk > 0) or not. */
static int run(const problem* P, int chunk, int split, double* out, double* lse) {
  if (check_problem(P)) return -1;
  int tq = total_tokens(P->cu_q, P->seqlen_q, P->batch);
  int max_sk = 0;
  for (int b = 0; b < P->batch; ++b) {
    int sk = seq_len(P->cu_k, P->seqlen_k, b);
    if (sk > max_sk) max_sk = sk;
  }
  int nunits = P->batch * P->hq;
  int err = 0;
#pragma omp parallel
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)(max_sk > 0 ? max_sk : 1));
    if (!scores) {
#pragma omp atomic write
      err = -2;
    }
#pragma omp for schedule(dynamic, 1)
    for (int u = 0; u < nunits; ++u) {
      if (!scores) continue;
      int b = u / P->hq, h = u % P->hq;
      int sq = seq_len(P->cu_q, P->seqlen_q, b);
      int sk = seq_len(P->cu_k, P->seqlen_k, b);
      int qs0 = seq_start(P->cu_q, P->seqlen_q, b);
      if (sk == 0) continue; /* rows of a query sequence with no keys: untouched */
      int klo = 0, khi = sk;
      if (chunk > 0) {
        klo = split * chunk;
        khi = klo + chunk;
        if (klo > sk) klo = sk;
        if (khi > sk) khi = sk;
      }
      for (int i = 0; i < sq; ++i) {
        int64_t t = qs0 + i;
        attend_row(P, b, h, i, klo, khi, scores, out + (t * P->hq + h) * P->dv,
                   lse + (int64_t)h * tq + t);
      }
    }
    free(scores);
  }
  return err;
}

/*
 * Full attention forward.  out: [Tq][Hq][Dv] doubles, lse: [Hq][Tq] doubles.
 * Rows of sequences with no keys are not written.
 */
int oracle_attention(const void* q, const void* k, const void* v, int dtype,
                     const int32_t* cu_q, const int32_t* cu_k, int batch,
                     int seqlen_q, int seqlen_k, int hq, int hkv, int dqk, int dv,
                     double scale, double q_descale, double k_descale,
                     double v_descale, int causal, int window_left,
                     int window_right, double* out, double* lse) {
  problem P = {q, k, v, dtype, cu_q, cu_k, batch, seqlen_q, seqlen_k,
               hq, hkv, dqk, dv, scale, q_descale, k_descale, v_descale,
               window_left, fold_causal(causal, window_right)};
  return run(&P, 0, 0, out, lse);
}

/*
 * Partial result of one split: keys [split*chunk, min((split+1)*chunk, sk_b))
 * of every sequence b.  out_part: [Tq][Hq][Dv], lse_part: [Hq][Tq].  Rows
 * whose range is empty or fully masked get (0, -inf); rows of sequences with
 * no keys are not written.
 */
int oracle_split_attention(const void* q, const void* k, const void* v, int dtype,
                           const int32_t* cu_q, const int32_t* cu_k, int batch,
                           int seqlen_q, int seqlen_k, int hq, int hkv, int dqk,
                           int dv, double scale, double q_descale,
                           double k_descale, double v_descale, int causal,
                           int window_left, int window_right, int chunk,
                           int split, double* out_part, double* lse_part) {
  if (chunk <= 0 || split < 0) return -1;
  problem P = {q, k, v, dtype, cu_q, cu_k, batch, seqlen_q, seqlen_k,
               hq, hkv, dqk, dv, scale, q_descale, k_descale, v_descale,
               window_left, fold_causal(causal, window_right)};
  return run(&P, chunk, split, out_part, lse_part);
}

/*
 * LSE-weighted combine of split partials.
 *   o_part   [S][Tq][Hq][Dv]    lse_part [S][Hq][Tq]
 * Sequence b uses its first ceil(sk_b / chunk) splits; rows of sequences with
 * no keys are not written.
 */
int oracle_combine(const double* o_part, const double* lse_part, int num_splits,
                   int chunk, const int32_t* cu_q, const int32_t* cu_k,
                   int batch, int seqlen_q, int seqlen_k, int hq, int dv,
                   double* out, double* lse) {
  if (chunk <= 0 || num_splits <= 0) return -1;
  int tq = total_tokens(cu_q, seqlen_q, batch);
  for (int b = 0; b < batch; ++b) {
    int sq = seq_len(cu_q, seqlen_q, b);
    int sk = seq_len(cu_k, seqlen_k, b);
    int qs0 = seq_start(cu_q, seqlen_q, b);
    if (sk == 0) continue;
    int nsb = (sk + chunk - 1) / chunk;
    if (nsb > num_splits) return -1;
    for (int h = 0; h < hq; ++h) {
      for (int i = 0; i < sq; ++i) {
        int64_t t = qs0 + i;
        double L = -INFINITY;
        for (int s = 0; s < nsb; ++s) {
          double x = lse_part[((int64_t)s * hq + h) * tq + t];
          if (x > L) L = x;
        }
        double* o = out + (t * hq + h) * dv;
        if (L == -INFINITY) {
          for (int e = 0; e < dv; ++e) o[e] = 0.0;
          lse[(int64_t)h * tq + t] = -INFINITY;
          continue;
        }
        double sum = 0.0;
        for (int s = 0; s < nsb; ++s)
          sum += exp(lse_part[((int64_t)s * hq + h) * tq + t] - L);
        double total = L + log(sum);
        for (int e = 0; e < dv; ++e) o[e] = 0.0;
        for (int s = 0; s < nsb; ++s) {
          double w = exp(lse_part[((int64_t)s * hq + h) * tq + t] - total);
          const double* os = o_part + (((int64_t)s * tq + t) * hq + h) * dv;
          for (int e = 0; e < dv; ++e) o[e] += w * os[e];
        }
        lse[(int64_t)h * tq + t] = total;
      }
    }
  }
  return 0;
}

/*
 * Selected rows only: row n is (query token rows_t[n], query head rows_h[n]),
 * tokens in the packed indexing of q.  out_rows: [nrows][Dv], lse_rows:
 * [nrows].  A row of a sequence with no keys is left untouched; the same
 * per-row computation as oracle_attention.
 */
int oracle_attention_rows(const void* q, const void* k, const void* v, int dtype,
                          const int32_t* cu_q, const int32_t* cu_k, int batch,
                          int seqlen_q, int seqlen_k, int hq, int hkv, int dqk,
                          int dv, double scale, double q_descale, double k_descale,
                          double v_descale, int causal, int window_left,
                          int window_right, const int32_t* rows_t,
                          const int32_t* rows_h, int nrows, double* out_rows,
                          double* lse_rows) {
  problem P = {q, k, v, dtype, cu_q, cu_k, batch, seqlen_q, seqlen_k,
               hq, hkv, dqk, dv, scale, q_descale, k_descale, v_descale,
               window_left, fold_causal(causal, window_right)};
  if (check_problem(&P)) return -1;
  int max_sk = 0;
  for (int b = 0; b < batch; ++b) {
    int sk = seq_len(cu_k, seqlen_k, b);
    if (sk > max_sk) max_sk = sk;
  }
  int err = 0;
#pragma omp parallel
  {
    double* scores = (double*)malloc(sizeof(double) * (size_t)(max_sk > 0 ? max_sk : 1));
#pragma omp for schedule(dynamic, 1)
    for (int n = 0; n < nrows; ++n) {
      if (!scores) continue;
      int t = rows_t[n], h = rows_h[n];
      int b = 0;
      while (b < batch && seq_start(cu_q, seqlen_q, b) + seq_len(cu_q, seqlen_q, b) <= t) ++b;
      if (b >= batch || h < 0 || h >= hq) {
#pragma omp atomic write
        err = -1;
        continue;
      }
      int sk = seq_len(cu_k, seqlen_k, b);
      if (sk == 0) continue;
      int i = t - seq_start(cu_q, seqlen_q, b);
      attend_row(&P, b, h, i, 0, sk, scores, out_rows + (int64_t)n * dv, lse_rows + n);
    }
    free(scores);
  }
  return err;
}

/* Threads the OpenMP runtime will use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
