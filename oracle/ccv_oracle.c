/*
 * ccv_oracle.c -- plain, slow, single-threaded fp64 oracle for the causal
 * depthwise conv1d forward.  TEST INFRASTRUCTURE ONLY: loaded by the tests,
 * the smoke check and the bench's cpu_baseline leg, never by the product.
 *
 * Every output is computed on its own from the definition (see ccv_oracle.h
 * for the formula and its sources); there is no tiling, no reuse of partial
 * sums and no reordering of the terms.  Build: gcc -O2 -ffp-contract=off
 * (no fused multiply-add, no fast-math), so the fp64 arithmetic is exactly
 * what is written here.  ora_fwd_threads runs the same per-output loop over
 * disjoint ranges of (b, c) rows on several POSIX threads (for timing on all host
 * cores); every output is still computed by the one function, so the results
 * are the single-threaded ones bit for bit.
 */
#define _POSIX_C_SOURCE 200809L
#include "ccv_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---- storage decoding ----------------------------------------------------- */

/* bfloat16 is the upper 16 bits of an IEEE binary32: widen and reinterpret. */
double ora_bf16_to_f64(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double ora_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24);                 /* subnormal: m * 2^-24 */
  } else if (e == 31) {
    v = (m == 0) ? INFINITY : NAN;
  } else {
    v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/1024) * 2^(e-15) */
  }
  return sign ? -v : v;
}

double ora_decode(const void* base, int32_t dtype, int64_t off) {
  switch (dtype) {
    case ORA_F32: {
      float f;
      memcpy(&f, (const char*)base + off * 4, 4);
      return (double)f;
    }
    case ORA_F16: {
      uint16_t h;
      memcpy(&h, (const char*)base + off * 2, 2);
      return ora_f16_to_f64(h);
    }
    case ORA_BF16: {
      uint16_t h;
      memcpy(&h, (const char*)base + off * 2, 2);
      return ora_bf16_to_f64(h);
    }
  }
  return NAN;
}

static int elt_size(int32_t dtype) { return dtype == ORA_F32 ? 4 : 2; }

/* ---- rounding to storage ---------------------------------------------------- */

/* fp64 -> binary32: the C conversion rounds to nearest, ties to even, in the
 * default floating-point environment; overflow gives +-inf. */
float ora_f64_to_f32(double v) { return (float)v; }

/* Round-half-to-even of a non-negative double to an integer-valued double,
 * written out (no dependence on the current rounding mode). */
static double rne_int(double q) {
  double fl = floor(q);
  double frac = q - fl;
  if (frac > 0.5) return fl + 1.0;
  if (frac < 0.5) return fl;
  return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* binary32 -> bfloat16, round to nearest even.  The kept value is the upper
 * 16 bits; the dropped 16 bits decide: above half -> round up, below -> down,
 * exactly half -> towards the even kept pattern.  Rounding the largest finite
 * values up carries into the exponent and yields infinity, as it should. */
uint16_t ora_f32_to_bf16(float v) {
  uint32_t bits;
  memcpy(&bits, &v, 4);
  if (isnan(v)) return (uint16_t)((bits >> 16) | 0x0040);   /* quiet NaN */
  uint32_t upper = bits >> 16;
  uint32_t lower = bits & 0xffffu;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
  return (uint16_t)upper;
}

/* binary32 -> binary16, round to nearest even, by scaling |v| exactly into the
 * target's integer significand range and rounding that. */
uint16_t ora_f32_to_f16(float v) {
  uint32_t bits;
  memcpy(&bits, &v, 4);
  uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
  if (isnan(v)) return (uint16_t)(sign | 0x7e00u);
  double a = fabs((double)v);
  if (isinf(v)) return (uint16_t)(sign | 0x7c00u);
  /* Largest finite binary16 is 65504 = (2 - 2^-10) * 2^15; the midpoint to the
   * next step (65536) is 65520, and a tie there goes to the even pattern,
   * which is the overflow.  So |v| >= 65520 rounds to infinity. */
  if (a >= 65520.0) return (uint16_t)(sign | 0x7c00u);
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: value = q * 2^-24 with integer q in [0, 1024];
     * q == 1024 is the smallest normal, whose encoding is also 1024. */
    double q = rne_int(a * ldexp(1.0, 24));
    return (uint16_t)(sign | (uint16_t)q);
  }
  int e;
  (void)frexp(a, &e);          /* a = f * 2^e, f in [0.5, 1) -> a in [2^(e-1), 2^e) */
  int ue = e - 1;              /* unbiased exponent: a in [2^ue, 2^(ue+1)) */
  double m = rne_int(ldexp(a, 10 - ue));   /* significand in [1024, 2048] */
  if (m == 2048.0) { m = 1024.0; ue += 1; }
  if (ue > 15) return (uint16_t)(sign | 0x7c00u);
  return (uint16_t)(sign | (uint16_t)((ue + 15) << 10) | (uint16_t)(m - 1024.0));
}

void ora_f32_to_bf16_array(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = ora_f32_to_bf16(in[i]);
}
void ora_f32_to_f16_array(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = ora_f32_to_f16(in[i]);
}
void ora_f16_to_f64_array(const uint16_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = ora_f16_to_f64(in[i]);
}
void ora_bf16_to_f64_array(const uint16_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = ora_bf16_to_f64(in[i]);
}

void ora_round_out(int32_t dtype, const double* y, int64_t n, void* out) {
  for (int64_t i = 0; i < n; ++i) {
    float o32 = ora_f64_to_f32(y[i]);
    if (dtype == ORA_F32) {
      memcpy((char*)out + i * 4, &o32, 4);
    } else {
      uint16_t h = (dtype == ORA_BF16) ? ora_f32_to_bf16(o32) : ora_f32_to_f16(o32);
      memcpy((char*)out + i * 2, &h, 2);
    }
  }
}

/* ---- the method ------------------------------------------------------------ */

/* Extended input: X~[b,c,j] = x[b,c,j] for j >= 0; for -(K-1) <= j < 0 the
 * history to the left of the block, initial_states[b,c,j+K-1] (time
 * ascending, so index K-2 is the step just before t = 0), or zero without it. */
double ora_xt(const ora_problem_t* p, int64_t b, int64_t c, int64_t j) {
  if (j >= 0)
    return ora_decode(p->x, p->x_dtype, b * p->xs[0] + c * p->xs[1] + j * p->xs[2]);
  if (p->init == NULL) return 0.0;
  int64_t i = j + p->K - 1;
  return ora_decode(p->init, p->x_dtype, b * p->is[0] + c * p->is[1] + i * p->is[2]);
}

/* Sequence id of extended position j of row b: seq_idx[b, j] for j >= 0.  The
 * history left of t = 0 is the history of the row's first sequence, so it carries
 * seq_idx[b, 0]; without a history (or with L = 0) it has no id.  Returns 0 when
 * the position has no id. */
static int ora_pos_id(const ora_problem_t* p, int64_t b, int64_t j, int32_t* id) {
  if (j >= 0) {
    *id = p->seq[b * p->L + j];
    return 1;
  }
  if (p->init == NULL || p->L == 0) return 0;
  *id = p->seq[b * p->L];
  return 1;
}

/* Whether term k of output t counts: always without seq_idx; with it, when its
 * source position has the output's sequence id. */
static int ora_keep(const ora_problem_t* p, int64_t b, int64_t t, int k) {
  if (p->seq == NULL) return 1;
  int32_t id;
  if (!ora_pos_id(p, b, t - p->K + 1 + k, &id)) return 0;
  return id == p->seq[b * p->L + t];
}

/* Whether extended position j survives into final_states: always without seq_idx;
 * with it, final_states are the history of the row's last sequence, so a position
 * of another sequence is zero there. */
static int ora_final_kept(const ora_problem_t* p, int64_t b, int64_t j) {
  if (p->seq == NULL || p->L == 0) return 1;
  int32_t id;
  return ora_pos_id(p, b, j, &id) && id == p->seq[b * p->L + p->L - 1];
}

int ora_point(const ora_problem_t* p, int64_t b, int64_t c, int64_t t,
              double* y, double* z, double* sabs) {
  if (b < 0 || b >= p->B || c < 0 || c >= p->C || t < 0 || t >= p->L) return -1;
  const int K = p->K;
  double acc = 0.0, s = 0.0;
  if (p->bias != NULL) {
    double beta = ora_decode(p->bias, p->w_dtype, c);
    acc = beta;
    s = fabs(beta);
  }
  for (int k = 0; k < K; ++k) {
    int64_t src = t - K + 1 + k;              /* w[c,K-1] meets the current step */
    if (!ora_keep(p, b, t, k)) continue;      /* dropped */
    double term = ora_decode(p->w, p->w_dtype, c * K + k) * ora_xt(p, b, c, src);
    acc += term;
    s += fabs(term);
  }
  double out = acc;
  if (p->silu) out = acc / (1.0 + exp(-acc));
  if (y) *y = out;
  if (z) *z = acc;
  if (sabs) *sabs = s;
  return 0;
}

/* Every output of rows r0 .. r1-1 (row r = b*C + c), in order. */
static int ora_rows(const ora_problem_t* p, int64_t r0, int64_t r1, double* y, double* sabs) {
  for (int64_t r = r0; r < r1; ++r) {
    const int64_t b = r / p->C, c = r % p->C;
    for (int64_t t = 0; t < p->L; ++t) {
      int64_t o = r * p->L + t;
      double yy, ss;
      if (ora_point(p, b, c, t, &yy, NULL, &ss) != 0) return -1;
      if (y) y[o] = yy;
      if (sabs) sabs[o] = ss;
    }
  }
  return 0;
}

int ora_fwd(const ora_problem_t* p, double* y, double* sabs) {
  return ora_rows(p, 0, p->B * p->C, y, sabs);
}

typedef struct {
  const ora_problem_t* p;
  double* y;
  double* sabs;
  int64_t r0, r1;
  int status;
} ora_rows_job;

static void* ora_rows_thread(void* arg) {
  ora_rows_job* j = (ora_rows_job*)arg;
  j->status = ora_rows(j->p, j->r0, j->r1, j->y, j->sabs);
  return NULL;
}

int ora_fwd_threads(const ora_problem_t* p, double* y, double* sabs, int nthreads) {
  enum { MAX_THREADS = 256 };
  const int64_t rows = p->B * p->C;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > MAX_THREADS) nthreads = MAX_THREADS;
  if ((int64_t)nthreads > rows) nthreads = rows > 0 ? (int)rows : 1;
  ora_rows_job jobs[MAX_THREADS];
  pthread_t tid[MAX_THREADS];
  int created[MAX_THREADS];
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = (ora_rows_job){p, y, sabs, rows * i / nthreads, rows * (i + 1) / nthreads, 0};
    /* range 0 runs on the calling thread, and so does any range whose thread fails to start */
    created[i] = i > 0 && pthread_create(&tid[i], NULL, ora_rows_thread, &jobs[i]) == 0;
  }
  for (int i = 0; i < nthreads; ++i)
    if (!created[i]) ora_rows_thread(&jobs[i]);
  int status = 0;
  for (int i = 0; i < nthreads; ++i) {
    if (created[i]) pthread_join(tid[i], NULL);
    status |= jobs[i].status;
  }
  return status ? -1 : 0;
}

int ora_points(const ora_problem_t* p, int64_t n, const int64_t* idx,
               double* y, double* sabs) {
  for (int64_t i = 0; i < n; ++i) {
    double yy, ss;
    if (ora_point(p, idx[3 * i], idx[3 * i + 1], idx[3 * i + 2], &yy, NULL, &ss) != 0)
      return -1;
    if (y) y[i] = yy;
    if (sabs) sabs[i] = ss;
  }
  return 0;
}

int ora_final_states(const ora_problem_t* p, void* fs) {
  const int K = p->K;
  const int es = elt_size(p->x_dtype);
  for (int64_t b = 0; b < p->B; ++b)
    for (int64_t c = 0; c < p->C; ++c)
      for (int i = 0; i < K - 1; ++i) {
        int64_t j = p->L - K + 1 + i;         /* the last K-1 positions of X~ */
        char* dst = (char*)fs + ((b * p->C + c) * (K - 1) + i) * es;
        if (!ora_final_kept(p, b, j)) {
          memset(dst, 0, es);
        } else if (j >= 0) {
          memcpy(dst, (const char*)p->x + (b * p->xs[0] + c * p->xs[1] + j * p->xs[2]) * es, es);
        } else if (p->init != NULL) {
          int64_t ii = j + K - 1;
          memcpy(dst, (const char*)p->init + (b * p->is[0] + c * p->is[1] + ii * p->is[2]) * es, es);
        } else {
          memset(dst, 0, es);
        }
      }
  return 0;
}

/* ---- diagnostic binary32 mode ------------------------------------------------ */

/* The same stencil (same extended input, same dropped terms) evaluated as a
 * binary32 accumulation with fused multiply-adds: acc starts at the bias (zero
 * without one) and takes acc = fmaf(w[c,k], X~, acc) for the kept terms in
 * ascending k, each step rounded once.  Every stored value is exact in binary32,
 * so only the K roundings of the running sum differ from the fp64 result.  No
 * activation.  A diagnostic, not the parity reference: the pages fix only that
 * the accumulation is fp32, not its order. */
int ora_point_f32(const ora_problem_t* p, int64_t b, int64_t c, int64_t t, float* z) {
  if (b < 0 || b >= p->B || c < 0 || c >= p->C || t < 0 || t >= p->L) return -1;
  const int K = p->K;
  float acc = 0.0f;
  if (p->bias != NULL) acc = (float)ora_decode(p->bias, p->w_dtype, c);
  for (int k = 0; k < K; ++k) {
    int64_t src = t - K + 1 + k;
    if (!ora_keep(p, b, t, k)) continue;
    float wv = (float)ora_decode(p->w, p->w_dtype, c * K + k);
    float xv = (float)ora_xt(p, b, c, src);
    acc = fmaf(wv, xv, acc);
  }
  *z = acc;
  return 0;
}

int ora_fwd_f32(const ora_problem_t* p, float* z) {
  for (int64_t b = 0; b < p->B; ++b)
    for (int64_t c = 0; c < p->C; ++c)
      for (int64_t t = 0; t < p->L; ++t)
        if (ora_point_f32(p, b, c, t, &z[(b * p->C + c) * p->L + t]) != 0) return -1;
  return 0;
}

int ora_points_f32(const ora_problem_t* p, int64_t n, const int64_t* idx, float* z) {
  for (int64_t i = 0; i < n; ++i)
    if (ora_point_f32(p, idx[3 * i], idx[3 * i + 1], idx[3 * i + 2], &z[i]) != 0) return -1;
  return 0;
}

/* ---- backward ------------------------------------------------------------------ */

int ora_bwd(const ora_problem_t* p, const ora_grad_t* g, double* dx, double* dinit,
            double* dw, double* db, double* ex, double* einit, double* ew, double* eb) {
  const int K = p->K;
  const int64_t B = p->B, C = p->C, L = p->L, H = K - 1;
  double* dz = malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
  double* edz = malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
  if (!dz || !edz) {
    free(dz);
    free(edz);
    return -1;
  }
  for (int64_t c = 0; c < C; ++c) {
    for (int k = 0; k < K; ++k) {
      if (dw) dw[c * K + k] = 0.0;
      if (ew) ew[c * K + k] = 0.0;
    }
    if (db) db[c] = 0.0;
    if (eb) eb[c] = 0.0;
  }
  for (int64_t b = 0; b < B; ++b)
    for (int64_t c = 0; c < C; ++c) {
      /* dz over the row: the pre-activation z is recomputed from the forward's terms. */
      for (int64_t t = 0; t < L; ++t) {
        double y, z, sz;
        ora_point(p, b, c, t, &y, &z, &sz);
        double go = ora_decode(g->dout, p->x_dtype, b * g->ds[0] + c * g->ds[1] + t * g->ds[2]);
        double slope = 1.0;
        if (p->silu) {
          double s = 1.0 / (1.0 + exp(-z));
          slope = s * (1.0 + z * (1.0 - s));
        }
        dz[t] = go * slope;
        edz[t] = fabs(dz[t]) + fabs(go) * sz;     /* |dz| plus its sensitivity to z's error */
      }
      /* dX~ at every extended position j, from the outputs t = j+K-1-k that read it. */
      for (int64_t j = -H; j < L; ++j) {
        double acc = 0.0, e = 0.0;
        for (int k = 0; k < K; ++k) {
          int64_t t = j + K - 1 - k;
          if (t < 0 || t >= L || !ora_keep(p, b, t, k)) continue;
          double wk = ora_decode(p->w, p->w_dtype, c * K + k);
          acc += wk * dz[t];
          e += fabs(wk) * edz[t];
        }
        if (g->dfs != NULL && j >= L - H && ora_final_kept(p, b, j)) {
          int64_t i = j - (L - H);
          double v = ora_decode(g->dfs, p->x_dtype, b * g->fs[0] + c * g->fs[1] + i * g->fs[2]);
          acc += v;
          e += fabs(v);
        }
        if (j >= 0) {
          int64_t o = (b * C + c) * L + j;
          if (dx) dx[o] = acc;
          if (ex) ex[o] = e;
        } else if (p->init != NULL) {
          int64_t o = (b * C + c) * H + (j + H);
          if (dinit) dinit[o] = acc;
          if (einit) einit[o] = e;
        }
      }
      /* Parameter gradients: every kept (t, k) term, summed over b and t. */
      for (int64_t t = 0; t < L; ++t) {
        for (int k = 0; k < K; ++k) {
          if (!ora_keep(p, b, t, k)) continue;
          double xv = ora_xt(p, b, c, t - K + 1 + k);
          if (dw) dw[c * K + k] += dz[t] * xv;
          if (ew) ew[c * K + k] += edz[t] * fabs(xv);
        }
        if (db) db[c] += dz[t];
        if (eb) eb[c] += edz[t];
      }
    }
  free(dz);
  free(edz);
  return 0;
}
