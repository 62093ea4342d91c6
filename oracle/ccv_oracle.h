/*
 * ccv_oracle.h -- plain CPU oracle for the causal depthwise conv1d forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
 * bench's cpu_baseline leg may load this library.  The GPU library never links
 * it and shares no code with it (no headers, helpers, tables or converters).
 *
 * What it computes (all arithmetic in fp64, single-threaded, one output at a time):
 *   z[b,c,t] = bias[c] + sum_{k=0}^{K-1} keep(t,k) * w[c,k] * X~[b,c,t-K+1+k]
 *   y        = z                      (no activation)
 *            = z / (1 + exp(-z))      (SiLU / swish)
 * following Ch.5 "Dao forward CUDA implementation", section "How adjacent
 * threads and chunks exchange history" (the stencil equation for z_i, with the
 * SiLU applied to the accumulator), and Ch.4 "Dao interface and source map",
 * section "Contract of the full-sequence interface" (argument table: weight is
 * ordered oldest -> current, bias is pre-activation, silu and swish are one
 * activation).  X~ is the input extended to the left by K-1 steps: the
 * initial_states row when given, zeros otherwise (Ch.5, section "Three kinds
 * of boundary handled separately").  keep(t,k) is 1 without seq_idx; with it,
 * a term counts only when its source position s = t-K+1+k is >= 0 and
 * seq_idx[b,s] == seq_idx[b,t] (same section, the seq_idx paragraph); a term
 * that does not count is skipped, never multiplied by zero.  With seq_idx and
 * initial_states together (a version limit of the pages' library, lifted here),
 * the history is the history of the row's first sequence: a term reaching left of
 * t = 0 counts when seq_idx[b,t] == seq_idx[b,0]; and final_states are the history
 * of the row's last sequence: an entry from another sequence is zero.
 *
 * Strides are in elements: offset(b,c,t) = b*s_B + c*s_C + t*s_L (Ch.4,
 * section "Why one shape still has two layouts", the offset equation).
 */
#ifndef CCV_ORACLE_H
#define CCV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage types.  The codes are the oracle's own. */
enum { ORA_F32 = 0, ORA_F16 = 1, ORA_BF16 = 2 };

typedef struct {
  int64_t B, C, L;
  int32_t K;               /* taps, >= 1 (the product accepts 2..4) */
  int32_t silu;            /* 0: identity, 1: SiLU */
  const void* x;           /* x[b,c,t] at x + b*xs[0] + c*xs[1] + t*xs[2] */
  int32_t x_dtype;
  int64_t xs[3];
  const void* w;           /* w[c,k] at w + c*K + k  (oldest -> current) */
  int32_t w_dtype;
  const void* bias;        /* NULL or bias[c], stored in w_dtype */
  const int32_t* seq;      /* NULL or seq[b,t] at seq + b*L + t */
  const void* init;        /* NULL or init[b,c,i] (i = 0..K-2, time ascending) */
  int64_t is[3];           /*   at init + b*is[0] + c*is[1] + i*is[2], x_dtype */
} ora_problem_t;

/* Exact value of one stored element as fp64. */
double ora_decode(const void* base, int32_t dtype, int64_t off);

/* The extended input X~[b,c,j] for j in [-(K-1), L-1]. */
double ora_xt(const ora_problem_t* p, int64_t b, int64_t c, int64_t j);

/* One output: y (after the activation), z (before it) and
 * sabs = |bias| + sum over kept terms of |w*X~|.  Returns 0, or -1 on bad indices. */
int ora_point(const ora_problem_t* p, int64_t b, int64_t c, int64_t t,
              double* y, double* z, double* sabs);

/* All outputs, written to y[(b*C+c)*L+t] and sabs[...] (either may be NULL). */
int ora_fwd(const ora_problem_t* p, double* y, double* sabs);

/* The same outputs as ora_fwd, computed by the same per-output function on up to
 * nthreads POSIX threads, each over a contiguous range of (b, c) rows: bit for bit
 * the single-threaded result (for timing the oracle on all host cores). */
int ora_fwd_threads(const ora_problem_t* p, double* y, double* sabs, int nthreads);

/* n sampled outputs; idx holds n (b,c,t) triples. */
int ora_points(const ora_problem_t* p, int64_t n, const int64_t* idx,
               double* y, double* sabs);

/* final_states[b,c,i] = X~[b,c,L-K+1+i] for i = 0..K-2, copied as raw bits of
 * x_dtype into fs[(b*C+c)*(K-1)+i] (Ch.5, section "Three kinds of boundary
 * handled separately": the last K-1 conv inputs, not activation outputs). */
int ora_final_states(const ora_problem_t* p, void* fs);

/* Rounding of the fp64 result to storage: o32 = RNE_f32(y); for 16-bit
 * storage, RNE of o32 to that format.  Writes n raw values of `dtype`. */
void ora_round_out(int32_t dtype, const double* y, int64_t n, void* out);

/* Converters, written from the IEEE-754 / bfloat16 definitions. */
float    ora_f64_to_f32(double v);
uint16_t ora_f32_to_bf16(float v);
uint16_t ora_f32_to_f16(float v);
double   ora_bf16_to_f64(uint16_t h);
double   ora_f16_to_f64(uint16_t h);
void     ora_f32_to_bf16_array(const float* in, uint16_t* out, int64_t n);
void     ora_f32_to_f16_array(const float* in, uint16_t* out, int64_t n);
void     ora_f16_to_f64_array(const uint16_t* in, double* out, int64_t n);
void     ora_bf16_to_f64_array(const uint16_t* in, double* out, int64_t n);

/* ---- backward ------------------------------------------------------------------
 * The gradient of the forward, written out by the chain rule (Ch.4 "Dao interface
 * and source map", section "How autograd links forward and backward": the
 * backward takes dout and, when the forward returned states, dfinal_states; it
 * returns dx, dweight, dbias and, with initial_states, their gradient; seq_idx
 * has none).  With z the pre-activation and X~ the extended input:
 *   dz[b,c,t]   = dout[b,c,t] * act'(z[b,c,t])      (SiLU': s(z) * (1 + z * (1 - s(z))))
 *   dX~[b,c,j]  = sum_k keep(t,k) w[c,k] dz[b,c,t] over t = j+K-1-k in [0, L)
 *                 + dfinal_states[b,c,j-(L-K+1)] when j >= L-K+1
 *   dx[b,c,t]   = dX~[b,c,t];   dinitial_states[b,c,i] = dX~[b,c,i-(K-1)]
 *   dw[c,k]     = sum_{b,t} keep(t,k) dz[b,c,t] X~[b,c,t-K+1+k];  db[c] = sum_{b,t} dz[b,c,t]
 * The error scales bound how far an fp32 evaluation may stray: for each gradient
 * element, the sum of the magnitudes of its terms, where each dz also carries
 * |dout| * S_z (the forward's sum of magnitudes of z). */
typedef struct {
  const void* dout;        /* dout[b,c,t] at dout + b*ds[0] + c*ds[1] + t*ds[2], x_dtype */
  int64_t ds[3];
  const void* dfs;         /* NULL or dfinal_states[b,c,i] at dfs + b*fs[0] + c*fs[1] + i*fs[2] */
  int64_t fs[3];
} ora_grad_t;

/* dx [B*C*L], dinit [B*C*(K-1)] (NULL when there are no initial_states), dw [C*K],
 * db [C], and their error scales ex, einit, ew, eb (same shapes; any may be NULL).
 * Returns 0, or -1 when scratch memory cannot be had. */
int ora_bwd(const ora_problem_t* p, const ora_grad_t* g, double* dx, double* dinit,
            double* dw, double* db, double* ex, double* einit, double* ew, double* eb);

/* Diagnostic binary32 mode: acc = bias (or 0), then acc = fmaf(w[c,k], X~, acc)
 * over the kept terms in ascending k; no activation.  Writes the binary32 sum. */
int ora_point_f32(const ora_problem_t* p, int64_t b, int64_t c, int64_t t, float* z);
int ora_fwd_f32(const ora_problem_t* p, float* z);            /* z[(b*C+c)*L+t] */
int ora_points_f32(const ora_problem_t* p, int64_t n, const int64_t* idx, float* z);

#ifdef __cplusplus
}
#endif
#endif
