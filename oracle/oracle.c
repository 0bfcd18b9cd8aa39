/*
 * oracle.c -- plain, slow, fp64 CPU definition of scaled-dot-product attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this
 * file; only the test suite, the smoke check and the CPU-baseline leg of the benchmark
 * do.  It shares no code, header or constant with the HIP library.
 *
 * What it computes (one row at a time, no tiling, no online softmax):
 *   "Profiling in PyTorch (part 3): attention" -- the naive causal attention section lists
 *   the five steps  scores = q.k^T ; scores *= scale ; masked positions -> -inf ;
 *   attn = softmax(scores, dim=-1) ; out = attn.v  and fixes the default scale to
 *   1/sqrt(head_dim).  The SDPA math-backend section of the same article adds the
 *   `_safe_softmax` rule: a row whose every position is masked must not produce NaN;
 *   this oracle returns a zero row for it and an LSE of -inf.
 *   The log-sum-exp of each row (natural log, in the scaled-score domain) is returned
 *   next to the output, as the FlashInfer DSA article's fused forward returns `lse`.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - mask polarity: a nonzero mask byte means "this key may be attended"; zero masks it.
 *   - causal alignment: top-left, key j is allowed for query i iff j <= i.
 *   - causal together with a mask: a key must pass both.
 *   - rank-3 [N,L,D] input is the rank-4 input with B=1, H=N (handled by the caller
 *     through strides; this file only sees (b,h,i,d) strides).
 *
 * Precision: every input element is decoded exactly to double (bf16 by a 16-bit shift
 * into the high half of an IEEE single, fp32 by conversion), all arithmetic is double,
 * dot products sum over d in ascending order, the softmax is the textbook two-pass form
 * (max, then exp and sum), and the probabilities are normalised before the product
 * with V, exactly in the order the five steps give.
 *
 * The backward (oracle_sdpa_bwd) is the derivative of the same function, written out with
 * the chain rule through the five steps: none of the pages defines a backward, but its
 * result is fixed by the forward; it is the step after the forward that the exported LSE
 * exists for (the fused forward of "[flashinfer] FlashInfer, Cake DSA 커널 최적화: Sparse
 * Attention 성능 2배 향상" returns `lse` for its backward, section 2).
 *
 * Parity pins: see tests/test_oracle_*.py (brute force, closed forms, invariants,
 * hand-derived golden cases, the library's fp64 math-backend SDPA; for the backward,
 * central finite differences of the forward oracle and the library's fp64 autograd).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2, ORACLE_F16 = 3 };

/* IEEE-754 binary16 from its fields: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Exponent 0 holds zero and the subnormals frac * 2^-24; exponent 31 holds the
 * infinities (frac 0) and NaNs; otherwise the value is (1024 + frac) * 2^(exp - 25). */
static double decode_f16(uint16_t h) {
  const int sign = h >> 15, ex = (h >> 10) & 0x1f, frac = h & 0x3ff;
  double mag;
  if (ex == 0) mag = ldexp((double)frac, -24);
  else if (ex == 31) mag = frac == 0 ? INFINITY : NAN;
  else mag = ldexp((double)(1024 + frac), ex - 25);
  return sign ? -mag : mag;
}

/* Exact decode of one element of a q/k/v tensor to double. */
static double load_elem(const void* base, int dtype, int64_t off) {
  if (dtype == ORACLE_F64) return ((const double*)base)[off];
  if (dtype == ORACLE_F32) return (double)((const float*)base)[off];
  if (dtype == ORACLE_F16) return decode_f16(((const uint16_t*)base)[off]);
  /* bf16: the 16 stored bits are the high half of an IEEE-754 binary32. */
  uint32_t bits = (uint32_t)((const uint16_t*)base)[off] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Is key j visible to query i of head (b,h)? (causal triangle and/or boolean mask) */
static int allowed(int is_causal, const uint8_t* mask, const int64_t* ms, int64_t b,
                   int64_t h, int64_t i, int64_t j) {
  if (is_causal && j > i) return 0;
  if (mask && mask[b * ms[0] + h * ms[1] + i * ms[2] + j * ms[3]] == 0) return 0;
  return 1;
}

/*
 * One output row: query i of head (b,h).  `s` and `p` are scratch of length Lk.
 * Writes D doubles to out_row and one double to *lse_out.
 */
static void one_row(int dtype, int64_t Lk, int64_t D, const void* q, const int64_t* qs,
                    const void* k, const int64_t* ks, const void* v, const int64_t* vs,
                    const uint8_t* mask, const int64_t* ms, const double* bias,
                    const int64_t* bs, int is_causal, double scale, int64_t b, int64_t h,
                    int64_t i, double* s, double* p, double* out_row, double* lse_out) {
  const int64_t qrow = b * qs[0] + h * qs[1] + i * qs[2];
  int any = 0;
  double m = -INFINITY;
  /* steps 1-3: scores of the visible keys, scaled after the dot product */
  for (int64_t j = 0; j < Lk; ++j) {
    if (!allowed(is_causal, mask, ms, b, h, i, j)) {
      s[j] = -INFINITY;
      continue;
    }
    const int64_t krow = b * ks[0] + h * ks[1] + j * ks[2];
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d)
      dot += load_elem(q, dtype, qrow + d * qs[3]) * load_elem(k, dtype, krow + d * ks[3]);
    s[j] = scale * dot;
    if (bias) { /* additive mask: a value added to the scaled score; -inf hides the key */
      s[j] += bias[b * bs[0] + h * bs[1] + i * bs[2] + j * bs[3]];
      if (s[j] == -INFINITY) continue;
    }
    if (!any || s[j] > m) m = s[j];
    any = 1;
  }
  if (!any) { /* every key masked: the safe softmax yields an all-zero row */
    for (int64_t d = 0; d < D; ++d) out_row[d] = 0.0;
    *lse_out = -INFINITY;
    return;
  }
  /* step 4: softmax over the visible keys, two passes (max above, exp+sum here) */
  double l = 0.0;
  for (int64_t j = 0; j < Lk; ++j) {
    p[j] = (s[j] == -INFINITY) ? 0.0 : exp(s[j] - m);
    l += p[j];
  }
  for (int64_t j = 0; j < Lk; ++j) p[j] /= l;
  /* step 5: out = attn . v */
  for (int64_t d = 0; d < D; ++d) {
    double acc = 0.0;
    for (int64_t j = 0; j < Lk; ++j)
      acc += p[j] * load_elem(v, dtype, b * vs[0] + h * vs[1] + j * vs[2] + d * vs[3]);
    out_row[d] = acc;
  }
  *lse_out = m + log(l);
}

/*
 * oracle_sdpa_fwd_bias -- the whole forward, or a chosen subset of its rows, with an optional
 * additive mask.
 *
 *   dtype        ORACLE_F32 / ORACLE_BF16 or ORACLE_F16 (raw 16-bit patterns) / ORACLE_F64,
 *                shared by q, k, v
 *   B,H,Lq,Lk,D  sizes; q is [B,H,Lq,D], k and v are [B,H,Lk,D] through the strides below
 *   qs,ks,vs     four element strides each, in (b, h, row, d) order; any value allowed
 *   mask, ms     optional byte mask addressed as mask[b*ms0 + h*ms1 + i*ms2 + j*ms3]
 *                (0 = masked); strides may be 0 to broadcast; NULL = no mask
 *   bias, bs     optional additive mask, doubles addressed as bias[b*bs0 + h*bs1 + i*bs2 +
 *                j*bs3] (strides may be 0 to broadcast), added to the scaled score of every
 *                visible key; -inf hides the key; NULL = none
 *   is_causal    nonzero: also hide keys j > i
 *   scale        multiplies q.k after the dot product
 *   rows, nrows  flat row ids r = (b*H + h)*Lq + i to evaluate; rows == NULL evaluates
 *                all B*H*Lq rows in that order (then nrows is ignored)
 *   out          [n, D] doubles, row-major, one row per evaluated row
 *   lse          [n] doubles (natural log), -inf for rows with no visible key
 *   nthreads     OpenMP threads (<= 0: the runtime's default)
 *
 * Returns 0 on success, 1 on a bad argument, 2 if scratch memory could not be allocated.
 */
int oracle_sdpa_fwd_bias(int dtype, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                         const void* q, const int64_t* qs, const void* k, const int64_t* ks,
                         const void* v, const int64_t* vs, const uint8_t* mask,
                         const int64_t* ms, const double* bias, const int64_t* bs,
                         int is_causal, double scale, const int64_t* rows, int64_t nrows,
                         double* out, double* lse, int nthreads) {
  if (dtype < ORACLE_F32 || dtype > ORACLE_F16) return 1;
  if (B < 0 || H < 0 || Lq < 0 || Lk < 0 || D < 0) return 1;
  if (!out || !lse || !qs || !ks || !vs || (mask && !ms) || (bias && !bs)) return 1;
  const int64_t n = rows ? nrows : B * H * Lq;
  if (n < 0) return 1;
  if (rows) {
    for (int64_t r = 0; r < n; ++r)
      if (rows[r] < 0 || rows[r] >= B * H * Lq) return 1;
  }
  int status = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)(Lk > 0 ? Lk : 1));
    double* p = (double*)malloc(sizeof(double) * (size_t)(Lk > 0 ? Lk : 1));
    if (!s || !p) {
#pragma omp atomic write
      status = 2;
    }
    /* every thread reaches the work-sharing loop; one without scratch only reports */
#pragma omp for schedule(dynamic, 8)
    for (int64_t r = 0; r < n; ++r) {
      if (!s || !p) continue;
      const int64_t flat = rows ? rows[r] : r;
      const int64_t i = flat % Lq;
      const int64_t bh = flat / Lq;
      one_row(dtype, Lk, D, q, qs, k, ks, v, vs, mask, ms, bias, bs, is_causal, scale, bh / H,
              bh % H, i,
              s, p, out + r * D, lse + r);
    }
    free(s);
    free(p);
  }
  return status;
}

/* oracle_sdpa_fwd -- oracle_sdpa_fwd_bias without an additive mask. */
int oracle_sdpa_fwd(int dtype, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                    const void* q, const int64_t* qs, const void* k, const int64_t* ks,
                    const void* v, const int64_t* vs, const uint8_t* mask, const int64_t* ms,
                    int is_causal, double scale, const int64_t* rows, int64_t nrows,
                    double* out, double* lse, int nthreads) {
  return oracle_sdpa_fwd_bias(dtype, B, H, Lq, Lk, D, q, qs, k, ks, v, vs, mask, ms, NULL, NULL,
                              is_causal, scale, rows, nrows, out, lse, nthreads);
}

/*
 * oracle_sdpa_bwd -- gradients of out = sdpa(q, k, v) for a given upstream gradient dout,
 * one head at a time, whole [Lq, Lk] matrices in fp64:
 *
 *   S   = scale * q.k^T (+ bias), hidden positions -inf   (the forward's steps 1-3)
 *   P   = row softmax of S; a row with every key hidden is all zero (safe softmax)
 *   dV  = P^T dout                                   (through step 5, out = P v)
 *   dP  = dout v^T
 *   dS  = P * (dP - rowsum(P * dP))                  (through step 4, the softmax Jacobian)
 *   dQ  = scale * dS k                               (through steps 1-2)
 *   dK  = scale * dS^T q
 *
 *   dtype, B..D, q/k/v and their strides, mask, is_causal, scale: as in oracle_sdpa_fwd
 *   bias, bs     optional additive mask as in oracle_sdpa_fwd_bias: S = scale * q.k^T + bias,
 *                -inf hides the key.  The bias is a constant of the forward (the SDPA call
 *                takes it as a given mask), so it shifts S and P but adds no term to the
 *                chain rule, and no gradient is produced for it; NULL = none
 *   dout, dos    upstream gradient [B,H,Lq,D] of q's dtype, four element strides
 *   dq           [B,H,Lq,D] doubles, row-major;  dk, dv: [B,H,Lk,D] doubles, row-major
 *   nthreads     OpenMP threads over heads (<= 0: the runtime's default)
 *
 * Returns 0 on success, 1 on a bad argument, 2 if scratch memory could not be allocated.
 */
int oracle_sdpa_bwd_bias(int dtype, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                         const void* q, const int64_t* qs, const void* k, const int64_t* ks,
                         const void* v, const int64_t* vs, const void* dout,
                         const int64_t* dos, const uint8_t* mask, const int64_t* ms,
                         const double* bias, const int64_t* bs, int is_causal, double scale,
                         double* dq, double* dk, double* dv, int nthreads) {
  if (dtype < ORACLE_F32 || dtype > ORACLE_F16) return 1;
  if (B < 0 || H < 0 || Lq < 0 || Lk < 0 || D < 0) return 1;
  if (!dq || !dk || !dv || !qs || !ks || !vs || !dos || (mask && !ms) || (bias && !bs))
    return 1;
  int status = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  const size_t mat = (size_t)(Lq > 0 ? Lq : 1) * (size_t)(Lk > 0 ? Lk : 1);
#pragma omp parallel
  {
    double* P = (double*)malloc(sizeof(double) * mat);
    double* dS = (double*)malloc(sizeof(double) * mat);
    if (!P || !dS) {
#pragma omp atomic write
      status = 2;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < B * H; ++bh) {
      if (!P || !dS) continue;
      const int64_t b = bh / H, h = bh % H;
      const int64_t qb = b * qs[0] + h * qs[1], kb = b * ks[0] + h * ks[1];
      const int64_t vb = b * vs[0] + h * vs[1], ob = b * dos[0] + h * dos[1];
      /* P: the forward's softmax, row by row */
      for (int64_t i = 0; i < Lq; ++i) {
        double* pr = P + i * Lk;
        double m = -INFINITY;
        int any = 0;
        for (int64_t j = 0; j < Lk; ++j) {
          if (!allowed(is_causal, mask, ms, b, h, i, j)) {
            pr[j] = -INFINITY;
            continue;
          }
          double dot = 0.0;
          for (int64_t d = 0; d < D; ++d)
            dot += load_elem(q, dtype, qb + i * qs[2] + d * qs[3]) *
                   load_elem(k, dtype, kb + j * ks[2] + d * ks[3]);
          pr[j] = scale * dot;
          if (bias) { /* the additive mask, as in the forward; -inf hides the key */
            pr[j] += bias[b * bs[0] + h * bs[1] + i * bs[2] + j * bs[3]];
            if (pr[j] == -INFINITY) continue;
          }
          if (!any || pr[j] > m) m = pr[j];
          any = 1;
        }
        double l = 0.0;
        for (int64_t j = 0; j < Lk; ++j) {
          pr[j] = (!any || pr[j] == -INFINITY) ? 0.0 : exp(pr[j] - m);
          l += pr[j];
        }
        for (int64_t j = 0; j < Lk; ++j) pr[j] = any ? pr[j] / l : 0.0;
      }
      /* dP = dout v^T, then dS = P (dP - rowsum(P dP)) */
      for (int64_t i = 0; i < Lq; ++i) {
        double rowsum = 0.0;
        for (int64_t j = 0; j < Lk; ++j) {
          double dot = 0.0;
          for (int64_t d = 0; d < D; ++d)
            dot += load_elem(dout, dtype, ob + i * dos[2] + d * dos[3]) *
                   load_elem(v, dtype, vb + j * vs[2] + d * vs[3]);
          dS[i * Lk + j] = dot;
          rowsum += P[i * Lk + j] * dot;
        }
        for (int64_t j = 0; j < Lk; ++j)
          dS[i * Lk + j] = P[i * Lk + j] * (dS[i * Lk + j] - rowsum);
      }
      /* dV = P^T dout, dK = scale dS^T q */
      for (int64_t j = 0; j < Lk; ++j)
        for (int64_t d = 0; d < D; ++d) {
          double av = 0.0, ak = 0.0;
          for (int64_t i = 0; i < Lq; ++i) {
            av += P[i * Lk + j] * load_elem(dout, dtype, ob + i * dos[2] + d * dos[3]);
            ak += dS[i * Lk + j] * load_elem(q, dtype, qb + i * qs[2] + d * qs[3]);
          }
          dv[(bh * Lk + j) * D + d] = av;
          dk[(bh * Lk + j) * D + d] = scale * ak;
        }
      /* dQ = scale dS k */
      for (int64_t i = 0; i < Lq; ++i)
        for (int64_t d = 0; d < D; ++d) {
          double a = 0.0;
          for (int64_t j = 0; j < Lk; ++j)
            a += dS[i * Lk + j] * load_elem(k, dtype, kb + j * ks[2] + d * ks[3]);
          dq[(bh * Lq + i) * D + d] = scale * a;
        }
    }
    free(P);
    free(dS);
  }
  return status;
}

/* oracle_sdpa_bwd -- oracle_sdpa_bwd_bias without an additive mask. */
int oracle_sdpa_bwd(int dtype, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                    const void* q, const int64_t* qs, const void* k, const int64_t* ks,
                    const void* v, const int64_t* vs, const void* dout, const int64_t* dos,
                    const uint8_t* mask, const int64_t* ms, int is_causal, double scale,
                    double* dq, double* dk, double* dv, int nthreads) {
  return oracle_sdpa_bwd_bias(dtype, B, H, Lq, Lk, D, q, qs, k, ks, v, vs, dout, dos, mask, ms,
                              NULL, NULL, is_causal, scale, dq, dk, dv, nthreads);
}

/* Threads the OpenMP runtime would use by default (reported next to CPU timings). */
int oracle_default_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
