/*
 * CPU oracle for the small-M decode GEMM and the per-layer projection chain.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table
 * or constant with the HIP library: it is a plain, slow, obviously correct
 * restatement of what the method computes.
 *
 * What it computes (Fleet, "Hierarchical Task-based Abstraction for
 * Megakernels on Multi-Die GPUs", reading note, Summary and section 4: each
 * Chiplet-task computes the sub-GEMM [M,K] x [K,N/8] of a decode projection
 * Y = X W; the news item "ROCm Low-Latency-GEMM" restates the same small-M
 * GEMM for the decode phase):
 *
 *   y[m][n] = sum_k x[m][k] * w[n][k]                     (1)
 *
 * with X row-major [M][K] and W stored K-major, [N][K] (one contiguous run of K
 * values per output column, the layout the per-chiplet weight pointer
 * base + k*(N/8)*K*sizeof(bf16) implies).  Inputs are bf16 bit patterns.  A
 * product of two bf16 values is exact in double, and the sum is accumulated in
 * double, in k order.  Alongside y the oracle returns a[m][n] = sum_k |x*w|,
 * the scale of the per-element tolerance.
 *
 * The chain (Fleet reading note, section 3f attack 2 and section 7b: gate and
 * up projections are concatenated and SiLU-gated; the projections of one
 * decoder layer run back to back) is, per layer l:
 *
 *   h1 = bf16(f32(x  . Wq^T))        Wq = the first q_cols rows of W_qkv
 *   h2 = bf16(f32(h1 . Wo^T))
 *   g|u = f32(h2 . Wgu^T)            g = columns [0,d_ff), u = [d_ff, 2 d_ff)
 *   a  = bf16(f32(silu(g) * u))      silu(v) = v / (1 + exp(-v)), in double
 *   x' = bf16(f32(a . Wdown^T))      the last layer also reports f32(a . Wdown^T)
 *
 * where f32() and bf16() round to nearest even.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* float -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN. */
uint16_t oracle_bf16_from_float(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  uint32_t keep = u >> 16;          /* truncated result */
  uint32_t rest = u & 0xffffu;      /* dropped bits */
  if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
  return (uint16_t)keep;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Equation (1).  y and absdot are [M][N] row-major; absdot may be NULL. */
void oracle_gemm(int M, int K, int N, const uint16_t* x, const uint16_t* w,
                 double* y, double* absdot) {
  long n;
#pragma omp parallel for schedule(dynamic, 16)
  for (n = 0; n < N; ++n) {
    const uint16_t* wn = w + (size_t)n * (size_t)K;
    for (int m = 0; m < M; ++m) {
      const uint16_t* xm = x + (size_t)m * (size_t)K;
      double s = 0.0, a = 0.0;
      for (int k = 0; k < K; ++k) {
        double p = bf16_value(xm[k]) * bf16_value(wn[k]);
        s += p;
        a += fabs(p);
      }
      y[(size_t)m * N + n] = s;
      if (absdot) absdot[(size_t)m * N + n] = a;
    }
  }
}

double oracle_silu(double v) { return v / (1.0 + exp(-v)); }

/* The SiLU gate of the chain on fp32 gate and up values: a = bf16(f32(silu(g) * u)),
 * silu in double (n values each). */
void oracle_silu_gate(long n, const float* g, const float* u, uint16_t* a) {
  for (long i = 0; i < n; ++i)
    a[i] = oracle_bf16_from_float((float)(oracle_silu((double)g[i]) * (double)u[i]));
}

/* One decoder-layer projection sequence (see the header).  All activations are
 * bf16 bits.  x_in [M][d], h1 [M][q], h2 [M][d], a [M][dff], x_out [M][d];
 * y_f32 [M][d] receives f32(a . Wdown^T) when not NULL.  The weights are
 * K-major: wq [q][d] (the first q rows of W_qkv), wo [d][q], wgu [2 dff][d],
 * wdown [d][dff]. */
void oracle_layer(int M, int d, int q, int dff, const uint16_t* x_in,
                  const uint16_t* wq, const uint16_t* wo, const uint16_t* wgu,
                  const uint16_t* wdown, uint16_t* h1, uint16_t* h2, uint16_t* a,
                  uint16_t* x_out, float* y_f32) {
  size_t big = (size_t)M * (size_t)(2 * dff > q ? (2 * dff > d ? 2 * dff : d) : (q > d ? q : d));
  double* y = (double*)malloc(big * sizeof(double));
  if (!y) abort();

  oracle_gemm(M, d, q, x_in, wq, y, NULL);
  for (size_t i = 0; i < (size_t)M * q; ++i) h1[i] = oracle_bf16_from_float((float)y[i]);

  oracle_gemm(M, q, d, h1, wo, y, NULL);
  for (size_t i = 0; i < (size_t)M * d; ++i) h2[i] = oracle_bf16_from_float((float)y[i]);

  oracle_gemm(M, d, 2 * dff, h2, wgu, y, NULL);
  for (int m = 0; m < M; ++m)
    for (int j = 0; j < dff; ++j) {
      float g = (float)y[(size_t)m * 2 * dff + j];
      float u = (float)y[(size_t)m * 2 * dff + dff + j];
      oracle_silu_gate(1, &g, &u, &a[(size_t)m * dff + j]);
    }

  oracle_gemm(M, dff, d, a, wdown, y, NULL);
  for (size_t i = 0; i < (size_t)M * d; ++i) {
    x_out[i] = oracle_bf16_from_float((float)y[i]);
    if (y_f32) y_f32[i] = (float)y[i];
  }
  free(y);
}
