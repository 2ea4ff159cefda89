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
 *
 * The whole decoder layer (Fleet reading note, TL;DR and Summary: about seven
 * operators per layer of a Qwen3-8B-shaped decoder; section 1, system scope:
 * grouped-query attention with 32 query and 8 key/value heads, RMSNorm,
 * residual adds, the SiLU-gated MLP) is, per layer, on the residual stream x:
 *
 *   n1  = bf16(rmsnorm(x) * w_attn)               rmsnorm(v) = v / sqrt(mean(v^2) + eps)
 *   qkv = bf16(f32(n1 . Wqkv^T))                  q: Hq heads, k and v: Hkv heads of hd values
 *   o   = bf16(attention(q, K|k, V|v))            per query head h, key/value head h / (Hq/Hkv),
 *                                                 over the T cached positions and the new one
 *   x1  = bf16(f32(x + f32(o . Wo^T)))
 *   n2  = bf16(rmsnorm(x1) * w_mlp)
 *   a   = bf16(f32(silu(g) * u)),  [g|u] = f32(n2 . Wgu^T)
 *   x'  = bf16(f32(x1 + f32(a . Wdown^T)))
 *
 * attention(q_h, K, V) = sum_t softmax_t(q_h . k_t / sqrt(hd)) v_t in double.
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


/* RMSNorm of each row of x [M][d] (bf16), times the weight w [d] (bf16):
 * out = bf16(f32(x / sqrt(mean(x^2) + eps) * w)), in double. */
void oracle_rmsnorm(int M, int d, const uint16_t* x, const uint16_t* w, double eps, uint16_t* out) {
  for (int m = 0; m < M; ++m) {
    const uint16_t* xm = x + (size_t)m * d;
    double ss = 0.0;
    for (int k = 0; k < d; ++k) ss += bf16_value(xm[k]) * bf16_value(xm[k]);
    const double inv = 1.0 / sqrt(ss / d + eps);
    for (int k = 0; k < d; ++k)
      out[(size_t)m * d + k] = oracle_bf16_from_float((float)(bf16_value(xm[k]) * inv * bf16_value(w[k])));
  }
}

/* Grouped-query decode attention for M sequences, one new token each.
 *   q       [M][Hq*hd]           the new token's queries (bf16)
 *   kc, vc  [M][Hkv][T][hd]      the T cached keys and values of each sequence (bf16)
 *   kn, vn  [M][Hkv*hd]          the new token's key and value (bf16), position T
 *   out     [M][Hq*hd]           bf16 of sum_t p_t v_t, p = softmax over t of q.k_t / sqrt(hd)
 * Query head h reads key/value head h / (Hq / Hkv).  Double throughout;
 * the softmax subtracts the maximum score. */
void oracle_gqa_decode(int M, int Hq, int Hkv, int hd, int T, const uint16_t* q, const uint16_t* kc,
                       const uint16_t* vc, const uint16_t* kn, const uint16_t* vn, uint16_t* out) {
  const int grp = Hq / Hkv;
  const double scale = 1.0 / sqrt((double)hd);
  double* s = (double*)malloc((size_t)(T + 1) * sizeof(double));
  double* acc = (double*)malloc((size_t)hd * sizeof(double));
  if (!s || !acc) abort();
  for (int m = 0; m < M; ++m)
    for (int h = 0; h < Hq; ++h) {
      const int g = h / grp;
      const uint16_t* qh = q + (size_t)m * Hq * hd + (size_t)h * hd;
      double mx = -INFINITY;
      for (int t = 0; t <= T; ++t) {
        const uint16_t* kt = t < T ? kc + (((size_t)m * Hkv + g) * T + t) * hd : kn + (size_t)m * Hkv * hd + (size_t)g * hd;
        double dot = 0.0;
        for (int i = 0; i < hd; ++i) dot += bf16_value(qh[i]) * bf16_value(kt[i]);
        s[t] = dot * scale;
        if (s[t] > mx) mx = s[t];
      }
      double l = 0.0;
      for (int t = 0; t <= T; ++t) {
        s[t] = exp(s[t] - mx);
        l += s[t];
      }
      for (int i = 0; i < hd; ++i) acc[i] = 0.0;
      for (int t = 0; t <= T; ++t) {
        const uint16_t* vt = t < T ? vc + (((size_t)m * Hkv + g) * T + t) * hd : vn + (size_t)m * Hkv * hd + (size_t)g * hd;
        for (int i = 0; i < hd; ++i) acc[i] += s[t] * bf16_value(vt[i]);
      }
      for (int i = 0; i < hd; ++i)
        out[(size_t)m * Hq * hd + (size_t)h * hd + i] = oracle_bf16_from_float((float)(acc[i] / l));
    }
  free(s);
  free(acc);
}

/* Residual add: out = bf16(f32(x + f32(y))), x bf16, y a projection's exact
 * (double) result; [n] elements. */
void oracle_residual(long n, const uint16_t* x, const double* y, uint16_t* out) {
  for (long i = 0; i < n; ++i)
    out[i] = oracle_bf16_from_float((float)(bf16_value(x[i]) + (double)(float)y[i]));
}
