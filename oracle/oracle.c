/*
 * CPU oracle for the forward pass of one sparse Mixture-of-Experts SwiGLU
 * feed-forward layer.
 *
 * TEST INFRASTRUCTURE.  Only the test-suite, the package smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU path never calls
 * it, links it or shares any code with it.
 *
 * What it computes (sources are the pages' titles and sections):
 *  - Router: "Mixture of experts: por que un modelo enorme apenas usa sus
 *    parametros" (josueisai), section "El router: la pieza que de verdad
 *    decide": a linear projection gives one score per expert, the k best are
 *    kept, and a softmax normalises only among the chosen ones.  The glossary
 *    "MoE (Mixture of Experts - Mezcla de Expertos)" (gotburnout), section 2
 *    diagram, writes the same as p = Softmax(TopK(W_g x)).
 *  - Experts: the glossary's section 3 pipeline, step 3: each chosen expert
 *    is a SwiGLU FFN.  Step 4 / diagram row 4: y = sum_i p_i * Expert_i(x).
 *  - Shared expert: glossary section 2, item 3 and diagram row 3: always
 *    active; added with coefficient 1 (it takes no router weight).
 *  - Packed layout: "Transformers v5 El Secreto Detras de los Modelos MoE Mas
 *    Rapidos" (smart-guide), section "La Solucion: WeightConverter": experts
 *    stacked on dim 0, the two input projections concatenated on dim 1, so one
 *    expert's gate_up block is [2F, D], first-listed projection first.
 *
 * Readings taken where the pages leave a step open:
 *  - The activated (SiLU) half is rows 0..F-1 of an expert's gate_up block;
 *    rows F..2F-1 multiply it elementwise.
 *  - The router's top-k decision is taken on fp32 logits (the precision the
 *    router's logits are defined in); ties go to the lower expert index; the
 *    chosen slots are ordered by descending logit.
 *  - No residual, no normalisation, no capacity limit: every token is
 *    computed by all of its k experts.
 *
 * Precision: bf16 inputs are widened exactly; every sum is accumulated in
 * double, in ascending index order; exp is the C library's double exp.  The
 * router logits are rounded once to fp32 before the selection.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static inline double bf(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

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

/* ------------------------------------------------------------------ router */

/* Logits of one token: l[e] = fp32( sum_d x[d] * W_g[e,d] + b[e] ). */
static void token_logits(const uint16_t* xt, const uint16_t* w_g, const float* bias,
                         int32_t D, int32_t E, float* l) {
  for (int32_t e = 0; e < E; ++e) {
    const uint16_t* w = w_g + (int64_t)e * D;
    double s = 0.0;
    for (int32_t d = 0; d < D; ++d) s += bf(xt[d]) * bf(w[d]);
    if (bias) s += (double)bias[e];
    l[e] = (float)s;
  }
}

/* Top-k by (key descending, index ascending), then softmax of the values l
 * over the chosen.  key == l unless a selection-only bias is in use.
 * margin = key_(k) - key_(k+1) with 1-based order statistics (+inf when k == E). */
static void token_topk_softmax(const float* key, const float* l, int32_t E, int32_t k,
                               unsigned char* taken, int32_t* ids, double* p, double* margin) {
  memset(taken, 0, (size_t)E);
  for (int32_t j = 0; j < k; ++j) {
    int32_t best = -1;
    for (int32_t e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || key[e] > key[best]) best = e; /* strict: the lower index wins ties */
    }
    taken[best] = 1;
    ids[j] = best;
  }
  if (margin) {
    if (k == E) {
      *margin = INFINITY;
    } else {
      int32_t next = -1;
      for (int32_t e = 0; e < E; ++e)
        if (!taken[e] && (next < 0 || key[e] > key[next])) next = e;
      *margin = (double)key[ids[k - 1]] - (double)key[next];
    }
  }
  double m = (double)l[ids[0]];
  for (int32_t j = 1; j < k; ++j)
    if ((double)l[ids[j]] > m) m = (double)l[ids[j]];
  double s[256];
  double tot = 0.0;
  for (int32_t j = 0; j < k; ++j) {
    s[j] = exp((double)l[ids[j]] - m);
    tot += s[j];
  }
  for (int32_t j = 0; j < k; ++j) p[j] = s[j] / tot;
}

/*
 * Route T tokens.
 *   x [T,D] bf16, w_g [E,D] bf16, bias [E] fp32 (NULL exactly when bias_mode == 0)
 *   bias_mode 1: the bias is part of the logit (it moves selection and weights).
 *   bias_mode 2: selection-only bias, the auxiliary-loss-free load balancer of
 *     the glossary "MoE (Mixture of Experts - Mezcla de Expertos)", section 2,
 *     item 4: the top-k is taken on key = fp32(l + b) (one fp32 add of the fp32
 *     logit and the bias), while the softmax runs over the plain logits l of
 *     the chosen experts, so the bias steers the load and never the weights.
 *   logits [T,E] fp32 out (the plain logits l) or NULL; ids [T,k] out;
 *   p [T,k] out; margin [T] out or NULL (taken on the selection keys)
 * Returns 0, or -1 on an invalid size or mode.
 */
int oracle_route_mode(const uint16_t* x, const uint16_t* w_g, const float* bias, int32_t bias_mode,
                      int64_t T, int32_t D, int32_t E, int32_t k, float* logits, int32_t* ids,
                      double* p, double* margin) {
  if (T < 0 || D <= 0 || E <= 0 || E > 256 || k <= 0 || k > E) return -1;
  if (bias_mode < 0 || bias_mode > 2 || (bias_mode != 0) != (bias != NULL)) return -1;
  int err = 0;
#pragma omp parallel
  {
    float* l = (float*)malloc(sizeof(float) * (size_t)E);
    float* key = (float*)malloc(sizeof(float) * (size_t)E);
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
    if (!l || !key || !taken) {
#pragma omp atomic write
      err = -2;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t t = 0; t < T; ++t) {
        token_logits(x + t * D, w_g, bias_mode == 1 ? bias : NULL, D, E, l);
        if (logits) memcpy(logits + t * E, l, sizeof(float) * (size_t)E);
        if (bias_mode == 2)
          for (int32_t e = 0; e < E; ++e) key[e] = l[e] + bias[e]; /* fp32 add */
        token_topk_softmax(bias_mode == 2 ? key : l, l, E, k, taken, ids + t * k, p + t * k,
                           margin ? margin + t : NULL);
      }
    }
    free(l);
    free(key);
    free(taken);
  }
  return err;
}

/* oracle_route_mode with the bias, when given, part of the logits (mode 1). */
int oracle_route(const uint16_t* x, const uint16_t* w_g, const float* bias, int64_t T, int32_t D,
                 int32_t E, int32_t k, float* logits, int32_t* ids, double* p, double* margin) {
  return oracle_route_mode(x, w_g, bias, bias ? 1 : 0, T, D, E, k, logits, ids, p, margin);
}

/* ----------------------------------------------------------------- experts */

/*
 * OCP 8-bit floating point E4M3 ("fn": no infinities), the format of the
 * quantised expert weights: sign bit, 4 exponent bits with bias 7, 3 mantissa
 * bits.  Exponent field 0 holds the subnormals m * 2^-9; S.1111.111 is NaN.
 * Per-expert quantised weights: "Mixture of Experts optimiza Transformers y
 * LLMs", section on the resources the method needs, and "Transformers v5 El
 * Secreto Detrás de los Modelos MoE Más Rápidos", section on its limits, name
 * per-expert quantisation without a format; this one is the reading taken.
 */
static double e4m3(uint8_t c) {
  const int sign = c >> 7, ex = (c >> 3) & 15, man = c & 7;
  double v;
  if (ex == 15 && man == 7) return NAN;
  if (ex == 0)
    v = ldexp((double)man, -9);
  else
    v = ldexp(1.0 + man / 8.0, ex - 7);
  return sign ? -v : v;
}

/* One expert matrix, row-major with `cols` columns: bf16 words, or (scale
 * != NULL) E4M3 bytes whose row r stands for e4m3(q[r][c]) * scale[r]. */
typedef struct {
  const void* w;
  const float* scale;
  int64_t cols;
} wmat;

static wmat wm(const void* base, const float* scale, int64_t row0, int64_t cols) {
  wmat m;
  m.cols = cols;
  m.scale = scale ? scale + row0 : NULL;
  m.w = scale ? (const void*)((const uint8_t*)base + row0 * cols)
              : (const void*)((const uint16_t*)base + row0 * cols);
  return m;
}

/* sum_c W[r][c] * v[c] with every weight dequantised exactly in double
 * (an E4M3 value times an fp32 scale needs 4 + 24 significant bits). */
static double row_dot(const wmat* m, int64_t r, const double* v) {
  double s = 0.0;
  if (m->scale) {
    const uint8_t* q = (const uint8_t*)m->w + r * m->cols;
    const double sc = (double)m->scale[r];
    for (int64_t c = 0; c < m->cols; ++c) s += e4m3(q[c]) * sc * v[c];
  } else {
    const uint16_t* b = (const uint16_t*)m->w + r * m->cols;
    for (int64_t c = 0; c < m->cols; ++c) s += bf(b[c]) * v[c];
  }
  return s;
}

/* yt[o] += coef * sum_f W_down[o,f] * h[f],  h[f] = SiLU(g_f) * u_f,
 * g_f = W_gu[f,:] . x,  u_f = W_gu[F+f,:] . x,  SiLU(g) = g / (1 + exp(-g)). */
static void swiglu_accumulate(const wmat* gu, const wmat* dn, int32_t F, int32_t D,
                              const double* xd, double* h, double coef, double* yt, int64_t* macs) {
  for (int32_t f = 0; f < F; ++f) {
    const double g = row_dot(gu, f, xd);
    const double u = row_dot(gu, F + f, xd);
    *macs += 2 * (int64_t)D;
    h[f] = g / (1.0 + exp(-g)) * u;
  }
  for (int32_t o = 0; o < D; ++o) {
    *macs += F;
    yt[o] += coef * row_dot(dn, o, h);
  }
}

/*
 * Expert outputs for n_tokens tokens given their routing, for one shard of
 * the experts (expert parallelism: "Mixture of Experts optimiza Transformers
 * y LLMs", section "Expert Parallelism"; "Transformers v5 El Secreto Detrás
 * de los Modelos MoE Más Rápidos", section "Paralelismo de Expertos"): only
 * the slots routed to experts e0 .. e0+n_local-1 contribute, and w_gate_up /
 * w_down hold just those n_local experts.  The shards' outputs add up to the
 * layer's (the shared expert is added by whichever call passes it).
 *   x [T,D] bf16 (rows picked by tokens[], or rows 0..n_tokens-1 when tokens is NULL)
 *   w_gate_up [n_local,2F,D], w_down [n_local,D,F]; ws_gate_up [2Fs,D], ws_down [D,Fs] or NULL
 *   fp8 == 0: those are bf16.  fp8 == 1: they are E4M3 bytes, and sgu [n_local,2F],
 *     sdn [n_local,D], ssgu [2Fs], ssdn [D] are the fp32 scales of their rows
 *   ids [*,k] (global expert ids), p [*,k]: the routing rows of the same tokens (indexed by token id)
 *   y [n_tokens, D] double out; macs: total multiply-adds performed (may be NULL)
 * Slots are accumulated in order j = 0..k-1, the shared expert last.
 */
int oracle_experts_q(const uint16_t* x, const void* w_gate_up, const void* w_down,
                     const void* ws_gate_up, const void* ws_down, int32_t fp8, const float* sgu,
                     const float* sdn, const float* ssgu, const float* ssdn, int32_t D, int32_t E,
                     int32_t e0, int32_t n_local, int32_t F, int32_t k, int32_t Fs,
                     const int32_t* ids, const double* p, const int64_t* tokens, int64_t n_tokens,
                     double* y, int64_t* macs) {
  if (D <= 0 || E <= 0 || F <= 0 || k <= 0 || k > E || Fs < 0 || n_tokens < 0) return -1;
  if (e0 < 0 || n_local < 0 || e0 + n_local > E) return -1;
  if (Fs > 0 && (!ws_gate_up || !ws_down)) return -1;
  if (fp8 != 0 && fp8 != 1) return -1;
  if (fp8 && (!sgu || !sdn || (Fs > 0 && (!ssgu || !ssdn)))) return -1;
  if (!fp8) sgu = sdn = ssgu = ssdn = NULL;
  int err = 0;
  int64_t total = 0;
  int32_t hmax = F > Fs ? F : Fs;
#pragma omp parallel reduction(+ : total)
  {
    double* xd = (double*)malloc(sizeof(double) * (size_t)D);
    double* h = (double*)malloc(sizeof(double) * (size_t)hmax);
    if (!xd || !h) {
#pragma omp atomic write
      err = -2;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t i = 0; i < n_tokens; ++i) {
        int64_t t = tokens ? tokens[i] : i;
        const uint16_t* xt = x + t * D;
        double* yt = y + i * D;
        for (int32_t d = 0; d < D; ++d) xd[d] = bf(xt[d]);
        for (int32_t d = 0; d < D; ++d) yt[d] = 0.0;
        for (int32_t j = 0; j < k; ++j) {
          int32_t e = ids[t * k + j] - e0; /* index inside this shard */
          if (e < 0 || e >= n_local) continue; /* another shard's expert */
          const wmat gu = wm(w_gate_up, sgu, (int64_t)e * 2 * F, D);
          const wmat dn = wm(w_down, sdn, (int64_t)e * D, F);
          swiglu_accumulate(&gu, &dn, F, D, xd, h, p[t * k + j], yt, &total);
        }
        if (Fs > 0) {
          const wmat gu = wm(ws_gate_up, ssgu, 0, D);
          const wmat dn = wm(ws_down, ssdn, 0, Fs);
          swiglu_accumulate(&gu, &dn, Fs, D, xd, h, 1.0, yt, &total);
        }
      }
    }
    free(xd);
    free(h);
  }
  if (macs) *macs = total;
  return err;
}

/* oracle_experts_q with bf16 weights. */
int oracle_experts_shard(const uint16_t* x, const uint16_t* w_gate_up, const uint16_t* w_down,
                         const uint16_t* ws_gate_up, const uint16_t* ws_down, int32_t D, int32_t E,
                         int32_t e0, int32_t n_local, int32_t F, int32_t k, int32_t Fs,
                         const int32_t* ids, const double* p, const int64_t* tokens,
                         int64_t n_tokens, double* y, int64_t* macs) {
  return oracle_experts_q(x, w_gate_up, w_down, ws_gate_up, ws_down, 0, NULL, NULL, NULL, NULL, D,
                          E, e0, n_local, F, k, Fs, ids, p, tokens, n_tokens, y, macs);
}

/* E4M3 decode of n codes (exposed for the tests). */
void oracle_e4m3_decode(const uint8_t* codes, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3(codes[i]);
}

/* Expert outputs with every expert present (the unsharded layer). */
int oracle_experts(const uint16_t* x, const uint16_t* w_gate_up, const uint16_t* w_down,
                   const uint16_t* ws_gate_up, const uint16_t* ws_down, int32_t D, int32_t E,
                   int32_t F, int32_t k, int32_t Fs, const int32_t* ids, const double* p,
                   const int64_t* tokens, int64_t n_tokens, double* y, int64_t* macs) {
  return oracle_experts_shard(x, w_gate_up, w_down, ws_gate_up, ws_down, D, E, 0, E, F, k, Fs, ids,
                              p, tokens, n_tokens, y, macs);
}

/* ---------------------------------------------------------------- backward */

/*
 * Backward pass of the layer for a given routing: the gradients of the scalar
 * sum_t <dy[t], y[t]> with respect to x, the router weight (and a bias inside
 * the logits), and every expert weight.  The pages' training sections ("Mixture
 * of Experts optimiza Transformers y LLMs", section on training; "Transformers
 * v5 El Secreto Detrás de los Modelos MoE Más Rápidos", section "Entrenamiento
 * MoE") give no formulas, so this is the chain rule of the forward pass above:
 *   O_j = W_down[e_j] h_j,  y = sum_j p_j O_j (+ shared),  p = softmax over the
 *   chosen logits.  The top-k choice is piecewise constant and passes no
 *   gradient; the softmax gives dl_j = p_j (dp_j - sum_i p_i dp_i) with
 *   dp_j = <dy, O_j> on the chosen logits, 0 on the others.
 *   SwiGLU: h = SiLU(g) u, SiLU'(g) = s (1 + g (1 - s)), s = 1 / (1 + e^-g).
 * Inputs: bf16 x [T,D], w_g [E,D], w_gate_up [E,2F,D], w_down [E,D,F], shared
 * ws_gate_up [2Fs,D], ws_down [D,Fs] (or NULL); ids/p [T,k] (the routing);
 * dy fp32 [T,D].  bias_mode: 1 when a bias is part of the logits (then dbias
 * gets sum_t dl[t,e]); otherwise dbias is zero (a selection-only bias passes
 * no gradient).  Outputs (double, overwritten): dx [T,D], dwg [E,D], dbias [E]
 * (or NULL), dwgu [E,2F,D], dwdn [E,D,F], dwsgu [2Fs,D], dwsdn [D,Fs] (NULL
 * without a shared expert), dp [T,k] (or NULL).  Weight gradients are summed
 * over tokens in ascending order.  Returns 0, -1 on invalid sizes, -2 on
 * allocation failure.
 */
int oracle_backward(const uint16_t* x, const uint16_t* w_g, const uint16_t* w_gate_up,
                    const uint16_t* w_down, const uint16_t* ws_gate_up, const uint16_t* ws_down,
                    int64_t T, int32_t D, int32_t E, int32_t F, int32_t k, int32_t Fs,
                    int32_t bias_mode, const int32_t* ids, const double* p, const float* dy,
                    double* dx, double* dwg, double* dbias, double* dwgu, double* dwdn,
                    double* dwsgu, double* dwsdn, double* dp_out) {
  if (T < 0 || D <= 0 || E <= 0 || F <= 0 || k <= 0 || k > E || Fs < 0) return -1;
  if (Fs > 0 && (!ws_gate_up || !ws_down || !dwsgu || !dwsdn)) return -1;
  for (int64_t a = 0; a < T * k; ++a)
    if (ids[a] < 0 || ids[a] >= E) return -1;
  const int64_t S = k + (Fs > 0 ? 1 : 0); /* slots per token, the shared expert last */
  const int32_t Fm = F > Fs ? F : Fs;
  /* per (token, slot): h, dg, du (Fm each), and the slot's dO scale and dl */
  double* hs = (double*)malloc(sizeof(double) * (size_t)(T * S * Fm + 1));
  double* dgs = (double*)malloc(sizeof(double) * (size_t)(T * S * Fm + 1));
  double* dus = (double*)malloc(sizeof(double) * (size_t)(T * S * Fm + 1));
  double* dls = (double*)malloc(sizeof(double) * (size_t)(T * k + 1));
  if (!hs || !dgs || !dus || !dls) {
    free(hs); free(dgs); free(dus); free(dls);
    return -2;
  }
  int err = 0;
  /* pass 1, per token: forward recomputation, dp, dl, SwiGLU backward, dx */
#pragma omp parallel
  {
    double* xd = (double*)malloc(sizeof(double) * (size_t)D);
    double* g = (double*)malloc(sizeof(double) * (size_t)Fm);
    double* u = (double*)malloc(sizeof(double) * (size_t)Fm);
    double* dpv = (double*)malloc(sizeof(double) * (size_t)k);
    if (!xd || !g || !u || !dpv) {
#pragma omp atomic write
      err = -2;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t t = 0; t < T; ++t) {
        for (int32_t d = 0; d < D; ++d) xd[d] = bf(x[t * D + d]);
        const float* dyt = dy + t * D;
        double* dxt = dx + t * D;
        for (int32_t d = 0; d < D; ++d) dxt[d] = 0.0;
        for (int64_t j = 0; j < S; ++j) {
          const int shared_slot = j == k;
          const int32_t e = shared_slot ? 0 : ids[t * k + j];
          const int32_t Fj = shared_slot ? Fs : F;
          const uint16_t* gu = shared_slot ? ws_gate_up : w_gate_up + (int64_t)e * 2 * F * D;
          const uint16_t* dn = shared_slot ? ws_down : w_down + (int64_t)e * D * F;
          const double coef = shared_slot ? 1.0 : p[t * k + j];
          double* h = hs + (t * S + j) * Fm;
          double* dg = dgs + (t * S + j) * Fm;
          double* du = dus + (t * S + j) * Fm;
          for (int32_t f = 0; f < Fj; ++f) {
            double a = 0.0, b = 0.0;
            for (int32_t d = 0; d < D; ++d) a += bf(gu[(int64_t)f * D + d]) * xd[d];
            for (int32_t d = 0; d < D; ++d) b += bf(gu[(int64_t)(Fj + f) * D + d]) * xd[d];
            g[f] = a;
            u[f] = b;
            h[f] = a / (1.0 + exp(-a)) * b;
          }
          /* dp_j = <dy, O_j> and dh = W_down^T (coef dy) */
          if (!shared_slot) {
            double s = 0.0;
            for (int32_t d = 0; d < D; ++d) {
              double o = 0.0;
              for (int32_t f = 0; f < Fj; ++f) o += bf(dn[(int64_t)d * Fj + f]) * h[f];
              s += (double)dyt[d] * o;
            }
            dpv[j] = s;
          }
          for (int32_t f = 0; f < Fj; ++f) {
            double dh = 0.0;
            for (int32_t d = 0; d < D; ++d) dh += coef * (double)dyt[d] * bf(dn[(int64_t)d * Fj + f]);
            const double sg = 1.0 / (1.0 + exp(-g[f]));
            dg[f] = dh * u[f] * sg * (1.0 + g[f] * (1.0 - sg));
            du[f] = dh * g[f] * sg;
          }
          for (int32_t d = 0; d < D; ++d) {
            double v = 0.0;
            for (int32_t f = 0; f < Fj; ++f)
              v += dg[f] * bf(gu[(int64_t)f * D + d]) + du[f] * bf(gu[(int64_t)(Fj + f) * D + d]);
            dxt[d] += v;
          }
        }
        /* softmax over the chosen logits */
        double sp = 0.0;
        for (int32_t j = 0; j < k; ++j) sp += p[t * k + j] * dpv[j];
        for (int32_t j = 0; j < k; ++j) {
          const double dl = p[t * k + j] * (dpv[j] - sp);
          dls[t * k + j] = dl;
          if (dp_out) dp_out[t * k + j] = dpv[j];
          const uint16_t* wr = w_g + (int64_t)ids[t * k + j] * D;
          for (int32_t d = 0; d < D; ++d) dxt[d] += dl * bf(wr[d]);
        }
      }
    }
    free(xd); free(g); free(u); free(dpv);
  }
  /* pass 2: weight gradients, one output row per iteration, tokens in order */
  if (!err) {
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < (int64_t)E * D; ++r) { /* dW_g[e,d], dW_down[e,d,:] */
      const int32_t e = (int32_t)(r / D), d = (int32_t)(r % D);
      double gsum = 0.0;
      double* dwr = dwdn + r * F;
      for (int32_t f = 0; f < F; ++f) dwr[f] = 0.0;
      for (int64_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j) {
          if (ids[t * k + j] != e) continue;
          gsum += dls[t * k + j] * bf(x[t * D + d]);
          const double c = p[t * k + j] * (double)dy[t * D + d];
          const double* h = hs + (t * S + j) * Fm;
          for (int32_t f = 0; f < F; ++f) dwr[f] += c * h[f];
        }
      dwg[r] = gsum;
    }
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < (int64_t)E * 2 * F; ++r) { /* dW_gate_up[e,r',:] */
      const int32_t e = (int32_t)(r / (2 * F)), q = (int32_t)(r % (2 * F));
      double* dwr = dwgu + r * D;
      for (int32_t d = 0; d < D; ++d) dwr[d] = 0.0;
      for (int64_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j) {
          if (ids[t * k + j] != e) continue;
          const double c = q < F ? dgs[(t * S + j) * Fm + q] : dus[(t * S + j) * Fm + q - F];
          for (int32_t d = 0; d < D; ++d) dwr[d] += c * bf(x[t * D + d]);
        }
    }
    if (dbias)
      for (int32_t e = 0; e < E; ++e) {
        double s = 0.0;
        if (bias_mode == 1)
          for (int64_t a = 0; a < T * k; ++a)
            if (ids[a] == e) s += dls[a];
        dbias[e] = s;
      }
    if (Fs > 0) {
#pragma omp parallel for schedule(dynamic, 4)
      for (int32_t d = 0; d < D; ++d) {
        double* dwr = dwsdn + (int64_t)d * Fs;
        for (int32_t f = 0; f < Fs; ++f) dwr[f] = 0.0;
        for (int64_t t = 0; t < T; ++t) {
          const double c = (double)dy[t * D + d];
          const double* h = hs + (t * S + k) * Fm;
          for (int32_t f = 0; f < Fs; ++f) dwr[f] += c * h[f];
        }
      }
#pragma omp parallel for schedule(dynamic, 4)
      for (int32_t q = 0; q < 2 * Fs; ++q) {
        double* dwr = dwsgu + (int64_t)q * D;
        for (int32_t d = 0; d < D; ++d) dwr[d] = 0.0;
        for (int64_t t = 0; t < T; ++t) {
          const double c = q < Fs ? dgs[(t * S + k) * Fm + q] : dus[(t * S + k) * Fm + q - Fs];
          for (int32_t d = 0; d < D; ++d) dwr[d] += c * bf(x[t * D + d]);
        }
      }
    }
  }
  free(hs); free(dgs); free(dus); free(dls);
  return err;
}

/* ------------------------------------------------------------------- align */

/*
 * Group the T*k assignments a = t*k + j by expert, for a given routing.
 * G = E groups (+1 shared group holding every token in order when shared != 0).
 *   counts[g]        number of rows of group g
 *   offsets[g]       exclusive prefix sum of counts            [G+1]
 *   padded[g]        exclusive prefix sum of ceil(count/BM)*BM [G+1]
 *   sorted_assign[i] the assignments in ascending (expert, a) order [T*k]
 *   row_of[a]        padded row of assignment a                 [T*k]
 *   row_token[r]     token of padded row r, -1 on padding rows  [padded[G]] (cap entries)
 *   tile_group[i]    group of BM-row tile i                     [padded[G]/BM]
 *   n_tiles          padded[G]/BM
 * Returns 0, -1 on invalid sizes or ids, -3 if cap is too small.
 */
int oracle_align(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t BM, int32_t shared,
                 int32_t* counts, int32_t* offsets, int32_t* padded, int32_t* sorted_assign,
                 int32_t* row_of, int32_t* row_token, int64_t cap, int32_t* tile_group,
                 int32_t* n_tiles) {
  if (T < 0 || k <= 0 || E <= 0 || BM <= 0) return -1;
  int32_t G = E + (shared ? 1 : 0);
  int64_t A = T * k;
  for (int32_t g = 0; g < G; ++g) counts[g] = 0;
  for (int64_t a = 0; a < A; ++a) {
    if (ids[a] < 0 || ids[a] >= E) return -1;
    counts[ids[a]]++;
  }
  if (shared) counts[E] = (int32_t)T;
  offsets[0] = 0;
  padded[0] = 0;
  for (int32_t g = 0; g < G; ++g) {
    offsets[g + 1] = offsets[g] + counts[g];
    padded[g + 1] = padded[g] + (counts[g] + BM - 1) / BM * BM;
  }
  if ((int64_t)padded[G] > cap) return -3;
  /* stable counting sort: scanning a upwards keeps ascending a inside each expert */
  int32_t* cursor = (int32_t*)calloc((size_t)G, sizeof(int32_t));
  if (!cursor) return -2;
  for (int64_t r = 0; r < padded[G]; ++r) row_token[r] = -1;
  for (int64_t a = 0; a < A; ++a) {
    int32_t e = ids[a];
    int32_t i = offsets[e] + cursor[e];
    int32_t r = padded[e] + cursor[e];
    cursor[e]++;
    sorted_assign[i] = (int32_t)a;
    row_of[a] = r;
    row_token[r] = (int32_t)(a / k);
  }
  if (shared)
    for (int64_t t = 0; t < T; ++t) row_token[padded[E] + t] = (int32_t)t;
  free(cursor);
  for (int32_t g = 0; g < G; ++g)
    for (int32_t i = padded[g] / BM; i < padded[g + 1] / BM; ++i) tile_group[i] = g;
  *n_tiles = padded[G] / BM;
  return 0;
}
