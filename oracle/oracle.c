/* CPU oracle of one Llama-style decode step.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg load this library.  The product path (the HIP
 * megakernel behind the C ABI) never links, loads or calls it, and this file
 * shares no code, header, table or constant generator with it.
 *
 * What it computes.  The megakernel page ("Why real-time inference wants a
 * megakernel", section "It increases compiler and verification burden") asks a
 * megakernel to keep the numerical behaviour of the program it replaces
 * through fusion and reordering, so the oracle is the plain, unfused
 * definition of one decode step of the workload the persistent-threads page
 * names (section 6: the Llama-3.2-1B forward pass for one token, through the
 * logits, with greedy decoding).  The pages never spell out the layer, so the
 * standard Llama-3 pre-norm decoder is taken:
 *
 *   x  = E[token]
 *   per layer:  a = RMSNorm(x) * g1;  q,k,v = split(W_qkv a)
 *               RoPE(q), RoPE(k) at position p = seq_len
 *               append k, v at p (stored in the cache's dtype)
 *               o_h = sum_{j<=p} softmax_j(q_h . K_j / sqrt(d)) V_j   (GQA)
 *               x += W_o o
 *               m = RMSNorm(x) * g2;  x += W_down (silu(W_gate m) * (W_up m))
 *   logits = E (RMSNorm(x) * g_f)    (tied head);  token = argmax
 *
 * Arithmetic is float64 throughout with plain sequential loops; weights are
 * read exactly (bf16 and f32 are subsets of f64).  The only roundings are the
 * ones the step itself defines: the KV cache stores k and v in its own dtype
 * (bf16 round-to-nearest-even, or f32), and the greedy choice is taken on the
 * logits rounded to float32, the precision the kernel decides in (lowest
 * index wins a tie).  OpenMP splits only independent output rows; each dot
 * product is one thread's sequential sum, so results do not depend on the
 * thread count.
 *
 * Readings of points the pages leave open (eps = 1e-5, rotate-half RoPE
 * pairs (i, i + d/2) with inverse frequency theta^(-2i/d) and no frequency
 * scaling, kv head of q head h = h / (Hq/Hkv), softmax scale 1/sqrt(d) over
 * positions 0..p inclusive, no biases, no embedding scale) are listed with the
 * rest of the design notes.  Whole-model values are parity unpinned against
 * the pages, which print no worked example; each building block is pinned by
 * the tests against library routines, closed forms and invariants.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

/* ---- number formats ---------------------------------------------------- */

/* Exact value of a bfloat16 bit pattern: the upper half of a float32. */
double oracle_bf16_value(uint16_t h) {
  union { uint32_t u; float f; } v;
  v.u = (uint32_t)h << 16;
  return (double)v.f;
}

/* Round a float64 to the nearest bfloat16, ties to even (8 significant bits,
 * exponent range of float32, subnormal quantum 2^-133). */
uint16_t oracle_round_bf16(double x) {
  if (isnan(x)) return (uint16_t)0x7FC0;
  const double a = fabs(x);
  double r;
  if (a == 0.0 || isinf(a)) {
    r = a;
  } else {
    int e = 0;
    frexp(a, &e);      /* a in [2^(e-1), 2^e) */
    int ex = e - 1;
    if (ex < -126) ex = -126;
    const double quantum = ldexp(1.0, ex - 7);
    r = nearbyint(a / quantum) * quantum; /* default rounding: nearest, ties even */
  }
  union { float f; uint32_t u; } v;
  v.f = (float)r; /* exact: r is a bfloat16 value, or overflows to inf */
  uint16_t bits = (uint16_t)(v.u >> 16);
  if (signbit(x)) bits |= 0x8000u;
  return bits;
}

static inline double weight_at(const void* w, int32_t dtype, int64_t i) {
  if (dtype == ORACLE_BF16) return oracle_bf16_value(((const uint16_t*)w)[i]);
  return (double)((const float*)w)[i];
}

static inline void cache_store(void* c, int32_t dtype, int64_t i, double x) {
  if (dtype == ORACLE_BF16) ((uint16_t*)c)[i] = oracle_round_bf16(x);
  else ((float*)c)[i] = (float)x;
}

/* ---- building blocks ----------------------------------------------------- */

/* y[r] = sum_c W[r][c] x[c], W row-major [rows][cols]. */
void oracle_matvec(const void* w, int32_t dtype, int32_t rows, int32_t cols,
                   const double* x, double* y) {
#pragma omp parallel for schedule(static)
  for (int32_t r = 0; r < rows; ++r) {
    double s = 0.0;
    const int64_t base = (int64_t)r * cols;
    for (int32_t c = 0; c < cols; ++c) s += weight_at(w, dtype, base + c) * x[c];
    y[r] = s;
  }
}

/* y = x / sqrt(mean(x^2) + eps) * g. */
void oracle_rmsnorm(const double* x, const float* g, int32_t n, double eps, double* y) {
  double ss = 0.0;
  for (int32_t i = 0; i < n; ++i) ss += x[i] * x[i];
  const double inv = 1.0 / sqrt(ss / (double)n + eps);
  for (int32_t i = 0; i < n; ++i) y[i] = x[i] * inv * (double)g[i];
}

/* Rotary embedding of one head vector at position pos, rotate-half pairing:
 * dims (i, i + d/2) rotate by the angle pos * theta^(-2i/d). */
void oracle_rope(double* v, int32_t head_dim, int32_t pos, double theta) {
  const int32_t half = head_dim / 2;
  for (int32_t i = 0; i < half; ++i) {
    const double ang = (double)pos * pow(theta, -2.0 * (double)i / (double)head_dim);
    const double c = cos(ang), s = sin(ang);
    const double a = v[i], b = v[i + half];
    v[i] = a * c - b * s;
    v[i + half] = b * c + a * s;
  }
}

double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

/* Decode attention of one sequence over its n cached positions.
 * q: [Hq][D] (float64); kc, vc: [Hkv][cap][D] in the cache dtype.
 * out: [Hq][D].  probs (optional): [Hq][n] softmax weights. */
void oracle_attention(const double* q, const void* kc, const void* vc, int32_t dtype,
                      int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t cap,
                      int32_t n, double* out, double* probs) {
  const int32_t group = n_q_heads / n_kv_heads;
  const double scale = 1.0 / sqrt((double)head_dim);
  double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int32_t h = 0; h < n_q_heads; ++h) {
    const int32_t g = h / group;
    const int64_t kv0 = (int64_t)g * cap * head_dim;
    double m = -INFINITY;
    for (int32_t j = 0; j < n; ++j) {
      double dot = 0.0;
      for (int32_t d = 0; d < head_dim; ++d)
        dot += q[h * head_dim + d] * weight_at(kc, dtype, kv0 + (int64_t)j * head_dim + d);
      s[j] = dot * scale;
      if (s[j] > m) m = s[j];
    }
    double z = 0.0;
    for (int32_t j = 0; j < n; ++j) {
      s[j] = exp(s[j] - m);
      z += s[j];
    }
    for (int32_t d = 0; d < head_dim; ++d) out[h * head_dim + d] = 0.0;
    for (int32_t j = 0; j < n; ++j) {
      const double p = s[j] / z;
      if (probs) probs[(int64_t)h * n + j] = p;
      for (int32_t d = 0; d < head_dim; ++d)
        out[h * head_dim + d] += p * weight_at(vc, dtype, kv0 + (int64_t)j * head_dim + d);
    }
  }
  free(s);
}

/* Greedy choice on the logits rounded to float32; the lowest index wins ties. */
int32_t oracle_argmax_f32(const double* logits, int32_t n) {
  int32_t best = -1;
  float bv = 0.0f;
  for (int32_t i = 0; i < n; ++i) {
    const float v = (float)logits[i];
    if (isnan(v)) continue;
    if (best < 0 || v > bv) {
      best = i;
      bv = v;
    }
  }
  return best;
}

/* ---- one decode step ------------------------------------------------------ */

int32_t oracle_step(const oracle_model* m, int32_t batch, int32_t cap, const int32_t* tokens_in,
                    void* kcache, void* vcache, int32_t* seq_len, double* logits,
                    int32_t* tokens_out) {
  if (!m || batch <= 0 || cap <= 0) return -1;
  const int32_t H = m->hidden, D = m->head_dim, Hq = m->n_q_heads, Hkv = m->n_kv_heads;
  const int32_t F = m->ffn, V = m->vocab, L = m->n_layers;
  if (Hkv <= 0 || Hq % Hkv != 0 || D % 2 != 0) return -1;
  for (int32_t b = 0; b < batch; ++b) {
    if (seq_len[b] < 0) continue;
    if (seq_len[b] >= cap) return -2;
    if (tokens_in[b] < 0 || tokens_in[b] >= V) return -3;
  }
  const int32_t qkv_rows = (Hq + 2 * Hkv) * D;
  double* x = (double*)malloc(sizeof(double) * H);
  double* a = (double*)malloc(sizeof(double) * H);
  double* qkv = (double*)malloc(sizeof(double) * qkv_rows);
  double* att = (double*)malloc(sizeof(double) * Hq * D);
  double* t = (double*)malloc(sizeof(double) * H);
  double* gate = (double*)malloc(sizeof(double) * F);
  double* up = (double*)malloc(sizeof(double) * F);
  const size_t elt = m->dtype == ORACLE_BF16 ? 2 : 4;

  for (int32_t b = 0; b < batch; ++b) {
    double* lg = logits + (int64_t)b * V;
    if (seq_len[b] < 0) { /* inactive slot: no work, token kept */
      for (int32_t i = 0; i < V; ++i) lg[i] = 0.0;
      tokens_out[b] = tokens_in[b];
      continue;
    }
    const int32_t p = seq_len[b];
    const int64_t tok = tokens_in[b];
    for (int32_t i = 0; i < H; ++i) x[i] = weight_at(m->embed, m->dtype, tok * H + i);

    for (int32_t l = 0; l < L; ++l) {
      oracle_rmsnorm(x, m->attn_norm[l], H, m->rms_eps, a);
      oracle_matvec(m->w_qkv[l], m->dtype, qkv_rows, H, a, qkv);
      double* q = qkv;
      double* k = qkv + (int64_t)Hq * D;
      double* v = qkv + (int64_t)(Hq + Hkv) * D;
      for (int32_t h = 0; h < Hq; ++h) oracle_rope(q + (int64_t)h * D, D, p, m->rope_theta);
      for (int32_t g = 0; g < Hkv; ++g) oracle_rope(k + (int64_t)g * D, D, p, m->rope_theta);
      /* cache slice of (layer l, sequence b): [Hkv][cap][D] */
      const int64_t slice = ((int64_t)l * batch + b) * Hkv * (int64_t)cap * D;
      char* kc = (char*)kcache + slice * elt;
      char* vc = (char*)vcache + slice * elt;
      for (int32_t g = 0; g < Hkv; ++g)
        for (int32_t d = 0; d < D; ++d) {
          const int64_t i = ((int64_t)g * cap + p) * D + d;
          cache_store(kc, m->dtype, i, k[(int64_t)g * D + d]);
          cache_store(vc, m->dtype, i, v[(int64_t)g * D + d]);
        }
      oracle_attention(q, kc, vc, m->dtype, Hq, Hkv, D, cap, p + 1, att, NULL);
      oracle_matvec(m->w_o[l], m->dtype, H, Hq * D, att, t);
      for (int32_t i = 0; i < H; ++i) x[i] += t[i];

      oracle_rmsnorm(x, m->mlp_norm[l], H, m->rms_eps, a);
      oracle_matvec(m->w_gate[l], m->dtype, F, H, a, gate);
      oracle_matvec(m->w_up[l], m->dtype, F, H, a, up);
      for (int32_t i = 0; i < F; ++i) gate[i] = oracle_silu(gate[i]) * up[i];
      oracle_matvec(m->w_down[l], m->dtype, H, F, gate, t);
      for (int32_t i = 0; i < H; ++i) x[i] += t[i];
    }
    oracle_rmsnorm(x, m->final_norm, H, m->rms_eps, a);
    oracle_matvec(m->embed, m->dtype, V, H, a, lg);
    tokens_out[b] = oracle_argmax_f32(lg, V);
    seq_len[b] = p + 1;
  }
  free(x); free(a); free(qkv); free(att); free(t); free(gate); free(up);
  return 0;
}

/* Prefill as the same step run token by token (teacher-forced): prompt is
 * [batch][T].  logits receives the last position's logits, tokens_out the
 * greedy token after the prompt. */
int32_t oracle_prefill(const oracle_model* m, int32_t batch, int32_t cap, const int32_t* prompt,
                       int32_t T, void* kcache, void* vcache, int32_t* seq_len, double* logits,
                       int32_t* tokens_out) {
  int32_t* tin = (int32_t*)malloc(sizeof(int32_t) * (size_t)batch);
  int32_t rc = 0;
  for (int32_t s = 0; s < T && rc == 0; ++s) {
    for (int32_t b = 0; b < batch; ++b) tin[b] = prompt[(int64_t)b * T + s];
    rc = oracle_step(m, batch, cap, tin, kcache, vcache, seq_len, logits, tokens_out);
  }
  free(tin);
  return rc;
}
