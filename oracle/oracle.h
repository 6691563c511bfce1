/* CPU oracle of one Llama-style decode step (test infrastructure only).
 * Declarations for oracle.c; nothing in the product path includes this file. */
#ifndef ORACLE_H
#define ORACLE_H
#include <stdint.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

typedef struct oracle_model {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  int32_t dtype;                  /* ORACLE_F32 or ORACLE_BF16: weights and KV cache */
  double rope_theta, rms_eps;
  const void* embed;              /* [vocab][hidden], also the tied LM head */
  const float* final_norm;        /* [hidden] */
  const float* const* attn_norm;  /* per layer [hidden] */
  const float* const* mlp_norm;   /* per layer [hidden] */
  const void* const* w_qkv;       /* per layer [(Hq+2Hkv)*D][hidden]: q rows, k rows, v rows */
  const void* const* w_o;         /* per layer [hidden][Hq*D] */
  const void* const* w_gate;      /* per layer [ffn][hidden] */
  const void* const* w_up;        /* per layer [ffn][hidden] */
  const void* const* w_down;      /* per layer [hidden][ffn] */
} oracle_model;

double oracle_bf16_value(uint16_t h);
uint16_t oracle_round_bf16(double x);
void oracle_matvec(const void* w, int32_t dtype, int32_t rows, int32_t cols, const double* x,
                   double* y);
void oracle_rmsnorm(const double* x, const float* g, int32_t n, double eps, double* y);
void oracle_rope(double* v, int32_t head_dim, int32_t pos, double theta);
double oracle_silu(double z);
void oracle_attention(const double* q, const void* kc, const void* vc, int32_t dtype,
                      int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t cap,
                      int32_t n, double* out, double* probs);
int32_t oracle_argmax_f32(const double* logits, int32_t n);
/* KV caches: [L][batch][Hkv][cap][D]; seq_len < 0 marks an inactive slot.
 * Returns 0, or -1 bad shape, -2 cache full, -3 token out of range. */
int32_t oracle_step(const oracle_model* m, int32_t batch, int32_t cap, const int32_t* tokens_in,
                    void* kcache, void* vcache, int32_t* seq_len, double* logits,
                    int32_t* tokens_out);
int32_t oracle_prefill(const oracle_model* m, int32_t batch, int32_t cap, const int32_t* prompt,
                       int32_t T, void* kcache, void* vcache, int32_t* seq_len, double* logits,
                       int32_t* tokens_out);
#endif
