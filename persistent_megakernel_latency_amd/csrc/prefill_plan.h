// prefill_plan.h -- the compiled form of a prompt prefill (time to first
// token), shared by the host builder and the gfx950 kernels.
//
// Time to first token is the latency the Llama-3.2-1B row of "One Megakernel
// is Not Enough" (Table III) measures for a 496-token prompt: the whole prompt
// goes through every layer at once (causal attention over the prompt), and the
// LM head on each sequence's last prompt position gives the first generated
// token.  The prefill is lowered to a tile DAG like the decode step (counter
// groups, claim queues in topological order), with tiles sized for a
// compute-bound workload: 128 prompt rows x 256 output columns x all of K per
// matrix-core tile, 64 queries x one kv head per attention tile.
#pragma once
#include <stdint.h>

#include "plan.h"

namespace wpk {

enum PrefillTileType : int32_t {
  P_EMBED = 0,   // layer 0: embedding rows of a row block -> residual stream, and their RMSNorm -> operand
  P_NORM1 = 1,   // attention-input RMSNorm of a row block (layers above 0)
  P_QKV = 2,     // QKV for (row block, four heads): RoPE, queries out, K/V appended to the cache
  P_ATTN = 3,    // causal attention for (sequence, kv head, 64-query block), the kv head's q heads together
  P_OPROJ = 4,   // o-projection + residual for (row block, 256 columns)
  P_NORM2 = 5,   // MLP-input RMSNorm of a row block
  P_GATEUP = 6,  // gate and up for (row block, 128 ffn columns) + SwiGLU
  P_DOWN = 7,    // down projection + residual for (row block, 256 columns)
  P_NORMF = 8,   // final RMSNorm of one sequence's last prompt row
  P_LM = 9,      // tied LM head on the last rows, 256 vocabulary columns, partial argmax
  P_ARGMAX = 10, // the first generated token of every sequence, seq_len = prompt length
  P_NTYPES = 11
};

// Tile fields (the 64-byte Tile of plan.h): type, layer, wait, signal, shard,
// id as in the decode step; r0 = row block (b * blocks per sequence + j),
// r1 = column block (norm tiles: which 16 rows of the row block), b =
// sequence, g = kv head, c = 64-query block.

constexpr int kPRows = 128;     // prompt rows of a row block (a matrix-core tile, a norm tile)
constexpr int kPCols = 256;     // output columns of a QKV / o / down tile (four heads)
constexpr int kPFfnCols = 128;  // SwiGLU columns of a gate/up tile (128 gate + 128 up weight rows)
constexpr int kPQueries = 64;   // queries of an attention tile (32 per wave, two waves per q head)
constexpr int kPKeys = 32;      // keys per attention step
constexpr int kPLmCols = 256;   // vocabulary columns of an LM-head tile
constexpr int kPThreads = 512;  // eight waves per worker (one worker per CU), all computing
constexpr int kPWaves = kPThreads / 64;
constexpr int kPNormSplit = kPRows / 16;  // norm tiles per row block (16 rows each)

// Per-layer device pointers.  Every activation buffer is per layer and
// written once per prefill, so a consumer never meets a line that was
// rewritten during the launch (see prefill.hip on coherence).  The operands
// of the matrix products (xn1, xn2, ao, h, and xf) are two bf16 planes, hi
// [R][K] then lo [R][K], with value = hi + lo (hi the fp32 value rounded to
// bf16, lo the remainder rounded to bf16: about 16 significant bits), the
// operand precision of the decode step's matrix-core tiles.
struct PLayer {
  const uint16_t* w_qkv;
  const uint16_t* w_o;
  const uint16_t* w_gate;
  const uint16_t* w_up;
  const uint16_t* w_down;
  const float* attn_norm;
  const float* mlp_norm;
  const float* x_in;   // [R][H] layer input (the previous layer's x_out, or x0)
  float* x_mid;        // [R][H] after attention
  float* x_out;        // [R][H] after the MLP
  uint16_t* xn1;       // [2][R][H] RMSNorm(x_in) * gain
  uint16_t* xn2;       // [2][R][H] RMSNorm(x_mid) * gain
  float* q;            // [R][Hq*D] rotated queries
  uint16_t* ao;        // [2][R][Hq*D] attention output
  uint16_t* h;         // [2][R][F] SwiGLU output
};

struct PParams {
  int32_t L, H, Hq, Hkv, D, F, V, B, cap, G, qkv_rows;
  int32_t P;      // prompt length (every sequence)
  int32_t Pp;     // rows per sequence, P rounded up to kPRows
  int32_t nrb_s;  // row blocks per sequence
  int32_t R;      // prompt rows of all sequences, B * Pp
  int32_t n_tiles, n_queues, n_workers;
  float eps, attn_scale;
  const uint16_t* embed;     // [V][H]
  const float* final_norm;   // [H]
  const PLayer* layers;      // [L], device memory
  float* x0;                 // [R][H] layer-0 input (embedding rows; padding rows zero)
  uint16_t* xf;              // [2][32][H] final-normed last prompt row per sequence (rows >= B zero)
  const float* rope_cos;     // [cap][D/2]
  const float* rope_sin;
  const int32_t* prompt;     // [B][P] token ids
  int32_t* tokens_out;       // [B] first generated token
  int32_t* seq_len;          // [B] set to P
  float* logits;             // [B][V] logits of the last prompt position
  uint16_t* kc;              // [L][B][Hkv][cap][D]
  uint16_t* vc;
  const Tile* tiles;         // by id
  const Tile* qtiles;        // claim-queue order
  const int32_t* queue_off;  // n_queues + 1
  const Group* groups;
  uint32_t* counters;        // group shards, stride kLine
  uint32_t* heads;           // claim head per queue, stride kLine
  uint32_t* ctl;             // control block (CTL_* words of plan.h)
  unsigned long long* argmax;  // [B][kArgmaxShards]
  int32_t* log;              // wpk_log_rec per tile
  uint64_t watchdog_ticks;
  const int32_t* worker_queue;  // claim queue of each worker
};

}  // namespace wpk
