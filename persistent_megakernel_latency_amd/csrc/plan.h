// plan.h -- the compiled form of one decode step, shared by the host builder,
// the host executors and the gfx950 kernels.
//
// The step is a DAG of tiles.  Every tile waits on at most one counter group
// and signals exactly one: a group counts the tiles that produce the tensor
// region its consumers read, so a consumer starts as soon as its own inputs
// are complete instead of at an operator boundary (the tile-to-tile tensor
// edges of "One Megakernel is Not Enough", Table I, cross-kernel readiness;
// the per-chunk dependency counters of the Llama-1B megakernel described in
// "persistent-threads-megakernels", section 6).
#pragma once
#include <stdint.h>

namespace wpk {

enum TileType : int32_t {
  T_QKV = 0,      // RMSNorm prologue, QKV rows, RoPE + KV-append epilogue
  T_ATTN = 1,     // split-KV decode attention partial over one KV chunk
  T_COMBINE = 2,  // merge of the partials of one (sequence, kv head)
  T_OPROJ = 3,    // output projection + residual
  T_GATEUP = 4,   // RMSNorm prologue, gate and up rows, SwiGLU epilogue
  T_DOWN = 5,     // down projection + residual
  T_LM = 6,       // final RMSNorm prologue, tied LM-head rows, partial argmax
  T_ARGMAX = 7,   // greedy token, seq_len advance (output conversion)
  // wide plans (batch above kMaxBatchGemv): the layer-0 embedding row of each
  // sequence into the bf16 operand the matrix-core tiles read (later RMSNorm
  // inputs are written by the tiles that produce them)
  T_NORM = 8,
  T_NORM2 = 9,    // not emitted (former per-sequence MLP-input norm)
  T_NORMF = 10,   // not emitted (former per-sequence final norm)
  // LDS forwarding: attention over every KV chunk of one (sequence, kv head),
  // each chunk's partial merged on chip into the next (the combine chained
  // onto the same worker; no partials in global memory, no combine tile)
  T_ATTNC = 11,
  T_NTYPES = 12
};

// One tile: 64 bytes, loaded with scalar loads by a worker.
struct Tile {
  int32_t type, layer, wait, signal;  // wait/signal: counter group id or -1
  int32_t shard;                      // counter shard of `signal` this tile increments
  int32_t r0, r1, rs;                 // GEMV: rows [r0, r0+rs) then [r1, r1+(rows-rs)) of its matrix
  int32_t rows;                       // GEMV: row capacity of the tile
  int32_t b, g, c;                    // ATTN: sequence, kv head, KV chunk; COMBINE, NORM*: b (, g); QKV: head
                                      // wide GEMM tiles: b = slices of the row block, c = this tile's slice
  int32_t kind;                       // QKV: 0 q rows, 1 k rows, 2 v rows; ATTN: KV chunks [c, c + kind)
  int32_t id;                         // tile id (index into the tile table and the log)
  int32_t fix;                        // wide GEMM tiles: row-block index (its arrival counter)
  int32_t pslot;                      // wide GEMM tiles: partial-sum slot of the row block's slice 0
};
static_assert(sizeof(Tile) == 64, "tile descriptor is 64 bytes");

// A counter group: `producers` tiles increment it once per step, spread over
// `shards` counters (each on its own 256-byte line) so that same-address
// atomics do not serialise.  Step e (from 0) is complete when the shards sum
// to (e + 1) * producers (modulo 2^32).
struct Group {
  int32_t producers, shard0, shards, pad;
};

constexpr int kThreads = 256;                         // threads per worker (4 wave64)
constexpr int kWaves = kThreads / 64;
constexpr int kChunks = 16;                           // 16-byte weight chunks per thread
constexpr int kSlotBytes = kThreads * kChunks * 16;   // one staging slot: 64 KiB
constexpr int kLine = 64;                             // uint32 stride of independent counters (256 B)
constexpr int kAttnChunk = 64;                        // KV positions per attention partial
constexpr int kHeadDim = 64;                          // the only head size built
constexpr int kMaxGroupHeads = 4;                     // q heads per kv head
constexpr int kArgmaxShards = 16;
constexpr int kMaxShards = 128;  // two per lane of a polling wave
constexpr int kMaxBatch = 32;
constexpr int kMaxBatchGemv = 4;   // above it a plan is wide: matrix-core tiles over all sequences
// Wide (matrix-core) tiles: 64 weight rows x a 512-column slice of K (64 KiB
// of bf16), all sequences.  The slices of a row block each leave a partial
// sum; the last one to finish adds them in slice order and runs the epilogue.
constexpr int kWideRows = 64;
constexpr int kWideK = 512;
constexpr int kWidePart = kWideRows * kMaxBatch;  // floats of one partial-sum slot
constexpr int kMaxLayers = 32;

// Control block: word offsets, each field on its own 256-byte line.
enum : int32_t {
  CTL_EPOCH = 0,     // steps completed
  CTL_EXIT = 64,     // workers that left the current step
  CTL_STATUS = 128,  // [0] error code, [1] tile, [2] worker, [3] epoch
  CTL_ABORT = 192,   // nonzero: every worker stops
  CTL_GO = 256,      // persistent grids: steps granted so far (an epoch), or kGoStop
  CTL_WORDS = 320
};

// Persistent grids: CTL_GO value that makes every worker leave, and the host
// doorbell value that asks for it.
constexpr uint32_t kGoStop = 0xFFFFFFFFu;
constexpr uint32_t kBellStop = 0xFFFFFFFFu;
constexpr int kPersistTimes = 4096;  // per-step device times kept (a ring)

// Per-layer pointers: weights (caller-owned) and this layer's activations.
// Field order matters to the wide kernels, which index runs of consecutive
// pointers: (attn_norm, mlp_norm), (x_in, x_mid, x_out), (xn1 .. xnf).
struct LayerBufs {
  const void* w_qkv;
  const void* w_o;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const float* attn_norm;
  const float* mlp_norm;
  const float* x_in;  // [B][H] layer input; nullptr for layer 0 (embedding gather)
  float* x_mid;       // [B][H] after attention
  float* x_out;       // [B][H] after the MLP
  float* q;           // [B][Hq*D] rotated queries
  float* part;        // [B][Hkv][nch][G][D+2] attention partials (m, l, o[D]), one per attention tile
  float* attn;        // [B][Hq*D] attention output
  float* h;           // [B][F] SwiGLU output
  // Wide plans: operands of the matrix-core tiles as a pair of bf16 planes,
  // hi [32][K] then lo [32][K], with value = hi + lo (hi is the value rounded
  // to bf16, lo the remainder rounded to bf16: about 16 significant bits).
  // Rows past B stay zero.
  // (xn1, xattn, xn2, xh, xnf are consecutive: the kernels index them)
  uint16_t* xn1;      // attention input (gain-scaled, see below)
  uint16_t* xattn;    // attention output
  uint16_t* xn2;      // MLP input (gain-scaled)
  uint16_t* xh;       // SwiGLU output
  uint16_t* xnf;      // final hidden state (gain-scaled; last layer only)
  const float* final_norm;  // the final RMSNorm gain (same in every layer)
  // Wide plans: the RMSNorm is split between producer and consumer.  The
  // operand planes xn1, xn2 and xnf hold gain * x (not yet divided by the
  // root mean square); the tile that writes a 64-row block of x also writes
  // that block's sum of squares per sequence here, [H/64][32], and the
  // consumer's epilogue scales its sums by 1 / sqrt(mean + eps).
  // (ss1, ss2, ssf are consecutive: the kernels index them)
  float* ss1;         // attention input
  float* ss2;         // MLP input
  float* ssf;         // final (last layer only)
};

// Per-layer weights as the kernels see them: kept inside the kernel arguments
// so that a tile's base pointers are scalar loads from constant memory.
struct LayerW {
  const void* w_qkv;
  const void* w_o;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const float* attn_norm;
  const float* mlp_norm;
};

// Everything a worker needs, passed by value to the kernel.
struct Params {
  int32_t L, H, Hq, Hkv, D, F, V, B, cap, nch, G, qkv_rows;
  int32_t attn_sub;  // KV chunks per attention tile: its chunks' partials merge into one (slot c / attn_sub)
  int32_t n_tiles, n_queues, n_workers, dtype;
  float eps, attn_scale;
  const void* embed;
  const float* final_norm;
  const LayerBufs* layers;  // host executors: per-layer pointers in host memory
  // device kernels: activations of layer l at act + l * act_layer + off_*
  float* act;
  int64_t act_layer;
  int32_t off_x_mid, off_x_out, off_q, off_part, off_attn, off_h;
  // wide plans: bf16 operand buffers, offsets in floats from the layer's base
  int32_t wide, off_xn1, off_xattn, off_xn2, off_xh, off_xnf;
  float* wpart;             // wide plans: partial sums, kWidePart floats per slot
  uint32_t* fixc;           // wide plans: arrival counter per row block, stride kLine
  LayerW lw[kMaxLayers];
  const float* rope_cos;  // [cap][D/2]
  const float* rope_sin;  // [cap][D/2]
  int32_t* tokens;
  int32_t* seq_len;
  float* logits;          // [B][V]
  char* kc;               // [L][B][Hkv][cap][D]
  char* vc;
  const Tile* tiles;
  const Tile* qtiles;       // the tile table in claim-queue order: qtiles[i] = tiles[queue[i]]
  const int32_t* queue;     // tile ids of all claim queues, concatenated
  const int32_t* queue_off; // queue q holds queue[queue_off[q] .. queue_off[q+1])
  const Group* groups;
  uint32_t* counters;       // group shards, stride kLine
  uint32_t* heads;          // claim head of each queue, stride kLine
  uint32_t* ctl;            // control block
  unsigned long long* argmax;  // [B][kArgmaxShards] packed (value, index) maxima
  int32_t* log;             // wpk_log_rec per tile, then per worker slot, then per-tile timings
  int32_t log_workers;      // worker record slots in the log (co-resident maximum)
  int32_t log_on, prefetch, drop_tile;
  uint32_t perturb;
  uint64_t watchdog_ticks;  // s_memrealtime ticks (100 MHz)
  // Cross-step persistence: with persist set the grid stays resident and runs
  // one step per grant.  The host rings host_bell (pinned host memory: the
  // number of steps it has asked for since the session began, or kBellStop);
  // worker 0 relays it to CTL_GO as the absolute epoch persist_base + bell;
  // the last worker out of each step publishes the steps done to host_done.
  int32_t persist;
  uint32_t persist_base;
  const uint32_t* host_bell;
  uint32_t* host_done;
  uint64_t idle_ticks;      // a grid left without a grant this long stops by itself
  uint64_t* step_times;     // [kPersistTimes][2]: grant seen, last worker out (s_memrealtime)
  // The claim queue of each worker (blockIdx.x): w mod n_queues for one
  // megakernel; with two co-resident megakernels (split plans) the first's
  // workers deal over its queues and the second's over the others.
  const int32_t* worker_queue;
};

}  // namespace wpk
