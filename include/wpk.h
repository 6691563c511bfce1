/* wpk.h -- C ABI of the MI355X (gfx950) decode-step megakernel.
 *
 * One recurring model update -- a Llama-style decode step: embedding gather,
 * RMSNorm, QKV projection, RoPE, KV-cache append, grouped-query decode
 * attention, output projection, SwiGLU MLP, tied LM head and greedy argmax --
 * runs as ONE kernel launch whose resident workers pull tiles of the step from
 * a device-side queue and start each tile when its dependency counter says its
 * inputs are complete.
 *
 * Where the operations come from:
 *  - "Why real-time inference wants a megakernel" (phbiojout.com), section
 *    "The unit of execution": a megakernel is one kernel that owns a
 *    multi-operation program including the coordination between operations;
 *    section "A concrete design: one WPK update": the compiler takes a graph of
 *    operations with cost estimates, the device does input conversion, the
 *    program and output conversion before publishing completion, and the host
 *    keeps admission, slot lifecycle and delivery.  wpk_build is that compile
 *    step for a declared operating point (model, capacity, context limit:
 *    section "The cohort is known"); wpk_step is one update.
 *  - "persistent-threads-megakernels" (tobiasrp.github.io), section 6: the
 *    Llama-3.2-1B forward pass for one token through the logits in one launch,
 *    with dependency counters that let a task start when its own input chunk is
 *    ready and weight loads for upcoming work started early.
 *  - "One Megakernel is Not Enough" (arXiv 2610.35336), Table I: tile graphs
 *    keep tile-to-tile tensor edges instead of barrier edges between kernels;
 *    one weight-staging slot per worker whose load is queued while the tile's
 *    predecessors run; W workers.
 *
 * Ownership: the caller owns every pointer it passes (weights, tokens, KV
 * cache, sequence lengths, logits) and keeps them alive while a plan that uses
 * them exists.  A plan owns its own device workspace and frees it in
 * wpk_destroy.  A plan is bound to the device that was current at build time,
 * is not thread-safe, and steps enqueued on one stream run in order.
 *
 * Errors: every call returns WPK_OK (0) or a negative WPK_E_* code; a NULL plan
 * from a build call means failure and wpk_last_error(NULL) says why (message
 * kept per thread).  Argument errors are reported synchronously.  Errors found
 * on the device (a full KV cache, a token id out of range, a watchdog timeout)
 * are latched in a device status word; wpk_sync() returns them, and from then
 * on the plan refuses to step (WPK_E_STATE) until WPK_OPT_RESET.  No C++
 * exception crosses this boundary.
 */
#ifndef WPK_H
#define WPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ---------------------------------------------------------- */
#define WPK_OK 0
#define WPK_E_ARG (-1)          /* bad argument or unsupported shape */
#define WPK_E_NOMEM (-2)        /* device or host allocation failed */
#define WPK_E_HIP (-3)          /* a HIP runtime call failed */
#define WPK_E_OCCUPANCY (-4)    /* the W workers cannot all be co-resident */
#define WPK_E_TIMEOUT (-5)      /* a worker's bounded wait ran out (device) */
#define WPK_E_CTX_FULL (-6)     /* seq_len reached the context capacity (device) */
#define WPK_E_TOKEN (-7)        /* an input token id is outside [0, vocab) (device) */
#define WPK_E_STATE (-8)        /* plan holds a latched device error; reset it */
#define WPK_E_NO_GPU (-9)       /* no usable gfx950 device */

/* ---- data types --------------------------------------------------------------- */
#define WPK_F32 0               /* float32 weights and KV cache */
#define WPK_BF16 1              /* bfloat16 weights and KV cache */

/* Stream handle: a hipStream_t, passed as an opaque pointer (NULL = the default
 * stream) so this header does not need the HIP headers. */
typedef void* wpk_stream_t;

/* A Llama-style decoder: pre-norm residual blocks, grouped-query attention with
 * rotate-half RoPE, SwiGLU MLP, tied LM head, no biases.
 * Matrices are row-major [out][in] in `dtype`; norm gains are float32.
 * For wpk_build / wpk_build_graph_baseline every pointer is DEVICE memory; for
 * wpk_build_host every pointer is HOST memory.  The per-layer pointer tables
 * themselves (attn_norm, w_qkv, ...) are host arrays of n_layers entries. */
typedef struct wpk_model_desc {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  int32_t tied_embeddings;       /* must be 1: lm_head = embed */
  float rope_theta, rms_eps;     /* e.g. 500000, 1e-5 */
  int32_t dtype;                 /* WPK_F32 | WPK_BF16 */
  const void* embed;             /* [vocab][hidden] */
  const float* final_norm;       /* [hidden] */
  const float* const* attn_norm; /* per layer [hidden] */
  const void* const* w_qkv;      /* per layer [(Hq + 2 Hkv) * head_dim][hidden]: q, k, v rows */
  const void* const* w_o;        /* per layer [hidden][Hq * head_dim] */
  const float* const* mlp_norm;  /* per layer [hidden] */
  const void* const* w_gate;     /* per layer [ffn][hidden] */
  const void* const* w_up;       /* per layer [ffn][hidden] */
  const void* const* w_down;     /* per layer [hidden][ffn] */
} wpk_model_desc;

/* KV cache, caller-owned.  k and v: [n_layers][batch][n_kv_heads][ctx_len][head_dim]
 * in the model dtype.  seq_len: int32[batch], the number of cached positions
 * of each sequence; a step appends at seq_len[b] and increments it; a negative
 * value marks an inactive slot (no append, token kept, logits undefined). */
typedef struct wpk_kv {
  void* k;
  void* v;
  int32_t* seq_len;
} wpk_kv;

/* Build-time tuning (all fields 0 = default). */
typedef struct wpk_build_opts {
  int32_t tile_bytes;       /* weight bytes per GEMV tile (default 65536; a multiple of 4096, at most 65536) */
  int32_t workers_per_cu;   /* resident workers per compute unit (default 2) */
  int32_t queue_shards;     /* claim queues the topological order is dealt over (default 8) */
  int32_t attn_chunk;       /* KV positions per attention partial tile (only 64 is built) */
  int32_t forward;          /* LDS forwarding of attention partials (batches above 4): one chained
                               tile per (sequence, kv head) walks its KV chunks and merges their
                               partials on chip, with no combine tiles.  1: on; 0 (default) or -1:
                               off (split tiles and combine tiles; faster at the built shapes) */
} wpk_build_opts;

typedef struct wpk_plan wpk_plan;

/* Compile the decode step for (model, batch, ctx_len) into a tile DAG, size the
 * workspace once and upload it.  Requirements: head_dim == 64,
 * n_q_heads * head_dim == hidden, n_q_heads / n_kv_heads <= 4, hidden and ffn
 * such that one weight row is 1..32 KiB and a power-of-two number of 16-byte
 * chunks, batch in [1, 32].  Batches above 4 run the projections, the MLP and
 * the LM head on the matrix cores (bf16 weights; hidden and ffn multiples of
 * 512, hidden at most 2048).  Returns NULL on error (see wpk_last_error(NULL)). */
wpk_plan* wpk_build(const wpk_model_desc* desc, int32_t batch, int32_t ctx_len);
wpk_plan* wpk_build_ex(const wpk_model_desc* desc, int32_t batch, int32_t ctx_len,
                       const wpk_build_opts* opts);

/* One decode step, enqueued on `stream` as a single launch.
 * tokens: device int32[batch]; on entry the current input token of each
 * sequence, on completion the greedy next token (so steps can be chained
 * without a host round trip).  logits: device float32[batch][vocab].
 * The call returns once the launch is enqueued; use wpk_sync to wait. */
int32_t wpk_step(wpk_plan* plan, int32_t* tokens, wpk_kv* kv, void* logits, wpk_stream_t stream);

/* Wait for the plan's last step and return the latched device status. */
int32_t wpk_sync(wpk_plan* plan);

void wpk_destroy(wpk_plan* plan);

/* Last error message of the plan, or of the calling thread if plan is NULL. */
const char* wpk_last_error(const wpk_plan* plan);

/* Runtime options (keys below).  Returns WPK_E_ARG for an unknown key/value. */
#define WPK_OPT_LOG 1             /* 1: record the per-tile execution log each step */
#define WPK_OPT_WATCHDOG_US 2     /* bound on any single wait, microseconds (default 2,000,000) */
#define WPK_OPT_PERTURB_SEED 3    /* != 0: sleep a pseudo-random time before each tile */
#define WPK_OPT_DEBUG_DROP_TILE 4 /* >= 0: that tile never publishes (watchdog test) */
#define WPK_OPT_RESET 5           /* clear the latched error, counters, queues and epoch */
#define WPK_OPT_PREFETCH 6        /* 1 (default): stage a tile's weights before its inputs are complete;
                                     0: only after (an ablation of the weight prefetch) */
#define WPK_OPT_WORKERS 7         /* number of resident workers W (<= the built maximum) */
#define WPK_OPT_LAUNCH 8          /* 0 (default): plain launch; 1: cooperative launch (measured ~20 us
                                     more per step).  Both are safe: claims follow the topological
                                     order, so a worker that is not yet resident holds no tile that
                                     anyone waits on */
int32_t wpk_set_option(wpk_plan* plan, int32_t key, int64_t value);

/* Per-tile execution log of the last logged step, one record per tile id. */
typedef struct wpk_log_rec {
  int32_t exec_count;   /* times the tile ran this step (must be 1) */
  int32_t wait_delta;   /* counter sum observed at start minus its target (must be 0) */
  int32_t worker;       /* worker (workgroup) that ran it */
  int32_t claim;        /* position in its claim queue */
  int64_t t_start;      /* s_memrealtime (100 MHz) after the wait was satisfied */
  int64_t t_end;        /* s_memrealtime before the tile published */
} wpk_log_rec;
/* Copies the n_tiles tile records.  On a device plan, when `bytes` holds
 * 3 * n_tiles + max_workers records, the rest follows in two parts:
 *  - max_workers worker records (slot w = workgroup w; only the first
 *    `workers` are written): exec_count = the HW_ID hardware register (wave,
 *    SIMD, CU, shader engine), wait_delta = the XCC_ID register, worker = w,
 *    claim = 0, t_start / t_end = s_memrealtime at kernel entry / before the
 *    exit count;
 *  - n_tiles timing records (wpk_tile_timing, 64 bytes each, by tile id).
 * All times are s_memrealtime ticks (100 MHz); a logged step also waits for
 * each slot's loads before its arithmetic, so it runs slightly slower. */
typedef struct wpk_tile_timing {
  int64_t t_claim;         /* control wave took the tile (before waiting on its group) */
  int64_t t_inputs;        /* inputs staged in LDS (last batch row) */
  int64_t t_slot_ready;    /* the last compute wave had its staged weights (last batch row) */
  int64_t t_compute_done;  /* the last compute wave finished its arithmetic */
  int64_t t_partials;      /* all partial sums ready: the control wave passed barrier B */
  int64_t t_end;           /* epilogue stores complete, before the publish */
  int64_t reserved[2];
} wpk_tile_timing;
int32_t wpk_get_log(wpk_plan* plan, void* host_dst, size_t bytes);

/* Shape of the built DAG. */
typedef struct wpk_plan_info {
  int32_t n_tiles;        /* tiles (= log records) */
  int32_t n_groups;       /* dependency counter groups */
  int32_t n_queue_shards; /* claim queues */
  int32_t workers;        /* W resident workers launched per step */
  int32_t max_workers;    /* co-residency limit found at build */
  int32_t rows_per_tile_h;/* rows of a K=hidden GEMV tile */
  int32_t rows_per_tile_f;/* rows of a K=ffn GEMV tile */
  int32_t attn_chunk;     /* KV positions per attention partial */
  int64_t workspace_bytes;
  int64_t weight_bytes;   /* bytes of weights one step streams */
} wpk_plan_info;
int32_t wpk_get_info(const wpk_plan* plan, wpk_plan_info* out);

/* Tile table of the DAG: for each tile id, its type (0 qkv, 1 attention
 * partial, 2 combine, 3 o-proj, 4 gate/up, 5 down, 6 lm-head, 7 argmax),
 * layer, the counter group it waits on (-1 none) and the group it signals
 * (-1 none).  Edge u -> v exists iff signal[u] == wait[v].  Arrays of n_tiles. */
int32_t wpk_get_dag(const wpk_plan* plan, int32_t* type, int32_t* layer, int32_t* wait,
                    int32_t* signal);

/* The same decode step as one kernel per operation (about 6 per layer),
 * captured once into a hipGraph and replayed by wpk_step: the conventional
 * baseline, sharing the megakernel's tile bodies.  The graph is captured on
 * the first wpk_step and re-captured if tokens/kv/logits pointers change. */
wpk_plan* wpk_build_graph_baseline(const wpk_model_desc* desc, int32_t batch, int32_t ctx_len);

/* ---- host-side executors (no GPU) ----------------------------------------------
 * wpk_build_host compiles the same DAG for a model in HOST memory.
 * wpk_serial_step runs one step's tiles on the CPU, one at a time, in a
 * topological order drawn from order_seed (Kahn's algorithm with a seeded
 * tie-break); with poison != 0 every intermediate buffer is filled with NaN
 * first, so a tile that ran before one of its producers poisons the result.
 * wpk_emulate_step runs the device protocol (claim from the sharded queues,
 * wait on counters with acquire loads, publish with release increments) with
 * n_threads std::threads as workers and seeded random delays.
 * Both fill the plan's log (wpk_get_log); all pointers are host memory. */
wpk_plan* wpk_build_host(const wpk_model_desc* desc, int32_t batch, int32_t ctx_len,
                         const wpk_build_opts* opts);
int32_t wpk_serial_step(wpk_plan* plan, int32_t* tokens, wpk_kv* kv, float* logits,
                        uint64_t order_seed, int32_t poison);
int32_t wpk_emulate_step(wpk_plan* plan, int32_t* tokens, wpk_kv* kv, float* logits,
                         int32_t n_threads, uint64_t seed);
/* Test hook for the host executors: drop the wait of tile `tile` (it no longer
 * waits on its counter group), or with tile = -1 restore the built DAG. */
int32_t wpk_debug_drop_edge(wpk_plan* plan, int32_t tile);
/* Inspection hook: copies the plan's activation arena (all per-layer
 * intermediate buffers, in the layout the host executors use, so the two can be
 * compared buffer by buffer) into host memory.  bytes must be at least the
 * arena size; *out_bytes receives it.  Device plans synchronize the device
 * first.  Returns 0 or a negative WPK_E code. */
int32_t wpk_debug_read_act(wpk_plan* plan, void* host_dst, size_t bytes, size_t* out_bytes);

#ifdef __cplusplus
}
#endif
#endif /* WPK_H */
