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
#define WPK_E_IDLE (-10)        /* a persistent grid waited longer than its idle limit for a step and left */
#define WPK_E_RANGE (-11)       /* a prefill activation of the fp16 products overflowed |x| >= 65520 (device) */

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
  int32_t barrier_edges;    /* ablation of the tile-to-tile tensor edges ("One Megakernel is Not
                               Enough", Table I, cross-kernel readiness): 1 makes every tile wait
                               for ALL tiles of the operator it reads from, as a per-operator
                               barrier would; 0 (default): only for the tiles producing its inputs */
  int32_t split_workers;    /* two co-resident megakernels ("One Megakernel is Not Enough": the
                               abstract, several megakernels sharing the GPU; Table I, smaller CTA
                               budget): 0 (default) runs the step as one megakernel; N > 0 gives the
                               attention and combine tiles a megakernel of their own: the last N
                               workers of the launch claim only from the attention and combine
                               queues, the others only from the queues of every other tile, and the
                               two wait on each other's tiles through the same counters.  Each needs
                               at least one worker per claim queue.  The workers' placement on CUs
                               is the dispatcher's (a CU-masked stream per megakernel, the MI355X
                               analogue of partitioning the streaming multiprocessors, could not be
                               created on the test machine).  Device plans from wpk_build_ex; no
                               persistent session; WPK_OPT_WORKERS is refused. */
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

/* Wait for the plan's last step and return the latched device status.
 * Source: "Why real-time inference wants a megakernel", section "What a
 * megakernel does not solve", under "It increases compiler and verification
 * burden": a megakernel must surface its failures (deadlock, a stuck
 * dependency) and keep enough execution state to locate them.  Device-side
 * errors are latched by the workers, never raised mid-step; wpk_sync is where
 * the host learns of them, with the failing tile, worker and step, and for a
 * watchdog timeout the first counter group that was short of publishes. */
int32_t wpk_sync(wpk_plan* plan);

void wpk_destroy(wpk_plan* plan);

/* Last error message of the plan, or of the calling thread if plan is NULL. */
const char* wpk_last_error(const wpk_plan* plan);

/* Runtime options (keys below).  Returns WPK_E_ARG for an unknown key/value.
 * Sources: the ablation keys switch the features that "One Megakernel is Not
 * Enough", Table I, models one at a time -- WPK_OPT_PREFETCH the weight
 * prefetch into the per-worker staging slot, WPK_OPT_WORKERS the worker count
 * W -- and WPK_OPT_LAUNCH the residency guarantee the persistent-threads page
 * asks of a persistent kernel (section 2: every worker resident for the whole
 * run).  WPK_OPT_LOG, WPK_OPT_WATCHDOG_US, WPK_OPT_DEBUG_DROP_TILE and
 * WPK_OPT_RESET serve the failure handling of "Why real-time inference wants a
 * megakernel", "What a megakernel does not solve" (find and survive a stuck
 * dependency); WPK_OPT_PERTURB_SEED exercises other claim and completion
 * orders, which must not change the numbers (same section: preserve numerical
 * behaviour through reordering).  Every key applies to later steps only. */
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
#define WPK_OPT_FIXED_REDUCER 9   /* host plans only, wpk_emulate_step: 1 makes each wide row block's
                                     last slice in claim order its reducer, which waits for the other
                                     slices' arrivals, instead of the last slice to arrive; device plans
                                     refuse it (a device run of this scheme once faulted, cause unknown) */
#define WPK_OPT_PERSIST_IDLE_US 10 /* persistent sessions: a grid left this long without a step leaves
                                      by itself and reports WPK_E_IDLE (default 2,000,000) */
int32_t wpk_set_option(wpk_plan* plan, int32_t key, int64_t value);

/* Per-tile execution log of the last logged step, one record per tile id.
 * Source: "Why real-time inference wants a megakernel", "What a megakernel
 * does not solve" ("It increases compiler and verification burden"): the
 * runtime records enough execution state to check that every task ran once,
 * after its dependencies, and to locate a failure.  Layout: dst receives
 * wpk_log_rec records (host memory, caller-owned, `bytes` long); returns
 * WPK_E_ARG if bytes cannot hold n_tiles records, WPK_E_HIP if the copy
 * fails.  Synchronous. */
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
  int64_t t_stored;        /* matrix-core GEMM tiles: the K slice's partial sums stored (else 0) */
  int64_t t_arrived;       /* matrix-core GEMM tiles: its arrival counted; bit 63 set for the last
                              slice of its row block, which then adds up the others (else 0) */
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

/* Source: the conventional execution the pages measure megakernels against --
 * "persistent-threads-megakernels", section 3 (one launch per operation, the
 * boundaries between them replayed from a captured graph) and section 7
 * (compare against the graph-replayed baseline) -- and the TensorRT-style
 * one-kernel-per-operator design of "One Megakernel is Not Enough".
 * The same decode step as one kernel per operation (about 6 per layer),
 * captured once into a hipGraph and replayed by wpk_step: the conventional
 * baseline, sharing the megakernel's tile bodies.  The graph is captured on
 * the first wpk_step and re-captured if tokens/kv/logits pointers change. */
wpk_plan* wpk_build_graph_baseline(const wpk_model_desc* desc, int32_t batch, int32_t ctx_len);

/* ---- cross-step persistence ------------------------------------------------------
 * Source: "Why real-time inference wants a megakernel", section "The unit of
 * execution" (the grid of a WPK stays resident across updates instead of
 * being launched per update) and section "A concrete design: one WPK update"
 * (the host keeps admission and delivery; the device publishes completion).
 * A session keeps the megakernel's grid resident and runs one decode step per
 * step the host rings, with no launch in between: the host writes a doorbell
 * in pinned host memory, worker 0 turns it into a grant in device memory,
 * every worker runs the step, and the last worker out advances the epoch and
 * writes the count of finished steps back to pinned host memory.  Steps chain
 * their tokens on the device, as with wpk_step (free-running greedy decoding);
 * tokens, kv and logits are device memory, caller-owned, and must not be
 * touched by the caller while the session runs.  The grid is launched
 * cooperatively (all workers co-resident) on `stream`.
 *
 * wpk_persist_begin: opens the session (the plan must be idle, with the log
 *   off); returns WPK_E_STATE if one is open or an error is latched.
 * wpk_persist_ring: asks for n_steps more steps (non-blocking).
 * wpk_persist_wait: waits until `steps` of the rung steps have finished;
 *   WPK_E_TIMEOUT after timeout_us (negative: no limit), WPK_E_STATE if the
 *   grid has already left.
 * wpk_persist_end: lets the rung steps finish, stops the grid, waits for it and
 *   returns its latched status, as wpk_sync does (WPK_E_IDLE if it left after
 *   the idle limit, WPK_OPT_PERSIST_IDLE_US).  wpk_step and wpk_sync refuse to
 *   run while a session is open; wpk_destroy ends an open session.
 * wpk_persist_times: after the session, two s_memrealtime stamps (100 MHz) per
 *   step into dst[2 * i], dst[2 * i + 1]: when worker 0 saw step i granted and
 *   when the last worker left it (the first n_steps of a 4096-entry ring). */
int32_t wpk_persist_begin(wpk_plan* plan, int32_t* tokens, wpk_kv* kv, void* logits, wpk_stream_t stream);
int32_t wpk_persist_ring(wpk_plan* plan, int32_t n_steps);
int32_t wpk_persist_wait(wpk_plan* plan, int32_t steps, int64_t timeout_us);
int32_t wpk_persist_end(wpk_plan* plan);
int32_t wpk_persist_times(wpk_plan* plan, int64_t* dst, int32_t n_steps);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * plan as wpk_build, with its whole workspace placed in a static device array
 * of WPK_STATIC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; no hipMalloc, hipFree or other allocating call is
 * made for device memory (host bookkeeping uses the C++ heap).  The caller
 * still passes tokens, the KV cache and logits to wpk_step.  A plan whose
 * workspace does not fit is refused (NULL; wpk_last_error(NULL) gives the
 * bytes it needs).  All static plans of one GPU share its array: building one
 * clears the part it uses and takes the array over, after which an earlier
 * static plan of that GPU refuses to step (WPK_E_STATE) until rebuilt.  Steps
 * of two static plans that overlap in time on one GPU race on the array.  The
 * batch-1 Llama-3.2-1B-shaped plan needs about 12 MiB; matrix-core plans
 * (batches above 4) of that model do not fit. */
#define WPK_STATIC_SCRATCH_BYTES (32u << 20)
wpk_plan* wpk_build_static(const wpk_model_desc* desc, int32_t batch, int32_t ctx_len);

/* ---- planner: the step time of a candidate design, predicted ----------------------
 * Source: "One Megakernel is Not Enough: Predicting Where to Cut for Streaming
 * Inference" -- the abstract and Table I: a planner takes per-operator
 * profiles, simulates the tile and event graph of each candidate design under
 * the modelled features (tile-to-tile readiness edges vs barrier edges,
 * weight prefetch into a one-slot staging buffer, the worker count W, kernel
 * boundaries of the conventional design) and picks the fastest.
 * wpk_simulate runs that simulation on the plan's own DAG and claim queues
 * (build it with the options of the candidate: barrier_edges, queue count;
 * a host plan is enough).  Costs are per tile type (indices of wpk_get_dag's
 * types), in microseconds: input staging after the wait, compute once the
 * weights are in, epilogue through the publish, and for matrix-core plans the
 * row-block reduction of the last K slice.  positions: host int32[batch],
 * the sequence lengths at step start (attention tiles stream the K/V of the
 * chunks holding positions; NULL counts none).  The conventional design
 * (conventional = 1) runs each operator as one kernel over `workers`
 * workgroups, separated by launch_gap_us, with no hops.  Returns WPK_E_ARG on a
 * bad parameter; deterministic; host only. */
#define WPK_SIM_TYPES 12
typedef struct wpk_sim_params {
  double hbm_GBps;           /* streaming bandwidth (one first-come server) */
  double load_latency_us;    /* latency of a staged load, on top of its streaming time */
  double hop_us;             /* last producer's publish to the consumer seeing its group complete */
  double launch_gap_us;      /* conventional design: between two operators' kernels */
  int32_t workers;           /* W (at least the plan's queue count) */
  int32_t prefetch;          /* 1: weights load when the slot frees; 0: once the inputs are complete */
  int32_t conventional;      /* 1: one kernel per operator instead of the megakernel */
  int32_t slots;             /* staging slots per worker (0 or 1: one; a design candidate above 1) */
  double stage_us[WPK_SIM_TYPES];
  double compute_us[WPK_SIM_TYPES];
  double epilogue_us[WPK_SIM_TYPES];
  double reduce_us[WPK_SIM_TYPES];  /* matrix-core plans: added to the epilogue of the K slice whose
                                       arrival completes its row block (it adds up the others) */
} wpk_sim_params;
typedef struct wpk_sim_result {
  double step_us;            /* predicted step time (last publish or last kernel end) */
  double hbm_bytes;          /* bytes the simulated step streamed */
  double achieved_GBps;      /* hbm_bytes / step_us */
  double worker_busy_frac;   /* share of worker time between a tile's start and its publish */
} wpk_sim_result;
int32_t wpk_simulate(const wpk_plan* plan, const wpk_sim_params* params, const int32_t* positions,
                     wpk_sim_result* out);

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

/* ---- prompt prefill: time to first token ---------------------------------------
 * Source: "One Megakernel is Not Enough", Table III (the Llama 3.2 1B row:
 * time to first token for a 496-token prompt, batches up to 48) and the
 * abstract and Table I (producer-consumer overlap of a split region with its
 * own smaller CTA budget; one megakernel against several co-resident ones and
 * against the conventional per-operator execution).  The prefill runs the
 * whole prompt of every sequence through every layer at once -- RMSNorm, QKV
 * with RoPE, the K/V of all prompt positions appended to the cache, causal
 * grouped-query attention over the prompt, o-projection, SwiGLU MLP -- and
 * the tied LM head on each sequence's last prompt position gives the first
 * generated token (greedy, lowest index on ties).  Matrix products run on the
 * matrix cores with fp32 accumulation.  QKV, the attention products and the
 * LM head take bf16 weights (or K/V) against activations split into bf16 hi +
 * lo parts (two products, ~16 significant bits); the o-projection, gate/up
 * and down take fp16 copies of their weights against fp16 activations (one
 * product, 11 bits).  The residual stream, RMSNorm, RoPE and softmax run in
 * fp32.  An activation entering an fp16 product that overflows (|x| >=
 * 65520) latches WPK_E_RANGE.
 *
 * wpk_build_prefill: model (DEVICE pointers, bf16 weights, hidden a multiple
 *   of 256 up to 4096, ffn a multiple of 128, n_q_heads + 2 n_kv_heads a
 *   multiple of 4; o-proj, gate, up and down weights inside the fp16 range,
 *   |w| < 65520), batch in [1, 32],
 *   ctx_len (the KV cache capacity), prompt_len in [1, ctx_len].  opts (NULL:
 *   defaults) picks the execution:
 *     WPK_PREFILL_MEGAKERNEL: one persistent kernel, all tiles;
 *     WPK_PREFILL_SPLIT: two co-resident megakernels in one launch -- the last
 *       split_workers workers (default an eighth) claim only the attention
 *       tiles, the others every other tile, and they wait on each other
 *       through the same counters;
 *     WPK_PREFILL_GRAPH: the conventional baseline, one kernel per (layer,
 *       operator) over the same tile bodies, captured once into a hipGraph.
 *   Returns NULL on error (wpk_prefill_last_error(NULL) says why).
 * wpk_build_prefill_host: the same DAG without a device (inspection only:
 *   get_info / get_dag; wpk_prefill refuses it).
 * wpk_prefill: prompt is device int32[batch][prompt_len]; kv as for wpk_step
 *   (the cache positions [0, prompt_len) of every sequence are overwritten,
 *   seq_len is set to prompt_len); logits: device float32[batch][vocab], the
 *   last prompt position's; tokens_out: device int32[batch], the first
 *   generated token.  One launch (or graph launch) enqueued on stream.  A token
 *   id outside [0, vocab) latches WPK_E_TOKEN (read by wpk_prefill_sync).
 * wpk_prefill_sync: waits for the last prefill and returns the latched device
 *   status (as wpk_sync); a latched plan refuses to run until WPK_OPT_RESET.
 * wpk_prefill_set_option: WPK_OPT_LOG (megakernel modes: per-tile log),
 *   WPK_OPT_WATCHDOG_US, WPK_OPT_RESET.
 * wpk_prefill_get_log: n_tiles wpk_log_rec of the last logged prefill
 *   (exec_count, wait_delta, worker, claim, start / end stamps).
 * wpk_prefill_get_dag: per tile id its type (wpk_prefill tile types below),
 *   layer, waited and signalled groups, and (if queue is not NULL) its claim
 *   queue.  Arrays of n_tiles.
 * Ownership and errors as for the decode step, except that a prefill plan
 * copies the layer matrices at build, repacked into the fragment-major
 * layout its matrix-core tiles load (QKV in bf16, the others in fp16; about
 * the size of the layer weights; the embedding is still read from the
 * caller's table): weights changed after the build are not seen by the
 * prefill. */
#define WPK_PREFILL_MEGAKERNEL 0
#define WPK_PREFILL_SPLIT 1
#define WPK_PREFILL_GRAPH 2
typedef struct wpk_prefill_opts {
  int32_t mode;            /* WPK_PREFILL_* (default 0) */
  int32_t split_workers;   /* WPK_PREFILL_SPLIT: workers of the attention megakernel (0: an eighth) */
  int32_t workers_per_cu;  /* 0 or 1: one eight-wave worker per compute unit (others are refused) */
} wpk_prefill_opts;
typedef struct wpk_prefill_info {
  int32_t n_tiles, n_groups, n_queues;
  int32_t workers;            /* workers launched (both megakernels of a split plan) */
  int32_t max_workers;        /* co-residency limit found at build */
  int32_t split_workers;      /* workers of the attention megakernel (split plans) */
  int32_t n_phases;           /* kernels of the per-operator baseline */
  int32_t rows_per_sequence;  /* prompt rows padded to the 128-row blocks */
  int64_t workspace_bytes;    /* device memory the plan owns, the repacked weights included */
  double flops;               /* matrix-product FLOPs of one prefill (2 per multiply-add) */
} wpk_prefill_info;
/* tile types of wpk_prefill_get_dag */
#define WPK_PTILE_EMBED 0
#define WPK_PTILE_NORM1 1
#define WPK_PTILE_QKV 2
#define WPK_PTILE_ATTN 3
#define WPK_PTILE_OPROJ 4
#define WPK_PTILE_NORM2 5
#define WPK_PTILE_GATEUP 6
#define WPK_PTILE_DOWN 7
#define WPK_PTILE_NORMF 8
#define WPK_PTILE_LM 9
#define WPK_PTILE_ARGMAX 10
typedef struct wpk_prefill_plan wpk_prefill_plan;
wpk_prefill_plan* wpk_build_prefill(const wpk_model_desc* desc, int32_t batch, int32_t ctx_len, int32_t prompt_len,
                                    const wpk_prefill_opts* opts);
wpk_prefill_plan* wpk_build_prefill_host(const wpk_model_desc* desc, int32_t batch, int32_t ctx_len,
                                         int32_t prompt_len, const wpk_prefill_opts* opts);
int32_t wpk_prefill(wpk_prefill_plan* plan, const int32_t* prompt, wpk_kv* kv, void* logits, int32_t* tokens_out,
                    wpk_stream_t stream);
int32_t wpk_prefill_sync(wpk_prefill_plan* plan);
void wpk_prefill_destroy(wpk_prefill_plan* plan);
const char* wpk_prefill_last_error(const wpk_prefill_plan* plan);
int32_t wpk_prefill_set_option(wpk_prefill_plan* plan, int32_t key, int64_t value);
int32_t wpk_prefill_get_log(wpk_prefill_plan* plan, void* host_dst, size_t bytes);
int32_t wpk_prefill_get_info(const wpk_prefill_plan* plan, wpk_prefill_info* out);
int32_t wpk_prefill_get_dag(const wpk_prefill_plan* plan, int32_t* type, int32_t* layer, int32_t* wait,
                            int32_t* signal, int32_t* queue);

/* The planner's prediction for a prefill design (source: "One Megakernel is
 * Not Enough", the abstract and Table I -- candidate designs simulated on
 * their tile and event graphs from per-operator profiles).  A discrete-event
 * replay of the plan's own DAG and claim queues: W workers (a split plan's
 * last split_workers claim only the attention queues), a tile starting when
 * its worker is free and its counter group complete plus hop_us, lasting its
 * measured cost (tile_us of its type; attention adds attn_step_us per
 * 32-key step of its causal span); with conventional = 1 each (layer,
 * operator) phase is one kernel over W workgroup slots, kernels separated by
 * launch_gap_us.  Prefill tiles are compute-bound, so no bandwidth server is
 * modelled (hbm_bytes and achieved_GBps are 0).  Host or device plans;
 * split_workers must be positive exactly for split plans.  Deterministic. */
typedef struct wpk_prefill_sim_params {
  double tile_us[11];      /* per WPK_PTILE_* type */
  double attn_step_us;
  double hop_us;
  double launch_gap_us;
  int32_t workers;
  int32_t split_workers;
  int32_t conventional;
  int32_t pad;
} wpk_prefill_sim_params;
int32_t wpk_prefill_simulate(const wpk_prefill_plan* plan, const wpk_prefill_sim_params* params,
                             wpk_sim_result* out);
/* Per tile id: the 32-key steps of an attention tile's causal span (the
 * keys of its last query, rounded up), 0 for other tiles -- the term the
 * simulation scales attn_step_us by.  Array of n_tiles. */
int32_t wpk_prefill_get_key_steps(const wpk_prefill_plan* plan, int32_t* key_steps);

#ifdef __cplusplus
}
#endif
#endif /* WPK_H */
