// builder.h -- host-side compilation of one decode step into a tile DAG.
#pragma once
#include <string>
#include <utility>
#include <vector>

#include "plan.h"
#include "wpk.h"

namespace wpk {

// The operating point a plan is compiled for and the tile geometry chosen.
struct Shape {
  int32_t L, H, Hq, Hkv, D, F, V, B, cap, dtype, elt;
  int32_t G;         // q heads per kv head
  int32_t qkv_rows;  // (Hq + 2 Hkv) * D
  int32_t nch;       // KV chunks covering the capacity
  int32_t cpr_h;     // 16-byte chunks in a weight row of length hidden
  int32_t cpr_f;     // ... of length ffn
  int32_t rows_h;    // rows of a K=hidden GEMV tile
  int32_t rows_qkv;  // rows of a QKV tile (RoPE pairs (i, i+D/2) stay together)
  int32_t rows_f;    // rows of a K=ffn GEMV tile
  int32_t tile_bytes, workers_per_cu, queue_shards;
  int32_t wide;      // batch above kMaxBatchGemv: matrix-core tiles, RMSNorm split between epilogues
  int32_t attn_sub;  // KV chunks per attention tile (one slot holds up to 64 KiB of K and V)
  int32_t forward;   // chained attention tiles (LDS forwarding of the partials to the combine)
  int32_t barrier_edges;  // ablation: each consumer waits on its whole producing operator
  int32_t split_workers;  // > 0: attention and combine tiles in a second co-resident megakernel
  float theta, eps;
};

struct Dag {
  std::vector<Tile> tiles;         // in global claim (topological) order; tiles[i].id == i
  std::vector<Group> groups;
  std::vector<int32_t> queue;      // claim queues, concatenated
  std::vector<int32_t> queue_off;  // n_queues + 1 offsets
  int32_t n_shard_slots = 0;
  int32_t n_fix = 0;     // wide plans: row blocks (arrival counters)
  int32_t n_pslots = 0;  // wide plans: partial-sum slots (one per wide GEMM tile)
  // split plans: queues [0, split_queues) hold every tile but attention and
  // combine (the first megakernel), the rest those (the second); 0: one region
  int32_t split_queues = 0;
  // runs of tiles of one (layer, type), in order: the operators of the
  // conventional one-kernel-per-operator baseline
  std::vector<std::pair<int32_t, int32_t>> phases;
};

// Checks the model/batch/context against what the kernels support and fills
// the tile geometry.  Returns an empty string or the reason for refusal.
std::string check_shape(const wpk_model_desc& d, int32_t batch, int32_t ctx_len,
                        const wpk_build_opts& o, Shape* out);

Dag build_dag(const Shape& s);

// Structural checks of a built DAG: ids, topological claim order, every
// output element produced exactly once, and every tile's inputs produced by
// the producers of the group it waits on.  Empty string when valid.
std::string validate_dag(const Shape& s, const Dag& d);

// Extra constraints of the gfx950 kernels: 32-bit offsets within a matrix or
// a KV cache slice, and GEMV tiles made of whole 4 KiB row slices.
std::string check_device_geometry(const Shape& s, const Dag& d);

// Weight bytes one step streams (matrices once each, norm gains once each).
int64_t step_weight_bytes(const Shape& s);

}  // namespace wpk
