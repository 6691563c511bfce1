// prefill_builder.h -- host-side compilation of a prompt prefill into a tile DAG.
#pragma once
#include <string>
#include <utility>
#include <vector>

#include "plan.h"
#include "prefill_plan.h"
#include "wpk.h"

namespace wpk {

struct PShape {
  int32_t L, H, Hq, Hkv, D, F, V, B, cap, G, qkv_rows;
  int32_t P, Pp, nrb_s, R;  // prompt length, rows per sequence, row blocks per sequence, rows
  int32_t nqb;              // 64-query attention blocks per sequence
  int32_t queue_shards;     // claim queues of each region
  int32_t split;            // attention tiles in a second co-resident megakernel (their own queues)
  float theta, eps;
};

struct PDag {
  std::vector<Tile> tiles;         // claim (topological) order; tiles[i].id == i
  std::vector<Group> groups;
  std::vector<int32_t> queue;      // claim queues, concatenated
  std::vector<int32_t> queue_off;  // n_queues + 1 offsets
  int32_t n_shard_slots = 0;
  int32_t split_queues = 0;        // split plans: queues [0, split_queues) hold every tile but attention
  std::vector<std::pair<int32_t, int32_t>> phases;  // runs of one (layer, type): the per-operator baseline
};

// Checks the model and prompt against what the prefill kernels support and
// fills the geometry.  Empty string, or the reason for refusal.
std::string check_prefill_shape(const wpk_model_desc& d, int32_t batch, int32_t ctx_len, int32_t prompt_len,
                                int32_t split, PShape* out);

PDag build_prefill_dag(const PShape& s);

// Structural checks: ids, every producer of a tile's group claimed before it,
// producer counts, every output region produced exactly once, and every
// tile's inputs produced by the group it waits on.  Empty string when valid.
std::string validate_prefill_dag(const PShape& s, const PDag& d);

// The planner's prediction for a prefill design: a discrete-event replay of
// the plan's DAG and claim queues with measured per-tile costs (see
// prefill_builder.cpp).  workers: W; split_workers: the attention pool of a
// split plan (0 otherwise); conventional: one kernel per operator phase.
struct PSimCost {
  double tile_us[P_NTYPES];  // per tile type (attention: fixed part)
  double attn_step_us;       // attention: per 32-key step of the tile's causal span
  double hop_us;             // a publish seen by a waiting worker
  double launch_gap_us;      // conventional: between two operators' kernels
};
double simulate_prefill(const PShape& s, const PDag& d, const PSimCost& c, int workers, int split_workers,
                        bool conventional, double* busy_frac);

// 32-key steps of an attention tile's causal span (0 for other tiles).
int32_t prefill_key_steps(const PShape& s, const Tile& t);

// FLOPs of the prefill's matrix products (QKV, o, gate/up, down over all
// prompt rows, causal QK and PV over the prompt, the LM head on the last rows).
double prefill_flops(const PShape& s);

}  // namespace wpk
