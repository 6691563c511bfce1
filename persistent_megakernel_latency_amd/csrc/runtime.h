// runtime.h -- the plan object behind the C ABI (host side).
#pragma once
#include <atomic>
#include <memory>
#include <string>
#include <vector>

#include "builder.h"
#include "plan.h"
#include "wpk.h"

namespace wpk {

// Host memory for a plan that runs on the CPU (serial executor / emulator).
struct HostWorkspace {
  std::vector<float> act;                     // all per-layer activation buffers
  std::vector<LayerBufs> layers;
  std::vector<float> rope_cos, rope_sin;      // [cap][D/2]
  std::unique_ptr<std::atomic<unsigned long long>[]> argmax;  // [B][kArgmaxShards]
  std::vector<float> wpart;                   // wide plans: partial-sum slots
  std::vector<uint32_t> fixc;                 // wide plans: arrival counters (stride kLine), zeroed per step
};

// RoPE table: cos/sin of pos * theta^(-2i/D), computed in float64, stored float32.
void rope_table(const Shape& s, std::vector<float>& cos_t, std::vector<float>& sin_t);

// Bytes of the per-layer activation buffers and their placement.
struct ActLayout {
  int64_t x_mid, x_out, q, part, attn, h;  // float offsets within a layer
  int64_t xn1, xattn, xn2, xh, xnf;        // wide plans: bf16 hi/lo planes [2][32][K] (float offsets; 0 size otherwise)
  int64_t ss1, ss2, ssf;                   // wide plans: RMSNorm sums of squares [H/64][32] (0 size otherwise)
  int64_t per_layer;
  int64_t total;                                      // floats for all layers
};
ActLayout act_layout(const Shape& s);

// Fill per-layer LayerBufs given the weight tables and an activation arena.
void fill_layers(const Shape& s, const wpk_model_desc& d, float* act, std::vector<LayerBufs>& out);

}  // namespace wpk

struct wpk_plan {
  bool host = false;      // compiled for the host executors only
  bool baseline = false;  // per-operator hipGraph baseline
  wpk::Shape s{};
  wpk::Dag dag;
  std::vector<int32_t> built_wait;  // waits as built (restored by wpk_debug_drop_edge(-1))
  wpk_model_desc desc{};
  std::vector<const void*> tables;  // copies of the caller's per-layer pointer tables
  std::string err;
  std::vector<wpk_log_rec> log;     // host copy of the last log
  int32_t latched = 0;              // device error seen by wpk_sync
  int32_t log_on = 0, prefetch = 1, drop_tile = -1, cooperative = 0;
  int32_t emu_fixed_reducer = 0;    // host emulator: fixed reducer per wide row block (WPK_OPT_FIXED_REDUCER)
  // cross-step persistence (wpk_persist_*)
  bool persist_open = false;
  uint32_t* host_words = nullptr;   // pinned host memory: [0] doorbell, [64] steps done
  uint32_t persist_requested = 0;   // steps rung since the session began
  uint64_t persist_idle_us = 2000000;
  uint64_t* d_step_times = nullptr; // inside the workspace: [kPersistTimes][2]
  uint32_t perturb = 0;
  uint64_t watchdog_us = 2000000;
  int64_t weight_bytes = 0;

  // host executors
  wpk::HostWorkspace hw;

  // device side (filled by the C ABI on a GPU)
  int device = -1;
  int n_cu = 0;
  int workers = 0, max_workers = 0;
  char* d_ws = nullptr;             // one allocation holding everything the plan owns
  bool static_ws = false;           // d_ws is the device's static scratch array (wpk_build_static)
  int64_t ws_bytes = 0;
  wpk::Params P{};                  // device pointers; step I/O filled per call
  const void* k_mega = nullptr;     // kernel handles
  const void* k_mega_log = nullptr;
  const void* k_phase = nullptr;
  const void* k_persist = nullptr;  // persistent grid kernel (narrow plans only)
  int dyn_lds = 0;                  // dynamic LDS bytes of the kernels (wide plans)
  // two co-resident megakernels (wpk_build_opts.split_workers): the last
  // split_workers workers of the launch form the second
  int split_workers = 0;
  void* last_stream = nullptr;
  // baseline graph
  void* graph_exec = nullptr;
  void* graph = nullptr;
  void* cap_tokens = nullptr;
  void* cap_kc = nullptr;
  void* cap_vc = nullptr;
  void* cap_seq = nullptr;
  void* cap_logits = nullptr;
  void* cap_stream = nullptr;
};
