// host_exec.h -- CPU executors of a built DAG (no GPU needed).
#pragma once
#include <cstdint>
#include <string>

#include "runtime.h"

namespace wpk {

// Build a plan whose weights and buffers are in host memory.
wpk_plan* make_host_plan(const wpk_model_desc& d, int32_t batch, int32_t ctx_len, const wpk_build_opts& o,
                         std::string* err);

// One step, tiles run one at a time in a seeded random topological order.
int32_t host_serial_step(wpk_plan* p, int32_t* tokens, wpk_kv* kv, float* logits, uint64_t seed,
                         bool poison);

// One step, the device claim/wait/publish protocol run by n_threads threads.
int32_t host_emulate_step(wpk_plan* p, int32_t* tokens, wpk_kv* kv, float* logits, int32_t n_threads,
                          uint64_t seed);

}  // namespace wpk
