// persist.hip -- cross-step persistence: the megakernel's grid kept resident
// across decode steps (a translation unit of its own; see worker.h).
#include "worker.h"

namespace wpk {

// ---- cross-step persistence ------------------------------------------------------------
// (WPK keeps "the same cooperative grid" resident across updates: "Why
// real-time inference wants a megakernel", sections "The unit of execution"
// and "A concrete design: one WPK update".)

__device__ __forceinline__ uint32_t ld_system(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ void st_system(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Control wave, at the start of step `epoch` of a persistent grid: true once
// the step is granted, false when every worker is to leave.  Worker 0 turns
// the host's doorbell into the grant (CTL_GO, an absolute epoch) and decides
// to stop on a stop bell, a latched error or after the idle limit; the others
// only read CTL_GO, so all workers take the same decision for every step.
__device__ __forceinline__ bool await_grant(const Params& P, uint32_t epoch, int lane) {
  const uint32_t want = epoch + 1u;
  const bool leader = blockIdx.x == 0;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    const uint32_t g = ld_sc1(&P.ctl[CTL_GO]);
    if (g == kGoStop) return false;
    if ((int32_t)(g - want) >= 0) {
      compiler_order();
      return true;
    }
    const uint64_t waited = __builtin_amdgcn_s_memrealtime() - t0;
    if (leader) {
      const uint32_t bell = ld_system(P.host_bell);
      uint32_t grant = 0;
      if (bell == kBellStop || ld_sc1(&P.ctl[CTL_STATUS]) != 0u || ld_sc1(&P.ctl[CTL_ABORT]) != 0u) {
        grant = kGoStop;
      } else if ((int32_t)(P.persist_base + bell - want) >= 0) {
        grant = P.persist_base + bell;
      } else if (waited > P.idle_ticks) {
        if (lane == 0) latch_error(P, WPK_E_IDLE, -1);
        grant = kGoStop;
      }
      if (grant != 0u) {
        if (lane == 0) st_sc1(&P.ctl[CTL_GO], grant);
        wait_all_memory();
        continue;
      }
    } else if (waited > P.idle_ticks + P.watchdog_ticks) {  // worker 0 always decides first
      if (lane == 0) latch_error(P, WPK_E_TIMEOUT, -1);
      return false;
    }
    __builtin_amdgcn_s_sleep(8);
  }
}

// Control wave, after its exit count: wait until the last worker out has
// rewound the queues and advanced the epoch (bounded).
__device__ __forceinline__ void await_epoch(const Params& P, uint32_t epoch, int lane) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (ld_sc1(&P.ctl[CTL_EPOCH]) == epoch) {
    if (ld_sc1(&P.ctl[CTL_ABORT]) != 0u) break;
    if (__builtin_amdgcn_s_memrealtime() - t0 > P.watchdog_ticks) {
      if (lane == 0) latch_error(P, WPK_E_TIMEOUT, -1);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  compiler_order();
}

// A persistent grid (narrow plans): the same worker loops as megakernel, one
// step per grant, with an epoch barrier between steps (the last worker out
// rewinds the queues and advances the epoch; the others wait for it).  Kept a
// kernel of its own so that the single-step kernel's code is unchanged: in one
// function with the single step the round loop made the compiler keep much
// more live across it (SGPR and VGPR spills to scratch in every instance).
// Matrix-core plans have no persistent instance: a matrix-core single-step
// kernel compiled with this loop faulted the device, cause not found.
template <typename WT, int CPR_H, int CPR_F>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void persistent_megakernel(Params P) {
  using SM = typename Lds<WT, CPR_H, CPR_F, false>::type;
  __shared__ SM sm;
  const int t = wpk_tid(), lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int q = (int)blockIdx.x % P.n_queues;
  const int qb = cload(P.queue_off, q), qn = cload(P.queue_off, q + 1) - qb;
  uint32_t* head = P.heads + (size_t)q * kLine;
  for (;;) {
    uint32_t epoch = 0;
    if (wave == 0) {
      epoch = ld_sc1(&P.ctl[CTL_EPOCH]);
      const bool run = await_grant(P, epoch, lane);
      if (run && blockIdx.x == 0 && lane == 0)
        __hip_atomic_store(&P.step_times[2 * ((epoch - P.persist_base) % kPersistTimes)],
                           (uint64_t)__builtin_amdgcn_s_memrealtime(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool dead = ld_sc1(&P.ctl[CTL_STATUS]) != 0u;
      // the first claim (-1: leave); compute wave 1 then claims each next tile
      int first = 0;
      if (lane == 0) first = !run ? -1 : dead ? qn : (int)atomic_add(head, 1u);
      step_start<WT>(P, sm, lane, first);
    }
    __syncthreads();
    const int cur = __builtin_amdgcn_readfirstlane(sm.first);
    if (cur < 0) break;
    if (wave == 0) control_loop<WT, CPR_H, CPR_F, false, false>(P, sm, cur, qb, qn, epoch, lane);
    else compute_loop<WT, CPR_H, CPR_F, false, false>(P, sm, cur, qb, qn, head, t - 64);
    __syncthreads();
    if (t == 0) {
      wait_all_memory();  // this worker's stores are complete before it counts itself out
      const uint32_t old = atomic_add(&P.ctl[CTL_EXIT], 1u);
      if (old == (uint32_t)P.n_workers - 1u) {
        compiler_order();
        for (int i = 0; i < P.n_queues; ++i) st_sc1(&P.heads[(size_t)i * kLine], 0u);
        st_sc1(&P.ctl[CTL_EXIT], 0u);
        wait_all_memory();  // the rewound queues are visible before the new epoch
        __hip_atomic_store(&P.step_times[2 * ((epoch - P.persist_base) % kPersistTimes) + 1],
                           (uint64_t)__builtin_amdgcn_s_memrealtime(), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        st_sc1(&P.ctl[CTL_EPOCH], epoch + 1u);
        wait_all_memory();  // the step's outputs and the epoch before the host hears of it
        st_system(P.host_done, epoch + 1u - P.persist_base);
      }
    }
    // the next step starts once every worker has left this one
    if (wave == 0) await_epoch(P, epoch, lane);
    __syncthreads();
  }
}

}  // namespace wpk

// The persistent-grid kernel for a (dtype, row geometry); 0 if there is none
// (matrix-core plans have none).
extern "C" int wpk_dev_persist_kernel(int dtype, int cpr_h, int cpr_f, int wide, const void** k) {
  using namespace wpk;
  *k = nullptr;
  if (wide) return 0;
#define WPK_PINST(DT, WT, H, F)                                                   \
  if (dtype == DT && cpr_h == H && cpr_f == F) {                                 \
    *k = reinterpret_cast<const void*>(&persistent_megakernel<WT, H, F>);        \
    return 1;                                                                    \
  }
  WPK_PINST(WPK_F32, float, 64, 256)
  WPK_PINST(WPK_BF16, uint16_t, 256, 1024)
  WPK_PINST(WPK_BF16, uint16_t, 64, 128)
  WPK_PINST(WPK_BF16, uint16_t, 64, 256)
#undef WPK_PINST
  return 0;
}
