// megakernel.hip -- the decode step as one persistent kernel launch on gfx950
// (the worker design is described in worker.h), the conventional
// one-kernel-per-operator baseline built from the same tile bodies, and the
// static workspace of allocation-free plans.
#include <mutex>

#include "worker.h"

namespace wpk {

template <typename WT, int CPR_H, int CPR_F, bool LOG, bool WIDE>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void megakernel(Params P) {
  using SM = typename Lds<WT, CPR_H, CPR_F, WIDE>::type;
  SM* smp;
  if constexpr (WIDE) {
    extern __shared__ __align__(16) unsigned char wpk_dyn_lds[];
    smp = reinterpret_cast<SM*>(wpk_dyn_lds);
  } else {
    __shared__ SM sm_static;
    smp = &sm_static;
  }
  SM& sm = *smp;
  const int t = wpk_tid(), lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int q = cload(P.worker_queue, (int)blockIdx.x);
  const int qb = cload(P.queue_off, q), qn = cload(P.queue_off, q + 1) - qb;
  uint32_t* head = P.heads + (size_t)q * kLine;
  uint32_t epoch = 0;
  const uint64_t t_entry = LOG ? __builtin_amdgcn_s_memrealtime() : 0;
  if (wave == 0) {
    epoch = ld_sc1(&P.ctl[CTL_EPOCH]);
    const bool dead = ld_sc1(&P.ctl[CTL_STATUS]) != 0u;
    // the first claim; compute wave 1 then claims each next tile
    int first = 0;
    if (lane == 0) first = dead ? qn : (int)atomic_add(head, 1u);
    step_start<WT>(P, sm, lane, first);
  }
  __syncthreads();
  const int cur = __builtin_amdgcn_readfirstlane(sm.first);
  if (wave == 0) control_loop<WT, CPR_H, CPR_F, LOG, WIDE>(P, sm, cur, qb, qn, epoch, lane);
  else compute_loop<WT, CPR_H, CPR_F, LOG, WIDE>(P, sm, cur, qb, qn, head, t - 64);
  // leave the step; the last worker out rewinds the queues and advances the epoch
  __syncthreads();
  if (LOG && t == 0) {
    // worker record after the tile records: hardware placement, residency span
    int32_t* rec = P.log + ((size_t)P.n_tiles + blockIdx.x) * 8;
    rec[0] = (int32_t)__builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_ID: wave, SIMD, CU, SE
    rec[1] = (int32_t)__builtin_amdgcn_s_getreg((31 << 11) | 20);  // XCC_ID
    rec[2] = (int32_t)blockIdx.x;
    rec[3] = 0;
    *(uint64_t*)(rec + 4) = t_entry;
    *(uint64_t*)(rec + 6) = __builtin_amdgcn_s_memrealtime();
  }
  if (t == 0) {
    const uint32_t old = atomic_add(&P.ctl[CTL_EXIT], 1u);
    if (old == (uint32_t)P.n_workers - 1u) {
      for (int i = 0; i < P.n_queues; ++i) st_sc1(&P.heads[(size_t)i * kLine], 0u);
      st_sc1(&P.ctl[CTL_EXIT], 0u);
      st_sc1(&P.ctl[CTL_EPOCH], epoch + 1u);
    }
  }
}


// One operator of the conventional baseline: one workgroup per tile, the same
// tile bodies and roles, no counters; kernel boundaries order the operators.
template <typename WT, int CPR_H, int CPR_F, bool WIDE>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void phase_kernel(Params P, int first) {
  using SM = typename Lds<WT, CPR_H, CPR_F, WIDE>::type;
  SM* smp;
  if constexpr (WIDE) {
    extern __shared__ __align__(16) unsigned char wpk_dyn_lds[];
    smp = reinterpret_cast<SM*>(wpk_dyn_lds);
  } else {
    __shared__ SM sm_static;
    smp = &sm_static;
  }
  SM& sm = *smp;
  const int t = wpk_tid(), lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const Tile T = cload(P.tiles, first + (int)blockIdx.x);
  if (wave == 0) step_start<WT>(P, sm, lane, 0);
  __syncthreads();
  const int npairs = n_passes<WIDE>(P, T, sm.pos[T.b]);
  // the roles never share registers: the slot is live only in the compute waves
  if (wave == 0) {
    int xkey = -1;
    AttnRun run;
    attn_run_init(run);
    for (int b = 0; b < npairs; ++b) {
      const Tile Tb = is_attn(T.type) ? sub_chunk(T, b) : T;
      const EpiIn e = ctl_pre<WT, CPR_H, CPR_F, WIDE>(P, Tb, b, sm, lane, xkey);
      __syncthreads();  // A
      __syncthreads();  // B
      ctl_post<WT, CPR_H, CPR_F, WIDE>(P, Tb, b, sm, e, lane, xkey);
      if (WIDE && is_attn(T.type) && attn_count(P, Tb, sm.pos[T.b]) > 0) attn_run_merge(P, run, sm, lane);
    }
    if (WIDE && T.type == T_ATTN) attn_run_partial(P, T, run, sm, lane);
    if (WIDE && T.type == T_ATTNC) attn_run_store<WIDE>(P, T, run, attn_active(P, sm.pos[T.b]), lane);
  } else {
    const int tc = t - 64;
    Slot s;
#pragma unroll
    for (int j = 0; j < kChunks; ++j) s.c[j] = u32x4{0u, 0u, 0u, 0u};
    const int valid = attn_valid(P, sm.pos[T.b]);
    const uint32_t voff = (uint32_t)tc * 16u;
    if (WIDE && is_gemv(T.type)) stage_wide(P, T, s, tc);
    else stage<WT, CPR_H, CPR_F>(P, WIDE && T.type == T_ATTNC ? attn_group<WT>(T, 0) : T, s, voff, valid);
    for (int b = 0; b < npairs; ++b) {
      const Tile Tb = is_attn(T.type) ? sub_chunk(T, b) : T;
      if (is_attn(T.type)) {
        if (b > 0) {
          if (WIDE && T.type == T_ATTNC && b % (kChunks / kv_chunks<WT>()) == 0)
            stage<WT, CPR_H, CPR_F>(P, attn_group<WT>(T, b), s, voff, valid);
          else
            slot_shift<WT>(s);
        }
        if (attn_count(P, Tb, sm.pos[T.b]) > 0) dump_kv<WT>(P, Tb, s, sm, tc);
      }
      __syncthreads();  // A
      launder(s);
      compute<WT, CPR_H, CPR_F, WIDE>(P, Tb, s, sm, tc);
      __syncthreads();  // B
    }
  }
}

}  // namespace wpk

// Kernel handles for a (dtype, row geometry, wide); 0 if that instance is not
// built.  *dyn_lds: dynamic LDS bytes the instance is launched with.
extern "C" int wpk_dev_kernels(int dtype, int cpr_h, int cpr_f, int wide, const void** mk, const void** mk_log,
                               const void** phase, int* dyn_lds) {
  using namespace wpk;
#define WPK_INST(DT, WT, H, F, W)                                                         \
  if (dtype == DT && cpr_h == H && cpr_f == F && (wide != 0) == W) {                      \
    *mk = reinterpret_cast<const void*>(&megakernel<WT, H, F, false, W>);                 \
    *mk_log = reinterpret_cast<const void*>(&megakernel<WT, H, F, true, W>);              \
    *phase = reinterpret_cast<const void*>(&phase_kernel<WT, H, F, W>);                   \
    *dyn_lds = W ? (int)sizeof(typename Lds<WT, H, F, W>::type) : 0;                      \
    return 1;                                                                             \
  }
  WPK_INST(WPK_F32, float, 64, 256, false)        // hidden 256, ffn 1024, f32 (tiny)
  WPK_INST(WPK_BF16, uint16_t, 256, 1024, false)  // hidden 2048, ffn 8192, bf16 (Llama-3.2-1B shape)
  WPK_INST(WPK_BF16, uint16_t, 64, 128, false)    // hidden 512, ffn 1024, bf16
  WPK_INST(WPK_BF16, uint16_t, 64, 256, false)    // hidden 512, ffn 2048, bf16
  WPK_INST(WPK_BF16, uint16_t, 256, 1024, true)   // Llama-3.2-1B shape, batches 5..32
  WPK_INST(WPK_BF16, uint16_t, 64, 128, true)     // hidden 512, ffn 1024, batches 5..32
#undef WPK_INST
  return 0;
}

// Threads per worker the kernels are built for (one control wave + compute waves).
extern "C" int wpk_dev_block_threads() { return wpk::kBlock; }

// ---- workspace for plans built without allocation ---------------------------------------
//
// A plan built by wpk_build_static keeps its whole workspace (counters, queues,
// tile tables, activations, partial sums, log) in this array instead of a
// hipMalloc allocation.  Every GPU the library runs on holds its own copy from
// module load until the process ends.  In host code `scratch` only names the
// host-side shadow of the symbol: its device address on the current device
// comes from hipGetSymbolAddress, looked up once per device below.
namespace {
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];
}  // namespace

// Device address and size of this device's scratch array.  The caller makes
// `device` current first.  Returns 0, or a negative code from wpk.h.
extern "C" int wpk_dev_static_scratch(int device, void** ptr, size_t* bytes) {
  if (device < 0 || device >= kScratchDevices || !ptr || !bytes) return WPK_E_ARG;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return WPK_E_HIP;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  *bytes = kScratchBytes;
  return WPK_OK;
}
