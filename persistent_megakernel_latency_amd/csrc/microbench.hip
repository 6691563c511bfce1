// Microbenchmarks that size the megakernel's tiles and synchronisation on gfx950.
//
// The Hazy Research Llama-1B megakernel, as the persistent-threads history page
// (section 6) describes it, wins by keeping weight loads streaming across
// operator boundaries; whether that is possible depends on three numbers of the
// machine, measured here:
//   1. the streaming-read ceiling of HBM for tile-shaped reads (contiguous
//      64 KiB blocks, as a worker's staging slot loads them), with and without
//      an agent-scope acquire/release per tile;
//   2. the throughput of device-scope atomics on one address (the work queue's
//      head and a shared dependency counter are such addresses);
//   3. the latency of a release/acquire round trip between two workgroups on
//      different XCDs (each XCD has its own L2).
// Each result is printed as one JSON line.  All waits are bounded by a
// wall-clock budget read from s_memrealtime (100 MHz), so no kernel here can
// spin forever.
#include <hip/hip_runtime.h>
#include <algorithm>

#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#define CHECK(x)                                                              \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_),       \
              __FILE__, __LINE__);                                            \
      exit(1);                                                                \
    }                                                                         \
  } while (0)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

static constexpr unsigned long long kSpinBudgetTicks = 200000000ull;  // 2 s

// ---------------------------------------------------------------------------
// 1. tile-shaped streaming read.  Block b reads blocks of 64 KiB (16 uint4 per
// thread, 256 threads) at tile index b, b+grid, ...  `mode` bits:
//   1: an agent-scope acquire fence before each tile;
//   2: a release fence plus a relaxed atomic add on a shared counter after
//      each tile (the fenced publish pattern);
//   4: non-temporal weight loads;
//   8: fence-free publish: 16 results stored with device-coherent (sc1)
//      stores, a wait for their completion, then a relaxed atomic add;
//  16: fence-free consume: a device-coherent poll of a counter, then the
//      tile's 8 KiB input vector read with device-coherent (sc1) loads;
//  32: as 16 but the input vector read with plain loads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_tile_read(const uint4* __restrict__ src,
                                                   long n_tiles, int mode,
                                                   unsigned* counters,
                                                   unsigned* sink,
                                                   const float* xvec,
                                                   float* results) {
  const int t = threadIdx.x;
  uint32_t acc = 0;
  __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void*)xvec, 0, 8192, 0x00020000);
  for (long tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    if (mode & 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (mode & 48) {
      const unsigned c = __hip_atomic_load(counters + 1024 + (blockIdx.x & 7) * 64, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      u32x4 xa, xb;
      if (mode & 16) {
        xa = __builtin_amdgcn_raw_buffer_load_b128(xr, t * 32, 0, 16);
        xb = __builtin_amdgcn_raw_buffer_load_b128(xr, t * 32 + 16, 0, 16);
      } else {
        xa = __builtin_amdgcn_raw_buffer_load_b128(xr, t * 32, 0, 0);
        xb = __builtin_amdgcn_raw_buffer_load_b128(xr, t * 32 + 16, 0, 0);
      }
      acc += c ^ xa.x ^ xa.w ^ xb.y ^ xb.z;
    }
    const u32x4* p = reinterpret_cast<const u32x4*>(src) + tile * 4096;  // 4096 x 16 B = 64 KiB
    u32x4 v[16];
    if (mode & 4) {
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = __builtin_nontemporal_load(p + j * 256 + t);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = p[j * 256 + t];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    if (mode & 2) {
      if (t == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_fetch_add(counters + (blockIdx.x & 7) * 64, 1u,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (mode & 8) {
      if (t < 64) {
        if (t < 16)
          __hip_atomic_store(results + (blockIdx.x * 16 + t), (float)(acc & 255u), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        if (t == 0)
          __hip_atomic_fetch_add(counters + (blockIdx.x & 7) * 64, 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x * blockDim.x + t] = acc;
}

// ---------------------------------------------------------------------------
// 2. same-address atomics: lane 0 of every block does `iters` fetch-adds on
// ctr[(block % n_addr) * 64].
// ---------------------------------------------------------------------------
__global__ void k_atomic(unsigned* ctr, int iters, int n_addr, unsigned* sink) {
  if (threadIdx.x != 0) return;
  unsigned s = 0;
  unsigned* c = ctr + (blockIdx.x % n_addr) * 64;
  for (int i = 0; i < iters; ++i)
    s += __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  sink[blockIdx.x] = s;
}

// ---------------------------------------------------------------------------
// 3. release/acquire ping-pong between block 0 and block `peer`.  With the
// round-robin dispatch of workgroups over the 8 XCDs, peer=1 sits on another
// XCD and peer=8 on the same one.  Blocks other than the two exit at once.
// out[0] = total ticks, out[1] = 1 if a wait ran out of budget.
// ---------------------------------------------------------------------------
__global__ void k_pingpong(unsigned* flags, int iters, int peer,
                           unsigned long long* out) {
  if (threadIdx.x != 0) return;
  if (blockIdx.x != 0 && (int)blockIdx.x != peer) return;
  const bool first = blockIdx.x == 0;
  unsigned* mine = flags + (first ? 0 : 64);
  unsigned* theirs = flags + (first ? 64 : 0);
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  bool timed_out = false;
  for (int i = 1; i <= iters && !timed_out; ++i) {
    if (first) __hip_atomic_store(mine, (unsigned)i, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long w0 = __builtin_amdgcn_s_memrealtime();
    while (__hip_atomic_load(theirs, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < (unsigned)i) {
      if (__builtin_amdgcn_s_memrealtime() - w0 > kSpinBudgetTicks) { timed_out = true; break; }
    }
    if (!first) __hip_atomic_store(mine, (unsigned)i, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memrealtime();
  if (first) {
    out[0] = t1 - t0;
    out[1] = timed_out ? 1ull : 0ull;
  } else if (timed_out) {
    out[1] = 1ull;
  }
}

// ---------------------------------------------------------------------------
// 4. cross-XCD message passing: pair k = (block 2k producer, block 2k+1
// consumer); round-robin dispatch puts them on different XCDs.  The producer
// writes `words` words of value i, publishes flag = i; the consumer waits for
// flag >= i, reads the words, counts those != i, then acks i.  proto:
//   0: producer device-coherent (sc1) stores + wait; consumer sc1 loads
//   1: producer sc1 stores + wait; consumer plain loads
//   2: producer plain stores + agent release fence; consumer agent acquire
//      fence + plain loads (the compiler's memory-model lowering)
//   3: producer plain stores + wait (no fence); consumer sc1 loads
// errs[0] = stale words seen, errs[1] = waits that ran out of budget,
// errs[2] = ticks spent by pair 0's consumer.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_mp(unsigned* flags, unsigned* data, int words, int iters,
                                           int proto, unsigned long long* errs) {
  const int pair = blockIdx.x >> 1;
  const bool producer = (blockIdx.x & 1) == 0;
  unsigned* flag = flags + pair * 128;
  unsigned* ack = flags + pair * 128 + 64;
  unsigned* d = data + (size_t)pair * words;
  const int lane = threadIdx.x;
  unsigned long long stale = 0, timeouts = 0;
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 1; i <= iters; ++i) {
    if (producer) {
      const unsigned long long w0 = __builtin_amdgcn_s_memrealtime();
      bool ok = true;
      while (__hip_atomic_load(ack, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (unsigned)(i - 1)) {
        if (__builtin_amdgcn_s_memrealtime() - w0 > kSpinBudgetTicks) { ok = false; break; }
      }
      if (!ok) { ++timeouts; break; }
      if (proto == 2) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      for (int w = lane; w < words; w += 64) {
        if (proto == 0 || proto == 1)
          __hip_atomic_store(d + w, (unsigned)i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          d[w] = (unsigned)i;
      }
      if (proto == 2) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      else __builtin_amdgcn_s_waitcnt(0);
      if (lane == 0) __hip_atomic_store(flag, (unsigned)i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      const unsigned long long w0 = __builtin_amdgcn_s_memrealtime();
      bool ok = true;
      while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (unsigned)i) {
        if (__builtin_amdgcn_s_memrealtime() - w0 > kSpinBudgetTicks) { ok = false; break; }
      }
      if (!ok) { ++timeouts; break; }
      if (proto == 2) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      for (int w = lane; w < words; w += 64) {
        unsigned v;
        if (proto == 0 || proto == 3)
          v = __hip_atomic_load(d + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          v = *(volatile unsigned*)(d + w);
        if (v != (unsigned)i) ++stale;
      }
      __builtin_amdgcn_s_waitcnt(0);
      if (proto == 2) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      if (lane == 0) __hip_atomic_store(ack, (unsigned)i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memrealtime();
  if (stale) atomicAdd(errs + 0, stale);
  if (timeouts) atomicAdd(errs + 1, timeouts);
  if (!producer && pair == 0 && lane == 0) errs[2] = t1 - t0;
}

// ---------------------------------------------------------------------------
// 5. latency of one dependent access, by cache policy: lane 0 of one block
// follows a pointer chain idx = p[idx] (stride 4 KiB + 64 B within `words`
// words) `iters` times with buffer loads of cache policy `aux` (0 plain,
// 1 sc0, 16 sc1, 17 sc0|sc1, 2 nt); mode 1: each step is instead a
// device-scope fetch-add with return; mode 2: an sc1 store followed by a wait
// for its completion.  out[0] = ticks, out[1] = final index (keeps the chain).
// ---------------------------------------------------------------------------
template <int AUX>
__device__ __forceinline__ uint32_t chase(__amdgpu_buffer_rsrc_t r, uint32_t idx) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, idx * 4, 0, AUX);
}
__global__ void k_latency(uint32_t* p, uint32_t words, int iters, int aux, int mode, unsigned long long* out) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, words * 4, 0x00020000);
  uint32_t idx = 0;
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
    if (mode == 1) {
      idx = __hip_atomic_fetch_add(p + idx, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) % words;
    } else if (mode == 2) {
      __hip_atomic_store(p + (words - 1 - (i & 1023)), (uint32_t)i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
    } else {
      switch (aux) {
        case 0: idx = chase<0>(r, idx); break;
        case 1: idx = chase<1>(r, idx); break;
        case 16: idx = chase<16>(r, idx); break;
        case 17: idx = chase<17>(r, idx); break;
        default: idx = chase<2>(r, idx); break;
      }
      idx %= words;
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memrealtime();
  out[0] = t1 - t0;
  out[1] = idx;
}

// ---- residency: how many workgroups of a given size and LDS / VGPR / SGPR
// footprint the dispatcher keeps on the GPU at once.  Every wave stays until
// the block's end (all threads spin, then a barrier); thread 0 records when
// the block ran and the host counts the largest number of overlapping blocks.
#define WPK_CLOBBER_V128 "v0","v1","v2","v3","v4","v5","v6","v7","v8","v9","v10","v11","v12","v13","v14","v15","v16","v17","v18","v19","v20","v21","v22","v23","v24","v25","v26","v27","v28","v29","v30","v31","v32","v33","v34","v35","v36","v37","v38","v39","v40","v41","v42","v43","v44","v45","v46","v47","v48","v49","v50","v51","v52","v53","v54","v55","v56","v57","v58","v59","v60","v61","v62","v63","v64","v65","v66","v67","v68","v69","v70","v71","v72","v73","v74","v75","v76","v77","v78","v79","v80","v81","v82","v83","v84","v85","v86","v87","v88","v89","v90","v91","v92","v93","v94","v95","v96","v97","v98","v99","v100","v101","v102","v103","v104","v105","v106","v107","v108","v109","v110","v111","v112","v113","v114","v115","v116","v117","v118","v119"
#define WPK_CLOBBER_V148 "v0","v1","v2","v3","v4","v5","v6","v7","v8","v9","v10","v11","v12","v13","v14","v15","v16","v17","v18","v19","v20","v21","v22","v23","v24","v25","v26","v27","v28","v29","v30","v31","v32","v33","v34","v35","v36","v37","v38","v39","v40","v41","v42","v43","v44","v45","v46","v47","v48","v49","v50","v51","v52","v53","v54","v55","v56","v57","v58","v59","v60","v61","v62","v63","v64","v65","v66","v67","v68","v69","v70","v71","v72","v73","v74","v75","v76","v77","v78","v79","v80","v81","v82","v83","v84","v85","v86","v87","v88","v89","v90","v91","v92","v93","v94","v95","v96","v97","v98","v99","v100","v101","v102","v103","v104","v105","v106","v107","v108","v109","v110","v111","v112","v113","v114","v115","v116","v117","v118","v119","v120","v121","v122","v123","v124","v125","v126","v127","v128","v129","v130","v131","v132","v133","v134","v135","v136","v137","v138","v139","v140","v141","v142","v143","v144","v145","v146","v147"
#define WPK_CLOBBER_S100 "s8","s9","s10","s11","s12","s13","s14","s15","s16","s17","s18","s19","s20","s21","s22","s23","s24","s25","s26","s27","s28","s29","s30","s31","s32","s33","s34","s35","s36","s37","s38","s39","s40","s41","s42","s43","s44","s45","s46","s47","s48","s49","s50","s51","s52","s53","s54","s55","s56","s57","s58","s59","s60","s61","s62","s63","s64","s65","s66","s67","s68","s69","s70","s71","s72","s73","s74","s75","s76","s77","s78","s79","s80","s81","s82","s83","s84","s85","s86","s87","s88","s89","s90","s91","s92","s93","s94","s95","s96","s97","s98","s99"
template <int NT, int LDSB, int VG, bool SG>
__global__ __launch_bounds__(NT) void k_resid(unsigned long long* out, int spin_ticks, int salt) {
  __shared__ float buf[LDSB / 4];
  for (int i = threadIdx.x; i < LDSB / 4; i += NT) buf[i] = (float)(i + salt);
  if (VG == 128) asm volatile("" ::: WPK_CLOBBER_V128);
  if (VG == 148) asm volatile("" ::: WPK_CLOBBER_V148);
  if (SG) asm volatile("" ::: WPK_CLOBBER_S100);
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  while (__builtin_amdgcn_s_memrealtime() - t0 < (unsigned long long)spin_ticks) __builtin_amdgcn_s_sleep(10);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned long long t1 = __builtin_amdgcn_s_memrealtime();
    out[2 * blockIdx.x] = t0;
    out[2 * blockIdx.x + 1] = t1 + (unsigned long long)(buf[(salt & 63) + 1] > 1e30f);
  }
}

template <int NT, int LDSB, int VG, bool SG>
static void resid_case(unsigned long long* d_out, int blocks) {
  const int spin = 3000;  // 30 us at 100 MHz
  void* fn = reinterpret_cast<void*>(&k_resid<NT, LDSB, VG, SG>);
  int per_cu = 0;
  CHECK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NT, 0));
  int salt = 0;
  void* args[] = {&d_out, (void*)&spin, &salt};
  const hipError_t e = hipLaunchCooperativeKernel(fn, dim3(blocks), dim3(NT), args, 0, 0);
  if (e != hipSuccess) {
    printf("{\"bench\": \"residency\", \"threads\": %d, \"lds\": %d, \"vgprs\": %d, \"sgpr100\": %d, \"blocks\": %d, "
           "\"occupancy_api_per_cu\": %d, \"error\": \"%s\"}\n", NT, LDSB, VG, (int)SG, blocks, per_cu, hipGetErrorString(e));
    fflush(stdout);
    (void)hipGetLastError();
    return;
  }
  CHECK(hipDeviceSynchronize());
  CHECK(hipGetLastError());
  std::vector<unsigned long long> h(2 * (size_t)blocks);
  CHECK(hipMemcpy(h.data(), d_out, h.size() * 8, hipMemcpyDeviceToHost));
  std::vector<std::pair<unsigned long long, int>> ev;
  for (int b = 0; b < blocks; ++b) {
    ev.push_back({h[2 * b], 1});
    ev.push_back({h[2 * b + 1], -1});
  }
  std::sort(ev.begin(), ev.end(), [](const std::pair<unsigned long long, int>& a, const std::pair<unsigned long long, int>& b) {
    return a.first != b.first ? a.first < b.first : a.second < b.second;
  });
  int cur = 0, best = 0;
  for (auto& x : ev) best = std::max(best, cur += x.second);
  printf("{\"bench\": \"residency\", \"threads\": %d, \"lds\": %d, \"vgprs\": %d, \"sgpr100\": %d, \"blocks\": %d, "
         "\"occupancy_api_per_cu\": %d, \"max_concurrent\": %d}\n", NT, LDSB, VG, (int)SG, blocks, per_cu, best);
  fflush(stdout);
}

// ---- poll storm: blocks 1.. poll (device-scope loads, each waiting for the
// previous) one of n_addr counters; block 0 meanwhile does dependent
// atomic adds on counter 0.  out[b] = ticks for the block's loop.
__global__ void k_poll(unsigned* ctr, int iters, int n_addr, int with_atomic, unsigned long long* out, unsigned* sink) {
  if (threadIdx.x != 0) return;
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
  unsigned s = 0;
  if (blockIdx.x == 0 && with_atomic) {
    for (int i = 0; i < iters; ++i) s += __hip_atomic_fetch_add(ctr + (s & 0u), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (blockIdx.x != 0) {
    unsigned* c = ctr + (size_t)(blockIdx.x % n_addr) * 64;
    for (int i = 0; i < iters; ++i) s += __hip_atomic_load(c + (s & 0u), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  out[blockIdx.x] = __builtin_amdgcn_s_memrealtime() - t0;
  sink[blockIdx.x] = s;
}

// ---- ping-pong under load: blocks 0 and 1 (64 threads, on different XCDs)
// bounce a counter with relaxed device-scope atomic adds and polls, the
// publish/poll pair of the megakernel's protocol; blocks 2.. (256 threads)
// stream 64 KiB tiles with non-temporal loads until block 0 finishes.
// out[0] = ticks for `iters` round trips, out[1] = 1 if a wait ran out.
// A scalar load that misses the scalar cache (glc), waited in the same asm
// statement: a poll that does not queue behind the vector memory pipeline.
__device__ __forceinline__ unsigned sload_glc(const unsigned* p) {
  unsigned v;
  asm volatile("s_load_dword %0, %1, 0x0 glc\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

template <bool SCALAR_POLL>
__global__ __launch_bounds__(256) void k_pp_loaded(unsigned* ctr, int iters, const uint4* src, long n_tiles,
                                                   unsigned long long* out, unsigned* sink) {
  const int t = threadIdx.x;
  if (blockIdx.x < 2) {
    if (t != 0) return;
    const bool first = blockIdx.x == 0;
    unsigned* mine = ctr + (first ? 0 : 64);
    unsigned* theirs = ctr + (first ? 64 : 0);
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    bool timed_out = false;
    for (int i = 1; i <= iters && !timed_out; ++i) {
      if (first) __hip_atomic_fetch_add(mine, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const unsigned long long w0 = __builtin_amdgcn_s_memrealtime();
      while ((SCALAR_POLL ? sload_glc(theirs) : __hip_atomic_load(theirs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) <
             (unsigned)i) {
        if (__builtin_amdgcn_s_memrealtime() - w0 > kSpinBudgetTicks) { timed_out = true; break; }
      }
      if (!first) __hip_atomic_fetch_add(mine, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (first) {
      out[0] = __builtin_amdgcn_s_memrealtime() - t0;
      out[1] = timed_out ? 1 : 0;
      __hip_atomic_store(ctr + 128, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // streamers stop
    }
    return;
  }
  uint32_t acc = 0;
  const long nb = gridDim.x - 2;
  for (long tile = blockIdx.x - 2; tile < n_tiles; tile += nb) {
    if (__hip_atomic_load(ctr + 128, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
    const u32x4* p = reinterpret_cast<const u32x4*>(src) + tile * 4096;
    u32x4 v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = __builtin_nontemporal_load(p + j * 256 + t);
#pragma unroll
    for (int j = 0; j < 16; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    if (tile + nb >= n_tiles) tile = blockIdx.x - 2 - nb;  // wrap around until told to stop
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x * blockDim.x + t] = acc;
}

// ---- publish detection: block 0 publishes (stores a timestamp, waits for it,
// adds 1 to line i % lines) every 20 us; blocks 1..N poll the sum over the
// lines with device-coherent loads and a short sleep, and record when they saw
// publish i.  out[2b] = summed detection ticks, out[2b+1] = the largest.
__global__ __launch_bounds__(64) void k_detect(unsigned* ctr, int lines, int iters, unsigned long long* tpub,
                                               unsigned long long* out, int* fail) {
  const int lane = threadIdx.x;
  if (blockIdx.x == 0) {
    if (lane != 0) return;
    for (int i = 1; i <= iters; ++i) {
      const unsigned long long w = __builtin_amdgcn_s_memrealtime();
      while (__builtin_amdgcn_s_memrealtime() - w < 2000) __builtin_amdgcn_s_sleep(2);
      const unsigned long long t = __builtin_amdgcn_s_memrealtime();
      __hip_atomic_store(&tpub[i], t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
      __hip_atomic_fetch_add(&ctr[(i % lines) * 64], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  unsigned long long acc = 0, mx = 0;
  for (int i = 1; i <= iters; ++i) {
    const unsigned long long w0 = __builtin_amdgcn_s_memrealtime();
    bool ok = false;
    while (__builtin_amdgcn_s_memrealtime() - w0 < kSpinBudgetTicks) {
      unsigned v = lane < lines ? __hip_atomic_load(&ctr[lane * 64], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
      if (v >= (unsigned)i) { ok = true; break; }
      __builtin_amdgcn_s_sleep(2);
    }
    const unsigned long long t = __builtin_amdgcn_s_memrealtime();
    if (!ok) { if (lane == 0) atomicAdd(fail, 1); break; }
    const unsigned long long tp = __hip_atomic_load(&tpub[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long d = t > tp ? t - tp : 0;
    acc += d;
    mx = d > mx ? d : mx;
  }
  if (lane == 0) { out[2 * blockIdx.x] = acc; out[2 * blockIdx.x + 1] = mx; }
}

// ---- round trip under load, by bytes in flight per streaming block: blocks 0
// and 1 (one lane each) bounce a counter; blocks 2.. stream 64 KiB tiles with
// NL 16-byte loads per thread in flight (NL/16 of a tile), until block 0 is
// done.  out[0] = ticks for the round trips, out[1] = 1 if a wait ran out,
// out[b] (b >= 2) = bytes block b streamed.
template <int NL>
__global__ __launch_bounds__(256) void k_rt_inflight(unsigned* ctr, int iters, const u32x4* src, long n_tiles,
                                                     unsigned long long* out, unsigned* sink) {
  const int t = threadIdx.x;
  if (blockIdx.x < 2) {
    if (t != 0) return;
    const bool first = blockIdx.x == 0;
    unsigned* mine = ctr + (first ? 0 : 64);
    unsigned* theirs = ctr + (first ? 64 : 0);
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    bool timed_out = false;
    for (int i = 1; i <= iters && !timed_out; ++i) {
      if (first) __hip_atomic_fetch_add(mine, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const unsigned long long w0 = __builtin_amdgcn_s_memrealtime();
      while (__hip_atomic_load(theirs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (unsigned)i) {
        if (__builtin_amdgcn_s_memrealtime() - w0 > kSpinBudgetTicks) { timed_out = true; break; }
      }
      if (!first) __hip_atomic_fetch_add(mine, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (first) {
      out[0] = __builtin_amdgcn_s_memrealtime() - t0;
      out[1] = timed_out ? 1 : 0;
      __hip_atomic_store(ctr + 128, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  uint32_t acc = 0;
  unsigned long long bytes = 0;
  const long nb = gridDim.x - 2;
  long tile = blockIdx.x - 2;
  const unsigned long long w0 = __builtin_amdgcn_s_memrealtime();
  while (true) {
    if (__hip_atomic_load(ctr + 128, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
    if (__builtin_amdgcn_s_memrealtime() - w0 > kSpinBudgetTicks) break;
    const u32x4* p = src + tile * 4096;
#pragma unroll
    for (int j0 = 0; j0 < 16; j0 += NL) {
      u32x4 v[NL];
#pragma unroll
      for (int j = 0; j < NL; ++j) v[j] = __builtin_nontemporal_load(p + (j0 + j) * 256 + t);
#pragma unroll
      for (int j = 0; j < NL; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
      __builtin_amdgcn_s_waitcnt(0);
    }
    bytes += 65536;
    tile += nb;
    if (tile >= n_tiles) tile = blockIdx.x - 2;
  }
  if (t == 0) out[blockIdx.x] = bytes;
  if (acc == 0x9e3779b9u) sink[blockIdx.x * 256 + t] = acc;
}

// ---- re-read bandwidth: 64 KiB tiles [tile0, tile0 + n_tiles) read by a
// grid-stride loop (whether a buffer that fits the memory-side cache is
// served faster the second time).
__global__ __launch_bounds__(256) void k_reread(const u32x4* __restrict__ src, long n_tiles, long tile0, unsigned* sink) {
  const int t = threadIdx.x;
  unsigned acc = 0;
  for (long k = blockIdx.x; k < n_tiles; k += gridDim.x) {
    const u32x4* p = src + (tile0 + k) * 4096;
    u32x4 v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = p[j * 256 + t];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  if (acc == 0x12345678u) sink[blockIdx.x] = acc;
}

// ---- weight-tile layouts: 64 KiB tiles streamed with non-temporal loads,
// 16 per thread, either as 1 KiB wave-contiguous pieces (FRAG = false) or in
// the matrix-core A-fragment order (FRAG = true: the tile viewed as 16 pieces
// of 4 KiB, wave w reading 512 columns of every piece, lane l piece l % 16 at
// 16-byte column group 4 (w * 16 + j) + l / 16), whose every load touches 64
// bytes of 16 pieces.
template <bool FRAG>
__global__ __launch_bounds__(256) void k_frag(const u32x4* __restrict__ src, long n_tiles, unsigned* sink) {
  const int t = threadIdx.x, w = t >> 6, l = t & 63;
  unsigned acc = 0;
  for (long k = blockIdx.x; k < n_tiles; k += gridDim.x) {
    const u32x4* p = src + k * 4096;
    u32x4 v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      v[j] = __builtin_nontemporal_load(FRAG ? p + (l & 15) * 256 + w * 64 + j * 4 + (l >> 4) : p + j * 256 + t);
#pragma unroll
    for (int j = 0; j < 16; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  if (acc == 0x12345678u) sink[blockIdx.x] = acc;
}

// ---- plain copy of a known number of bytes: the calibration kernel for the
// FETCH_SIZE / WRITE_SIZE hardware counters (16 bytes per thread per step).
__global__ __launch_bounds__(256) void k_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst, long n16) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n16; i += (long)gridDim.x * 256) dst[i] = src[i];
}

static double time_ms(hipEvent_t a, hipEvent_t b) {
  float ms = 0;
  CHECK(hipEventElapsedTime(&ms, a, b));
  return ms;
}


// ---------------------------------------------------------------------------
// X/W streaming: each 256-thread block reads 64 KiB weight tiles from HBM
// (non-temporal) and, per tile, XR x 64 KiB of a small activation buffer that
// stays in L2 (device-coherent loads), either into registers in batches of 16
// loads per thread (LDSX = false) or straight into a 32 KiB LDS area with
// LDS-direct loads in batches of 8 per thread (LDSX = true).
// ---------------------------------------------------------------------------
template <bool LDSX>
__global__ __launch_bounds__(256) void k_xw(const u32x4* __restrict__ w, long n_tiles, const float* xbuf,
                                            int xr, unsigned* sink) {
  __shared__ u32x4 lds[2048];  // 32 KiB
  const int t = threadIdx.x;
  uint32_t acc = 0;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)xbuf, 0, 262144, 0x00020000);
  for (long tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const u32x4* p = w + tile * 4096;
    u32x4 v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = __builtin_nontemporal_load(p + j * 256 + t);
    for (int b = 0; b < xr * 16; b += 16) {
      if (!LDSX) {
        u32x4 x[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
          x[j] = __builtin_amdgcn_raw_buffer_load_b128(r, ((uint32_t)((tile * 7 + b + j) * 256 + t) * 16u) & 262143u, 0, 16);
#pragma unroll
        for (int j = 0; j < 16; ++j) acc += x[j].x ^ x[j].w;
      } else {
        const int wv = t >> 6, ln = t & 63;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                r, (__attribute__((address_space(3))) void*)&lds[wv * 512 + j * 64],
                16, ((uint32_t)((tile * 7 + b + h * 8 + j) * 256 + t) * 16u) & 262143u, 0, 0, 16);
          __builtin_amdgcn_s_waitcnt(0);
          acc += lds[wv * 512 + (ln + h) % 512].x;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x * blockDim.x + t] = acc;
}

int main(int argc, char** argv) {
  int dev = 0;
  CHECK(hipSetDevice(dev));
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, dev));
  const int n_cu = prop.multiProcessorCount;
  printf("{\"device\": \"%s\", \"gcn_arch\": \"%s\", \"cus\": %d, \"l2_bytes\": %d, \"clock_khz\": %d}\n",
         prop.name, prop.gcnArchName, n_cu, prop.l2CacheSize, prop.clockRate);
  fflush(stdout);

  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));

  // ---- 1. tile-shaped streaming reads over 4 GiB ----
  const long n_tiles = 65536;  // 64 Ki tiles x 64 KiB = 4 GiB
  const size_t bytes = (size_t)n_tiles * 65536;
  uint4* src = nullptr;
  unsigned* sink = nullptr;
  unsigned* counters = nullptr;
  CHECK(hipMalloc(&src, bytes));
  CHECK(hipMemset(src, 1, bytes));
  CHECK(hipMalloc(&sink, sizeof(unsigned) * 256 * 8192));
  CHECK(hipMalloc(&counters, 4096 * sizeof(unsigned)));
  CHECK(hipMemset(counters, 0, 4096 * sizeof(unsigned)));
  float* xvec = nullptr;
  float* results = nullptr;
  CHECK(hipMalloc(&xvec, 8192));
  CHECK(hipMemset(xvec, 0, 8192));
  CHECK(hipMalloc(&results, sizeof(float) * 16 * 8192));
  const std::string which = argc > 1 ? argv[1] : "all";
  if (which == "poll") {
    const int blocks = 513, iters = 2000;
    unsigned long long* d_out = nullptr;
    unsigned* ctr = nullptr;
    unsigned* snk = nullptr;
    CHECK(hipMalloc(&d_out, sizeof(unsigned long long) * blocks));
    CHECK(hipMalloc(&ctr, sizeof(unsigned) * 64 * 256));
    CHECK(hipMalloc(&snk, sizeof(unsigned) * blocks));
    CHECK(hipMemset(ctr, 0, sizeof(unsigned) * 64 * 256));
    for (int with_atomic : {0, 1})
      for (int n_addr : {1, 4, 16, 64, 256}) {
        hipLaunchKernelGGL(k_poll, dim3(blocks), dim3(64), 0, 0, ctr, iters, n_addr, with_atomic, d_out, snk);
        CHECK(hipDeviceSynchronize());
        CHECK(hipGetLastError());
        std::vector<unsigned long long> h(blocks);
        CHECK(hipMemcpy(h.data(), d_out, sizeof(unsigned long long) * blocks, hipMemcpyDeviceToHost));
        double poll = 0;
        for (int b = 1; b < blocks; ++b) poll += (double)h[b];
        poll = poll / (blocks - 1) * 10.0 / iters;  // ns per dependent poll
        printf("{\"bench\": \"poll_storm\", \"pollers\": %d, \"addresses\": %d, \"with_atomic\": %d, "
               "\"ns_per_poll\": %.1f, \"atomic_ns\": %.1f, \"polls_per_s_per_address\": %.3g}\n",
               blocks - 1, n_addr, with_atomic, poll, with_atomic ? h[0] * 10.0 / iters : 0.0,
               (blocks - 1) / (double)n_addr / (poll * 1e-9));
        fflush(stdout);
      }
    CHECK(hipFree(d_out));
    CHECK(hipFree(ctr));
    CHECK(hipFree(snk));
    return 0;
  }
  if (which == "detect") {
    const int iters = 200;
    unsigned* ctr = nullptr;
    unsigned long long *tpub = nullptr, *d_out = nullptr;
    int* fail = nullptr;
    CHECK(hipMalloc(&ctr, 64 * 64 * sizeof(unsigned)));
    CHECK(hipMalloc(&tpub, (iters + 1) * sizeof(unsigned long long)));
    CHECK(hipMalloc(&d_out, 2 * 1024 * sizeof(unsigned long long)));
    CHECK(hipMalloc(&fail, sizeof(int)));
    for (int lines : {1, 4, 16})
      for (int pollers : {16, 128, 512}) {
        CHECK(hipMemset(ctr, 0, 64 * 64 * sizeof(unsigned)));
        CHECK(hipMemset(tpub, 0, (iters + 1) * sizeof(unsigned long long)));
        CHECK(hipMemset(d_out, 0, 2 * 1024 * sizeof(unsigned long long)));
        CHECK(hipMemset(fail, 0, sizeof(int)));
        hipLaunchKernelGGL(k_detect, dim3(pollers + 1), dim3(64), 0, 0, ctr, lines, iters, tpub, d_out, fail);
        CHECK(hipDeviceSynchronize());
        CHECK(hipGetLastError());
        std::vector<unsigned long long> h(2 * (pollers + 1));
        int hf = 0;
        CHECK(hipMemcpy(h.data(), d_out, h.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost));
        CHECK(hipMemcpy(&hf, fail, sizeof(int), hipMemcpyDeviceToHost));
        double sum = 0, mx = 0;
        for (int b = 1; b <= pollers; ++b) {
          sum += (double)h[2 * b];
          mx = (double)h[2 * b + 1] > mx ? (double)h[2 * b + 1] : mx;
        }
        printf("{\"bench\": \"publish_detect\", \"lines\": %d, \"pollers\": %d, \"mean_us\": %.2f, \"max_us\": %.2f, "
               "\"timeouts\": %d}\n", lines, pollers, sum / pollers / iters / 100.0, mx / 100.0, hf);
        fflush(stdout);
      }
    CHECK(hipFree(ctr));
    CHECK(hipFree(tpub));
    CHECK(hipFree(d_out));
    CHECK(hipFree(fail));
    return 0;
  }
  if (which == "rtload") {
    const int iters = 2000;
    const long rt_tiles = 32768;  // the first 2 GiB of the read buffer
    unsigned long long* d_out = nullptr;
    unsigned* ctr = nullptr;
    CHECK(hipMalloc(&d_out, 4096 * sizeof(unsigned long long)));
    CHECK(hipMalloc(&ctr, 4096 * sizeof(unsigned)));
    const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
    for (int grid : {2, 2 + n_cu, 2 + 2 * n_cu})
      for (int nl : {4, 8, 16}) {
        CHECK(hipMemset(ctr, 0, 4096 * sizeof(unsigned)));
        CHECK(hipMemset(d_out, 0, 4096 * sizeof(unsigned long long)));
        if (nl == 4) hipLaunchKernelGGL(k_rt_inflight<4>, dim3(grid), dim3(256), 0, 0, ctr, iters, s4, rt_tiles, d_out, sink);
        if (nl == 8) hipLaunchKernelGGL(k_rt_inflight<8>, dim3(grid), dim3(256), 0, 0, ctr, iters, s4, rt_tiles, d_out, sink);
        if (nl == 16) hipLaunchKernelGGL(k_rt_inflight<16>, dim3(grid), dim3(256), 0, 0, ctr, iters, s4, rt_tiles, d_out, sink);
        CHECK(hipDeviceSynchronize());
        CHECK(hipGetLastError());
        std::vector<unsigned long long> h(grid);
        CHECK(hipMemcpy(h.data(), d_out, grid * sizeof(unsigned long long), hipMemcpyDeviceToHost));
        double tot = 0;
        for (int b = 2; b < grid; ++b) tot += (double)h[b];
        const double us = h[0] / 100.0;
        printf("{\"bench\": \"round_trip_under_load\", \"streamers\": %d, \"inflight_KiB_per_streamer\": %d, "
               "\"round_trip_ns\": %.0f, \"stream_GBps\": %.0f, \"timed_out\": %llu}\n",
               grid - 2, nl * 4, us * 1000.0 / iters, us > 0 ? tot / us / 1e3 : 0.0, h[1]);
        fflush(stdout);
      }
    CHECK(hipFree(d_out));
    CHECK(hipFree(ctr));
    return 0;
  }
  if (which == "reread") {
    const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
    const long flush_tiles = 16384, flush0 = n_tiles - flush_tiles;  // the last GiB, other data
    for (long mib : {16L, 64L, 128L, 192L, 256L, 320L, 512L, 1024L}) {
      const long nt = mib * 16;  // 64 KiB tiles
      const long reps = mib <= 256 ? 20 : 4;
      float best = 1e30f, cold = 0;
      for (int trial = 0; trial < 3; ++trial) {
        hipLaunchKernelGGL(k_reread, dim3(2 * n_cu), dim3(256), 0, 0, s4, flush_tiles, flush0, sink);
        CHECK(hipEventRecord(e0));
        hipLaunchKernelGGL(k_reread, dim3(2 * n_cu), dim3(256), 0, 0, s4, nt, 0L, sink);
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        cold = (float)time_ms(e0, e1);
        CHECK(hipEventRecord(e0));
        for (long r = 0; r < reps; ++r)
          hipLaunchKernelGGL(k_reread, dim3(2 * n_cu), dim3(256), 0, 0, s4, nt, 0L, sink);
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        const float ms = (float)time_ms(e0, e1) / reps;
        best = ms < best ? ms : best;
      }
      CHECK(hipGetLastError());
      const double b = (double)nt * 65536;
      printf("{\"bench\": \"reread\", \"MiB\": %ld, \"first_read_GBps\": %.0f, \"reread_GBps\": %.0f}\n", mib,
             b / cold / 1e6, b / best / 1e6);
      fflush(stdout);
    }
    return 0;
  }
  if (which == "frag") {
    // 4 GiB of 64 KiB tiles, contiguous pieces against A-fragment order
    const u32x4* s4 = reinterpret_cast<const u32x4*>(src);
    for (int frag : {0, 1, 0, 1})
      for (int per_cu : {1, 2}) {
        const int grid = n_cu * per_cu;
        float best = 1e30f;
        for (int rep = 0; rep < 3; ++rep) {
          CHECK(hipEventRecord(e0));
          if (frag) hipLaunchKernelGGL(k_frag<true>, dim3(grid), dim3(256), 0, 0, s4, n_tiles, sink);
          else hipLaunchKernelGGL(k_frag<false>, dim3(grid), dim3(256), 0, 0, s4, n_tiles, sink);
          CHECK(hipEventRecord(e1));
          CHECK(hipEventSynchronize(e1));
          CHECK(hipGetLastError());
          const float ms = (float)time_ms(e0, e1);
          best = ms < best ? ms : best;
        }
        printf("{\"bench\": \"tile_layout\", \"fragment_order\": %d, \"blocks_per_cu\": %d, \"ms\": %.3f, "
               "\"GBps\": %.0f}\n", frag, per_cu, best, bytes / (best * 1e6));
        fflush(stdout);
      }
    return 0;
  }
  if (which == "resid") {
    unsigned long long* d_out = nullptr;
    CHECK(hipMalloc(&d_out, sizeof(unsigned long long) * 2 * 4 * n_cu));
    resid_case<320, 16384, 0, false>(d_out, 2 * n_cu);
    resid_case<320, 53840, 148, true>(d_out, 2 * n_cu);
    resid_case<320, 53840, 128, true>(d_out, 2 * n_cu);
    resid_case<320, 16384, 148, false>(d_out, 2 * n_cu);
    resid_case<256, 53840, 148, true>(d_out, 2 * n_cu);
    resid_case<576, 53840, 148, true>(d_out, n_cu);
    resid_case<576, 53840, 128, true>(d_out, n_cu);
    resid_case<320, 16384, 128, false>(d_out, 3 * n_cu);
    CHECK(hipFree(d_out));
    return 0;
  }
  if (which == "xw") {
    // weight tiles over 4 GiB plus xr x their bytes of L2-resident activations
    float* xb = nullptr;
    CHECK(hipMalloc(&xb, 262144));
    CHECK(hipMemset(xb, 0, 262144));
    for (int ldsx : {0, 1})
      for (int xr : {0, 1, 2, 4})
        for (int per_cu : {1, 2}) {
          const int grid = n_cu * per_cu;
          for (int rep = 0; rep < 2; ++rep) {
            CHECK(hipEventRecord(e0));
            if (ldsx)
              hipLaunchKernelGGL(k_xw<true>, dim3(grid), dim3(256), 0, 0, reinterpret_cast<const u32x4*>(src),
                                 n_tiles, xb, xr, sink);
            else
              hipLaunchKernelGGL(k_xw<false>, dim3(grid), dim3(256), 0, 0, reinterpret_cast<const u32x4*>(src),
                                 n_tiles, xb, xr, sink);
            CHECK(hipEventRecord(e1));
            CHECK(hipEventSynchronize(e1));
            CHECK(hipGetLastError());
            const double ms = time_ms(e0, e1);
            if (rep == 1)
              printf("{\"bench\": \"xw\", \"lds_direct\": %d, \"x_per_w\": %d, \"blocks_per_cu\": %d, "
                     "\"ms\": %.3f, \"w_GBps\": %.1f, \"total_GBps\": %.1f}\n",
                     ldsx, xr, per_cu, ms, bytes / (ms * 1e6), bytes * (1.0 + xr) / (ms * 1e6));
            fflush(stdout);
          }
        }
    CHECK(hipFree(xb));
    return 0;
  }
  if (which == "copy") {
    // 1 GiB from the read buffer into a second buffer, five times
    const size_t cbytes = (size_t)1 << 30;
    u32x4* dst = nullptr;
    CHECK(hipMalloc(&dst, cbytes));
    for (int r = 0; r < 5; ++r) {
      CHECK(hipEventRecord(e0));
      hipLaunchKernelGGL(k_copy, dim3(n_cu * 8), dim3(256), 0, 0, reinterpret_cast<const u32x4*>(src), dst,
                         (long)(cbytes / 16));
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      CHECK(hipGetLastError());
      const double ms = time_ms(e0, e1);
      printf("{\"bench\": \"copy\", \"bytes_read\": %zu, \"bytes_written\": %zu, \"ms\": %.4f, \"GBps\": %.1f}\n",
             cbytes, cbytes, ms, 2.0 * cbytes / (ms * 1e6));
      fflush(stdout);
    }
    CHECK(hipFree(dst));
    return 0;
  }
  if (which == "ppload") {
    unsigned long long* d_out = nullptr;
    CHECK(hipMalloc(&d_out, sizeof(unsigned long long) * 2));
    for (int scalar : {0, 1})
    for (int streamers : {0, 256, 512, 768}) {
      CHECK(hipMemset(counters, 0, 4096 * sizeof(unsigned)));
      const int iters = 2000;
      if (scalar)
        hipLaunchKernelGGL(k_pp_loaded<true>, dim3(2 + streamers), dim3(256), 0, 0, counters, iters, src, n_tiles, d_out, sink);
      else
        hipLaunchKernelGGL(k_pp_loaded<false>, dim3(2 + streamers), dim3(256), 0, 0, counters, iters, src, n_tiles, d_out, sink);
      CHECK(hipDeviceSynchronize());
      CHECK(hipGetLastError());
      unsigned long long h[2];
      CHECK(hipMemcpy(h, d_out, sizeof(h), hipMemcpyDeviceToHost));
      printf("{\"bench\": \"pingpong_under_load\", \"poll\": \"%s\", \"streaming_blocks\": %d, \"round_trip_ns\": %.1f, \"timed_out\": %llu}\n",
             scalar ? "scalar_glc" : "vector_sc1", streamers, h[0] * 10.0 / iters, h[1]);
      fflush(stdout);
    }
    CHECK(hipFree(d_out));
    return 0;
  }
  const int per_cu[] = {1, 2, 4, 8};
  for (int mode : {0, 1, 2, 3, 4, 8, 16, 32, 24, 40}) {
    if (which != "all" && which != "read") break;
    for (int pc : per_cu) {
      const int grid = n_cu * pc;  // grid-stride over n_tiles: every tile index < n_tiles
      hipLaunchKernelGGL(k_tile_read, dim3(grid), dim3(256), 0, 0, src, n_tiles, mode, counters, sink, xvec, results);
      CHECK(hipEventRecord(e0));
      const int reps = 5;
      for (int r = 0; r < reps; ++r)
        hipLaunchKernelGGL(k_tile_read, dim3(grid), dim3(256), 0, 0, src, n_tiles, mode, counters, sink, xvec, results);
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      CHECK(hipGetLastError());
      const double ms = time_ms(e0, e1) / reps;
      printf("{\"bench\": \"tile_read\", \"mode\": %d, \"blocks_per_cu\": %d, \"ms\": %.4f, \"GBps\": %.1f}\n",
             mode, pc, ms, bytes / ms / 1e6);
      fflush(stdout);
    }
  }

  // ---- 2. same-address atomic throughput ----
  const int addrs[] = {1, 8, 64};
  for (int na : addrs) {
    if (which != "all" && which != "atomic") break;
    for (int pc : {1, 4}) {
      const int grid = n_cu * pc;
      const int iters = 64;
      CHECK(hipMemset(counters, 0, 4096 * sizeof(unsigned)));
      hipLaunchKernelGGL(k_atomic, dim3(grid), dim3(64), 0, 0, counters, iters, na, sink);
      CHECK(hipEventRecord(e0));
      hipLaunchKernelGGL(k_atomic, dim3(grid), dim3(64), 0, 0, counters, iters, na, sink);
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      CHECK(hipGetLastError());
      const double ms = time_ms(e0, e1);
      const double n = (double)grid * iters;
      std::vector<unsigned> hc(4096);
      CHECK(hipMemcpy(hc.data(), counters, 4096 * sizeof(unsigned), hipMemcpyDeviceToHost));
      unsigned long long total = 0;
      for (int a = 0; a < na; ++a) total += hc[a * 64];
      const bool exact = total == (unsigned long long)(2.0 * n);
      printf("{\"bench\": \"atomic\", \"addresses\": %d, \"blocks\": %d, \"atomics\": %.0f, \"ms\": %.4f, \"Mops\": %.1f, \"ns_per_op_per_address\": %.2f, \"count_exact\": %s}\n",
             na, grid, n, ms, n / ms / 1e3, ms * 1e6 / (n / na), exact ? "true" : "false");
      fflush(stdout);
    }
  }

  // ---- 3. release/acquire ping-pong ----
  unsigned long long* pp_out = nullptr;
  CHECK(hipMalloc(&pp_out, 2 * sizeof(unsigned long long)));
  for (int peer : {1, 8, 2, 4}) {
    if (which != "all" && which != "pingpong") break;
    const int iters = 2000;
    CHECK(hipMemset(counters, 0, 4096 * sizeof(unsigned)));
    CHECK(hipMemset(pp_out, 0, 2 * sizeof(unsigned long long)));
    hipLaunchKernelGGL(k_pingpong, dim3(peer + 1), dim3(64), 0, 0, counters, iters, peer, pp_out);
    CHECK(hipDeviceSynchronize());
    CHECK(hipGetLastError());
    unsigned long long h[2];
    CHECK(hipMemcpy(h, pp_out, sizeof(h), hipMemcpyDeviceToHost));
    printf("{\"bench\": \"pingpong\", \"peer_block\": %d, \"round_trip_ns\": %.1f, \"timed_out\": %llu}\n",
           peer, h[0] * 10.0 / iters, h[1]);
    fflush(stdout);
  }

  // ---- 4. message passing across XCDs ----
  if (which == "all" || which == "mp") {
    const int words = 2048, iters = 2000;
    unsigned* mpdata = nullptr;
    unsigned long long* errs = nullptr;
    CHECK(hipMalloc(&mpdata, sizeof(unsigned) * words * 8));
    CHECK(hipMalloc(&errs, 4 * sizeof(unsigned long long)));
    for (int proto : {0, 1, 2, 3}) {
      for (int pairs : {1, 8}) {
        CHECK(hipMemset(counters, 0, 4096 * sizeof(unsigned)));
        CHECK(hipMemset(mpdata, 0, sizeof(unsigned) * words * 8));
        CHECK(hipMemset(errs, 0, 4 * sizeof(unsigned long long)));
        hipLaunchKernelGGL(k_mp, dim3(2 * pairs), dim3(64), 0, 0, counters, mpdata, words, iters, proto, errs);
        CHECK(hipDeviceSynchronize());
        CHECK(hipGetLastError());
        unsigned long long h[3];
        CHECK(hipMemcpy(h, errs, sizeof(h), hipMemcpyDeviceToHost));
        printf("{\"bench\": \"message_passing\", \"proto\": %d, \"pairs\": %d, \"words\": %d, \"iters\": %d, \"stale_words\": %llu, \"timeouts\": %llu, \"ns_per_iter\": %.1f}\n",
               proto, pairs, words, iters, h[0], h[1], h[2] * 10.0 / iters);
        fflush(stdout);
      }
    }
    CHECK(hipFree(mpdata));
    CHECK(hipFree(errs));
  }

  // ---- 5. access latency by cache policy ----
  if (which == "all" || which == "latency") {
    unsigned long long* lo = nullptr;
    CHECK(hipMalloc(&lo, 2 * sizeof(unsigned long long)));
    for (uint32_t words : {1u << 18, 1u << 28}) {  // 1 MiB (cache resident), 1 GiB (HBM)
      std::vector<uint32_t> chain(words);
      const uint32_t stride = 1040;  // 4 KiB + 64 B in words
      for (uint32_t i = 0; i < words; ++i) chain[i] = (uint32_t)(((uint64_t)i + stride) % words);
      uint32_t* d = reinterpret_cast<uint32_t*>(src);  // reuse the 4 GiB read buffer
      CHECK(hipMemcpy(d, chain.data(), (size_t)words * 4, hipMemcpyHostToDevice));
      for (int mode = 0; mode < 3; ++mode) {
        for (int aux : {0, 1, 16, 17, 2}) {
          if (mode != 0 && aux != 0) continue;
          const int iters = 2000;
          hipLaunchKernelGGL(k_latency, dim3(1), dim3(64), 0, 0, d, words, iters, aux, mode, lo);  // warm
          hipLaunchKernelGGL(k_latency, dim3(1), dim3(64), 0, 0, d, words, iters, aux, mode, lo);
          CHECK(hipDeviceSynchronize());
          CHECK(hipGetLastError());
          unsigned long long h[2];
          CHECK(hipMemcpy(h, lo, sizeof(h), hipMemcpyDeviceToHost));
          printf("{\"bench\": \"latency\", \"bytes\": %llu, \"mode\": \"%s\", \"aux\": %d, \"ns\": %.1f}\n",
                 (unsigned long long)words * 4, mode == 0 ? "load" : (mode == 1 ? "atomic_add_ret" : "sc1_store_wait"),
                 aux, h[0] * 10.0 / iters);
          fflush(stdout);
        }
      }
    }
    CHECK(hipFree(lo));
  }

  CHECK(hipFree(xvec));
  CHECK(hipFree(results));
  CHECK(hipFree(src));
  CHECK(hipFree(sink));
  CHECK(hipFree(counters));
  CHECK(hipFree(pp_out));
  return 0;
}
