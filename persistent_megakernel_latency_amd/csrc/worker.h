// worker.h -- the device side of the decode-step megakernel: memory
// primitives, tile bodies, the control and compute waves' loops.  Included
// by megakernel.hip (the single-step megakernel and the per-operator baseline)
// and by persist.hip (the persistent grid), each its own translation unit, so
// that one kernel's code does not change the other's code generation.
//
// megakernel.hip -- the decode step as one persistent kernel on gfx950.
//
// Structure (what the pages describe, re-designed for MI355X):
//  * A megakernel owns the multi-operation program and the coordination between
//    operations ("Why real-time inference wants a megakernel", "The unit of
//    execution"); the host launches once per step and the GPU walks the
//    schedule: wait for the dependencies, run, signal the consumers (section
//    "What the megakernel changes").
//  * Workers are resident workgroups, several per CU (one launch of at most
//    the co-resident count), that claim tiles from device-side queues in a
//    topological order.  Each worker has one staging slot: the claimed tile's
//    weights are loaded into it before the tile's dependency counter is
//    checked, so weight streaming continues while predecessors finish
//    ("One Megakernel is Not Enough", Table I, weight prefetch; the Llama-1B
//    megakernel of "persistent-threads-megakernels", section 6, starts weight
//    loads for upcoming work early).
//  * Dependencies are counter groups (tile-to-tile tensor edges, Table I), not
//    operator barriers.
//
// A worker is one control wave plus four compute waves.  On CDNA a wave can
// only consume its loads in issue order (one vector-memory counter), so a wave
// that keeps 64 KiB of weights in flight cannot also take a quick round trip to
// a counter or an activation.  The roles are therefore split: the compute
// waves only stream weights and multiply (they issue the next tile's weight
// loads the moment they finish the current tile), while the control wave
// claims tiles, polls counters, stages activations into LDS, runs the
// epilogues, stores results and publishes.  The two sides meet at two
// workgroup barriers per tile (A: inputs staged; B: partial sums ready).
//
// Synchronisation, measured with microbench.hip on an MI355X:
//  * An agent-scope acquire fence (L2 invalidate) per 64 KiB tile cut streaming
//    reads from 6.2 to 2.2 TB/s and a release fence (L2 write-back) to 1.2 TB/s,
//    because each of the 8 XCDs has its own L2.  No fence is used in the hot
//    path: the control wave writes tile outputs with device-coherent (sc1,
//    write-through) stores, waits for their completion, then bumps the counter
//    with a relaxed device-scope atomic (performed past the L2s); consumers
//    read counters and activations with device-coherent (sc1) loads.  A
//    cross-XCD message-passing test of exactly this protocol saw no stale word
//    in 2000 x 8 rounds; plain stores in its place were stale.
//  * One address takes ~88 M atomics/s, so each counter group is spread over up
//    to 128 shards (two producers per shard) and tiles are claimed from 8
//    queues.  A phase's producers finish within a few microseconds of each
//    other, and their increments of one line queue behind each other: a batch-1
//    step took 963, 857, 818 and 772 us with 128, 32, 8 and 2 producers per
//    shard.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.h"
#include "wide_layout.h"
#include "wpk.h"

namespace wpk {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kBlock = kThreads + 64;  // one control wave + four compute waves

struct Slot {
  u32x4 c[kChunks];  // the tile's weights (or K/V chunk)
  u32x4 g[2];        // RMSNorm gains of this thread's columns (fp32 bits; 1.0 without a norm)
};

template <typename WT>
struct WT_ {
  static constexpr int EPC = 16 / sizeof(WT);              // elements per 16-byte chunk
  // LDS pitch (elements) of K rows [position][dim] and of transposed V rows
  // [dim][position]: 16-byte aligned rows, so each lane reads its row with
  // 16-byte loads (8 lanes of a pass cover all 32 banks)
  static constexpr int KP = sizeof(WT) == 2 ? 72 : 68;
};

template <typename WT, int KMAX>
struct alignas(16) Smem {
  union alignas(16) {
    float xs[KMAX];  // activation row of the current GEMV tile
    struct {
      WT ks[kAttnChunk * WT_<WT>::KP];  // attention tiles: K chunk, row per position
      WT vt[kHeadDim * WT_<WT>::KP];    // V chunk transposed, row per head dimension
    };
  };
  float red[kWaves][64];                       // per compute wave partial row sums
  float outs[kMaxGroupHeads][kHeadDim + 2];    // attention partial (m, l, o) per q head
  alignas(16) float qs[kMaxGroupHeads][kHeadDim];
  alignas(16) float ps[kMaxGroupHeads][kAttnChunk];
  int pos[kMaxBatch];  // seq_len of each sequence at step start
  int tok[kMaxBatch];  // input token of each sequence (validated)
  int ids[2];          // claim index of the next tile, by iteration parity
  alignas(16) int tnext[2][16];  // the next tile's descriptor, by iteration parity (compute wave 1 fetches it)
  uint64_t t_ready, t_done;  // logged steps: compute wave 1 saw its slot, finished its arithmetic
  float xinv;  // 1 / RMS of the staged activation row (1 without a norm), applied with the gains
  int first;
  int stop;
};

// The thread index, made opaque to the optimiser.  Inside the persistent tile
// loop the compiler would otherwise hoist every tile type's per-lane address
// arithmetic out of the loop and keep it all live, which multiplies the
// register footprint of the merged kernel (the register-pressure cost of
// megakernels the persistent-threads page discusses in section 4).
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}
__device__ __forceinline__ int wpk_tid() { return opaque((int)threadIdx.x); }

// ---- memory primitives ------------------------------------------------------------------

__device__ __forceinline__ u32x4 ld_nt(const void* p) { return __builtin_nontemporal_load((const u32x4*)p); }

__device__ __forceinline__ uint32_t ld_sc1(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_sc1(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_sc1(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint16_t ld_sc1(const uint16_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_sc1(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_sc1(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_sc1(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_sc1(uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t atomic_add(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16 bytes of fp32 activations with a device-coherent (sc1) buffer load.
__device__ __forceinline__ u32x4 ld_sc1_x4(const float* base, int32_t float_off) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, 0x7FFFFFFF, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b128(r, float_off * 4, 0, 16 /* sc1 */);
}

// 16 bytes stored with a device-coherent (sc1) buffer store.
__device__ __forceinline__ void st_sc1_x4(void* base, uint32_t byte_off, u32x4 v) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7FFFFFFF, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, 16 /* sc1 */);
}

// 8 bytes stored with a device-coherent (sc1) buffer store.
__device__ __forceinline__ void st_sc1_x2(void* base, uint32_t byte_off, u32x2 v) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7FFFFFFF, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b64(v, r, byte_off, 0, 16 /* sc1 */);
}

// Read-only tables (tiles, groups, queues) through the constant address space:
// uniform loads from it become scalar loads that do not count against the
// vector-memory counter.
template <class T>
__device__ __forceinline__ T cload(const T* p, int i) {
  static_assert(sizeof(T) % 4 == 0, "table entries are whole 32-bit words");
  T v;
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int W = sizeof(T) / 4;
  const int32_t __attribute__((address_space(4)))* src =
      (const int32_t __attribute__((address_space(4)))*)(const void*)p + (size_t)i * W;
  int32_t w[W];
#pragma unroll
  for (int k = 0; k < W; ++k) w[k] = src[k];
  __builtin_memcpy(&v, w, sizeof(T));
#else
  v = p[i];  // the host compilation pass never runs device code
#endif
  return v;
}

// Activations of layer l (one arena, fixed offsets per layer).
__device__ __forceinline__ float* act(const Params& P, int l, int32_t off) {
  return P.act + (size_t)l * P.act_layer + off;
}
__device__ __forceinline__ const float* x_in(const Params& P, int l) {
  return l == 0 ? nullptr : act(P, l - 1, P.off_x_out);
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// two floats rounded to bf16 (to nearest, ties to even; one v_cvt_pk_bf16_f32,
// which matches the bit-level rounding on every non-NaN input, denormals
// included, and gives a quiet NaN for a NaN) in one word, a in the low half
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
__device__ __forceinline__ uint16_t to_bf16(float f) { return (uint16_t)(cvt_bf16x2(f, 0.f) & 0xFFFFu); }
// f as bf16 hi + lo parts: two words, element pairs (a, b) in the low and high halves
__device__ __forceinline__ void split_hilo2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = cvt_bf16x2(a, b);
  lo = cvt_bf16x2(a - bf16_lo(hi), b - bf16_hi(hi));
}

// a.lo * b.lo + a.hi * b.hi + c over the bf16 halves of two 32-bit words
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

template <typename WT>
__device__ __forceinline__ void unpack(u32x4 c, float* o);
template <>
__device__ __forceinline__ void unpack<uint16_t>(u32x4 c, float* o) {
  o[0] = bf16_lo(c.x); o[1] = bf16_hi(c.x); o[2] = bf16_lo(c.y); o[3] = bf16_hi(c.y);
  o[4] = bf16_lo(c.z); o[5] = bf16_hi(c.z); o[6] = bf16_lo(c.w); o[7] = bf16_hi(c.w);
}
template <>
__device__ __forceinline__ void unpack<float>(u32x4 c, float* o) {
  o[0] = __uint_as_float(c.x); o[1] = __uint_as_float(c.y); o[2] = __uint_as_float(c.z); o[3] = __uint_as_float(c.w);
}

template <typename WT>
__device__ __forceinline__ float elt(const WT* a, int i) {
  if (sizeof(WT) == 2) return bf16_lo(((const uint16_t*)a)[i]);
  return ((const float*)a)[i];
}

// ---- cross-lane exchanges in registers ----------------------------------------------------
// (data-parallel-primitive moves within a row of 16 lanes, and the lane-swap
// moves between rows; a shuffle through the LDS crossbar would cost a round
// trip to the LDS per step)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
// The value of lane l ^ M, for M below 16.
template <int M>
__device__ __forceinline__ uint32_t xlane(uint32_t v) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8, "within a row of 16 lanes");
  if constexpr (M == 1) return dpp_u32<0xB1>(v);                   // quad permute 1,0,3,2
  else if constexpr (M == 2) return dpp_u32<0x4E>(v);              // quad permute 2,3,0,1
  else if constexpr (M == 4) return dpp_u32<0x141>(dpp_u32<0x1B>(v));  // quad reverse, then half-row mirror
  else return dpp_u32<0x128>(v);                                   // row rotate by 8
}
// The values of lanes l and l ^ M, in an order that depends on the lane (for
// commutative combinations: the result is the same bits in both lanes).
template <int M>
__device__ __forceinline__ void xpair(uint32_t v, uint32_t& a, uint32_t& b) {
  static_assert(M >= 1 && M <= 32 && (M & (M - 1)) == 0, "lane distance");
  if constexpr (M < 16) {
    a = v;
    b = xlane<M>(v);
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    a = r[0];
    b = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    a = r[0];
    b = r[1];
  }
}
template <int M>
__device__ __forceinline__ float xsum(float v) {
  uint32_t a, b;
  xpair<M>(__float_as_uint(v), a, b);
  return __uint_as_float(a) + __uint_as_float(b);
}
template <int M>
__device__ __forceinline__ float xmax(float v) {
  uint32_t a, b;
  xpair<M>(__float_as_uint(v), a, b);
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
template <int M>
__device__ __forceinline__ unsigned long long xmax_u64(unsigned long long v) {
  uint32_t al, bl, ah, bh;
  xpair<M>((uint32_t)v, al, bl);
  xpair<M>((uint32_t)(v >> 32), ah, bh);
  const unsigned long long a = (unsigned long long)ah << 32 | al, b = (unsigned long long)bh << 32 | bl;
  return a > b ? a : b;
}
// Sum or maximum over aligned groups of N lanes (N a power of two up to 64).
template <int N, int M = 1>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (M < N) return group_sum<N, 2 * M>(xsum<M>(v));
  else return v;
}
template <int N, int M = 1>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (M < N) return group_max<N, 2 * M>(xmax<M>(v));
  else return v;
}
template <int N, int M = 1>
__device__ __forceinline__ unsigned long long group_max_u64(unsigned long long v) {
  if constexpr (M < N) return group_max_u64<N, 2 * M>(xmax_u64<M>(v));
  else return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }
// Sum over the wave, wave-uniform.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += xlane<1>(v);
  v += xlane<2>(v);
  v += xlane<4>(v);
  v += xlane<8>(v);
  uint32_t a, b;
  xpair<16>(v, a, b);
  v = a + b;
  xpair<32>(v, a, b);
  return __builtin_amdgcn_readfirstlane(a + b);
}
__device__ __forceinline__ float wave_max(float v) { return group_max<64>(v); }

// lane l holds the wave-wide sum of value index scatter_index<N>(l).
// One level of the reduce-scatter: lanes exchange half their values with
// the lane M away, keeping the half their bit M selects.
template <int N, int M, int n>
__device__ __forceinline__ void rs_level(float (&v)[N], int lane) {
  if constexpr (n > 1) {
    const bool up = (lane & M) != 0;
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
      const float lo = v[i], hi = v[i + n / 2];  // selects on values, not on an index
      const float send = up ? lo : hi;
      const float keep = up ? hi : lo;
      v[i] = keep + __uint_as_float(xlane<M>(__float_as_uint(send)));
    }
    rs_level<N, 2 * M, n / 2>(v, lane);
  }
}
template <int N, int M>
__device__ __forceinline__ float rs_tail(float r) {
  if constexpr (M < 64) return rs_tail<N, 2 * M>(xsum<M>(r));
  else return r;
}
template <int N>
__device__ __forceinline__ float wave_reduce_scatter(float (&v)[N], int lane) {
  static_assert(N <= 16, "levels exchange within rows of 16 lanes");
  rs_level<N, 1, N>(v, lane);
  return rs_tail<N, N>(v[0]);
}
template <int N>
__device__ __forceinline__ int scatter_index(int lane) {
  int idx = 0;
#pragma unroll
  for (int s = 0, n = N; n > 1; ++s, n >>= 1)
    if ((lane >> s) & 1) idx += n / 2;
  return idx;
}

__device__ __forceinline__ void latch_error(const Params& P, int32_t code, int32_t tile) {
  uint32_t zero = 0;
  if (__hip_atomic_compare_exchange_strong(&P.ctl[CTL_STATUS], &zero, (uint32_t)code, __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
    st_sc1(&P.ctl[CTL_STATUS + 1], (uint32_t)tile);
    st_sc1(&P.ctl[CTL_STATUS + 2], (uint32_t)blockIdx.x);
    st_sc1(&P.ctl[CTL_STATUS + 3], P.ctl[CTL_EPOCH]);
  }
  st_sc1(&P.ctl[CTL_ABORT], 1u);
}

__device__ __forceinline__ bool is_gemv(int type) {
  return type == T_QKV || type == T_OPROJ || type == T_GATEUP || type == T_DOWN || type == T_LM;
}

// Greedy choice key: the float's bits mapped so that unsigned order is float
// order, then the inverted index, so a 64-bit maximum picks the largest value
// and, among equal values, the lowest index.  -0 is taken as +0 (they compare
// equal, so the lower index wins between them) and a NaN gives the key 0,
// below every number: it is never chosen, as a float comparison never
// prefers it.
__device__ __forceinline__ unsigned long long pack_max(float v, int idx) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0ull;
  if (u == 0x80000000u) u = 0u;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)idx);
}

// Compiler-only ordering points of the hand-off protocol (no instruction is
// emitted).  The publish is a relaxed device-scope increment issued after the
// wave's device-coherent stores have completed (s_waitcnt); the consumer reads
// inputs with device-coherent loads after its poll saw the group complete.
// Nothing in the relaxed atomics themselves stops the compiler from moving a
// store below the completion wait or an input load above the successful poll,
// so both sides are pinned here.
__device__ __forceinline__ void compiler_order() { asm volatile("" ::: "memory"); }

// Wait until every memory operation this wave issued has completed (stores
// performed, loads and LDS-direct loads landed), with no memory access of the
// surrounding code moved across the wait.
__device__ __forceinline__ void wait_all_memory() {
  compiler_order();
  __builtin_amdgcn_s_waitcnt(0);
  compiler_order();
}

// ---- GEMV geometry ------------------------------------------------------------------------
//
// A GEMV tile is `rows` weight rows (two segments, so RoPE pairs (i, i+D/2) and
// gate/up pairs land in one tile) of a matrix with K columns, CPR 16-byte
// chunks per row.  Compute thread tc owns chunk j*256 + tc of the tile for
// j < 16, so each of its 16 loads is one fully coalesced 4 KiB piece.

template <int CPR>
struct Geo {
  static constexpr int LPR = CPR >= kThreads ? CPR / kThreads : 1;  // chunks of one row per thread
  static constexpr int NV = kChunks / LPR;                          // rows a thread contributes to
  static constexpr int ROWS = kThreads * kChunks / CPR;             // rows of a full tile
  static constexpr int WPR = CPR >= kThreads ? kWaves : CPR / 64;   // compute waves sharing a row
  static_assert(CPR >= 64 && ROWS <= 64, "unsupported row length");
};

// ============================ compute waves ===================================================

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, 0, 0x7FFFFFFF, 0x00020000);
}

// Where slice j of a tile's weights is: chunk j of thread tc is 16 bytes at
// lane offset tc*16 into slice j, a 4 KiB run of memory at a wave-uniform
// offset, read with one buffer load (resource and slice offset in scalar
// registers, one lane offset):
//  * GEMV: slice j is row (j / SPR) * SR of the tile (SR = 256 / CPR rows per
//    slice for short rows, SPR = CPR / 256 slices per row for long ones); the
//    device plan keeps segment boundaries and tile sizes on whole slices, so a
//    slice never straddles the two row segments.  Slices past a short tile or
//    past the matrix re-read its last valid slice (their sums are never stored).
//  * ATTN: for each KV chunk of the tile in turn, slices of K then V; lanes
//    past the cache capacity read its last chunk (those positions are never
//    used); chunks past the sequence read nothing.
//  * the remaining slots of an attention tile and every slot of a combine or
//    argmax tile read one 16-byte word (no HBM traffic; the value is unused).
template <typename WT, int CPR_H, int CPR_F>
struct SliceMap {
  static constexpr int RB = kHeadDim * (int)sizeof(WT);  // K/V bytes per position
  static constexpr int PPS = 4096 / RB;                  // positions per slice
  static constexpr int NS = kAttnChunk / PPS;            // slices of K (and of V)
  __amdgpu_buffer_rsrc_t rs0, rs1;
  bool gemv, attn;
  int limit, sh_spr, sr, rowb;

  int n_valid;  // attention: positions of the sequence in the cache this step

  __device__ __forceinline__ SliceMap(const Params& P, const Tile& T, int valid = 0) {
    const LayerW& lw = P.lw[T.layer];
    const int ty = T.type;
    gemv = is_gemv(ty);
    attn = ty == T_ATTN || ty == T_ATTNC;
    n_valid = valid;
    const void* w0 = P.embed;
    const void* w1 = P.embed;
    limit = P.V;
    int cpr = CPR_H;
    switch (ty) {
      case T_QKV: w0 = w1 = lw.w_qkv; limit = P.qkv_rows; break;
      case T_OPROJ: w0 = w1 = lw.w_o; limit = P.H; break;
      case T_GATEUP: w0 = lw.w_gate; w1 = lw.w_up; limit = P.F; break;
      case T_DOWN: w0 = w1 = lw.w_down; limit = P.H; cpr = CPR_F; break;
      case T_ATTN:
      case T_ATTNC: {
        const size_t sl = ((((size_t)T.layer * P.B + T.b) * P.Hkv + T.g) * P.cap) * RB;
        w0 = P.kc + sl;
        w1 = P.vc + sl;
        break;
      }
      default: break;
    }
    rs0 = rsrc(w0);
    rs1 = rsrc(w1);
    sh_spr = cpr >= kThreads ? __builtin_ctz(cpr / kThreads) : 0;
    sr = cpr >= kThreads ? 1 : kThreads / cpr;
    rowb = cpr * 16;
  }
  // slice j: its resource, its byte offset, and the largest lane offset that
  // stays inside valid data
  __device__ __forceinline__ void at(const Params& P, const Tile& T, int j, __amdgpu_buffer_rsrc_t& r, int& soff,
                                     uint32_t& last) const {
    const int row = min((j >> sh_spr) * sr, T.rows - sr);
    const bool seg1 = row >= T.rs;
    const int mrow = min(seg1 ? T.r1 + (row - T.rs) : T.r0 + row, limit - sr);
    const int g_off = mrow * rowb + (j & ((1 << sh_spr) - 1)) * 4096;
    const int u = j / (2 * NS), jj = j % (2 * NS);  // chunk of the tile, slice within it
    const int c = T.c + u;
    const int p0 = min(c * kAttnChunk + (jj % NS) * PPS, P.cap - 1);
    const bool a_real = u < T.kind && c * kAttnChunk < n_valid;
    const int a_off = a_real ? p0 * RB : 0;
    const uint32_t a_last = a_real ? (uint32_t)(P.cap - p0) * RB - 16u : 0u;
    soff = gemv ? g_off : (attn ? a_off : 0);
    last = gemv ? 0xFFFFFFF0u : (attn ? a_last : 0u);
    r = (gemv ? seg1 : (attn && jj >= NS && a_real)) ? rs1 : rs0;
  }
};

// Stages the tile's weights into the slot, and the RMSNorm gains of the
// columns this thread multiplies (loaded first, so waiting for them does not
// wait for the weights).  Combine and argmax tiles read nothing of use.
template <typename WT, int CPR_H, int CPR_F>
__device__ __forceinline__ void stage(const Params& P, const Tile& T, Slot& s, uint32_t voff, int n_valid = 0) {
  static_assert(CPR_H <= kThreads, "gains in the slot cover one chunk per thread");
  constexpr int EPC = WT_<WT>::EPC;
  const LayerW& lw = P.lw[T.layer];
  const int ty = T.type;
  const float* gain = ty == T_QKV ? lw.attn_norm : ty == T_GATEUP ? lw.mlp_norm : ty == T_LM ? P.final_norm : nullptr;
  if (gain) {
    const uint32_t goff = (voff / 16u % (uint32_t)CPR_H) * (EPC * 4);
    const __amdgpu_buffer_rsrc_t rg = rsrc(gain);
    s.g[0] = __builtin_amdgcn_raw_buffer_load_b128(rg, goff, 0, 0);
    s.g[1] = EPC == 8 ? __builtin_amdgcn_raw_buffer_load_b128(rg, goff + 16u, 0, 0) : s.g[0];
  } else {
    s.g[0] = s.g[1] = u32x4{0x3f800000u, 0x3f800000u, 0x3f800000u, 0x3f800000u};
  }
  const SliceMap<WT, CPR_H, CPR_F> m(P, T, n_valid);
#pragma unroll
  for (int j = 0; j < kChunks; ++j) {
    __amdgpu_buffer_rsrc_t r;
    int soff;
    uint32_t last;
    m.at(P, T, j, r, soff, last);
    s.c[j] = __builtin_amdgcn_raw_buffer_load_b128(r, min(voff, last), soff, 2 /* nt */);
  }
}



// Partial row sums of the staged tile against the activation row in LDS
// (times the RMSNorm gains the slot carries, for the K = hidden operators).
template <typename WT, int CPR, bool GAIN, int KMAX>
__device__ __forceinline__ void cmp_gemv(const Slot& s, Smem<WT, KMAX>& sm, int tc0) {
  const int tc = opaque(tc0);
  using G = Geo<CPR>;
  constexpr int EPC = WT_<WT>::EPC;
  static_assert(!GAIN || G::LPR == 1, "gains cover one column chunk per thread");
  const int lane = tc & 63, cw = tc >> 6;
  float acc[G::NV];
#pragma unroll
  for (int v = 0; v < G::NV; ++v) acc[v] = 0.f;
  float x[EPC];  // one column chunk: held for the whole tile when LPR == 1
  if (G::LPR == 1) {
    const int col = CPR >= kThreads ? tc : tc % CPR;
#pragma unroll
    for (int e = 0; e < EPC; e += 4) {
      const f32x4 v = *(const f32x4*)&sm.xs[col * EPC + e];
      x[e] = v.x; x[e + 1] = v.y; x[e + 2] = v.z; x[e + 3] = v.w;
    }
    if (GAIN) {
      const float xi = sm.xinv;
#pragma unroll
      for (int e = 0; e < EPC; ++e) x[e] *= __uint_as_float(s.g[e / 4][e % 4]) * xi;
    }
  }
  if constexpr (sizeof(WT) == 2 && G::LPR == 1) {
    // bf16 weights, one column chunk per thread: the chunk's activations as
    // hi + lo bf16 pairs (about 16 significant bits), split once per tile, so
    // each pair of weights takes two bf16 dot products instead of two unpacks
    // and two fp32 multiply-adds
    uint32_t xh[EPC / 2], xl[EPC / 2];
#pragma unroll
    for (int i = 0; i < EPC / 2; ++i) {
      xh[i] = cvt_bf16x2(x[2 * i], x[2 * i + 1]);
      xl[i] = cvt_bf16x2(x[2 * i] - bf16_lo(xh[i]), x[2 * i + 1] - bf16_hi(xh[i]));
    }
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      float a = acc[j];
#pragma unroll
      for (int i = 0; i < EPC / 2; ++i) {
        a = dot2_bf16(s.c[j][i], xh[i], a);
        a = dot2_bf16(s.c[j][i], xl[i], a);
      }
      acc[j] = a;
    }
  } else {
#pragma unroll
  for (int j = 0; j < kChunks; ++j) {
    if (G::LPR > 1) {  // chunks cycle through LPR columns: read this one from LDS
      const int col = (j % G::LPR) * kThreads + tc;
#pragma unroll
      for (int e = 0; e < EPC; e += 4) {
        const f32x4 v = *(const f32x4*)&sm.xs[col * EPC + e];
        x[e] = v.x; x[e + 1] = v.y; x[e + 2] = v.z; x[e + 3] = v.w;
      }
    }
    float w[EPC];
    unpack<WT>(s.c[j], w);
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[j / G::LPR] = fmaf(w[e], x[e], acc[j / G::LPR]);
  }
  }
  const float r = wave_reduce_scatter<G::NV>(acc, lane);
  if (lane < G::NV) sm.red[cw][scatter_index<G::NV>(lane)] = r;
}

// Staged K/V chunk -> LDS rows, except the row of the position being appended
// this step, which the control wave writes (it was staged before it existed).
template <typename WT, int KMAX>
__device__ __forceinline__ void dump_kv(const Params& P, const Tile& T, const Slot& s, Smem<WT, KMAX>& sm, int tc0) {
  const int tc = opaque(tc0);
  constexpr int CPP = kHeadDim * sizeof(WT) / 16, KCH = kAttnChunk * CPP, EPC = WT_<WT>::EPC;
  constexpr int KP = WT_<WT>::KP;
  const int p = sm.pos[T.b];
  const int skip = p - T.c * kAttnChunk;
#pragma unroll
  for (int j = 0; j < 2 * KCH / kThreads; ++j) {
    const int flat = j * kThreads + tc;
    const bool isv = flat >= KCH;  // uniform per j
    const int f = isv ? flat - KCH : flat;
    const int pos = f / CPP, dc = f % CPP;
    if (pos == skip) continue;
    if (!isv) {
      *(u32x4*)(sm.ks + pos * KP + dc * EPC) = s.c[j];
    } else {
      float w[EPC];
      unpack<WT>(s.c[j], w);
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        WT* d = sm.vt + (dc * EPC + e) * KP + pos;
        if (sizeof(WT) == 2) *(uint16_t*)d = (uint16_t)(__float_as_uint(w[e]) >> 16);
        else *(float*)d = w[e];
      }
    }
  }
}

__device__ __forceinline__ int attn_count(const Params& P, const Tile& T, int p) {
  const int n = p < 0 ? 0 : min(p + 1, P.cap);
  return max(0, min(kAttnChunk, n - T.c * kAttnChunk));
}

// Positions of a sequence in the cache this step (its own position included).
__device__ __forceinline__ int attn_valid(const Params& P, int p) { return p < 0 ? 0 : min(p + 1, P.cap); }

// Slot chunks one KV chunk occupies (K then V of 64 positions).
template <typename WT>
constexpr int kv_chunks() {
  return 2 * kAttnChunk * (kHeadDim * (int)sizeof(WT) / 16) / kThreads;
}

// The next KV chunk of a multi-chunk attention tile moves to the front of the
// slot (register moves; the slot is never indexed with a run-time value).
template <typename WT>
__device__ __forceinline__ void slot_shift(Slot& s) {
  constexpr int CH = kv_chunks<WT>();
#pragma unroll
  for (int j = 0; j + CH < kChunks; ++j) s.c[j] = s.c[j + CH];
}

__device__ __forceinline__ Tile sub_chunk(const Tile& T, int u) {
  Tile U = T;
  U.c = T.c + u;
  return U;
}

__device__ __forceinline__ bool is_attn(int type) { return type == T_ATTN || type == T_ATTNC; }

// KV chunks holding positions of the sequence this step.
__device__ __forceinline__ int attn_active(const Params& P, int p) {
  return (attn_valid(P, p) + kAttnChunk - 1) / kAttnChunk;
}

// Passes of a tile: the sequences of a narrow GEMV tile, the KV chunks of an
// attention tile (a chained one: only the chunks holding positions), else one.
template <bool WIDE>
__device__ __forceinline__ int n_passes(const Params& P, const Tile& T, int p) {
  if (!WIDE && is_gemv(T.type)) return P.B;
  if (T.type == T_ATTN) return T.kind;
  if (WIDE && T.type == T_ATTNC) return max(1, attn_active(P, p));  // at least one (empty) pass
  return 1;
}

// The chunks of a chained attention tile the slot holds from chunk c0 on.
template <typename WT>
__device__ __forceinline__ Tile attn_group(const Tile& T, int c0) {
  constexpr int S = kChunks / kv_chunks<WT>();
  Tile G = T;
  G.c = c0;
  G.kind = min(S, T.kind - c0);
  return G;
}

// Running merge of the chunk partials of an attention tile (control wave;
// lane = head dimension), fed from LDS: a wide plan's tile stores one merged
// partial for its chunks, a chained tile the merged and normalised output.
struct AttnRun {
  float M[kMaxGroupHeads], L[kMaxGroupHeads], O[kMaxGroupHeads];
};
__device__ __forceinline__ void attn_run_init(AttnRun& r) {
#pragma unroll
  for (int h = 0; h < kMaxGroupHeads; ++h) {
    r.M[h] = -INFINITY;
    r.L[h] = 0.f;
    r.O[h] = 0.f;
  }
}
template <typename WT, int KMAX>
__device__ __forceinline__ void attn_run_merge(const Params& P, AttnRun& r, const Smem<WT, KMAX>& sm, int lane) {
#pragma unroll
  for (int h = 0; h < kMaxGroupHeads; ++h) {
    if (h >= P.G) break;
    // m and l are one value per head: scalar registers
    const float m = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sm.outs[h][0])));
    const float l = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(sm.outs[h][1])));
    const float o = sm.outs[h][2 + lane];
    const float Mn = fmaxf(r.M[h], m);
    const float keep = __expf(r.M[h] - Mn), w = __expf(m - Mn);
    r.L[h] = fmaf(r.L[h], keep, l * w);
    r.O[h] = fmaf(r.O[h], keep, o * w);
    r.M[h] = Mn;
  }
}
// The merged partial of a wide plan's attention tile, at partial slot
// T.c / attn_sub (nothing for a tile past its sequence: never read).
template <typename WT, int KMAX>
__device__ __forceinline__ void attn_run_partial(const Params& P, const Tile& T, const AttnRun& r,
                                                 const Smem<WT, KMAX>& sm, int lane) {
  if (attn_count(P, T, sm.pos[T.b]) == 0) return;
  float* out = act(P, T.layer, P.off_part) +
               ((((size_t)T.b * P.Hkv + T.g) * P.nch + T.c / P.attn_sub) * P.G) * (P.D + 2);
#pragma unroll
  for (int h = 0; h < kMaxGroupHeads; ++h) {
    if (h >= P.G) break;
    float* o = out + h * (P.D + 2);
    st_sc1(o + 2 + lane, r.O[h]);
    if (lane == 0) {
      st_sc1(o, r.M[h]);
      st_sc1(o + 1, r.L[h]);
    }
  }
}

// The merged output of the group's q heads: fp32 rows, or the hi/lo operand
// planes of the o-proj in a wide plan.  No chunk at all (an inactive slot): 0.
template <bool WIDE>
__device__ __forceinline__ void attn_run_store(const Params& P, const Tile& T, const AttnRun& r, int nact, int lane) {
#pragma unroll
  for (int h = 0; h < kMaxGroupHeads; ++h) {
    if (h >= P.G) break;
    const float o = nact == 0 ? 0.f : r.O[h] / r.L[h];
    const size_t at = (size_t)T.b * P.H + (size_t)(T.g * P.G + h) * P.D + lane;
    if (WIDE) {
      uint16_t* xa = (uint16_t*)act(P, T.layer, P.off_xattn);
      const uint16_t hi = to_bf16(o);
      st_sc1(xa + at, hi);
      st_sc1(xa + (size_t)kMaxBatch * P.H + at, to_bf16(o - bf16_lo(hi)));
    } else {
      st_sc1(act(P, T.layer, P.off_attn) + at, o);
    }
  }
}


#ifndef WPK_ATTN_GROUP
#define WPK_ATTN_GROUP 1
#endif

// Attention partial of a bf16 KV chunk on the matrix cores
// (v_mfma_f32_16x16x32_bf16), the kv head's q heads as the columns:
//  * scores S^T = K Q^T: A = K rows from LDS (lane l: position l % 16 of a
//    16-position block, dims 8 (l / 16) + 32 s ..), B = the queries scaled
//    by 1/sqrt(D) as hi + lo bf16 parts (lane l: q head l % 16, zero past the
//    group; K is bf16 and exact, so the two products keep ~16 bits of q).
//    Every compute wave computes all 64 positions (16 products): lane l then
//    holds positions 16 kb + 4 (l / 16) + e of head l % 16, and the softmax
//    over the chunk (positions past its count masked) needs only exchanges
//    between the four lanes of a head.
//  * weighted values O^T = V^T P^T: wave w takes head dims 16 w .. +15; A =
//    the transposed V rows from LDS, B = the lane's own probabilities as hi +
//    lo bf16, both in the K order 8 (l / 16) + 4 j + e <-> position
//    32 t + 16 j + 4 (l / 16) + e of 32-position step t.  V values of
//    positions past the count are zeroed (the cache holds anything there).
// Lane l ends with dims 16 w + 4 (l / 16) + e of head l % 16.
// Used by the matrix-core plans (batch 5-32).  Measured at batch 32: the
// pass's arithmetic fell from ~1.4 us on the vector units to ~0.3 us, the step
// by ~1% (2216 -> 2194 us): an attention tile's time is its K/V chunks
// streaming in (~7.6 us from its start to its inputs being staged), not its
// arithmetic.  Narrow plans keep the vector-unit pass below: in their
// 128-register budget, next to the 64-register slot, this one spilled and the
// batch-1 step was ~1% slower.
template <typename WT, int KMAX>
__device__ __forceinline__ void cmp_attn_mx(const Params& P, const Tile& T, Smem<WT, KMAX>& sm, int tc0) {
  static_assert(sizeof(WT) == 2 && kHeadDim == 64 && kAttnChunk == 64 && kWaves == 4, "bf16, 64 dims, 64 positions");
  constexpr int KP = WT_<WT>::KP;
  const int tc = opaque(tc0);
  const int lane = tc & 63, w = __builtin_amdgcn_readfirstlane(tc >> 6);
  const int cnt = attn_count(P, T, sm.pos[T.b]);
  if (cnt == 0) return;
  const int l15 = lane & 15, g4 = lane >> 4;
  const bool live = l15 < P.G;
  bf16x8 qh[2], ql[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const float* qr = &sm.qs[live ? l15 : 0][32 * s + 8 * g4];
    const float sc = live ? P.attn_scale : 0.f;
    const f32x4 a = *(const f32x4*)qr * sc, b = *(const f32x4*)(qr + 4) * sc;
    uint32_t h[4], l[4];
    split_hilo2(a[0], a[1], h[0], l[0]);
    split_hilo2(a[2], a[3], h[1], l[1]);
    split_hilo2(b[0], b[1], h[2], l[2]);
    split_hilo2(b[2], b[3], h[3], l[3]);
    qh[s] = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
    ql[s] = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
  }
  const uint16_t* ks = (const uint16_t*)sm.ks;
  f32x4 st[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const uint16_t* kr = ks + (16 * kb + l15) * KP + 8 * g4;
    const bf16x8 k0 = *(const bf16x8*)kr, k1 = *(const bf16x8*)(kr + 32);
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qh[0], z, 0, 0, 0);
    z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, ql[0], z, 0, 0, 0);
    z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qh[1], z, 0, 0, 0);
    z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, ql[1], z, 0, 0, 0);
    st[kb] = z;
  }
  float m = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = 16 * kb + 4 * g4 + e < cnt ? st[kb][e] : -INFINITY;
      st[kb][e] = v;
      m = fmaxf(m, v);
    }
  m = xmax<32>(xmax<16>(m));
  float l = 0.f;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
    for (int e = 0; e < 4; ++e) st[kb][e] = __expf(st[kb][e] - m);
    l += (st[kb][0] + st[kb][1]) + (st[kb][2] + st[kb][3]);
  }
  l = xsum<32>(xsum<16>(l));
  const uint16_t* vr = (const uint16_t*)sm.vt + (16 * w + l15) * KP + 4 * g4;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    uint32_t ph[4], pl[4], vv[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const f32x4 pr = st[2 * t + j];
      split_hilo2(pr[0], pr[1], ph[2 * j], pl[2 * j]);
      split_hilo2(pr[2], pr[3], ph[2 * j + 1], pl[2 * j + 1]);
      const int p0 = 32 * t + 16 * j + 4 * g4;  // positions p0 .. p0 + 3
      const u32x2 v = *(const u32x2*)(vr + 32 * t + 16 * j);
      vv[2 * j] = p0 + 1 < cnt ? v.x : p0 < cnt ? (v.x & 0xFFFFu) : 0u;
      vv[2 * j + 1] = p0 + 3 < cnt ? v.y : p0 + 2 < cnt ? (v.y & 0xFFFFu) : 0u;
    }
    const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{vv[0], vv[1], vv[2], vv[3]});
    o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, __builtin_bit_cast(bf16x8, u32x4{ph[0], ph[1], ph[2], ph[3]}), o,
                                                0, 0, 0);
    o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, __builtin_bit_cast(bf16x8, u32x4{pl[0], pl[1], pl[2], pl[3]}), o,
                                                0, 0, 0);
  }
  if (live) {
    float* out = &sm.outs[l15][2 + 16 * w + 4 * g4];
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = o[e];
    if (w == 0 && g4 == 0) {
      sm.outs[l15][0] = m;
      sm.outs[l15][1] = l;
    }
  }
}

// Attention partial: compute wave h = q head h of the group, lane = position
// (scores) then lane = head dimension (weighted values).  Both loops are
// unrolled so that the LDS reads of a row are in flight together.
template <typename WT, int KMAX>
__device__ __forceinline__ void cmp_attn(const Params& P, const Tile& T, Smem<WT, KMAX>& sm, int tc0) {
  const int tc = opaque(tc0);
  constexpr int KP = WT_<WT>::KP, EPC = WT_<WT>::EPC;
  const int lane = tc & 63, h = tc >> 6;
  const int cnt = attn_count(P, T, sm.pos[T.b]);
  if (h >= P.G || cnt == 0) return;
  // Both loops go over groups of two 16-byte row chunks; the next group's LDS
  // reads are issued before this group's products (scheduling barriers keep
  // them there), so the reads overlap the arithmetic instead of each one
  // being waited for.  The multiply-add order is the plain loop's.
  constexpr int QPC = EPC / 4;  // 16-byte query (or weight) reads per row chunk
  constexpr int GC = WPK_ATTN_GROUP;  // row chunks per group
  float sc = -INFINITY;
  if (lane < cnt) {
    const WT* kr = sm.ks + lane * KP;
    const float* qh = &sm.qs[h][0];
    float d0 = 0.f, d1 = 0.f;
    u32x4 kc[GC];
    f32x4 qc[GC * QPC];
#pragma unroll
    for (int i = 0; i < GC; ++i) kc[i] = *(const u32x4*)(kr + i * EPC);
#pragma unroll
    for (int j = 0; j < GC * QPC; ++j) qc[j] = *(const f32x4*)(qh + 4 * j);
#pragma unroll
    for (int g = 0; g < kHeadDim / (GC * EPC); ++g) {
      const int dn = (g + 1) * GC * EPC;
      u32x4 kn[GC];
      f32x4 qn[GC * QPC];
      if (dn < kHeadDim) {
#pragma unroll
        for (int i = 0; i < GC; ++i) kn[i] = *(const u32x4*)(kr + dn + i * EPC);
#pragma unroll
        for (int j = 0; j < GC * QPC; ++j) qn[j] = *(const f32x4*)(qh + dn + 4 * j);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < GC; ++i) {
        float k[EPC];
        unpack<WT>(kc[i], k);
#pragma unroll
        for (int e = 0; e < EPC; e += 4) {
          const f32x4 q = qc[i * QPC + e / 4];
          d0 = fmaf(q.x, k[e], d0);
          d1 = fmaf(q.y, k[e + 1], d1);
          d0 = fmaf(q.z, k[e + 2], d0);
          d1 = fmaf(q.w, k[e + 3], d1);
        }
      }
      if (dn < kHeadDim) {
#pragma unroll
        for (int i = 0; i < GC; ++i) kc[i] = kn[i];
#pragma unroll
        for (int j = 0; j < GC * QPC; ++j) qc[j] = qn[j];
      }
    }
    sc = (d0 + d1) * P.attn_scale;
  }
  const float m = wave_max(sc);
  const float e = lane < cnt ? __expf(sc - m) : 0.f;
  const float l = wave_sum(e);
  sm.ps[h][lane] = e;
  // weighted values: lane = head dimension, its transposed V row read 16 bytes
  // at a time over the whole chunk (all reads in flight together); positions
  // past the chunk's count hold no data and are masked
  const WT* vr = sm.vt + lane * KP;
  const float* ph = &sm.ps[h][0];
  float o0 = 0.f, o1 = 0.f;
  u32x4 vc[GC];
  f32x4 pc[GC * QPC];
#pragma unroll
  for (int i = 0; i < GC; ++i) vc[i] = *(const u32x4*)(vr + i * EPC);
#pragma unroll
  for (int j = 0; j < GC * QPC; ++j) pc[j] = *(const f32x4*)(ph + 4 * j);
#pragma unroll
  for (int g = 0; g < kAttnChunk / (GC * EPC); ++g) {
    const int jn = (g + 1) * GC * EPC;
    u32x4 vn[GC];
    f32x4 pn[GC * QPC];
    if (jn < kAttnChunk) {
#pragma unroll
      for (int i = 0; i < GC; ++i) vn[i] = *(const u32x4*)(vr + jn + i * EPC);
#pragma unroll
      for (int j = 0; j < GC * QPC; ++j) pn[j] = *(const f32x4*)(ph + jn + 4 * j);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < GC; ++i) {
      const int j0 = g * GC * EPC + i * EPC;
      float v[EPC];
      unpack<WT>(vc[i], v);
#pragma unroll
      for (int u = 0; u < EPC; u += 4) {
        const f32x4 pw = pc[i * QPC + u / 4];
        o0 = fmaf(pw.x, j0 + u < cnt ? v[u] : 0.f, o0);
        o1 = fmaf(pw.y, j0 + u + 1 < cnt ? v[u + 1] : 0.f, o1);
        o0 = fmaf(pw.z, j0 + u + 2 < cnt ? v[u + 2] : 0.f, o0);
        o1 = fmaf(pw.w, j0 + u + 3 < cnt ? v[u + 3] : 0.f, o1);
      }
    }
    if (jn < kAttnChunk) {
#pragma unroll
      for (int i = 0; i < GC; ++i) vc[i] = vn[i];
#pragma unroll
      for (int j = 0; j < GC * QPC; ++j) pc[j] = pn[j];
    }
  }
  sm.outs[h][2 + lane] = o0 + o1;
  if (lane == 0) {
    sm.outs[h][0] = m;
    sm.outs[h][1] = l;
  }
}

// Merge of the attention partials of one (sequence, kv head): compute wave h
// merges q head h (lane = head dimension), reading the chunks in batches of
// 16 with all of a batch's loads in flight together, and rescaling the running
// sums when a batch raises the maximum.  The wave waits for its stores, so the
// tile is complete when the control wave publishes after barrier B.
template <typename WT, bool WIDE, int KMAX>
__device__ __forceinline__ void cmp_combine(const Params& P, const Tile& T, const Smem<WT, KMAX>& sm, int tc0) {
  const int tc = opaque(tc0);
  const int lane = tc & 63, h = tc >> 6;
  if (h >= P.G) return;
  const int p = sm.pos[T.b];
  const int n = p < 0 ? 0 : min(p + 1, P.cap);
  const int nact = ((n + kAttnChunk - 1) / kAttnChunk + P.attn_sub - 1) / P.attn_sub;  // one partial per tile
  float* dst = act(P, T.layer, P.off_attn) + (size_t)T.b * P.Hq * P.D + (size_t)(T.g * P.G + h) * P.D;
  const float* part = act(P, T.layer, P.off_part) + (((size_t)T.b * P.Hkv + T.g) * P.nch * P.G + h) * (P.D + 2);
  const int stride = P.G * (P.D + 2);
  float M = -INFINITY, L = 0.f, O = 0.f;
  for (int c0 = 0; c0 < nact; c0 += 16) {
    const int nb = min(16, nact - c0);
    const int k = lane & 15;
    const float* pk = part + (size_t)(c0 + min(k, nb - 1)) * stride;
    const float mk = ld_sc1(pk), lk = ld_sc1(pk + 1);
    float o[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) o[c] = c < nb ? ld_sc1(part + (size_t)(c0 + c) * stride + 2 + lane) : 0.f;
    const float mb = group_max<16>(mk);
    const float Mn = fmaxf(M, mb);
    const float keep = __expf(M - Mn);
    const float wk = k < nb ? __expf(mk - Mn) : 0.f;
    const float lb = group_sum<16>(wk * lk);
    float ob = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) ob = fmaf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), c)), o[c], ob);
    L = fmaf(L, keep, lb);
    O = fmaf(O, keep, ob);
    M = Mn;
  }
  const float o = nact == 0 ? 0.f : O / L;
  if (WIDE) {  // the o-proj operand: hi and lo bf16 planes
    uint16_t* xa = (uint16_t*)act(P, T.layer, P.off_xattn);
    const size_t at = (size_t)T.b * P.H + (size_t)(T.g * P.G + h) * P.D + lane;
    const uint16_t hi = to_bf16(o);
    st_sc1(xa + at, hi);
    st_sc1(xa + (size_t)kMaxBatch * P.H + at, to_bf16(o - bf16_lo(hi)));
  } else {
    st_sc1(dst + lane, o);
  }
  wait_all_memory();
}

// ---- wide (matrix-core) tiles ---------------------------------------------------------------
//
// Batches above four: a tile is 64 weight rows x a 512-column slice of K for
// every sequence, on v_mfma_f32_16x16x32_bf16.  Compute wave w owns rows
// [16w, 16w+16) of the tile; chunk j of its slot is the A fragment of k-step j
// (lane l: row l % 16, columns 32j + 8(l / 16) .. +7).  The operand slice sits
// in LDS as 1 KiB B fragments (lane l: sequence l % 16 of a half, the same
// eight columns), hi and lo bf16 planes each: an operand value is hi + lo, so
// the product keeps about 16 significant bits of the fp32 activation.  Each
// slice leaves a partial sum of its rows; the row block's last slice to
// arrive adds them in slice order and runs the epilogue.

constexpr int kWideSteps = kWideK / 32;                     // k-steps of a slice
constexpr int kWideFrags = kWideSteps * 2 * 2;              // x sequence halves x hi/lo planes
static_assert(kWideFrags == kWidePieces, "the operand area of the reduction layout");
constexpr int kWideKmax = kWideFrags * 256 + kWidePart;     // LDS floats: B fragments, then the partial sums

__device__ __forceinline__ int wfrag(int ks, int h, int pl) { return (ks * 2 + h) * 2 + pl; }

// The tile descriptor in scalar registers.  It is wave-uniform; this keeps
// the compiler from indexing the kernel arguments (the per-layer weight
// table) with a vector register, which it can only do from a private copy.
__device__ __forceinline__ Tile uni(const Tile& T) {
  int32_t w[16];
  __builtin_memcpy(w, &T, sizeof(Tile));
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i] = __builtin_amdgcn_readfirstlane(w[i]);
  Tile U;
  __builtin_memcpy(&U, w, sizeof(Tile));
  return U;
}

template <typename WT, int KMAX>
__device__ __forceinline__ float* cpart(Smem<WT, KMAX>& sm) {
  return sm.xs + kWideFrags * 256;
}

// A wide tile's weight matrices (segment 0 and 1), K, row count, and the
// operand buffer it reads.  Pointers come from the per-layer table in device
// memory and kernel-argument values are read before they are selected: a
// select between two kernel-argument addresses makes the compiler copy all the
// arguments to private memory.
struct WideOp {
  const void* w0;
  const void* w1;
  const uint16_t* x;
  int K, limit;
};
__device__ __forceinline__ WideOp wide_op(const Params& P, const Tile& T0) {
  const Tile T = uni(T0);
  const LayerBufs lb = cload(P.layers, T.layer);
  const void* emb = P.embed;
  int32_t H = P.H, F = P.F, V = P.V, R = P.qkv_rows;
  asm volatile("" : "+s"(emb), "+s"(H), "+s"(F), "+s"(V), "+s"(R));
  // the operand pointer: one of the five consecutive fields xn1 .. xnf of the
  // table (an indexed scalar load, not a switch the compiler turns into a
  // private lookup table)
  const int xi = T.type == T_QKV ? 0 : T.type == T_OPROJ ? 1 : T.type == T_GATEUP ? 2 : T.type == T_DOWN ? 3 : 4;
  const uint16_t* x = cload((const uint16_t* const*)&P.layers[T.layer].xn1, xi);
  switch (T.type) {
    case T_QKV: return WideOp{lb.w_qkv, lb.w_qkv, x, H, R};
    case T_OPROJ: return WideOp{lb.w_o, lb.w_o, x, H, H};
    case T_GATEUP: return WideOp{lb.w_gate, lb.w_up, x, H, F};
    case T_DOWN: return WideOp{lb.w_down, lb.w_down, x, F, H};
    default: return WideOp{emb, emb, x, H, V};  // LM head: tiles carry the last layer
  }
}

// The slot of a wide tile: sixteen A fragments per compute wave.  Rows past
// the matrix (a ragged last LM block) re-read its last row; their sums are
// never stored.
__device__ __forceinline__ void stage_wide(const Params& P, const Tile& T0, Slot& s, int tc0) {
  const int tc = opaque(tc0);
  const Tile T = uni(T0);
  const int lane = tc & 63, w = __builtin_amdgcn_readfirstlane(tc >> 6);
  const WideOp o = wide_op(P, T);
  const bool seg1 = 16 * w >= T.rs;  // segments break on whole compute-wave row groups
  const int r = 16 * w + (lane & 15);
  const int mrow = min(seg1 ? T.r1 + (r - T.rs) : T.r0 + r, o.limit - 1);
  const __amdgpu_buffer_rsrc_t rs = rsrc(seg1 ? o.w1 : o.w0);
  const uint32_t voff = ((uint32_t)mrow * (uint32_t)o.K + (uint32_t)(T.c * kWideK + 8 * (lane >> 4))) * 2u;
#pragma unroll
  for (int j = 0; j < kChunks; ++j) s.c[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 64 * j, 2 /* nt */);
}

// The slice's products: per k-step, the A fragment times the hi and the lo B
// fragment of each sequence half; then the 16 x 16 accumulators to the
// partial-sum area, laid out as [half][tile row][16 sequences].
template <typename WT, int KMAX>
__device__ __forceinline__ void cmp_wide(const Params& P, const Slot& s, Smem<WT, KMAX>& sm, int tc0) {
  const int tc = opaque(tc0);
  const int lane = tc & 63, w = tc >> 6;
  const bool two = P.B > 16;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const uint32_t* xf = (const uint32_t*)sm.xs + lane * 4;
  // the k-step loop in two straight-line versions (one or two sequence
  // halves), the B fragments of step ks + 1 read while step ks multiplies, so
  // the LDS reads are in flight behind the matrix-core work instead of each
  // one waited for
  if (two) {
    bf16x8 b[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) b[f] = *(const bf16x8*)(xf + wfrag(0, f >> 1, f & 1) * 256);
#pragma unroll
    for (int ks = 0; ks < kWideSteps; ++ks) {
      bf16x8 nb[4];
      if (ks + 1 < kWideSteps) {
#pragma unroll
        for (int f = 0; f < 4; ++f) nb[f] = *(const bf16x8*)(xf + wfrag(ks + 1, f >> 1, f & 1) * 256);
      }
      __builtin_amdgcn_sched_barrier(0);  // the next step's reads stay ahead of this step's products
      const bf16x8 a = __builtin_bit_cast(bf16x8, s.c[ks]);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[0], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[2], acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[1], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[3], acc1, 0, 0, 0);
      if (ks + 1 < kWideSteps) {
#pragma unroll
        for (int f = 0; f < 4; ++f) b[f] = nb[f];
      }
    }
  } else {
    bf16x8 b[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) b[f] = *(const bf16x8*)(xf + wfrag(0, 0, f) * 256);
#pragma unroll
    for (int ks = 0; ks < kWideSteps; ++ks) {
      bf16x8 nb[2];
      if (ks + 1 < kWideSteps) {
#pragma unroll
        for (int f = 0; f < 2; ++f) nb[f] = *(const bf16x8*)(xf + wfrag(ks + 1, 0, f) * 256);
      }
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 a = __builtin_bit_cast(bf16x8, s.c[ks]);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[0], acc0, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[1], acc0, 0, 0, 0);
      if (ks + 1 < kWideSteps) {
#pragma unroll
        for (int f = 0; f < 2; ++f) b[f] = nb[f];
      }
    }
  }
  float* cp = cpart(sm);
  const int row = 16 * w + 4 * (lane >> 4), s16 = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) cp[(row + i) * 16 + s16] = acc0[i];
  if (two) {
#pragma unroll
    for (int i = 0; i < 4; ++i) cp[(kWideRows + row + i) * 16 + s16] = acc1[i];
  }
}

template <typename WT, int CPR_H, int CPR_F, bool WIDE, int KMAX>
__device__ __forceinline__ void compute(const Params& P, const Tile& T, const Slot& s, Smem<WT, KMAX>& sm, int tc) {
  if constexpr (WIDE) {
    switch (T.type) {
      case T_QKV:
      case T_OPROJ:
      case T_GATEUP:
      case T_DOWN:
      case T_LM: cmp_wide<WT>(P, s, sm, tc); break;
      case T_ATTN:
      case T_ATTNC:
        if constexpr (sizeof(WT) == 2) cmp_attn_mx<WT>(P, T, sm, tc);
        else cmp_attn<WT>(P, T, sm, tc);
        break;
      case T_COMBINE: cmp_combine<WT, true>(P, T, sm, tc); break;
      default: break;  // norm and argmax tiles are control-wave work
    }
    return;
  }
  switch (T.type) {
    case T_QKV:
    case T_OPROJ:
    case T_GATEUP:
    case T_LM: cmp_gemv<WT, CPR_H, true>(s, sm, tc); break;
    case T_DOWN: cmp_gemv<WT, CPR_F, false>(s, sm, tc); break;
    case T_ATTN:
    case T_ATTNC: cmp_attn<WT>(P, T, sm, tc); break;
    case T_COMBINE: cmp_combine<WT, false>(P, T, sm, tc); break;
    default: break;  // argmax is control-wave work
  }
}

// ============================ control wave ====================================================

// Stages the activation row of a GEMV tile for sequence b into LDS, applying
// the RMSNorm prologue (x / sqrt(mean(x^2) + eps) * gain) for the operators
// that have one; the embedding row of the token is layer 0's input (device-side
// input conversion).
template <typename WT, int K, bool EMBED, int KMAX>
__device__ __forceinline__ void ctl_input(const Params& P, const float* src, const float* gain, int b,
                                          Smem<WT, KMAX>& sm, int lane0) {
  const int lane = opaque(lane0);
  constexpr int NQ = K / 256;  // 1 KiB pieces of the row: 16 bytes per lane each
  static_assert(K % 256 == 0, "row length");
  if (!EMBED || src != nullptr) {
    // Device-coherent (sc1) loads straight into LDS: every piece in flight at
    // once, no registers held; then the norm, if any, in place.
    const __amdgpu_buffer_rsrc_t r = rsrc(src + (size_t)b * K);
#pragma unroll
    for (int i = 0; i < NQ; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)&sm.xs[256 * i], 16,
                                               (uint32_t)lane * 16u, 1024 * i, 0, 16 /* sc1 */);
    wait_all_memory();
    if (!gain) {
      sm.xinv = 1.f;
      return;
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const f32x4 v = *(const f32x4*)&sm.xs[256 * i + 4 * lane];
      ss = fmaf(v.x, v.x, ss); ss = fmaf(v.y, v.y, ss); ss = fmaf(v.z, v.z, ss); ss = fmaf(v.w, v.w, ss);
    }
    ss = wave_sum(ss);
    // the compute waves scale the row by 1 / RMS together with the gains
    sm.xinv = 1.0f / sqrtf(ss / (float)K + P.eps);
    return;
  }
  if constexpr (!EMBED) return;
  // layer 0: the token's embedding row (model dtype -> fp32), with the norm;
  // the compute waves apply the gains, which they stage with the weights
  constexpr int EPC = WT_<WT>::EPC;
  constexpr int NG = K / (64 * EPC);  // 16-byte chunks per lane
  static_assert(K % (64 * EPC) == 0, "row length");
  float v[NG * EPC];
  const char* row = (const char*)P.embed + (size_t)sm.tok[b] * K * sizeof(WT);
#pragma unroll
  for (int g = 0; g < NG; ++g) unpack<WT>(*(const u32x4*)(row + (size_t)(lane + 64 * g) * 16), &v[g * EPC]);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NG * EPC; ++i) ss = fmaf(v[i], v[i], ss);
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)K + P.eps);
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int c = 0; c < EPC; c += 4) {
      f32x4 o;
      o.x = v[g * EPC + c] * inv;
      o.y = v[g * EPC + c + 1] * inv;
      o.z = v[g * EPC + c + 2] * inv;
      o.w = v[g * EPC + c + 3] * inv;
      *(f32x4*)&sm.xs[(lane + 64 * g) * EPC + c] = o;
    }
  sm.xinv = 1.f;
}

// Values the epilogue needs, loaded together with the inputs.
struct EpiIn {
  float res;     // residual row (o-proj, down)
  float cs, sn;  // RoPE cos/sin (q and k rows)
};

template <typename WT, int KMAX>
__device__ __forceinline__ EpiIn ctl_preload(const Params& P, const Tile& T, int b, const Smem<WT, KMAX>& sm,
                                             int lane0) {
  const int lane = opaque(lane0);
  EpiIn e{0.f, 1.f, 0.f};
  const int p = sm.pos[b];
  switch (T.type) {
    case T_QKV:
      if (T.kind < 2 && lane < T.rs && p >= 0 && p < P.cap) {
        const int base = T.kind == 0 ? T.g * P.D : (P.Hq + T.g) * P.D;
        const int dim = T.r0 + lane - base;
        e.cs = P.rope_cos[p * (P.D / 2) + dim];
        e.sn = P.rope_sin[p * (P.D / 2) + dim];
      }
      break;
    case T_OPROJ:
      if (lane < T.rows && T.r0 + lane < P.H) {
        const int row = T.r0 + lane;
        if (T.layer == 0) {
          const WT* ep = (const WT*)P.embed + (size_t)sm.tok[b] * P.H + row;
          e.res = sizeof(WT) == 2 ? bf16_lo(*(const uint16_t*)ep) : *(const float*)ep;
        } else {
          e.res = ld_sc1(x_in(P, T.layer) + (size_t)b * P.H + row);
        }
      }
      break;
    case T_DOWN:
      if (lane < T.rows && T.r0 + lane < P.H) e.res = ld_sc1(act(P, T.layer, P.off_x_mid) + (size_t)b * P.H + T.r0 + lane);
      break;
    default:
      break;
  }
  return e;
}

// Full row sum of row `lane` of the tile from the compute waves' partials.
template <int CPR, typename WT, int KMAX>
__device__ __forceinline__ float row_sum(const Smem<WT, KMAX>& sm, int lane) {
  using G = Geo<CPR>;
  float y = 0.f;
  if (lane < G::ROWS) {
    if (CPR >= kThreads) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) y += sm.red[w][lane];
    } else {
      constexpr int S = kThreads / CPR;  // rows interleaved per value index
      const int v = lane / S, grp = lane % S;
#pragma unroll
      for (int w = 0; w < G::WPR; ++w) y += sm.red[grp * G::WPR + w][v];
    }
  }
  return y;
}

template <typename WT, int CPR, int KMAX>
__device__ __forceinline__ void ctl_gemv_out(const Params& P, const Tile& T, int b, const Smem<WT, KMAX>& sm,
                                             const EpiIn& e, int lane0) {
  const int lane = opaque(lane0);
  const float y = row_sum<CPR>(sm, lane);
  // the paired row (RoPE / gate-up): lane + rs, within a row of lanes for rs = 8
  const float y2 = T.rs == 8 ? __uint_as_float(xlane<8>(__float_as_uint(y))) : __shfl(y, min(lane + T.rs, 63));
  const int l = T.layer;
  const int p = sm.pos[b];
  switch (T.type) {
    case T_QKV: {
      if (p < 0) break;  // inactive slot: nothing to append
      if (p >= P.cap) {
        if (lane == 0) latch_error(P, WPK_E_CTX_FULL, T.id);
        break;
      }
      const int half = P.D / 2;
      if (T.kind < 2) {
        if (lane < T.rs) {
          const int head = T.g;
          const int base = T.kind == 0 ? head * P.D : (P.Hq + head) * P.D;
          const int dim = T.r0 + lane - base;
          const float ra = y * e.cs - y2 * e.sn, rb = y2 * e.cs + y * e.sn;
          if (T.kind == 0) {
            float* q = act(P, l, P.off_q) + (size_t)b * P.Hq * P.D + head * P.D;
            st_sc1(q + dim, ra);
            st_sc1(q + dim + half, rb);
          } else {
            const size_t at = ((((size_t)l * P.B + b) * P.Hkv + head) * P.cap + p) * P.D;
            if (sizeof(WT) == 2) {
              st_sc1((uint16_t*)P.kc + at + dim, to_bf16(ra));
              st_sc1((uint16_t*)P.kc + at + dim + half, to_bf16(rb));
            } else {
              st_sc1((float*)P.kc + at + dim, ra);
              st_sc1((float*)P.kc + at + dim + half, rb);
            }
          }
        }
      } else if (lane < T.rows) {
        const int base = (P.Hq + P.Hkv + T.g) * P.D;
        const int mrow = lane < T.rs ? T.r0 + lane : T.r1 + (lane - T.rs);
        const size_t at = ((((size_t)l * P.B + b) * P.Hkv + T.g) * P.cap + p) * P.D + (mrow - base);
        if (sizeof(WT) == 2) st_sc1((uint16_t*)P.vc + at, to_bf16(y));
        else st_sc1((float*)P.vc + at, y);
      }
      break;
    }
    case T_OPROJ:
      if (lane < T.rows && T.r0 + lane < P.H) st_sc1(act(P, l, P.off_x_mid) + (size_t)b * P.H + T.r0 + lane, e.res + y);
      break;
    case T_GATEUP:
      if (lane < T.rs && T.r0 + lane < P.F)
        st_sc1(act(P, l, P.off_h) + (size_t)b * P.F + T.r0 + lane, y / (1.0f + __expf(-y)) * y2);
      break;
    case T_DOWN:
      if (lane < T.rows && T.r0 + lane < P.H) st_sc1(act(P, l, P.off_x_out) + (size_t)b * P.H + T.r0 + lane, e.res + y);
      break;
    case T_LM: {
      const int row = T.r0 + lane;
      unsigned long long key = 0;
      if (lane < T.rows && row < P.V) {
        P.logits[(size_t)b * P.V + row] = y;
        key = pack_max(y, row);
      }
      key = group_max_u64<64>(key);
      if (lane == 0)
        __hip_atomic_fetch_max(&P.argmax[b * kArgmaxShards + T.id % kArgmaxShards], key, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
  }
}

// Attention inputs: the K/V row appended this step, if it falls in this
// chunk, and (first chunk of the tile only; they stay in LDS for the others)
// the group's queries.
template <typename WT, int KMAX>
__device__ __forceinline__ void ctl_attn_patch(const Params& P, const Tile& T, Smem<WT, KMAX>& sm, int lane) {
  constexpr int KP = WT_<WT>::KP;
  const int p = sm.pos[T.b];
  const int start = T.c * kAttnChunk;
  if (p >= start && p < start + kAttnChunk && p < P.cap) {
    const size_t at = ((((size_t)T.layer * P.B + T.b) * P.Hkv + T.g) * P.cap + p) * kHeadDim + lane;
    WT* kd = sm.ks + (p - start) * KP + lane;
    WT* vd = sm.vt + lane * KP + (p - start);
    if (sizeof(WT) == 2) {
      *(uint16_t*)kd = ld_sc1((const uint16_t*)P.kc + at);
      *(uint16_t*)vd = ld_sc1((const uint16_t*)P.vc + at);
    } else {
      *(float*)kd = ld_sc1((const float*)P.kc + at);
      *(float*)vd = ld_sc1((const float*)P.vc + at);
    }
  }
}

template <typename WT, int KMAX>
__device__ __forceinline__ void ctl_attn_in(const Params& P, const Tile& T, Smem<WT, KMAX>& sm, int lane0,
                                            bool first = true) {
  const int lane = opaque(lane0);
  if (attn_count(P, T, sm.pos[T.b]) == 0) return;
  if (!first) {
    ctl_attn_patch<WT>(P, T, sm, lane);
    return;
  }
  const float* q = act(P, T.layer, P.off_q) + (size_t)T.b * P.Hq * P.D + (size_t)T.g * P.G * P.D;
  float qv[kMaxGroupHeads];
#pragma unroll
  for (int h = 0; h < kMaxGroupHeads; ++h) qv[h] = h < P.G ? ld_sc1(q + h * P.D + lane) : 0.f;
  ctl_attn_patch<WT>(P, T, sm, lane);
#pragma unroll
  for (int h = 0; h < kMaxGroupHeads; ++h)
    if (h < P.G) sm.qs[h][lane] = qv[h];
}

template <typename WT, int KMAX>
__device__ __forceinline__ void ctl_attn_out(const Params& P, const Tile& T, const Smem<WT, KMAX>& sm, int lane0) {
  const int lane = opaque(lane0);
  if (attn_count(P, T, sm.pos[T.b]) == 0) return;  // past the sequence: the combine never reads it
  float* out = act(P, T.layer, P.off_part) + ((((size_t)T.b * P.Hkv + T.g) * P.nch + T.c) * P.G) * (P.D + 2);
  for (int h = 0; h < P.G; ++h) {
    float* o = out + h * (P.D + 2);
    st_sc1(o + 2 + lane, sm.outs[h][2 + lane]);
    if (lane == 0) {
      st_sc1(o, sm.outs[h][0]);
      st_sc1(o + 1, sm.outs[h][1]);
    }
  }
}

// Output conversion: greedy token and sequence advance.  Lane b*16 + s of a
// group of four sequences takes shard s of sequence b (and clears it for the
// next step); a 16-lane max reduction gives the packed (value, lowest index)
// maximum.
template <typename WT, int KMAX>
__device__ __forceinline__ void ctl_argmax(const Params& P, const Smem<WT, KMAX>& sm, int lane0) {
  const int lane = opaque(lane0);
  constexpr int SEQS = 64 / kArgmaxShards;
  for (int b0 = 0; b0 < P.B; b0 += SEQS) {
    const int b = b0 + lane / kArgmaxShards;
    unsigned long long best = 0;
    if (b < P.B)
      best = __hip_atomic_exchange(&P.argmax[(size_t)b0 * kArgmaxShards + lane], 0ull, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    best = group_max_u64<kArgmaxShards>(best);
    if (b < P.B && lane % kArgmaxShards == 0) {
      const int p = sm.pos[b];
      if (p >= 0 && p < P.cap) {
        st_sc1(&P.tokens[b], (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull)));
        st_sc1(&P.seq_len[b], p + 1);
      }
    }
  }
}

// ---- wide tiles: control wave ---------------------------------------------------------------

// The operand slice of a wide tile into LDS as B fragments: one LDS-direct
// device-coherent load per 1 KiB fragment (lane l: sequence 16h + l % 16,
// columns k0 + 32ks + 8(l / 16) .. +7 of the hi or lo plane), all in flight
// together.  Sequences past the batch read the zero rows of the buffer.
template <typename WT, int KMAX>
__device__ __forceinline__ void ctl_stage_x(const Params& P, const Tile& T0, Smem<WT, KMAX>& sm, int lane0) {
  const int lane = opaque(lane0);
  const Tile T = uni(T0);
  const WideOp o = wide_op(P, T);
  const __amdgpu_buffer_rsrc_t r = rsrc(o.x);
  const uint32_t voff = (uint32_t)((lane & 15) * o.K + 8 * (lane >> 4)) * 2u;
  const int nh = P.B > 16 ? 2 : 1;
  const int k0 = T.c * kWideK;
  for (int h = 0; h < nh; ++h)
#pragma unroll
    for (int ks = 0; ks < kWideSteps; ++ks)
#pragma unroll
      for (int pl = 0; pl < 2; ++pl) {
        const int soff = (pl * kMaxBatch * o.K + h * 16 * o.K + k0 + 32 * ks) * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(sm.xs + wfrag(ks, h, pl) * 256), 16, voff, soff, 0,
            16 /* sc1 */);
      }
  wait_all_memory();
}

__device__ __forceinline__ void st_hilo(uint16_t* plane0, size_t plane_elems, size_t at, float v) {
  const uint16_t hi = to_bf16(v);
  st_sc1(plane0 + at, hi);
  st_sc1(plane0 + plane_elems + at, to_bf16(v - bf16_lo(hi)));
}

// After barrier B of a wide tile: store this slice's partial sums, count its
// arrival; the row block's last slice loads the others (LDS-direct, into the
// operand area, up to 64 KiB at a time), adds all of them in slice order and
// runs the epilogue.  Lane l holds sequence 16h + l % 16 of rows l / 16 + 4m.
// True if this was the last slice (the operand area was overwritten).
// Logged steps: tw[0] = partial sums stored, tw[1] = arrival counted (its
// sign bit set for the last slice).
#ifndef WPK_WIDE_SUM_READS
#define WPK_WIDE_SUM_READS 4
#endif
constexpr int kWideSumReads = WPK_WIDE_SUM_READS;  // 16-byte LDS reads in flight per group of adds
template <typename WT, int KMAX, bool LOG = false>
__device__ __forceinline__ bool ctl_wide_post(const Params& P, const Tile& T0, Smem<WT, KMAX>& sm, int lane0,
                                              uint64_t* tw = nullptr) {
  const int lane = opaque(lane0);
  const Tile T = uni(T0);
  const int nh = P.B > 16 ? 2 : 1;
  const int per = WPK_WIDE_SLOT_PIECES(nh);  // 1 KiB pieces of a partial-sum slot
  const float* cp = cpart(sm);
  float* mine = P.wpart + (size_t)(T.pslot + T.c) * kWidePart;
  for (int i = 0; i < per; ++i)
    st_sc1_x4(mine, (uint32_t)(i * 64 + lane) * 16u, *(const u32x4*)(cp + (i * 64 + lane) * 4));
  wait_all_memory();
  if constexpr (LOG) tw[0] = __builtin_amdgcn_s_memrealtime();
  uint32_t old = 0;
  if (lane == 0) old = atomic_add(&P.fixc[(size_t)T.fix * kLine], 1u);
  old = __builtin_amdgcn_readfirstlane(__shfl(old, 0));
  if constexpr (LOG) tw[1] = __builtin_amdgcn_s_memrealtime() | ((int)old + 1 == T.b ? (1ull << 63) : 0ull);
  if ((int)old + 1 != T.b) return false;
  compiler_order();  // the other slices' partial sums are read only after their arrivals are counted
  // the last slice: no other slice of this row block touches the counter
  // again this step; it counts from zero in the next
  if (lane == 0) st_sc1(&P.fixc[(size_t)T.fix * kLine], 0u);
  // the slice sums: z[4h + k] holds rows lane / 4 + 16k of sequences
  // 16h + 4(lane % 4) .. +3, which is 16 consecutive bytes of a partial-sum
  // slot ([half][row][16 sequences] floats): one 16-byte LDS read per value
  // group, the 64 lanes of a read covering 1 KiB without bank conflicts
  float z[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) z[i] = 0.f;
  const int q = lane >> 4, s16 = lane & 15;
  const int l = T.layer;
  // o-proj and down: the residual and the next RMSNorm's gain, loaded together
  // with the other slices' partial sums (one round trip for all)
  const bool resid = T.type == T_OPROJ || T.type == T_DOWN;
  float rv[32];  // set (and live) only on the residual path
  // RMSNorm site this epilogue writes (o-proj: the MLP input of this layer;
  // down: the next layer's attention input, or after the last layer the final
  // norm's input): 0 attention input, 1 MLP input, 2 final
  const int last = l == P.L - 1;
  const int site = T.type == T_OPROJ ? 1 : 2 * last;
  const LayerBufs* nb = P.layers + (T.type == T_OPROJ ? l : l + 1 - last);
  if (resid) {
#pragma unroll
    for (int i = 0; i < 32; ++i) rv[i] = 0.f;
    // in the store mapping of the epilogue: entry 4i + k of lane l is row
    // 4(l % 16) + k of sequence 4i + l / 16
    const LayerBufs* lbp = P.layers + l;
    // o-proj: x_in (layer 0: the embedding row); down: x_mid (consecutive table fields)
    const float* res = cload((const float* const*)&lbp->x_in, T.type == T_OPROJ ? 0 : 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = 4 * i + q;
      if (i >= 4 * nh || n >= P.B) continue;
      if (res) {
        const u32x4 v = ld_sc1_x4(res, n * P.H + T.r0 + 4 * s16);
        rv[4 * i + 0] = __uint_as_float(v.x);
        rv[4 * i + 1] = __uint_as_float(v.y);
        rv[4 * i + 2] = __uint_as_float(v.z);
        rv[4 * i + 3] = __uint_as_float(v.w);
      } else {  // layer 0: the token's embedding row (bf16 weights: wide plans are bf16 only)
        const uint2 e = *(const uint2*)((const uint16_t*)P.embed + (size_t)sm.tok[n] * P.H + T.r0 + 4 * s16);
        rv[4 * i + 0] = __uint_as_float(e.x << 16);
        rv[4 * i + 1] = __uint_as_float(e.x & 0xFFFF0000u);
        rv[4 * i + 2] = __uint_as_float(e.y << 16);
        rv[4 * i + 3] = __uint_as_float(e.y & 0xFFFF0000u);
      }
    }
    const float* gsel = cload((const float* const*)&nb->attn_norm, site == 1 ? 1 : 0);
    const float* gfin = cload((const float* const*)&nb->final_norm, 0);
    const float* gain = site == 2 ? gfin : gsel;
    // the row block's 64 gains into the (otherwise unused) row-sum area
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(gain), (__attribute__((address_space(3))) void*)&sm.red[0][0], 4,
                                             (uint32_t)lane * 4u, T.r0 * 4, 0, 0);
  }
  // QKV, gate/up and LM head: the sums of squares of their operand's rows
  // (every 64-row block, per sequence), into the top of the operand area
  const bool consumer = T.type == T_QKV || T.type == T_GATEUP || T.type == T_LM;
  const int nrb = P.H / kWideRows;
  const int ssp = WPK_WIDE_SS_PIECES(nrb);  // 1 KiB pieces of the table [nrb][32]
  if (consumer) {
    const float* ssc = cload((const float* const*)&P.layers[l].ss1, T.type == T_QKV ? 0 : T.type == T_GATEUP ? 1 : 2);
    const __amdgpu_buffer_rsrc_t r = rsrc(ssc);
    for (int i = 0; i < ssp; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(sm.xs + (kWideFrags - ssp + i) * 256), 16,
          (uint32_t)lane * 16u, i * 1024, 0, 16 /* sc1 */);
  }
  // q and k rows: the RoPE factors of each sequence's position, [n][D/2] cos
  // then sin, into pieces 48..55 of the operand area (above the slices of a
  // K = hidden row block, below the sums of squares)
  float* const rl = sm.xs + WPK_WIDE_ROPE_PIECE * 256;
  if (T.type == T_QKV && T.kind < 2) {
    const __amdgpu_buffer_rsrc_t rc = rsrc(P.rope_cos), rs = rsrc(P.rope_sin);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = 8 * j + (lane >> 3);
      int p = n < P.B ? sm.pos[n] : 0;
      p = p < 0 || p >= P.cap ? 0 : p;
      const uint32_t voff = (uint32_t)(p * (kHeadDim / 2) + 4 * (lane & 7)) * 4u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (__attribute__((address_space(3))) void*)(rl + j * 256), 16,
                                               voff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(rl + (4 + j) * 256),
                                               16, voff, 0, 0, 0);
    }
  }
  // slices of a batch in LDS slots, the own slice skipped (it stays in the
  // compute waves' partial-sum area)
  const int fit = WPK_WIDE_FIT(nh);  // slots the operand area holds (wide_layout.h)
  for (int s0 = 0; s0 < T.b; s0 += fit + WPK_WIDE_ADVANCE(s0, T.c, fit)) {
    const int own = WPK_WIDE_HAS_OWN(s0, T.c, fit);
    const int s1 = min(T.b, s0 + fit + own);
    for (int sl = s0; sl < s1; ++sl) {
      if (sl == T.c) continue;
      const int slot = WPK_WIDE_SLOT_OF(sl, s0, T.c, own);
      const __amdgpu_buffer_rsrc_t r = rsrc(P.wpart + (size_t)(T.pslot + sl) * kWidePart);
      for (int i = 0; i < per; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void*)(sm.xs + (slot * per + i) * 256), 16,
            (uint32_t)lane * 16u, i * 1024, 0, 16 /* sc1 */);
    }
    wait_all_memory();
    for (int sl = s0; sl < s1; ++sl) {
      const int slot = WPK_WIDE_SLOT_OF(sl, s0, T.c, own);
      const float* src = sl == T.c ? cp : sm.xs + slot * per * 256;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h >= nh) break;
        // a half's four reads in flight together, then the adds (slice order
        // per value: the sums do not depend on the lane mapping)
#pragma unroll
        for (int k0 = 0; k0 < 4; k0 += kWideSumReads) {
          f32x4 t[kWideSumReads];
#pragma unroll
          for (int k = 0; k < kWideSumReads; ++k) t[k] = *(const f32x4*)(src + h * 1024 + (k0 + k) * 256 + 4 * lane);
#pragma unroll
          for (int k = 0; k < kWideSumReads; ++k) {
            float* zz = z + 4 * (4 * h + k0 + k);
            zz[0] += t[k].x;
            zz[1] += t[k].y;
            zz[2] += t[k].z;
            zz[3] += t[k].w;
          }
        }
      }
    }
  }
  if (consumer) {  // divide by the root mean square of the operand's row
    // sequence n = lane % 32: lanes n and n + 32 add the even and the odd row
    // blocks (at most 32: hidden <= 2048), each with its reads in flight
    // together and a fixed tree, then each other's sum; the 32 factors go
    // through LDS (the attention query area, unused by GEMM tiles) to the
    // lanes holding those sequences
    const float* ssl = sm.xs + (kWideFrags - ssp) * 256;
    const int n = lane & 31, par = lane >> 5;
    float a[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) a[j] = 2 * j + par < nrb ? ssl[(2 * j + par) * kMaxBatch + n] : 0.f;
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
      for (int j = 0; j < w; ++j) a[j] += a[j + w];
    const float sum = xsum<32>(a[0]);
    float* inv = &sm.qs[0][0];
    if (par == 0) inv[n] = 1.0f / sqrtf(sum / (float)P.H + P.eps);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h >= nh) break;
      const f32x4 iv = *(const f32x4*)&inv[16 * h + 4 * (lane & 3)];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float* zz = z + 4 * (4 * h + k);
        zz[0] *= iv.x;
        zz[1] *= iv.y;
        zz[2] *= iv.z;
        zz[3] *= iv.w;
      }
    }
  }
  // The sums into LDS ([sequence][row], pitch 68: conflict-free both ways;
  // the operand area is free after the slice sums), read back in the store
  // mapping: lane l owns rows 4(l % 16) .. +3 of sequence 4i + l / 16, so
  // sixteen lanes store a sequence's 64 rows with full 16- or 8-byte stores.
  constexpr int TP = 68;
  static_assert(TP == kWideTransposePitch, "the transposition pitch of the reduction layout");
  float* tr = sm.xs;
  {
    const int rr = lane >> 2, sq = 4 * (lane & 3);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h >= nh) break;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float* v = z + 4 * (4 * h + k);
        float* d = tr + (16 * h + sq) * TP + rr + 16 * k;
        d[0] = v[0];
        d[TP] = v[1];
        d[2 * TP] = v[2];
        d[3 * TP] = v[3];
      }
    }
  }
  const int r4 = 4 * s16;
  switch (T.type) {
    case T_QKV: {
      // rows [0, 32) are head dimensions [0, 32), rows [32, 64) dimensions
      // [32, 64): a RoPE pair is rows d and d + 32, on lanes s16 and s16 + 8
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i >= 4 * nh) break;
        const int n = 4 * i + q;
        const int p = n < P.B ? sm.pos[n] : -1;
        if (p < 0) continue;  // past the batch, or an inactive slot: nothing to append
        if (p >= P.cap) {
          latch_error(P, WPK_E_CTX_FULL, T.id);
          continue;
        }
        const f32x4 own = *(const f32x4*)&tr[n * TP + r4];
        const size_t at = ((((size_t)l * P.B + n) * P.Hkv + T.g) * P.cap + p) * P.D + r4;
        if (T.kind == 2) {
          st_sc1_x2((uint16_t*)P.vc, (uint32_t)(at * 2), u32x2{cvt_bf16x2(own.x, own.y), cvt_bf16x2(own.z, own.w)});
          continue;
        }
        const int lo = r4 < 32;  // this lane holds the first rows of its pairs
        const f32x4 oth = *(const f32x4*)&tr[n * TP + (lo ? r4 + 32 : r4 - 32)];
        const int d = r4 & 31;
        const f32x4 cs = *(const f32x4*)&rl[n * 32 + d], sn = *(const f32x4*)&rl[1024 + n * 32 + d];
        // dimension d: a cos - b sin; dimension d + 32: b cos + a sin (a = row d, b = row d + 32)
        const float sg = lo ? -1.f : 1.f;
        const float o0 = own.x * cs.x + sg * oth.x * sn.x, o1 = own.y * cs.y + sg * oth.y * sn.y,
                    o2 = own.z * cs.z + sg * oth.z * sn.z, o3 = own.w * cs.w + sg * oth.w * sn.w;
        if (T.kind == 0) {
          // a wave-uniform base (the buffer descriptor lives in scalar
          // registers); the sequence goes into the per-lane offset
          float* qd = act(P, l, P.off_q) + T.g * P.D;
          st_sc1_x4(qd, (uint32_t)(n * P.Hq * P.D + r4) * 4u,
                    u32x4{__float_as_uint(o0), __float_as_uint(o1), __float_as_uint(o2), __float_as_uint(o3)});
        } else {
          st_sc1_x2((uint16_t*)P.kc, (uint32_t)(at * 2), u32x2{cvt_bf16x2(o0, o1), cvt_bf16x2(o2, o3)});
        }
      }
      break;
    }
    case T_OPROJ:
    case T_DOWN: {
      // o-proj: x_mid = x_in + y; down: x_out = x_mid + y (consecutive table
      // fields); then gain * x as the next RMSNorm's operand and this row
      // block's sums of squares.  The sums go through LDS ([sequence][row],
      // pitch 68: conflict-free both ways) into the store mapping, where a
      // lane owns four consecutive rows and sixteen lanes a sequence's 64.
      const LayerBufs* lbp = P.layers + l;
      float* dst = cload((float* const*)&lbp->x_mid, T.type == T_OPROJ ? 0 : 1);
      uint16_t* plane = cload((uint16_t* const*)&nb->xn1, 2 * site);
      float* ssd = cload((float* const*)&nb->ss1, site);
      const f32x4 g4 = *(const f32x4*)&sm.red[0][4 * s16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i >= 4 * nh) break;
        const int n = 4 * i + q;
        const f32x4 v = *(const f32x4*)&tr[n * TP + 4 * s16];
        const float x0 = rv[4 * i] + v.x, x1 = rv[4 * i + 1] + v.y, x2 = rv[4 * i + 2] + v.z,
                    x3 = rv[4 * i + 3] + v.w;
        float sq = fmaf(x3, x3, fmaf(x2, x2, fmaf(x1, x1, x0 * x0)));
        if (n < P.B) {
          const uint32_t at = (uint32_t)(n * P.H + T.r0 + 4 * s16);
          st_sc1_x4(dst, at * 4u,
                    u32x4{__float_as_uint(x0), __float_as_uint(x1), __float_as_uint(x2), __float_as_uint(x3)});
          const float g0 = g4.x * x0, g1 = g4.y * x1, g2 = g4.z * x2, g3 = g4.w * x3;
          uint32_t h01, l01, h23, l23;
          split_hilo2(g0, g1, h01, l01);
          split_hilo2(g2, g3, h23, l23);
          st_sc1_x2(plane, at * 2u, u32x2{h01, h23});
          st_sc1_x2(plane, (uint32_t)(kMaxBatch * P.H) * 2u + at * 2u, u32x2{l01, l23});
        }
        sq = group_sum<16>(sq);
        if (s16 == 0 && n < P.B) st_sc1(ssd + (T.r0 / kWideRows) * kMaxBatch + n, sq);
      }
      break;
    }
    case T_GATEUP: {
      // rows [0, 32) are gate rows, [32, 64) the up rows of the same h columns
      uint16_t* xh = (uint16_t*)act(P, l, P.off_xh);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i >= 4 * nh) break;
        const int n = 4 * i + q;
        if (n >= P.B || s16 >= 8) continue;
        const f32x4 g = *(const f32x4*)&tr[n * TP + r4], u = *(const f32x4*)&tr[n * TP + 32 + r4];
        const float h0 = g.x / (1.0f + __expf(-g.x)) * u.x, h1 = g.y / (1.0f + __expf(-g.y)) * u.y,
                    h2 = g.z / (1.0f + __expf(-g.z)) * u.z, h3 = g.w / (1.0f + __expf(-g.w)) * u.w;
        const uint32_t at = (uint32_t)(n * P.F + T.r0 + r4) * 2u;
        uint32_t a01, b01, a23, b23;
        split_hilo2(h0, h1, a01, b01);
        split_hilo2(h2, h3, a23, b23);
        st_sc1_x2(xh, at, u32x2{a01, a23});
        st_sc1_x2(xh, (uint32_t)(kMaxBatch * P.F) * 2u + at, u32x2{b01, b23});
      }
      break;
    }
    default: {  // LM head: logits and the block's per-sequence maximum
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i >= 4 * nh) break;
        const int n = 4 * i + q;
        unsigned long long key = 0;
        if (n < P.B) {
          const f32x4 v = *(const f32x4*)&tr[n * TP + r4];
          const float vv[4] = {v.x, v.y, v.z, v.w};
          const int row0 = T.r0 + r4;
          float* lg = P.logits + (size_t)n * P.V + row0;
          if (row0 + 3 < P.V && (P.V & 3) == 0) {
            *(f32x4*)lg = v;  // four logits in one 16-byte store (rows of a vocab that is a multiple of 4)
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (row0 + k < P.V) lg[k] = vv[k];
          }
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            if (row0 + k < P.V) {
              const unsigned long long c = pack_max(vv[k], row0 + k);
              key = c > key ? c : key;
            }
          }
        }
        key = group_max_u64<16>(key);
        if (s16 == 0 && n < P.B)
          __hip_atomic_fetch_max(&P.argmax[n * kArgmaxShards + T.id % kArgmaxShards], key, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
      break;
    }
  }
  return true;
}

// The layer-0 tile of one sequence in a wide plan: its embedding row as the
// first QKV operand, gain * x in the hi/lo planes, and the row's sum of
// squares per 64-column block (the QKV epilogue divides by the root mean
// square).  Lane l holds columns 512g + 8l .. +7, so eight consecutive lanes
// cover one block.
template <typename WT, int KMAX>
__device__ __forceinline__ void ctl_norm(const Params& P, const Tile& T0, const Smem<WT, KMAX>& sm, int lane0) {
  const int lane = opaque(lane0);
  const Tile T = uni(T0);
  const int b = T.b, K = P.H;
  const int ng = K / 512;
  const LayerBufs* lbp = P.layers;
  const float* gain = cload((const float* const*)&lbp->attn_norm, 0);
  uint16_t* dst = cload((uint16_t* const*)&lbp->xn1, 0);
  float* ss = cload((float* const*)&lbp->ss1, 0);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    if (g >= ng) break;
    const int e = 512 * g + 8 * lane;
    float v[8];
    const u32x4 c = *(const u32x4*)((const uint16_t*)P.embed + (size_t)sm.tok[b] * K + e);
    unpack<uint16_t>(c, v);
    const f32x4 g0 = *(const f32x4*)(gain + e), g1 = *(const f32x4*)(gain + e + 4);
    const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    uint32_t hw[4], lw[4];
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float y0 = v[i] * gg[i], y1 = v[i + 1] * gg[i + 1];
      sq = fmaf(v[i], v[i], sq);
      sq = fmaf(v[i + 1], v[i + 1], sq);
      split_hilo2(y0, y1, hw[i / 2], lw[i / 2]);
    }
    st_sc1_x4(dst, (uint32_t)(b * K + e) * 2u, u32x4{hw[0], hw[1], hw[2], hw[3]});
    st_sc1_x4(dst, (uint32_t)((kMaxBatch + b) * K + e) * 2u, u32x4{lw[0], lw[1], lw[2], lw[3]});
    sq = group_sum<8>(sq);
    if ((lane & 7) == 0) st_sc1(ss + (8 * g + lane / 8) * kMaxBatch + b, sq);
  }
}

template <typename WT, int CPR_H, int CPR_F, bool WIDE, int KMAX>
__device__ __forceinline__ EpiIn ctl_pre(const Params& P, const Tile& T, int b, Smem<WT, KMAX>& sm, int lane,
                                         int& xkey) {
  constexpr int KH = CPR_H * 16 / sizeof(WT), KF = CPR_F * 16 / sizeof(WT);
  EpiIn e{0.f, 1.f, 0.f};
  if constexpr (WIDE) {
    if (is_gemv(T.type)) {
      // The operand slice stays in LDS for the worker's next tile of the
      // same operator and K slice (with queues dealt round-robin, a worker
      // keeps meeting the same slice of a four-slice operator), unless a
      // row-block reduction or an attention tile has overwritten it since.
      const int key = (T.layer * T_NTYPES + T.type) * 64 + T.c;
      if (key != xkey) {
        ctl_stage_x<WT>(P, T, sm, lane);
        xkey = key;
      }
    } else if (is_attn(T.type)) {
      ctl_attn_in<WT>(P, T, sm, lane, b == 0);
      xkey = -1;
    }
    return e;
  }
  if (is_gemv(T.type)) {
    // one activation row serves consecutive tiles of an operator (batch 1)
    const int key = T.layer * T_NTYPES + T.type;
    e = ctl_preload<WT>(P, T, b, sm, lane);
    if (P.B > 1 || key != xkey) {
      // the activation row and RMSNorm gain of each GEMV operator; a null
      // source is layer 0's embedding row, a null gain a plain copy
      const int ty = T.type, l = T.layer;
      if (ty == T_DOWN) {
        ctl_input<WT, KF, false>(P, act(P, l, P.off_h), nullptr, b, sm, lane);
      } else {
        const float* src = ty == T_QKV ? x_in(P, l)
                         : ty == T_OPROJ ? act(P, l, P.off_attn)
                         : ty == T_GATEUP ? act(P, l, P.off_x_mid)
                                          : act(P, P.L - 1, P.off_x_out);
        const float* gain = ty == T_QKV ? P.lw[l].attn_norm
                          : ty == T_GATEUP ? P.lw[l].mlp_norm
                          : ty == T_LM ? P.final_norm
                                       : nullptr;
        ctl_input<WT, KH, true>(P, src, gain, b, sm, lane);
      }
      xkey = P.B > 1 ? -1 : key;
    }
  } else if (is_attn(T.type)) {
    ctl_attn_in<WT>(P, T, sm, lane, b == 0);
    xkey = -1;  // the K/V chunk overlays the activation row
  }
  return e;
}

template <typename WT, int CPR_H, int CPR_F, bool WIDE, int KMAX, bool LOG = false>
__device__ __forceinline__ void ctl_post(const Params& P, const Tile& T, int b, Smem<WT, KMAX>& sm, const EpiIn& e,
                                         int lane, int& xkey, uint64_t* tw = nullptr) {
  if constexpr (WIDE) {
    switch (T.type) {
      case T_QKV:
      case T_OPROJ:
      case T_GATEUP:
      case T_DOWN:
      case T_LM:
        if (ctl_wide_post<WT, KMAX, LOG>(P, T, sm, lane, tw)) xkey = -1;  // the reduction used the operand area
        break;
      case T_ARGMAX: ctl_argmax<WT>(P, sm, lane); break;  // attention: merged by the caller
      case T_NORM: ctl_norm<WT>(P, T, sm, lane); break;
      default: break;
    }
    return;
  }
  switch (T.type) {
    case T_DOWN: ctl_gemv_out<WT, CPR_F>(P, T, b, sm, e, lane); break;
    case T_QKV:
    case T_OPROJ:
    case T_GATEUP:
    case T_LM: ctl_gemv_out<WT, CPR_H>(P, T, b, sm, e, lane); break;
    case T_ATTN: ctl_attn_out<WT>(P, T, sm, lane); break;
    case T_ARGMAX: ctl_argmax<WT>(P, sm, lane); break;
    default: break;
  }
}

// The control wave waits until the tile's counter group is complete for this
// step.  Bounded: past the watchdog budget it latches WPK_E_TIMEOUT naming the
// tile and raises the abort flag, which every other waiting worker also sees.
template <bool WIDE>
__device__ __forceinline__ bool wait_group(const Params& P, const Tile& T, uint32_t epoch, int32_t* delta,
                                           int lane) {
  const Group G = cload(P.groups, T.wait);
  const uint32_t target = (epoch + 1u) * (uint32_t)G.producers;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (uint32_t n = 0;; ++n) {
    const uint32_t v0 = lane < G.shards ? ld_sc1(&P.counters[(size_t)(G.shard0 + lane) * kLine]) : 0u;
    const uint32_t v1 = lane + 64 < G.shards ? ld_sc1(&P.counters[(size_t)(G.shard0 + lane + 64) * kLine]) : 0u;
    const uint32_t sum = wave_sum_u32(v0 + v1);  // G.shards <= kMaxShards = 128
    if ((int32_t)(sum - target) >= 0) {
      *delta = (int32_t)(sum - target);
      compiler_order();  // the tile's input loads stay after the poll that saw them complete
      return true;
    }
    // Narrow plans read the abort flag every 16th poll: a round trip per poll
    // to one line that every waiting worker reads halves the poll rate (1.2%
    // of a batch-1 step).  Wide plans read it every poll: their faster polls
    // add more load than they save (+2% at batch 32).
    if ((WIDE || (n & 15u) == 15u) && ld_sc1(&P.ctl[CTL_ABORT])) return false;
    if (__builtin_amdgcn_s_memrealtime() - t0 > P.watchdog_ticks) {
      if (lane == 0) latch_error(P, WPK_E_TIMEOUT, T.id);
      return false;
    }
    __builtin_amdgcn_s_sleep(WIDE ? 1 : 2);
  }
}

__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16; x *= 0x7FEB352Du; x ^= x >> 15; x *= 0x846CA68Bu; x ^= x >> 16;
  return x;
}

// ============================ the worker loops ================================================

// Barrier C (the tile is published before the compute waves stage the next
// one) is skipped after LM-head tiles and wide tiles, whose epilogues may then
// queue behind the next weights.  A wide tile's control wave reuses the
// operand LDS area for the slice sums, so C stays when the next tile is an
// attention tile (its compute waves fill that area before barrier A).
template <bool WIDE>
__device__ __forceinline__ bool need_c(const Tile& T, int next_type) {
  // a wide plan's attention tile followed by another: the next tile's K/V
  // chunks stream into the slot (and its first chunk into the K/V rows of the
  // LDS) while the control wave merges the last pass and stores the partial,
  // which read only the pass outputs and registers (-0.7% at batch 32)
  if (WIDE && T.type == T_ATTN && next_type == T_ATTN) return false;
  if (!(T.type == T_LM || (WIDE && is_gemv(T.type)))) return true;
  if (!WIDE || next_type < 0) return false;
  return is_attn(next_type);
}

// Wide plans: compute wave 1, which claims the next tile, loads its descriptor
// while its weights stream in and leaves it in LDS before barrier A, so that
// after barrier B the compute waves stage the next weights without a
// scalar-cache miss in between.  (Narrow plans load it in each role: there
// the wait for wave 1 at barrier A would lie on the critical path, and the
// control wave's load hides behind its poll for the tile's inputs.)
__device__ __forceinline__ void put_tile(int* dst, const Tile& T, int lane) {
  int32_t w[16];
  __builtin_memcpy(w, &T, sizeof(Tile));
  int v = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) v = lane == k ? w[k] : v;
  if (lane < 16) dst[lane] = v;
}
__device__ __forceinline__ Tile get_tile(const int* src) {
  int32_t w[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) w[k] = __builtin_amdgcn_readfirstlane(src[k]);
  Tile T;
  __builtin_memcpy(&T, w, sizeof(Tile));
  return T;
}

// Publishes a worker's run of LM-head tiles at once: their logits stores and
// argmax updates have completed, then one increment by the run's length (the
// group counts its total over all shards, so any shard serves).
__device__ __forceinline__ void flush_lm(const Params& P, int group, int& count, int lane) {
  wait_all_memory();
  if (lane == 0) {
    const Group G = cload(P.groups, group);
    atomic_add(&P.counters[(size_t)(G.shard0 + (int)blockIdx.x % G.shards) * kLine], (uint32_t)count);
  }
  count = 0;
}

template <typename WT, int CPR_H, int CPR_F, bool LOG, bool WIDE, int KMAX>
__device__ __forceinline__ void control_loop(const Params& P, Smem<WT, KMAX>& sm, int cur, int qb, int qn,
                                             uint32_t epoch, int lane0) {
  int it = 0;
  int done_group = -1;  // a group already seen complete this step (groups never un-complete)
  int xkey = -1;        // which activation row sm.xs holds
  // LM-head tiles feed only the final argmax: a worker publishes its run of
  // them with one wait and one increment when the run ends
  int lm_group = -1, lm_count = 0;
  // the control wave's polls and publishes go ahead of the compute waves'
  // weight loads in the CU's instruction arbitration
  __builtin_amdgcn_s_setprio(3);
  while (cur < qn) {
    // lane index made opaque per tile, so per-lane address arithmetic of all
    // tile types is not hoisted out of the loop and kept live across it
    const int lane = opaque(lane0);
    const uint64_t t_claim = LOG ? __builtin_amdgcn_s_memrealtime() : 0;
    // the descriptor: loaded at the end of the previous iteration (narrow
    // plans) or by compute wave 1 (wide plans), and left in LDS
    const Tile T = it ? get_tile(sm.tnext[WIDE ? it & 1 : 0]) : cload(P.qtiles, qb + cur);
    const int id = T.id;
    if (lm_count && T.type != T_LM) flush_lm(P, lm_group, lm_count, lane);
    int32_t delta = 0;
    bool ok = true;
    // an attention chunk past its sequence reads and writes nothing (its
    // combine never reads it): it only publishes, without waiting, except in
    // logged steps, which check that every tile starts after its producers
    const bool idle = is_attn(T.type) && attn_count(P, T, sm.pos[T.b]) == 0;
    if (T.wait >= 0 && (LOG || (T.wait != done_group && !idle))) {
      ok = wait_group<WIDE>(P, T, epoch, &delta, lane);
      if (ok) done_group = T.wait;
    }
    if (lane == 0) sm.stop = ok ? 0 : 1;
    if (!P.prefetch) __syncthreads();  // W: the compute waves may load the weights now
    if (!ok) {
      __syncthreads();  // A
      __syncthreads();  // B
      break;
    }
    if (P.perturb)
      for (uint32_t k = hash32((uint32_t)id ^ P.perturb) & 31u; k; --k) __builtin_amdgcn_s_sleep(8);
    const uint64_t t_start = LOG ? __builtin_amdgcn_s_memrealtime() : 0;
    const int npairs = n_passes<WIDE>(P, T, sm.pos[T.b]);
    uint64_t t_inputs = 0, t_partials = 0, t_ready = 0, t_done = 0;
    uint64_t tw[2] = {0, 0};  // logged matrix-core GEMM tiles: partials stored, arrival counted
    AttnRun run;
    attn_run_init(run);
    for (int b = 0; b < npairs; ++b) {
      // an attention tile's passes are its KV chunks
      const Tile Tb = is_attn(T.type) ? sub_chunk(T, b) : T;
      const EpiIn e = ctl_pre<WT, CPR_H, CPR_F, WIDE>(P, Tb, b, sm, lane, xkey);
      if (LOG) {
        t_inputs = __builtin_amdgcn_s_memrealtime();
        if (lane == 0) sm.t_ready = sm.t_done = 0;
      }
      __syncthreads();  // A: inputs staged
      __syncthreads();  // B: partial sums ready
      if (LOG) {
        t_partials = __builtin_amdgcn_s_memrealtime();
        t_ready = sm.t_ready;
        t_done = sm.t_done;
      }
      ctl_post<WT, CPR_H, CPR_F, WIDE, KMAX, LOG>(P, Tb, b, sm, e, lane, xkey, tw);
      if (WIDE && is_attn(T.type) && attn_count(P, Tb, sm.pos[T.b]) > 0) attn_run_merge(P, run, sm, lane);
    }
    if (WIDE && T.type == T_ATTN) attn_run_partial(P, T, run, sm, lane);
    if (WIDE && T.type == T_ATTNC) attn_run_store<WIDE>(P, T, run, attn_active(P, sm.pos[T.b]), lane);
    // publish: this wave made every global store of the tile; once they have
    // completed, one relaxed device-scope increment of the tile's counter shard
    const bool batch = T.type == T_LM && T.signal >= 0;
    if (batch) {
      lm_group = T.signal;
      lm_count += id != P.drop_tile;
    } else {
      wait_all_memory();
    }
    if (lane == 0) {
      if (LOG) {
        int32_t* rec = P.log + (size_t)id * 8;
        __hip_atomic_fetch_add(rec, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        rec[1] = delta;
        rec[2] = (int32_t)blockIdx.x;
        rec[3] = cur;
        const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
        *(uint64_t*)(rec + 4) = t_start;
        *(uint64_t*)(rec + 6) = t_end;
        uint64_t* tm = (uint64_t*)(P.log + ((size_t)P.n_tiles + P.log_workers) * 8) + (size_t)id * 8;
        tm[0] = t_claim;
        tm[1] = t_inputs;
        tm[2] = t_ready;
        tm[3] = t_done;
        tm[4] = t_partials;
        tm[5] = t_end;
        tm[6] = tw[0];
        tm[7] = tw[1];
      }
      if (!batch && T.signal >= 0 && id != P.drop_tile) {
        const Group G = cload(P.groups, T.signal);
        atomic_add(&P.counters[(size_t)(G.shard0 + T.shard) * kLine], 1u);
      }
    }
    // C: published; the compute waves may load the next tile.  LM-head tiles
    // skip it: only the final argmax depends on them, so their epilogue may
    // queue behind the next weights, which then stream without a gap.  The
    // next claim was written by compute wave 1 before this tile's barrier B.
    const int nxt = __builtin_amdgcn_readfirstlane(sm.ids[(it + 1) & 1]);
    // narrow plans: the next descriptor, fetched after the publish (so the
    // scalar-cache miss delays neither the publish nor the next poll) and
    // left in LDS for this wave and, past barrier C, the compute waves
    if (!WIDE && nxt < qn) put_tile(sm.tnext[0], cload(P.qtiles, qb + nxt), lane);
    if (need_c<WIDE>(T, WIDE && nxt < qn ? __builtin_amdgcn_readfirstlane(sm.tnext[(it + 1) & 1][0]) : -1))
      __syncthreads();
    cur = nxt;
    ++it;
  }
  if (lm_count) flush_lm(P, lm_group, lm_count, lane0);
}

// Redefines the slot in place (no copy), once per batch row: the unpacked
// weights then depend on the row and are not hoisted out of the batch loop,
// where they would need twice the slot's registers.
__device__ __forceinline__ void launder(Slot& s) {
  asm volatile("" : "+v"(s.c[0]), "+v"(s.c[1]), "+v"(s.c[2]), "+v"(s.c[3]), "+v"(s.c[4]), "+v"(s.c[5]),
               "+v"(s.c[6]), "+v"(s.c[7]));
  asm volatile("" : "+v"(s.c[8]), "+v"(s.c[9]), "+v"(s.c[10]), "+v"(s.c[11]), "+v"(s.c[12]), "+v"(s.c[13]),
               "+v"(s.c[14]), "+v"(s.c[15]));
}

template <typename WT, int CPR_H, int CPR_F, bool LOG, bool WIDE, int KMAX>
__device__ __forceinline__ void compute_loop(const Params& P, Smem<WT, KMAX>& sm, int cur, int qb, int qn,
                                             uint32_t* head, int tc0) {
  const uint32_t voff = (uint32_t)tc0 * 16u;
  Slot s;
#pragma unroll
  for (int j = 0; j < kChunks; ++j) s.c[j] = u32x4{0u, 0u, 0u, 0u};
  int it = -1;  // claim iteration of the current tile
  int nx = cur;
  bool c_taken = false;  // the previous tile ended with barrier C
  while (nx < qn) {
    // The slot is free (the previous tile's arithmetic is done and its
    // barrier B passed, so the control wave is already running that tile's
    // epilogue): stage this tile's weights; they stream in while the control
    // wave publishes, claims, waits for the tile's inputs and stages them.
    // Claim the next tile here rather than in the control wave: a wave's
    // memory operations complete in issue order, so an atomic (slow while the
    // weights stream) would hold up every later wait of the control wave,
    // while here it returns ahead of the weights this wave waits for anyway.
    // wide plans: from LDS (compute wave 1 fetched it); narrow plans: from
    // LDS after barrier C (the control wave fetched it), else loaded here
    const Tile T = it >= 0 && (WIDE || c_taken) ? get_tile(sm.tnext[WIDE ? (it + 1) & 1 : 0])
                                                : cload(P.qtiles, qb + nx);
    uint32_t ahead = 0;
    if (tc0 == 0) ahead = atomic_add(head, 1u);
    // without weight prefetch (an ablation), the weights are loaded only once
    // the control wave has seen the tile's inputs complete (barrier W)
    if (!P.prefetch) __syncthreads();  // W
    const int valid = attn_valid(P, sm.pos[T.b]);
    if (WIDE && is_gemv(T.type)) stage_wide(P, T, s, tc0);
    else stage<WT, CPR_H, CPR_F>(P, WIDE && T.type == T_ATTNC ? attn_group<WT>(T, 0) : T, s, voff, valid);
    ++it;
    if (WIDE && tc0 < 64) {
      // the next claim and its descriptor, read by every wave after barrier
      // A (double-buffered by iteration parity: the current tile's copy may
      // still be being read)
      const int nxt = __builtin_amdgcn_readfirstlane((int)ahead);
      if (tc0 == 0) sm.ids[(it + 1) & 1] = nxt;
      if (nxt < qn) put_tile(sm.tnext[(it + 1) & 1], cload(P.qtiles, qb + nxt), tc0);
    }
    const int tc = opaque(tc0);
    const int npairs = n_passes<WIDE>(P, T, sm.pos[T.b]);
    bool stop = false;
    for (int b = 0; b < npairs; ++b) {
      const Tile Tb = is_attn(T.type) ? sub_chunk(T, b) : T;
      if (is_attn(T.type)) {
        // the next KV chunk: already in the slot, or (chained tiles) the
        // slot's next fill
        if (b > 0) {
          if (WIDE && T.type == T_ATTNC && b % (kChunks / kv_chunks<WT>()) == 0)
            stage<WT, CPR_H, CPR_F>(P, attn_group<WT>(T, b), s, voff, valid);
          else
            slot_shift<WT>(s);
        }
        if (attn_count(P, Tb, sm.pos[T.b]) > 0) dump_kv<WT>(P, Tb, s, sm, tc);
      }
      __syncthreads();  // A
      if (__builtin_amdgcn_readfirstlane(sm.stop)) {
        __syncthreads();  // B
        stop = true;
        break;
      }
      if (LOG) {  // timing only: the slot's loads are complete here (latest compute wave)
        wait_all_memory();
        if ((tc & 63) == 0)
          __hip_atomic_fetch_max(&sm.t_ready, (uint64_t)__builtin_amdgcn_s_memrealtime(), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      if (!WIDE && b == 0 && tc == 0) sm.ids[(it + 1) & 1] = (int)ahead;  // read after B
      launder(s);
      compute<WT, CPR_H, CPR_F, WIDE>(P, Tb, s, sm, tc);
      if (LOG && (tc & 63) == 0)
        __hip_atomic_fetch_max(&sm.t_done, (uint64_t)__builtin_amdgcn_s_memrealtime(), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
      __syncthreads();  // B
    }
    if (stop) break;
    // Keep the next tile's loads after this tile's arithmetic: hoisting them
    // above it would keep two slots live.
    __builtin_amdgcn_sched_barrier(0);
    nx = __builtin_amdgcn_readfirstlane(sm.ids[(it + 1) & 1]);
    c_taken = need_c<WIDE>(T, WIDE && nx < qn ? __builtin_amdgcn_readfirstlane(sm.tnext[(it + 1) & 1][0]) : -1);
    if (c_taken) __syncthreads();  // C
  }
}

template <int CPR_H, int CPR_F, typename WT>
constexpr int kmax() {
  return (CPR_H > CPR_F ? CPR_H : CPR_F) * 16 / (int)sizeof(WT);
}

// Step start: sequence positions and tokens (both fixed until the step's last
// tile), the worker's first claim.
template <typename WT, int KMAX>
__device__ __forceinline__ void step_start(const Params& P, Smem<WT, KMAX>& sm, int lane, int first) {
  if (lane < P.B) {
    const int32_t p = ld_sc1(&P.seq_len[lane]);
    int32_t tk = ld_sc1(&P.tokens[lane]);
    if (tk < 0 || tk >= P.V) {
      if (p >= 0) latch_error(P, WPK_E_TOKEN, -1);
      tk = 0;
    }
    sm.pos[lane] = p;
    sm.tok[lane] = tk;
  }
  if (lane == 0) {
    sm.first = first;
    sm.stop = 0;
  }
}

// The worker loop: claim (from this worker's queue, in topological order),
// stage the tile's weights, wait for its counter group, run it, publish.
// Wide instances take their LDS (about 77 KiB: the operand slice and the
// partial sums) as dynamic shared memory: two workers still fit a CU's 160 KiB,
// and the compiler, which only sees static LDS, keeps the register budget of
// four waves per SIMD.
template <typename WT, int CPR_H, int CPR_F, bool WIDE>
struct Lds {
  static constexpr int KMAX = WIDE ? kWideKmax : kmax<CPR_H, CPR_F, WT>();
  using type = Smem<WT, KMAX>;
};

}  // namespace wpk
