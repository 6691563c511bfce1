// megakernel.hip -- the decode step as one persistent kernel on gfx950.
//
// Structure (what the pages describe, re-designed for MI355X):
//  * A megakernel owns the multi-operation program and the coordination between
//    operations ("Why real-time inference wants a megakernel", "The unit of
//    execution"); the host launches once per step and the GPU walks the schedule:
//    wait for the dependencies, run, signal the consumers (section "What the
//    megakernel changes").
//  * Workers are resident workgroups, several per CU, all co-resident
//    (cooperative launch), that claim tiles from device-side queues in a
//    topological order.  Each worker has one staging slot: the claimed tile's
//    weights are loaded into it before the tile's dependency counter is
//    checked, so weight streaming continues while predecessors finish
//    ("One Megakernel is Not Enough", Table I, weight prefetch; the Llama-1B
//    megakernel of "persistent-threads-megakernels", section 6, starts weight
//    loads for upcoming work early).
//  * Dependencies are counter groups (tile-to-tile tensor edges, Table I), not
//    operator barriers.
//
// gfx950 specifics, measured with microbench.hip on an MI355X:
//  * An agent-scope acquire fence (L2 invalidate) per 64 KiB tile cut streaming
//    reads from 6.2 to 2.2 TB/s and a release fence (L2 write-back) to 1.2 TB/s,
//    because each of the 8 XCDs has its own L2.  The kernel therefore uses no
//    fences in its hot path: tile outputs are written with device-coherent
//    (sc1, write-through) stores and a wait for their completion, counters are
//    bumped with relaxed device-scope atomics (performed past the L2s), and
//    consumers read counters and activations with device-coherent (sc1) loads.
//    A cross-XCD message-passing test of exactly this protocol saw no stale
//    word in 2000 x 8 rounds; plain stores in its place were stale.
//  * One address takes ~88 M atomics/s, so each counter group is spread over up
//    to 16 shards and tiles are claimed from 8 queues.
//  * Weights stream with 16-byte non-temporal loads, 16 per thread, so a worker
//    keeps a whole 64 KiB tile in flight.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.h"
#include "wpk.h"

namespace wpk {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct Slot {
  u32x4 c[kChunks];
};

template <typename WT>
struct WT_ {
  static constexpr int EPC = 16 / sizeof(WT);   // elements per 16-byte chunk
  static constexpr int PITCH = sizeof(WT) == 2 ? 66 : 65;  // LDS row pitch of a K/V chunk (conflict-free)
};

template <typename WT>
struct Smem {
  float red[kWaves][64];
  float yrow[64];
  float nrm[kWaves];
  float qs[kMaxGroupHeads][kHeadDim];
  float ps[kMaxGroupHeads][kAttnChunk];
  WT ks[kAttnChunk * WT_<WT>::PITCH];
  WT vs[kAttnChunk * WT_<WT>::PITCH];
  int next[2];
  int first;
  int ok;
  int delta;
};

// The thread index, made opaque to the optimiser.  Inside the persistent tile
// loop the compiler would otherwise hoist every tile type's per-lane address
// arithmetic out of the loop and keep it all live, which multiplies the
// register footprint of the merged kernel (the register-pressure cost of
// megakernels the persistent-threads page discusses in section 4).
__device__ __forceinline__ int wpk_tid() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

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

// Read-only tables (tiles, groups, queues) through the constant address space:
// uniform loads from it become scalar loads that do not count against the
// vector-memory counter the weight stream uses.
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

__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Elements of one 16-byte chunk as floats.
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
__device__ __forceinline__ float dot_chunk(u32x4 c, const float* x, float acc) {
  float w[WT_<WT>::EPC];
  unpack<WT>(c, w);
#pragma unroll
  for (int e = 0; e < WT_<WT>::EPC; ++e) acc = fmaf(w[e], x[e], acc);
  return acc;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += (uint32_t)__shfl_xor((int)v, m);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// Sum over all threads of the worker; every thread gets the result.
template <typename WT>
__device__ __forceinline__ float block_sum(float v, Smem<WT>& sm) {
  v = wave_sum(v);
  const int t = wpk_tid();
  if ((t & 63) == 0) sm.nrm[t >> 6] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) s += sm.nrm[w];
  __syncthreads();
  return s;
}

// Reduce-scatter of N per-lane values over the 64 lanes of a wave: after it,
// lane l holds the wave-wide sum of value index scatter_index<N>(l).
template <int N>
__device__ __forceinline__ float wave_reduce_scatter(float (&v)[N], int lane) {
#pragma unroll
  for (int s = 0, n = N; n > 1; ++s, n >>= 1) {
    const int m = 1 << s;
    const bool up = (lane & m) != 0;
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
      const float send = up ? v[i] : v[i + n / 2];
      const float keep = up ? v[i + n / 2] : v[i];
      v[i] = keep + __shfl_xor(send, m);
    }
  }
  float r = v[0];
#pragma unroll
  for (int m = N; m < 64; m <<= 1) r += __shfl_xor(r, m);
  return r;
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

// ---- GEMV tiles ----------------------------------------------------------------------------
//
// A GEMV tile is `rows` weight rows (two segments, so RoPE pairs (i, i+D/2) and
// gate/up pairs land in one tile) of a matrix with K columns, CPR 16-byte
// chunks per row.  Thread t owns chunk j*256 + t of the tile for j < 16, so
// each of its 16 loads is one fully coalesced 4 KiB wavefront-set of the tile.

template <int CPR>
struct Geo {
  static constexpr int LPR = CPR >= kThreads ? CPR / kThreads : 1;  // chunks of one row per thread
  static constexpr int NV = kChunks / LPR;                          // rows a thread contributes to
  static constexpr int ROWS = kThreads * kChunks / CPR;             // rows of a full tile
  static constexpr int WPR = CPR >= kThreads ? kWaves : CPR / 64;   // waves sharing a row
  static_assert(CPR >= 64 && ROWS <= 64, "unsupported row length");
};

template <int CPR>
__device__ __forceinline__ void stage_gemv(const void* w0, const void* w1, int r0, int r1, int rs, int rows,
                                           int limit, Slot& s) {
  const int t = wpk_tid();
#pragma unroll
  for (int j = 0; j < kChunks; ++j) {
    // Rows past the tile or the matrix are clamped to a valid row, so every
    // load is unconditional; their (duplicate) sums are never stored.
    const int flat = j * kThreads + t;
    const int row = min(flat / CPR, rows - 1);
    const int col = flat % CPR;
    const bool seg1 = row >= rs;
    const int mrow = min(seg1 ? r1 + (row - rs) : r0 + row, limit - 1);
    const char* base = (const char*)(seg1 ? w1 : w0);
    s.c[j] = ld_nt(base + (size_t)mrow * (CPR * 16) + (size_t)col * 16);
  }
}

// This thread's activations for sequence b (the columns of its chunks), with
// the RMSNorm prologue for the operators that have one.
template <typename WT, int CPR>
__device__ __forceinline__ void gemv_input(const Params& P, const Tile& T, int b, int tok,
                                           float (&x)[Geo<CPR>::LPR * WT_<WT>::EPC], Smem<WT>& sm) {
  constexpr int EPC = WT_<WT>::EPC, LPR = Geo<CPR>::LPR;
  const int t = wpk_tid();
  const LayerW& lw = P.lw[T.layer];
  const float* src = nullptr;
  const float* gain = nullptr;
  int K = P.H;
  switch (T.type) {
    case T_QKV: src = x_in(P, T.layer); gain = lw.attn_norm; break;
    case T_OPROJ: src = act(P, T.layer, P.off_attn); break;
    case T_GATEUP: src = act(P, T.layer, P.off_x_mid); gain = lw.mlp_norm; break;
    case T_DOWN: src = act(P, T.layer, P.off_h); K = P.F; break;
    default: src = act(P, P.L - 1, P.off_x_out); gain = P.final_norm; break;
  }
#pragma unroll
  for (int k = 0; k < LPR; ++k) {
    const int col = CPR >= kThreads ? k * kThreads + t : t % CPR;
    if (src == nullptr) {  // layer-0 input: the embedding row of the token (input conversion)
      const u32x4 c = *(const u32x4*)((const char*)P.embed + ((size_t)tok * P.H * sizeof(WT)) + (size_t)col * 16);
      unpack<WT>(c, &x[k * EPC]);
    } else {
#pragma unroll
      for (int e = 0; e < EPC; e += 4) {
        const u32x4 c = ld_sc1_x4(src, b * K + col * EPC + e);
        x[k * EPC + e + 0] = __uint_as_float(c.x);
        x[k * EPC + e + 1] = __uint_as_float(c.y);
        x[k * EPC + e + 2] = __uint_as_float(c.z);
        x[k * EPC + e + 3] = __uint_as_float(c.w);
      }
    }
  }
  if (gain) {
    float ss = 0.f;
    if (CPR >= kThreads || t < CPR) {
#pragma unroll
      for (int i = 0; i < LPR * EPC; ++i) ss = fmaf(x[i], x[i], ss);
    }
    ss = block_sum(ss, sm);
    const float inv = 1.0f / sqrtf(ss / (float)K + P.eps);
#pragma unroll
    for (int k = 0; k < LPR; ++k) {
      const int col = CPR >= kThreads ? k * kThreads + t : t % CPR;
#pragma unroll
      for (int e = 0; e < EPC; ++e) x[k * EPC + e] = x[k * EPC + e] * inv * gain[col * EPC + e];
    }
  }
}

// Row sums of the tile for the thread's activations, into sm.yrow[0 .. ROWS).
template <typename WT, int CPR>
__device__ __forceinline__ void gemv_rows(const Slot& s, const float (&x)[Geo<CPR>::LPR * WT_<WT>::EPC],
                                          Smem<WT>& sm) {
  using G = Geo<CPR>;
  constexpr int EPC = WT_<WT>::EPC;
  const int t = wpk_tid(), lane = t & 63, wave = t >> 6;
  float acc[G::NV];
#pragma unroll
  for (int v = 0; v < G::NV; ++v) acc[v] = 0.f;
#pragma unroll
  for (int j = 0; j < kChunks; ++j) {
    // Opaque copy: keeps the compiler from hoisting the unpacked (2x wider)
    // weights out of the caller's batch loop, which would double the slot's
    // register footprint.
    u32x4 c = s.c[j];
    asm volatile("" : "+v"(c));
    acc[j / G::LPR] = dot_chunk<WT>(c, &x[(j % G::LPR) * EPC], acc[j / G::LPR]);
  }
  const float r = wave_reduce_scatter<G::NV>(acc, lane);
  if (lane < G::NV) sm.red[wave][scatter_index<G::NV>(lane)] = r;
  __syncthreads();
  if (t < G::ROWS) {
    float y = 0.f;
    if (CPR >= kThreads) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) y += sm.red[w][t];
    } else {
      constexpr int S = kThreads / CPR;  // rows interleaved per value index
      const int v = t / S, grp = t % S;
#pragma unroll
      for (int w = 0; w < G::WPR; ++w) y += sm.red[grp * G::WPR + w][v];
    }
    sm.yrow[t] = y;
  }
  __syncthreads();
}

__device__ __forceinline__ unsigned long long pack_max(float v, int idx) {
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)idx);
}

template <typename WT, int CPR>
__device__ __forceinline__ void gemv_tile(const Params& P, const Tile& T, const Slot& s, Smem<WT>& sm) {
  using G = Geo<CPR>;
  const int t = wpk_tid();
  const int l = T.layer;
  for (int b = 0; b < P.B; ++b) {
    const int32_t p = ld_sc1(&P.seq_len[b]);
    if (T.type == T_QKV && p < 0) continue;  // inactive slot: nothing to append
    int tok = 0;
    if (T.layer == 0 && (T.type == T_QKV || T.type == T_OPROJ)) {
      tok = P.tokens[b];
      if (tok < 0 || tok >= P.V) {
        if (p >= 0 && t == 0) latch_error(P, WPK_E_TOKEN, T.id);
        tok = 0;
      }
    }
    float x[G::LPR * WT_<WT>::EPC];
    gemv_input<WT, CPR>(P, T, b, tok, x, sm);
    gemv_rows<WT, CPR>(s, x, sm);
    const float* y = sm.yrow;
    switch (T.type) {
      case T_QKV: {
        if (p >= P.cap) {
          if (t == 0) latch_error(P, WPK_E_CTX_FULL, T.id);
          break;
        }
        const int half = P.D / 2;
        if (T.kind < 2) {
          const int head = T.g;
          const int base = T.kind == 0 ? head * P.D : (P.Hq + head) * P.D;
          if (t < T.rs) {
            const int dim = T.r0 + t - base;
            const float cs = P.rope_cos[p * half + dim], sn = P.rope_sin[p * half + dim];
            const float a = y[t], bb = y[T.rs + t];
            const float ra = a * cs - bb * sn, rb = bb * cs + a * sn;
            if (T.kind == 0) {
              float* q = act(P, l, P.off_q) + (size_t)b * P.Hq * P.D + head * P.D;
              st_sc1(q + dim, ra);
              st_sc1(q + dim + half, rb);
            } else {
              const size_t at = ((((size_t)T.layer * P.B + b) * P.Hkv + head) * P.cap + p) * P.D;
              WT* kc = (WT*)P.kc + at;
              if (sizeof(WT) == 2) {
                st_sc1((uint16_t*)kc + dim, to_bf16(ra));
                st_sc1((uint16_t*)kc + dim + half, to_bf16(rb));
              } else {
                st_sc1((float*)kc + dim, ra);
                st_sc1((float*)kc + dim + half, rb);
              }
            }
          }
        } else if (t < T.rows) {
          const int base = (P.Hq + P.Hkv + T.g) * P.D;
          const int mrow = t < T.rs ? T.r0 + t : T.r1 + (t - T.rs);
          const size_t at = ((((size_t)T.layer * P.B + b) * P.Hkv + T.g) * P.cap + p) * P.D + (mrow - base);
          if (sizeof(WT) == 2) st_sc1((uint16_t*)P.vc + at, to_bf16(y[t]));
          else st_sc1((float*)P.vc + at, y[t]);
        }
        break;
      }
      case T_OPROJ:
        if (t < T.rows && T.r0 + t < P.H) {
          const int row = T.r0 + t;
          float xin;
          if (T.layer == 0) {
            const WT* e = (const WT*)P.embed + (size_t)tok * P.H + row;
            xin = sizeof(WT) == 2 ? bf16_lo(*(const uint16_t*)e) : *(const float*)e;
          } else {
            xin = ld_sc1(x_in(P, l) + (size_t)b * P.H + row);
          }
          st_sc1(act(P, l, P.off_x_mid) + (size_t)b * P.H + row, xin + y[t]);
        }
        break;
      case T_GATEUP:
        if (t < T.rs && T.r0 + t < P.F) {
          const float g = y[t], u = y[T.rs + t];
          st_sc1(act(P, l, P.off_h) + (size_t)b * P.F + T.r0 + t, g / (1.0f + __expf(-g)) * u);
        }
        break;
      case T_DOWN:
        if (t < T.rows && T.r0 + t < P.H) {
          const int row = T.r0 + t;
          st_sc1(act(P, l, P.off_x_out) + (size_t)b * P.H + row, ld_sc1(act(P, l, P.off_x_mid) + (size_t)b * P.H + row) + y[t]);
        }
        break;
      case T_LM:
        if (t < 64) {
          const int row = T.r0 + t;
          unsigned long long key = 0;
          if (t < T.rows && row < P.V) {
            P.logits[(size_t)b * P.V + row] = y[t];
            key = pack_max(y[t], row);
          }
#pragma unroll
          for (int m = 1; m < 64; m <<= 1) {
            const unsigned long long o = __shfl_xor(key, m);
            key = o > key ? o : key;
          }
          if (t == 0)
            __hip_atomic_fetch_max(&P.argmax[b * kArgmaxShards + T.id % kArgmaxShards], key, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        break;
    }
    __syncthreads();
  }
}

// ---- attention ---------------------------------------------------------------------------
//
// Split-KV decode attention (the chunked KV of FlashInfer's persistent kernel and
// the partial + reduction tasks of ThunderMLA, "persistent-threads-megakernels"
// section 6): one tile handles 64 cached positions of one (sequence, kv head)
// for all the q heads of its group; the K/V chunk is the tile's staged "weights".

template <typename WT>
__device__ __forceinline__ void stage_attn(const Params& P, const Tile& T, Slot& s) {
  constexpr int CPP = kHeadDim * sizeof(WT) / 16;  // chunks per position
  constexpr int KCH = kAttnChunk * CPP;            // chunks of K (and of V) per tile
  const int t = wpk_tid();
  const size_t slice = (((size_t)T.layer * P.B + T.b) * P.Hkv + T.g) * P.cap;
  const int start = T.c * kAttnChunk;
#pragma unroll
  for (int j = 0; j < 2 * KCH / kThreads; ++j) {
    const int flat = j * kThreads + t;
    const bool isv = flat >= KCH;
    const int f = isv ? flat - KCH : flat;
    const int pos = min(start + f / CPP, P.cap - 1);  // positions past the capacity are never used
    const int dc = f % CPP;
    s.c[j] = ld_nt((isv ? P.vc : P.kc) + ((slice + pos) * kHeadDim) * sizeof(WT) + (size_t)dc * 16);
  }
  // Define the whole slot on every path: with entries left undefined here the
  // optimiser can no longer keep the slot in registers and spills it to
  // scratch, serialising the weight loads.
#pragma unroll
  for (int j = 2 * KCH / kThreads; j < kChunks; ++j) s.c[j] = u32x4{0u, 0u, 0u, 0u};
}

template <typename WT>
__device__ __forceinline__ float lds_elt(const WT* a, int i) {
  if (sizeof(WT) == 2) return bf16_lo(((const uint16_t*)a)[i]);
  return ((const float*)a)[i];
}

template <typename WT>
__device__ __forceinline__ void attn_tile(const Params& P, const Tile& T, const Slot& s, Smem<WT>& sm) {
  constexpr int CPP = kHeadDim * sizeof(WT) / 16, KCH = kAttnChunk * CPP, EPC = WT_<WT>::EPC;
  constexpr int PITCH = WT_<WT>::PITCH;
  const int t = wpk_tid(), lane = t & 63, wave = t >> 6;
  const int32_t p = ld_sc1(&P.seq_len[T.b]);
  const int n = p < 0 ? 0 : min(p + 1, P.cap);
  const int start = T.c * kAttnChunk;
  const int cnt = max(0, min(kAttnChunk, n - start));
  float* out = act(P, T.layer, P.off_part) + ((((size_t)T.b * P.Hkv + T.g) * P.nch + T.c) * P.G) * (P.D + 2);
  if (cnt == 0) {
    if (wave < P.G) {
      float* o = out + wave * (P.D + 2);
      st_sc1(o + 2 + lane, 0.f);
      if (lane == 0) {
        st_sc1(o, -INFINITY);
        st_sc1(o + 1, 0.f);
      }
    }
    return;
  }
  // staged K/V chunk -> LDS, one row per position
#pragma unroll
  for (int j = 0; j < 2 * KCH / kThreads; ++j) {
    const int flat = j * kThreads + t;
    const bool isv = flat >= KCH;
    const int f = isv ? flat - KCH : flat;
    const int pos = f / CPP, dc = f % CPP;
    WT* dst = (isv ? sm.vs : sm.ks) + pos * PITCH + dc * EPC;
    if (sizeof(WT) == 2) {
      uint32_t* d32 = (uint32_t*)dst;  // row pitch 132 B keeps 4-byte alignment
      d32[0] = s.c[j].x; d32[1] = s.c[j].y; d32[2] = s.c[j].z; d32[3] = s.c[j].w;
    } else {
      float* d = (float*)dst;
      d[0] = __uint_as_float(s.c[j].x); d[1] = __uint_as_float(s.c[j].y);
      d[2] = __uint_as_float(s.c[j].z); d[3] = __uint_as_float(s.c[j].w);
    }
  }
  // queries of the group (written by this step's QKV tiles)
  if (wave < P.G)
    sm.qs[wave][lane] = ld_sc1(act(P, T.layer, P.off_q) + (size_t)T.b * P.Hq * P.D + (size_t)(T.g * P.G + wave) * P.D + lane);
  __syncthreads();
  // position p was appended by this step's QKV tiles after the chunk was staged
  if (p >= start && p < start + kAttnChunk && p < P.cap && t < 2 * kHeadDim) {
    const size_t at = ((((size_t)T.layer * P.B + T.b) * P.Hkv + T.g) * P.cap + p) * kHeadDim;
    const bool isv = t >= kHeadDim;
    const int d = t & (kHeadDim - 1);
    WT* dst = (isv ? sm.vs : sm.ks) + (p - start) * PITCH + d;
    const WT* src = (const WT*)(isv ? P.vc : P.kc) + at + d;
    if (sizeof(WT) == 2) *(uint16_t*)dst = ld_sc1((const uint16_t*)src);
    else *(float*)dst = ld_sc1((const float*)src);
  }
  __syncthreads();
  // scores: wave h = q head, lane j = position
  float m = -INFINITY, l = 0.f;
  if (wave < P.G) {
    float sc = -INFINITY;
    if (lane < cnt) {
      float dot = 0.f;
      const WT* kr = sm.ks + lane * PITCH;
#pragma unroll 16
      for (int d = 0; d < kHeadDim; ++d) dot = fmaf(sm.qs[wave][d], lds_elt<WT>(kr, d), dot);
      sc = dot * P.attn_scale;
    }
    m = wave_max(sc);
    const float e = lane < cnt ? __expf(sc - m) : 0.f;
    l = wave_sum(e);
    sm.ps[wave][lane] = e;
  }
  __syncthreads();
  if (wave < P.G) {
    float o = 0.f;
    for (int j = 0; j < cnt; ++j) o = fmaf(sm.ps[wave][j], lds_elt<WT>(sm.vs + j * PITCH, lane), o);
    float* dst = out + wave * (P.D + 2);
    st_sc1(dst + 2 + lane, o);
    if (lane == 0) {
      st_sc1(dst, m);
      st_sc1(dst + 1, l);
    }
  }
}

template <typename WT>
__device__ __forceinline__ void combine_tile(const Params& P, const Tile& T) {
  const int t = wpk_tid(), lane = t & 63, wave = t >> 6;
  if (wave >= P.G) return;
  const int32_t p = ld_sc1(&P.seq_len[T.b]);
  const int n = p < 0 ? 0 : min(p + 1, P.cap);
  const int nact = (n + kAttnChunk - 1) / kAttnChunk;
  float* dst = act(P, T.layer, P.off_attn) + (size_t)T.b * P.Hq * P.D + (size_t)(T.g * P.G + wave) * P.D;
  const float* part = act(P, T.layer, P.off_part) + (((size_t)T.b * P.Hkv + T.g) * P.nch * P.G + wave) * (P.D + 2);
  const size_t stride = (size_t)P.G * (P.D + 2);
  if (nact == 0) {
    st_sc1(dst + lane, 0.f);
    return;
  }
  float M = -INFINITY;
  for (int c = 0; c < nact; ++c) M = fmaxf(M, ld_sc1(part + c * stride));
  float L = 0.f, o = 0.f;
  for (int c = 0; c < nact; ++c) {
    const float w = __expf(ld_sc1(part + c * stride) - M);
    L = fmaf(ld_sc1(part + c * stride + 1), w, L);
    o = fmaf(ld_sc1(part + c * stride + 2 + lane), w, o);
  }
  st_sc1(dst + lane, o / L);
}

// Output conversion: greedy token and sequence advance.
__device__ __forceinline__ void argmax_tile(const Params& P) {
  const int t = wpk_tid();
  if (t < P.B) {
    unsigned long long best = 0;
    for (int s = 0; s < kArgmaxShards; ++s) {
      unsigned long long* a = &P.argmax[t * kArgmaxShards + s];
      const unsigned long long v = __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      best = v > best ? v : best;
      __hip_atomic_store(a, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const int32_t p = ld_sc1(&P.seq_len[t]);
    if (p >= 0 && p < P.cap) {
      st_sc1(&P.tokens[t], (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull)));
      st_sc1(&P.seq_len[t], p + 1);
    }
  }
}

// ---- dispatch -------------------------------------------------------------------------------

template <typename WT, int CPR_H, int CPR_F>
__device__ __forceinline__ void stage(const Params& P, const Tile& T, Slot& s) {
  const LayerW& lw = P.lw[T.layer];
  switch (T.type) {
    case T_QKV: stage_gemv<CPR_H>(lw.w_qkv, lw.w_qkv, T.r0, T.r1, T.rs, T.rows, P.qkv_rows, s); break;
    case T_OPROJ: stage_gemv<CPR_H>(lw.w_o, lw.w_o, T.r0, T.r1, T.rs, T.rows, P.H, s); break;
    case T_GATEUP: stage_gemv<CPR_H>(lw.w_gate, lw.w_up, T.r0, T.r1, T.rs, T.rows, P.F, s); break;
    case T_DOWN: stage_gemv<CPR_F>(lw.w_down, lw.w_down, T.r0, T.r1, T.rs, T.rows, P.H, s); break;
    case T_LM: stage_gemv<CPR_H>(P.embed, P.embed, T.r0, T.r1, T.rs, T.rows, P.V, s); break;
    case T_ATTN: stage_attn<WT>(P, T, s); break;
    default: break;
  }
}

template <typename WT, int CPR_H, int CPR_F>
__device__ __forceinline__ void run_tile(const Params& P, const Tile& T, const Slot& s, Smem<WT>& sm) {
  switch (T.type) {
    case T_QKV:
    case T_OPROJ:
    case T_GATEUP:
    case T_LM: gemv_tile<WT, CPR_H>(P, T, s, sm); break;
    case T_DOWN: gemv_tile<WT, CPR_F>(P, T, s, sm); break;
    case T_ATTN: attn_tile<WT>(P, T, s, sm); break;
    case T_COMBINE: combine_tile<WT>(P, T); break;
    case T_ARGMAX: argmax_tile(P); break;
    default: break;
  }
}

// Wave 0 of a worker waits until the tile's counter group is complete for this
// step.  Bounded: past the watchdog budget it latches WPK_E_TIMEOUT naming the
// tile and raises the abort flag, which every other waiting worker also sees.
__device__ __forceinline__ bool wait_group(const Params& P, const Tile& T, uint32_t epoch, int32_t* delta) {
  const Group G = cload(P.groups, T.wait);
  const uint32_t target = (epoch + 1u) * (uint32_t)G.producers;
  const int lane = wpk_tid() & 63;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    const uint32_t v = lane < G.shards ? ld_sc1(&P.counters[(size_t)(G.shard0 + lane) * kLine]) : 0u;
    const uint32_t sum = wave_sum_u32(v);
    if ((int32_t)(sum - target) >= 0) {
      *delta = (int32_t)(sum - target);
      return true;
    }
    if (ld_sc1(&P.ctl[CTL_ABORT])) return false;
    if (__builtin_amdgcn_s_memrealtime() - t0 > P.watchdog_ticks) {
      if (lane == 0) latch_error(P, WPK_E_TIMEOUT, T.id);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16; x *= 0x7FEB352Du; x ^= x >> 15; x *= 0x846CA68Bu; x ^= x >> 16;
  return x;
}

// The worker loop: claim (from this worker's queue, in topological order),
// stage the tile's weights, wait for its counter group, run it, publish.
template <typename WT, int CPR_H, int CPR_F, bool LOG>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void megakernel(Params P) {
  __shared__ Smem<WT> sm;
  const int t = wpk_tid(), lane = t & 63, wave = t >> 6;
  const int w = blockIdx.x;
  const uint32_t epoch = ld_sc1(&P.ctl[CTL_EPOCH]);
  const bool dead = ld_sc1(&P.ctl[CTL_STATUS]) != 0u;
  const int q = w % P.n_queues;
  const int qb = cload(P.queue_off, q), qn = cload(P.queue_off, q + 1) - qb;
  uint32_t* head = P.heads + (size_t)q * kLine;
  if (t == 0) sm.first = dead ? qn : (int)atomic_add(head, 1u);
  __syncthreads();
  int ci = __builtin_amdgcn_readfirstlane(sm.first);
  int parity = 0;
  while (ci < qn) {
    const int id = cload(P.queue, qb + ci);
    const Tile T = cload(P.tiles, id);
    Slot s;
    if (P.prefetch) stage<WT, CPR_H, CPR_F>(P, T, s);
    if (wave == 0) {
      uint32_t next = 0;
      if (lane == 0) next = atomic_add(head, 1u);
      int32_t delta = 0;
      bool ok = true;
      if (T.wait >= 0) ok = wait_group(P, T, epoch, &delta);
      if (lane == 0) {
        sm.next[parity] = (int)next;
        sm.ok = ok;
        sm.delta = delta;
      }
    }
    __syncthreads();
    if (!sm.ok) break;
    if (!P.prefetch) stage<WT, CPR_H, CPR_F>(P, T, s);
    if (P.perturb) {
      for (uint32_t k = hash32((uint32_t)id ^ P.perturb) & 31u; k; --k) __builtin_amdgcn_s_sleep(8);
    }
    const uint64_t t_start = LOG ? __builtin_amdgcn_s_memrealtime() : 0;
    run_tile<WT, CPR_H, CPR_F>(P, T, s, sm);
    // publish: every wave's device-coherent stores have completed, then one
    // relaxed device-scope increment of the tile's counter shard
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t == 0) {
      if (LOG) {
        int32_t* rec = P.log + (size_t)id * 8;
        __hip_atomic_fetch_add(rec, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        rec[1] = sm.delta;
        rec[2] = w;
        rec[3] = ci;
        const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
        *(uint64_t*)(rec + 4) = t_start;
        *(uint64_t*)(rec + 6) = t_end;
      }
      if (T.signal >= 0 && id != P.drop_tile) {
        const Group G = cload(P.groups, T.signal);
        atomic_add(&P.counters[(size_t)(G.shard0 + T.shard) * kLine], 1u);
      }
    }
    ci = __builtin_amdgcn_readfirstlane(sm.next[parity]);
    parity ^= 1;
  }
  // leave the step; the last worker out rewinds the queues and advances the epoch
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (t == 0) {
    const uint32_t old = atomic_add(&P.ctl[CTL_EXIT], 1u);
    if (old == (uint32_t)P.n_workers - 1u) {
      for (int i = 0; i < P.n_queues; ++i) st_sc1(&P.heads[(size_t)i * kLine], 0u);
      st_sc1(&P.ctl[CTL_EXIT], 0u);
      st_sc1(&P.ctl[CTL_EPOCH], epoch + 1u);
    }
  }
}

// One operator of the conventional baseline: one workgroup per tile, no
// counters; kernel boundaries order the operators.
template <typename WT, int CPR_H, int CPR_F>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void phase_kernel(Params P, int first) {
  __shared__ Smem<WT> sm;
  const int id = first + (int)blockIdx.x;
  const Tile T = cload(P.tiles, id);
  Slot s;
  stage<WT, CPR_H, CPR_F>(P, T, s);
  run_tile<WT, CPR_H, CPR_F>(P, T, s, sm);
}

}  // namespace wpk

// Kernel handles for a (dtype, row geometry); 0 if that instance is not built.
extern "C" int wpk_dev_kernels(int dtype, int cpr_h, int cpr_f, const void** mk, const void** mk_log,
                               const void** phase) {
  using namespace wpk;
#define WPK_INST(DT, WT, H, F)                                                 \
  if (dtype == DT && cpr_h == H && cpr_f == F) {                                \
    *mk = reinterpret_cast<const void*>(&megakernel<WT, H, F, false>);          \
    *mk_log = reinterpret_cast<const void*>(&megakernel<WT, H, F, true>);       \
    *phase = reinterpret_cast<const void*>(&phase_kernel<WT, H, F>);            \
    return 1;                                                                   \
  }
  WPK_INST(WPK_F32, float, 64, 256)      // tiny: hidden 256, ffn 1024, f32
  WPK_INST(WPK_BF16, uint16_t, 256, 1024)  // Llama-3.2-1B shape: hidden 2048, ffn 8192, bf16
  WPK_INST(WPK_BF16, uint16_t, 64, 128)  // hidden 512, ffn 1024, bf16
  WPK_INST(WPK_BF16, uint16_t, 64, 256)  // hidden 512, ffn 2048, bf16
#undef WPK_INST
  return 0;
}
