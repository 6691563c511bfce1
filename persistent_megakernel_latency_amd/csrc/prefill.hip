// prefill.hip -- the prompt prefill (time to first token) as one persistent
// kernel on gfx950, and the conventional one-kernel-per-operator baseline
// built from the same tile bodies.
//
// A worker is one workgroup of eight waves per compute unit, all computing:
// prefill tiles are compute-bound (a matrix-core tile is 128 x 256 x K), so
// the decode step's split into a latency-hiding control wave and
// weight-streaming compute waves buys nothing here, and one wide tile per CU
// fetches each k-step's fragments once for all eight waves (two 128 x 128
// tiles side by side on one CU would fetch the operand rows twice).  Wave 0
// polls the tile's counter group; thread 0 claims the next tile while the
// current one runs, then publishes.
//
// Coherence.  The eight XCDs' L2 caches are not coherent with each other.
// Outputs are written with device-coherent (sc1, write-through) stores, and
// the publish is a relaxed device-scope increment after they completed (the
// decode step's protocol).  Inputs are read with ordinary, cacheable loads:
// every activation buffer of a layer is written exactly once per prefill and
// read only after its counter group completed, so no L2 or L1 can hold a
// stale copy of a line a tile reads (a cache only holds lines read during
// this launch, and each line is read only after its one write; the caches
// start clean at every kernel boundary).  This lets the 24 QKV tiles of a
// row block share its operand rows through the L2 of their XCD.
#include "prefill_plan.h"
#include "worker.h"

namespace wpk {
namespace {

constexpr int kVtPitch = 40;  // bf16 elements per transposed V row (32 keys + pad)

constexpr int kGBlocks = 32;  // 1 KiB fragment blocks of a matrix-core k-step: 16 weight, 8 operand hi, 8 lo
constexpr int kGStages = 4;   // LDS stages of the matrix-core k-loop (128 KiB)

struct PSmem {
  union alignas(16) {
    uint16_t vt[2][kHeadDim][kVtPitch];  // attention: one key step of V, [dim][key]
    u32x4 gs[kGStages][kGBlocks][64];    // matrix-core tiles: four k-steps of fragments, 16 bytes per lane
  };
  float nss[kPWaves][16];  // norm tiles: each wave's sums of squares of the 16 rows
  int claim[2];
  int stop;
};

__device__ __forceinline__ void p_latch(const PParams& P, int32_t code, int32_t tile) {
  uint32_t zero = 0;
  if (__hip_atomic_compare_exchange_strong(&P.ctl[CTL_STATUS], &zero, (uint32_t)code, __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
    st_sc1(&P.ctl[CTL_STATUS + 1], (uint32_t)tile);
    st_sc1(&P.ctl[CTL_STATUS + 2], (uint32_t)blockIdx.x);
    st_sc1(&P.ctl[CTL_STATUS + 3], ld_sc1(&P.ctl[CTL_EPOCH]));
  }
  st_sc1(&P.ctl[CTL_ABORT], 1u);
}

// Bounded wait for the tile's counter group (wave 0; the same sharded
// counters and epoch targets as the decode step).
__device__ __forceinline__ bool p_wait(const PParams& P, const Tile& T, uint32_t epoch, int32_t* delta, int lane) {
  const Group G = cload(P.groups, T.wait);
  const uint32_t target = (epoch + 1u) * (uint32_t)G.producers;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    const uint32_t v0 = lane < G.shards ? ld_sc1(&P.counters[(size_t)(G.shard0 + lane) * kLine]) : 0u;
    const uint32_t v1 = lane + 64 < G.shards ? ld_sc1(&P.counters[(size_t)(G.shard0 + lane + 64) * kLine]) : 0u;
    const uint32_t sum = wave_sum_u32(v0 + v1);
    if ((int32_t)(sum - target) >= 0) {
      *delta = (int32_t)(sum - target);
      compiler_order();
      return true;
    }
    if (ld_sc1(&P.ctl[CTL_ABORT])) return false;
    if (__builtin_amdgcn_s_memrealtime() - t0 > P.watchdog_ticks) {
      if (lane == 0) p_latch(P, WPK_E_TIMEOUT, T.id);
      return false;
    }
    __builtin_amdgcn_s_sleep(4);
  }
}

// A buffer resource from a pointer that is the same in every lane, built from
// scalar copies of it: the compiler would otherwise keep a resource chosen by
// a select or derived through a switch in vector registers and wrap every
// load in a loop over its distinct values.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t urs(const void* p) {
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return rsrc((const void*)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
// An LDS address as the LDS-destination operand of a buffer load.
__device__ __forceinline__ __attribute__((address_space(3))) void* lds_ptr(void* p) {
  return (__attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ u32x2 bf16x4(f32x4 v) { return u32x2{cvt_bf16x2(v[0], v[1]), cvt_bf16x2(v[2], v[3])}; }
// Device-coherent (sc1) stores through a wave-uniform buffer resource; the
// per-lane part of the address is the byte offset.
__device__ __forceinline__ void st16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 16 /* sc1 */);
}
__device__ __forceinline__ void st8(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 16 /* sc1 */);
}
// Four fp32 values as bf16 hi + lo parts (value = hi + lo), 8 bytes into each
// plane of an operand buffer.
__device__ __forceinline__ void st_hilo4(__amdgpu_buffer_rsrc_t hi, __amdgpu_buffer_rsrc_t lo, uint32_t off, f32x4 v) {
  uint32_t h0, h1, l0, l1;
  split_hilo2(v[0], v[1], h0, l0);
  split_hilo2(v[2], v[3], h1, l1);
  st8(hi, off, u32x2{h0, h1});
  st8(lo, off, u32x2{l0, l1});
}
// Eight fp32 values as a bf16x8 hi part and a bf16x8 lo part.
__device__ __forceinline__ bf16x8 hilo8(f32x4 a, f32x4 b, bf16x8& lo) {
  uint32_t h[4], l[4];
  split_hilo2(a[0], a[1], h[0], l[0]);
  split_hilo2(a[2], a[3], h[1], l[1]);
  split_hilo2(b[0], b[1], h[2], l[2]);
  split_hilo2(b[2], b[3], h[3], l[3]);
  lo = as_bf16x8(u32x4{l[0], l[1], l[2], l[3]});
  return as_bf16x8(u32x4{h[0], h[1], h[2], h[3]});
}

// fp16 operands (the o-projection, gate/up and down products): one plane,
// one product per fragment.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// two floats as fp16 (round to nearest even), a in the low half; over is set
// if a finite value is beyond the fp16 range (it would round to infinity)
__device__ __forceinline__ uint32_t cvt_f16x2(float a, float b, bool& over) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  over |= (fabsf(a) >= 65520.f) | (fabsf(b) >= 65520.f);
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, f16x2));
}
// Four fp32 values as fp16, 8 bytes into an operand plane.
__device__ __forceinline__ void st_f16x4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v, bool& over) {
  st8(r, off, u32x2{cvt_f16x2(v[0], v[1], over), cvt_f16x2(v[2], v[3], over)});
}
// A wave that saw an fp16 overflow latches WPK_E_RANGE.
__device__ __forceinline__ void range_check(const PParams& P, const Tile& T, bool over, int lane) {
  if (__builtin_amdgcn_ballot_w64(over) != 0 && lane == 0) p_latch(P, WPK_E_RANGE, T.id);
}

// Fragment-major ("packed") layout of a bf16 matrix-core operand with K
// columns: blocks of 16 rows x 32 columns, one 1 KiB block per (16 rows,
// k-step) in row-block-major order, and inside a block lane l's 16 bytes at
// 16 l hold row l % 16, columns 8 (l / 16) .. +7 -- the register layout of a
// v_mfma_f32_16x16x32_bf16 operand.  A wave then loads a fragment as one
// contiguous KiB (eight whole cache lines); in row-major order the same
// fragment is sixteen half-used lines, and the loads, not the matrix cores,
// set the pace (measured: a 128 x 128 x 2048 tile took 88 us row-major).
// Byte offset of element (r, k), 4-element aligned groups stay contiguous.
__device__ __forceinline__ uint32_t pk(uint32_t r, uint32_t k, uint32_t K) {
  return (((r >> 4) * (K >> 5) + (k >> 5)) * 64u + (r & 15u) + 16u * ((k & 31u) >> 3)) * 16u + (k & 7u) * 2u;
}

// ---- RMSNorm of rows -------------------------------------------------------------------------
// y = x / sqrt(mean(x^2) + eps) * gain, stored as the hi and lo bf16 planes
// of the packed matrix-core operand (F16: one fp16 plane).  Returns whether a
// value overflowed fp16.  A norm tile takes 16 rows; wave w takes
// an eighth of the columns in the fragment layout (lane l: row l % 16,
// columns 8 (l / 16) .. +7 of each 32-column k-step), so every store is one
// contiguous KiB per wave and all of a wave's loads of a pass are in flight
// at once.  Sums of squares: each lane in column order, the four lanes of a
// row with lane swaps, then the eight waves' parts in a fixed order through
// LDS.  Second pass: the rows are read again (from the
// cache), scaled and stored.  src(r, k, a, b) gives 8 fp32 values of row r
// from column k.
template <bool F16, typename SRC>
__device__ __forceinline__ bool norm_rows16(const PParams& P, int r0, const SRC& src, const float* gain,
                                            __amdgpu_buffer_rsrc_t yh, __amdgpu_buffer_rsrc_t yl,
                                            __amdgpu_buffer_rsrc_t xc, bool copy, PSmem& sm, int w, int lane) {
  const int r = r0 + (lane & 15), c8 = 8 * (lane >> 4), nks = P.H / 32, q = nks / kPWaves, k0 = w * q;
  float ss = 0.f;
#pragma unroll 16
  for (int ks = k0; ks < k0 + q; ++ks) {
    f32x4 a, b;
    src(r, 32 * ks + c8, a, b);
    ss += ((a[0] * a[0] + a[1] * a[1]) + (a[2] * a[2] + a[3] * a[3])) +
          ((b[0] * b[0] + b[1] * b[1]) + (b[2] * b[2] + b[3] * b[3]));
  }
  ss = xsum<16>(ss);
  ss = xsum<32>(ss);
  if (lane < 16) sm.nss[w][lane] = ss;
  __syncthreads();
  const int rr = lane & 15;
  const float tot = ((sm.nss[0][rr] + sm.nss[1][rr]) + (sm.nss[2][rr] + sm.nss[3][rr])) +
                    ((sm.nss[4][rr] + sm.nss[5][rr]) + (sm.nss[6][rr] + sm.nss[7][rr]));
  const float inv = 1.0f / sqrtf(tot / (float)P.H + P.eps);
  const uint32_t blk = (uint32_t)(r0 >> 4) * (uint32_t)nks * 1024u + (uint32_t)lane * 16u;
  bool over = false;
#pragma unroll 16
  for (int ks = k0; ks < k0 + q; ++ks) {
    const int k = 32 * ks + c8;
    f32x4 a, b;
    src(r, k, a, b);
    if (copy) {
      const uint32_t xo = ((uint32_t)r * (uint32_t)P.H + (uint32_t)k) * 4u;
      st16(xc, xo, __builtin_bit_cast(u32x4, a));
      st16(xc, xo + 16u, __builtin_bit_cast(u32x4, b));
    }
    const f32x4 ga = *(const f32x4*)(gain + k), gb = *(const f32x4*)(gain + k + 4);
    a = a * inv * ga;
    b = b * inv * gb;
    if (F16) {
      st16(yh, blk + (uint32_t)ks * 1024u,
           u32x4{cvt_f16x2(a[0], a[1], over), cvt_f16x2(a[2], a[3], over), cvt_f16x2(b[0], b[1], over),
                 cvt_f16x2(b[2], b[3], over)});
    } else {
      uint32_t h[4], l[4];
      split_hilo2(a[0], a[1], h[0], l[0]);
      split_hilo2(a[2], a[3], h[1], l[1]);
      split_hilo2(b[0], b[1], h[2], l[2]);
      split_hilo2(b[2], b[3], h[3], l[3]);
      st16(yh, blk + (uint32_t)ks * 1024u, u32x4{h[0], h[1], h[2], h[3]});
      st16(yl, blk + (uint32_t)ks * 1024u, u32x4{l[0], l[1], l[2], l[3]});
    }
  }
  return over;
}

// A norm tile: rows 16 sub .. +15 of its row block.  Layer 0 gathers the
// embedding rows (token ids checked; padding rows past the prompt are zero)
// and keeps them as the residual stream.
__device__ void norm_tile(const PParams& P, const Tile& T, PSmem& sm, int tid) {
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const PLayer Lw = cload(P.layers, T.layer);
  const size_t plane = (size_t)P.R * P.H;
  uint16_t* y = T.type == P_NORM2 ? Lw.xn2 : Lw.xn1;
  const __amdgpu_buffer_rsrc_t yh = urs(y), yl = urs(y + plane), xc = urs(P.x0);
  const int r0 = T.r0 * kPRows + 16 * T.r1;
  if (T.type == P_EMBED) {
    const int r = r0 + (lane & 15), b = r / P.Pp, p = r - b * P.Pp;
    int tok = 0;
    if (p < P.P) {
      tok = P.prompt[(size_t)b * P.P + p];
      if (tok < 0 || tok >= P.V) {
        if (w == 0) p_latch(P, WPK_E_TOKEN, T.id);
        tok = 0;
      }
    }
    const uint16_t* er = P.embed + (size_t)tok * P.H;
    const bool pad = p >= P.P;
    auto src = [&](int, int k, f32x4& a, f32x4& bb) {
      const u32x4 e = *(const u32x4*)(er + k);
      a = pad ? f32x4{0.f, 0.f, 0.f, 0.f} : f32x4{bf16_lo(e.x), bf16_hi(e.x), bf16_lo(e.y), bf16_hi(e.y)};
      bb = pad ? f32x4{0.f, 0.f, 0.f, 0.f} : f32x4{bf16_lo(e.z), bf16_hi(e.z), bf16_lo(e.w), bf16_hi(e.w)};
    };
    norm_rows16<false>(P, r0, src, Lw.attn_norm, yh, yl, xc, true, sm, w, lane);
  } else {
    const float* x = T.type == P_NORM1 ? Lw.x_in : Lw.x_mid;
    auto src = [&](int r, int k, f32x4& a, f32x4& bb) {
      const float* xr = x + (size_t)r * P.H + k;
      a = *(const f32x4*)xr;
      bb = *(const f32x4*)(xr + 4);
    };
    if (T.type == P_NORM1) {
      norm_rows16<false>(P, r0, src, Lw.attn_norm, yh, yl, xc, false, sm, w, lane);
    } else {  // the gate/up operand: fp16
      const bool over = norm_rows16<true>(P, r0, src, Lw.mlp_norm, yh, yl, xc, false, sm, w, lane);
      range_check(P, T, over, lane);
    }
  }
}

// The final norm of one sequence's last prompt row (xf row b): wave 0, the
// 64 lanes across the row (all of its chunks loaded at once), stored into
// row b of the packed xf.  Only row b is touched: the other sequences' rows
// may not be complete yet, and reading a line before its producer has
// written it could leave a stale copy in this XCD's cache.
constexpr int kNormChunks = 16;  // 16-byte chunks per lane for hidden up to 4096
__device__ void normf_tile(const PParams& P, const Tile& T, int tid) {
  if (tid >= 64) return;
  const int lane = tid, nc = P.H / 4;
  const PLayer Lw = cload(P.layers, P.L - 1);
  const float* x = Lw.x_out + ((size_t)T.b * P.Pp + P.P - 1) * P.H;
  f32x4 v[kNormChunks];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < kNormChunks; ++k)
    if (lane + 64 * k < nc) v[k] = *(const f32x4*)(x + 4 * (lane + 64 * k));
#pragma unroll
  for (int k = 0; k < kNormChunks; ++k)
    if (lane + 64 * k < nc) ss += (v[k][0] * v[k][0] + v[k][1] * v[k][1]) + (v[k][2] * v[k][2] + v[k][3] * v[k][3]);
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)P.H + P.eps);
  const __amdgpu_buffer_rsrc_t yh = urs(P.xf), yl = urs(P.xf + (size_t)kMaxBatch * P.H);
#pragma unroll
  for (int k = 0; k < kNormChunks; ++k) {
    const int c = lane + 64 * k;
    if (c < nc) st_hilo4(yh, yl, pk((uint32_t)T.b, 4u * c, (uint32_t)P.H), v[k] * inv * *(const f32x4*)(P.final_norm + 4 * c));
  }
}

// ---- matrix-core tiles: 128 prompt rows x 256 output columns x all of K ----------------------
//
// v_mfma_f32_16x16x32_bf16 with the weights as the A operand (lane l: weight
// row l % 16, eight K values from 8 (l / 16)) and the activations as B (lane
// l: prompt row l % 16, the same K values), twice: the operand's hi and lo
// bf16 planes (bf16 weights are exact, so the two products keep about 16
// significant bits of the activations); the 16 x 16 result leaves lane l
// four consecutive output columns 4 (l / 16) + e of prompt row l % 16, so
// epilogues store 8 or 16 contiguous bytes per lane.  Wave w computes rows
// 64 (w & 1) .. +63 and columns 64 (w >> 1) .. +63 (one head of QKV): four
// column blocks j x four row blocks i.
//
// A k-step (32 of K) needs 32 fragment blocks of 1 KiB (16 bytes per lane in
// fragment order): 16 weight blocks of 16 rows, 8 operand blocks of 16 rows
// in the hi plane and 8 in the lo plane.  Each wave fetches 4 of them
// straight into an LDS stage (buffer loads with the LDS as destination: lane
// l's 16 bytes land at 16 l of the block, the fragment layout), then every
// wave reads its 12 blocks from LDS.  Each block is fetched from the caches
// once per tile instead of once per wave that uses it, and nothing passes
// through registers on its way into LDS: staging through registers and
// ds_write cost a k-step about 0.75 us against 0.54 us this way (measured,
// 8 waves per CU, products included), LDS writes being the slow half of the
// LDS's bandwidth.
// F16 (o-projection, gate/up, down): fp16 weights against one fp16 operand
// plane -- 24 blocks per k-step (16 weight, 8 operand), each wave fetching
// weight blocks 2w, 2w+1 and operand block w, and 16 products per wave.
template <bool F16>
__device__ void gemm_tile(const PParams& P, const Tile& T0, PSmem& sm, int tid) {
  const Tile T = uni(T0);
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = w & 1, wc = w >> 1, l15 = lane & 15, g4 = lane >> 4;
  const PLayer Lw = cload(P.layers, T.layer);
  const uint16_t* A;
  const uint16_t* W0;
  const uint16_t* W1;
  int K, wrow0;  // first weight row of this wave's column blocks (gate/up: of its gate and up halves)
  switch (T.type) {
    case P_QKV: A = Lw.xn1, W0 = W1 = Lw.w_qkv, K = P.H, wrow0 = T.r1 * kPCols + 64 * wc; break;
    case P_OPROJ: A = Lw.ao, W0 = W1 = Lw.w_o, K = P.H, wrow0 = T.r1 * kPCols + 64 * wc; break;
    case P_GATEUP: A = Lw.xn2, W0 = Lw.w_gate, W1 = Lw.w_up, K = P.H, wrow0 = T.r1 * kPFfnCols + 32 * wc; break;
    default: A = Lw.h, W0 = W1 = Lw.w_down, K = P.F, wrow0 = T.r1 * kPCols + 64 * wc; break;
  }
  const bool gu = T.type == P_GATEUP;
  const int row0 = T.r0 * kPRows + 64 * wr;
  // this wave's loads: weight blocks 2w, 2w+1 (block jj: column group jj / 4, block jj % 4 of it),
  // operand block w of the hi and of the lo plane
  const __amdgpu_buffer_rsrc_t ra = urs(A), rl = urs(A + (size_t)P.R * K);
  uint32_t gv[3];
  __amdgpu_buffer_rsrc_t gr[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int jj = 2 * w + q, c = jj >> 2, j = jj & 3;
    const int row = gu ? T.r1 * kPFfnCols + 32 * c + 16 * (j & 1) : T.r1 * kPCols + 16 * jj;
    gr[q] = urs(gu && j >= 2 ? W1 : W0);
    // packed operands: the fragment of 16 rows at k-step ks is the KiB at
    // (row block * K / 32 + ks) * 1024, the lane's 16 bytes at 16 lane
    gv[q] = ((uint32_t)(row >> 4) * (uint32_t)(K >> 5) * 64u + lane) * 16u;
  }
  gv[2] = ((uint32_t)(T.r0 * (kPRows / 16) + w) * (uint32_t)(K >> 5) * 64u + lane) * 16u;
  // this wave's blocks of k-step ks into LDS stage st
  auto fetch = [&](int st, int ks) {
    const uint32_t so = (uint32_t)ks * 1024u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(gr[0], lds_ptr(&sm.gs[st][2 * w][0]), 16, gv[0], so, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(gr[1], lds_ptr(&sm.gs[st][2 * w + 1][0]), 16, gv[1], so, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, lds_ptr(&sm.gs[st][16 + w][0]), 16, gv[2], so, 0, 0);
    if (!F16) __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, lds_ptr(&sm.gs[st][24 + w][0]), 16, gv[2], so, 0, 0);
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // fragments of one k-step from an LDS stage: 4 weight blocks, the hi and lo
  // planes of 4 operand blocks
  struct Frag {
    bf16x8 b[4], a[4], al[4];
  };
  auto fread = [&](int st, Frag& f) {
#pragma unroll
    for (int j = 0; j < 4; ++j) f.b[j] = as_bf16x8(sm.gs[st][4 * wc + j][lane]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f.a[i] = as_bf16x8(sm.gs[st][16 + 4 * wr + i][lane]);
      if (!F16) f.al[i] = as_bf16x8(sm.gs[st][24 + 4 * wr + i][lane]);
    }
  };
  // the hi products, then the lo products: no two consecutive products share
  // an accumulator (fp16: the one product per pair)
  auto products = [&](const Frag& f) {
    if (F16) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[j][i] = mfma16(__builtin_bit_cast(f16x8, f.b[j]), __builtin_bit_cast(f16x8, f.a[i]), acc[j][i]);
      return;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[j][i] = mfma(f.b[j], f.a[i], acc[j][i]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[j][i] = mfma(f.b[j], f.al[i], acc[j][i]);
  };
  // Pipeline over k-steps h: four LDS stages (step h in stage h % 4) and two
  // fragment sets in turn.  In step h a wave issues the fetch of step h + 3
  // into its stage (last read in step h - 2: its reads completed before that
  // data's products in step h - 1), reads step h + 1's fragments from LDS,
  // runs step h's products, waits for its fetch of step h + 2 (issued in
  // step h - 1; only this step's NF fetches may still be in flight) and
  // meets the others at a barrier, after which step h + 2's stage is
  // complete.  So a fetch has two steps of products to land in.  The k-loop
  // issues no other vector-memory operation, and the counter retires them in
  // order, so "at most NF outstanding" is exactly "step h + 2 has landed".
  // The barrier is a bare s_barrier between compiler-only fences: a
  // workgroup fence there would wait for every outstanding LDS-destination
  // load, this step's included.  Past the last step the fetch repeats it
  // (never used).
  constexpr int NF = F16 ? 3 : 4;  // fetches per wave and k-step
  const int nk = K / 32;
  auto kc = [&](int ks) { return min(ks, nk - 1); };
  auto step_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F70 | NF);  // vmcnt(NF), expcnt and lgkmcnt unconstrained
    compiler_order();
    __builtin_amdgcn_s_barrier();
    compiler_order();
  };
  Frag F0, F1;
  fetch(0, 0);
  fetch(1, kc(1));
  fetch(2, kc(2));
  step_barrier();  // steps 0 and 1 landed
  fread(0, F0);
#define WPK_GEMM_STEP(I, FN, FC)                                            \
  {                                                                         \
    const int h = h0 + (I);                                                 \
    fetch(((I) + 3) % 4, kc(h + 3));                                        \
    __builtin_amdgcn_sched_barrier(0);                                      \
    fread(((I) + 1) % 4, FN);                                               \
    if (h < nk) products(FC);                                               \
    step_barrier();                                                         \
  }
  for (int h0 = 0; h0 < nk; h0 += 4) {
    WPK_GEMM_STEP(0, F1, F0)
    WPK_GEMM_STEP(1, F0, F1)
    WPK_GEMM_STEP(2, F1, F0)
    WPK_GEMM_STEP(3, F0, F1)
  }
#undef WPK_GEMM_STEP

  // epilogues: lane holds columns c_j + 4 (lane / 16) + e of prompt row r_i
  const int e4 = 4 * (lane >> 4);
  switch (T.type) {
    case P_QKV: {
      const int hh = T.r1 * (kPCols / kHeadDim) + wc;  // head of this wave's 64 columns: q heads, then k, then v
      const bool isq = hh < P.Hq, isk = !isq && hh < P.Hq + P.Hkv;
      const __amdgpu_buffer_rsrc_t rd = urs(isq ? (void*)Lw.q : isk ? (void*)P.kc : (void*)P.vc);
      const int kh = isk ? hh - P.Hq : hh - P.Hq - P.Hkv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = row0 + 16 * i + (lane & 15);
        const int bq = r / P.Pp, p = r - bq * P.Pp;
        if (p >= P.P) continue;  // padding rows: nothing stored
        f32x4 y[4] = {acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
        if (hh < P.Hq + P.Hkv) {
          // rotate-half RoPE: dims d < 32 pair with d + 32 (blocks j and j + 2)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const f32x4 cs = *(const f32x4*)(P.rope_cos + (size_t)p * 32 + 16 * j + e4);
            const f32x4 sn = *(const f32x4*)(P.rope_sin + (size_t)p * 32 + 16 * j + e4);
            const f32x4 x1 = acc[j][i], x2 = acc[j + 2][i];
            y[j] = x1 * cs - x2 * sn;
            y[j + 2] = x2 * cs + x1 * sn;
          }
        }
        if (isq) {
          const uint32_t o = ((uint32_t)r * (uint32_t)P.Hq + (uint32_t)hh) * kHeadDim;
#pragma unroll
          for (int j = 0; j < 4; ++j) st16(rd, (o + 16 * j + e4) * 4u, __builtin_bit_cast(u32x4, y[j]));
        } else {
          const uint32_t o = (uint32_t)(((((size_t)T.layer * P.B + bq) * P.Hkv + kh) * P.cap + p) * kHeadDim);
#pragma unroll
          for (int j = 0; j < 4; ++j) st8(rd, (o + 16 * j + e4) * 2u, bf16x4(y[j]));
        }
      }
      break;
    }
    case P_OPROJ:
    case P_DOWN: {
      const float* xs = T.type == P_OPROJ ? Lw.x_in : Lw.x_mid;
      const __amdgpu_buffer_rsrc_t rd = urs(T.type == P_OPROJ ? Lw.x_mid : Lw.x_out);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t ro = (uint32_t)(row0 + 16 * i + (lane & 15)) * (uint32_t)P.H;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t c = (uint32_t)(wrow0 + 16 * j + e4);
          const f32x4 v = *(const f32x4*)(xs + ro + c) + acc[j][i];
          st16(rd, (ro + c) * 4u, __builtin_bit_cast(u32x4, v));
        }
      }
      break;
    }
    default: {  // P_GATEUP: h = silu(gate) * up, blocks 0-1 gate and 2-3 up of the same columns; the down operand (fp16)
      const __amdgpu_buffer_rsrc_t hh = urs(Lw.h);
      bool over = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const f32x4 g = acc[j][i], u = acc[j + 2][i];
          f32x4 hv;
#pragma unroll
          for (int e = 0; e < 4; ++e) hv[e] = g[e] / (1.0f + __expf(-g[e])) * u[e];
          st_f16x4(hh, pk((uint32_t)(row0 + 16 * i + (lane & 15)), (uint32_t)(wrow0 + 16 * j + e4), (uint32_t)P.F), hv,
                   over);
        }
      }
      range_check(P, T, over, lane);
      break;
    }
  }
}

// ---- causal attention: (sequence, kv head, 64 queries) ------------------------------------------
//
// Wave w takes q head w % 4 of the kv head's group and queries 32 (w / 4) ..
// +31 of the tile (waves past the group size idle); every wave of the
// worker shares the staged V of a step.
// Per step of 32 keys, on the matrix cores:
//  * S^T = K Q^T: A = K rows from the cache (lane l: key l % 16, dims
//    8 (l / 16) ..), B = the wave's queries (query l % 16), scaled by 1/sqrt(D)
//    and split into hi + lo bf16 parts (two products; K in the cache is bf16
//    and exact).  Lane l gets keys 4 (l / 16) + e of query l % 16 for each
//    16-key block.
//  * The online softmax (max, rescale, exponentials) runs per query in that
//    layout; the four lanes of a query combine maxima with lane swaps.
//  * O^T += V^T P^T: B = the lane's own eight probabilities (hi + lo bf16), in
//    K order 8 (l / 16) + 4 kb + e <-> key 16 kb + 4 (l / 16) + e; A = V from
//    LDS, staged transposed ([dim][key]) by all eight waves, read in that
//    same key order.  Lane l accumulates dims 4 (l / 16) + e of query l % 16.
// Causality masks keys past each query and past the prompt; V rows past the
// prompt are staged as zeros, K rows past it re-read the last prompt row.
// Rounding the queries or the probabilities to plain bf16 alone moves the
// last-position logits of the 16-layer model by about 2e-2, hence the pairs.
constexpr int kPQB = 2;  // 16-query blocks per wave
static_assert(kPQueries == 2 * 16 * kPQB && kPWaves == 2 * kMaxGroupHeads, "attention waves: 4 heads x 2 query halves");

__device__ void attn_tile(const PParams& P, const Tile& T0, PSmem& sm, int tid) {
  const Tile T = uni(T0);
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const PLayer Lw = cload(P.layers, T.layer);
  const int q0 = T.c * kPQueries, nq = min(kPQueries, P.P - q0), kend = q0 + nq;
  const int nsteps = (kend + kPKeys - 1) / kPKeys;
  const int hw = w & (kMaxGroupHeads - 1), qw = q0 + 16 * kPQB * (w >> 2);  // this wave's first query
  const bool active = hw < P.G && qw < kend;  // waves whose queries are all padding idle too
  const int h = T.g * P.G + (hw < P.G ? hw : 0);
  const size_t kvpos = (((size_t)T.layer * P.B + T.b) * P.Hkv + T.g) * P.cap;  // position 0 of this kv head
  const __amdgpu_buffer_rsrc_t rk = urs(P.kc + kvpos * kHeadDim), rv = urs(P.vc + kvpos * kHeadDim);
  const int l15 = lane & 15, g4 = lane >> 4;

  // queries (B operand) as hi + lo bf16
  bf16x8 qh[kPQB][2], ql[kPQB][2];
#pragma unroll
  for (int i = 0; i < kPQB; ++i) {
    const float* qr = Lw.q + ((size_t)T.b * P.Pp + qw + 16 * i + l15) * P.Hq * kHeadDim + h * kHeadDim;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f32x4 x0 = *(const f32x4*)(qr + 32 * s + 8 * g4) * P.attn_scale;
      const f32x4 x1 = *(const f32x4*)(qr + 32 * s + 8 * g4 + 4) * P.attn_scale;
      qh[i][s] = hilo8(x0, x1, ql[i][s]);
    }
  }
  // K fragments of a step (A operand), rows clamped into the prompt
  auto kload = [&](int k0, u32x4 (&kf)[2][2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = min(k0 + 16 * kb + l15, kend - 1);
#pragma unroll
      for (int s = 0; s < 2; ++s) kf[kb][s] = ld16(rk, (uint32_t)(key * kHeadDim + 32 * s + 8 * g4) * 2u, 0);
    }
  };
  // V staging: thread t loads dims 4 (t % 16) .. +3 of key t / 16 of the step
  static_assert(kPThreads == kPKeys * kHeadDim / 4, "V staging: one 8-byte chunk per thread");
  const int vkey = tid >> 4, vd0 = 4 * (tid & 15);
  auto vload = [&](int k0) -> u32x2 {
    const int key = k0 + vkey;
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rv, (uint32_t)(min(key, kend - 1) * kHeadDim + vd0) * 2u, 0, 0);
    return key < kend ? v : u32x2{0u, 0u};
  };
  auto vstore = [&](int buf, u32x2 v) {
    sm.vt[buf][vd0][vkey] = (uint16_t)(v.x & 0xFFFFu);
    sm.vt[buf][vd0 + 1][vkey] = (uint16_t)(v.x >> 16);
    sm.vt[buf][vd0 + 2][vkey] = (uint16_t)(v.y & 0xFFFFu);
    sm.vt[buf][vd0 + 3][vkey] = (uint16_t)(v.y >> 16);
  };

  float m[kPQB], lsum[kPQB];
  f32x4 o[4][kPQB];  // [dim block][query block]
#pragma unroll
  for (int i = 0; i < kPQB; ++i) {
    m[i] = -INFINITY;
    lsum[i] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  u32x4 kf[2][2];
  u32x2 vreg = vload(0);
  kload(0, kf);
  for (int ks = 0; ks < nsteps; ++ks) {
    const int k0 = ks * kPKeys, buf = ks & 1;
    vstore(buf, vreg);
    __syncthreads();  // this step's V staged; every wave is past step ks - 1 (its buffer is free)
    // the next step's loads, unconditional (past the last step they repeat it)
    const int kn = min(ks + 1, nsteps - 1) * kPKeys;
    u32x4 nkf[2][2];
    vreg = vload(kn);
    kload(kn, nkf);
    // a step past this wave's last query is masked whole: skipped (the wave's
    // SIMD partner, the other query half of the same head, runs alone)
    if (active && k0 <= qw + 16 * kPQB - 1) {
      f32x4 st[2][kPQB];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < kPQB; ++i) {
          f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            z = mfma(as_bf16x8(kf[kb][s]), qh[i][s], z);
            z = mfma(as_bf16x8(kf[kb][s]), ql[i][s], z);
          }
          st[kb][i] = z;
        }
      bf16x8 ph[kPQB], pl[kPQB];
#pragma unroll
      for (int i = 0; i < kPQB; ++i) {
        const int qpos = qw + 16 * i + l15;
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = k0 + 16 * kb + 4 * g4 + e;
            const float v = (key <= qpos && key < kend) ? st[kb][i][e] : -INFINITY;
            st[kb][i][e] = v;
            mx = fmaxf(mx, v);
          }
        mx = xmax<16>(mx);
        mx = xmax<32>(mx);
        const float mn = fmaxf(m[i], mx);
        const float alpha = __expf(m[i] - mn);
        m[i] = mn;
        f32x4 p0, p1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p0[e] = __expf(st[0][i][e] - mn);
          p1[e] = __expf(st[1][i][e] - mn);
        }
        lsum[i] = lsum[i] * alpha + ((p0[0] + p0[1]) + (p0[2] + p0[3])) + ((p1[0] + p1[1]) + (p1[2] + p1[3]));
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db][i] *= alpha;
        ph[i] = hilo8(p0, p1, pl[i]);
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const uint16_t* vr = &sm.vt[buf][16 * db + l15][0];
        const u32x2 v0 = *(const u32x2*)(vr + 4 * g4);
        const u32x2 v1 = *(const u32x2*)(vr + 16 + 4 * g4);
        const bf16x8 vf = as_bf16x8(u32x4{v0.x, v0.y, v1.x, v1.y});
#pragma unroll
        for (int i = 0; i < kPQB; ++i) {
          o[db][i] = mfma(vf, ph[i], o[db][i]);
          o[db][i] = mfma(vf, pl[i], o[db][i]);
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < 2; ++s) kf[kb][s] = nkf[kb][s];
  }
  if (!active) return;
  // the o-projection's operand: one fp16 plane
  const __amdgpu_buffer_rsrc_t oh = urs(Lw.ao);
  bool over = false;
#pragma unroll
  for (int i = 0; i < kPQB; ++i) {
    float lt = xsum<16>(lsum[i]);
    lt = xsum<32>(lt);
    const int qpos = qw + 16 * i + l15;
    if (qpos >= P.P) continue;
    const float inv = 1.0f / lt;
    const uint32_t orow = (uint32_t)T.b * P.Pp + qpos, ocol = (uint32_t)h * kHeadDim + 4 * g4;
#pragma unroll
    for (int db = 0; db < 4; ++db) st_f16x4(oh, pk(orow, ocol + 16 * db, (uint32_t)(P.Hq * kHeadDim)), o[db][i] * inv, over);
  }
  range_check(P, T, over, lane);
}

// ---- LM head on the last prompt rows: 256 vocabulary columns per tile ------------------------
// Wave w: vocabulary rows 32 w .. +31 of the tile (two 16-row blocks) against
// 16 sequences at a time (the final-normed rows, hi and lo bf16 planes).  Logits are stored in
// fp32; the partial greedy choice (value, lowest index) goes to one of 16
// shards per sequence with a 64-bit atomic maximum.
__device__ void lm_tile(const PParams& P, const Tile& T0, int tid) {
  const Tile T = uni(T0);
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l15 = lane & 15, g4 = lane >> 4;
  const int v0 = T.r1 * kPLmCols + 32 * w;
  const __amdgpu_buffer_rsrc_t re = urs(P.embed), rx = urs(P.xf), rxl = urs(P.xf + (size_t)kMaxBatch * P.H);
  uint32_t ve[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) ve[j] = (uint32_t)min(v0 + 16 * j + l15, P.V - 1) * (uint32_t)P.H * 2u + 16u * g4;
  for (int sg = 0; sg * 16 < P.B; ++sg) {
    const uint32_t vx = ((uint32_t)sg * (uint32_t)(P.H >> 5) * 64u + lane) * 16u;  // packed xf
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll 8
    for (int k0 = 0; k0 < P.H; k0 += 32) {
      const uint32_t so = (uint32_t)k0 * 2u, sx = (uint32_t)k0 * 32u;
      const bf16x8 x = as_bf16x8(ld16(rx, vx, sx)), xl = as_bf16x8(ld16(rxl, vx, sx));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8 e = as_bf16x8(ld16(re, ve[j], so));
        acc[j] = mfma(e, x, acc[j]);
        acc[j] = mfma(e, xl, acc[j]);
      }
    }
    const int seq = 16 * sg + l15;
    unsigned long long best = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int v = v0 + 16 * j + 4 * g4;
      if (seq < P.B) {
        float* lg = P.logits + (size_t)seq * P.V;
        if (v + 3 < P.V && (P.V & 3) == 0) {
          *(f32x4*)(lg + v) = acc[j];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (v + e < P.V) lg[v + e] = acc[j][e];
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (v + e < P.V) {
          const unsigned long long k = pack_max(acc[j][e], v + e);
          best = k > best ? k : best;
        }
    }
    best = xmax_u64<16>(best);
    best = xmax_u64<32>(best);
    if (g4 == 0 && seq < P.B && best)
      __hip_atomic_fetch_max(&P.argmax[(size_t)seq * kArgmaxShards + (T.r1 * kPWaves + w) % kArgmaxShards], best,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The first generated token: the shards' maximum per sequence (and the shards
// cleared for the next prefill), seq_len = prompt length.
__device__ void argmax_tile(const PParams& P, int tid) {
  if (tid >= 64) return;
  const int lane = tid;
  constexpr int SEQS = 64 / kArgmaxShards;
  for (int b0 = 0; b0 < P.B; b0 += SEQS) {
    const int b = b0 + lane / kArgmaxShards;
    unsigned long long best = 0;
    if (b < P.B)
      best = __hip_atomic_exchange(&P.argmax[(size_t)b0 * kArgmaxShards + lane], 0ull, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    best = group_max_u64<kArgmaxShards>(best);
    if (b < P.B && lane % kArgmaxShards == 0) {
      st_sc1(&P.tokens_out[b], (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull)));
      st_sc1(&P.seq_len[b], P.P);
    }
  }
}

__device__ __forceinline__ void run_tile(const PParams& P, const Tile& T, PSmem& sm, int tid) {
  switch (T.type) {
    case P_EMBED:
    case P_NORM1:
    case P_NORM2: norm_tile(P, T, sm, tid); break;
    case P_QKV: gemm_tile<false>(P, T, sm, tid); break;
    case P_OPROJ:
    case P_GATEUP:
    case P_DOWN: gemm_tile<true>(P, T, sm, tid); break;
    case P_ATTN: attn_tile(P, T, sm, tid); break;
    case P_NORMF: normf_tile(P, T, tid); break;
    case P_LM: lm_tile(P, T, tid); break;
    default: argmax_tile(P, tid); break;
  }
}

}  // namespace

// The persistent prefill: each worker claims from its queue in topological
// order (the next claim in flight while a tile runs), waits for the tile's
// group, runs it with all eight waves, waits for its stores and publishes.
// The last worker out rewinds the queues and advances the epoch.
template <bool LOG>
__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(2))) void prefill_megakernel(PParams P) {
  __shared__ PSmem sm;
  const int tid = wpk_tid(), lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = cload(P.worker_queue, (int)blockIdx.x);
  const int qb = cload(P.queue_off, q), qn = cload(P.queue_off, q + 1) - qb;
  uint32_t* head = P.heads + (size_t)q * kLine;
  const uint32_t epoch = ld_sc1(&P.ctl[CTL_EPOCH]);
  if (tid == 0) {
    sm.claim[0] = ld_sc1(&P.ctl[CTL_STATUS]) != 0u ? qn : (int)atomic_add(head, 1u);
    sm.stop = 0;
  }
  __syncthreads();
  int cur = __builtin_amdgcn_readfirstlane(sm.claim[0]);
  // a group wave 0 has seen complete (groups never un-complete within a
  // launch): consecutive tiles of a queue mostly wait on the same row block's
  // group, and each poll is a memory round trip (logged runs poll every tile:
  // the log records the counter each start saw)
  int done_group = -1;
  for (int it = 0; cur < qn; ++it) {
    const Tile T = uni(cload(P.qtiles, qb + cur));
    if (tid == 0) sm.claim[(it + 1) & 1] = (int)atomic_add(head, 1u);
    int32_t delta = 0;
    if (wave == 0 && T.wait >= 0 && (LOG || T.wait != done_group)) {
      if (p_wait(P, T, epoch, &delta, lane)) done_group = T.wait;
      else if (lane == 0) sm.stop = 1;
    }
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(sm.stop)) break;
    const uint64_t t_start = LOG ? __builtin_amdgcn_s_memrealtime() : 0;
    // the thread index made opaque per tile: the tile bodies' per-lane address
    // arithmetic is then not hoisted out of the loop and kept live across it
    run_tile(P, T, sm, opaque(tid));
    wait_all_memory();
    __syncthreads();
    if (tid == 0) {
      if (LOG) {
        int32_t* rec = P.log + (size_t)T.id * 8;
        __hip_atomic_fetch_add(rec, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        rec[1] = delta;
        rec[2] = (int32_t)blockIdx.x;
        rec[3] = cur;
        *(uint64_t*)(rec + 4) = t_start;
        *(uint64_t*)(rec + 6) = __builtin_amdgcn_s_memrealtime();
        wait_all_memory();
      }
      if (T.signal >= 0) {
        const Group G = cload(P.groups, T.signal);
        atomic_add(&P.counters[(size_t)(G.shard0 + T.shard) * kLine], 1u);
      }
    }
    cur = __builtin_amdgcn_readfirstlane(sm.claim[(it + 1) & 1]);
  }
  __syncthreads();
  if (tid == 0) {
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
__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(2))) void prefill_phase(PParams P,
                                                                                                      int first) {
  __shared__ PSmem sm;
  const Tile T = uni(cload(P.tiles, first + (int)blockIdx.x));
  run_tile(P, T, sm, wpk_tid());
}

}  // namespace wpk

namespace wpk {
// Repacks a row-major bf16 matrix [rows][K] (rows a multiple of 16, K of 32)
// into the packed fragment-major layout the matrix-core tiles load: one
// thread per 16-byte chunk.  to_f16: the values converted to fp16 (exact for
// bf16 magnitudes in [2^-14, 65504]; smaller ones become fp16 subnormals,
// within 2^-25 of the value), and *flag set if one is beyond the fp16 range.
__global__ __launch_bounds__(256) void prefill_pack(const uint16_t* src, uint16_t* dst, int rows, int K, int to_f16,
                                                    int* flag) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t per_row = (size_t)K / 8;
  if (i >= (size_t)rows * per_row) return;
  const uint32_t r = (uint32_t)(i / per_row), k = (uint32_t)(i % per_row) * 8u;
  u32x4 v = *(const u32x4*)(src + i * 8);
  if (to_f16) {
    bool over = false;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = cvt_f16x2(bf16_lo(w[e]), bf16_hi(w[e]), over);
    v = u32x4{o[0], o[1], o[2], o[3]};
    if (over) __hip_atomic_fetch_or(flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  *(u32x4*)((char*)dst + pk(r, k, (uint32_t)K)) = v;
}
}  // namespace wpk

// Launches the repacking of one matrix on `stream` (asynchronous).
extern "C" int wpk_dev_prefill_pack(const void* src, void* dst, int rows, int K, int to_f16, int* flag, void* stream) {
  const size_t chunks = (size_t)rows * (size_t)K / 8;
  const unsigned grid = (unsigned)((chunks + 255) / 256);
  hipLaunchKernelGGL(wpk::prefill_pack, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const uint16_t*)src,
                     (uint16_t*)dst, rows, K, to_f16, flag);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int wpk_dev_prefill_kernels(const void** mk, const void** mk_log, const void** phase) {
  *mk = reinterpret_cast<const void*>(&wpk::prefill_megakernel<false>);
  *mk_log = reinterpret_cast<const void*>(&wpk::prefill_megakernel<true>);
  *phase = reinterpret_cast<const void*>(&wpk::prefill_phase);
  return 1;
}
