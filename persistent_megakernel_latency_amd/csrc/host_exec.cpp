// host_exec.cpp -- the tile DAG run on the CPU.
//
// Two executors share one set of CPU tile bodies (float32, sequential sums):
//  * the serial executor runs tiles one at a time in a topological order drawn
//    at random (Kahn's algorithm with a seeded tie-break).  Any valid order
//    must give bit-identical results, and with NaN-poisoned intermediates a
//    tile that runs before one of its producers poisons the logits;
//  * the emulator runs the device protocol itself -- claim from the sharded
//    queues in topological order, poll a counter group, publish with one
//    increment -- on std::threads with random delays.  The orderings are the
//    device's, written in the C++ memory model: the device publishes with a
//    relaxed atomic after waiting for its own stores to complete and reads its
//    inputs after the poll that saw them complete, so here a release fence
//    precedes each relaxed publish and an acquire fence follows each satisfied
//    relaxed poll.  ThreadSanitizer does not model standalone fences, so a
//    build with WPK_TSAN_ORDERINGS folds each fence into its atomic (release
//    increment, acquire poll loads: the same happens-before edges), which lets
//    a sanitizer build of the emulator check every data access the protocol is
//    meant to order.
// The "final participant publishes" and phase-barrier logic of the WPK design
// ("Why real-time inference wants a megakernel", one WPK update) is replaced
// here, as on the device, by counter groups released per tile.
#include "host_exec.h"

#include <atomic>
#include <chrono>
#include <cmath>
#include <cstring>
#include <limits>
#include <thread>

namespace wpk {

// ---- shared layout helpers ---------------------------------------------------------

void rope_table(const Shape& s, std::vector<float>& cos_t, std::vector<float>& sin_t) {
  const int half = s.D / 2;
  cos_t.resize((size_t)s.cap * half);
  sin_t.resize((size_t)s.cap * half);
  for (int p = 0; p < s.cap; ++p)
    for (int i = 0; i < half; ++i) {
      const double ang = (double)p * std::pow((double)s.theta, -2.0 * i / s.D);
      cos_t[(size_t)p * half + i] = (float)std::cos(ang);
      sin_t[(size_t)p * half + i] = (float)std::sin(ang);
    }
}

ActLayout act_layout(const Shape& s) {
  ActLayout a{};
  auto r64 = [](int64_t x) { return (x + 63) & ~(int64_t)63; };  // 256-byte aligned
  int64_t at = 0;
  a.x_mid = at; at += r64((int64_t)s.B * s.H);
  a.x_out = at; at += r64((int64_t)s.B * s.H);
  a.q = at;     at += r64((int64_t)s.B * s.Hq * s.D);
  a.part = at;  at += r64((int64_t)s.B * s.Hkv * s.nch * s.G * (s.D + 2));
  a.attn = at;  at += r64((int64_t)s.B * s.Hq * s.D);
  a.h = at;     at += r64((int64_t)s.B * s.F);
  // wide operands: bf16 hi/lo planes [2][32][K] take 32 * K floats; rows past the batch stay zero
  const int64_t wb = s.wide ? (int64_t)kMaxBatch : 0;  // two bf16 planes of 32 rows
  a.xn1 = at;   at += r64(wb * s.H);
  a.xattn = at; at += r64(wb * s.Hq * s.D);
  a.xn2 = at;   at += r64(wb * s.H);
  a.xh = at;    at += r64(wb * s.F);
  a.xnf = at;   at += r64(wb * s.H);
  // wide plans: per 64-row block and sequence, the sum of squares of the
  // RMSNorm input rows (attention input, MLP input, final)
  const int64_t ssz = s.wide ? (int64_t)(s.H / kWideRows) * kMaxBatch : 0;
  a.ss1 = at;   at += r64(ssz);
  a.ss2 = at;   at += r64(ssz);
  a.ssf = at;   at += r64(ssz);
  a.per_layer = at;
  a.total = at * s.L;
  return a;
}

void fill_layers(const Shape& s, const wpk_model_desc& d, float* act, std::vector<LayerBufs>& out) {
  const ActLayout a = act_layout(s);
  out.resize(s.L);
  for (int l = 0; l < s.L; ++l) {
    float* base = act + a.per_layer * l;
    LayerBufs& lb = out[l];
    lb.w_qkv = d.w_qkv[l];
    lb.w_o = d.w_o[l];
    lb.w_gate = d.w_gate[l];
    lb.w_up = d.w_up[l];
    lb.w_down = d.w_down[l];
    lb.attn_norm = d.attn_norm[l];
    lb.mlp_norm = d.mlp_norm[l];
    lb.x_mid = base + a.x_mid;
    lb.x_out = base + a.x_out;
    lb.q = base + a.q;
    lb.part = base + a.part;
    lb.attn = base + a.attn;
    lb.h = base + a.h;
    lb.xn1 = (uint16_t*)(base + a.xn1);
    lb.xattn = (uint16_t*)(base + a.xattn);
    lb.xn2 = (uint16_t*)(base + a.xn2);
    lb.xh = (uint16_t*)(base + a.xh);
    lb.xnf = (uint16_t*)(base + a.xnf);
    lb.x_in = l == 0 ? nullptr : out[l - 1].x_out;
    lb.final_norm = (const float*)d.final_norm;
    lb.ss1 = base + a.ss1;
    lb.ss2 = base + a.ss2;
    lb.ssf = base + a.ssf;
  }
}

// ---- CPU tile bodies ----------------------------------------------------------------

namespace {

inline float wval(const void* w, int32_t dtype, int64_t i) {
  if (dtype == WPK_BF16) {
    const uint32_t u = (uint32_t)((const uint16_t*)w)[i] << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
  }
  return ((const float*)w)[i];
}

inline uint16_t to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

inline void cache_put(char* base, int32_t dtype, int64_t i, float v) {
  if (dtype == WPK_BF16) ((uint16_t*)base)[i] = to_bf16(v);
  else ((float*)base)[i] = v;
}

inline float bf16v(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Stores v as the hi/lo bf16 pair of a wide operand buffer [2][32][K].
inline void xput(uint16_t* x, int K, int b, int i, float v) {
  const int64_t at = (int64_t)b * K + i;
  const uint16_t hi = to_bf16(v);
  x[at] = hi;
  x[(int64_t)kMaxBatch * K + at] = to_bf16(v - bf16v(hi));
}

// Greedy choice key, as on the device: float order, then the lowest index;
// -0 counts as +0 and a NaN is never chosen.
inline uint64_t pack_max(float v, int32_t idx) {
  uint32_t u;
  std::memcpy(&u, &v, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0;
  if (u == 0x80000000u) u = 0u;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)idx);
}

struct Ctx {
  const Params& P;
  std::atomic<unsigned long long>* argmax;
  std::atomic<int32_t>* status;
  int64_t wpart_len = 0;   // floats of the partial-sum slots (bounds of every access)
  int64_t fixc_len = 0;    // words of the arrival counters
  bool fixed_reducer = false;         // emulator option, wide plans (see run_gemv)
  const std::atomic<int32_t>* abort = nullptr;
};

// The device protocol's orderings (see the file comment).
inline void publish_fence() {
#ifndef WPK_TSAN_ORDERINGS
  std::atomic_thread_fence(std::memory_order_release);
#endif
}
inline void acquire_fence() {
#ifndef WPK_TSAN_ORDERINGS
  std::atomic_thread_fence(std::memory_order_acquire);
#endif
}
#ifdef WPK_TSAN_ORDERINGS
constexpr std::memory_order kPublishOrder = std::memory_order_release;
constexpr std::memory_order kPollOrder = std::memory_order_acquire;
constexpr int kPublishOrderB = __ATOMIC_RELEASE, kPollOrderB = __ATOMIC_ACQUIRE, kArriveOrder = __ATOMIC_ACQ_REL;
#else
constexpr std::memory_order kPublishOrder = std::memory_order_relaxed;
constexpr std::memory_order kPollOrder = std::memory_order_relaxed;
constexpr int kPublishOrderB = __ATOMIC_RELAXED, kPollOrderB = __ATOMIC_RELAXED, kArriveOrder = __ATOMIC_RELAXED;
#endif

void set_status(Ctx& c, int32_t code) {
  int32_t z = 0;
  c.status->compare_exchange_strong(z, code);
}

int32_t token_of(Ctx& c, int b) {
  const int32_t t = c.P.tokens[b];
  if (c.P.seq_len[b] >= 0 && (t < 0 || t >= c.P.V)) {
    set_status(c, WPK_E_TOKEN);
    return 0;
  }
  return (t < 0 || t >= c.P.V) ? 0 : t;
}

// A wide operand element: the hi and lo bf16 planes of a [2][32][K] buffer.
inline float xget(const uint16_t* x, int K, int b, int i) {
  const int64_t at = (int64_t)b * K + i;
  return bf16v(x[at]) + bf16v(x[(int64_t)kMaxBatch * K + at]);
}

// Wide plans: the RMSNorm split between the tile that produces a 64-row
// block of x (it writes gain * x as the bf16 operand and the block's sum of
// squares) and the tile that consumes the operand (its epilogue divides by
// the root mean square, read from all blocks' sums in block order).
void put_norm_rows(const Params& P, uint16_t* plane, float* ss, const float* gain, int b, int64_t r0,
                   const float* x) {
  float sq = 0.f;
  for (int r = 0; r < kWideRows; ++r) {
    xput(plane, P.H, b, (int)(r0 + r), gain[r0 + r] * x[r]);
    sq += x[r] * x[r];
  }
  ss[(r0 / kWideRows) * kMaxBatch + b] = sq;
}

float inv_rms(const Params& P, const float* ss, int b) {
  float sum = 0.f;
  for (int rb = 0; rb < P.H / kWideRows; ++rb) sum += ss[rb * kMaxBatch + b];
  return 1.0f / std::sqrt(sum / (float)P.H + P.eps);
}

// Input vector of a GEMV tile for sequence b, with its RMSNorm prologue.  In
// a wide plan it is the operand row (gain * x for the normalised inputs) the
// producing tile wrote; the consumer's epilogue divides by the root mean square.
void gemv_input(Ctx& c, const Tile& T, int b, std::vector<float>& x) {
  const Params& P = c.P;
  const LayerBufs& lb = P.layers[T.layer];
  if (P.wide) {
    const uint16_t* src = nullptr;
    int K = P.H;
    switch (T.type) {
      case T_QKV: src = lb.xn1; break;
      case T_OPROJ: src = lb.xattn; break;
      case T_GATEUP: src = lb.xn2; break;
      case T_DOWN: src = lb.xh; K = P.F; break;
      default: src = P.layers[P.L - 1].xnf; break;
    }
    // only this tile's K slice: it waits for the tiles producing those
    // columns and no others, so the rest of the row may still be being written
    x.assign(K, 0.f);
    const int k0 = T.c * kWideK, k1 = std::min(K, k0 + kWideK);
    for (int i = k0; i < k1; ++i) x[i] = xget(src, K, b, i);
    return;
  }
  const float* gain = nullptr;
  int K = P.H;
  switch (T.type) {
    case T_QKV:
      gain = lb.attn_norm;
      if (T.layer == 0) {
        const int64_t tok = token_of(c, b);
        x.resize(P.H);
        for (int i = 0; i < P.H; ++i) x[i] = wval(P.embed, P.dtype, tok * P.H + i);
      } else {
        x.assign(lb.x_in + (int64_t)b * P.H, lb.x_in + (int64_t)(b + 1) * P.H);
      }
      break;
    case T_OPROJ:
      x.assign(lb.attn + (int64_t)b * P.H, lb.attn + (int64_t)(b + 1) * P.H);
      break;
    case T_GATEUP:
      gain = lb.mlp_norm;
      x.assign(lb.x_mid + (int64_t)b * P.H, lb.x_mid + (int64_t)(b + 1) * P.H);
      break;
    case T_DOWN:
      K = P.F;
      x.assign(lb.h + (int64_t)b * P.F, lb.h + (int64_t)(b + 1) * P.F);
      break;
    case T_LM: {
      gain = P.final_norm;
      const float* xo = P.layers[P.L - 1].x_out;
      x.assign(xo + (int64_t)b * P.H, xo + (int64_t)(b + 1) * P.H);
      break;
    }
  }
  if (gain) {
    float ss = 0.f;
    for (int i = 0; i < K; ++i) ss += x[i] * x[i];
    const float inv = 1.0f / std::sqrt(ss / (float)K + P.eps);
    for (int i = 0; i < K; ++i) x[i] = x[i] * inv * gain[i];
  }
}

void run_gemv(Ctx& c, const Tile& T) {
  const Params& P = c.P;
  const LayerBufs& lb = P.layers[T.layer];
  const void* w0;
  const void* w1;
  int K = P.H, limit;
  switch (T.type) {
    case T_QKV: w0 = w1 = lb.w_qkv; limit = P.qkv_rows; break;
    case T_OPROJ: w0 = w1 = lb.w_o; limit = P.H; break;
    case T_GATEUP: w0 = lb.w_gate; w1 = lb.w_up; limit = P.F; break;
    case T_DOWN: w0 = w1 = lb.w_down; K = P.F; limit = P.H; break;
    default: w0 = w1 = P.embed; limit = P.V; break;
  }
  std::vector<float> x, y(T.rows);
  // wide plans: this tile's K slice; its partial sums go to its slot, and the
  // row block's last slice adds all slots in slice order
  const int k0 = P.wide ? T.c * kWideK : 0, k1 = P.wide ? k0 + kWideK : K;
  // partial sums of slice `slice`, bounds-checked against the slot area
  float dummy = 0.f;
  auto part = [&](int slice, int r, int b) -> float& {
    const int64_t i = (int64_t)(T.pslot + slice) * kWidePart + ((b / 16) * kWideRows + r) * 16 + b % 16;
    if (slice < 0 || slice >= T.b || r < 0 || r >= kWideRows || b < 0 || b >= kMaxBatch || i < 0 ||
        i >= c.wpart_len) {
      set_status(c, WPK_E_ARG);
      return dummy;
    }
    return P.wpart[i];
  };
  if (P.wide) {
    for (int b = 0; b < P.B; ++b) {
      gemv_input(c, T, b, x);
      for (int r = 0; r < T.rows; ++r) {
        const bool seg1 = r >= T.rs;
        const int64_t mrow = std::min<int64_t>(seg1 ? T.r1 + (r - T.rs) : T.r0 + r, limit - 1);
        const void* w = seg1 ? w1 : w0;
        float acc = 0.f;
        for (int k = k0; k < k1; ++k) acc += wval(w, P.dtype, mrow * K + k) * x[k];
        part(T.c, r, b) = acc;
      }
    }
    const int64_t fi = (int64_t)T.fix * kLine;
    if (fi < 0 || fi >= c.fixc_len || T.c < 0 || T.c >= T.b) {
      set_status(c, WPK_E_ARG);
      return;
    }
    uint32_t* arrivals = &P.fixc[fi];
    if (!c.fixed_reducer) {
      // the last slice to arrive adds up the row block (the device's scheme)
      publish_fence();
      const uint32_t old = __atomic_fetch_add(arrivals, 1u, kArriveOrder);
      if ((int32_t)(old + 1u) != T.b) return;  // not the row block's last slice
      acquire_fence();
    } else if (T.c != T.b - 1) {
      // a fixed reducer, the row block's last slice in claim order: the others
      // only count their arrival and go on (no reply awaited)
      publish_fence();
      __atomic_fetch_add(arrivals, 1u, kPublishOrderB);
      return;
    } else {
      // the reducer waits, bounded, until every other slice has arrived; its
      // siblings precede it in the topological claim order, so the lowest
      // unfinished tile always progresses and the wait ends
      const auto t0 = std::chrono::steady_clock::now();
      while (__atomic_load_n(arrivals, kPollOrderB) != (uint32_t)(T.b - 1)) {
        if ((c.abort && c.abort->load(std::memory_order_relaxed)) ||
            std::chrono::steady_clock::now() - t0 > std::chrono::seconds(20)) {
          set_status(c, WPK_E_TIMEOUT);
          return;
        }
        std::this_thread::yield();
      }
      acquire_fence();
      __atomic_store_n(arrivals, 0u, __ATOMIC_RELAXED);  // no other slice touches it again this step
    }
  }
  for (int b = 0; b < P.B; ++b) {
    const int32_t p = P.seq_len[b];
    if (T.type == T_QKV && p < 0) continue;
    if (P.wide) {
      for (int r = 0; r < T.rows; ++r) {
        float acc = 0.f;
        for (int sl = 0; sl < T.b; ++sl) acc += part(sl, r, b);
        y[r] = acc;
      }
      // the RMSNorm of the operand, divided out here
      const float* ss = T.type == T_QKV ? lb.ss1 : T.type == T_GATEUP ? lb.ss2 : T.type == T_LM ? lb.ssf : nullptr;
      if (ss) {
        const float inv = inv_rms(P, ss, b);
        for (int r = 0; r < T.rows; ++r) y[r] *= inv;
      }
    } else {
      gemv_input(c, T, b, x);
      for (int r = 0; r < T.rows; ++r) {
        const bool seg1 = r >= T.rs;
        const int64_t mrow = seg1 ? T.r1 + (r - T.rs) : T.r0 + r;
        y[r] = 0.f;
        if (mrow >= limit) continue;
        const void* w = seg1 ? w1 : w0;
        float acc = 0.f;
        for (int k = 0; k < K; ++k) acc += wval(w, P.dtype, mrow * K + k) * x[k];
        y[r] = acc;
      }
    }
    switch (T.type) {
      case T_QKV: {
        if (p >= P.cap) {
          set_status(c, WPK_E_CTX_FULL);
          break;
        }
        const int half = P.D / 2;
        if (T.kind < 2) {
          const int head = T.g;
          const int64_t base = T.kind == 0 ? (int64_t)head * P.D : (int64_t)(P.Hq + head) * P.D;
          for (int i = 0; i < T.rs; ++i) {
            const int dim = (int)(T.r0 + i - base);
            const float cs = P.rope_cos[(int64_t)p * half + dim], sn = P.rope_sin[(int64_t)p * half + dim];
            const float a = y[i], bb = y[T.rs + i];
            const float ra = a * cs - bb * sn, rb = bb * cs + a * sn;
            if (T.kind == 0) {
              lb.q[(int64_t)b * P.Hq * P.D + head * P.D + dim] = ra;
              lb.q[(int64_t)b * P.Hq * P.D + head * P.D + dim + half] = rb;
            } else {
              const int64_t at = ((((int64_t)T.layer * P.B + b) * P.Hkv + head) * P.cap + p) * P.D;
              cache_put(P.kc, P.dtype, at + dim, ra);
              cache_put(P.kc, P.dtype, at + dim + half, rb);
            }
          }
        } else {
          const int64_t base = (int64_t)(P.Hq + P.Hkv + T.g) * P.D;
          const int64_t at = ((((int64_t)T.layer * P.B + b) * P.Hkv + T.g) * P.cap + p) * P.D;
          for (int r = 0; r < T.rows; ++r) {
            const int64_t mrow = r < T.rs ? T.r0 + r : T.r1 + (r - T.rs);
            cache_put(P.vc, P.dtype, at + (mrow - base), y[r]);
          }
        }
        break;
      }
      case T_OPROJ:
        for (int r = 0; r < T.rows; ++r) {
          const int64_t row = T.r0 + r;
          if (row >= P.H) continue;
          float xin;
          if (T.layer == 0) xin = wval(P.embed, P.dtype, (int64_t)token_of(c, b) * P.H + row);
          else xin = lb.x_in[(int64_t)b * P.H + row];
          lb.x_mid[(int64_t)b * P.H + row] = xin + y[r];
        }
        if (P.wide) put_norm_rows(P, lb.xn2, lb.ss2, lb.mlp_norm, b, T.r0, lb.x_mid + (int64_t)b * P.H + T.r0);
        break;
      case T_GATEUP:
        for (int i = 0; i < T.rs; ++i) {
          const int64_t j = T.r0 + i;
          if (j >= P.F) continue;
          const float g = y[i], u = y[T.rs + i];
          const float hv = g / (1.0f + std::exp(-g)) * u;
          if (P.wide) xput(lb.xh, P.F, b, j, hv);
          else lb.h[(int64_t)b * P.F + j] = hv;
        }
        break;
      case T_DOWN:
        for (int r = 0; r < T.rows; ++r) {
          const int64_t row = T.r0 + r;
          if (row >= P.H) continue;
          lb.x_out[(int64_t)b * P.H + row] = lb.x_mid[(int64_t)b * P.H + row] + y[r];
        }
        if (P.wide) {  // the next layer's attention input, or the final norm's
          const float* xo = lb.x_out + (int64_t)b * P.H + T.r0;
          if (T.layer + 1 < P.L) {
            const LayerBufs& nx = P.layers[T.layer + 1];
            put_norm_rows(P, nx.xn1, nx.ss1, nx.attn_norm, b, T.r0, xo);
          } else {
            put_norm_rows(P, lb.xnf, lb.ssf, P.final_norm, b, T.r0, xo);
          }
        }
        break;
      case T_LM: {
        uint64_t best = 0;
        for (int r = 0; r < T.rows; ++r) {
          const int64_t row = T.r0 + r;
          if (row >= P.V) continue;
          P.logits[(int64_t)b * P.V + row] = y[r];
          const uint64_t k = pack_max(y[r], (int32_t)row);
          if (k > best) best = k;
        }
        std::atomic<unsigned long long>& slot = c.argmax[b * kArgmaxShards + T.id % kArgmaxShards];
        unsigned long long cur = slot.load(std::memory_order_relaxed);
        while (best > cur && !slot.compare_exchange_weak(cur, best, std::memory_order_relaxed)) {
        }
        break;
      }
    }
  }
}

// The partial (m, l, o[D]) of each q head of the group over one KV chunk,
// into out[G][D+2]; false if the chunk holds no position of the sequence.
bool attn_partial(Ctx& c, const Tile& T, int chunk, float* out) {
  const Params& P = c.P;
  const LayerBufs& lb = P.layers[T.layer];
  const int32_t p = P.seq_len[T.b];
  const int n = p < 0 ? 0 : std::min(p + 1, P.cap);
  const int start = chunk * kAttnChunk;
  const int cnt = std::max(0, std::min(kAttnChunk, n - start));
  if (cnt == 0) return false;
  const int64_t slice = (((int64_t)T.layer * P.B + T.b) * P.Hkv + T.g) * P.cap;
  for (int h = 0; h < P.G; ++h) {
    float* o_h = out + h * (P.D + 2);
    const float* q = lb.q + (int64_t)T.b * P.Hq * P.D + (int64_t)(T.g * P.G + h) * P.D;
    float s[kAttnChunk];
    float m = -std::numeric_limits<float>::infinity();
    for (int j = 0; j < cnt; ++j) {
      float dot = 0.f;
      for (int d = 0; d < P.D; ++d) dot += q[d] * wval(P.kc, P.dtype, (slice + start + j) * P.D + d);
      s[j] = dot * P.attn_scale;
      m = std::max(m, s[j]);
    }
    float l = 0.f;
    for (int j = 0; j < cnt; ++j) {
      s[j] = std::exp(s[j] - m);
      l += s[j];
    }
    o_h[0] = m;
    o_h[1] = l;
    for (int d = 0; d < P.D; ++d) {
      float o = 0.f;
      for (int j = 0; j < cnt; ++j) o += s[j] * wval(P.vc, P.dtype, (slice + start + j) * P.D + d);
      o_h[2 + d] = o;
    }
  }
  return true;
}

// Running merge of partials: acc = merge(acc, part), both [G][D+2]; acc starts
// with m = -inf, l = 0, o = 0.
void merge_partial(const Params& P, float* acc, const float* part) {
  for (int h = 0; h < P.G; ++h) {
    float* a = acc + h * (P.D + 2);
    const float* b = part + h * (P.D + 2);
    const float M = std::max(a[0], b[0]);
    const float ka = std::exp(a[0] - M), kb = std::exp(b[0] - M);
    a[1] = a[1] * ka + b[1] * kb;
    for (int d = 0; d < P.D; ++d) a[2 + d] = a[2 + d] * ka + b[2 + d] * kb;
    a[0] = M;
  }
}

void init_partial(const Params& P, std::vector<float>& acc) {
  acc.assign((size_t)P.G * (P.D + 2), 0.f);
  for (int h = 0; h < P.G; ++h) acc[(size_t)h * (P.D + 2)] = -std::numeric_limits<float>::infinity();
}

// An attention tile covers T.kind consecutive KV chunks; their partials are
// merged on chip into one, stored at partial slot T.c / attn_sub (a tile past
// its sequence stores nothing: the combine never reads that slot).
void run_attn(Ctx& c, const Tile& T) {
  const Params& P = c.P;
  const LayerBufs& lb = P.layers[T.layer];
  std::vector<float> acc, part((size_t)P.G * (P.D + 2));
  init_partial(P, acc);
  bool any = false;
  for (int u = 0; u < std::max(1, T.kind); ++u)
    if (attn_partial(c, T, T.c + u, part.data())) {
      merge_partial(P, acc.data(), part.data());
      any = true;
    }
  if (!any) return;
  float* out = lb.part + (((int64_t)T.b * P.Hkv + T.g) * P.nch + T.c / P.attn_sub) * P.G * (P.D + 2);
  std::copy(acc.begin(), acc.end(), out);
}

// A chained attention tile (LDS forwarding): every chunk's partial merged in
// turn, then normalised into the attention output.
void run_attnc(Ctx& c, const Tile& T) {
  const Params& P = c.P;
  const LayerBufs& lb = P.layers[T.layer];
  std::vector<float> acc, part((size_t)P.G * (P.D + 2));
  init_partial(P, acc);
  bool any = false;
  for (int ch = 0; ch < P.nch; ++ch)
    if (attn_partial(c, T, ch, part.data())) {
      merge_partial(P, acc.data(), part.data());
      any = true;
    }
  for (int h = 0; h < P.G; ++h) {
    const float* a = acc.data() + h * (P.D + 2);
    for (int d = 0; d < P.D; ++d) {
      const float v = any ? a[2 + d] / a[1] : 0.f;
      const int64_t col = (int64_t)(T.g * P.G + h) * P.D + d;
      if (P.wide) xput(lb.xattn, P.Hq * P.D, T.b, (int)col, v);
      else lb.attn[(int64_t)T.b * P.Hq * P.D + col] = v;
    }
  }
}

void run_combine(Ctx& c, const Tile& T) {
  const Params& P = c.P;
  const LayerBufs& lb = P.layers[T.layer];
  const int32_t p = P.seq_len[T.b];
  const int n = p < 0 ? 0 : std::min(p + 1, P.cap);
  // one partial per attention tile: the tiles holding positions
  const int nact = ((n + kAttnChunk - 1) / kAttnChunk + P.attn_sub - 1) / P.attn_sub;
  for (int h = 0; h < P.G; ++h) {
    const int64_t at = (int64_t)T.b * P.Hq * P.D + (int64_t)(T.g * P.G + h) * P.D;
    float* dst = lb.attn + at;
    auto put = [&](int d, float v) {
      if (P.wide) xput(lb.xattn, P.Hq * P.D, T.b, (T.g * P.G + h) * P.D + d, v);  // the o-proj operand
      else dst[d] = v;
    };
    if (nact == 0) {
      for (int d = 0; d < P.D; ++d) put(d, 0.f);
      continue;
    }
    auto part = [&](int ch) {
      return lb.part + ((((int64_t)T.b * P.Hkv + T.g) * P.nch + ch) * P.G + h) * (P.D + 2);
    };
    float M = -std::numeric_limits<float>::infinity();
    for (int ch = 0; ch < nact; ++ch) M = std::max(M, part(ch)[0]);
    float L = 0.f;
    for (int ch = 0; ch < nact; ++ch) L += part(ch)[1] * std::exp(part(ch)[0] - M);
    for (int d = 0; d < P.D; ++d) {
      float o = 0.f;
      for (int ch = 0; ch < nact; ++ch) o += part(ch)[2 + d] * std::exp(part(ch)[0] - M);
      put(d, o / L);
    }
  }
}

void run_argmax(Ctx& c) {
  const Params& P = c.P;
  for (int b = 0; b < P.B; ++b) {
    unsigned long long best = 0;
    for (int s = 0; s < kArgmaxShards; ++s) {
      best = std::max(best, (unsigned long long)c.argmax[b * kArgmaxShards + s].load(std::memory_order_relaxed));
      c.argmax[b * kArgmaxShards + s].store(0, std::memory_order_relaxed);
    }
    const int32_t p = P.seq_len[b];
    if (p < 0 || p >= P.cap) continue;
    P.tokens[b] = (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
    P.seq_len[b] = p + 1;
  }
}

// Wide plans, layer 0: one sequence's embedding row as the first QKV operand.
void run_norm(Ctx& c, const Tile& T) {
  const Params& P = c.P;
  const LayerBufs& lb = P.layers[0];
  const int b = T.b, K = P.H;
  const int64_t tok = token_of(c, b);
  std::vector<float> x(kWideRows);
  for (int r0 = 0; r0 < K; r0 += kWideRows) {
    for (int r = 0; r < kWideRows; ++r) x[r] = wval(P.embed, P.dtype, tok * K + r0 + r);
    put_norm_rows(P, lb.xn1, lb.ss1, lb.attn_norm, b, r0, x.data());
  }
}

void run_tile(Ctx& c, const Tile& T) {
  switch (T.type) {
    case T_NORM: run_norm(c, T); break;
    case T_ATTN: run_attn(c, T); break;
    case T_COMBINE: run_combine(c, T); break;
    case T_ATTNC: run_attnc(c, T); break;
    case T_ARGMAX: run_argmax(c); break;
    default: run_gemv(c, T); break;
  }
}

Params host_params(wpk_plan* p, int32_t* tokens, wpk_kv* kv, float* logits) {
  const Shape& s = p->s;
  Params P{};
  P.L = s.L; P.H = s.H; P.Hq = s.Hq; P.Hkv = s.Hkv; P.D = s.D; P.F = s.F; P.V = s.V;
  P.B = s.B; P.cap = s.cap; P.nch = s.nch; P.G = s.G; P.qkv_rows = s.qkv_rows;
  P.attn_sub = s.attn_sub;
  P.n_tiles = (int32_t)p->dag.tiles.size();
  P.dtype = s.dtype;
  P.eps = s.eps;
  P.attn_scale = 1.0f / std::sqrt((float)s.D);
  P.embed = p->desc.embed;
  P.final_norm = p->desc.final_norm;
  P.layers = p->hw.layers.data();
  const ActLayout a = act_layout(s);
  P.act = p->hw.act.data();
  P.act_layer = a.per_layer;
  P.off_x_mid = (int32_t)a.x_mid;
  P.off_x_out = (int32_t)a.x_out;
  P.off_q = (int32_t)a.q;
  P.off_part = (int32_t)a.part;
  P.off_attn = (int32_t)a.attn;
  P.off_h = (int32_t)a.h;
  P.wide = s.wide;
  P.off_xn1 = (int32_t)a.xn1;
  P.off_xattn = (int32_t)a.xattn;
  P.off_xn2 = (int32_t)a.xn2;
  P.off_xh = (int32_t)a.xh;
  P.off_xnf = (int32_t)a.xnf;
  P.wpart = p->hw.wpart.data();
  P.fixc = p->hw.fixc.data();
  P.rope_cos = p->hw.rope_cos.data();
  P.rope_sin = p->hw.rope_sin.data();
  P.tokens = tokens;
  P.seq_len = kv->seq_len;
  P.logits = logits;
  P.kc = (char*)kv->k;
  P.vc = (char*)kv->v;
  P.tiles = p->dag.tiles.data();
  P.groups = p->dag.groups.data();
  return P;
}

void poison(wpk_plan* p, const Params& P) {
  const float nan = std::numeric_limits<float>::quiet_NaN();
  // a float NaN whose two halves are bf16 NaNs too, for the bf16 operand rows
  const uint32_t nan2 = 0x7FC07FC0u;
  float nanw;
  std::memcpy(&nanw, &nan2, 4);
  std::fill(p->hw.act.begin(), p->hw.act.end(), nanw);
  std::fill(p->hw.wpart.begin(), p->hw.wpart.end(), nan);
  std::fill(P.logits, P.logits + (int64_t)P.B * P.V, nan);
  // the slot each active sequence is about to append: a read of it before the
  // tile that writes it sees NaN
  for (int b = 0; b < P.B; ++b) {
    const int32_t pos = P.seq_len[b];
    if (pos < 0 || pos >= P.cap) continue;
    for (int l = 0; l < P.L; ++l)
      for (int g = 0; g < P.Hkv; ++g) {
        const int64_t at = ((((int64_t)l * P.B + b) * P.Hkv + g) * P.cap + pos) * P.D;
        for (int d = 0; d < P.D; ++d) {
          cache_put(P.kc, P.dtype, at + d, nan);
          cache_put(P.vc, P.dtype, at + d, nan);
        }
      }
  }
}

uint64_t mix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ULL;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

bool args_ok(wpk_plan* p, int32_t* tokens, wpk_kv* kv, float* logits) {
  if (!p || !p->host) return false;
  if (!tokens || !kv || !kv->k || !kv->v || !kv->seq_len || !logits) {
    p->err = "null argument";
    return false;
  }
  return true;
}

}  // namespace

wpk_plan* make_host_plan(const wpk_model_desc& d, int32_t batch, int32_t ctx_len, const wpk_build_opts& o,
                         std::string* err) {
  Shape s;
  std::string e = check_shape(d, batch, ctx_len, o, &s);
  if (!e.empty()) {
    *err = e;
    return nullptr;
  }
  std::unique_ptr<wpk_plan> p(new wpk_plan());
  p->host = true;
  p->s = s;
  p->desc = d;
  // keep our own copy of the per-layer pointer tables
  p->tables.resize(7 * (size_t)s.L);
  const void* const* src[7] = {(const void* const*)d.attn_norm, d.w_qkv, d.w_o, (const void* const*)d.mlp_norm,
                               d.w_gate, d.w_up, d.w_down};
  for (int k = 0; k < 7; ++k)
    for (int l = 0; l < s.L; ++l) p->tables[(size_t)k * s.L + l] = src[k][l];
  p->desc.attn_norm = (const float* const*)&p->tables[0];
  p->desc.w_qkv = &p->tables[(size_t)1 * s.L];
  p->desc.w_o = &p->tables[(size_t)2 * s.L];
  p->desc.mlp_norm = (const float* const*)&p->tables[(size_t)3 * s.L];
  p->desc.w_gate = &p->tables[(size_t)4 * s.L];
  p->desc.w_up = &p->tables[(size_t)5 * s.L];
  p->desc.w_down = &p->tables[(size_t)6 * s.L];
  p->dag = build_dag(s);
  e = validate_dag(s, p->dag);
  if (!e.empty()) {
    *err = "invalid DAG: " + e;
    return nullptr;
  }
  for (const Tile& t : p->dag.tiles) p->built_wait.push_back(t.wait);
  p->weight_bytes = step_weight_bytes(s);
  const ActLayout a = act_layout(s);
  p->hw.act.assign((size_t)a.total, 0.f);
  fill_layers(s, p->desc, p->hw.act.data(), p->hw.layers);
  p->hw.wpart.assign((size_t)p->dag.n_pslots * kWidePart, 0.f);
  p->hw.fixc.assign((size_t)p->dag.n_fix * kLine, 0u);
  rope_table(s, p->hw.rope_cos, p->hw.rope_sin);
  p->hw.argmax.reset(new std::atomic<unsigned long long>[(size_t)s.B * kArgmaxShards]);
  for (int i = 0; i < s.B * kArgmaxShards; ++i) p->hw.argmax[i].store(0);
  p->log.assign(p->dag.tiles.size(), wpk_log_rec{});
  return p.release();
}

int32_t host_serial_step(wpk_plan* p, int32_t* tokens, wpk_kv* kv, float* logits, uint64_t seed, bool poison_on) {
  if (!args_ok(p, tokens, kv, logits)) return WPK_E_ARG;
  Params P = host_params(p, tokens, kv, logits);
  std::fill(p->hw.fixc.begin(), p->hw.fixc.end(), 0u);
  if (poison_on) poison(p, P);
  std::atomic<int32_t> status{0};
  Ctx c{P, p->hw.argmax.get(), &status};
  c.wpart_len = (int64_t)p->hw.wpart.size();
  c.fixc_len = (int64_t)p->hw.fixc.size();
  const auto& tiles = p->dag.tiles;
  const auto& groups = p->dag.groups;
  const int32_t n = (int32_t)tiles.size();
  std::vector<std::vector<int32_t>> waiters(groups.size());
  std::vector<int32_t> ready, count(groups.size(), 0);
  for (const Tile& t : tiles) {
    if (t.wait < 0) ready.push_back(t.id);
    else waiters[t.wait].push_back(t.id);
  }
  std::fill(p->log.begin(), p->log.end(), wpk_log_rec{});
  uint64_t rng = seed;
  int32_t done = 0;
  while (!ready.empty()) {
    rng = mix64(rng);
    const size_t k = (size_t)(rng % ready.size());
    const int32_t id = ready[k];
    ready[k] = ready.back();
    ready.pop_back();
    const Tile& T = tiles[id];
    wpk_log_rec& L = p->log[id];
    L.exec_count += 1;
    L.wait_delta = T.wait < 0 ? 0 : count[T.wait] - groups[T.wait].producers;
    L.worker = 0;
    L.claim = done;
    L.t_start = 2 * (int64_t)done;
    run_tile(c, T);
    L.t_end = 2 * (int64_t)done + 1;
    ++done;
    if (T.signal >= 0 && ++count[T.signal] == groups[T.signal].producers)
      for (int32_t w : waiters[T.signal]) ready.push_back(w);
  }
  if (done != n) {
    p->err = "serial executor stalled: " + std::to_string(n - done) + " tiles never became ready";
    return WPK_E_TIMEOUT;
  }
  return status.load();
}

int32_t host_emulate_step(wpk_plan* p, int32_t* tokens, wpk_kv* kv, float* logits, int32_t n_threads,
                          uint64_t seed) {
  if (!args_ok(p, tokens, kv, logits)) return WPK_E_ARG;
  const Dag& d = p->dag;
  const int32_t nq = (int32_t)d.queue_off.size() - 1;
  if (n_threads < nq || n_threads > 256) {
    p->err = "n_threads must be in [queue shards, 256]";
    return WPK_E_ARG;
  }
  Params P = host_params(p, tokens, kv, logits);
  std::fill(p->hw.fixc.begin(), p->hw.fixc.end(), 0u);
  std::atomic<int32_t> status{0};
  Ctx c{P, p->hw.argmax.get(), &status};
  c.wpart_len = (int64_t)p->hw.wpart.size();
  c.fixc_len = (int64_t)p->hw.fixc.size();
  c.fixed_reducer = p->emu_fixed_reducer != 0;
  std::unique_ptr<std::atomic<uint32_t>[]> counters(new std::atomic<uint32_t>[d.n_shard_slots]);
  for (int i = 0; i < d.n_shard_slots; ++i) counters[i].store(0);
  std::unique_ptr<std::atomic<uint32_t>[]> heads(new std::atomic<uint32_t>[nq]);
  for (int i = 0; i < nq; ++i) heads[i].store(0);
  const int32_t n = (int32_t)d.tiles.size();
  std::unique_ptr<std::atomic<int32_t>[]> exec(new std::atomic<int32_t>[n]);
  for (int i = 0; i < n; ++i) exec[i].store(0);
  std::atomic<int32_t> abort{0};
  c.abort = &abort;
  std::fill(p->log.begin(), p->log.end(), wpk_log_rec{});
  const auto t0 = std::chrono::steady_clock::now();
  auto now_ns = [&] {
    return (int64_t)std::chrono::duration_cast<std::chrono::nanoseconds>(std::chrono::steady_clock::now() - t0).count();
  };
  auto worker = [&](int w) {
    const int q = w % nq;
    const int32_t qb = d.queue_off[q], qn = d.queue_off[q + 1] - qb;
    uint64_t rng = mix64(seed ^ (uint64_t)w * 0x9E37ULL);
    for (;;) {
      const uint32_t ci = heads[q].fetch_add(1, std::memory_order_relaxed);
      if ((int32_t)ci >= qn || abort.load(std::memory_order_relaxed)) break;
      const int32_t id = d.queue[qb + ci];
      const Tile& T = d.tiles[id];
      rng = mix64(rng);
      for (uint64_t k = rng % 8; k; --k) std::this_thread::yield();
      int32_t delta = 0;
      if (T.wait >= 0) {
        const Group& G = d.groups[T.wait];
        const auto w0 = std::chrono::steady_clock::now();
        for (;;) {
          uint32_t sum = 0;
          for (int s = 0; s < G.shards; ++s) sum += counters[G.shard0 + s].load(kPollOrder);
          if ((int32_t)(sum - (uint32_t)G.producers) >= 0) {
            delta = (int32_t)(sum - (uint32_t)G.producers);
            acquire_fence();  // the tile's input reads stay after the poll that saw them complete
            break;
          }
          if (abort.load(std::memory_order_relaxed)) return;
          if (std::chrono::steady_clock::now() - w0 > std::chrono::seconds(20)) {
            int32_t z = 0;
            status.compare_exchange_strong(z, WPK_E_TIMEOUT);
            abort.store(1);
            return;
          }
          std::this_thread::yield();
        }
      }
      wpk_log_rec& L = p->log[id];
      L.wait_delta = delta;
      L.worker = w;
      L.claim = (int32_t)ci;
      L.t_start = now_ns();
      exec[id].fetch_add(1, std::memory_order_relaxed);
      run_tile(c, T);
      L.t_end = now_ns();
      if (T.signal >= 0) {
        const Group& G = d.groups[T.signal];
        publish_fence();  // the tile's output writes happen before its publish
        counters[G.shard0 + T.shard].fetch_add(1, kPublishOrder);
      }
    }
  };
  std::vector<std::thread> th;
  for (int w = 0; w < n_threads; ++w) th.emplace_back(worker, w);
  for (auto& t : th) t.join();
  for (int i = 0; i < n; ++i) p->log[i].exec_count = exec[i].load();
  if (abort.load()) {
    p->err = "emulated worker timed out waiting on a counter";
    return WPK_E_TIMEOUT;
  }
  return status.load();
}

}  // namespace wpk
