// builder.cpp -- lowers one decode step to a tile DAG.
//
// Following "One Megakernel is Not Enough" (Table I): the barrier edges
// between consecutive operators are dropped and only tile-to-tile tensor edges
// are kept; each consumer waits on one counter group that counts exactly the
// tiles producing the region it reads.  Tiles are emitted in a topological
// order that doubles as the claim order of the device queues: because every
// producer precedes its consumers, the lowest unfinished tile always has all of
// its inputs and is held (or about to be claimed) by a worker whose earlier
// tiles are done, so the resident workers can never all wait on work nobody
// will do (the deadlock hazard of "persistent-threads-megakernels", section 4).
#include "builder.h"

#include <algorithm>
#include <cstdio>
#include <map>
#include <tuple>

namespace wpk {

static bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

std::string check_shape(const wpk_model_desc& d, int32_t batch, int32_t ctx_len,
                        const wpk_build_opts& o, Shape* out) {
  Shape s{};
  s.L = d.n_layers;
  s.H = d.hidden;
  s.Hq = d.n_q_heads;
  s.Hkv = d.n_kv_heads;
  s.D = d.head_dim;
  s.F = d.ffn;
  s.V = d.vocab;
  s.B = batch;
  s.cap = ctx_len;
  s.dtype = d.dtype;
  s.theta = d.rope_theta;
  s.eps = d.rms_eps;
  if (s.L <= 0 || s.H <= 0 || s.Hq <= 0 || s.Hkv <= 0 || s.F <= 0 || s.V <= 0)
    return "model dimensions must be positive";
  if (s.L > kMaxLayers) return "at most 32 layers";
  if (d.dtype != WPK_F32 && d.dtype != WPK_BF16) return "dtype must be WPK_F32 or WPK_BF16";
  if (!d.tied_embeddings) return "only tied embeddings (lm_head = embed) are built";
  if (s.D != kHeadDim) return "head_dim must be 64";
  if (s.Hq % s.Hkv != 0) return "n_q_heads must be a multiple of n_kv_heads";
  s.G = s.Hq / s.Hkv;
  if (s.G > kMaxGroupHeads) return "at most 4 q heads per kv head";
  if (s.Hq * s.D != s.H) return "n_q_heads * head_dim must equal hidden";
  if (batch < 1 || batch > kMaxBatch) return "batch must be in [1, 32]";
  s.wide = batch > kMaxBatchGemv;
  if (ctx_len < 1) return "ctx_len must be positive";
  if (!(d.rms_eps >= 0.0f) || !(d.rope_theta > 0.0f)) return "rms_eps >= 0 and rope_theta > 0 required";
  s.elt = d.dtype == WPK_F32 ? 4 : 2;
  const int64_t rb_h = (int64_t)s.H * s.elt, rb_f = (int64_t)s.F * s.elt;
  if (rb_h % 16 || rb_f % 16) return "weight rows must be whole 16-byte chunks";
  s.cpr_h = (int32_t)(rb_h / 16);
  s.cpr_f = (int32_t)(rb_f / 16);
  if (!is_pow2(s.cpr_h) || !is_pow2(s.cpr_f) || s.cpr_h < 64 || s.cpr_f < 64 || s.cpr_h > 2048 ||
      s.cpr_f > 2048)
    return "hidden*elt and ffn*elt must be powers of two between 1 KiB and 32 KiB";
  s.tile_bytes = o.tile_bytes ? o.tile_bytes : kSlotBytes;
  if (s.tile_bytes % 4096 || s.tile_bytes < 4096 || s.tile_bytes > kSlotBytes)
    return "tile_bytes must be a multiple of 4096 in [4096, 65536]";
  s.rows_h = (int32_t)(s.tile_bytes / rb_h);
  s.rows_f = (int32_t)(s.tile_bytes / rb_f);
  if (s.rows_h < 2 || s.rows_f < 1) return "tile_bytes too small for one row pair";
  if (s.rows_h > 64) s.rows_h = 64;
  s.rows_h &= ~1;
  int rq = 1;
  while (rq * 2 <= std::min(s.rows_h, s.D)) rq *= 2;
  s.rows_qkv = rq;
  if (s.rows_f > 64) s.rows_f = 64;
  if (s.wide) {
    // matrix-core tiles: 64 rows (one head of QKV) x 512-column slices of K
    if (s.dtype != WPK_BF16) return "batches above 4 need bf16 weights";
    if (s.H % kWideK || s.F % kWideK) return "batches above 4 need hidden and ffn to be multiples of 512";
    if (s.D != kWideRows) return "batches above 4 need head_dim 64";
    // the last slice of a K = hidden row block loads the other slices'
    // partial sums, the RoPE factors and the RMSNorm sums of squares into one
    // 64 KiB LDS area
    if (s.H > 2048) return "batches above 4 need hidden <= 2048";
    s.rows_h = s.rows_qkv = s.rows_f = kWideRows;
  }
  s.workers_per_cu = o.workers_per_cu ? o.workers_per_cu : 2;
  if (s.workers_per_cu < 1 || s.workers_per_cu > 8) return "workers_per_cu must be in [1, 8]";
  s.queue_shards = o.queue_shards ? o.queue_shards : 8;
  if (s.queue_shards < 1 || s.queue_shards > 64) return "queue_shards must be in [1, 64]";
  if (o.attn_chunk && o.attn_chunk != kAttnChunk) return "attn_chunk must be 64";
  s.qkv_rows = (s.Hq + 2 * s.Hkv) * s.D;
  s.nch = (s.cap + kAttnChunk - 1) / kAttnChunk;
  // Batch 1-4: one KV chunk per attention tile (few tiles, as many in
  // parallel as possible).  Wide plans have tiles to spare: as many chunks as
  // the slot holds, so a tile's claim and hand-off cover more work.
  s.attn_sub = s.wide ? kSlotBytes / (2 * kAttnChunk * s.D * s.elt) : 1;
  if (o.forward < -1 || o.forward > 1) return "forward must be -1, 0 or 1";
  s.forward = o.forward == 1;  // measured slower at the built shapes: off unless asked for
  if (s.forward && !s.wide) return "LDS forwarding of attention partials is built for batches above 4";
  if (o.barrier_edges != 0 && o.barrier_edges != 1) return "barrier_edges must be 0 or 1";
  s.barrier_edges = o.barrier_edges;
  if (o.split_workers < 0) return "split_workers must be >= 0";
  s.split_workers = o.split_workers;
  *out = s;
  return "";
}

int64_t step_weight_bytes(const Shape& s) {
  const int64_t per_layer = (int64_t)s.qkv_rows * s.H + (int64_t)s.H * s.H + 3LL * s.F * s.H;
  return (per_layer * s.L + (int64_t)s.V * s.H) * s.elt + (int64_t)(2 * s.L + 1) * s.H * 4;
}

namespace {

struct Emitter {
  Dag d;
  int32_t group() {
    d.groups.push_back(Group{0, 0, 0, 0});
    return (int32_t)d.groups.size() - 1;
  }
  Tile& tile(int32_t type, int32_t layer, int32_t wait, int32_t signal) {
    Tile t{};
    t.type = type;
    t.layer = layer;
    t.wait = wait;
    t.signal = signal;
    t.r1 = -1;
    t.kind = -1;
    t.id = (int32_t)d.tiles.size();
    d.tiles.push_back(t);
    return d.tiles.back();
  }
  Tile& gemv(int32_t type, int32_t layer, int32_t wait, int32_t signal, int32_t r0, int32_t r1,
             int32_t rs, int32_t rows) {
    Tile& t = tile(type, layer, wait, signal);
    t.r0 = r0;
    t.r1 = r1;
    t.rs = rs;
    t.rows = rows;
    return t;
  }
  // A chained attention tile: all KV chunks of (sequence b, kv head g).
  Tile& attnc(int32_t layer, int32_t wait, int32_t signal, int32_t b, int32_t g, int32_t nch) {
    Tile& t = tile(T_ATTNC, layer, wait, signal);
    t.b = b;
    t.g = g;
    t.c = 0;
    t.kind = nch;
    return t;
  }
  // The slices of one wide row block: slice c waits on wait_of(c); all signal
  // `signal`.
  template <class F>
  void wide(int32_t type, int32_t layer, F wait_of, int32_t signal, int32_t r0, int32_t r1, int32_t rs,
            int32_t K, int32_t kind = -1, int32_t head = 0) {
    const int32_t nsl = K / kWideK;
    for (int32_t c = 0; c < nsl; ++c) {
      Tile& t = gemv(type, layer, wait_of(c), signal, r0, r1, rs, kWideRows);
      t.b = nsl;
      t.c = c;
      t.fix = d.n_fix;
      t.pslot = d.n_pslots;
      t.kind = kind;
      t.g = head;
    }
    d.n_fix += 1;
    d.n_pslots += nsl;
  }
};

}  // namespace

namespace {

Dag finish_dag(const Shape& s, Emitter& e);

// The counter groups of one operator's consumers: one per consumer input
// region (tile-to-tile edges), or, as the barrier-edge ablation, a single
// group shared by all of them, so that every consumer waits for the whole
// producing operator.
void fill_groups(Emitter& e, std::vector<int32_t>& gs, int32_t barrier) {
  const int32_t one = barrier ? e.group() : -1;
  for (auto& g : gs) g = barrier ? one : e.group();
}

// Wide plans (batch above kMaxBatchGemv).  Layer 0 starts with a tile per
// sequence that writes the embedding row as the first QKV operand.  Per layer:
// QKV row blocks of one head each (two segments, dimensions [0, D/2) and
// [D/2, D), so a RoPE pair is rows i and i + D/2 of the tile), attention of kv
// head g waiting on its q, k and v heads; output-projection slices, each
// waiting only on the combines of the heads in its K slice; gate/up row blocks
// (32 gate + 32 up rows) waiting on the o-proj; down slices, each waiting only
// on the gate/up row blocks of its K slice.  Then the LM-head row blocks.  The
// RMSNorms need no tiles of their own: the o-proj and down epilogues write
// gain * x and per-block sums of squares, and the QKV, gate/up and LM-head
// epilogues divide by the root mean square.
void build_wide(const Shape& s, Emitter& e) {
  const int32_t D = s.D;
  const int32_t n_os = s.H / kWideK;            // o-proj K slices
  const int32_t n_ds = s.F / kWideK;            // down K slices
  const int32_t hpb = kWideRows / 2;             // h columns per gate/up row block
  auto same = [](int32_t w) { return [w](int32_t) { return w; }; };
  int32_t g_x = -1;
  for (int32_t l = 0; l < s.L; ++l) {
    int32_t g_qkv_in = g_x;
    if (l == 0) {
      g_qkv_in = e.group();
      for (int32_t b = 0; b < s.B; ++b) e.tile(T_NORM, 0, -1, g_qkv_in).b = b;
    }
    std::vector<int32_t> g_attn(s.Hkv), g_comb(s.B * s.Hkv), g_o(n_os), g_dn(n_ds);
    fill_groups(e, g_attn, s.barrier_edges);
    fill_groups(e, g_comb, s.barrier_edges);
    fill_groups(e, g_o, s.barrier_edges);
    const int32_t g_xm = e.group();
    fill_groups(e, g_dn, s.barrier_edges);
    const int32_t g_next = e.group();
    for (int32_t g = 0; g < s.Hkv; ++g) {
      for (int32_t k = 0; k < s.G; ++k) {
        const int32_t head = g * s.G + k;
        e.wide(T_QKV, l, same(g_qkv_in), g_attn[g], head * D, head * D + D / 2, D / 2, s.H, 0, head);
      }
      const int32_t kb = (s.Hq + g) * D, vb = (s.Hq + s.Hkv + g) * D;
      e.wide(T_QKV, l, same(g_qkv_in), g_attn[g], kb, kb + D / 2, D / 2, s.H, 1, g);
      e.wide(T_QKV, l, same(g_qkv_in), g_attn[g], vb, vb + D / 2, D / 2, s.H, 2, g);
    }
    if (s.forward) {  // each feeds the o-proj slice holding its kv head's q heads
      for (int32_t b = 0; b < s.B; ++b)
        for (int32_t g = 0; g < s.Hkv; ++g) e.attnc(l, g_attn[g], g_o[g * s.G * D / kWideK], b, g, s.nch);
    } else {
      for (int32_t b = 0; b < s.B; ++b)
        for (int32_t g = 0; g < s.Hkv; ++g)
          for (int32_t c = 0; c < s.nch; c += s.attn_sub) {
            Tile& t = e.tile(T_ATTN, l, g_attn[g], g_comb[b * s.Hkv + g]);
            t.b = b;
            t.g = g;
            t.c = c;
            t.kind = std::min(s.attn_sub, s.nch - c);
          }
      for (int32_t b = 0; b < s.B; ++b)
        for (int32_t g = 0; g < s.Hkv; ++g) {
          // the o-proj slice holding this kv head's q heads
          Tile& t = e.tile(T_COMBINE, l, g_comb[b * s.Hkv + g], g_o[g * s.G * D / kWideK]);
          t.b = b;
          t.g = g;
        }
    }
    for (int32_t r = 0; r < s.H; r += kWideRows)
      e.wide(T_OPROJ, l, [&](int32_t c) { return g_o[c]; }, g_xm, r, r + kWideRows, kWideRows, s.H);
    for (int32_t j = 0; j < s.F; j += hpb)
      e.wide(T_GATEUP, l, same(g_xm), g_dn[j / kWideK], j, j, hpb, s.H);
    for (int32_t r = 0; r < s.H; r += kWideRows)
      e.wide(T_DOWN, l, [&](int32_t c) { return g_dn[c]; }, g_next, r, r + kWideRows, kWideRows, s.F);
    g_x = g_next;
  }
  const int32_t g_am = e.group();
  for (int32_t r = 0; r < s.V; r += kWideRows)
    e.wide(T_LM, s.L - 1, same(g_x), g_am, r, r + kWideRows, kWideRows, s.H);
  e.tile(T_ARGMAX, s.L - 1, g_am, -1);
}

}  // namespace

Dag build_dag(const Shape& s) {
  Emitter e;
  if (s.wide) {
    build_wide(s, e);
    return finish_dag(s, e);
  }
  const int32_t D = s.D, half = s.D / 2;
  int32_t g_x = -1;  // group the current layer's QKV tiles wait on (-1: layer 0)
  for (int32_t l = 0; l < s.L; ++l) {
    std::vector<int32_t> g_attn(s.Hkv), g_comb(s.B * s.Hkv);
    fill_groups(e, g_attn, s.barrier_edges);
    fill_groups(e, g_comb, s.barrier_edges);
    const int32_t g_o = e.group(), g_gu = e.group(), g_dn = e.group();
    const int32_t g_qkv_in = g_x;

    // QKV: for each kv group, the q heads of the group, then its k head, then
    // its v head, so attention of group g depends on a contiguous run.
    const int32_t rs_q = s.rows_qkv / 2;
    for (int32_t g = 0; g < s.Hkv; ++g) {
      for (int32_t k = 0; k <= s.G + 1; ++k) {
        const int32_t kind = k < s.G ? 0 : (k == s.G ? 1 : 2);
        const int32_t head = kind == 0 ? g * s.G + k : g;
        const int32_t base = kind == 0 ? head * D : (kind == 1 ? (s.Hq + g) * D : (s.Hq + s.Hkv + g) * D);
        if (kind < 2) {
          for (int32_t i0 = 0; i0 < half; i0 += rs_q) {
            Tile& t = e.gemv(T_QKV, l, g_qkv_in, g_attn[g], base + i0, base + half + i0, rs_q, s.rows_qkv);
            t.kind = kind;
            t.g = head;
          }
        } else {
          for (int32_t i0 = 0; i0 < D; i0 += s.rows_qkv) {
            Tile& t = e.gemv(T_QKV, l, g_qkv_in, g_attn[g], base + i0, base + i0 + rs_q, rs_q, s.rows_qkv);
            t.kind = 2;
            t.g = head;
          }
        }
      }
    }
    if (s.forward) {
      for (int32_t b = 0; b < s.B; ++b)
        for (int32_t g = 0; g < s.Hkv; ++g) e.attnc(l, g_attn[g], g_o, b, g, s.nch);
    } else {
      for (int32_t b = 0; b < s.B; ++b)
        for (int32_t g = 0; g < s.Hkv; ++g)
          for (int32_t c = 0; c < s.nch; ++c) {
            Tile& t = e.tile(T_ATTN, l, g_attn[g], g_comb[b * s.Hkv + g]);
            t.b = b;
            t.g = g;
            t.c = c;
            t.kind = 1;
          }
      for (int32_t b = 0; b < s.B; ++b)
        for (int32_t g = 0; g < s.Hkv; ++g) {
          Tile& t = e.tile(T_COMBINE, l, g_comb[b * s.Hkv + g], g_o);
          t.b = b;
          t.g = g;
        }
    }
    for (int32_t r = 0; r < s.H; r += s.rows_h) e.gemv(T_OPROJ, l, g_o, g_gu, r, r + s.rows_h, s.rows_h, s.rows_h);
    const int32_t rs_gu = s.rows_h / 2;
    for (int32_t j = 0; j < s.F; j += rs_gu) e.gemv(T_GATEUP, l, g_gu, g_dn, j, j, rs_gu, s.rows_h);
    const int32_t g_next = e.group();  // x of the next layer, or the LM head's input
    for (int32_t r = 0; r < s.H; r += s.rows_f) e.gemv(T_DOWN, l, g_dn, g_next, r, r + s.rows_f, s.rows_f, s.rows_f);
    g_x = g_next;
  }
  const int32_t g_am = e.group();
  for (int32_t r = 0; r < s.V; r += s.rows_h) e.gemv(T_LM, s.L - 1, g_x, g_am, r, r + s.rows_h, s.rows_h, s.rows_h);
  e.tile(T_ARGMAX, s.L - 1, g_am, -1);
  return finish_dag(s, e);
}

namespace {

Dag finish_dag(const Shape& s, Emitter& e) {
  Dag& d = e.d;
  // producers and shards: two producers per shard, up to kMaxShards (a
  // phase's increments of one counter line serialise)
  for (const Tile& t : d.tiles)
    if (t.signal >= 0) d.groups[t.signal].producers++;
  int32_t slot = 0;
  for (Group& g : d.groups) {
    int32_t want = (g.producers + 1) / 2, sh = 1;
    while (sh < want && sh < kMaxShards) sh *= 2;
    g.shards = sh;
    g.shard0 = slot;
    slot += sh;
  }
  d.n_shard_slots = slot;
  std::vector<int32_t> seen(d.groups.size(), 0);
  for (Tile& t : d.tiles)
    if (t.signal >= 0) t.shard = seen[t.signal]++ % d.groups[t.signal].shards;

  // claim queues: the topological order dealt round-robin (split plans: each
  // region's tiles, in topological order, over that region's queues)
  const int32_t nq = s.queue_shards;
  const int32_t nr = s.split_workers > 0 ? 2 : 1;
  auto region = [&](const Tile& t) {
    return nr == 2 && (t.type == T_ATTN || t.type == T_ATTNC || t.type == T_COMBINE) ? 1 : 0;
  };
  d.queue_off.assign(nr * nq + 1, 0);
  for (int32_t r = 0; r < nr; ++r) {
    std::vector<int32_t> ids;
    for (size_t i = 0; i < d.tiles.size(); ++i)
      if (region(d.tiles[i]) == r) ids.push_back((int32_t)i);
    for (int32_t q = 0; q < nq; ++q) {
      d.queue_off[r * nq + q] = (int32_t)d.queue.size();
      for (size_t i = q; i < ids.size(); i += nq) d.queue.push_back(ids[i]);
    }
  }
  d.queue_off[nr * nq] = (int32_t)d.queue.size();
  d.split_queues = nr == 2 ? nq : 0;

  // operator runs for the baseline
  for (size_t i = 0; i < d.tiles.size();) {
    size_t j = i;
    while (j < d.tiles.size() && d.tiles[j].type == d.tiles[i].type && d.tiles[j].layer == d.tiles[i].layer) ++j;
    d.phases.emplace_back((int32_t)i, (int32_t)(j - i));
    i = j;
  }
  return d;
}

}  // namespace

namespace {

// Half-open interval set with coverage queries.
struct Cover {
  std::vector<std::pair<int64_t, int64_t>> iv;
  void add(int64_t a, int64_t b) {
    if (a < b) iv.emplace_back(a, b);
  }
  void seal() {
    std::sort(iv.begin(), iv.end());
    std::vector<std::pair<int64_t, int64_t>> m;
    for (auto& p : iv) {
      if (!m.empty() && p.first <= m.back().second) m.back().second = std::max(m.back().second, p.second);
      else m.push_back(p);
    }
    iv.swap(m);
  }
  bool covers(int64_t a, int64_t b) const {
    if (a >= b) return true;
    auto it = std::upper_bound(iv.begin(), iv.end(), std::make_pair(a, INT64_MAX));
    if (it == iv.begin()) return false;
    --it;
    return it->first <= a && it->second >= b;
  }
};

bool is_gemm(int32_t type) {
  return type == T_QKV || type == T_OPROJ || type == T_GATEUP || type == T_DOWN || type == T_LM;
}

// Output rows of a GEMM operator, and (wide plans) its K slices: the flat
// index of row r of slice c is c * rows + r.
int64_t gemm_rows(const Shape& s, int32_t type) {
  return type == T_QKV ? s.qkv_rows : type == T_LM ? s.V : type == T_GATEUP ? s.F : s.H;
}
int32_t gemm_slices(const Shape& s, int32_t type) {
  return s.wide ? (type == T_DOWN ? s.F : s.H) / kWideK : 1;
}

// The region of its operator's output tensor a tile writes, as intervals of a
// flat index, keyed by (layer, type).  A wide GEMM tile writes its rows of its
// K slice (the partial sums the row block's last slice adds up).
void outputs(const Shape& s, const Tile& t, std::vector<std::pair<int64_t, int64_t>>& out) {
  out.clear();
  auto clip = [](int64_t a, int64_t b, int64_t lim) { return std::make_pair(std::min(a, lim), std::min(b, lim)); };
  switch (t.type) {
    case T_QKV:
    case T_OPROJ:
    case T_DOWN:
    case T_LM: {
      const int64_t lim = gemm_rows(s, t.type), at = s.wide ? (int64_t)t.c * lim : 0;
      auto p = clip(t.r0, t.r0 + t.rs, lim);
      out.emplace_back(at + p.first, at + p.second);
      if (t.rows > t.rs) {
        p = clip(t.r1, t.r1 + (t.rows - t.rs), lim);
        out.emplace_back(at + p.first, at + p.second);
      }
      break;
    }
    case T_GATEUP: {
      const int64_t at = s.wide ? (int64_t)t.c * s.F : 0;
      auto p = clip(t.r0, t.r0 + t.rs, s.F);  // h rows (gate and up rows pair up)
      out.emplace_back(at + p.first, at + p.second);
      break;
    }
    case T_ATTN: {  // its KV chunks' partials
      const int64_t i = ((int64_t)t.b * s.Hkv + t.g) * s.nch + t.c;
      out.emplace_back(i, i + t.kind);
      break;
    }
    case T_COMBINE:
    case T_ATTNC: {  // the attention output of its q heads
      const int64_t base = (int64_t)t.b * s.Hq * s.D + (int64_t)t.g * s.G * s.D;
      out.emplace_back(base, base + (int64_t)s.G * s.D);
      break;
    }
    case T_ARGMAX:
      out.emplace_back(0, s.B);
      break;
    case T_NORM:
      out.emplace_back(t.b, t.b + 1);  // one sequence's operand row
      break;
  }
}

// The tensor a tile type writes: a chained attention tile writes what a
// combine tile would.
int32_t out_type(int32_t type) { return type == T_ATTNC ? T_COMBINE : type; }

struct Need {
  int32_t layer, type;
  int64_t a, b;
};

// What a tile reads from tensors produced in the same step.
void inputs(const Shape& s, const Tile& t, std::vector<Need>& need) {
  need.clear();
  const int32_t l = t.layer;
  if (s.wide) {
    // rows [a, b) of a GEMM operator's output: every K slice of them
    auto rows = [&](int32_t layer, int32_t type, int64_t a, int64_t b) {
      const int64_t lim = gemm_rows(s, type);
      for (int32_t c = 0; c < gemm_slices(s, type); ++c) need.push_back({layer, type, c * lim + a, c * lim + b});
    };
    switch (t.type) {
      case T_NORM:  // layer 0 only: the embedding rows
        break;
      case T_QKV:  // the operand and sums of squares of every row block of x
        if (l == 0) need.push_back({0, T_NORM, 0, s.B});
        else rows(l - 1, T_DOWN, 0, s.H);
        break;
      case T_ATTN:
      case T_ATTNC: {
        const int64_t qa = (int64_t)t.g * s.G * s.D, ka = ((int64_t)s.Hq + t.g) * s.D,
                      va = ((int64_t)s.Hq + s.Hkv + t.g) * s.D;
        rows(l, T_QKV, qa, qa + (int64_t)s.G * s.D);
        rows(l, T_QKV, ka, ka + s.D);
        rows(l, T_QKV, va, va + s.D);
        break;
      }
      case T_COMBINE: {
        const int64_t i = ((int64_t)t.b * s.Hkv + t.g) * s.nch;
        need.push_back({l, T_ATTN, i, i + s.nch});
        break;
      }
      case T_OPROJ:  // the attention output columns of its K slice, every sequence
        for (int32_t b = 0; b < s.B; ++b) {
          const int64_t a = (int64_t)b * s.Hq * s.D + (int64_t)t.c * kWideK;
          need.push_back({l, T_COMBINE, a, a + kWideK});
        }
        break;
      case T_GATEUP:
        rows(l, T_OPROJ, 0, s.H);
        break;
      case T_DOWN:  // the h columns of its K slice
        rows(l, T_GATEUP, (int64_t)t.c * kWideK, (int64_t)(t.c + 1) * kWideK);
        break;
      case T_LM:
        rows(s.L - 1, T_DOWN, 0, s.H);
        break;
      case T_ARGMAX:
        rows(s.L - 1, T_LM, 0, s.V);
        break;
    }
    return;
  }
  switch (t.type) {
    case T_QKV:
      if (l > 0) need.push_back({l - 1, T_DOWN, 0, s.H});
      break;
    case T_ATTN:
    case T_ATTNC: {
      const int64_t qa = (int64_t)t.g * s.G * s.D;
      need.push_back({l, T_QKV, qa, qa + (int64_t)s.G * s.D});
      const int64_t ka = ((int64_t)s.Hq + t.g) * s.D;
      need.push_back({l, T_QKV, ka, ka + s.D});
      const int64_t va = ((int64_t)s.Hq + s.Hkv + t.g) * s.D;
      need.push_back({l, T_QKV, va, va + s.D});
      break;
    }
    case T_COMBINE: {
      const int64_t i = ((int64_t)t.b * s.Hkv + t.g) * s.nch;
      need.push_back({l, T_ATTN, i, i + s.nch});
      break;
    }
    case T_OPROJ:
      need.push_back({l, T_COMBINE, 0, (int64_t)s.B * s.Hq * s.D});
      break;
    case T_GATEUP:
      need.push_back({l, T_OPROJ, 0, s.H});
      break;
    case T_DOWN:
      need.push_back({l, T_GATEUP, 0, s.F});
      break;
    case T_LM:
      need.push_back({s.L - 1, T_DOWN, 0, s.H});
      break;
    case T_ARGMAX:
      need.push_back({s.L - 1, T_LM, 0, s.V});
      break;
  }
}

}  // namespace

std::string validate_dag(const Shape& s, const Dag& d) {
  char msg[256];
  const int32_t n = (int32_t)d.tiles.size();
  std::vector<std::vector<int32_t>> producers(d.groups.size());
  for (int32_t i = 0; i < n; ++i) {
    const Tile& t = d.tiles[i];
    if (t.id != i) return "tile ids are not their positions";
    if (t.signal >= (int32_t)d.groups.size() || t.wait >= (int32_t)d.groups.size()) return "group id out of range";
    if (t.signal >= 0) producers[t.signal].push_back(i);
  }
  for (size_t g = 0; g < d.groups.size(); ++g)
    if ((int32_t)producers[g].size() != d.groups[g].producers) return "group producer count mismatch";
  // topological claim order: every producer of a tile's group comes before it
  for (int32_t i = 0; i < n; ++i) {
    const Tile& t = d.tiles[i];
    if (t.wait < 0) continue;
    if (producers[t.wait].empty()) {
      snprintf(msg, sizeof msg, "tile %d waits on group %d that has no producers", i, t.wait);
      return msg;
    }
    if (producers[t.wait].back() >= i) {
      snprintf(msg, sizeof msg, "tile %d precedes its producer %d: the order is not topological (cycle?)", i,
               producers[t.wait].back());
      return msg;
    }
  }
  // every output element written exactly once per (layer, type)
  std::map<std::pair<int32_t, int32_t>, std::vector<std::pair<int64_t, int64_t>>> written;
  std::vector<std::pair<int64_t, int64_t>> out;
  for (const Tile& t : d.tiles) {
    outputs(s, t, out);
    auto& w = written[{t.layer, out_type(t.type)}];
    for (auto& p : out)
      if (p.first < p.second) w.push_back(p);
  }
  for (auto& kv : written) {
    auto v = kv.second;
    std::sort(v.begin(), v.end());
    int64_t at = 0;
    for (auto& p : v) {
      if (p.first != at) {
        snprintf(msg, sizeof msg, "layer %d type %d: element %lld written %s", kv.first.first, kv.first.second,
                 (long long)std::min(at, p.first), p.first > at ? "never" : "twice");
        return msg;
      }
      at = p.second;
    }
    const int32_t type = kv.first.second;
    const int64_t want = is_gemm(type) ? gemm_rows(s, type) * gemm_slices(s, type)
                         : type == T_ATTN ? (int64_t)s.B * s.Hkv * s.nch
                         : type == T_COMBINE ? (int64_t)s.B * s.Hq * s.D
                                             : s.B;
    if (at != want) {
      snprintf(msg, sizeof msg, "layer %d type %d covers %lld of %lld elements", kv.first.first, type,
               (long long)at, (long long)want);
      return msg;
    }
  }
  // inputs covered by the wait group's producers
  std::vector<Need> need;
  std::map<int32_t, std::map<std::pair<int32_t, int32_t>, Cover>> cover_of_group;
  for (const Tile& t : d.tiles) {
    inputs(s, t, need);
    if (need.empty()) continue;
    if (t.wait < 0) {
      snprintf(msg, sizeof msg, "tile %d reads tensors of this step but waits on nothing", t.id);
      return msg;
    }
    auto it = cover_of_group.find(t.wait);
    if (it == cover_of_group.end()) {
      auto& cg = cover_of_group[t.wait];
      for (int32_t p : producers[t.wait]) {
        outputs(s, d.tiles[p], out);
        for (auto& iv : out) cg[{d.tiles[p].layer, out_type(d.tiles[p].type)}].add(iv.first, iv.second);
      }
      for (auto& c : cg) c.second.seal();
      it = cover_of_group.find(t.wait);
    }
    for (const Need& nd : need) {
      auto c = it->second.find({nd.layer, nd.type});
      if (c == it->second.end() || !c->second.covers(nd.a, nd.b)) {
        snprintf(msg, sizeof msg, "tile %d (type %d layer %d) reads [%lld, %lld) of layer %d type %d not produced by group %d",
                 t.id, t.type, t.layer, (long long)nd.a, (long long)nd.b, nd.layer, nd.type, t.wait);
        return msg;
      }
    }
  }
  // queues hold every tile exactly once, each in increasing (topological) order
  std::vector<int32_t> count(n, 0);
  for (size_t q = 0; q + 1 < d.queue_off.size(); ++q)
    for (int32_t i = d.queue_off[q]; i < d.queue_off[q + 1]; ++i) {
      if (d.queue[i] < 0 || d.queue[i] >= n) return "queue entry out of range";
      count[d.queue[i]]++;
      if (i > d.queue_off[q] && d.queue[i] <= d.queue[i - 1]) return "queue not in topological order";
    }
  for (int32_t i = 0; i < n; ++i)
    if (count[i] != 1) return "a tile is not queued exactly once";
  return "";
}

std::string check_device_geometry(const Shape& s, const Dag& d) {
  // byte offsets inside one matrix or one (layer, sequence, kv head) cache
  // slice are 32-bit and bounded by the buffer resource's 2^31 - 1 records
  const int64_t lim = 0x7FFFFFFF;
  const int64_t rb_h = (int64_t)s.cpr_h * 16, rb_f = (int64_t)s.cpr_f * 16;
  if ((int64_t)s.V * rb_h > lim || (int64_t)s.qkv_rows * rb_h > lim || (int64_t)s.F * rb_h > lim ||
      (int64_t)s.H * rb_f > lim || (int64_t)s.cap * s.D * s.elt > lim)
    return "a weight matrix or a KV cache slice exceeds 2 GiB";
  if (s.wide) return "";  // wide tiles address rows per lane and clamp a ragged last block
  // a 4 KiB slice of a tile holds 256 / cpr whole rows when a row is shorter
  // than a slice; segments, tiles and matrices must break on whole slices
  for (const Tile& t : d.tiles) {
    if (t.type != T_QKV && t.type != T_OPROJ && t.type != T_GATEUP && t.type != T_DOWN && t.type != T_LM)
      continue;
    const int32_t cpr = t.type == T_DOWN ? s.cpr_f : s.cpr_h;
    const int32_t sr = cpr >= kThreads ? 1 : kThreads / cpr;
    if (t.rows < sr || t.rows % sr || t.rs % sr || t.r0 % sr || t.r1 % sr)
      return "tile_bytes too small for whole 4 KiB row slices";
  }
  const int32_t sr_h = s.cpr_h >= kThreads ? 1 : kThreads / s.cpr_h;
  const int32_t sr_f = s.cpr_f >= kThreads ? 1 : kThreads / s.cpr_f;
  if (s.V % sr_h || s.qkv_rows % sr_h || s.F % sr_h || s.H % sr_h || s.H % sr_f)
    return "vocab and projection row counts must fill whole 4 KiB slices";
  return "";
}

}  // namespace wpk
