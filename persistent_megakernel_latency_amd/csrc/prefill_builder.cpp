// prefill_builder.cpp -- the prompt prefill as a tile DAG.
//
// Per layer, in claim order (operator-major across sequences, so the first
// sequences' later operators become ready while the last sequences' earlier
// ones still run):
//   NORM1 / EMBED (row block)  ->  QKV (row block, 4 heads)
//   ->  ATTN (sequence, kv head, query block: waits for the whole sequence's
//       K and V, the causal span of its last query block)
//   ->  OPROJ (row block, 256 columns)  ->  NORM2 (row block)
//   ->  GATEUP (row block, 128 ffn columns)  ->  DOWN (row block, 256 columns)
//   ->  the next layer's NORM1 of the same row block.
// After the last layer: NORMF per sequence (its last prompt row), the LM-head
// tiles, and one ARGMAX tile.  Counter groups are per row block (per
// sequence for the attention input), the tile-to-tile edges of "One
// Megakernel is Not Enough", Table I.
#include "prefill_builder.h"

#include <algorithm>
#include <cstdio>
#include <functional>
#include <map>
#include <queue>
#include <set>
#include <tuple>

namespace wpk {

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

std::string check_prefill_shape(const wpk_model_desc& d, int32_t batch, int32_t ctx_len, int32_t prompt_len,
                                int32_t split, PShape* out) {
  PShape s{};
  s.L = d.n_layers;
  s.H = d.hidden;
  s.Hq = d.n_q_heads;
  s.Hkv = d.n_kv_heads;
  s.D = d.head_dim;
  s.F = d.ffn;
  s.V = d.vocab;
  s.B = batch;
  s.cap = ctx_len;
  s.P = prompt_len;
  s.theta = d.rope_theta;
  s.eps = d.rms_eps;
  if (s.L <= 0 || s.H <= 0 || s.Hq <= 0 || s.Hkv <= 0 || s.F <= 0 || s.V <= 0)
    return "model dimensions must be positive";
  if (s.L > kMaxLayers) return "at most 32 layers";
  if (d.dtype != WPK_BF16) return "the prefill is built for bf16 weights";
  if (!d.tied_embeddings) return "only tied embeddings (lm_head = embed) are built";
  if (s.D != kHeadDim) return "head_dim must be 64";
  if (s.Hq % s.Hkv != 0) return "n_q_heads must be a multiple of n_kv_heads";
  s.G = s.Hq / s.Hkv;
  if (s.G > kMaxGroupHeads) return "at most 4 q heads per kv head";
  if (s.Hq * s.D != s.H) return "n_q_heads * head_dim must equal hidden";
  if (s.H % kPCols || s.H > 4096) return "hidden must be a multiple of 256, at most 4096";
  if (s.F % kPFfnCols) return "ffn must be a multiple of 128";
  s.qkv_rows = (s.Hq + 2 * s.Hkv) * s.D;
  if (s.qkv_rows % kPCols) return "n_q_heads + 2 n_kv_heads must be a multiple of 4 (QKV tiles hold four heads)";
  if (batch < 1 || batch > kMaxBatch) return "batch must be in [1, 32]";
  if (ctx_len < 1) return "ctx_len must be positive";
  if (prompt_len < 1 || prompt_len > ctx_len) return "prompt_len must be in [1, ctx_len]";
  if (!(d.rms_eps >= 0.0f) || !(d.rope_theta > 0.0f)) return "rms_eps >= 0 and rope_theta > 0 required";
  s.Pp = (int32_t)ceil_div(s.P, kPRows) * kPRows;
  s.nrb_s = s.Pp / kPRows;
  s.nqb = (int32_t)ceil_div(s.P, kPQueries);
  const int64_t R = (int64_t)s.B * s.Pp;
  s.R = (int32_t)R;
  // 32-bit byte offsets within one buffer (buffer loads and stores)
  const int64_t big = std::max({R * s.F * 2, R * s.H * 4, (int64_t)s.V * s.H * 2,
                                (int64_t)s.L * s.B * s.Hkv * s.cap * s.D * 2, (int64_t)s.F * s.H * 2});
  if (big >= ((int64_t)1 << 31)) return "a buffer of this prefill would exceed 2 GiB (32-bit offsets)";
  if (split != 0 && split != 1) return "split must be 0 or 1";
  s.split = split;
  s.queue_shards = 8;
  *out = s;
  return "";
}

PDag build_prefill_dag(const PShape& s) {
  PDag d;
  const int nq0 = s.queue_shards, nq1 = s.split ? s.queue_shards : 0;
  std::vector<std::vector<int32_t>> queues(nq0 + nq1);
  auto group = [&]() {
    d.groups.push_back(Group{0, 0, 0, 0});
    return (int32_t)d.groups.size() - 1;
  };
  auto add = [&](int32_t type, int32_t layer, int32_t wait, int32_t signal, int32_t rb, int32_t cb, int32_t b,
                 int32_t g, int32_t c, int32_t queue) {
    Tile t{};
    t.type = type;
    t.layer = layer;
    t.wait = wait;
    t.signal = signal;
    t.r0 = rb;
    t.r1 = cb;
    t.b = b;
    t.g = g;
    t.c = c;
    t.id = (int32_t)d.tiles.size();
    t.fix = -1;
    t.pslot = -1;
    d.tiles.push_back(t);
    queues[queue].push_back(t.id);
  };
  const int nrb = s.B * s.nrb_s;
  const int ncq = s.qkv_rows / kPCols, nch = s.H / kPCols, ncf = s.F / kPFfnCols;
  // groups of the previous layer's down tiles per row block (the next norm waits on them)
  std::vector<int32_t> down_g(nrb, -1);
  for (int l = 0; l < s.L; ++l) {
    std::vector<int32_t> n1_g(nrb), qkv_g(s.B), at_g(nrb), o_g(nrb), n2_g(nrb), gu_g(nrb), dn_g(nrb);
    for (int rb = 0; rb < nrb; ++rb) n1_g[rb] = group();
    for (int b = 0; b < s.B; ++b) qkv_g[b] = group();
    for (int rb = 0; rb < nrb; ++rb) {
      at_g[rb] = group();
      o_g[rb] = group();
      n2_g[rb] = group();
      gu_g[rb] = group();
      dn_g[rb] = group();
    }
    auto rq = [&](int rb) { return rb % nq0; };  // norm tiles: one queue (XCD) per row block
    // matrix-core tiles: the tile's index within its operator, round robin over
    // the queues (as a grid's workgroups go round robin over the XCDs).  With
    // 8, 64 or 8 column blocks per row block (o, gate/up, down) each XCD keeps
    // a fixed eighth of the weight columns for every row block, reused from
    // its L2, instead of streaming the whole matrix once per row block.
    auto cq = [&](int rb, int cb, int ncols) { return (rb * ncols + cb) % nq0; };
    // norms: kPNormSplit tiles of 16 rows per row block (a norm is on every
    // layer's critical path; one tile per row block took ~130 us)
    for (int rb = 0; rb < nrb; ++rb)
      for (int sub = 0; sub < kPNormSplit; ++sub)
        add(l == 0 ? P_EMBED : P_NORM1, l, l == 0 ? -1 : down_g[rb], n1_g[rb], rb, sub, rb / s.nrb_s, 0, 0, rq(rb));
    for (int rb = 0; rb < nrb; ++rb)
      for (int cb = 0; cb < ncq; ++cb)
        add(P_QKV, l, n1_g[rb], qkv_g[rb / s.nrb_s], rb, cb, rb / s.nrb_s, 0, 0, cq(rb, cb, ncq));
    for (int b = 0; b < s.B; ++b)
      for (int qb = 0; qb < s.nqb; ++qb)
        for (int g = 0; g < s.Hkv; ++g) {
          const int rb = b * s.nrb_s + qb * kPQueries / kPRows;
          const int q = (b * s.Hkv + g) % nq0;
          add(P_ATTN, l, qkv_g[b], at_g[rb], rb, 0, b, g, qb, s.split ? nq0 + q : q);
        }
    for (int rb = 0; rb < nrb; ++rb)
      for (int cb = 0; cb < nch; ++cb) add(P_OPROJ, l, at_g[rb], o_g[rb], rb, cb, rb / s.nrb_s, 0, 0, cq(rb, cb, nch));
    for (int rb = 0; rb < nrb; ++rb)
      for (int sub = 0; sub < kPNormSplit; ++sub) add(P_NORM2, l, o_g[rb], n2_g[rb], rb, sub, rb / s.nrb_s, 0, 0, rq(rb));
    for (int rb = 0; rb < nrb; ++rb)
      for (int cb = 0; cb < ncf; ++cb) add(P_GATEUP, l, n2_g[rb], gu_g[rb], rb, cb, rb / s.nrb_s, 0, 0, cq(rb, cb, ncf));
    for (int rb = 0; rb < nrb; ++rb)
      for (int cb = 0; cb < nch; ++cb) add(P_DOWN, l, gu_g[rb], dn_g[rb], rb, cb, rb / s.nrb_s, 0, 0, cq(rb, cb, nch));
    down_g = dn_g;
  }
  const int nf_g = group(), lm_g = group();
  for (int b = 0; b < s.B; ++b) {
    const int rb = b * s.nrb_s + (s.P - 1) / kPRows;
    add(P_NORMF, s.L - 1, down_g[rb], nf_g, rb, 0, b, 0, 0, b % nq0);
  }
  const int nlm = (int)ceil_div(s.V, kPLmCols);
  for (int cb = 0; cb < nlm; ++cb) add(P_LM, s.L - 1, nf_g, lm_g, 0, cb, 0, 0, 0, cb % nq0);
  add(P_ARGMAX, s.L - 1, lm_g, -1, 0, 0, 0, 0, 0, 0);

  // producers and shards: two producers per shard, up to kMaxShards (a
  // polling wave sums the shards, two per lane)
  for (const Tile& t : d.tiles)
    if (t.signal >= 0) d.groups[t.signal].producers++;
  int32_t slot = 0;
  for (Group& g : d.groups) {
    const int32_t want = std::max(1, std::min<int32_t>(kMaxShards, (g.producers + 1) / 2));
    g.shards = want;
    g.shard0 = slot;
    slot += want;
  }
  d.n_shard_slots = slot;
  std::vector<int32_t> seen(d.groups.size(), 0);
  for (Tile& t : d.tiles)
    if (t.signal >= 0) t.shard = seen[t.signal]++ % d.groups[t.signal].shards;
  d.queue_off.push_back(0);
  for (const auto& q : queues) {
    d.queue.insert(d.queue.end(), q.begin(), q.end());
    d.queue_off.push_back((int32_t)d.queue.size());
  }
  d.split_queues = s.split ? nq0 : 0;
  // operator phases (runs of one (layer, type) in id order)
  for (int32_t i = 0; i < (int32_t)d.tiles.size();) {
    int32_t j = i;
    while (j < (int32_t)d.tiles.size() && d.tiles[j].type == d.tiles[i].type && d.tiles[j].layer == d.tiles[i].layer)
      ++j;
    d.phases.push_back({i, j - i});
    i = j;
  }
  return d;
}

std::string validate_prefill_dag(const PShape& s, const PDag& d) {
  char msg[256];
  const int32_t n = (int32_t)d.tiles.size();
  std::vector<std::vector<int32_t>> producers(d.groups.size());
  for (int32_t i = 0; i < n; ++i) {
    const Tile& t = d.tiles[i];
    if (t.id != i) return "tile ids must equal their index";
    if (t.type < 0 || t.type >= P_NTYPES) return "unknown tile type";
    if (t.wait >= (int32_t)d.groups.size() || t.signal >= (int32_t)d.groups.size()) return "group id out of range";
    if (t.signal >= 0) producers[t.signal].push_back(i);
  }
  for (size_t g = 0; g < d.groups.size(); ++g) {
    if ((int32_t)producers[g].size() != d.groups[g].producers) return "group producer count mismatch";
    if (d.groups[g].shards < 1 || d.groups[g].shards > kMaxShards) return "group shard count out of range";
  }
  for (int32_t i = 0; i < n; ++i) {
    const Tile& t = d.tiles[i];
    if (t.wait < 0) {
      if (t.type != P_EMBED) return "only the embedding tiles start without a wait";
      continue;
    }
    if (producers[t.wait].empty()) return "a tile waits on a group without producers";
    if (producers[t.wait].back() >= i) {
      snprintf(msg, sizeof msg, "tile %d waits on group %d whose producer %d comes later in claim order", i, t.wait,
               producers[t.wait].back());
      return msg;
    }
  }
  // every output region exactly once
  const int nrb = s.B * s.nrb_s;
  std::map<std::tuple<int, int, int, int, int>, int> cnt;  // (type, layer, a, b, c)
  for (const Tile& t : d.tiles) {
    switch (t.type) {
      case P_EMBED: case P_NORM1: case P_NORM2: cnt[{t.type, t.layer, t.r0, t.r1, 0}]++; break;
      case P_QKV: case P_OPROJ: case P_GATEUP: case P_DOWN: cnt[{t.type, t.layer, t.r0, t.r1, 0}]++; break;
      case P_ATTN: cnt[{t.type, t.layer, t.b, t.g, t.c}]++; break;
      case P_NORMF: cnt[{t.type, t.layer, t.b, 0, 0}]++; break;
      case P_LM: cnt[{t.type, t.layer, t.r1, 0, 0}]++; break;
      default: cnt[{t.type, t.layer, 0, 0, 0}]++; break;
    }
  }
  for (const auto& kv : cnt)
    if (kv.second != 1) return "an output region is produced more than once";
  const int ncq = s.qkv_rows / kPCols, nch = s.H / kPCols, ncf = s.F / kPFfnCols;
  const int64_t want = (int64_t)s.L * nrb * (2 * kPNormSplit + ncq + 2 * nch + ncf) + (int64_t)s.L * s.B * s.nqb * s.Hkv + s.B +
                       ceil_div(s.V, kPLmCols) + 1;
  if ((int64_t)cnt.size() != want || (int64_t)n != want) return "the tiles do not cover the prefill";
  // inputs: each consumer's group holds exactly the producers of what it reads
  auto expect = [&](const Tile& t, const Tile& p) -> bool {
    switch (t.type) {
      case P_NORM1: return p.type == P_DOWN && p.layer == t.layer - 1 && p.r0 == t.r0;
      case P_QKV: return (p.type == P_EMBED || p.type == P_NORM1) && p.layer == t.layer && p.r0 == t.r0;
      case P_ATTN: return p.type == P_QKV && p.layer == t.layer && p.b == t.b;
      case P_OPROJ:
        return p.type == P_ATTN && p.layer == t.layer && p.b == t.b && p.c * kPQueries / kPRows == t.r0 % s.nrb_s;
      case P_NORM2: return p.type == P_OPROJ && p.layer == t.layer && p.r0 == t.r0;
      case P_GATEUP: return p.type == P_NORM2 && p.layer == t.layer && p.r0 == t.r0;
      case P_DOWN: return p.type == P_GATEUP && p.layer == t.layer && p.r0 == t.r0;
      case P_NORMF: return p.type == P_DOWN && p.layer == s.L - 1 && p.r0 == t.r0;
      case P_LM: return p.type == P_NORMF;
      case P_ARGMAX: return p.type == P_LM;
      default: return false;
    }
  };
  auto want_producers = [&](const Tile& t) -> int64_t {
    switch (t.type) {
      case P_NORM1: case P_NORM2: return nch;
      case P_QKV: case P_GATEUP: return kPNormSplit;
      case P_ATTN: return (int64_t)s.nrb_s * ncq;
      case P_OPROJ: {
        const int j = t.r0 % s.nrb_s;
        int nqblk = 0;
        for (int qb = 0; qb < s.nqb; ++qb) nqblk += qb * kPQueries / kPRows == j;
        return (int64_t)nqblk * s.Hkv;
      }
      case P_DOWN: return ncf;
      case P_NORMF: return nch;
      case P_LM: return s.B;
      case P_ARGMAX: return ceil_div(s.V, kPLmCols);
      default: return 0;
    }
  };
  for (const Tile& t : d.tiles) {
    if (t.wait < 0) continue;
    for (int32_t p : producers[t.wait])
      if (!expect(t, d.tiles[p])) {
        snprintf(msg, sizeof msg, "tile %d (type %d) waits on tile %d (type %d), which it does not read", t.id, t.type,
                 p, d.tiles[p].type);
        return msg;
      }
    if ((int64_t)producers[t.wait].size() != want_producers(t)) {
      snprintf(msg, sizeof msg, "tile %d (type %d) waits on %zu producers, expected %lld", t.id, t.type,
               producers[t.wait].size(), (long long)want_producers(t));
      return msg;
    }
  }
  // queues: a partition of the tiles, each in claim order; split plans keep
  // attention tiles (only) in the second region
  std::vector<int> seen(n, 0);
  const int32_t nq = (int32_t)d.queue_off.size() - 1;
  for (int32_t q = 0; q < nq; ++q) {
    int32_t last = -1;
    for (int32_t k = d.queue_off[q]; k < d.queue_off[q + 1]; ++k) {
      const int32_t id = d.queue[k];
      if (id < 0 || id >= n || id <= last) return "a claim queue is not in claim order";
      last = id;
      seen[id]++;
      if (d.split_queues && ((q >= d.split_queues) != (d.tiles[id].type == P_ATTN)))
        return "split plans keep attention tiles, and only those, in the second region";
    }
  }
  for (int32_t i = 0; i < n; ++i)
    if (seen[i] != 1) return "the claim queues do not partition the tiles";
  return "";
}

// The prefill as the planner sees it ("One Megakernel is Not Enough": the
// tile and event graph of a candidate design simulated from per-operator
// profiles).  Prefill tiles are compute-bound, so a tile's time is its
// measured cost (attention: a fixed part plus one per 32-key step of its
// causal span); no bandwidth server is modelled.
//  * megakernel / split: W workers, worker w claiming from its queue (w mod Q,
//    or its region's queues in a split plan), in queue order, a tile when its
//    worker is free; it starts when its counter group is complete plus a hop
//    and ends its cost later, publishing then;
//  * conventional: each (layer, operator) phase is one kernel over W
//    workgroup slots (a tile goes to the earliest free slot), the next
//    kernel starting a launch gap after the last tile of the previous one.
double simulate_prefill(const PShape& s, const PDag& d, const PSimCost& c, int workers, int split_workers,
                        bool conventional, double* busy_frac) {
  const int32_t n = (int32_t)d.tiles.size();
  std::vector<double> cost(n);
  double work = 0;
  for (int32_t i = 0; i < n; ++i) {
    const Tile& t = d.tiles[i];
    const double u = c.tile_us[t.type] + c.attn_step_us * prefill_key_steps(s, t);
    cost[i] = u;
    work += u;
  }
  double span = 0;
  if (conventional) {
    double t0 = 0;
    for (const auto& ph : d.phases) {
      std::priority_queue<double, std::vector<double>, std::greater<double>> slots;
      for (int w = 0; w < std::min(workers, ph.second); ++w) slots.push(t0);
      double end = t0;
      for (int32_t k = 0; k < ph.second; ++k) {
        const double st = slots.top();
        slots.pop();
        const double e = st + cost[ph.first + k];
        end = std::max(end, e);
        slots.push(e);
      }
      span = end;
      t0 = end + c.launch_gap_us;
    }
  } else {
    const int32_t nq = (int32_t)d.queue_off.size() - 1, q0 = d.split_queues ? d.split_queues : nq;
    const int w0 = workers - split_workers;
    // groups: producers remaining and completion time
    std::vector<int32_t> left(d.groups.size());
    std::vector<double> done(d.groups.size(), 0.0);
    for (size_t g = 0; g < d.groups.size(); ++g) left[g] = d.groups[g].producers;
    std::vector<double> end(n, -1.0);
    // each queue: its workers' free times; a queue's next tile goes to its
    // earliest free worker.  Tiles are processed in global claim (id) order,
    // which is topological, so every producer's end is known first.
    std::vector<std::priority_queue<double, std::vector<double>, std::greater<double>>> free_at(nq);
    for (int w = 0; w < workers; ++w) {
      const int q = !split_workers ? w % nq : w < w0 ? w % q0 : q0 + (w - w0) % (nq - q0);
      free_at[q].push(0.0);
    }
    std::vector<int32_t> queue_of(n);
    for (int32_t q = 0; q < nq; ++q)
      for (int32_t k = d.queue_off[q]; k < d.queue_off[q + 1]; ++k) queue_of[d.queue[k]] = q;
    // Claims within a queue happen in queue order as workers come free; with
    // ids in topological order and each queue's tiles in id order, replaying
    // tiles in id order assigns each to its queue's earliest free worker at
    // that point, as the device does up to ties.
    for (int32_t i = 0; i < n; ++i) {
      const Tile& t = d.tiles[i];
      auto& fq = free_at[queue_of[i]];
      const double wf = fq.top();
      fq.pop();
      double st = wf;
      if (t.wait >= 0) st = std::max(st, done[t.wait] + c.hop_us);
      end[i] = st + cost[i];
      fq.push(end[i]);
      if (t.signal >= 0) {
        done[t.signal] = std::max(done[t.signal], end[i]);
        --left[t.signal];
      }
      span = std::max(span, end[i]);
    }
  }
  if (busy_frac) *busy_frac = span > 0 ? work / (span * workers) : 0.0;
  return span;
}

int32_t prefill_key_steps(const PShape& s, const Tile& t) {
  if (t.type != P_ATTN) return 0;
  const int kend = std::min(s.P, (t.c + 1) * kPQueries);
  return (kend + kPKeys - 1) / kPKeys;
}

double prefill_flops(const PShape& s) {
  const double rows = (double)s.B * s.P;
  const double per_row = 2.0 * ((double)s.qkv_rows * s.H + (double)s.H * s.H + 2.0 * s.F * s.H + (double)s.H * s.F);
  // causal attention: query i attends to i + 1 keys; QK and PV, 2 flops per multiply-add
  const double pairs = (double)s.P * (s.P + 1) / 2.0;
  const double attn = 4.0 * pairs * s.D * s.Hq * s.B;
  return s.L * (rows * per_row + attn) + 2.0 * s.B * (double)s.V * s.H;
}

}  // namespace wpk
