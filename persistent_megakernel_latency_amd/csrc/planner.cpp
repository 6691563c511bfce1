// planner.cpp -- predicts a decode step's time for a candidate design by
// simulating its tile graph (the planner of "One Megakernel is Not Enough":
// per-operator profiles in, the tile and event graph simulated under the
// Table I feature rules, the best design out).
//
// The simulation runs the plan's own DAG, claim queues and counter groups:
//  * W workers, worker w claiming from queue w mod Q in queue order; a worker
//    claims its next tile when it stages the current one's weights (the
//    kernel's claim-ahead), so it holds at most one staged and one claimed
//    tile;
//  * one staging slot per worker (or S slots, a design candidate): a tile's
//    weights start loading when its slot is free -- the slot of the tile S
//    places earlier on the same worker (weight prefetch, Table I) -- or,
//    without prefetch, once its inputs are complete; HBM is one first-come
//    server at the streaming bandwidth, each load also paying a fixed
//    latency;
//  * a tile starts when its counter group is complete plus a hop (publish
//    seen by the poller) and its worker's previous tile has published; then
//    input staging, compute (once its weights are in) and epilogue, per tile
//    type, from measured profiles; its publish counts towards its group;
//  * barrier edges are a property of the DAG (build with barrier_edges=1), and
//    so is a split into two co-resident megakernels (split_workers): the last
//    split_workers workers then claim only the attention and combine queues,
//    the others only the rest;
//  * the conventional design runs each operator as one kernel over W
//    resident workgroups (ceil(tiles / W) waves), kernels separated by a
//    launch gap, with no hops (kernel boundaries order the operators).
#include <algorithm>
#include <cstdint>
#include <cmath>
#include <queue>
#include <vector>

#include "runtime.h"

namespace wpk {
namespace {

constexpr double kInf = 1e300;

// Bytes a tile streams from HBM (weights, or the K/V of the chunks holding
// positions of its sequence this step).
double tile_bytes(const Shape& s, const Tile& t, const int32_t* pos) {
  switch (t.type) {
    case T_QKV:
    case T_OPROJ:
    case T_GATEUP:
    case T_LM:
      return s.wide ? (double)kWideRows * kWideK * s.elt : (double)t.rows * s.H * s.elt;
    case T_DOWN:
      return s.wide ? (double)kWideRows * kWideK * s.elt : (double)t.rows * s.F * s.elt;
    case T_ATTN:
    case T_ATTNC: {
      const int p = pos ? pos[t.b] : 0;
      const int n = p < 0 ? 0 : std::min(p + 1, s.cap);
      double b = 0;
      const int c1 = t.type == T_ATTNC ? s.nch : t.c + std::max(1, t.kind);
      for (int c = t.c; c < c1; ++c) b += std::max(0, std::min(kAttnChunk, n - c * kAttnChunk));
      return b * s.D * 2.0 * s.elt;
    }
    default:
      return 0.0;
  }
}

struct Hbm {
  double bw, lat, free_at = 0;
  // a load issued at t: done after the latency, or when the server has
  // streamed it behind the loads issued before it
  double load(double t, double bytes) {
    if (bytes <= 0) return t;
    const double start = std::max(t, free_at);
    free_at = start + bytes / bw;
    return std::max(t + lat, free_at);
  }
};

// One claimed tile of a worker.  The kernel's timing relations:
//   top    = max(claim, slot free after the previous tile): the compute waves
//            reach the tile, issue the next claim, and (with prefetch) stage
//            its weights;
//   start  = max(previous publish, group complete + hop): the control wave
//            saw the inputs complete (without prefetch, the weights load now);
//   c1     = max(start + input staging, weights in) + compute;
//   pub    = c1 + epilogue;
//   slot free = pub where the kernel keeps barrier C, else c1.
struct Rec {
  int32_t tile = -1;
  double claim = 0, top = kInf, load_end = kInf, start = kInf, c1 = kInf, pub = kInf;
  double frees = kInf;  // when this tile's slot takes another tile's weights (final once started)
  bool top_sched = false, start_sched = false, waiting = false;
};

struct Worker {
  int q = 0;
  std::vector<Rec> recs;  // tiles in claim order
  size_t cur = 0;         // the tile the control wave works on next
};

enum Ev { TOP = 0, CLAIM = 1, START = 2, PUBLISH = 3 };
// Events at equal times run by kind, then first come first served (so every
// worker's first claim goes out before any claim-ahead, as at kernel start).
struct Event {
  double t;
  int kind, w;
  size_t k;
  uint64_t seq;
  bool operator>(const Event& o) const {
    if (t != o.t) return t > o.t;
    if (kind != o.kind) return kind > o.kind;
    return seq > o.seq;
  }
};

struct Sim {
  const Shape& s;
  const Dag& d;
  const wpk_sim_params& sp;
  const int32_t* pos;
  Hbm hbm;
  std::vector<Worker> ws;
  std::vector<int32_t> head;              // per queue
  std::vector<int32_t> remaining;         // per group: publishes still missing
  std::vector<double> done_at;            // per group: completion time
  std::vector<std::vector<int>> waiters;  // per group: workers whose next tile waits on it
  std::vector<int32_t> arrivals;          // matrix-core plans: K slices started, per row block
  std::priority_queue<Event, std::vector<Event>, std::greater<Event>> ev;
  uint64_t seq = 0;
  void push(double t, int kind, int w, size_t k) { ev.push(Event{t, kind, w, k, seq++}); }
  double end = 0, busy = 0, bytes = 0;

  int slots = 1;

  Sim(const Shape& s_, const Dag& d_, const wpk_sim_params& sp_, const int32_t* pos_)
      : s(s_), d(d_), sp(sp_), pos(pos_), hbm{sp_.hbm_GBps * 1e3, sp_.load_latency_us},
        slots(std::max(1, sp_.slots)) {}

  double cost(const double* a, int type) const { return type >= 0 && type < WPK_SIM_TYPES ? a[type] : 0.0; }

  // Barrier C (the next weights wait for the publish) is kept after every
  // tile except LM-head tiles and, in matrix-core plans, GEMM tiles.
  bool barrier_c(const Tile& t) const {
    const bool gemm = t.type == T_QKV || t.type == T_OPROJ || t.type == T_GATEUP || t.type == T_DOWN || t.type == T_LM;
    return !(t.type == T_LM || (s.wide && gemm));
  }

  // A matrix-core K slice's share of its row block's reduction: the slice
  // that arrives last (here: starts last) adds up the others.
  double reduction(const Tile& T) {
    if (!s.wide || T.fix < 0 || T.fix >= (int32_t)arrivals.size() || T.b <= 1) return 0.0;
    const bool gemm = T.type == T_QKV || T.type == T_OPROJ || T.type == T_GATEUP || T.type == T_DOWN || T.type == T_LM;
    if (!gemm) return 0.0;
    return ++arrivals[T.fix] == T.b ? cost(sp.reduce_us, T.type) : 0.0;
  }

  // Tile k of a worker stages into the slot that tile k - S frees.
  void schedule_top(int w, size_t k) {
    Worker& W = ws[w];
    Rec& r = W.recs[k];
    if (r.top_sched) return;
    double free_at = 0.0;
    if (k >= (size_t)slots) {
      const Rec& o = W.recs[k - slots];
      if (!o.start_sched || o.start >= kInf) return;  // not final until that tile has started
      free_at = o.frees;
    }
    r.top_sched = true;
    push(std::max(r.claim, free_at), TOP, w, k);
  }

  // The control wave takes its next tile once the previous one has published
  // and the tile's group is complete.
  void consider_start(int w, double now) {
    Worker& W = ws[w];
    if (W.cur >= W.recs.size()) return;
    Rec& r = W.recs[W.cur];
    if (r.start_sched) return;
    const double prev = W.cur == 0 ? 0.0 : W.recs[W.cur - 1].pub;
    if (prev >= kInf) return;
    const Tile& T = d.tiles[r.tile];
    double ready = prev;
    if (T.wait >= 0) {
      if (remaining[T.wait] > 0) {
        if (!r.waiting) {
          r.waiting = true;
          waiters[T.wait].push_back(w);
        }
        return;
      }
      ready = std::max(ready, done_at[T.wait] + sp.hop_us);
    }
    r.start_sched = true;
    push(std::max(ready, now), START, w, W.cur);
  }

  void claim(int w, double t) {
    Worker& W = ws[w];
    const int32_t qb = d.queue_off[W.q], qn = d.queue_off[W.q + 1] - qb;
    if (head[W.q] >= qn) return;
    Rec r;
    r.tile = d.queue[qb + head[W.q]++];
    r.claim = t;
    W.recs.push_back(r);
    schedule_top(w, W.recs.size() - 1);
    consider_start(w, t);
  }

  void run_megakernel() {
    const int nq = (int)d.queue_off.size() - 1;
    ws.assign(sp.workers, Worker{});
    head.assign(nq, 0);
    remaining.assign(d.groups.size(), 0);
    done_at.assign(d.groups.size(), 0.0);
    waiters.assign(d.groups.size(), {});
    for (size_t g = 0; g < d.groups.size(); ++g) remaining[g] = d.groups[g].producers;
    arrivals.assign(d.n_fix, 0);
    // split plans: the first megakernel's workers claim from its queues, the
    // second's (the last split_workers) from the attention and combine queues
    const int q0 = d.split_queues ? d.split_queues : nq, w1 = d.split_queues ? s.split_workers : 0;
    const int w0 = sp.workers - w1;
    for (int w = 0; w < sp.workers; ++w) {
      ws[w].q = w < w0 ? w % q0 : q0 + (w - w0) % (nq - q0);
      push(0.0, CLAIM, w, 0);
    }
    while (!ev.empty()) {
      const Event e = ev.top();
      ev.pop();
      Worker& W = ws[e.w];
      switch (e.kind) {
        case CLAIM:
          claim(e.w, e.t);
          break;
        case TOP: {
          Rec& r = W.recs[e.k];
          r.top = e.t;
          if (sp.prefetch) {
            const double b = tile_bytes(s, d.tiles[r.tile], pos);
            bytes += b;
            r.load_end = hbm.load(e.t, b);
          }
          push(e.t, CLAIM, e.w, 0);  // the next claim goes out as the slot is staged
          break;
        }
        case START: {
          Rec& r = W.recs[e.k];
          const Tile& T = d.tiles[r.tile];
          r.start = e.t;
          if (!sp.prefetch) {
            const double b = tile_bytes(s, T, pos);
            bytes += b;
            r.load_end = hbm.load(std::max(e.t, r.top), b);
          }
          const double in = e.t + cost(sp.stage_us, T.type);
          r.c1 = std::max(in, r.load_end) + cost(sp.compute_us, T.type);
          r.pub = r.c1 + cost(sp.epilogue_us, T.type) + reduction(T);
          busy += r.pub - e.t;
          r.frees = barrier_c(T) ? r.pub : r.c1;
          if (e.k + slots < W.recs.size()) schedule_top(e.w, e.k + slots);
          push(r.pub, PUBLISH, e.w, e.k);
          break;
        }
        case PUBLISH: {
          const Tile& T = d.tiles[W.recs[e.k].tile];
          end = std::max(end, e.t);
          W.cur = e.k + 1;
          if (T.signal >= 0 && --remaining[T.signal] == 0) {
            done_at[T.signal] = e.t;
            std::vector<int> wake;
            wake.swap(waiters[T.signal]);
            for (int v : wake) consider_start(v, e.t);
          }
          consider_start(e.w, e.t);
          break;
        }
      }
    }
  }

  void run_conventional() {
    arrivals.assign(d.n_fix, 0);
    double t = 0;
    for (const auto& ph : d.phases) {
      t += sp.launch_gap_us;
      std::priority_queue<double, std::vector<double>, std::greater<double>> slots;
      for (int w = 0; w < sp.workers; ++w) slots.push(t);
      double phase_end = t;
      for (int32_t i = ph.first; i < ph.first + ph.second; ++i) {
        const Tile& T = d.tiles[i];
        const double ts = slots.top();
        slots.pop();
        const double b = tile_bytes(s, T, pos);
        bytes += b;
        const double le = hbm.load(ts, b);
        const double in = ts + cost(sp.stage_us, T.type);
        const double te = std::max(in, le) + cost(sp.compute_us, T.type) + cost(sp.epilogue_us, T.type) +
                          reduction(T);
        busy += te - ts;
        slots.push(te);
        phase_end = std::max(phase_end, te);
      }
      t = phase_end;
    }
    end = t;
  }
};

}  // namespace
}  // namespace wpk

using namespace wpk;

extern "C" int32_t wpk_simulate(const wpk_plan* p, const wpk_sim_params* sp, const int32_t* positions,
                                wpk_sim_result* out) {
  if (!p || !sp || !out) return WPK_E_ARG;
  const int32_t nq = (int32_t)p->dag.queue_off.size() - 1;
  if (p->dag.split_queues && !sp->conventional &&
      (p->s.split_workers < nq - p->dag.split_queues || sp->workers - p->s.split_workers < p->dag.split_queues))
    return WPK_E_ARG;  // each megakernel needs a worker per queue
  if (sp->workers < nq || sp->workers > 65536 || !(sp->hbm_GBps > 0) ||
      sp->load_latency_us < 0 || sp->hop_us < 0 || sp->launch_gap_us < 0)
    return WPK_E_ARG;
  Sim sim(p->s, p->dag, *sp, positions);
  if (sp->conventional) sim.run_conventional();
  else sim.run_megakernel();
  out->step_us = sim.end;
  out->hbm_bytes = sim.bytes;
  out->achieved_GBps = sim.end > 0 ? sim.bytes / sim.end / 1e3 : 0.0;
  out->worker_busy_frac = sim.end > 0 ? sim.busy / (sim.end * sp->workers) : 0.0;
  return WPK_OK;
}
