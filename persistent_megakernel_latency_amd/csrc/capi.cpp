// capi.cpp -- the C ABI declared in include/wpk.h.
//
// wpk_build compiles the step for a declared operating point (model, batch
// capacity, context limit), the compile-time scheduling of "Why real-time
// inference wants a megakernel" (sections "The cohort is known" and "A
// concrete design: one WPK update"): the builder fixes the tiles, their
// dependency counters, the claim order, the worker count W and the whole
// memory plan once; wpk_step is then a single launch.
#include <hip/hip_runtime.h>

#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "host_exec.h"
#include "runtime.h"

extern "C" int wpk_dev_kernels(int dtype, int cpr_h, int cpr_f, int wide, const void** mk, const void** mk_log,
                               const void** phase, int* dyn_lds);
extern "C" int wpk_dev_persist_kernel(int dtype, int cpr_h, int cpr_f, int wide, const void** k);
extern "C" int wpk_dev_block_threads();
extern "C" int wpk_dev_static_scratch(int device, void** ptr, size_t* bytes);

using namespace wpk;

namespace {

thread_local std::string g_err;

// The static plan that currently owns each device's scratch array (plans
// built by wpk_build_static share one array per device; the latest owns it).
std::mutex g_owner_mu;
std::map<int, const wpk_plan*> g_scratch_owner;

wpk_plan* fail(const std::string& m) {
  g_err = m;
  return nullptr;
}

std::string hip_msg(const char* what, hipError_t e) { return std::string(what) + ": " + hipGetErrorString(e); }

int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

struct Layout {
  int64_t ctl, heads, counters, argmax, tiles, qtiles, groups, queue, queue_off, layers, rope_cos, rope_sin, act, log,
      wpart, fixc, step_times, wqueue, total;
};

Layout layout(const Shape& s, const Dag& d, int32_t max_workers) {
  Layout L{};
  int64_t at = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = at;
    at = align256(at + bytes);
    return o;
  };
  const int32_t nq = (int32_t)d.queue_off.size() - 1;
  L.ctl = take(CTL_WORDS * 4);
  L.heads = take((int64_t)nq * kLine * 4);
  L.counters = take((int64_t)d.n_shard_slots * kLine * 4);
  L.argmax = take((int64_t)s.B * kArgmaxShards * 8);
  L.tiles = take((int64_t)d.tiles.size() * sizeof(Tile));
  L.qtiles = take((int64_t)d.queue.size() * sizeof(Tile));
  L.groups = take((int64_t)d.groups.size() * sizeof(Group));
  L.queue = take((int64_t)d.queue.size() * 4);
  L.queue_off = take((int64_t)d.queue_off.size() * 4);
  L.layers = take((int64_t)s.L * sizeof(LayerBufs));
  L.rope_cos = take((int64_t)s.cap * (s.D / 2) * 4);
  L.rope_sin = take((int64_t)s.cap * (s.D / 2) * 4);
  L.act = take(act_layout(s).total * 4);
  // tile records, worker records, tile timings (two record sizes each)
  L.log = take((3 * (int64_t)d.tiles.size() + max_workers) * sizeof(wpk_log_rec));
  L.wpart = take((int64_t)d.n_pslots * kWidePart * 4);
  L.fixc = take((int64_t)d.n_fix * kLine * 4);
  L.step_times = take((int64_t)kPersistTimes * 2 * 8);
  L.wqueue = take((int64_t)max_workers * 4);
  L.total = at;
  return L;
}

void copy_tables(wpk_plan* p, const wpk_model_desc& d) {
  const int L = d.n_layers;
  p->desc = d;
  p->tables.resize(7 * (size_t)L);
  const void* const* src[7] = {(const void* const*)d.attn_norm, d.w_qkv, d.w_o, (const void* const*)d.mlp_norm,
                               d.w_gate, d.w_up, d.w_down};
  for (int k = 0; k < 7; ++k)
    for (int l = 0; l < L; ++l) p->tables[(size_t)k * L + l] = src[k][l];
  p->desc.attn_norm = (const float* const*)&p->tables[0];
  p->desc.w_qkv = &p->tables[(size_t)1 * L];
  p->desc.w_o = &p->tables[(size_t)2 * L];
  p->desc.mlp_norm = (const float* const*)&p->tables[(size_t)3 * L];
  p->desc.w_gate = &p->tables[(size_t)4 * L];
  p->desc.w_up = &p->tables[(size_t)5 * L];
  p->desc.w_down = &p->tables[(size_t)6 * L];
}

bool desc_ok(const wpk_model_desc* d, std::string* why) {
  if (!d) {
    *why = "null model description";
    return false;
  }
  if (!d->embed || !d->final_norm || !d->attn_norm || !d->w_qkv || !d->w_o || !d->mlp_norm || !d->w_gate ||
      !d->w_up || !d->w_down || d->n_layers <= 0) {
    *why = "model description has a null pointer or no layers";
    return false;
  }
  for (int l = 0; l < d->n_layers; ++l)
    if (!d->attn_norm[l] || !d->w_qkv[l] || !d->w_o[l] || !d->mlp_norm[l] || !d->w_gate[l] || !d->w_up[l] ||
        !d->w_down[l]) {
      *why = "null weight pointer in layer " + std::to_string(l);
      return false;
    }
  return true;
}

wpk_plan* build_device(const wpk_model_desc* desc, int32_t batch, int32_t ctx_len, const wpk_build_opts* opts,
                       bool baseline, bool static_ws = false) {
  std::string why;
  if (!desc_ok(desc, &why)) return fail(why);
  wpk_build_opts o{};
  if (opts) o = *opts;
  Shape s;
  why = check_shape(*desc, batch, ctx_len, o, &s);
  if (!why.empty()) return fail(why);
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) return fail("no HIP device");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(hip_msg("hipGetDevice", e));
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return fail(hip_msg("hipGetDeviceProperties", e));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(std::string("built for gfx950, found ") + prop.gcnArchName);
  const void *mk = nullptr, *mk_log = nullptr, *phase = nullptr, *persist = nullptr;
  int dyn = 0;
  (void)wpk_dev_persist_kernel(s.dtype, s.cpr_h, s.cpr_f, s.wide, &persist);
  if (!wpk_dev_kernels(s.dtype, s.cpr_h, s.cpr_f, s.wide, &mk, &mk_log, &phase, &dyn))
    return fail("no kernel instance for this dtype / hidden / ffn / batch (cpr_h=" + std::to_string(s.cpr_h) +
                ", cpr_f=" + std::to_string(s.cpr_f) + ", wide=" + std::to_string(s.wide) + ")");
  if (dyn > 0)
    for (const void* k : {mk, mk_log, phase}) {
      e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, dyn);
      if (e != hipSuccess) return fail(hip_msg("dynamic LDS size", e));
    }

  std::unique_ptr<wpk_plan> p(new wpk_plan());
  p->baseline = baseline;
  p->s = s;
  p->device = dev;
  p->n_cu = prop.multiProcessorCount;
  copy_tables(p.get(), *desc);
  p->dag = build_dag(s);
  why = validate_dag(s, p->dag);
  if (!why.empty()) return fail("invalid DAG: " + why);
  why = check_device_geometry(s, p->dag);
  if (!why.empty()) return fail(why);
  for (const Tile& t : p->dag.tiles) p->built_wait.push_back(t.wait);
  p->weight_bytes = step_weight_bytes(s);
  p->k_mega = mk;
  p->k_mega_log = mk_log;
  p->k_phase = phase;
  p->k_persist = persist;
  p->dyn_lds = dyn;

  int per_cu = 0, per_cu_log = 0;
  const int block = wpk_dev_block_threads();
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, mk, block, dyn);
  if (e != hipSuccess) return fail(hip_msg("occupancy query", e));
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_log, mk_log, block, dyn);
  if (e != hipSuccess) return fail(hip_msg("occupancy query", e));
  per_cu = std::min(per_cu, per_cu_log);
  p->max_workers = per_cu * p->n_cu;
  p->workers = std::min(s.workers_per_cu, per_cu) * p->n_cu;
  if (p->workers < s.queue_shards) {
    g_err = "occupancy too low: " + std::to_string(p->max_workers) + " co-resident workers";
    return nullptr;
  }
  if (s.split_workers > 0) {
    if (baseline || static_ws) return fail("split_workers: megakernel plans from wpk_build_ex only");
    const int w1 = s.split_workers;
    if (w1 < s.queue_shards || p->workers - w1 < s.queue_shards)
      return fail("split_workers must leave each megakernel at least one worker per claim queue (" +
                  std::to_string(s.queue_shards) + ") of the " + std::to_string(p->workers) + " workers");
    p->split_workers = w1;
  }

  const Layout L = layout(s, p->dag, p->max_workers);
  if (static_ws) {
    // no allocation: the workspace is this device's scratch array
    void* sp = nullptr;
    size_t cap_bytes = 0;
    const int rc = wpk_dev_static_scratch(dev, &sp, &cap_bytes);
    if (rc != WPK_OK) return fail("static scratch: address lookup failed on device " + std::to_string(dev));
    if ((size_t)L.total > cap_bytes)
      return fail("static scratch: this plan needs a " + std::to_string(L.total) + "-byte workspace, above the " +
                  std::to_string(cap_bytes) + "-byte static array (use wpk_build)");
    p->d_ws = (char*)sp;
    p->static_ws = true;
  } else {
    e = hipMalloc((void**)&p->d_ws, L.total);
    if (e != hipSuccess) return fail(hip_msg("hipMalloc workspace", e));
  }
  p->ws_bytes = L.total;
  auto release_ws = [&]() {
    if (!p->static_ws) (void)hipFree(p->d_ws);
    p->d_ws = nullptr;
  };
  char* w = p->d_ws;
  auto up = [&](int64_t off, const void* src, size_t bytes) { return hipMemcpy(w + off, src, bytes, hipMemcpyHostToDevice); };
  e = hipMemset(w, 0, L.total);
  std::vector<LayerBufs> lbs;
  fill_layers(s, p->desc, (float*)(w + L.act), lbs);
  std::vector<float> rc, rsn;
  rope_table(s, rc, rsn);
  if (e == hipSuccess) e = up(L.tiles, p->dag.tiles.data(), p->dag.tiles.size() * sizeof(Tile));
  std::vector<Tile> qt;
  for (int32_t id : p->dag.queue) qt.push_back(p->dag.tiles[id]);
  if (e == hipSuccess) e = up(L.qtiles, qt.data(), qt.size() * sizeof(Tile));
  if (e == hipSuccess) e = up(L.groups, p->dag.groups.data(), p->dag.groups.size() * sizeof(Group));
  if (e == hipSuccess) e = up(L.queue, p->dag.queue.data(), p->dag.queue.size() * 4);
  if (e == hipSuccess) e = up(L.queue_off, p->dag.queue_off.data(), p->dag.queue_off.size() * 4);
  if (e == hipSuccess) e = up(L.layers, lbs.data(), lbs.size() * sizeof(LayerBufs));
  if (e == hipSuccess) e = up(L.rope_cos, rc.data(), rc.size() * 4);
  if (e == hipSuccess) e = up(L.rope_sin, rsn.data(), rsn.size() * 4);
  {
    // each worker's claim queue (split plans: the first megakernel's workers
    // over its queues, the last split_workers over the attention queues)
    const int32_t nq = (int32_t)p->dag.queue_off.size() - 1, q0 = p->dag.split_queues;
    const int32_t w0 = p->workers - p->split_workers;
    std::vector<int32_t> wq(p->max_workers);
    for (int32_t w = 0; w < p->max_workers; ++w)
      wq[w] = !p->split_workers ? w % nq : w < w0 ? w % q0 : q0 + (w - w0) % (nq - q0);
    if (e == hipSuccess) e = up(L.wqueue, wq.data(), wq.size() * 4);
  }
  if (e != hipSuccess) {
    release_ws();
    return fail(hip_msg("workspace upload", e));
  }
  Params& P = p->P;
  P.L = s.L; P.H = s.H; P.Hq = s.Hq; P.Hkv = s.Hkv; P.D = s.D; P.F = s.F; P.V = s.V;
  P.B = s.B; P.cap = s.cap; P.nch = s.nch; P.G = s.G; P.qkv_rows = s.qkv_rows;
  P.attn_sub = s.attn_sub;
  P.n_tiles = (int32_t)p->dag.tiles.size();
  P.n_queues = (int32_t)p->dag.queue_off.size() - 1;
  P.n_workers = p->workers;  // both megakernels' workers: the exit count
  P.worker_queue = (const int32_t*)(w + L.wqueue);
  P.dtype = s.dtype;
  P.eps = s.eps;
  P.attn_scale = 1.0f / std::sqrt((float)s.D);
  P.embed = p->desc.embed;
  P.final_norm = p->desc.final_norm;
  P.layers = (const LayerBufs*)(w + L.layers);
  {
    const ActLayout a = act_layout(s);
    P.act = (float*)(w + L.act);
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
    P.wpart = (float*)(w + L.wpart);
    P.fixc = (uint32_t*)(w + L.fixc);
    for (int l = 0; l < s.L; ++l)
      P.lw[l] = LayerW{p->desc.w_qkv[l], p->desc.w_o[l], p->desc.w_gate[l], p->desc.w_up[l], p->desc.w_down[l],
                       p->desc.attn_norm[l], p->desc.mlp_norm[l]};
  }
  P.rope_cos = (const float*)(w + L.rope_cos);
  P.rope_sin = (const float*)(w + L.rope_sin);
  P.tiles = (const Tile*)(w + L.tiles);
  P.qtiles = (const Tile*)(w + L.qtiles);
  P.queue = (const int32_t*)(w + L.queue);
  P.queue_off = (const int32_t*)(w + L.queue_off);
  P.groups = (const Group*)(w + L.groups);
  P.counters = (uint32_t*)(w + L.counters);
  P.heads = (uint32_t*)(w + L.heads);
  P.ctl = (uint32_t*)(w + L.ctl);
  P.argmax = (unsigned long long*)(w + L.argmax);
  P.log = (int32_t*)(w + L.log);
  P.log_workers = p->max_workers;
  P.log_on = 0;
  P.prefetch = 1;
  P.drop_tile = -1;
  P.perturb = 0;
  P.watchdog_ticks = p->watchdog_us * 100;
  P.persist = 0;
  P.step_times = (uint64_t*)(w + L.step_times);
  p->d_step_times = P.step_times;
  p->log.assign(p->dag.tiles.size(), wpk_log_rec{});
  if (baseline) {
    hipStream_t cs;
    e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
    if (e != hipSuccess) {
      release_ws();
      return fail(hip_msg("hipStreamCreate", e));
    }
    p->cap_stream = cs;
  }
  if (static_ws) {
    std::lock_guard<std::mutex> lk(g_owner_mu);
    g_scratch_owner[dev] = p.get();
  }
  return p.release();
}

int32_t plan_fail(wpk_plan* p, int32_t code, const std::string& m) {
  if (p) p->err = m;
  else g_err = m;
  return code;
}

int32_t capture_baseline(wpk_plan* p) {
  if (p->graph_exec) {
    (void)hipGraphExecDestroy((hipGraphExec_t)p->graph_exec);
    p->graph_exec = nullptr;
  }
  if (p->graph) {
    (void)hipGraphDestroy((hipGraph_t)p->graph);
    p->graph = nullptr;
  }
  hipStream_t cs = (hipStream_t)p->cap_stream;
  hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return plan_fail(p, WPK_E_HIP, hip_msg("hipStreamBeginCapture", e));
  for (const auto& ph : p->dag.phases) {
    int32_t first = ph.first;
    void* args[] = {(void*)&p->P, (void*)&first};
    e = hipLaunchKernel(p->k_phase, dim3(ph.second), dim3(wpk_dev_block_threads()), args, p->dyn_lds, cs);
    if (e != hipSuccess) break;
  }
  hipGraph_t g = nullptr;
  const hipError_t e2 = hipStreamEndCapture(cs, &g);
  if (e != hipSuccess) return plan_fail(p, WPK_E_HIP, hip_msg("baseline launch during capture", e));
  if (e2 != hipSuccess) return plan_fail(p, WPK_E_HIP, hip_msg("hipStreamEndCapture", e2));
  hipGraphExec_t ge = nullptr;
  e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    return plan_fail(p, WPK_E_HIP, hip_msg("hipGraphInstantiate", e));
  }
  p->graph = g;
  p->graph_exec = ge;
  return WPK_OK;
}

}  // namespace

extern "C" {

wpk_plan* wpk_build(const wpk_model_desc* desc, int32_t batch, int32_t ctx_len) {
  return build_device(desc, batch, ctx_len, nullptr, false);
}

wpk_plan* wpk_build_ex(const wpk_model_desc* desc, int32_t batch, int32_t ctx_len, const wpk_build_opts* opts) {
  return build_device(desc, batch, ctx_len, opts, false);
}

wpk_plan* wpk_build_graph_baseline(const wpk_model_desc* desc, int32_t batch, int32_t ctx_len) {
  return build_device(desc, batch, ctx_len, nullptr, true);
}

wpk_plan* wpk_build_static(const wpk_model_desc* desc, int32_t batch, int32_t ctx_len) {
  return build_device(desc, batch, ctx_len, nullptr, false, true);
}

int32_t wpk_step(wpk_plan* p, int32_t* tokens, wpk_kv* kv, void* logits, wpk_stream_t stream) {
  if (!p) return plan_fail(nullptr, WPK_E_ARG, "null plan");
  if (p->host) return plan_fail(p, WPK_E_ARG, "host plan: use wpk_serial_step / wpk_emulate_step");
  if (p->latched) return plan_fail(p, WPK_E_STATE, "plan holds device error " + std::to_string(p->latched) + "; reset it");
  if (p->persist_open) return plan_fail(p, WPK_E_STATE, "a persistent session is open on this plan");
  if (!tokens || !kv || !kv->k || !kv->v || !kv->seq_len || !logits)
    return plan_fail(p, WPK_E_ARG, "null tokens, kv or logits");
  if (p->static_ws) {
    std::lock_guard<std::mutex> lk(g_owner_mu);
    if (g_scratch_owner[p->device] != p)
      return plan_fail(p, WPK_E_STATE, "the static scratch of device " + std::to_string(p->device) +
                                           " now holds a later static plan's workspace; rebuild this plan");
  }
  hipStream_t st = (hipStream_t)stream;
  Params& P = p->P;
  P.tokens = tokens;
  P.seq_len = kv->seq_len;
  P.logits = (float*)logits;
  P.kc = (char*)kv->k;
  P.vc = (char*)kv->v;
  p->last_stream = stream;
  hipError_t e;
  if (p->baseline) {
    if (!p->graph_exec || p->cap_tokens != tokens || p->cap_kc != kv->k || p->cap_vc != kv->v ||
        p->cap_seq != kv->seq_len || p->cap_logits != logits) {
      const int32_t rc = capture_baseline(p);
      if (rc != WPK_OK) return rc;
      p->cap_tokens = tokens;
      p->cap_kc = kv->k;
      p->cap_vc = kv->v;
      p->cap_seq = kv->seq_len;
      p->cap_logits = logits;
    }
    e = hipGraphLaunch((hipGraphExec_t)p->graph_exec, st);
    if (e != hipSuccess) return plan_fail(p, WPK_E_HIP, hip_msg("hipGraphLaunch", e));
    return WPK_OK;
  }
  P.log_on = p->log_on;
  if (p->log_on) {
    e = hipMemsetAsync(P.log, 0, (3 * p->dag.tiles.size() + p->max_workers) * sizeof(wpk_log_rec), st);
    if (e != hipSuccess) return plan_fail(p, WPK_E_HIP, hip_msg("hipMemsetAsync log", e));
  }
  void* args[] = {(void*)&P};
  if (!p->cooperative)
    e = hipLaunchKernel(p->log_on ? p->k_mega_log : p->k_mega, dim3(p->workers), dim3(wpk_dev_block_threads()),
                        args, p->dyn_lds, st);
  else
    e = hipLaunchCooperativeKernel(p->log_on ? p->k_mega_log : p->k_mega, dim3(p->workers),
                                   dim3(wpk_dev_block_threads()), args, p->dyn_lds, st);
  if (e != hipSuccess) return plan_fail(p, WPK_E_HIP, hip_msg("megakernel launch", e));
  return WPK_OK;
}

int32_t wpk_sync(wpk_plan* p) {
  if (!p) return plan_fail(nullptr, WPK_E_ARG, "null plan");
  if (p->host) return WPK_OK;
  if (p->persist_open) return plan_fail(p, WPK_E_STATE, "a persistent session is open: use wpk_persist_end");
  hipError_t e = hipStreamSynchronize((hipStream_t)p->last_stream);
  if (e != hipSuccess) return plan_fail(p, WPK_E_HIP, hip_msg("hipStreamSynchronize", e));
  uint32_t st[4];
  e = hipMemcpy(st, p->P.ctl + CTL_STATUS, sizeof st, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return plan_fail(p, WPK_E_HIP, hip_msg("status read", e));
  if (st[0] != 0) {
    p->latched = (int32_t)st[0];
    char m[320];
    snprintf(m, sizeof m, "device error %d at tile %u (worker %u, step %u)", (int32_t)st[0], st[1], st[2], st[3]);
    p->err = m;
    if ((int32_t)st[0] == WPK_E_TIMEOUT) {
      // Name the root cause: the first counter group (groups are numbered in
      // topological order) that did not receive all of its increments.
      std::vector<uint32_t> ctr((size_t)p->dag.n_shard_slots * kLine);
      if (hipMemcpy(ctr.data(), p->P.counters, ctr.size() * 4, hipMemcpyDeviceToHost) == hipSuccess) {
        for (size_t g = 0; g < p->dag.groups.size(); ++g) {
          const Group& G = p->dag.groups[g];
          uint32_t sum = 0;
          for (int s = 0; s < G.shards; ++s) sum += ctr[(size_t)(G.shard0 + s) * kLine];
          const uint32_t target = (st[3] + 1u) * (uint32_t)G.producers;
          if ((int32_t)(sum - target) < 0) {
            snprintf(m, sizeof m, "; first incomplete group %zu: %d of %d publishes this step", g,
                     (int32_t)(sum - st[3] * (uint32_t)G.producers), G.producers);
            p->err += m;
            break;
          }
        }
      }
    }
    return p->latched;
  }
  return WPK_OK;
}

void wpk_destroy(wpk_plan* p) {
  if (!p) return;
  if (p->persist_open) (void)wpk_persist_end(p);
  if (p->host_words) (void)hipHostFree(p->host_words);
  if (p->graph_exec) (void)hipGraphExecDestroy((hipGraphExec_t)p->graph_exec);
  if (p->graph) (void)hipGraphDestroy((hipGraph_t)p->graph);
  if (p->cap_stream) (void)hipStreamDestroy((hipStream_t)p->cap_stream);

  if (p->d_ws) {
    (void)hipDeviceSynchronize();
    if (p->static_ws) {
      std::lock_guard<std::mutex> lk(g_owner_mu);
      if (g_scratch_owner[p->device] == p) g_scratch_owner.erase(p->device);
    } else {
      (void)hipFree(p->d_ws);
    }
  }
  delete p;
}

const char* wpk_last_error(const wpk_plan* p) { return p ? p->err.c_str() : g_err.c_str(); }

int32_t wpk_set_option(wpk_plan* p, int32_t key, int64_t value) {
  if (!p) return plan_fail(nullptr, WPK_E_ARG, "null plan");
  Params& P = p->P;
  switch (key) {
    case WPK_OPT_LOG:
      p->log_on = value != 0;
      return WPK_OK;
    case WPK_OPT_WATCHDOG_US:
      if (value <= 0) return plan_fail(p, WPK_E_ARG, "watchdog must be positive");
      p->watchdog_us = (uint64_t)value;
      P.watchdog_ticks = (uint64_t)value * 100;
      return WPK_OK;
    case WPK_OPT_PERTURB_SEED:
      P.perturb = (uint32_t)value;
      p->perturb = (uint32_t)value;
      return WPK_OK;
    case WPK_OPT_DEBUG_DROP_TILE:
      if (value < -1 || value >= (int64_t)p->dag.tiles.size()) return plan_fail(p, WPK_E_ARG, "tile out of range");
      P.drop_tile = (int32_t)value;
      p->drop_tile = (int32_t)value;
      return WPK_OK;
    case WPK_OPT_PREFETCH:
      P.prefetch = value != 0;
      p->prefetch = (int32_t)(value != 0);
      return WPK_OK;
    case WPK_OPT_LAUNCH:
      if (value != 0 && value != 1) return plan_fail(p, WPK_E_ARG, "launch must be 0 or 1");
      p->cooperative = (int32_t)value;
      return WPK_OK;
    case WPK_OPT_PERSIST_IDLE_US:
      if (value <= 0) return plan_fail(p, WPK_E_ARG, "idle limit must be positive");
      p->persist_idle_us = (uint64_t)value;
      return WPK_OK;
    case WPK_OPT_FIXED_REDUCER:
      if (!p->host) return plan_fail(p, WPK_E_ARG, "the fixed reducer is an option of the host emulator only");
      if (value != 0 && value != 1) return plan_fail(p, WPK_E_ARG, "fixed reducer must be 0 or 1");
      p->emu_fixed_reducer = (int32_t)value;
      return WPK_OK;
    case WPK_OPT_WORKERS:
      if (value < (int64_t)p->s.queue_shards || value > p->max_workers)
        return plan_fail(p, WPK_E_ARG, "workers must be in [queue shards, max co-resident]");
      if (p->split_workers) return plan_fail(p, WPK_E_ARG, "a split plan's worker counts are fixed when it is built");
      p->workers = (int32_t)value;
      P.n_workers = (int32_t)value;
      return WPK_OK;
    case WPK_OPT_RESET: {
      if (p->host) {
        p->latched = 0;
        return WPK_OK;
      }
      hipError_t e = hipDeviceSynchronize();
      if (e == hipSuccess) e = hipMemset(P.ctl, 0, CTL_WORDS * 4);
      if (e == hipSuccess) e = hipMemset(P.heads, 0, (size_t)P.n_queues * kLine * 4);
      if (e == hipSuccess) e = hipMemset(P.counters, 0, (size_t)p->dag.n_shard_slots * kLine * 4);
      if (e == hipSuccess) e = hipMemset(P.argmax, 0, (size_t)p->s.B * kArgmaxShards * 8);
      if (e == hipSuccess && p->dag.n_fix) e = hipMemset(P.fixc, 0, (size_t)p->dag.n_fix * kLine * 4);
      if (e == hipSuccess) e = hipDeviceSynchronize();
      if (e != hipSuccess) return plan_fail(p, WPK_E_HIP, hip_msg("reset", e));
      p->latched = 0;
      return WPK_OK;
    }
  }
  return plan_fail(p, WPK_E_ARG, "unknown option key");
}

int32_t wpk_get_log(wpk_plan* p, void* dst, size_t bytes) {
  if (!p || !dst) return plan_fail(p, WPK_E_ARG, "null argument");
  const size_t need = p->dag.tiles.size() * sizeof(wpk_log_rec);
  if (bytes < need) return plan_fail(p, WPK_E_ARG, "log buffer too small");
  if (p->host) {
    std::memcpy(dst, p->log.data(), need);
    return WPK_OK;
  }
  // with room for them, the worker record slots and the tile timings follow
  const size_t full = (3 * p->dag.tiles.size() + p->max_workers) * sizeof(wpk_log_rec);
  hipError_t e = hipMemcpy(dst, p->P.log, bytes >= full ? full : need, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return plan_fail(p, WPK_E_HIP, hip_msg("log read", e));
  return WPK_OK;
}

int32_t wpk_get_info(const wpk_plan* p, wpk_plan_info* out) {
  if (!p || !out) return WPK_E_ARG;
  out->n_tiles = (int32_t)p->dag.tiles.size();
  out->n_groups = (int32_t)p->dag.groups.size();
  out->n_queue_shards = (int32_t)p->dag.queue_off.size() - 1;
  out->workers = p->workers;
  out->max_workers = p->max_workers;
  out->rows_per_tile_h = p->s.rows_h;
  out->rows_per_tile_f = p->s.rows_f;
  out->attn_chunk = kAttnChunk;
  out->workspace_bytes = p->ws_bytes;
  out->weight_bytes = p->weight_bytes;
  return WPK_OK;
}

int32_t wpk_get_dag(const wpk_plan* p, int32_t* type, int32_t* layer, int32_t* wait, int32_t* signal) {
  if (!p || !type || !layer || !wait || !signal) return WPK_E_ARG;
  for (size_t i = 0; i < p->dag.tiles.size(); ++i) {
    type[i] = p->dag.tiles[i].type;
    layer[i] = p->dag.tiles[i].layer;
    wait[i] = p->dag.tiles[i].wait;
    signal[i] = p->dag.tiles[i].signal;
  }
  return WPK_OK;
}

wpk_plan* wpk_build_host(const wpk_model_desc* desc, int32_t batch, int32_t ctx_len, const wpk_build_opts* opts) {
  std::string why;
  if (!desc_ok(desc, &why)) return fail(why);
  wpk_build_opts o{};
  if (opts) o = *opts;
  wpk_plan* p = make_host_plan(*desc, batch, ctx_len, o, &why);
  if (!p) return fail(why);
  return p;
}

int32_t wpk_serial_step(wpk_plan* p, int32_t* tokens, wpk_kv* kv, float* logits, uint64_t order_seed, int32_t poison) {
  if (!p || !p->host) return plan_fail(p, WPK_E_ARG, "wpk_serial_step needs a host plan");
  return host_serial_step(p, tokens, kv, logits, order_seed, poison != 0);
}

int32_t wpk_emulate_step(wpk_plan* p, int32_t* tokens, wpk_kv* kv, float* logits, int32_t n_threads, uint64_t seed) {
  if (!p || !p->host) return plan_fail(p, WPK_E_ARG, "wpk_emulate_step needs a host plan");
  return host_emulate_step(p, tokens, kv, logits, n_threads, seed);
}

int32_t wpk_debug_read_act(wpk_plan* p, void* dst, size_t bytes, size_t* out_bytes) {
  if (!p) return plan_fail(nullptr, WPK_E_ARG, "null plan");
  const size_t need = (size_t)act_layout(p->s).total * 4;
  if (out_bytes) *out_bytes = need;
  if (!dst) return WPK_OK;
  if (bytes < need) return plan_fail(p, WPK_E_ARG, "buffer smaller than the activation arena");
  if (p->host) {
    std::memcpy(dst, p->hw.act.data(), need);
    return WPK_OK;
  }
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(dst, p->P.act, need, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return plan_fail(p, WPK_E_HIP, hip_msg("activation read", e));
  return WPK_OK;
}

// ---- cross-step persistence ---------------------------------------------------------------

int32_t wpk_persist_begin(wpk_plan* p, int32_t* tokens, wpk_kv* kv, void* logits, wpk_stream_t stream) {
  if (!p) return plan_fail(nullptr, WPK_E_ARG, "null plan");
  if (p->host || p->baseline) return plan_fail(p, WPK_E_ARG, "persistent sessions run megakernel device plans");
  if (!p->k_persist)
    return plan_fail(p, WPK_E_ARG, "persistent sessions are built for batches up to 4 (no matrix-core instance)");
  if (p->split_workers) return plan_fail(p, WPK_E_ARG, "persistent sessions run one megakernel (not a split plan)");
  if (p->persist_open) return plan_fail(p, WPK_E_STATE, "a persistent session is already open");
  if (p->latched) return plan_fail(p, WPK_E_STATE, "plan holds device error " + std::to_string(p->latched) + "; reset it");
  if (p->log_on) return plan_fail(p, WPK_E_ARG, "the per-tile log records one step: switch it off first");
  if (!tokens || !kv || !kv->k || !kv->v || !kv->seq_len || !logits)
    return plan_fail(p, WPK_E_ARG, "null tokens, kv or logits");
  if (p->static_ws) {
    std::lock_guard<std::mutex> lk(g_owner_mu);
    if (g_scratch_owner[p->device] != p)
      return plan_fail(p, WPK_E_STATE, "the static scratch now holds a later static plan's workspace");
  }
  hipError_t e = hipSuccess;
  if (!p->host_words) {
    e = hipHostMalloc((void**)&p->host_words, 512, hipHostMallocCoherent | hipHostMallocMapped);
    if (e != hipSuccess) return plan_fail(p, WPK_E_NOMEM, hip_msg("hipHostMalloc doorbell", e));
  }
  // the plan is idle: its last step (if any) is finished
  if (p->last_stream) {
    e = hipStreamSynchronize((hipStream_t)p->last_stream);
    if (e != hipSuccess) return plan_fail(p, WPK_E_HIP, hip_msg("hipStreamSynchronize", e));
  }
  uint32_t epoch = 0;
  e = hipMemcpy(&epoch, p->P.ctl + CTL_EPOCH, 4, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpy(p->P.ctl + CTL_GO, &epoch, 4, hipMemcpyHostToDevice);  // nothing granted yet
  if (e != hipSuccess) return plan_fail(p, WPK_E_HIP, hip_msg("session setup", e));
  __atomic_store_n(&p->host_words[0], 0u, __ATOMIC_RELEASE);
  __atomic_store_n(&p->host_words[64], 0u, __ATOMIC_RELEASE);
  p->persist_requested = 0;
  Params P = p->P;
  P.tokens = tokens;
  P.seq_len = kv->seq_len;
  P.logits = (float*)logits;
  P.kc = (char*)kv->k;
  P.vc = (char*)kv->v;
  P.log_on = 0;
  P.persist = 1;
  P.persist_base = epoch;
  uint32_t* dev_words = nullptr;
  e = hipHostGetDevicePointer((void**)&dev_words, p->host_words, 0);
  if (e != hipSuccess || !dev_words) return plan_fail(p, WPK_E_HIP, hip_msg("hipHostGetDevicePointer", e));
  P.host_bell = dev_words;
  P.host_done = dev_words + 64;
  P.idle_ticks = p->persist_idle_us * 100;
  void* args[] = {(void*)&P};
  // every worker waits for every other at each step boundary: the grid must
  // be co-resident, which a cooperative launch guarantees (or refuses)
  e = hipLaunchCooperativeKernel(p->k_persist, dim3(p->workers), dim3(wpk_dev_block_threads()), args, p->dyn_lds,
                                 (hipStream_t)stream);
  if (e != hipSuccess) return plan_fail(p, WPK_E_HIP, hip_msg("persistent launch", e));
  p->last_stream = stream;
  p->persist_open = true;
  return WPK_OK;
}

int32_t wpk_persist_ring(wpk_plan* p, int32_t n_steps) {
  if (!p) return plan_fail(nullptr, WPK_E_ARG, "null plan");
  if (!p->persist_open) return plan_fail(p, WPK_E_STATE, "no persistent session is open");
  if (n_steps <= 0 || (uint64_t)p->persist_requested + (uint64_t)n_steps >= kBellStop)
    return plan_fail(p, WPK_E_ARG, "n_steps must be positive");
  p->persist_requested += (uint32_t)n_steps;
  __atomic_store_n(&p->host_words[0], p->persist_requested, __ATOMIC_RELEASE);
  return WPK_OK;
}

int32_t wpk_persist_wait(wpk_plan* p, int32_t steps, int64_t timeout_us) {
  if (!p) return plan_fail(nullptr, WPK_E_ARG, "null plan");
  if (!p->persist_open) return plan_fail(p, WPK_E_STATE, "no persistent session is open");
  if (steps < 0 || (uint32_t)steps > p->persist_requested)
    return plan_fail(p, WPK_E_ARG, "can only wait for steps that were rung");
  const auto t0 = std::chrono::steady_clock::now();
  for (uint64_t k = 0;; ++k) {
    if (__atomic_load_n(&p->host_words[64], __ATOMIC_ACQUIRE) >= (uint32_t)steps) return WPK_OK;
    if ((k & 1023u) == 1023u) {
      // the grid left early (an error, or its idle limit): report it
      if (hipStreamQuery((hipStream_t)p->last_stream) == hipSuccess) {
        if (__atomic_load_n(&p->host_words[64], __ATOMIC_ACQUIRE) >= (uint32_t)steps) return WPK_OK;
        return plan_fail(p, WPK_E_STATE, "the persistent grid has left; wpk_persist_end reports why");
      }
      if (timeout_us >= 0 &&
          std::chrono::steady_clock::now() - t0 > std::chrono::microseconds(timeout_us))
        return plan_fail(p, WPK_E_TIMEOUT, "persistent steps not done within the timeout");
    }
  }
}

int32_t wpk_persist_end(wpk_plan* p) {
  if (!p) return plan_fail(nullptr, WPK_E_ARG, "null plan");
  if (!p->persist_open) return plan_fail(p, WPK_E_STATE, "no persistent session is open");
  // the steps already rung run first; then the stop bell
  (void)wpk_persist_wait(p, (int32_t)p->persist_requested, (int64_t)(p->persist_idle_us + p->watchdog_us) * 4);
  __atomic_store_n(&p->host_words[0], kBellStop, __ATOMIC_RELEASE);
  p->persist_open = false;
  hipError_t e = hipStreamSynchronize((hipStream_t)p->last_stream);
  if (e != hipSuccess) return plan_fail(p, WPK_E_HIP, hip_msg("hipStreamSynchronize", e));
  return wpk_sync(p);
}

int32_t wpk_persist_times(wpk_plan* p, int64_t* dst, int32_t n_steps) {
  if (!p || !dst) return plan_fail(p, WPK_E_ARG, "null argument");
  if (p->host || !p->d_step_times) return plan_fail(p, WPK_E_ARG, "device plans only");
  if (p->persist_open) return plan_fail(p, WPK_E_STATE, "end the persistent session first");
  if (n_steps < 0 || n_steps > kPersistTimes) return plan_fail(p, WPK_E_ARG, "at most 4096 steps are kept");
  hipError_t e = hipMemcpy(dst, p->d_step_times, (size_t)n_steps * 16, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return plan_fail(p, WPK_E_HIP, hip_msg("step times read", e));
  return WPK_OK;
}

int32_t wpk_debug_drop_edge(wpk_plan* p, int32_t tile) {
  if (!p || !p->host) return plan_fail(p, WPK_E_ARG, "edges can only be dropped on host plans");
  if (tile == -1) {
    for (size_t i = 0; i < p->dag.tiles.size(); ++i) p->dag.tiles[i].wait = p->built_wait[i];
    return WPK_OK;
  }
  if (tile < 0 || tile >= (int32_t)p->dag.tiles.size()) return plan_fail(p, WPK_E_ARG, "tile out of range");
  p->dag.tiles[tile].wait = -1;
  return WPK_OK;
}

}  // extern "C"
