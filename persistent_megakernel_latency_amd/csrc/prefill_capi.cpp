// prefill_capi.cpp -- the prompt-prefill entry points of include/wpk.h.
//
// wpk_build_prefill compiles the prefill of a fixed prompt length for a batch
// (the operating point is declared up front, as for the decode step) into a
// tile DAG and sizes one device workspace; wpk_prefill is then one launch (one
// megakernel, two co-resident megakernels, or the per-operator hipGraph
// baseline, as built).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <memory>
#include <string>
#include <vector>

#include "prefill_builder.h"
#include "prefill_plan.h"
#include "wpk.h"

extern "C" int wpk_dev_prefill_kernels(const void** mk, const void** mk_log, const void** phase);
extern "C" int wpk_dev_prefill_pack(const void* src, void* dst, int rows, int K, int to_f16, int* flag, void* stream);

using namespace wpk;

struct wpk_prefill_plan {
  bool host = false;
  int32_t mode = WPK_PREFILL_MEGAKERNEL;
  PShape s{};
  PDag dag;
  std::string err;
  int32_t latched = 0, log_on = 0;
  uint64_t watchdog_us = 2000000;
  int device = -1, n_cu = 0, workers = 0, max_workers = 0, split_workers = 0;
  char* d_ws = nullptr;
  int64_t ws_bytes = 0;
  // the layer matrices repacked at build into the fragment-major layout the
  // matrix-core tiles load (the caller's row-major weights are not read later)
  uint16_t* d_wpk = nullptr;
  int64_t wpk_bytes = 0;
  PParams P{};
  const void* k_mega = nullptr;
  const void* k_mega_log = nullptr;
  const void* k_phase = nullptr;
  void* last_stream = nullptr;
  // per-operator baseline graph and the I/O pointers it was captured with
  void* graph = nullptr;
  void* graph_exec = nullptr;
  void* cap_stream = nullptr;
  const void* cap_io[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
};

namespace {

thread_local std::string g_perr;

wpk_prefill_plan* pfail(const std::string& m) {
  g_perr = m;
  return nullptr;
}

int32_t plan_err(wpk_prefill_plan* p, int32_t code, const std::string& m) {
  if (p) p->err = m;
  else g_perr = m;
  return code;
}

std::string hip_msg(const char* what, hipError_t e) { return std::string(what) + ": " + hipGetErrorString(e); }

int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

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

struct PLayout {
  int64_t ctl, heads, counters, argmax, tiles, qtiles, groups, queue_off, layers, rope_cos, rope_sin, x0, xf, act,
      act_layer, log, wqueue, pack_flag, total;
  // per-layer buffer offsets within act_layer bytes
  int64_t x_mid, x_out, xn1, xn2, q, ao, h;
};

PLayout playout(const PShape& s, const PDag& d, int32_t max_workers) {
  PLayout L{};
  int64_t at = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = at;
    at = align256(at + bytes);
    return o;
  };
  const int64_t R = s.R, nq = (int64_t)d.queue_off.size() - 1;
  L.ctl = take(CTL_WORDS * 4);
  L.heads = take(nq * kLine * 4);
  L.counters = take((int64_t)d.n_shard_slots * kLine * 4);
  L.argmax = take((int64_t)s.B * kArgmaxShards * 8);
  L.tiles = take((int64_t)d.tiles.size() * sizeof(Tile));
  L.qtiles = take((int64_t)d.queue.size() * sizeof(Tile));
  L.groups = take((int64_t)d.groups.size() * sizeof(Group));
  L.queue_off = take((int64_t)d.queue_off.size() * 4);
  L.layers = take((int64_t)s.L * sizeof(PLayer));
  L.rope_cos = take((int64_t)s.cap * (s.D / 2) * 4);
  L.rope_sin = take((int64_t)s.cap * (s.D / 2) * 4);
  L.x0 = take(R * s.H * 4);
  L.xf = take((int64_t)kMaxBatch * s.H * 4);  // hi and lo planes
  L.log = take((int64_t)d.tiles.size() * sizeof(wpk_log_rec));
  L.wqueue = take((int64_t)max_workers * 4);
  L.pack_flag = take(4);  // set by the weight repacking if a weight is outside the fp16 range
  // per-layer activations, each buffer 256-byte aligned
  int64_t la = 0;
  auto lt = [&](int64_t bytes) {
    const int64_t o = la;
    la = align256(la + bytes);
    return o;
  };
  L.x_mid = lt(R * s.H * 4);
  L.x_out = lt(R * s.H * 4);
  L.xn1 = lt(R * s.H * 4);  // the QKV operand: bf16 hi and lo planes
  L.xn2 = lt(R * s.H * 2);  // the o-proj, gate/up and down operands: one fp16 plane
  L.q = lt(R * s.Hq * s.D * 4);
  L.ao = lt(R * s.Hq * s.D * 2);
  L.h = lt(R * s.F * 2);
  L.act_layer = la;
  L.act = take(la * s.L);
  L.total = at;
  return L;
}

wpk_prefill_plan* build(const wpk_model_desc* desc, int32_t batch, int32_t ctx_len, int32_t prompt_len,
                        const wpk_prefill_opts* opts, bool host) {
  std::string why;
  if (!desc_ok(desc, &why)) return pfail(why);
  wpk_prefill_opts o{};
  if (opts) o = *opts;
  if (o.mode < WPK_PREFILL_MEGAKERNEL || o.mode > WPK_PREFILL_GRAPH) return pfail("unknown prefill mode");
  if (o.split_workers < 0) return pfail("split_workers must be >= 0");
  if (o.split_workers && o.mode != WPK_PREFILL_SPLIT) return pfail("split_workers applies to the split mode only");
  const int wpc = o.workers_per_cu ? o.workers_per_cu : 1;
  if (wpc != 1) return pfail("workers_per_cu must be 1: a prefill worker is eight waves and fills a compute unit");
  PShape s;
  why = check_prefill_shape(*desc, batch, ctx_len, prompt_len, o.mode == WPK_PREFILL_SPLIT, &s);
  if (!why.empty()) return pfail(why);
  std::unique_ptr<wpk_prefill_plan> p(new wpk_prefill_plan());
  p->host = host;
  p->mode = o.mode;
  p->s = s;
  p->dag = build_prefill_dag(s);
  why = validate_prefill_dag(s, p->dag);
  if (!why.empty()) return pfail("invalid prefill DAG: " + why);
  if (host) return p.release();

  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) return pfail("no HIP device");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return pfail(hip_msg("hipGetDevice", e));
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return pfail(hip_msg("hipGetDeviceProperties", e));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return pfail(std::string("built for gfx950, found ") + prop.gcnArchName);
  (void)wpk_dev_prefill_kernels(&p->k_mega, &p->k_mega_log, &p->k_phase);
  p->device = dev;
  p->n_cu = prop.multiProcessorCount;
  int per_cu = 0, per_cu_log = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, p->k_mega, kPThreads, 0);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_log, p->k_mega_log, kPThreads, 0);
  if (e != hipSuccess) return pfail(hip_msg("occupancy query", e));
  per_cu = std::min(per_cu, per_cu_log);
  p->max_workers = per_cu * p->n_cu;
  p->workers = std::min(wpc, per_cu) * p->n_cu;
  if (p->workers < 2 * s.queue_shards) return pfail("occupancy too low: " + std::to_string(p->max_workers) + " workers");
  if (o.mode == WPK_PREFILL_SPLIT) {
    const int w1 = o.split_workers ? o.split_workers : std::max(s.queue_shards, p->workers / 8);
    if (w1 < s.queue_shards || p->workers - w1 < s.queue_shards)
      return pfail("split_workers must leave each megakernel at least one worker per claim queue (" +
                   std::to_string(s.queue_shards) + ") of the " + std::to_string(p->workers) + " workers");
    p->split_workers = w1;
  }

  const PLayout L = playout(s, p->dag, p->max_workers);
  e = hipMalloc((void**)&p->d_ws, L.total);
  if (e != hipSuccess) return pfail(hip_msg("hipMalloc prefill workspace", e));
  p->ws_bytes = L.total;
  char* w = p->d_ws;
  auto up = [&](int64_t off, const void* src, size_t bytes) {
    return hipMemcpy(w + off, src, bytes, hipMemcpyHostToDevice);
  };
  // zero: counters, heads, control, argmax shards, the padding rows of the
  // queries and attention outputs (never written) and the rows of xf past
  // the batch
  e = hipMemset(w, 0, L.total);
  // packed copies of the layer matrices: qkv, o, gate, up, down per layer
  const int64_t per_layer_w = (int64_t)s.qkv_rows * s.H + (int64_t)s.H * s.H + 3 * (int64_t)s.F * s.H;
  p->wpk_bytes = per_layer_w * s.L * 2;
  if (e == hipSuccess) e = hipMalloc((void**)&p->d_wpk, p->wpk_bytes);
  if (e != hipSuccess) {
    (void)hipFree(p->d_ws);
    p->d_ws = nullptr;
    p->d_wpk = nullptr;
    return pfail(hip_msg("hipMalloc packed weights", e));
  }
  std::vector<PLayer> lay(s.L);
  for (int l = 0; l < s.L; ++l) {
    char* a = w + L.act + (int64_t)l * L.act_layer;
    PLayer& y = lay[l];
    uint16_t* wl = p->d_wpk + per_layer_w * l;
    const struct {
      const void* src;
      int rows, K;
    } mats[5] = {{desc->w_qkv[l], s.qkv_rows, s.H}, {desc->w_o[l], s.H, s.H}, {desc->w_gate[l], s.F, s.H},
                 {desc->w_up[l], s.F, s.H}, {desc->w_down[l], s.H, s.F}};
    uint16_t* dst[5];
    for (int m = 0; m < 5; ++m) {
      dst[m] = wl;
      // QKV stays bf16 (its operand is the hi + lo bf16 pair); o, gate, up and
      // down become fp16, the format of their single-plane operands
      if (wpk_dev_prefill_pack(mats[m].src, wl, mats[m].rows, mats[m].K, m > 0 ? 1 : 0, (int*)(w + L.pack_flag),
                               nullptr) != 0)
        e = hipErrorLaunchFailure;
      wl += (int64_t)mats[m].rows * mats[m].K;
    }
    y.w_qkv = dst[0];
    y.w_o = dst[1];
    y.w_gate = dst[2];
    y.w_up = dst[3];
    y.w_down = dst[4];
    y.attn_norm = desc->attn_norm[l];
    y.mlp_norm = desc->mlp_norm[l];
    y.x_mid = (float*)(a + L.x_mid);
    y.x_out = (float*)(a + L.x_out);
    y.xn1 = (uint16_t*)(a + L.xn1);
    y.xn2 = (uint16_t*)(a + L.xn2);
    y.q = (float*)(a + L.q);
    y.ao = (uint16_t*)(a + L.ao);
    y.h = (uint16_t*)(a + L.h);
    y.x_in = l == 0 ? (const float*)(w + L.x0) : lay[l - 1].x_out;
  }
  std::vector<float> rc((size_t)s.cap * (s.D / 2)), rsn(rc.size());
  for (int pos = 0; pos < s.cap; ++pos)
    for (int i = 0; i < s.D / 2; ++i) {
      // cos / sin of pos * theta^(-2i/D) in float64, stored float32 (the decode step's table)
      const double ang = (double)pos * std::pow((double)s.theta, -2.0 * i / s.D);
      rc[(size_t)pos * (s.D / 2) + i] = (float)std::cos(ang);
      rsn[(size_t)pos * (s.D / 2) + i] = (float)std::sin(ang);
    }
  std::vector<Tile> qt;
  for (int32_t id : p->dag.queue) qt.push_back(p->dag.tiles[id]);
  const int32_t nq = (int32_t)p->dag.queue_off.size() - 1, q0 = p->dag.split_queues;
  const int32_t w0 = p->workers - p->split_workers;
  std::vector<int32_t> wq(p->max_workers);
  for (int32_t k = 0; k < p->max_workers; ++k)
    wq[k] = !p->split_workers ? k % nq : k < w0 ? k % q0 : q0 + (k - w0) % (nq - q0);
  if (e == hipSuccess) e = up(L.tiles, p->dag.tiles.data(), p->dag.tiles.size() * sizeof(Tile));
  if (e == hipSuccess) e = up(L.qtiles, qt.data(), qt.size() * sizeof(Tile));
  if (e == hipSuccess) e = up(L.groups, p->dag.groups.data(), p->dag.groups.size() * sizeof(Group));
  if (e == hipSuccess) e = up(L.queue_off, p->dag.queue_off.data(), p->dag.queue_off.size() * 4);
  if (e == hipSuccess) e = up(L.layers, lay.data(), lay.size() * sizeof(PLayer));
  if (e == hipSuccess) e = up(L.rope_cos, rc.data(), rc.size() * 4);
  if (e == hipSuccess) e = up(L.rope_sin, rsn.data(), rsn.size() * 4);
  if (e == hipSuccess) e = up(L.wqueue, wq.data(), wq.size() * 4);
  if (e == hipSuccess) e = hipDeviceSynchronize();  // the weight repacking
  int32_t out_of_range = 0;
  if (e == hipSuccess) e = hipMemcpy(&out_of_range, w + L.pack_flag, 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess || out_of_range) {
    (void)hipFree(p->d_ws);
    (void)hipFree(p->d_wpk);
    p->d_ws = nullptr;
    p->d_wpk = nullptr;
    if (e == hipSuccess)
      return pfail("an o-proj, gate, up or down weight is outside the fp16 range (|w| >= 65520): the prefill "
                   "multiplies those matrices in fp16");
    return pfail(hip_msg("prefill workspace upload / weight repacking", e));
  }
  PParams& P = p->P;
  P.L = s.L; P.H = s.H; P.Hq = s.Hq; P.Hkv = s.Hkv; P.D = s.D; P.F = s.F; P.V = s.V;
  P.B = s.B; P.cap = s.cap; P.G = s.G; P.qkv_rows = s.qkv_rows;
  P.P = s.P; P.Pp = s.Pp; P.nrb_s = s.nrb_s; P.R = s.R;
  P.n_tiles = (int32_t)p->dag.tiles.size();
  P.n_queues = nq;
  P.n_workers = p->workers;
  P.eps = s.eps;
  P.attn_scale = 1.0f / std::sqrt((float)s.D);
  P.embed = (const uint16_t*)desc->embed;
  P.final_norm = desc->final_norm;
  P.layers = (const PLayer*)(w + L.layers);
  P.x0 = (float*)(w + L.x0);
  P.xf = (uint16_t*)(w + L.xf);
  P.rope_cos = (const float*)(w + L.rope_cos);
  P.rope_sin = (const float*)(w + L.rope_sin);
  P.tiles = (const Tile*)(w + L.tiles);
  P.qtiles = (const Tile*)(w + L.qtiles);
  P.queue_off = (const int32_t*)(w + L.queue_off);
  P.groups = (const Group*)(w + L.groups);
  P.counters = (uint32_t*)(w + L.counters);
  P.heads = (uint32_t*)(w + L.heads);
  P.ctl = (uint32_t*)(w + L.ctl);
  P.argmax = (unsigned long long*)(w + L.argmax);
  P.log = (int32_t*)(w + L.log);
  P.watchdog_ticks = p->watchdog_us * 100;
  P.worker_queue = (const int32_t*)(w + L.wqueue);
  if (o.mode == WPK_PREFILL_GRAPH) {
    hipStream_t cs;
    e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
    if (e != hipSuccess) {
      (void)hipFree(p->d_ws);
      (void)hipFree(p->d_wpk);
      p->d_ws = nullptr;
      p->d_wpk = nullptr;
      return pfail(hip_msg("hipStreamCreate", e));
    }
    p->cap_stream = cs;
  }
  return p.release();
}

int32_t capture(wpk_prefill_plan* p) {
  if (p->graph_exec) (void)hipGraphExecDestroy((hipGraphExec_t)p->graph_exec);
  if (p->graph) (void)hipGraphDestroy((hipGraph_t)p->graph);
  p->graph_exec = p->graph = nullptr;
  hipStream_t cs = (hipStream_t)p->cap_stream;
  hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return plan_err(p, WPK_E_HIP, hip_msg("hipStreamBeginCapture", e));
  for (const auto& ph : p->dag.phases) {
    int32_t first = ph.first;
    void* args[] = {(void*)&p->P, (void*)&first};
    e = hipLaunchKernel(p->k_phase, dim3(ph.second), dim3(kPThreads), args, 0, cs);
    if (e != hipSuccess) break;
  }
  hipGraph_t g = nullptr;
  const hipError_t e2 = hipStreamEndCapture(cs, &g);
  if (e != hipSuccess) return plan_err(p, WPK_E_HIP, hip_msg("prefill phase launch during capture", e));
  if (e2 != hipSuccess) return plan_err(p, WPK_E_HIP, hip_msg("hipStreamEndCapture", e2));
  hipGraphExec_t ge = nullptr;
  e = hipGraphInstantiate(&ge, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    return plan_err(p, WPK_E_HIP, hip_msg("hipGraphInstantiate", e));
  }
  p->graph = g;
  p->graph_exec = ge;
  return WPK_OK;
}

}  // namespace

extern "C" {

wpk_prefill_plan* wpk_build_prefill(const wpk_model_desc* desc, int32_t batch, int32_t ctx_len, int32_t prompt_len,
                                    const wpk_prefill_opts* opts) {
  return build(desc, batch, ctx_len, prompt_len, opts, false);
}

wpk_prefill_plan* wpk_build_prefill_host(const wpk_model_desc* desc, int32_t batch, int32_t ctx_len,
                                         int32_t prompt_len, const wpk_prefill_opts* opts) {
  return build(desc, batch, ctx_len, prompt_len, opts, true);
}

int32_t wpk_prefill(wpk_prefill_plan* p, const int32_t* prompt, wpk_kv* kv, void* logits, int32_t* tokens_out,
                    wpk_stream_t stream) {
  if (!p) return plan_err(nullptr, WPK_E_ARG, "null plan");
  if (p->host) return plan_err(p, WPK_E_ARG, "host plan: the DAG only");
  if (p->latched) return plan_err(p, WPK_E_STATE, "plan holds device error " + std::to_string(p->latched));
  if (!prompt || !kv || !kv->k || !kv->v || !kv->seq_len || !logits || !tokens_out)
    return plan_err(p, WPK_E_ARG, "null prompt, kv, logits or tokens_out");
  PParams& P = p->P;
  P.prompt = prompt;
  P.kc = (uint16_t*)kv->k;
  P.vc = (uint16_t*)kv->v;
  P.seq_len = kv->seq_len;
  P.logits = (float*)logits;
  P.tokens_out = tokens_out;
  hipStream_t st = (hipStream_t)stream;
  p->last_stream = stream;
  hipError_t e;
  if (p->mode == WPK_PREFILL_GRAPH) {
    const void* io[6] = {prompt, kv->k, kv->v, kv->seq_len, logits, tokens_out};
    if (!p->graph_exec || std::memcmp(io, p->cap_io, sizeof io) != 0) {
      const int32_t rc = capture(p);
      if (rc != WPK_OK) return rc;
      std::memcpy(p->cap_io, io, sizeof io);
    }
    e = hipGraphLaunch((hipGraphExec_t)p->graph_exec, st);
    if (e != hipSuccess) return plan_err(p, WPK_E_HIP, hip_msg("hipGraphLaunch", e));
    return WPK_OK;
  }
  if (p->log_on) {
    e = hipMemsetAsync(P.log, 0, p->dag.tiles.size() * sizeof(wpk_log_rec), st);
    if (e != hipSuccess) return plan_err(p, WPK_E_HIP, hip_msg("hipMemsetAsync log", e));
  }
  void* args[] = {(void*)&P};
  e = hipLaunchKernel(p->log_on ? p->k_mega_log : p->k_mega, dim3(p->workers), dim3(kPThreads), args, 0, st);
  if (e != hipSuccess) return plan_err(p, WPK_E_HIP, hip_msg("prefill megakernel launch", e));
  return WPK_OK;
}

int32_t wpk_prefill_sync(wpk_prefill_plan* p) {
  if (!p) return plan_err(nullptr, WPK_E_ARG, "null plan");
  if (p->host) return WPK_OK;
  hipError_t e = hipStreamSynchronize((hipStream_t)p->last_stream);
  if (e != hipSuccess) return plan_err(p, WPK_E_HIP, hip_msg("hipStreamSynchronize", e));
  uint32_t st[4];
  e = hipMemcpy(st, p->P.ctl + CTL_STATUS, sizeof st, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return plan_err(p, WPK_E_HIP, hip_msg("status read", e));
  if (st[0] != 0) {
    p->latched = (int32_t)st[0];
    char m[256];
    snprintf(m, sizeof m, "device error %d at tile %u (worker %u, launch %u)", (int32_t)st[0], st[1], st[2], st[3]);
    p->err = m;
    return p->latched;
  }
  return WPK_OK;
}

void wpk_prefill_destroy(wpk_prefill_plan* p) {
  if (!p) return;
  if (p->graph_exec) (void)hipGraphExecDestroy((hipGraphExec_t)p->graph_exec);
  if (p->graph) (void)hipGraphDestroy((hipGraph_t)p->graph);
  if (p->cap_stream) (void)hipStreamDestroy((hipStream_t)p->cap_stream);
  if (p->d_ws || p->d_wpk) {
    (void)hipDeviceSynchronize();
    if (p->d_ws) (void)hipFree(p->d_ws);
    if (p->d_wpk) (void)hipFree(p->d_wpk);
  }
  delete p;
}

const char* wpk_prefill_last_error(const wpk_prefill_plan* p) { return p ? p->err.c_str() : g_perr.c_str(); }

int32_t wpk_prefill_set_option(wpk_prefill_plan* p, int32_t key, int64_t value) {
  if (!p) return plan_err(nullptr, WPK_E_ARG, "null plan");
  switch (key) {
    case WPK_OPT_LOG:
      if (p->mode == WPK_PREFILL_GRAPH && value) return plan_err(p, WPK_E_ARG, "the graph baseline keeps no log");
      p->log_on = value != 0;
      return WPK_OK;
    case WPK_OPT_WATCHDOG_US:
      if (value <= 0) return plan_err(p, WPK_E_ARG, "watchdog must be positive");
      p->watchdog_us = (uint64_t)value;
      p->P.watchdog_ticks = (uint64_t)value * 100;
      return WPK_OK;
    case WPK_OPT_RESET: {
      if (p->host) {
        p->latched = 0;
        return WPK_OK;
      }
      PParams& P = p->P;
      hipError_t e = hipDeviceSynchronize();
      if (e == hipSuccess) e = hipMemset(P.ctl, 0, CTL_WORDS * 4);
      if (e == hipSuccess) e = hipMemset(P.heads, 0, (size_t)P.n_queues * kLine * 4);
      if (e == hipSuccess) e = hipMemset(P.counters, 0, (size_t)p->dag.n_shard_slots * kLine * 4);
      if (e == hipSuccess) e = hipMemset(P.argmax, 0, (size_t)p->s.B * kArgmaxShards * 8);
      if (e == hipSuccess) e = hipDeviceSynchronize();
      if (e != hipSuccess) return plan_err(p, WPK_E_HIP, hip_msg("reset", e));
      p->latched = 0;
      return WPK_OK;
    }
  }
  return plan_err(p, WPK_E_ARG, "unknown or unsupported option key for a prefill plan");
}

int32_t wpk_prefill_get_log(wpk_prefill_plan* p, void* dst, size_t bytes) {
  if (!p || !dst) return plan_err(p, WPK_E_ARG, "null argument");
  if (p->host) return plan_err(p, WPK_E_ARG, "host plans keep no log");
  const size_t need = p->dag.tiles.size() * sizeof(wpk_log_rec);
  if (bytes < need) return plan_err(p, WPK_E_ARG, "log buffer too small");
  const hipError_t e = hipMemcpy(dst, p->P.log, need, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return plan_err(p, WPK_E_HIP, hip_msg("log read", e));
  return WPK_OK;
}

int32_t wpk_prefill_get_info(const wpk_prefill_plan* p, wpk_prefill_info* out) {
  if (!p || !out) return WPK_E_ARG;
  out->n_tiles = (int32_t)p->dag.tiles.size();
  out->n_groups = (int32_t)p->dag.groups.size();
  out->n_queues = (int32_t)p->dag.queue_off.size() - 1;
  out->workers = p->workers;
  out->max_workers = p->max_workers;
  out->split_workers = p->split_workers;
  out->n_phases = (int32_t)p->dag.phases.size();
  out->rows_per_sequence = p->s.Pp;
  out->workspace_bytes = p->ws_bytes + p->wpk_bytes;
  out->flops = prefill_flops(p->s);
  return WPK_OK;
}

int32_t wpk_prefill_get_dag(const wpk_prefill_plan* p, int32_t* type, int32_t* layer, int32_t* wait, int32_t* signal,
                            int32_t* queue) {
  if (!p || !type || !layer || !wait || !signal) return WPK_E_ARG;
  for (size_t i = 0; i < p->dag.tiles.size(); ++i) {
    type[i] = p->dag.tiles[i].type;
    layer[i] = p->dag.tiles[i].layer;
    wait[i] = p->dag.tiles[i].wait;
    signal[i] = p->dag.tiles[i].signal;
  }
  if (queue) {
    const int32_t nq = (int32_t)p->dag.queue_off.size() - 1;
    for (int32_t q = 0; q < nq; ++q)
      for (int32_t k = p->dag.queue_off[q]; k < p->dag.queue_off[q + 1]; ++k) queue[p->dag.queue[k]] = q;
  }
  return WPK_OK;
}

int32_t wpk_prefill_simulate(const wpk_prefill_plan* p, const wpk_prefill_sim_params* sp, wpk_sim_result* out) {
  if (!p || !sp || !out) return WPK_E_ARG;
  if (sp->workers < p->s.queue_shards * (p->s.split ? 2 : 1)) return WPK_E_ARG;
  if ((sp->split_workers > 0) != (p->s.split != 0) || sp->split_workers < 0) return WPK_E_ARG;
  if (p->s.split && (sp->split_workers < p->s.queue_shards || sp->workers - sp->split_workers < p->s.queue_shards))
    return WPK_E_ARG;
  if (sp->conventional != 0 && sp->conventional != 1) return WPK_E_ARG;
  if (sp->conventional && p->s.split) return WPK_E_ARG;
  PSimCost c{};
  for (int k = 0; k < P_NTYPES; ++k) {
    if (!(sp->tile_us[k] >= 0)) return WPK_E_ARG;
    c.tile_us[k] = sp->tile_us[k];
  }
  if (!(sp->attn_step_us >= 0) || !(sp->hop_us >= 0) || !(sp->launch_gap_us >= 0)) return WPK_E_ARG;
  c.attn_step_us = sp->attn_step_us;
  c.hop_us = sp->hop_us;
  c.launch_gap_us = sp->launch_gap_us;
  double busy = 0;
  out->step_us = simulate_prefill(p->s, p->dag, c, sp->workers, sp->split_workers, sp->conventional != 0, &busy);
  out->hbm_bytes = 0;
  out->achieved_GBps = 0;
  out->worker_busy_frac = busy;
  return WPK_OK;
}

int32_t wpk_prefill_get_key_steps(const wpk_prefill_plan* p, int32_t* key_steps) {
  if (!p || !key_steps) return WPK_E_ARG;
  for (size_t i = 0; i < p->dag.tiles.size(); ++i) key_steps[i] = prefill_key_steps(p->s, p->dag.tiles[i]);
  return WPK_OK;
}

}  // extern "C"
