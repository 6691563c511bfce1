// Driver for a ThreadSanitizer build of the protocol emulator (host_exec.cpp
// compiled with WPK_TSAN_ORDERINGS and -fsanitize=thread; no GPU, no HIP).
//
// It builds two small models in host memory -- a float32 decoder run as a
// batch-2 GEMV plan and a bf16 decoder run as a batch-8 matrix-core plan (K
// slices, row-block reductions) -- and runs the device claim/poll/publish
// protocol with 16 worker threads, several seeds, comparing every result bit
// for bit with the serial executor.  The wide plan also runs with the fixed
// reducer per row block.  With "drop", one output-projection tile no longer
// waits for its inputs: the sanitizer must then report a race (the positive
// control that shows the build would see one).
#include <cmath>
#include <cstdio>
#include <cstring>
#include <memory>
#include <string>
#include <vector>

#include "host_exec.h"

using namespace wpk;

namespace {

uint64_t rng_state = 0x243F6A8885A308D3ull;
double uniform() {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return ((rng_state >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}
double normal() { return std::sqrt(-2.0 * std::log(uniform())) * std::cos(6.283185307179586 * uniform()); }

uint16_t bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

struct Model {
  wpk_model_desc d{};
  std::vector<std::vector<char>> mats;
  std::vector<std::vector<float>> gains;
  std::vector<const void*> qkv, o, gate, up, down;
  std::vector<const float*> an, mn;
  int elt;

  const void* mat(size_t n) {
    mats.emplace_back(n * elt);
    for (size_t i = 0; i < n; ++i) {
      const float v = (float)(0.02 * normal());
      if (elt == 2) ((uint16_t*)mats.back().data())[i] = bf16(v);
      else ((float*)mats.back().data())[i] = v;
    }
    return mats.back().data();
  }
  const float* gain(int n) {
    gains.emplace_back(n);
    for (auto& g : gains.back()) g = (float)(1.0 + 0.1 * normal());
    return gains.back().data();
  }
  Model(int L, int H, int Hq, int Hkv, int F, int V, int dtype) {
    elt = dtype == WPK_BF16 ? 2 : 4;
    mats.reserve(64);
    gains.reserve(64);
    d.n_layers = L; d.hidden = H; d.n_q_heads = Hq; d.n_kv_heads = Hkv; d.head_dim = 64; d.ffn = F;
    d.vocab = V; d.tied_embeddings = 1; d.rope_theta = 500000.f; d.rms_eps = 1e-5f; d.dtype = dtype;
    d.embed = mat((size_t)V * H);
    d.final_norm = gain(H);
    for (int l = 0; l < L; ++l) {
      qkv.push_back(mat((size_t)(Hq + 2 * Hkv) * 64 * H));
      o.push_back(mat((size_t)H * H));
      gate.push_back(mat((size_t)F * H));
      up.push_back(mat((size_t)F * H));
      down.push_back(mat((size_t)H * F));
      an.push_back(gain(H));
      mn.push_back(gain(H));
    }
    d.attn_norm = an.data(); d.w_qkv = qkv.data(); d.w_o = o.data(); d.mlp_norm = mn.data();
    d.w_gate = gate.data(); d.w_up = up.data(); d.w_down = down.data();
  }
};

struct State {
  std::vector<char> k, v;
  std::vector<int32_t> seq, tok;
  std::vector<float> logits;
  wpk_kv kv{};
  State(const Model& m, int B, int cap, const std::vector<int32_t>& lens) {
    const size_t n = (size_t)m.d.n_layers * B * m.d.n_kv_heads * cap * 64 * m.elt;
    k.resize(n);
    v.resize(n);
    for (size_t i = 0; i < n / m.elt; ++i) {
      const float a = (float)(0.9 * normal()), b = (float)(0.9 * normal());
      if (m.elt == 2) {
        ((uint16_t*)k.data())[i] = bf16(a);
        ((uint16_t*)v.data())[i] = bf16(b);
      } else {
        ((float*)k.data())[i] = a;
        ((float*)v.data())[i] = b;
      }
    }
    seq = lens;
    for (int b = 0; b < B; ++b) tok.push_back((int32_t)((b * 131 + 7) % m.d.vocab));
    logits.assign((size_t)B * m.d.vocab, 0.f);
    kv.k = k.data();
    kv.v = v.data();
    kv.seq_len = seq.data();
  }
  bool same(const State& o) const {
    return k == o.k && v == o.v && seq == o.seq && tok == o.tok &&
           std::memcmp(logits.data(), o.logits.data(), logits.size() * 4) == 0;
  }
};

int run(const char* name, const Model& m, int B, int cap, const std::vector<int32_t>& lens, bool drop, bool fixed) {
  std::string err;
  std::unique_ptr<wpk_plan> p(make_host_plan(m.d, B, cap, wpk_build_opts{}, &err));
  if (!p) {
    std::printf("%s: build failed: %s\n", name, err.c_str());
    return 1;
  }
  State ref(m, B, cap, lens);
  rng_state = 0x243F6A8885A308D3ull;  // the same cache contents for every state
  State ref2(m, B, cap, lens);
  (void)ref2;
  int32_t rc = host_serial_step(p.get(), ref.tok.data(), &ref.kv, ref.logits.data(), 1, false);
  if (rc != 0) {
    std::printf("%s: serial step failed (%d)\n", name, rc);
    return 1;
  }
  if (drop) {
    for (auto& t : p->dag.tiles)
      if (t.type == T_OPROJ && t.layer == 1) {
        t.wait = -1;
        break;
      }
  }
  p->emu_fixed_reducer = fixed ? 1 : 0;
  int bad = 0;
  for (uint64_t seed = 1; seed <= 3; ++seed) {
    rng_state = 0x243F6A8885A308D3ull;
    State st(m, B, cap, lens);
    rng_state = 0x243F6A8885A308D3ull;
    State fresh(m, B, cap, lens);
    (void)fresh;
    rc = host_emulate_step(p.get(), st.tok.data(), &st.kv, st.logits.data(), 16, seed);
    if (rc != 0) {
      std::printf("%s: emulated step failed (%d) %s\n", name, rc, p->err.c_str());
      return 1;
    }
    if (!drop && !st.same(ref)) {
      std::printf("%s: seed %llu differs from the serial executor\n", name, (unsigned long long)seed);
      ++bad;
    }
  }
  std::printf("%s: %s\n", name, bad ? "MISMATCH" : "ok");
  return bad ? 1 : 0;
}

}  // namespace

int main(int argc, char** argv) {
  const bool drop = argc > 1 && std::strcmp(argv[1], "drop") == 0;
  int rc = 0;
  {
    rng_state = 0x9E3779B97F4A7C15ull;
    Model tiny(2, 256, 4, 2, 1024, 1024, WPK_F32);
    rng_state = 0x243F6A8885A308D3ull;
    rc |= run("float32 batch 2", tiny, 2, 100, {40, 90}, drop, false);
  }
  if (!drop) {
    rng_state = 0x9E3779B97F4A7C15ull;
    Model mini(2, 512, 8, 2, 1024, 1000, WPK_BF16);
    const std::vector<int32_t> lens = {63, 64, 1, 100, 7, 128, 90, -1};
    rng_state = 0x243F6A8885A308D3ull;
    rc |= run("bf16 batch 8 (matrix-core plan)", mini, 8, 140, lens, false, false);
    rng_state = 0x243F6A8885A308D3ull;
    rc |= run("bf16 batch 8, fixed reducer", mini, 8, 140, lens, false, true);
  }
  return rc;
}
