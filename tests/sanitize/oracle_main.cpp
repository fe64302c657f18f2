// Host driver that runs the oracle's entry points on small dense and
// routed-expert decoders, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_sanitizers.py.  The oracle has no
// header (its Python binding declares the ABI); the declarations below mirror
// it.  Weights come from a local linear congruential generator: the run
// checks memory safety and finiteness, not values.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

extern "C" {
typedef struct {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate;
  int32_t n_experts, top_k, expert_intermediate, vocab, tied_embeddings;
  double rms_eps, rope_theta;
} orc_shape;
typedef struct orc_model orc_model;
const char* orc_last_error(void);
void orc_rmsnorm(const double* x, const double* g, int64_t n, double eps, double* y);
void orc_rope(double* v, int64_t D, int64_t pos, double theta);
void orc_attention(const double* q, const uint16_t* K, const uint16_t* V, int64_t T, int64_t D, int64_t stride,
                   double* o, double* wts);
void orc_route(const double* logits, int32_t E, int32_t k, int32_t* experts, double* weights);
double orc_route_gap(const double* logits, int32_t E, int32_t k, const int32_t* experts);
orc_model* orc_create(const orc_shape* s, int32_t batch, int32_t cap, int32_t nthreads);
void orc_destroy(orc_model* m);
int32_t orc_set_weight(orc_model* m, const char* name, const uint16_t* data, int64_t rows, int64_t cols);
uint16_t* orc_kv(orc_model* m, int32_t which);
int64_t orc_kv_elems(const orc_model* m);
int32_t orc_decode(orc_model* m, const int32_t* tokens, const int32_t* positions, double* logits, double* resid);
int32_t orc_full_forward(orc_model* m, const int32_t* tokens, int32_t n, double* logits_last);
double orc_last_routing_gap(const orc_model* m, int32_t b);
int32_t orc_last_router_logits(const orc_model* m, int32_t layer, int32_t b, double* out);
int32_t orc_force_routing(orc_model* m, const int32_t* experts);
int32_t orc_last_routing(const orc_model* m, int32_t layer, int32_t b, int32_t* experts, double* weights);
}

static uint32_t lcg = 12345u;
static uint16_t rnd_bf16(float scale) {
  lcg = lcg * 1664525u + 1013904223u;
  const float u = ((float)(lcg >> 8) / 16777216.0f - 0.5f) * 2.0f * scale;
  uint32_t b;
  std::memcpy(&b, &u, 4);
  return (uint16_t)(b >> 16);
}
static std::vector<uint16_t> mat(int64_t r, int64_t c, float scale) {
  std::vector<uint16_t> v((size_t)(r * c));
  for (auto& x : v) x = rnd_bf16(scale);
  return v;
}
static std::vector<uint16_t> ones(int64_t n) { return std::vector<uint16_t>((size_t)n, (uint16_t)0x3F80); }

static int fail(const char* what) {
  std::printf("FAIL %s: %s\n", what, orc_last_error());
  return 1;
}

static int run(const orc_shape& s, int B, int cap, int steps) {
  orc_model* m = orc_create(&s, B, cap, 3);
  if (!m) return fail("create");
  std::vector<std::vector<uint16_t>> keep;
  auto set = [&](const std::string& n, std::vector<uint16_t> v, int64_t r, int64_t c) {
    keep.push_back(std::move(v));
    return orc_set_weight(m, n.c_str(), keep.back().data(), r, c);
  };
  const int H = s.hidden, D = s.head_dim, Hq = s.n_q_heads, Hkv = s.n_kv_heads, V = s.vocab;
  int rc = set("embed", mat(V, H, 0.5f), V, H) | set("final_norm", ones(H), H, 1);
  if (!s.tied_embeddings) rc |= set("lm_head", mat(V, H, 0.05f), V, H);
  for (int l = 0; l < s.n_layers; ++l) {
    const std::string p = "layers." + std::to_string(l) + ".";
    rc |= set(p + "in_norm", ones(H), H, 1) | set(p + "post_norm", ones(H), H, 1);
    rc |= set(p + "q_norm", ones(D), D, 1) | set(p + "k_norm", ones(D), D, 1);
    rc |= set(p + "wq", mat(Hq * D, H, 0.05f), Hq * D, H) | set(p + "wk", mat(Hkv * D, H, 0.05f), Hkv * D, H);
    rc |= set(p + "wv", mat(Hkv * D, H, 0.05f), Hkv * D, H) | set(p + "wo", mat(H, Hq * D, 0.05f), H, Hq * D);
    if (s.n_experts == 0) {
      const int I = s.intermediate;
      rc |= set(p + "w_gate", mat(I, H, 0.05f), I, H) | set(p + "w_up", mat(I, H, 0.05f), I, H);
      rc |= set(p + "w_down", mat(H, I, 0.05f), H, I);
    } else {
      const int I = s.expert_intermediate;
      rc |= set(p + "router", mat(s.n_experts, H, 0.05f), s.n_experts, H);
      for (int e = 0; e < s.n_experts; ++e) {
        const std::string q = p + "experts." + std::to_string(e) + ".";
        rc |= set(q + "w_gate", mat(I, H, 0.05f), I, H) | set(q + "w_up", mat(I, H, 0.05f), I, H);
        rc |= set(q + "w_down", mat(H, I, 0.05f), H, I);
      }
    }
  }
  if (rc) return fail("set_weight");
  // a prefilled cache: random rows below each sequence's start position
  uint16_t* K = orc_kv(m, 0);
  uint16_t* Vc = orc_kv(m, 1);
  for (int64_t i = 0; i < orc_kv_elems(m); ++i) {
    K[i] = rnd_bf16(1.0f);
    Vc[i] = rnd_bf16(1.0f);
  }
  std::vector<int32_t> tok(B), pos(B);
  std::vector<double> logits((size_t)B * V), resid((size_t)B * H);
  for (int st = 0; st < steps; ++st) {
    for (int b = 0; b < B; ++b) {
      tok[b] = (7 * b + 3 * st) % V;
      pos[b] = (b * 5 + st) % cap;  // includes position 0 (a cache holding only the new row)
    }
    if (orc_decode(m, tok.data(), pos.data(), logits.data(), resid.data())) return fail("decode");
    for (double v : logits)
      if (!std::isfinite(v)) return fail("non-finite logits");
    if (s.n_experts) {
      std::vector<int32_t> ex((size_t)s.n_layers * B * s.top_k), e1(s.top_k);
      std::vector<double> w1(s.top_k), rl(s.n_experts);
      for (int l = 0; l < s.n_layers; ++l)
        for (int b = 0; b < B; ++b) {
          if (orc_last_routing(m, l, b, e1.data(), w1.data())) return fail("last_routing");
          if (orc_last_router_logits(m, l, b, rl.data())) return fail("router_logits");
          for (int j = 0; j < s.top_k; ++j) ex[((size_t)l * B + b) * s.top_k + j] = (e1[j] + 1) % s.n_experts;
        }
      for (int b = 0; b < B; ++b)
        if (!(orc_last_routing_gap(m, b) >= 0.0)) return fail("routing gap");
      if (orc_force_routing(m, ex.data())) return fail("force_routing");
      if (orc_decode(m, tok.data(), pos.data(), logits.data(), nullptr)) return fail("forced decode");
      if (orc_force_routing(m, nullptr)) return fail("unforce");
    }
  }
  std::vector<int32_t> prompt(9);
  for (int i = 0; i < 9; ++i) prompt[i] = (11 * i) % V;
  if (orc_full_forward(m, prompt.data(), 9, logits.data())) return fail("full_forward");
  orc_destroy(m);
  return 0;
}

int main() {
  // primitives at their edges: one position, an all-equal routing row
  std::vector<double> x(64, 0.5), g(64, 1.0), y(64), q(64, 0.1), o(64), w(1);
  orc_rmsnorm(x.data(), g.data(), 64, 1e-6, y.data());
  orc_rmsnorm(x.data(), nullptr, 64, 1e-6, y.data());
  orc_rope(y.data(), 64, 0, 1e6);
  orc_rope(y.data(), 64, 4095, 1e6);
  std::vector<uint16_t> kv = mat(3, 64, 1.0f);
  orc_attention(q.data(), kv.data(), kv.data(), 1, 64, 64, o.data(), w.data());
  std::vector<double> lg(8, 1.0), rw(2);
  std::vector<int32_t> re(2);
  orc_route(lg.data(), 8, 2, re.data(), rw.data());
  if (orc_route_gap(lg.data(), 8, 2, re.data()) != 0.0) return fail("tie gap");
  // decoders: dense (untied and tied) and routed experts, ragged positions
  orc_shape dense{2, 128, 4, 2, 64, 256, 0, 0, 0, 512, 0, 1e-6, 1e6};
  orc_shape tied = dense;
  tied.tied_embeddings = 1;
  orc_shape moe{2, 128, 4, 2, 64, 0, 8, 2, 64, 512, 0, 1e-6, 1e6};
  if (run(dense, 3, 24, 3) || run(tied, 1, 16, 2) || run(moe, 2, 16, 2)) return 1;
  std::printf("oracle ok\n");
  return 0;
}
