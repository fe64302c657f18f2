// oracle.cpp - plain CPU reference decoder.  TEST INFRASTRUCTURE ONLY.
//
// Only the tests, the smoke check and the benchmark's CPU-baseline leg may
// load this library.  It shares no code, header, table or helper with the HIP
// decoder; both sides only read the same bf16 bytes made by the synth module.
//
// What it computes: one autoregressive decode step of a Qwen3-style decoder
// (dense SwiGLU MLP or top-k routed experts), the computation the MPK pages
// fuse into one persistent kernel (page "MPK: A Compiler and Runtime for
// Mega-Kernelizing Tensor Programs", abstract; review page 2512.22219, section
// 2.1: the fused scope is attention + MatMul + RMSNorm).  The pages never
// write the model's formulas down, so each step below follows the plainest
// Qwen3 reading; each such reading is pinned by a test in tests/test_oracle_pins.py.
//
// Arithmetic: IEEE double throughout.  bf16 weights and cache entries are
// widened exactly.  The only roundings to bf16 are the ones the method itself
// stores: a new key/value entering the KV cache.
//
// Pins (tests/test_oracle_pins.py): RoPE identity at position 0 and a closed
// form angle, RMSNorm closed form, softmax rows summing to one, attention
// against brute force / equal keys / a single position, matvec against numpy,
// SwiGLU closed forms, routing against a full sort and the one-expert
// reduction, incremental decode equal to a full causal recompute, batch
// invariance, and the whole decoder against an independent torch fp64 model.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <condition_variable>
#include <cstdint>
#include <cstring>
#include <functional>
#include <map>
#include <mutex>
#include <stdexcept>
#include <string>
#include <thread>
#include <vector>

namespace {

// ---------------------------------------------------------------- bf16
double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// Storing a value in bf16: the nearest float, then round-to-nearest-even to
// the upper 16 bits.
uint16_t double_to_bf16(double v) {
  float f = (float)v;
  uint32_t x;
  std::memcpy(&x, &f, 4);
  if ((x & 0x7f800000u) == 0x7f800000u) return (uint16_t)((x >> 16) | ((x & 0xffffu) ? 0x40u : 0u));
  x += 0x7fffu + ((x >> 16) & 1u);
  return (uint16_t)(x >> 16);
}

// ---------------------------------------------------------------- threads
// A small fixed pool; parallel_for splits [0, n) into contiguous blocks.
class Pool {
 public:
  explicit Pool(int n) : n_(std::max(1, n)) {
    for (int i = 1; i < n_; ++i) th_.emplace_back([this, i] { loop(i); });
  }
  ~Pool() {
    {
      std::lock_guard<std::mutex> g(m_);
      stop_ = true;
      ++gen_;
    }
    cv_.notify_all();
    for (auto& t : th_) t.join();
  }
  int size() const { return n_; }
  void parallel_for(int64_t n, const std::function<void(int64_t, int64_t)>& f) {
    if (n <= 0) return;
    if (n_ == 1 || n < 2 * n_) {
      f(0, n);
      return;
    }
    {
      std::lock_guard<std::mutex> g(m_);
      job_ = &f;
      jn_ = n;
      pending_ = n_ - 1;
      ++gen_;
    }
    cv_.notify_all();
    run_block(0, f, n);
    std::unique_lock<std::mutex> lk(m_);
    done_cv_.wait(lk, [this] { return pending_ == 0; });
    job_ = nullptr;
  }

 private:
  void run_block(int i, const std::function<void(int64_t, int64_t)>& f, int64_t n) {
    int64_t per = (n + n_ - 1) / n_;
    int64_t b = (int64_t)i * per, e = std::min(n, b + per);
    if (b < e) f(b, e);
  }
  void loop(int i) {
    uint64_t seen = 0;
    for (;;) {
      const std::function<void(int64_t, int64_t)>* f;
      int64_t n;
      {
        std::unique_lock<std::mutex> lk(m_);
        cv_.wait(lk, [&] { return gen_ != seen; });
        seen = gen_;
        if (stop_) return;
        f = job_;
        n = jn_;
      }
      run_block(i, *f, n);
      {
        std::lock_guard<std::mutex> g(m_);
        if (--pending_ == 0) done_cv_.notify_all();
      }
    }
  }
  int n_;
  std::vector<std::thread> th_;
  std::mutex m_;
  std::condition_variable cv_, done_cv_;
  const std::function<void(int64_t, int64_t)>* job_ = nullptr;
  int64_t jn_ = 0;
  int pending_ = 0;
  uint64_t gen_ = 0;
  bool stop_ = false;
};

thread_local std::string g_err;

}  // namespace

extern "C" {

typedef struct {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate;
  int32_t n_experts, top_k, expert_intermediate, vocab, tied_embeddings;
  double rms_eps, rope_theta;
} orc_shape;

const char* orc_last_error(void) { return g_err.c_str(); }

// ---------------------------------------------------------------- primitives
// Each primitive is also exported so the pins can test it on its own.

// RMSNorm: y = x / sqrt(mean(x^2) + eps) * g.   (g may be null: gain 1)
void orc_rmsnorm(const double* x, const double* g, int64_t n, double eps, double* y) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
  double r = 1.0 / std::sqrt(ss / (double)n + eps);
  for (int64_t i = 0; i < n; ++i) y[i] = x[i] * r * (g ? g[i] : 1.0);
}

// y[i] = sum_k W[i,k] x[k], W bf16 row-major [n_out, n_in].
void orc_matvec_rows(const uint16_t* W, const double* x, int64_t n_in, int64_t r0, int64_t r1, double* y) {
  for (int64_t i = r0; i < r1; ++i) {
    const uint16_t* w = W + i * n_in;
    double acc = 0.0;
    for (int64_t k = 0; k < n_in; ++k) acc += bf16_to_double(w[k]) * x[k];
    y[i] = acc;
  }
}
void orc_matvec(const uint16_t* W, const double* x, int64_t n_out, int64_t n_in, double* y) {
  orc_matvec_rows(W, x, n_in, 0, n_out, y);
}

// RoPE, rotate-half pairing (i, i + D/2): the angle of pair i at position p is
// p * theta^(-2i/D).
void orc_rope(double* v, int64_t D, int64_t pos, double theta) {
  int64_t h = D / 2;
  for (int64_t i = 0; i < h; ++i) {
    double ang = (double)pos * std::pow(theta, -2.0 * (double)i / (double)D);
    double c = std::cos(ang), s = std::sin(ang);
    double a = v[i], b = v[i + h];
    v[i] = a * c - b * s;
    v[i + h] = b * c + a * s;
  }
}

// Single-head attention over T cached positions: s_t = q.K_t / sqrt(D),
// w = softmax(s) (max subtracted), o = sum_t w_t V_t.  K, V are bf16 with row
// stride `stride` elements.  `wts` (optional) receives the T softmax weights.
void orc_attention(const double* q, const uint16_t* K, const uint16_t* V, int64_t T, int64_t D, int64_t stride,
                   double* o, double* wts) {
  std::vector<double> s((size_t)std::max<int64_t>(T, 1));
  double scale = 1.0 / std::sqrt((double)D);
  double m = -INFINITY;
  for (int64_t t = 0; t < T; ++t) {
    double acc = 0.0;
    for (int64_t d = 0; d < D; ++d) acc += q[d] * bf16_to_double(K[t * stride + d]);
    s[t] = acc * scale;
    m = std::max(m, s[t]);
  }
  double den = 0.0;
  for (int64_t t = 0; t < T; ++t) {
    s[t] = std::exp(s[t] - m);
    den += s[t];
  }
  for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
  for (int64_t t = 0; t < T; ++t) {
    double w = s[t] / den;
    if (wts) wts[t] = w;
    for (int64_t d = 0; d < D; ++d) o[d] += w * bf16_to_double(V[t * stride + d]);
  }
}

double orc_silu(double z) { return z / (1.0 + std::exp(-z)); }

// Router: p = softmax(logits[0..E)); the k largest p (ties: lower index
// first); weights renormalised over the chosen k.
void orc_route(const double* logits, int32_t E, int32_t k, int32_t* experts, double* weights) {
  std::vector<double> p((size_t)E);
  double m = -INFINITY;
  for (int e = 0; e < E; ++e) m = std::max(m, logits[e]);
  double den = 0.0;
  for (int e = 0; e < E; ++e) {
    p[e] = std::exp(logits[e] - m);
    den += p[e];
  }
  for (int e = 0; e < E; ++e) p[e] /= den;
  std::vector<char> taken((size_t)E, 0);
  double tot = 0.0;
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int e = 0; e < E; ++e)
      if (!taken[e] && (best < 0 || p[e] > p[best])) best = e;
    taken[best] = 1;
    experts[j] = best;
    weights[j] = p[best];
    tot += p[best];
  }
  for (int j = 0; j < k; ++j) weights[j] /= tot;
}

// Weights of a given choice of k experts: the softmax over all E router
// logits, renormalised over the chosen experts (the same definition as
// orc_route, with the choice taken as input instead of the k largest).
void orc_route_weights(const double* logits, int32_t E, int32_t k, const int32_t* experts, double* weights) {
  double m = -INFINITY;
  for (int e = 0; e < E; ++e) m = std::max(m, logits[e]);
  double den = 0.0;
  for (int e = 0; e < E; ++e) den += std::exp(logits[e] - m);
  double tot = 0.0;
  for (int j = 0; j < k; ++j) {
    weights[j] = std::exp(logits[experts[j]] - m) / den;
    tot += weights[j];
  }
  for (int j = 0; j < k; ++j) weights[j] /= tot;
}

// How close a top-k choice came to a tie: the smallest logit among the k
// chosen experts minus the largest logit among the others (0 for an exact
// tie across the boundary; +inf when k = E).
double orc_route_gap(const double* logits, int32_t E, int32_t k, const int32_t* experts) {
  std::vector<char> chosen((size_t)E, 0);
  for (int j = 0; j < k; ++j) chosen[experts[j]] = 1;
  double lo_in = INFINITY, hi_out = -INFINITY;
  for (int e = 0; e < E; ++e) {
    if (chosen[e]) lo_in = std::min(lo_in, logits[e]);
    else hi_out = std::max(hi_out, logits[e]);
  }
  return lo_in - hi_out;
}

}  // extern "C"

// ---------------------------------------------------------------- the model
struct orc_model {
  orc_shape s{};
  int32_t B = 0, cap = 0;
  std::map<std::string, const uint16_t*> w;
  std::map<std::string, std::pair<int64_t, int64_t>> dims;
  std::vector<uint16_t> K, V;  // [L][B][Hkv][cap][D]
  Pool* pool = nullptr;
  // routing of the last decode step: [L][B][top_k]
  std::vector<int32_t> route_e;
  std::vector<double> route_w;
  std::vector<double> route_gap;  // [L][B]: smallest chosen logit minus largest unchosen logit
  std::vector<double> route_logits;  // [L][B][E]: router logits of the last decode step
  // optional forced expert choice [L][B][top_k] for the next decode steps
  std::vector<int32_t> forced;
};

namespace {

const uint16_t* need(orc_model* m, const std::string& name, int64_t rows, int64_t cols) {
  auto it = m->w.find(name);
  if (it == m->w.end()) throw std::runtime_error("missing tensor " + name);
  auto d = m->dims[name];
  if (d.first != rows || d.second != cols)
    throw std::runtime_error("tensor " + name + " has the wrong shape");
  return it->second;
}

std::vector<double> gain(orc_model* m, const std::string& name, int64_t n) {
  const uint16_t* g = need(m, name, n, 1);
  std::vector<double> v((size_t)n);
  for (int64_t i = 0; i < n; ++i) v[i] = bf16_to_double(g[i]);
  return v;
}

void matvec_par(orc_model* m, const uint16_t* W, const double* x, int64_t n_out, int64_t n_in, double* y) {
  m->pool->parallel_for(n_out, [&](int64_t a, int64_t b) { orc_matvec_rows(W, x, n_in, a, b, y); });
}

size_t kv_index(const orc_model* m, int l, int b, int g, int64_t pos) {
  const orc_shape& s = m->s;
  return ((((size_t)l * m->B + b) * s.n_kv_heads + g) * (size_t)m->cap + (size_t)pos) * (size_t)s.head_dim;
}

// SwiGLU MLP: down( silu(gate h) * (up h) ).
void mlp(orc_model* m, const std::string& pre, const double* h, int64_t H, int64_t I, double* out) {
  std::vector<double> g((size_t)I), u((size_t)I);
  matvec_par(m, need(m, pre + "w_gate", I, H), h, I, H, g.data());
  matvec_par(m, need(m, pre + "w_up", I, H), h, I, H, u.data());
  for (int64_t i = 0; i < I; ++i) g[i] = orc_silu(g[i]) * u[i];
  matvec_par(m, need(m, pre + "w_down", H, I), g.data(), H, I, out);
}

// The per-layer body shared by incremental decode and the full recompute.
// `kv_at(t)` gives the bf16 K and V rows of position t for kv head g.
// x is the residual stream of one sequence at position `pos`; it is updated
// in place.  The new k/v (already rounded to bf16) are returned in kb/vb.
struct LayerIO {
  std::vector<uint16_t> kb, vb;  // [Hkv][D]
};

void attention_block(orc_model* m, int l, double* x, int64_t pos,
                     const std::function<void(int g, int64_t t, const uint16_t** k, const uint16_t** v)>& kv_at,
                     const std::function<void(int g, const uint16_t* k, const uint16_t* v)>& store_kv) {
  const orc_shape& s = m->s;
  const int64_t H = s.hidden, D = s.head_dim, Hq = s.n_q_heads, Hkv = s.n_kv_heads, G = Hq / Hkv;
  const std::string pre = "layers." + std::to_string(l) + ".";
  std::vector<double> h((size_t)H);
  std::vector<double> gin = gain(m, pre + "in_norm", H);
  orc_rmsnorm(x, gin.data(), H, s.rms_eps, h.data());
  std::vector<double> q((size_t)(Hq * D)), k((size_t)(Hkv * D)), v((size_t)(Hkv * D));
  matvec_par(m, need(m, pre + "wq", Hq * D, H), h.data(), Hq * D, H, q.data());
  matvec_par(m, need(m, pre + "wk", Hkv * D, H), h.data(), Hkv * D, H, k.data());
  matvec_par(m, need(m, pre + "wv", Hkv * D, H), h.data(), Hkv * D, H, v.data());
  std::vector<double> gq = gain(m, pre + "q_norm", D), gk = gain(m, pre + "k_norm", D);
  for (int64_t hh = 0; hh < Hq; ++hh) {
    orc_rmsnorm(&q[hh * D], gq.data(), D, s.rms_eps, &q[hh * D]);
    orc_rope(&q[hh * D], D, pos, s.rope_theta);
  }
  std::vector<uint16_t> kb((size_t)D), vb((size_t)D);
  for (int64_t g = 0; g < Hkv; ++g) {
    orc_rmsnorm(&k[g * D], gk.data(), D, s.rms_eps, &k[g * D]);
    orc_rope(&k[g * D], D, pos, s.rope_theta);
    for (int64_t d = 0; d < D; ++d) {
      kb[d] = double_to_bf16(k[g * D + d]);
      vb[d] = double_to_bf16(v[g * D + d]);
    }
    store_kv((int)g, kb.data(), vb.data());
  }
  // attention over positions 0..pos of the cache (pos itself holds the new entry)
  std::vector<double> att((size_t)(Hq * D));
  const int64_t T = pos + 1;
  std::vector<uint16_t> Kg((size_t)(T * D)), Vg((size_t)(T * D));
  for (int64_t g = 0; g < Hkv; ++g) {
    for (int64_t t = 0; t < T; ++t) {
      const uint16_t *kr, *vr;
      kv_at((int)g, t, &kr, &vr);
      std::memcpy(&Kg[t * D], kr, D * 2);
      std::memcpy(&Vg[t * D], vr, D * 2);
    }
    for (int64_t j = 0; j < G; ++j) {
      int64_t hh = g * G + j;
      orc_attention(&q[hh * D], Kg.data(), Vg.data(), T, D, D, &att[hh * D], nullptr);
    }
  }
  std::vector<double> o((size_t)H);
  matvec_par(m, need(m, pre + "wo", H, Hq * D), att.data(), H, Hq * D, o.data());
  for (int64_t i = 0; i < H; ++i) x[i] += o[i];
}

void ffn_block(orc_model* m, int l, int b, double* x) {
  const orc_shape& s = m->s;
  const int64_t H = s.hidden;
  const std::string pre = "layers." + std::to_string(l) + ".";
  std::vector<double> h((size_t)H), y((size_t)H);
  std::vector<double> gp = gain(m, pre + "post_norm", H);
  orc_rmsnorm(x, gp.data(), H, s.rms_eps, h.data());
  if (s.n_experts == 0) {
    mlp(m, pre, h.data(), H, s.intermediate, y.data());
    for (int64_t i = 0; i < H; ++i) x[i] += y[i];
    return;
  }
  const int E = s.n_experts, Kt = s.top_k;
  std::vector<double> r((size_t)E);
  matvec_par(m, need(m, pre + "router", E, H), h.data(), E, H, r.data());
  std::vector<int32_t> ex((size_t)Kt);
  std::vector<double> wt((size_t)Kt);
  if (b >= 0 && !m->forced.empty()) {
    // a given choice (another decoder's valid routing), weighted by the definition
    for (int j = 0; j < Kt; ++j) ex[j] = m->forced[((size_t)l * m->B + b) * Kt + j];
    orc_route_weights(r.data(), E, Kt, ex.data(), wt.data());
  } else {
    orc_route(r.data(), E, Kt, ex.data(), wt.data());
  }
  if (b >= 0) {
    for (int j = 0; j < Kt; ++j) {
      m->route_e[((size_t)l * m->B + b) * Kt + j] = ex[j];
      m->route_w[((size_t)l * m->B + b) * Kt + j] = wt[j];
    }
    std::copy(r.begin(), r.end(), m->route_logits.begin() + ((size_t)l * m->B + b) * E);
    // how close the top-k choice came to a tie (in logit units): a decision
    // another precision may take differently when this is tiny
    m->route_gap[(size_t)l * m->B + b] = orc_route_gap(r.data(), E, Kt, ex.data());
  }
  std::vector<double> acc((size_t)H, 0.0);
  for (int j = 0; j < Kt; ++j) {
    mlp(m, pre + "experts." + std::to_string(ex[j]) + ".", h.data(), H, s.expert_intermediate, y.data());
    for (int64_t i = 0; i < H; ++i) acc[i] += wt[j] * y[i];
  }
  for (int64_t i = 0; i < H; ++i) x[i] += acc[i];
}

void logits_of(orc_model* m, const double* x, double* out) {
  const orc_shape& s = m->s;
  const int64_t H = s.hidden, V = s.vocab;
  std::vector<double> h((size_t)H);
  std::vector<double> gf = gain(m, "final_norm", H);
  orc_rmsnorm(x, gf.data(), H, s.rms_eps, h.data());
  const uint16_t* W = s.tied_embeddings ? need(m, "embed", V, H) : need(m, "lm_head", V, H);
  matvec_par(m, W, h.data(), V, H, out);
}

void embed_row(orc_model* m, int32_t tok, double* x) {
  const int64_t H = m->s.hidden;
  const uint16_t* E = need(m, "embed", m->s.vocab, H);
  if (tok < 0 || tok >= m->s.vocab) throw std::runtime_error("token id out of range");
  for (int64_t i = 0; i < H; ++i) x[i] = bf16_to_double(E[(int64_t)tok * H + i]);
}

}  // namespace

extern "C" {

orc_model* orc_create(const orc_shape* s, int32_t batch, int32_t cap, int32_t nthreads) {
  try {
    if (!s || batch <= 0 || cap <= 0) throw std::runtime_error("bad arguments");
    if (s->n_q_heads % s->n_kv_heads != 0 || s->head_dim % 2 != 0) throw std::runtime_error("bad head layout");
    auto* m = new orc_model();
    m->s = *s;
    m->B = batch;
    m->cap = cap;
    size_t kvn = (size_t)s->n_layers * batch * s->n_kv_heads * (size_t)cap * s->head_dim;
    m->K.assign(kvn, 0);
    m->V.assign(kvn, 0);
    if (nthreads <= 0) nthreads = (int)std::max(1u, std::thread::hardware_concurrency());
    m->pool = new Pool(nthreads);
    if (s->n_experts > 0) {
      m->route_e.assign((size_t)s->n_layers * batch * s->top_k, -1);
      m->route_w.assign((size_t)s->n_layers * batch * s->top_k, 0.0);
      m->route_gap.assign((size_t)s->n_layers * batch, INFINITY);
      m->route_logits.assign((size_t)s->n_layers * batch * s->n_experts, 0.0);
    }
    return m;
  } catch (const std::exception& e) {
    g_err = e.what();
    return nullptr;
  }
}

void orc_destroy(orc_model* m) {
  if (!m) return;
  delete m->pool;
  delete m;
}

int32_t orc_threads(const orc_model* m) { return m ? m->pool->size() : 0; }

// Borrow a bf16 tensor (the caller keeps it alive).  Vectors use cols = 1.
int32_t orc_set_weight(orc_model* m, const char* name, const uint16_t* data, int64_t rows, int64_t cols) {
  if (!m || !name || !data || rows <= 0 || cols <= 0) {
    g_err = "bad arguments";
    return -1;
  }
  m->w[name] = data;
  m->dims[name] = {rows, cols};
  return 0;
}

uint16_t* orc_kv(orc_model* m, int32_t which) { return which == 0 ? m->K.data() : m->V.data(); }
int64_t orc_kv_elems(const orc_model* m) { return (int64_t)m->K.size(); }

// One decode step for every sequence b: token tokens[b] at position
// positions[b].  Writes its new K/V at that position of the oracle's own
// cache and attends over positions 0..positions[b].  logits: [B][V];
// resid (optional): the final residual stream [B][H].
int32_t orc_decode(orc_model* m, const int32_t* tokens, const int32_t* positions, double* logits, double* resid) {
  try {
    const orc_shape& s = m->s;
    const int64_t H = s.hidden, D = s.head_dim;
    for (int b = 0; b < m->B; ++b) {
      const int64_t pos = positions[b];
      if (pos < 0 || pos >= m->cap) throw std::runtime_error("position outside the cache");
      std::vector<double> x((size_t)H);
      embed_row(m, tokens[b], x.data());
      for (int l = 0; l < s.n_layers; ++l) {
        attention_block(
            m, l, x.data(), pos,
            [&](int g, int64_t t, const uint16_t** k, const uint16_t** v) {
              *k = &m->K[kv_index(m, l, b, g, t)];
              *v = &m->V[kv_index(m, l, b, g, t)];
            },
            [&](int g, const uint16_t* k, const uint16_t* v) {
              std::memcpy(&m->K[kv_index(m, l, b, g, pos)], k, D * 2);
              std::memcpy(&m->V[kv_index(m, l, b, g, pos)], v, D * 2);
            });
        ffn_block(m, l, b, x.data());
      }
      logits_of(m, x.data(), logits + (size_t)b * s.vocab);
      if (resid) std::memcpy(resid + (size_t)b * H, x.data(), H * sizeof(double));
    }
    return 0;
  } catch (const std::exception& e) {
    g_err = e.what();
    return -1;
  }
}

// Full causal recompute without the cache: tokens[0..n) at positions 0..n-1
// through every layer, each layer computing its keys/values for all positions
// (rounded to bf16 as the cache would store them).  Returns the logits of the
// last position.  Used to pin the incremental KV-cache path.
int32_t orc_full_forward(orc_model* m, const int32_t* tokens, int32_t n, double* logits_last) {
  try {
    const orc_shape& s = m->s;
    const int64_t H = s.hidden, D = s.head_dim, Hkv = s.n_kv_heads;
    if (n <= 0) throw std::runtime_error("empty sequence");
    std::vector<std::vector<double>> xs((size_t)n, std::vector<double>((size_t)H));
    for (int t = 0; t < n; ++t) embed_row(m, tokens[t], xs[t].data());
    for (int l = 0; l < s.n_layers; ++l) {
      // keys/values of every position of this layer, [t][g][D]
      std::vector<uint16_t> Kl((size_t)n * Hkv * D), Vl((size_t)n * Hkv * D);
      // pass 1: the attention block of every position needs the keys of all
      // earlier positions of this layer, so positions are processed in order
      // and each one's k/v is stored before the next position's attention.
      for (int t = 0; t < n; ++t) {
        attention_block(
            m, l, xs[t].data(), t,
            [&](int g, int64_t u, const uint16_t** k, const uint16_t** v) {
              *k = &Kl[((size_t)u * Hkv + g) * D];
              *v = &Vl[((size_t)u * Hkv + g) * D];
            },
            [&](int g, const uint16_t* k, const uint16_t* v) {
              std::memcpy(&Kl[((size_t)t * Hkv + g) * D], k, D * 2);
              std::memcpy(&Vl[((size_t)t * Hkv + g) * D], v, D * 2);
            });
        ffn_block(m, l, -1, xs[t].data());
      }
    }
    logits_of(m, xs[n - 1].data(), logits_last);
    return 0;
  } catch (const std::exception& e) {
    g_err = e.what();
    return -1;
  }
}

// Smallest routing gap (chosen minus unchosen router logit) of sequence b
// over all layers of the last orc_decode; +inf for dense models.
double orc_last_routing_gap(const orc_model* m, int32_t b) {
  double g = INFINITY;
  if (!m || m->s.n_experts == 0) return g;
  for (int l = 0; l < m->s.n_layers; ++l) g = std::min(g, m->route_gap[(size_t)l * m->B + b]);
  return g;
}

// Router logits of (layer, b) in the last orc_decode: E values.
int32_t orc_last_router_logits(const orc_model* m, int32_t layer, int32_t b, double* out) {
  if (!m || m->s.n_experts == 0 || layer < 0 || layer >= m->s.n_layers || b < 0 || b >= m->B) return -1;
  const int E = m->s.n_experts;
  std::copy(m->route_logits.begin() + ((size_t)layer * m->B + b) * E,
            m->route_logits.begin() + ((size_t)layer * m->B + b + 1) * E, out);
  return 0;
}

// Force the expert choice of the following orc_decode calls: experts
// [L][B][top_k] (each row k distinct ids), weighted by orc_route_weights; NULL
// restores the top-k choice.  The full causal recompute is never forced.
int32_t orc_force_routing(orc_model* m, const int32_t* experts) {
  if (!m || m->s.n_experts == 0) {
    g_err = "no routed experts";
    return -1;
  }
  if (!experts) {
    m->forced.clear();
    return 0;
  }
  const int E = m->s.n_experts, Kt = m->s.top_k;
  const size_t n = (size_t)m->s.n_layers * m->B * Kt;
  for (size_t i = 0; i < n; i += Kt) {
    for (int j = 0; j < Kt; ++j) {
      const int e = experts[i + j];
      if (e < 0 || e >= E) {
        g_err = "forced expert id out of range";
        return -1;
      }
      for (int u = 0; u < j; ++u)
        if (experts[i + u] == e) {
          g_err = "forced experts of one (layer, sequence) must be distinct";
          return -1;
        }
    }
  }
  m->forced.assign(experts, experts + n);
  return 0;
}

// Routing chosen by the last orc_decode for (layer, b): top_k experts and weights.
int32_t orc_last_routing(const orc_model* m, int32_t layer, int32_t b, int32_t* experts, double* weights) {
  if (!m || m->s.n_experts == 0) return -1;
  const int Kt = m->s.top_k;
  for (int j = 0; j < Kt; ++j) {
    experts[j] = m->route_e[((size_t)layer * m->B + b) * Kt + j];
    weights[j] = m->route_w[((size_t)layer * m->B + b) * Kt + j];
  }
  return 0;
}

}  // extern "C"
