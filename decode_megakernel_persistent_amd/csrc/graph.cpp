// graph.cpp - host-side compiler from a decoder shape to the task/event tables.
//
// Steps (MPK review page 2512.22219, section 2.4, which names event fusion,
// normalisation to at most one dependency and one trigger event per task, and
// BFS linearisation so that an event's fan-out is one [first, last] range; MPK
// abstract: operators are lowered to an SM-level task graph):
//   1. tiling      - every operator becomes CU-sized tasks, each with the
//                    word ranges it reads and writes (footprints)
//   2. edges       - read-after-write, write-after-read and write-after-write
//                    conflicts between footprints give task edges
//   3. reduction   - an edge u->t is dropped when another dependency of t
//                    already has every task of u's operator as an ancestor
//   4. fusion      - consumers with identical dependency sets share one event
//                    whose target is the number of producers
//   5. normalise   - a task with several dependency events gets empty tasks
//                    feeding one fresh event; a task with several trigger
//                    events triggers one fresh event whose empty dependents
//                    trigger the originals
//   6. linearise   - breadth-first over events from the root tasks; the
//                    dependents of each event get consecutive ids
//   7. assign      - each event's range is dealt round-robin over the workers
//                    from a rotating offset; work-list routing tasks go to the
//                    dispatch wavefront
#include "graph.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <deque>
#include <fstream>
#include <map>
#include <numeric>
#include <sstream>
#include <unordered_map>

namespace mk {

const char* op_kind_name(int32_t k) {
  static const char* names[] = {"empty", "embed", "qkv",    "attn",     "merge",    "oproj",  "gateup",
                                "down",  "lmhead", "router", "route", "moe_gu", "moe_down", "combine"};
  return (k >= 0 && k < OP_KINDS) ? names[k] : "?";
}

namespace {

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Split n rows into `tiles` near-equal tiles whose sizes are multiples of granule.
std::vector<std::pair<int32_t, int32_t>> split_rows(int32_t n, int32_t tiles, int32_t granule) {
  int32_t blocks = n / granule;
  tiles = std::max(1, std::min(tiles, blocks));
  std::vector<std::pair<int32_t, int32_t>> out;
  for (int32_t i = 0; i < tiles; ++i) {
    int64_t b0 = (int64_t)blocks * i / tiles, b1 = (int64_t)blocks * (i + 1) / tiles;
    out.push_back({(int32_t)(b0 * granule), (int32_t)((b1 - b0) * granule)});
  }
  return out;
}

struct Builder {
  Graph& g;
  explicit Builder(Graph& gg) : g(gg) {}

  int32_t buf(const std::string& name, int64_t words, bool virt = false) {
    Buffer b;
    b.name = name;
    b.words = words;
    b.off = virt ? -2 : -1;  // -2 marks virtual; real offsets assigned by layout()
    g.bufs.push_back(b);
    return (int32_t)g.bufs.size() - 1;
  }
  int32_t op(int32_t kind, int32_t layer, int32_t K, int32_t N, int32_t norm_in) {
    OpInst o;
    o.kind = kind;
    o.layer = layer;
    o.K = K;
    o.N = N;
    o.norm_in = norm_in;
    o.first_raw = (int32_t)g.raw.size();
    g.ops.push_back(o);
    return (int32_t)g.ops.size() - 1;
  }
  RawTask& task(int32_t op, int32_t a0 = 0, int32_t a1 = 0, int32_t a2 = 0, int32_t a3 = 0, int32_t a4 = 0) {
    RawTask t;
    t.op = op;
    t.a[0] = a0;
    t.a[1] = a1;
    t.a[2] = a2;
    t.a[3] = a3;
    t.a[4] = a4;
    g.raw.push_back(t);
    g.ops[op].ntasks++;
    return g.raw.back();
  }
  static void rd(RawTask& t, int32_t b, int64_t lo, int64_t n) { t.fp.push_back({b, lo, lo + n, false}); }
  static void wr(RawTask& t, int32_t b, int64_t lo, int64_t n) { t.fp.push_back({b, lo, lo + n, true}); }
};

// ---------------------------------------------------------------- tiling
void build_decoder_ops(Graph& g) {
  Builder bd(g);
  const mk_model_shape& s = g.shape;
  const int32_t B = g.B, H = s.hidden, Hq = s.n_q_heads, Hkv = s.n_kv_heads, D = s.head_dim, G = Hq / Hkv;
  const int32_t L = s.n_layers, V = s.vocab, W = g.W, C = g.C, gr = g.granule;
  const int32_t RG = (G + 2) * D;          // qkv rows of one kv head group
  const int32_t QN = Hkv * RG;             // qkv row length per sequence
  const int32_t PW = G * (D + 2);          // partial words of one (b, g, chunk)
  // Tiles per GEMV op: one per worker, more if the per-row results of a tile
  // (batch x rows x mult floats) would not fit the LDS result area.
  // rows per tile: the per-row results of a tile (batch x rows x mult floats)
  // must fit the LDS result area; MFMA tiles hold at most 32 row groups
  auto max_rows = [&](int32_t mult) {
    int32_t r = std::max(1, kRowResultFloats / (mult * B));
    if (g.gemv == MK_GEMV_MFMA) r = std::min(r, 512 / mult);
    return r;
  };
  auto ntiles = [&](int32_t rows, int32_t mult) {
    const int32_t mr = max_rows(mult) / gr * gr;
    return std::max(W, (rows + mr - 1) / std::max(mr, 1));
  };

  int32_t x_in = bd.buf("x0", (int64_t)B * H);
  {
    int32_t o = bd.op(OP_EMBED, -1, 0, H, 0);
    g.ops[o].out_buf = x_in;
    for (int32_t b = 0; b < B; ++b) {
      RawTask& t = bd.task(o, b);
      Builder::wr(t, x_in, (int64_t)b * H, H);
    }
  }
  for (int32_t l = 0; l < L; ++l) {
    const std::string ls = "." + std::to_string(l);
    int32_t qkv = bd.buf("qkv" + ls, (int64_t)B * QN);
    int32_t part = bd.buf("part" + ls, (int64_t)B * Hkv * C * PW);
    int32_t attn = bd.buf("attn" + ls, (int64_t)B * Hq * D);
    int32_t xo = bd.buf("xo" + ls, (int64_t)B * H);
    int32_t xd = bd.buf("xd" + ls, (int64_t)B * H);
    int32_t kvnew = bd.buf("kvnew" + ls, (int64_t)B * Hkv, true);

    // QKV: tiles aligned to kv-head groups so that each attention group
    // depends on exactly its own tiles.
    {
      int32_t o = bd.op(OP_QKV, l, H, QN, 1);
      g.ops[o].in_buf = x_in;
      g.ops[o].out_buf = qkv;
      const int32_t mr = max_rows(1) / gr * gr;
      int32_t tpg = std::max(std::max(1, W / Hkv), (RG + mr - 1) / mr);
      int32_t tile = 0;
      for (int32_t gi = 0; gi < Hkv; ++gi) {
        for (auto rr : split_rows(RG, tpg, gr)) {
          int32_t row = gi * RG + rr.first;
          RawTask& t = bd.task(o, tile++, row, rr.second, row * H);
          Builder::rd(t, x_in, 0, (int64_t)B * H);
          for (int32_t b = 0; b < B; ++b) Builder::wr(t, qkv, (int64_t)b * QN + row, rr.second);
        }
      }
    }
    // Attention chunks: (b, g, chunk); the last chunk appends the new k/v.
    // With merge_tasks == 2 the op is joint: the last chunk of (b, g) to
    // finish reads every chunk's partial and writes the merged heads.
    const bool fused = g.opts.merge_tasks == 2;
    {
      int32_t o = bd.op(OP_ATTN, l, D, 0, 0);
      g.ops[o].in_buf = qkv;
      g.ops[o].out_buf = part;
      if (fused) {
        g.ops[o].joint = true;
        g.ops[o].aux_buf = -3;  // arrival counters of this layer (separate scratch region)
        g.ops[o].aux2_buf = attn;
      }
      for (int32_t b = 0; b < B; ++b)
        for (int32_t gi = 0; gi < Hkv; ++gi)
          for (int32_t c = 0; c < C; ++c) {
            RawTask& t = bd.task(o, b, gi, c);
            Builder::rd(t, qkv, (int64_t)b * QN + (int64_t)gi * RG, RG);
            Builder::wr(t, part, (((int64_t)b * Hkv + gi) * C + c) * PW, PW);
            if (c == C - 1) Builder::wr(t, kvnew, (int64_t)b * Hkv + gi, 1);
            if (fused) {
              Builder::rd(t, part, ((int64_t)b * Hkv + gi) * C * PW, (int64_t)C * PW);
              Builder::wr(t, attn, (int64_t)b * Hq * D + (int64_t)gi * G * D, (int64_t)G * D);
            }
          }
    }
    if (!fused) {
      // merge tasks: S slices of the G*D outputs of each (b, g), each slice
      // combining the C partials of its outputs (S = 1: one task per group)
      const int32_t S = g.merge_slices;
      int32_t o = bd.op(OP_MERGE, l, D, 0, 0);
      g.ops[o].in_buf = part;
      g.ops[o].out_buf = attn;
      for (int32_t b = 0; b < B; ++b)
        for (int32_t gi = 0; gi < Hkv; ++gi)
          for (auto rr : split_rows(G * D, S, 1)) {
            RawTask& t = bd.task(o, b, gi, rr.first, rr.second);
            Builder::rd(t, part, ((int64_t)b * Hkv + gi) * C * PW, (int64_t)C * PW);
            Builder::wr(t, attn, (int64_t)b * Hq * D + (int64_t)gi * G * D + rr.first, rr.second);
          }
    }
    {
      int32_t o = bd.op(OP_OPROJ, l, Hq * D, H, 0);
      g.ops[o].in_buf = attn;
      g.ops[o].res_buf = x_in;
      g.ops[o].out_buf = xo;
      int32_t tile = 0;
      for (auto rr : split_rows(H, ntiles(H, 1), gr)) {
        RawTask& t = bd.task(o, tile++, rr.first, rr.second, rr.first * (Hq * D));
        Builder::rd(t, attn, 0, (int64_t)B * Hq * D);
        for (int32_t b = 0; b < B; ++b) {
          Builder::rd(t, x_in, (int64_t)b * H + rr.first, rr.second);
          Builder::wr(t, xo, (int64_t)b * H + rr.first, rr.second);
        }
      }
    }
    if (s.n_experts == 0) {
      const int32_t I = s.intermediate;
      int32_t act = bd.buf("act" + ls, (int64_t)B * I);
      {
        int32_t o = bd.op(OP_GATEUP, l, H, I, 1);
        g.ops[o].in_buf = xo;
        g.ops[o].out_buf = act;
        int32_t tile = 0;
        for (auto rr : split_rows(I, ntiles(I, 2), gr)) {
          RawTask& t = bd.task(o, tile++, rr.first, rr.second, 2 * rr.first * H);
          Builder::rd(t, xo, 0, (int64_t)B * H);
          for (int32_t b = 0; b < B; ++b) Builder::wr(t, act, (int64_t)b * I + rr.first, rr.second);
        }
      }
      {
        int32_t o = bd.op(OP_DOWN, l, I, H, 0);
        g.ops[o].in_buf = act;
        g.ops[o].res_buf = xo;
        g.ops[o].out_buf = xd;
        int32_t tile = 0;
        for (auto rr : split_rows(H, ntiles(H, 1), gr)) {
          RawTask& t = bd.task(o, tile++, rr.first, rr.second, rr.first * I);
          Builder::rd(t, act, 0, (int64_t)B * I);
          for (int32_t b = 0; b < B; ++b) {
            Builder::rd(t, xo, (int64_t)b * H + rr.first, rr.second);
            Builder::wr(t, xd, (int64_t)b * H + rr.first, rr.second);
          }
        }
      }
    } else {
      const int32_t E = s.n_experts, K = s.top_k, Ie = s.expert_intermediate;
      int32_t rlog = bd.buf("rlog" + ls, (int64_t)B * E);
      // routing table: per sequence K (expert, weight) pairs; per expert its
      // token count and slots; the active-expert list
      int32_t route = bd.buf("route" + ls, (int64_t)B * K * 2 + (int64_t)E * (B + 1) + E + 1);
      int32_t mact = bd.buf("mact" + ls, (int64_t)B * K * Ie);
      int32_t my = bd.buf("my" + ls, (int64_t)B * K * H);
      {
        int32_t o = bd.op(OP_ROUTER, l, H, E, 1);
        g.ops[o].in_buf = xo;
        g.ops[o].out_buf = rlog;
        int32_t tile = 0;
        for (auto rr : split_rows(E, std::max(1, std::min(W, E / std::max(gr, 16))), gr)) {
          RawTask& t = bd.task(o, tile++, rr.first, rr.second, rr.first * H);
          Builder::rd(t, xo, 0, (int64_t)B * H);
          for (int32_t b = 0; b < B; ++b) Builder::wr(t, rlog, (int64_t)b * E + rr.first, rr.second);
        }
      }
      {
        int32_t o = bd.op(OP_ROUTE, l, E, K, 0);
        g.ops[o].in_buf = rlog;
        g.ops[o].out_buf = route;
        RawTask& t = bd.task(o, 0);
        Builder::rd(t, rlog, 0, (int64_t)B * E);
        Builder::wr(t, route, 0, g.bufs[route].words);
      }
      {
        int32_t o = bd.op(OP_MOE_GU, l, H, Ie, 1);
        g.ops[o].joint = true;
        g.ops[o].in_buf = xo;
        g.ops[o].aux_buf = route;
        g.ops[o].out_buf = mact;
        for (int32_t sl = 0; sl < W; ++sl) {
          RawTask& t = bd.task(o, sl);
          Builder::rd(t, route, 0, g.bufs[route].words);
          Builder::rd(t, xo, 0, (int64_t)B * H);
          Builder::wr(t, mact, 0, g.bufs[mact].words);
        }
      }
      {
        int32_t o = bd.op(OP_MOE_DOWN, l, Ie, H, 0);
        g.ops[o].joint = true;
        g.ops[o].in_buf = mact;
        g.ops[o].aux_buf = route;
        g.ops[o].out_buf = my;
        for (int32_t sl = 0; sl < W; ++sl) {
          RawTask& t = bd.task(o, sl);
          Builder::rd(t, route, 0, g.bufs[route].words);
          Builder::rd(t, mact, 0, g.bufs[mact].words);
          Builder::wr(t, my, 0, g.bufs[my].words);
        }
      }
      {
        int32_t o = bd.op(OP_COMBINE, l, K, H, 0);
        g.ops[o].in_buf = my;
        g.ops[o].aux_buf = route;
        g.ops[o].res_buf = xo;
        g.ops[o].out_buf = xd;
        int32_t tile = 0;
        for (auto rr : split_rows(H, W, 1)) {
          RawTask& t = bd.task(o, tile++, rr.first, rr.second);
          Builder::rd(t, route, 0, (int64_t)B * K * 2);
          Builder::rd(t, my, 0, g.bufs[my].words);
          for (int32_t b = 0; b < B; ++b) {
            Builder::rd(t, xo, (int64_t)b * H + rr.first, rr.second);
            Builder::wr(t, xd, (int64_t)b * H + rr.first, rr.second);
          }
        }
      }
    }
    x_in = xd;
  }
  {
    int32_t logits = bd.buf("logits", (int64_t)B * V, true);
    int32_t o = bd.op(OP_LMHEAD, -1, H, V, 1);
    g.ops[o].in_buf = x_in;
    g.ops[o].out_buf = logits;
    // one tile per worker unless a tile would exceed 1024 rows
    int32_t per = (V + W - 1) / W;
    int32_t nt = std::max(W * std::max(1, (per + 1023) / 1024), ntiles(V, 1));
    int32_t tile = 0;
    for (auto rr : split_rows(V, nt, gr)) {
      RawTask& t = bd.task(o, tile++, rr.first, rr.second, rr.first * H);
      Builder::rd(t, x_in, 0, (int64_t)B * H);
      for (int32_t b = 0; b < B; ++b) Builder::wr(t, logits, (int64_t)b * V + rr.first, rr.second);
    }
  }
}

// ---------------------------------------------------------------- edges
struct Seg {
  int64_t end;
  int32_t writer_op = -1;
  std::vector<int32_t> writers, readers;
};
using SegMap = std::map<int64_t, Seg>;

void split_at(SegMap& m, int64_t pos) {
  auto it = m.upper_bound(pos);
  if (it == m.begin()) return;
  --it;
  if (it->first == pos || it->second.end <= pos) return;
  Seg tail = it->second;
  it->second.end = pos;
  m.emplace(pos, std::move(tail));
}

bool derive_edges(Graph& g, std::vector<std::vector<int32_t>>& deps, std::string* err) {
  const int32_t n = (int32_t)g.raw.size();
  std::vector<SegMap> st(g.bufs.size());
  for (size_t b = 0; b < g.bufs.size(); ++b) {
    Seg s;
    s.end = g.bufs[b].words;
    st[b].emplace(0, s);
  }
  deps.assign(n, {});
  // Readers only matter for write-after-read edges, i.e. while a later op
  // still writes the buffer; single-assignment buffers skip that bookkeeping.
  std::vector<int32_t> last_write_op(g.bufs.size(), -1);
  for (int32_t oi = 0; oi < (int32_t)g.ops.size(); ++oi)
    for (int32_t t = g.ops[oi].first_raw; t < g.ops[oi].first_raw + g.ops[oi].ntasks; ++t)
      for (const Footprint& f : g.raw[t].fp)
        if (f.write) last_write_op[f.buf] = std::max(last_write_op[f.buf], oi);
  for (int32_t oi = 0; oi < (int32_t)g.ops.size(); ++oi) {
    const OpInst& op = g.ops[oi];
    const int32_t t0 = op.first_raw, t1 = op.first_raw + op.ntasks;
    for (int32_t t = t0; t < t1; ++t) {
      for (const Footprint& f : g.raw[t].fp) {
        if (f.begin < 0 || f.end > g.bufs[f.buf].words || f.begin >= f.end) {
          *err = "footprint out of range in op " + std::string(op_kind_name(op.kind));
          return false;
        }
        SegMap& m = st[f.buf];
        auto it = m.upper_bound(f.begin);
        --it;
        for (; it != m.end() && it->first < f.end; ++it) {
          for (int32_t w : it->second.writers)
            if (deps[t].empty() || deps[t].back() != w) deps[t].push_back(w);
          if (f.write)
            for (int32_t r : it->second.readers)
              if (deps[t].empty() || deps[t].back() != r) deps[t].push_back(r);
        }
      }
      std::sort(deps[t].begin(), deps[t].end());
      deps[t].erase(std::unique(deps[t].begin(), deps[t].end()), deps[t].end());
    }
    // update: writes first, then reads
    for (int pass = 0; pass < 2; ++pass) {
      for (int32_t t = t0; t < t1; ++t) {
        for (const Footprint& f : g.raw[t].fp) {
          if (f.write != (pass == 0)) continue;
          if (!f.write && oi >= last_write_op[f.buf] && !(g.ops[oi].joint)) {
            // no later writer: only the same-op read/write conflict check remains
            SegMap& m = st[f.buf];
            auto it = m.upper_bound(f.begin);
            --it;
            for (; it != m.end() && it->first < f.end; ++it)
              if (it->second.writer_op == oi)
                for (int32_t w : it->second.writers)
                  if (w != t) {
                    *err = "a task reads words another task of its op writes";
                    return false;
                  }
            continue;
          }
          SegMap& m = st[f.buf];
          split_at(m, f.begin);
          split_at(m, f.end);
          for (auto it = m.find(f.begin); it != m.end() && it->first < f.end; ++it) {
            Seg& s = it->second;
            if (f.write) {
              if (s.writer_op != oi) {
                s.writer_op = oi;
                s.writers.assign(1, t);
                s.readers.clear();
              } else {
                if (!op.joint) {
                  *err = "two tasks of one op write the same words (" + std::string(op_kind_name(op.kind)) + ")";
                  return false;
                }
                s.writers.push_back(t);
              }
            } else {
              if (s.writer_op == oi && !op.joint) {
                for (int32_t w : s.writers)
                  if (w != t) {
                    *err = "a task reads words another task of its op writes";
                    return false;
                  }
              }
              if (s.readers.empty() || s.readers.back() != t) s.readers.push_back(t);
            }
          }
        }
      }
    }
  }
  for (auto& d : deps) {
    std::sort(d.begin(), d.end());
    d.erase(std::unique(d.begin(), d.end()), d.end());
  }
  return true;
}

// ---------------------------------------------------------------- reduction
void reduce_edges(Graph& g, std::vector<std::vector<int32_t>>& deps) {
  const int32_t n = (int32_t)g.raw.size();
  const int32_t nops = (int32_t)g.ops.size();
  const int32_t words = (nops + 63) / 64;
  std::vector<uint64_t> fa((size_t)n * words, 0);
  std::vector<int32_t> op_of(n);
  for (int32_t oi = 0; oi < nops; ++oi)
    for (int32_t t = g.ops[oi].first_raw; t < g.ops[oi].first_raw + g.ops[oi].ntasks; ++t) op_of[t] = oi;
  std::vector<uint64_t> U(words);
  for (int32_t t = 0; t < n; ++t) {
    std::fill(U.begin(), U.end(), 0);
    for (int32_t u : deps[t])
      for (int32_t w = 0; w < words; ++w) U[w] |= fa[(size_t)u * words + w];
    uint64_t* F = &fa[(size_t)t * words];
    for (int32_t w = 0; w < words; ++w) F[w] = U[w];
    // whole operators among the direct dependencies
    size_t i = 0;
    while (i < deps[t].size()) {
      int32_t oi = op_of[deps[t][i]];
      size_t j = i;
      while (j < deps[t].size() && op_of[deps[t][j]] == oi) ++j;
      if ((int32_t)(j - i) == g.ops[oi].ntasks) F[oi / 64] |= 1ull << (oi % 64);
      i = j;
    }
    std::vector<int32_t> keep;
    keep.reserve(deps[t].size());
    for (int32_t u : deps[t]) {
      int32_t oi = op_of[u];
      if (!(U[oi / 64] >> (oi % 64) & 1ull)) keep.push_back(u);
    }
    deps[t].swap(keep);
  }
}

}  // namespace

// ---------------------------------------------------------------- back end
bool finish_graph(Graph& g, std::string* err) {
  std::vector<std::vector<int32_t>> deps;
  if (!derive_edges(g, deps, err)) return false;
  std::vector<std::pair<int32_t, int32_t>> raw_edges;
  for (int32_t t = 0; t < (int32_t)deps.size(); ++t)
    for (int32_t u : deps[t]) raw_edges.push_back({u, t});
  reduce_edges(g, deps);
  int64_t nred = 0;
  for (auto& d : deps) nred += (int64_t)d.size();
  g.n_reduced_edges = nred;

  // Empty tasks get their own operator entry.
  int32_t empty_op = (int32_t)g.ops.size();
  {
    OpInst e;
    e.kind = OP_EMPTY;
    e.first_raw = (int32_t)g.raw.size();
    e.ntasks = 0;
    g.ops.push_back(e);
  }
  const int32_t n0 = (int32_t)g.raw.size();

  // ---- fusion: one event per distinct dependency set (or one per edge when
  // fusion is off), target = number of producers.
  std::vector<std::vector<int32_t>> ev_prod;                 // producers of each event
  std::vector<std::vector<int32_t>> tdep(n0), ttrig(n0);     // per task
  if (g.fuse) {
    std::map<std::vector<int32_t>, int32_t> by_set;
    for (int32_t t = 0; t < n0; ++t) {
      if (deps[t].empty()) continue;
      auto it = by_set.find(deps[t]);
      int32_t e;
      if (it == by_set.end()) {
        e = (int32_t)ev_prod.size();
        by_set.emplace(deps[t], e);
        ev_prod.push_back(deps[t]);
      } else {
        e = it->second;
      }
      tdep[t].push_back(e);
    }
  } else {
    for (int32_t t = 0; t < n0; ++t)
      for (int32_t u : deps[t]) {
        tdep[t].push_back((int32_t)ev_prod.size());
        ev_prod.push_back({u});
      }
  }
  for (int32_t e = 0; e < (int32_t)ev_prod.size(); ++e)
    for (int32_t u : ev_prod[e]) ttrig[u].push_back(e);
  // Terminal event of the logits: the lm_head tiles trigger it and no task of
  // the step waits on it; a multi-step launch waits on it before embedding the
  // next step's tokens, and its count checks that every tile ran.
  int32_t lm_raw_event = -1;
  {
    std::vector<int32_t> lm;
    for (int32_t t = 0; t < n0; ++t)
      if (g.raw[t].op >= 0 && g.ops[g.raw[t].op].kind == OP_LMHEAD && ttrig[t].empty()) lm.push_back(t);
    if (!lm.empty()) {
      lm_raw_event = (int32_t)ev_prod.size();
      ev_prod.push_back(lm);
      for (int32_t u : lm) ttrig[u].push_back(lm_raw_event);
    }
  }

  // ---- normalisation
  auto new_empty = [&](int32_t dep, int32_t trig) {
    RawTask t;
    t.op = empty_op;
    std::memset(t.a, 0, sizeof t.a);
    g.raw.push_back(t);
    g.ops[empty_op].ntasks++;
    tdep.push_back(dep >= 0 ? std::vector<int32_t>{dep} : std::vector<int32_t>{});
    ttrig.push_back(trig >= 0 ? std::vector<int32_t>{trig} : std::vector<int32_t>{});
    return (int32_t)g.raw.size() - 1;
  };
  // (i) several dependency events -> empty tasks x_j (dep e_j) all triggering e'
  for (int32_t t = 0; t < n0; ++t) {
    if (tdep[t].size() <= 1) continue;
    std::vector<int32_t> old = tdep[t];
    int32_t ep = (int32_t)ev_prod.size();
    ev_prod.push_back({});
    for (int32_t e : old) {
      int32_t x = new_empty(e, ep);
      ev_prod[ep].push_back(x);
    }
    tdep[t].assign(1, ep);
  }
  // (ii) several trigger events -> one fresh event e' whose empty dependents
  // y_j trigger the original events in place of the task
  const int32_t n1 = (int32_t)g.raw.size();
  for (int32_t u = 0; u < n1; ++u) {
    if (ttrig[u].size() <= 1) continue;
    std::vector<int32_t> old = ttrig[u];
    int32_t ep = (int32_t)ev_prod.size();
    ev_prod.push_back({u});
    ttrig[u].assign(1, ep);
    for (int32_t e : old) {
      int32_t y = new_empty(ep, e);
      for (int32_t& p : ev_prod[e])
        if (p == u) p = y;
    }
  }
  const int32_t n = (int32_t)g.raw.size();
  const int32_t ne = (int32_t)ev_prod.size();
  g.n_empty = n - n0;

  // ---- BFS linearisation
  std::vector<std::vector<int32_t>> consumers(ne);
  for (int32_t t = 0; t < n; ++t)
    if (!tdep[t].empty()) consumers[tdep[t][0]].push_back(t);
  std::vector<int32_t> pending(ne);
  for (int32_t e = 0; e < ne; ++e) pending[e] = (int32_t)ev_prod[e].size();
  std::vector<int32_t> id(n, -1);
  std::vector<int32_t> order;  // task ids -> raw
  order.reserve(n);
  std::vector<int32_t> ev_first(ne, 0), ev_last(ne, -1), ev_bfs;
  std::deque<int32_t> q;
  auto give = [&](int32_t t) {
    id[t] = (int32_t)order.size();
    order.push_back(t);
  };
  auto after = [&](int32_t t) {
    for (int32_t e : ttrig[t])
      if (--pending[e] == 0) q.push_back(e);
  };
  std::vector<int32_t> roots;
  for (int32_t t = 0; t < n; ++t)
    if (tdep[t].empty()) roots.push_back(t);
  for (int32_t t : roots) give(t);
  for (int32_t t : roots) after(t);
  int32_t roots_end = (int32_t)order.size();
  while (!q.empty()) {
    int32_t e = q.front();
    q.pop_front();
    ev_bfs.push_back(e);
    ev_first[e] = (int32_t)order.size();
    for (int32_t t : consumers[e]) give(t);
    ev_last[e] = (int32_t)order.size() - 1;
    for (int32_t t : consumers[e]) after(t);
  }
  if ((int32_t)order.size() != n) {
    *err = "task graph has a cycle";
    return false;
  }
  // renumber events in BFS order
  std::vector<int32_t> ev_new(ne, -1);
  for (int32_t i = 0; i < (int32_t)ev_bfs.size(); ++i) ev_new[ev_bfs[i]] = i;
  if ((int32_t)ev_bfs.size() != ne) {
    *err = "unreachable event";
    return false;
  }
  g.lm_event = lm_raw_event >= 0 ? ev_new[lm_raw_event] : -1;
  g.lm_tiles = lm_raw_event >= 0 ? (int32_t)ev_prod[lm_raw_event].size() : 0;
  g.events.assign(ne, Event{});
  for (int32_t e = 0; e < ne; ++e) {
    Event& ev = g.events[ev_new[e]];
    ev.need = (int32_t)ev_prod[e].size();
    ev.producers = ev.need;
    ev.first = consumers[e].empty() ? 0 : ev_first[e];
    ev.last = consumers[e].empty() ? -1 : ev_last[e];
  }
  g.tasks.assign(n, Task{});
  g.raw_to_id = id;
  for (int32_t i = 0; i < n; ++i) {
    const RawTask& r = g.raw[order[i]];
    Task& t = g.tasks[i];
    t.op = r.op;
    t.dep = tdep[order[i]].empty() ? -1 : ev_new[tdep[order[i]][0]];
    t.trig = ttrig[order[i]].empty() ? -1 : ev_new[ttrig[order[i]][0]];
    t.a0 = r.a[0];
    t.a1 = r.a[1];
    t.a2 = r.a[2];
    t.a3 = r.a[3];
    t.a4 = r.a[4];
  }
  g.raw_edges.clear();
  for (auto& e : raw_edges) g.raw_edges.push_back({id[e.first], id[e.second]});

  // ---- assignment (workers 0..W-1; the dispatch wavefront is agent W)
  std::vector<std::vector<int32_t>> lists(g.W + 1);
  int32_t off = 0;
  auto deal = [&](int32_t first, int32_t last) {
    int32_t k = 0;
    for (int32_t i = first; i <= last; ++i) {
      if (g.ops[g.tasks[i].op].kind == OP_ROUTE) {
        lists[g.W].push_back(i);
      } else {
        lists[(off + k) % g.W].push_back(i);
        ++k;
      }
    }
    off = (off + k) % g.W;
  };
  std::vector<std::pair<int32_t, int32_t>> ranges;
  if (roots_end > 0) ranges.push_back({0, roots_end - 1});
  for (int32_t e = 0; e < ne; ++e)
    if (g.events[e].last >= g.events[e].first) ranges.push_back({g.events[e].first, g.events[e].last});
  std::sort(ranges.begin(), ranges.end());
  for (auto& r : ranges) deal(r.first, r.second);
  g.wl_off.assign(g.W + 2, 0);
  g.wl_ids.clear();
  for (int32_t w = 0; w <= g.W; ++w) {
    g.wl_off[w] = (int32_t)g.wl_ids.size();
    g.wl_ids.insert(g.wl_ids.end(), lists[w].begin(), lists[w].end());
  }
  g.wl_off[g.W + 1] = (int32_t)g.wl_ids.size();

  // ---- launch-per-task ranges: one launch per (event range, operator) run
  g.launch_first.clear();
  g.launch_count.clear();
  for (auto& r : ranges) {
    int32_t i = r.first;
    while (i <= r.second) {
      int32_t j = i;
      while (j + 1 <= r.second && g.tasks[j + 1].op == g.tasks[i].op) ++j;
      g.launch_first.push_back(i);
      g.launch_count.push_back(j - i + 1);
      i = j + 1;
    }
  }
  return validate_graph(g, err);
}

bool validate_graph(const Graph& g, std::string* err) {
  const int32_t n = (int32_t)g.tasks.size(), ne = (int32_t)g.events.size();
  std::vector<int32_t> trig_count(ne, 0), max_prod_id(ne, -1);
  for (int32_t i = 0; i < n; ++i) {
    const Task& t = g.tasks[i];
    if (t.dep < -1 || t.dep >= ne || t.trig < -1 || t.trig >= ne) {
      *err = "event index out of range";
      return false;
    }
    if (t.trig >= 0) {
      trig_count[t.trig]++;
      max_prod_id[t.trig] = std::max(max_prod_id[t.trig], i);
    }
    if (t.dep >= 0) {
      const Event& e = g.events[t.dep];
      if (i < e.first || i > e.last) {
        *err = "task outside its event's range";
        return false;
      }
    }
  }
  for (int32_t e = 0; e < ne; ++e) {
    const Event& ev = g.events[e];
    if (ev.need != trig_count[e] || ev.need <= 0) {
      *err = "event need differs from its number of triggering tasks";
      return false;
    }
    for (int32_t i = ev.first; i <= ev.last; ++i)
      if (g.tasks[i].dep != e) {
        *err = "event range not contiguous";
        return false;
      }
    if (ev.last >= ev.first && max_prod_id[e] >= ev.first) {
      *err = "ids not topological";
      return false;
    }
  }
  // worker lists: a partition of the ids, each list increasing
  std::vector<char> seen(n, 0);
  for (int32_t w = 0; w + 1 < (int32_t)g.wl_off.size(); ++w)
    for (int32_t k = g.wl_off[w]; k < g.wl_off[w + 1]; ++k) {
      int32_t id = g.wl_ids[k];
      if (id < 0 || id >= n || seen[id]) {
        *err = "worker lists are not a partition";
        return false;
      }
      seen[id] = 1;
      if (k > g.wl_off[w] && g.wl_ids[k - 1] >= id) {
        *err = "worker list not increasing";
        return false;
      }
    }
  for (int32_t i = 0; i < n; ++i)
    if (!seen[i]) {
      *err = "task not assigned";
      return false;
    }
  return true;
}

// ---------------------------------------------------------------- layout
namespace {

void layout(Graph& g) {
  const mk_model_shape& s = g.shape;
  const int32_t H = s.hidden, Hq = s.n_q_heads, Hkv = s.n_kv_heads, D = s.head_dim, G = Hq / Hkv;
  const int32_t V = s.vocab, L = s.n_layers;
  const bool swz = g.gemv == MK_GEMV_MFMA;
  const int32_t wkind = swz ? CopyJob::SWZ16 : CopyJob::ROWS;
  int64_t a = 0;
  auto take = [&](int64_t bytes) {
    int64_t o = a;
    a = align_up(a + bytes, 256);
    return o;
  };
  auto rows = [&](const std::string& t, int64_t r0, int64_t nr, int64_t cols, int64_t dst, int32_t kind) {
    CopyJob c;
    c.tensor = t;
    c.row0 = r0;
    c.nrows = nr;
    c.cols = cols;
    c.dst = dst;
    c.kind = kind;
    g.copies.push_back(c);
  };
  auto gain = [&](const std::string& t, int64_t n) {
    int64_t o = take(n * 4);
    rows(t, 0, n, 1, o, CopyJob::GAIN_F32);
    return o;
  };
  int64_t embed_off = take((int64_t)V * H * 2);
  rows("embed", 0, V, H, embed_off, CopyJob::ROWS);
  g.weight_bytes_step = 0;
  for (OpInst& op : g.ops) {
    const std::string p = "layers." + std::to_string(op.layer) + ".";
    switch (op.kind) {
      case OP_EMBED:
        op.w_off = embed_off;
        break;
      case OP_QKV: {
        op.w_off = take((int64_t)op.N * H * 2);
        int64_t dst = op.w_off;
        for (int32_t gi = 0; gi < Hkv; ++gi) {
          rows(p + "wq", (int64_t)gi * G * D, (int64_t)G * D, H, dst, wkind);
          dst += (int64_t)G * D * H * 2;
          rows(p + "wk", (int64_t)gi * D, D, H, dst, wkind);
          dst += (int64_t)D * H * 2;
          rows(p + "wv", (int64_t)gi * D, D, H, dst, wkind);
          dst += (int64_t)D * H * 2;
        }
        op.g_off = gain(p + "in_norm", H);
        g.weight_bytes_step += (int64_t)op.N * H * 2;
        break;
      }
      case OP_ATTN:
        op.g_off = gain(p + "q_norm", D);
        op.g2_off = gain(p + "k_norm", D);
        break;
      case OP_OPROJ:
        op.w_off = take((int64_t)H * Hq * D * 2);
        rows(p + "wo", 0, H, (int64_t)Hq * D, op.w_off, wkind);
        g.weight_bytes_step += (int64_t)H * Hq * D * 2;
        break;
      case OP_GATEUP: {
        const int32_t I = op.N;
        op.w_off = take(2LL * I * H * 2);
        for (int32_t t = op.first_raw; t < op.first_raw + op.ntasks; ++t) {
          const RawTask& r = g.raw[t];
          int64_t dst = op.w_off + (int64_t)r.a[3] * 2;
          rows(p + "w_gate", r.a[1], r.a[2], H, dst, wkind);
          rows(p + "w_up", r.a[1], r.a[2], H, dst + (int64_t)r.a[2] * H * 2, wkind);
        }
        op.g_off = gain(p + "post_norm", H);
        g.weight_bytes_step += 2LL * I * H * 2;
        break;
      }
      case OP_DOWN:
        op.w_off = take((int64_t)H * op.K * 2);
        rows(p + "w_down", 0, H, op.K, op.w_off, wkind);
        g.weight_bytes_step += (int64_t)H * op.K * 2;
        break;
      case OP_ROUTER:
        op.w_off = take((int64_t)op.N * H * 2);
        rows(p + "router", 0, op.N, H, op.w_off, wkind);
        op.g_off = gain(p + "post_norm", H);
        g.weight_bytes_step += (int64_t)op.N * H * 2;
        break;
      case OP_MOE_GU: {
        // per expert: [gate rows | up rows] in 16-row interleaved tiles of Ie
        const int32_t E = s.n_experts, Ie = s.expert_intermediate;
        op.w_off = take((int64_t)E * 2 * Ie * H * 2);
        for (int32_t e = 0; e < E; ++e) {
          int64_t base = op.w_off + (int64_t)e * 2 * Ie * H * 2;
          std::string q = p + "experts." + std::to_string(e) + ".";
          for (int32_t r0 = 0; r0 < Ie; r0 += 16) {
            int64_t dst = base + (int64_t)r0 * 2 * H * 2;
            rows(q + "w_gate", r0, 16, H, dst, CopyJob::ROWS);
            rows(q + "w_up", r0, 16, H, dst + 16LL * H * 2, CopyJob::ROWS);
          }
        }
        op.g_off = gain(p + "post_norm", H);
        break;
      }
      case OP_MOE_DOWN: {
        const int32_t E = s.n_experts, Ie = s.expert_intermediate;
        op.w_off = take((int64_t)E * H * Ie * 2);
        for (int32_t e = 0; e < E; ++e)
          rows(p + "experts." + std::to_string(e) + ".w_down", 0, H, Ie, op.w_off + (int64_t)e * H * Ie * 2,
               CopyJob::ROWS);
        break;
      }
      case OP_LMHEAD:
        if (s.tied_embeddings && !swz) {
          op.w_off = embed_off;
        } else {
          op.w_off = take((int64_t)V * H * 2);
          rows(s.tied_embeddings ? "embed" : "lm_head", 0, V, H, op.w_off, wkind);
        }
        op.g_off = gain("final_norm", H);
        g.weight_bytes_step += (int64_t)V * H * 2;
        break;
      default:
        break;
    }
  }
  g.off_invfreq = take((int64_t)(D / 2) * 8);
  g.off_geom = take(sizeof(Geom));
  g.off_ops = take((int64_t)g.ops.size() * sizeof(OpDesc));
  g.off_ops_static = take((int64_t)g.ops.size() * sizeof(OpDesc));
  g.off_tasks = take((int64_t)g.tasks.size() * sizeof(Task));
  g.off_events = take((int64_t)std::max<size_t>(1, g.events.size()) * sizeof(Event));
  g.off_wloff = take((int64_t)g.wl_off.size() * 4);
  g.off_wlids = take((int64_t)std::max<size_t>(1, g.wl_ids.size()) * 4);
  g.arena_bytes = a;

  // scratch
  int64_t sc = 0;
  g.off_counters = sc;
  sc = align_up(sc + (int64_t)g.events.size() * kEventBytes, 256);
  g.off_status = sc;
  sc = align_up(sc + ST_WORDS * 4, 256);
  g.off_progress = sc;  // one word per agent: 1 + id of the task it is in, 0xFFFFFFFF when done
  sc = align_up(sc + (int64_t)(g.W + 1) * 4, 256);
  g.off_arrive = sc;    // attention arrival counters: [L][B][Hkv] x one 128-byte line
  sc = align_up(sc + (int64_t)g.shape.n_layers * g.B * g.shape.n_kv_heads * kCounterStride * 4, 256);
  g.off_state_end = sc; // counters .. here are the event state cleared by a reset
  for (Buffer& b : g.bufs) {
    if (b.off == -2) continue;
    b.off = sc;
    sc = align_up(sc + b.words * 8, 256);
  }
  g.off_cand = sc;  // greedy candidates of the lm_head tiles: [tile][B] x (value, id) tagged words
  sc = align_up(sc + (int64_t)std::max(1, g.lm_tiles) * g.B * 2 * 8, 256);
  if (s.n_experts > 0) {
    g.off_route_hist = sc;  // {expert, weight} [kRouteHistSteps][L][B][top_k]
    sc = align_up(sc + (int64_t)kRouteHistSteps * L * g.B * s.top_k * 8, 256);
  }
  g.scratch_bytes = sc;
  g.trace_bytes = g.opts.trace ? (int64_t)g.tasks.size() * (int64_t)sizeof(mk_trace_rec) : 0;
}

}  // namespace

uint32_t graph_magic(const Graph& g) {
  uint32_t h = 2166136261u;
  auto mix = [&](int64_t v) {
    for (int i = 0; i < 8; ++i) {
      h ^= (uint32_t)(v >> (8 * i)) & 0xffu;
      h *= 16777619u;
    }
  };
  mix(g.tasks.size());
  mix(g.events.size());
  mix(g.ops.size());
  mix(g.B);
  mix(g.cap);
  mix(g.W);
  mix(g.C);
  mix(g.gemv);
  mix(g.shape.n_layers);
  mix(g.shape.hidden);
  mix(g.shape.vocab);
  return h | 1u;
}

// Odd-numbered XCDs see event counters later and stream weights more slowly
// than even-numbered ones (measured per XCD from the timing trace: at the 8B
// batch-1 shape, gate-up tiles on odd XCDs start ~1 us later and run ~9%
// longer), so the last tile of every operator lands on an odd XCD.  For the
// O, gate-up, down and lm_head operators of VALU graphs (one dependency event
// each, so their row split does not change any edge), the rows are re-split
// after assignment: a tile whose worker w has w mod 8 odd gets
// opts.xcd_rows_pct percent of the rows of a tile on an even XCD.  Worker w
// runs on XCD w mod 8 (the device deals workgroups round-robin over the
// XCDs; the trace records it).  Runs before layout(), which places gate-up
// weights per tile.  Measured at the 8B batch-1 shape (same box, 64 steps,
// twice each), equal tiles are fastest: 78% 3.361, 85% 3.341, 92% 3.319,
// 100% 3.268, 104% 3.273, 108% 3.394, 115% 3.406 ms; the per-XCD lateness
// follows the contention rather than the work, so equal tiles stay the
// default and the split is an option.
constexpr int32_t kDefaultXcdRowsPct = 100;
static void balance_xcd_rows(Graph& g) {
  const int32_t pct = g.opts.xcd_rows_pct ? g.opts.xcd_rows_pct : kDefaultXcdRowsPct;
  if (pct == 100 || g.gemv != MK_GEMV_VALU) return;
  std::vector<int32_t> worker(g.tasks.size(), -1);
  for (int32_t w = 0; w < g.W; ++w)
    for (int32_t k = g.wl_off[w]; k < g.wl_off[w + 1]; ++k) worker[(size_t)g.wl_ids[k]] = w;
  for (OpInst& op : g.ops) {
    if (op.kind != OP_OPROJ && op.kind != OP_GATEUP && op.kind != OP_DOWN && op.kind != OP_LMHEAD) continue;
    const int32_t n = op.ntasks;
    if (n < 2) continue;
    int64_t R = 0;
    std::vector<double> wt((size_t)n);
    double wsum = 0.0;
    for (int32_t i = 0; i < n; ++i) {
      const RawTask& r = g.raw[(size_t)(op.first_raw + i)];
      R += r.a[2];
      const int32_t w = worker[(size_t)g.raw_to_id[(size_t)(op.first_raw + i)]];
      wt[(size_t)i] = (w >= 0 && (w % 8) % 2 == 1) ? pct / 100.0 : 1.0;
      wsum += wt[(size_t)i];
    }
    if (R < n) continue;
    // contiguous tiles in the original order, sizes proportional to the weights, at least one row each
    double acc = 0.0;
    int32_t r0 = 0;
    for (int32_t i = 0; i < n; ++i) {
      acc += wt[(size_t)i];
      int32_t r1 = i + 1 == n ? (int32_t)R : (int32_t)std::llround((double)R * acc / wsum);
      r1 = std::max(r1, r0 + 1);
      r1 = std::min<int32_t>(r1, (int32_t)R - (n - 1 - i));
      RawTask& r = g.raw[(size_t)(op.first_raw + i)];
      Task& t = g.tasks[(size_t)g.raw_to_id[(size_t)(op.first_raw + i)]];
      const int32_t a3 = op.kind == OP_GATEUP ? 2 * r0 * op.K : r0 * op.K;
      r.a[1] = t.a1 = r0;
      r.a[2] = t.a2 = r1 - r0;
      r.a[3] = t.a3 = a3;
      r0 = r1;
    }
  }
}

// With opts.lds_ring, batch-1 VALU GEMV tiles whose rows are whole kilobytes
// and whose input, segments and rows fit the LDS ring's areas are fed through
// the LDS weight ring (loader wavefronts stream the weights, see device.h).  The segment
// size, in KB, is the largest of 4, 2, 1 dividing every such op's row bytes
// (one size per graph, so that segments of consecutive tiles can share the
// loader's in-flight accounting).  Returns it, or 0 when no op qualifies.
static int32_t assign_ring(Graph& g) {
  if (g.B != 1 || g.gemv != MK_GEMV_VALU || !g.opts.lds_ring) return 0;
  std::vector<int32_t> max_rows(g.ops.size(), 0);
  for (const Task& t : g.tasks) {
    const OpInst& o = g.ops[(size_t)t.op];
    if (o.kind == OP_QKV || o.kind == OP_OPROJ || o.kind == OP_GATEUP || o.kind == OP_DOWN || o.kind == OP_LMHEAD)
      max_rows[(size_t)t.op] = std::max(max_rows[(size_t)t.op], o.kind == OP_GATEUP ? 2 * t.a2 : t.a2);
  }
  int32_t u = 4;
  std::vector<size_t> cand;
  for (size_t i = 0; i < g.ops.size(); ++i) {
    const OpInst& o = g.ops[i];
    if (max_rows[i] == 0 || o.K % 512 != 0 || o.K > kRingMaxK || max_rows[i] > kRingMaxRows) continue;
    while ((o.K * 2) % (u * 1024) != 0) u /= 2;
    cand.push_back(i);
  }
  // segments per tile must fit the partials area (dropping an op keeps u valid)
  bool any = false;
  for (size_t i : cand) {
    if ((int64_t)max_rows[i] * (g.ops[i].K * 2 / (u * 1024)) > kRingMaxSegs) continue;
    g.ops[i].ring = true;
    any = true;
  }
  return any ? u : 0;
}

Graph* compile_decoder(const mk_model_shape& s, int32_t batch, int32_t cap, const mk_build_opts& o, int32_t workers,
                       bool fuse, std::string* err) {
  auto bad = [&](const char* m) -> Graph* {
    *err = m;
    return nullptr;
  };
  if (s.n_layers <= 0 || s.hidden <= 0 || s.n_q_heads <= 0 || s.n_kv_heads <= 0 || s.head_dim <= 0 || s.vocab <= 0)
    return bad("shape fields must be positive");
  if (s.n_q_heads % s.n_kv_heads) return bad("n_q_heads must be a multiple of n_kv_heads");
  if (s.head_dim % 64 || s.head_dim > 128) return bad("head_dim must be 64 or 128");
  {
    const int32_t gq = s.n_q_heads / s.n_kv_heads;
    if (gq != 1 && gq != 2 && gq != 4 && gq != 8) return bad("query heads per kv head must be 1, 2, 4 or 8");
  }
  if (o.merge_tasks < 0 || o.merge_tasks > 2) return bad("merge_tasks must be 0, 1 or 2");
  if (o.attn_chunks > 64) return bad("attn_chunks must be <= 64");
  if (s.hidden % 64) return bad("hidden must be a multiple of 64");
  if (s.n_experts == 0 && (s.intermediate <= 0 || s.intermediate % 16)) return bad("intermediate must be a positive multiple of 16");
  if (s.n_experts > 0 && (s.top_k <= 0 || s.top_k > s.n_experts || s.top_k > 8 || s.expert_intermediate % 16 ||
                          s.expert_intermediate <= 0 || s.n_experts > 256))
    return bad("bad expert configuration (top_k <= 8, expert_intermediate multiple of 16, <= 256 experts)");
  if (s.n_experts > 0 && (batch > 8 || s.expert_intermediate > 1024 || s.hidden % 64 || s.hidden > 4096))
    return bad("routed experts support batch <= 8, expert_intermediate <= 1024 and hidden <= 4096");
  if (batch <= 0 || batch > 16) return bad("batch must be in 1..16");
  if (cap <= 0 || cap > (1 << 20)) return bad("max_ctx out of range");
  if (workers <= 0 || workers > 4096) return bad("worker count out of range");
  for (int i = 0; i < 2; ++i)
    if (o.reserved[i]) return bad("reserved options must be zero");
  if (o.xcd_rows_pct != 0 && (o.xcd_rows_pct < 50 || o.xcd_rows_pct > 150))
    return bad("xcd_rows_pct must be 0 or in 50..150");
  if (o.lds_ring < 0 || o.lds_ring > 1) return bad("lds_ring must be 0 or 1");
  if (o.prefetch_loads < 0 || o.prefetch_loads > 64) return bad("prefetch_loads must be in 0..64");
  if (o.trace < 0 || o.trace > 2) return bad("trace must be 0, 1 or 2");
  if (o.no_watchdog && s.n_experts > 0) return bad("no_watchdog: routed-expert graphs need the dispatch wavefront");

  Graph* g = new Graph();
  g->shape = s;
  g->B = batch;
  g->cap = cap;
  g->opts = o;
  g->W = workers;
  g->fuse = fuse;
  int32_t gm = o.gemv;
  if (gm == MK_GEMV_AUTO) gm = batch > 4 ? MK_GEMV_MFMA : MK_GEMV_VALU;
  if (gm != MK_GEMV_VALU && gm != MK_GEMV_MFMA) {
    delete g;
    return bad("unknown gemv mode");
  }
  if (gm == MK_GEMV_VALU && batch > 4) {
    delete g;
    return bad("the VALU GEMV path supports batch <= 4; use MFMA");
  }
  if (gm == MK_GEMV_VALU) {
    int64_t kmax = std::max<int64_t>({s.hidden, (int64_t)s.n_q_heads * s.head_dim, s.intermediate, s.expert_intermediate});
    if (kmax * batch > kStageFloats) {
      delete g;
      return bad("batch x input length exceeds the VALU staging area; use MFMA");
    }
  }
  g->gemv = gm;
  g->granule = gm == MK_GEMV_MFMA ? 16 : 1;
  if (gm == MK_GEMV_MFMA) {
    const int32_t I = s.n_experts ? s.expert_intermediate : s.intermediate;
    if (s.hidden % 32 || I % 32 || s.vocab % 16 || (s.n_q_heads * s.head_dim) % 32) {
      delete g;
      return bad("MFMA GEMV needs hidden/intermediate multiples of 32 and vocab multiple of 16");
    }
  }
  const int32_t bh = batch * s.n_kv_heads;
  int32_t C = o.attn_chunks;
  if (C <= 0) C = std::max(1, std::min(workers / std::max(1, bh), std::max(1, cap / 32)));
  // the scores of one chunk (G heads x chunk length, padded to whole value
  // passes of 16 rows) must fit the LDS score area
  const int64_t Gq = s.n_q_heads / s.n_kv_heads;
  while (Gq * ((cap + C - 1) / C + 16) > kScoreFloats) ++C;
  // the merge gives each chunk one lane of a wavefront
  if (C > 64) {
    delete g;
    return bad("attention needs more than 64 chunks per (sequence, kv head) for this context; reduce max_ctx");
  }
  g->C = C;
  if (o.merge_tasks == 1) g->merge_slices = 1;
  else g->merge_slices = (int32_t)std::max<int64_t>(1, std::min<int64_t>(C, Gq * s.head_dim / 16));
  build_decoder_ops(*g);
  if (!finish_graph(*g, err)) {
    delete g;
    return nullptr;
  }
  balance_xcd_rows(*g);
  layout(*g);
  Geom& ge = g->geom;
  ge.ring_u = assign_ring(*g);
  ge.B = batch;
  ge.H = s.hidden;
  ge.Hq = s.n_q_heads;
  ge.Hkv = s.n_kv_heads;
  ge.D = s.head_dim;
  ge.G = s.n_q_heads / s.n_kv_heads;
  ge.I = s.intermediate;
  ge.V = s.vocab;
  ge.L = s.n_layers;
  ge.C = g->C;
  ge.mfma = g->gemv == MK_GEMV_MFMA ? 1 : 0;
  ge.lm_event = g->lm_event;
  ge.lm_tiles = g->lm_tiles;
  ge.cap = cap;
  ge.E = s.n_experts;
  ge.topk = s.top_k;
  ge.Ie = s.expert_intermediate;
  ge.qkv_stride = s.n_kv_heads * (ge.G + 2) * s.head_dim;
  ge.part_stride = s.head_dim + 2;
  ge.n_events = (int32_t)g->events.size();
  ge.n_tasks = (int32_t)g->tasks.size();
  ge.n_workers = workers;
  ge.n_ops = (int32_t)g->ops.size();
  ge.eps = s.rms_eps;
  ge.attn_scale = (float)(1.0 / std::sqrt((double)s.head_dim));
  ge.magic = graph_magic(*g);
  return g;
}

void dump_json(const Graph& g, const std::string& path) {
  std::ofstream f(path);
  f << "{\n  \"batch\": " << g.B << ", \"max_ctx\": " << g.cap << ", \"workers\": " << g.W
    << ", \"attn_chunks\": " << g.C << ", \"gemv\": \"" << (g.gemv == MK_GEMV_MFMA ? "mfma" : "valu") << "\",\n";
  f << "  \"ops\": [";
  for (size_t i = 0; i < g.ops.size(); ++i)
    f << (i ? ", " : "") << "{\"kind\": \"" << op_kind_name(g.ops[i].kind) << "\", \"layer\": " << g.ops[i].layer
      << ", \"tasks\": " << g.ops[i].ntasks << "}";
  f << "],\n  \"events\": [";
  for (size_t i = 0; i < g.events.size(); ++i)
    f << (i ? ", " : "") << "[" << g.events[i].need << ", " << g.events[i].first << ", " << g.events[i].last << "]";
  f << "],\n  \"tasks\": [";
  for (size_t i = 0; i < g.tasks.size(); ++i) {
    const Task& t = g.tasks[i];
    f << (i ? ", " : "") << "[" << t.op << ", " << t.dep << ", " << t.trig << ", " << t.a0 << ", " << t.a1 << ", "
      << t.a2 << ", " << t.a3 << "]";
  }
  f << "],\n  \"worker_lists\": [";
  for (size_t w = 0; w + 1 < g.wl_off.size(); ++w) {
    f << (w ? ", " : "") << "[";
    for (int32_t k = g.wl_off[w]; k < g.wl_off[w + 1]; ++k) f << (k > g.wl_off[w] ? ", " : "") << g.wl_ids[k];
    f << "]";
  }
  f << "]\n}\n";
}

}  // namespace mk
