// sim_main.cpp - host-only driver for the graph compiler and the protocol
// simulator, built with ThreadSanitizer (build_tsan) and with AddressSanitizer
// plus UndefinedBehaviorSanitizer (build_asan): compiles small decoder graphs,
// runs the protocol on one host thread per worker for several steps and
// checks every trace.  Arguments: workers, steps, and "all" for the wider set
// of graphs (routed experts, merge modes, an odd worker count).
// Exit status 0 = all checks passed.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "graph.h"

static int run_one(const mk_model_shape& s, int batch, const mk_build_opts& o, int workers, bool fuse, int steps,
                   const char* label) {
  std::string err;
  mk::Graph* g = mk::compile_decoder(s, batch, 64, o, workers, fuse, &err);
  if (!g) {
    std::printf("compile failed (%s): %s\n", label, err.c_str());
    return 2;
  }
  std::vector<mk_trace_rec> recs(g->tasks.size());
  std::vector<uint32_t> cnt(g->events.size());
  int64_t n = 0;
  int32_t rc = mk::simulate(*g, 0, steps, 0, 5000, recs.data(), (int64_t)recs.size(), &n, cnt.data(), &err);
  if (rc != MK_OK) {
    std::printf("simulate failed (%s): %s\n", label, err.c_str());
    delete g;
    return 3;
  }
  if (!mk::check_trace(*g, recs.data(), n, (uint32_t)(steps - 1), cnt.data(), (uint32_t)steps, &err)) {
    std::printf("trace check failed (%s): %s\n", label, err.c_str());
    delete g;
    return 4;
  }
  std::printf("%s fuse=%d tasks=%zu events=%zu empty=%lld: %d steps ok\n", label, fuse ? 1 : 0, g->tasks.size(),
              g->events.size(), (long long)g->n_empty, steps);
  delete g;
  return 0;
}

int main(int argc, char** argv) {
  const int workers = argc > 1 ? std::atoi(argv[1]) : 8;
  const int steps = argc > 2 ? std::atoi(argv[2]) : 3;
  const bool all = argc > 3 && std::strcmp(argv[3], "all") == 0;
  const mk_model_shape dense{2, 256, 4, 2, 64, 768, 0, 0, 0, 4096, 0, 1e-6f, 1e6};
  const mk_build_opts o{};
  for (int fuse = 1; fuse >= 0; --fuse)
    if (int rc = run_one(dense, 1, o, workers, fuse != 0, steps, "dense")) return rc;
  if (!all) return 0;
  const mk_model_shape moe{2, 256, 4, 2, 64, 0, 8, 2, 64, 4096, 0, 1e-6f, 1e6};
  mk_build_opts m1{}, m2{}, c7{};
  m1.merge_tasks = 1;
  m2.merge_tasks = 2;
  c7.attn_chunks = 7;
  if (int rc = run_one(moe, 2, o, workers, true, steps, "moe")) return rc;
  if (int rc = run_one(moe, 3, o, workers + 1, false, steps, "moe-odd-workers")) return rc;
  if (int rc = run_one(dense, 2, m1, workers, true, steps, "merge-per-group")) return rc;
  if (int rc = run_one(dense, 2, m2, workers, true, steps, "merge-fused")) return rc;
  if (int rc = run_one(dense, 3, c7, workers - 1, false, steps, "chunks7")) return rc;
  return 0;
}
