// sim_main.cpp - host-only driver for the protocol simulator, built with
// ThreadSanitizer: compiles a small decoder graph, runs the protocol on one
// host thread per worker for several steps and checks every trace.
// Exit status 0 = all checks passed.
#include <cstdio>
#include <string>
#include <vector>

#include "graph.h"

int main(int argc, char** argv) {
  const int workers = argc > 1 ? std::atoi(argv[1]) : 8;
  const int steps = argc > 2 ? std::atoi(argv[2]) : 3;
  mk_model_shape s{2, 256, 4, 2, 64, 768, 0, 0, 0, 4096, 0, 1e-6f, 1e6};
  mk_build_opts o{};
  std::string err;
  for (int fuse = 1; fuse >= 0; --fuse) {
    mk::Graph* g = mk::compile_decoder(s, 1, 64, o, workers, fuse != 0, &err);
    if (!g) {
      std::printf("compile failed: %s\n", err.c_str());
      return 2;
    }
    std::vector<mk_trace_rec> recs(g->tasks.size());
    std::vector<uint32_t> cnt(g->events.size());
    int64_t n = 0;
    int32_t rc = mk::simulate(*g, 0, steps, 0, 5000, recs.data(), (int64_t)recs.size(), &n, cnt.data(), &err);
    if (rc != MK_OK) {
      std::printf("simulate failed: %s\n", err.c_str());
      return 3;
    }
    if (!mk::check_trace(*g, recs.data(), n, (uint32_t)(steps - 1), cnt.data(), (uint32_t)steps, &err)) {
      std::printf("trace check failed: %s\n", err.c_str());
      return 4;
    }
    std::printf("fuse=%d tasks=%zu events=%zu empty=%lld: %d steps ok\n", fuse, g->tasks.size(), g->events.size(),
                (long long)g->n_empty, steps);
    delete g;
  }
  return 0;
}
