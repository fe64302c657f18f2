// sim.cpp - host-only pieces of the runtime protocol: the trace checker and a
// simulator that runs the real task/event tables on host threads.
//
// Protocol being checked (MPK review page 2512.22219, section 2.4: with at most
// one dependency and one trigger event per task, in-kernel scheduling needs
// only atomicAdd on event counters and local state): a task may start only
// after its dependency event's counter reached need * (step + 1); when done it
// adds one to its trigger event's counter.
#include <atomic>
#include <chrono>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "graph.h"

namespace mk {

namespace {
thread_local std::string g_err;
}

void set_error(const std::string& msg) { g_err = msg; }

bool check_trace(const Graph& g, const mk_trace_rec* recs, int64_t n, uint32_t step, const uint32_t* counters,
                 uint32_t steps_done, std::string* err) {
  const int64_t nt = (int64_t)g.tasks.size();
  const int32_t ne = (int32_t)g.events.size();
  auto fail = [&](const std::string& m) {
    *err = m;
    return false;
  };
  if (n != nt) return fail("trace has " + std::to_string(n) + " records but the graph has " + std::to_string(nt) + " tasks");
  std::vector<int64_t> at(nt, -1);
  for (int64_t i = 0; i < n; ++i) {
    const mk_trace_rec& r = recs[i];
    if (r.task < 0 || r.task >= nt) return fail("trace record with task id out of range: " + std::to_string(r.task));
    if (at[r.task] >= 0) return fail("task " + std::to_string(r.task) + " executed more than once");
    if (r.step != step) return fail("task " + std::to_string(r.task) + " recorded step " + std::to_string(r.step));
    if (r.t_end < r.t_start) return fail("task " + std::to_string(r.task) + " ended before it started");
    at[r.task] = i;
  }
  // (iii) a task starts only after every trigger of its dependency event ended
  std::vector<int64_t> max_end(ne, -1);
  for (int64_t t = 0; t < nt; ++t) {
    int32_t e = g.tasks[t].trig;
    if (e >= 0) max_end[e] = std::max<int64_t>(max_end[e], recs[at[t]].t_end);
  }
  for (int64_t t = 0; t < nt; ++t) {
    int32_t e = g.tasks[t].dep;
    if (e < 0) continue;
    const mk_trace_rec& r = recs[at[t]];
    if ((int64_t)r.t_start <= max_end[e])
      return fail("task " + std::to_string(t) + " started (ticket " + std::to_string(r.t_start) +
                  ") before a producer of event " + std::to_string(e) + " ended (ticket " + std::to_string(max_end[e]) + ")");
    // (iv) the counter it observed had reached the target
    uint64_t target = (uint64_t)g.events[e].need * steps_done;
    if (r.dep_seen < target)
      return fail("task " + std::to_string(t) + " saw counter " + std::to_string(r.dep_seen) + " of event " +
                  std::to_string(e) + " below target " + std::to_string(target));
  }
  // (ii) every counter equals need * steps exactly
  if (counters) {
    for (int32_t e = 0; e < ne; ++e)
      if ((uint64_t)counters[e] != (uint64_t)g.events[e].need * steps_done)
        return fail("event " + std::to_string(e) + " counter " + std::to_string(counters[e]) + " != need " +
                    std::to_string(g.events[e].need) + " x " + std::to_string(steps_done));
  }
  return true;
}

int32_t simulate(const Graph& g, int32_t threads, int32_t steps, int32_t fault, int32_t timeout_ms,
                 mk_trace_rec* recs, int64_t cap, int64_t* n, uint32_t* counters, std::string* err) {
  const int32_t agents = g.W + 1;
  const int64_t nt = (int64_t)g.tasks.size();
  const int32_t ne = (int32_t)g.events.size();
  if (threads != 0 && threads < agents) {
    *err = "the simulator needs one thread per agent (workers + dispatcher)";
    return MK_ERR_ARG;
  }
  if (steps < 1 || cap < nt || !recs || !n) {
    *err = "bad simulate arguments";
    return MK_ERR_ARG;
  }
  if (timeout_ms <= 0) timeout_ms = 2000;
  std::vector<std::atomic<uint32_t>> ctr(ne);
  for (auto& c : ctr) c.store(0);
  std::atomic<uint32_t> ticket{0};
  std::atomic<int64_t> nrec{0};
  std::atomic<int32_t> status{MK_OK};
  std::atomic<int32_t> bad_task{-1};

  // fault victims
  int32_t victim = -1;
  std::vector<char> slow_producer(nt, 0);
  if (fault == 1 || fault == 2) {
    for (int64_t t = 0; t < nt; ++t)
      if (g.tasks[t].trig >= 0) {
        victim = (int32_t)t;
        break;
      }
  } else if (fault == 3) {
    // the first task of some agent's list that has a dependency, whose earlier
    // list entries are roots, and none of whose producers run on that agent
    std::vector<int32_t> agent_of(nt, -1);
    for (int32_t a = 0; a < agents; ++a)
      for (int32_t k = g.wl_off[a]; k < g.wl_off[a + 1]; ++k) agent_of[g.wl_ids[k]] = a;
    for (int32_t a = agents - 1; a >= 0 && victim < 0; --a) {
      for (int32_t k = g.wl_off[a]; k < g.wl_off[a + 1]; ++k) {
        int32_t id = g.wl_ids[k];
        int32_t e = g.tasks[id].dep;
        if (e < 0) continue;
        bool ok = true;
        for (int64_t t = 0; t < nt; ++t)
          if (g.tasks[t].trig == e && agent_of[t] == a) ok = false;
        if (ok) {
          victim = id;
          for (int64_t t = 0; t < nt; ++t)
            if (g.tasks[t].trig == e) slow_producer[t] = 1;
        }
        break;
      }
    }
  }
  if (fault != 0 && victim < 0) {
    *err = "no task suitable for the requested fault";
    return MK_ERR_ARG;
  }

  for (int32_t step = 0; step < steps; ++step) {
    ticket.store(0);
    nrec.store(0);
    std::vector<std::thread> th;
    th.reserve(agents);
    for (int32_t a = 0; a < agents; ++a) {
      th.emplace_back([&, a, step] {
        for (int32_t k = g.wl_off[a]; k < g.wl_off[a + 1]; ++k) {
          if (status.load() != MK_OK) return;
          const int32_t id = g.wl_ids[k];
          const Task& t = g.tasks[id];
          uint32_t seen = 0;
          uint32_t start = 0;
          bool early = fault == 3 && id == victim && step == 0;
          if (early) start = ticket.fetch_add(1);
          if (t.dep >= 0 && !early) {
            const uint32_t target = (uint32_t)g.events[t.dep].need * (uint32_t)(step + 1);
            auto t0 = std::chrono::steady_clock::now();
            while ((seen = ctr[t.dep].load(std::memory_order_acquire)) < target) {
              if (status.load() != MK_OK) return;
              if (std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(timeout_ms)) {
                int32_t ok = MK_OK;
                if (status.compare_exchange_strong(ok, MK_ERR_TIMEOUT)) bad_task.store(id);
                return;
              }
              std::this_thread::yield();
            }
          } else if (t.dep >= 0) {
            seen = ctr[t.dep].load(std::memory_order_acquire);
          }
          if (slow_producer[id] && step == 0) std::this_thread::sleep_for(std::chrono::milliseconds(20));
          if (!early) start = ticket.fetch_add(1);
          // the task body is a no-op here
          uint32_t end = ticket.fetch_add(1);
          int64_t slot = nrec.fetch_add(1);
          if (slot < cap) {
            mk_trace_rec& r = recs[slot];
            r.task = id;
            r.worker = (int16_t)a;
            r.xcc = (int16_t)(a % 8);
            r.t_start = start;
            r.t_end = end;
            r.dep_seen = seen;
            r.step = (uint32_t)step;
            r.clk_start = r.clk_end = 0;
          }
          if (t.trig >= 0) {
            if (!(fault == 1 && id == victim)) ctr[t.trig].fetch_add(1, std::memory_order_release);
            if (fault == 2 && id == victim && step == 0) ctr[t.trig].fetch_add(1, std::memory_order_release);
          }
        }
      });
    }
    for (auto& x : th) x.join();
    if (status.load() != MK_OK) {
      *err = "simulated wait timed out at task " + std::to_string(bad_task.load());
      *n = nrec.load();
      return status.load();
    }
  }
  *n = nrec.load();
  if (counters)
    for (int32_t e = 0; e < ne; ++e) counters[e] = ctr[e].load();
  return MK_OK;
}

}  // namespace mk

extern "C" {

const char* mk_last_error(void) { return mk::g_err.c_str(); }

mk_status mk_check_trace(const mk_graph* g, const mk_trace_rec* recs, int64_t n, uint32_t step,
                         const uint32_t* counters) {
  if (!g || !g->G || !recs) {
    mk::set_error("mk_check_trace: null argument");
    return MK_ERR_ARG;
  }
  if (g->G->opts.trace == 2) {
    mk::set_error("mk_check_trace: a timing trace (trace = 2) carries no tickets; build with trace = 1");
    return MK_ERR_ARG;
  }
  std::string err;
  // `step` is the epoch of the traced step; counters are totals after it
  if (!mk::check_trace(*g->G, recs, n, step, counters, step + 1, &err)) {
    mk::set_error(err);
    return MK_ERR_TRACE;
  }
  return MK_OK;
}

mk_status mk_simulate(const mk_graph* g, int32_t threads, int32_t steps, int32_t fault, int32_t timeout_ms,
                      mk_trace_rec* recs, int64_t cap, int64_t* n, uint32_t* counters) {
  if (!g || !g->G) {
    mk::set_error("mk_simulate: null graph");
    return MK_ERR_ARG;
  }
  std::string err;
  int32_t rc = mk::simulate(*g->G, threads, steps, fault, timeout_ms, recs, cap, n, counters, &err);
  if (rc != MK_OK) mk::set_error(err);
  return rc;
}

}  // extern "C"
