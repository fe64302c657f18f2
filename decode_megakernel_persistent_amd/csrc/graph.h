// graph.h - host-side task-graph compiler (no HIP dependency).
#pragma once
#include <cstdint>
#include <string>
#include <vector>

#include "mk.h"
#include "tables.h"

namespace mk {

// A read or write footprint: words [begin, end) of buffer `buf`.
struct Footprint {
  int32_t buf;
  int64_t begin, end;
  bool write;
};

// Host view of one operator instance.
struct OpInst {
  int32_t kind = OP_EMPTY, layer = -1;
  int32_t K = 0, N = 0, norm_in = 0;
  int32_t first_raw = 0, ntasks = 0;  // raw task range
  bool joint = false;                 // tasks jointly write the op's outputs (work-list slots)
  int64_t w_off = -1;                 // arena byte offset of the weight block
  int64_t g_off = -1, g2_off = -1;    // arena byte offsets of fp32 gains
  int32_t in_buf = -1, res_buf = -1, out_buf = -1, aux_buf = -1, aux2_buf = -1;
  bool ring = false;                  // batch-1 GEMV tiles fed through the LDS weight ring
};

// Activation buffer in scratch (tagged 64-bit words), or a virtual buffer
// (logits, KV slots) that exists only for dependency analysis.
struct Buffer {
  std::string name;
  int64_t words = 0;
  int64_t off = -1;  // scratch byte offset; -1 = virtual
};

// How one piece of a logical tensor lands in the arena.
struct CopyJob {
  enum Kind : int32_t { ROWS = 0, SWZ16 = 1, GAIN_F32 = 2 };
  std::string tensor;
  int64_t row0 = 0, nrows = 0, cols = 0;
  int64_t dst = 0;  // arena byte offset
  int32_t kind = ROWS;
};

struct RawTask {
  int32_t op;
  int32_t a[5];
  std::vector<Footprint> fp;
};

struct Graph {
  mk_model_shape shape{};
  int32_t B = 0, cap = 0;
  mk_build_opts opts{};
  int32_t W = 0;        // workers
  int32_t C = 0;        // attention chunks per (sequence, kv head)
  int32_t merge_slices = 1;  // merge tasks per (sequence, kv head)
  int32_t gemv = 0;     // MK_GEMV_VALU or MK_GEMV_MFMA
  int32_t granule = 1;  // GEMV tile row granule
  bool fuse = true;     // event fusion (off only for compiler tests)
  Geom geom{};

  std::vector<OpInst> ops;
  std::vector<Buffer> bufs;
  std::vector<RawTask> raw;
  std::vector<Task> tasks;    // linearised
  std::vector<Event> events;
  std::vector<int32_t> raw_to_id;           // raw index -> task id
  std::vector<int32_t> wl_off, wl_ids;      // worker lists (W workers + the dispatcher at index W)
  std::vector<int32_t> launch_first, launch_count;  // launch-per-task ranges (BFS order)
  std::vector<std::pair<int32_t, int32_t>> raw_edges;  // (producer, consumer) task ids
  int64_t n_empty = 0, n_reduced_edges = 0;
  int32_t lm_event = -1, lm_tiles = 0;  // terminal event of the lm_head tiles, and their count

  // layout
  std::vector<CopyJob> copies;
  int64_t arena_bytes = 0, scratch_bytes = 0, trace_bytes = 0;
  int64_t off_geom = 0, off_ops = 0, off_tasks = 0, off_events = 0, off_wloff = 0, off_wlids = 0, off_invfreq = 0;
  int64_t off_ops_static = 0;  // the operator table again, its buffers in the library's static scratch
  int64_t off_counters = 0, off_status = 0, off_progress = 0, off_arrive = 0, off_state_end = 0, off_cand = 0;
  int64_t off_route_hist = -1;  // routed experts: expert choice history (kRouteHistSteps steps), else -1
  int64_t weight_bytes_step = 0;
};

// Compile a decoder step graph.  Returns nullptr and sets *err on failure.
Graph* compile_decoder(const mk_model_shape& s, int32_t batch, int32_t cap, const mk_build_opts& o, int32_t workers,
                       bool fuse, std::string* err);

// Shared back end, also used for arbitrary DAGs in tests: given raw tasks with
// footprints (or explicit edges), derive edges, reduce, fuse, normalise,
// linearise and assign.
bool finish_graph(Graph& g, std::string* err);

// Check the structural invariants: <=1 dep/trig event per task, contiguous
// event ranges, topological ids, need == number of triggering tasks.
bool validate_graph(const Graph& g, std::string* err);

uint32_t graph_magic(const Graph& g);

void dump_json(const Graph& g, const std::string& path);

const char* op_kind_name(int32_t k);

// Thread-local message behind mk_last_error().
void set_error(const std::string& msg);

// Verify a trace against the graph (the checks of mk_check_trace).
bool check_trace(const Graph& g, const mk_trace_rec* recs, int64_t n, uint32_t step, const uint32_t* counters,
                 uint32_t steps_done, std::string* err);

// Run the protocol on host threads (see mk_simulate).  Returns MK_OK or an error status.
int32_t simulate(const Graph& g, int32_t threads, int32_t steps, int32_t fault, int32_t timeout_ms, mk_trace_rec* recs,
                 int64_t cap, int64_t* n, uint32_t* counters, std::string* err);

}  // namespace mk

// The handle behind the C ABI.  Device-side members are opaque here so that
// host-only code (compiler, simulator, checker) builds without HIP.
struct mk_graph {
  mk::Graph* G = nullptr;
  void* arena = nullptr;
  void* scratch = nullptr;
  void* trace = nullptr;
  void* side_stream = nullptr;
  void* ev_a = nullptr;
  void* ev_b = nullptr;
  int32_t mode = 0, per_task_launch = 0, device = -1;
  bool loaded = false;
  uint32_t epoch = 0;  // steps whose events counted since the last reset
  uint32_t persistent_steps = 0;  // of those, steps run by persistent launches (worker arrival/done counts)
  uint32_t tag = 1;    // data tag of the next step
  uint64_t budget_ticks = 0;
  int32_t last_steps = 0;   // steps of the last launch (mk_read_routing)
  uint32_t last_tag0 = 0;   // data tag of that launch's first step
  void* static_scr = nullptr;  // the library's static scratch on this graph's device, when the graph fits it
  bool last_static = false;    // the last step ran on the static scratch (mk_decode_step_noalloc)
};
