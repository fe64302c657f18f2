/*
 * mk.h - C ABI of the persistent decode megakernel for MI355X (gfx950).
 *
 * One call of mk_decode_step runs one autoregressive decode step of a
 * Qwen3-style decoder (dense SwiGLU MLP, or top-k routed experts) for a batch
 * of sequences, either
 *   - PERSISTENT: one launch of a worker kernel with one workgroup resident on
 *     every compute unit plus a one-wavefront dispatch kernel on a second
 *     stream; workers run their statically assigned task lists and wait only on
 *     atomic event counters (MPK page "Mirage Persistent Kernel (MPK)", sections
 *     3.2 and 5.1: one compute kernel launched with one block per worker plus a
 *     dispatch-only scheduler kernel on its own stream), or
 *   - LAUNCH_PER_TASK: the same task bodies, one kernel launch per operator
 *     range in the same order, stream order replacing the events (the
 *     kernel-per-operator baseline of the same pages, section 3.2, and of the
 *     Spheron article "Compile a Megakernel With Mirage", section
 *     "Kernel-Per-Operator Dispatch").
 *
 * The task graph comes from a host compiler (mk_build_graph): every operator
 * is tiled into CU-sized tasks, events are fused and normalised so that each
 * task waits on at most one event and triggers at most one, and the graph is
 * BFS-linearised so that each event's dependents are one contiguous task range
 * (MPK review page 2512.22219, section 2.4; MPK abstract: an SM-level task
 * graph executed with decentralised in-kernel scheduling).
 *
 * Conventions
 *  - Every device pointer is memory the CALLER allocated and owns (PyTorch in
 *    the bundled binding).  The library never allocates or frees device memory;
 *    it owns only the host-side mk_graph and one internal HIP stream.
 *  - bf16 tensors are raw IEEE bfloat16 bit patterns (uint16), row-major
 *    [out, in] as in a linear layer.
 *  - Calls that take a stream enqueue asynchronous work on it; results are
 *    valid after the caller synchronises that stream.  Argument and shape
 *    errors are reported synchronously and nothing is enqueued.
 *  - Every call returns MK_OK (0) or a negative mk_status; mk_last_error()
 *    gives a message for the calling thread's last failure.  No C++ exception
 *    crosses this boundary.
 *  - One mk_graph must not be used from two host threads at once, and steps
 *    of one graph must be issued in order on one stream.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mk_status;
#define MK_OK 0
#define MK_ERR_ARG (-1)          /* bad argument (null pointer, out-of-range value) */
#define MK_ERR_SHAPE (-2)        /* shapes inconsistent or unsupported */
#define MK_ERR_HIP (-3)          /* a HIP runtime call failed */
#define MK_ERR_NOT_RESIDENT (-4) /* workers could not all be co-resident */
#define MK_ERR_TIMEOUT (-5)      /* a device wait exceeded its time budget (watchdog) */
#define MK_ERR_TRACE (-6)        /* the task trace violates the graph */
#define MK_ERR_STATE (-7)        /* call out of order (e.g. decode before load) */

typedef struct mk_graph mk_graph;

/* Model shape.  Dense models set n_experts = 0; routed models set
 * n_experts/top_k/expert_intermediate and leave intermediate = 0.
 * head_dim must be a multiple of 64 and at most 128; n_q_heads must be a
 * multiple of n_kv_heads. */
typedef struct {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, intermediate;
  int32_t n_experts, top_k, expert_intermediate, vocab, tied_embeddings;
  float rms_eps;     /* RMSNorm epsilon (1e-6) */
  double rope_theta; /* RoPE base (1e6) */
} mk_model_shape;

#define MK_PERSISTENT 0
#define MK_LAUNCH_PER_TASK 1

#define MK_GEMV_AUTO 0 /* VALU dot products up to batch 4, MFMA skinny GEMM above */
#define MK_GEMV_VALU 1
#define MK_GEMV_MFMA 2

typedef struct {
  int32_t mode;            /* MK_PERSISTENT or MK_LAUNCH_PER_TASK (mk_set_mode can switch) */
  int32_t per_task_launch; /* launch-per-task only: 1 = one launch per task (stress mode) */
  int32_t num_workers;     /* 0 = the device's compute-unit count */
  int32_t trace;           /* 1 = record one mk_trace_rec per executed task (global tickets, for
                              mk_check_trace); 2 = timing trace: clocks only, record i = task i,
                              no atomics on the task's path (tickets are 0); 0 = off */
  int32_t attn_chunks;     /* attention chunks per (sequence, kv head); 0 = auto */
  int32_t gemv;            /* MK_GEMV_* */
  int32_t spin_timeout_us; /* watchdog budget of any single device wait; 0 = 2 s */
  int32_t no_fusion;       /* 1 = one event per dependency edge (analysis only: normalisation then
                              inserts empty tasks); 0 = fuse events (default) */
  int32_t merge_tasks;     /* how the attention chunks' partials are combined: 0 = merge tasks, each
                              combining one slice of a (sequence, kv head)'s outputs (default);
                              1 = one merge task per (sequence, kv head); 2 = no merge tasks: the
                              last chunk of each (sequence, kv head) to finish merges them */
  int32_t no_watchdog;     /* 1 = persistent mode launches no dispatch wavefront (no residency
                              handshake, no step watchdog; the workers' own bounded waits remain).
                              For profilers that serialise kernel dispatches.  Rejected with
                              MK_ERR_ARG when the graph has dispatcher tasks (routed experts). */
  int32_t prefetch_loads;  /* GEMV weight loads per lane (16 bytes each) issued before a task's
                              dependency wait; 0 = per-operator default */
  int32_t late_trigger;    /* 1 = GEMV tasks trigger their event after storing their outputs;
                              0 = once their last weight loads are issued (consumers re-read
                              words whose step tag is not yet current; default) */
  int32_t lds_ring;        /* 1 = batch-1 GEMV tiles whose rows are whole KB are fed through an LDS
                              ring by four loader wavefronts (LDS-DMA loads) that run ahead into the
                              worker's next tile; 0 = weights stream through registers (default,
                              faster as measured) */
  int32_t xcd_rows_pct;    /* batch <= 4 VALU GEMV tiles of the O, gate-up, down and lm_head operators:
                              rows of a tile whose worker runs on an odd-numbered XCD (worker w runs
                              on XCD w mod 8), in percent of the rows of a tile on an even-numbered
                              XCD (odd XCDs see events later and stream slower); 0 = default,
                              100 = equal tiles, else 50..150 */
  int32_t reserved[2];     /* must be zero */
} mk_build_opts;

/* One logical tensor handed to mk_load_weights.  Names:
 *   embed [V,H], final_norm [H], lm_head [V,H] (absent when tied),
 *   layers.{l}.{in_norm [H], wq [Hq*D,H], wk [Hkv*D,H], wv [Hkv*D,H],
 *               q_norm [D], k_norm [D], wo [H,Hq*D], post_norm [H]}
 *   dense:  layers.{l}.{w_gate [I,H], w_up [I,H], w_down [H,I]}
 *   routed: layers.{l}.router [E,H], layers.{l}.experts.{e}.{w_gate,w_up [Ie,H], w_down [H,Ie]}
 * Vectors use cols = 1.  data is bf16; on_device = 1 if data is device memory. */
typedef struct {
  const char* name;
  const void* data;
  int64_t rows, cols;
  int32_t on_device;
} mk_tensor;

/* The caller's bf16 KV cache (device memory), in one of two layouts:
 *  - contiguous (page_size = 0): k and v each [L][B][Hkv][capacity][D];
 *  - paged (page_size > 0), the layout of paged attention that a serving
 *    pipeline keeps inside the megakernel (review page of arXiv 2512.22219,
 *    adoption paragraph: continuous batching and paged attention run inside
 *    the mega-kernel): k and v are pools [L][n_pages][Hkv][page_size][D];
 *    page_table [B][capacity / page_size] (device int32) gives the physical
 *    page of every logical page of a sequence, so position t of sequence b
 *    is row t % page_size of page page_table[b][t / page_size].  page_size is
 *    a power of two, at least 16, dividing capacity; one layer's pool must
 *    stay below 4 GiB.  A page number outside 0..n_pages-1 met by a step is
 *    reported by mk_check (MK_ERR_ARG); nothing is written through it.
 * positions[b] of a step is the slot that step writes; attention covers slots
 * 0..positions[b] of sequence b.  capacity must equal the graph's max_ctx.
 * The library reads the struct at each call (mk_capture_lpt_graph: once). */
typedef struct {
  void* k;
  void* v;
  int32_t capacity;
  int32_t page_size;          /* 0 = contiguous */
  const int32_t* page_table;  /* paged: [B][capacity / page_size], device memory */
  int32_t n_pages;            /* paged: pages in each of the k and v pools */
  int32_t reserved;           /* must be zero */
} mk_kv_cache;

/* One record per executed task (trace mode).  Tickets (trace = 1) come from
 * one global atomic counter: start is taken after the task's dependency wait
 * succeeded, end is taken before its trigger.  In the timing trace (trace =
 * 2) the two ticket fields hold clocks instead: t_start the clock at task
 * entry (its worker done with the previous task), t_end the clock when the
 * dependency wait began (the pre-wait weight loads issued). */
typedef struct {
  int32_t task;     /* task id (BFS order) */
  int16_t worker;   /* worker (workgroup) index; -1 in launch-per-task mode */
  int16_t xcc;      /* hardware XCC (chiplet) id the task ran on */
  uint32_t t_start; /* global ticket at start (timing trace: clock at task entry) */
  uint32_t t_end;   /* global ticket at end, before the trigger (timing trace: clock when the wait began) */
  uint32_t dep_seen;/* dependency counter value observed when the wait ended */
  uint32_t step;    /* step epoch */
  uint32_t clk_start, clk_end; /* low 32 bits of the 100 MHz device wall clock */
} mk_trace_rec;

typedef struct {
  int64_t tasks;             /* tasks per step, including empty ones */
  int64_t empty_tasks;       /* tasks inserted by normalisation */
  int64_t events;            /* events after fusion and normalisation */
  int64_t ops;               /* operator instances */
  int64_t workers;
  int64_t launches_per_step; /* launch-per-task mode, range granularity */
  int64_t raw_edges;         /* task dependency edges before reduction */
  int64_t reduced_edges;     /* after transitive reduction */
  int64_t max_tasks_per_worker;
  int64_t weight_bytes;      /* weight bytes one step streams (dense) */
  int64_t arena_bytes, scratch_bytes, trace_bytes;
  int32_t batch, max_ctx, attn_chunks, gemv;
  int32_t ring_kb;           /* KB per LDS-ring segment of batch-1 GEMV tiles, 0 = no ring tiles */
  int32_t ring_ops;          /* operator instances whose tiles are fed through the LDS ring */
} mk_stats;

/* Compile the task graph for a model shape, batch and KV capacity (host only;
 * no device work): tiling, event fusion, normalisation to at most one
 * dependency and one trigger event per task, BFS linearisation, assignment to
 * workers (review page of arXiv 2512.22219, section 2.4; the compile half of
 * the survey page's compile-and-run pipeline, section 3.1).  *out receives a
 * new graph, freed by mk_destroy_graph.  Errors: MK_ERR_ARG, MK_ERR_SHAPE. */
mk_status mk_build_graph(const mk_model_shape* shape, int32_t batch, int32_t max_ctx, const mk_build_opts* opts,
                         mk_graph** out);

/* Bytes of caller-allocated device memory the graph needs:
 *   arena   - packed weights and the read-only task tables (256 B aligned)
 *   scratch - event counters, status words and inter-task activations
 *   trace   - trace records (0 unless opts.trace)
 * The pages' runtime keeps the task graph and the tensors between tasks in
 * device memory for the one resident kernel (survey page on MPK, section 3:
 * a runtime that launches and drives the compiled megakernel); here the
 * caller allocates that memory.  Pure query: no device work.
 * Errors: MK_ERR_ARG (null argument). */
mk_status mk_workspace_size(const mk_graph* g, size_t* arena_bytes, size_t* scratch_bytes, size_t* trace_bytes);

/* Repack the logical tensors into the arena in per-task order, upload the
 * task tables, and clear the scratch.  Asynchronous on `stream` (a
 * hipStream_t; NULL = default stream); host tensors are staged synchronously.
 * Every tensor of the shape must be present exactly once.  This is the step
 * before the timed decode in the pages' demo, where the model is built and
 * its weights placed once and the decode is then a single call (survey page
 * on MPK, section 5.3).  The tensors stay owned by the caller and may be freed
 * after the stream is synchronised.
 * Errors: MK_ERR_ARG (missing/duplicate/misshapen tensor), MK_ERR_HIP. */
mk_status mk_load_weights(mk_graph* g, const mk_tensor* tensors, int32_t n, void* d_arena, void* d_scratch,
                          void* d_trace, void* stream);

/* Run one decode step: tokens d_tokens[B] (int32) at positions d_positions[B]
 * (int32, 0 <= pos < capacity), reading/writing the KV cache, and writing
 * fp32 logits d_logits[B][V].  Asynchronous on `stream`.  In persistent mode
 * this is the single launch per step of the pages' megakernel timeline (survey
 * page on MPK, section 3.2: one launch, one resident kernel, a dispatch-only
 * scheduler beside it); in launch-per-task mode it is that section's baseline
 * of one launch per operator range.
 * Errors: MK_ERR_STATE (weights not loaded, or a previous step failed and was
 * not cleared by mk_check), MK_ERR_ARG, MK_ERR_HIP, MK_ERR_NOT_RESIDENT. */
mk_status mk_decode_step(mk_graph* g, const int32_t* d_tokens, const int32_t* d_positions, const mk_kv_cache* kv,
                         float* d_logits, void* stream);

/* Greedy decode of n_steps steps in ONE persistent launch: the whole decode
 * loop inside the megakernel, as the MPK pages' single mpk() call runs the
 * generation (survey page on MPK, section 5, the demo's decode loop).
 * Step 0 embeds d_tokens[B] at d_positions[B]; step s > 0 embeds the greedy
 * token of step s-1 (argmax of its fp32 logits, ties to the lower id) at
 * d_positions[b] + s.  The argmax is reduced on the device from per-tile
 * candidates of the lm_head; the next step's embedding waits for the previous
 * step's lm_head event.  d_tokens_out[n_steps][B] (int32, device, nullable
 * when n_steps == 1) receives every step's greedy token; d_logits[B][V] holds
 * the last step's logits.  Caller-owned buffers; d_tokens and d_positions are
 * not modified.  Needs 0 <= d_positions[b] + n_steps - 1 < capacity (else the
 * attention bounds check clamps the position and mk_check then reports
 * MK_ERR_ARG, position out of range), the persistent mode, and a graph built
 * without trace when n_steps > 1.
 * Errors: as mk_decode_step; MK_ERR_ARG for n_steps outside 1..4096, for
 * token output or n_steps > 1 in launch-per-task mode, or for n_steps > 1
 * with a trace. */
mk_status mk_decode_steps(mk_graph* g, const int32_t* d_tokens, const int32_t* d_positions, const mk_kv_cache* kv,
                          float* d_logits, int32_t* d_tokens_out, int32_t n_steps, void* stream);

/* mk_decode_step for callers that cannot allocate device memory around a
 * step (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same step, run on a scratch area the library holds
 * in a static device array of 64 MiB, one per GPU, kept until the process
 * ends, instead of the scratch given to mk_load_weights.  It calls no
 * allocating routine.  Graphs whose scratch (mk_workspace_size) exceeds 64 MiB
 * are rejected with MK_ERR_ARG; the batch-1 decoders up to the 8B shape fit.
 * Every call clears the event state it needs (a fill kernel on `stream`) and
 * takes a data tag no earlier call on the device used, so calls may follow
 * each other with different graphs; calls that overlap on one GPU (other
 * streams, other threads) race on the shared array.  Afterwards mk_check,
 * mk_read_trace, mk_read_counters and mk_read_routing read this call's state.
 * The graph's own scratch and its step count are left as they were.
 * Errors: as mk_decode_step. */
mk_status mk_decode_step_noalloc(mk_graph* g, const int32_t* d_tokens, const int32_t* d_positions,
                                 const mk_kv_cache* kv, float* d_logits, void* stream);

/* Launch-per-task mode captured once into a HIP graph and replayed: the same
 * task bodies and launch sequence as mode MK_LAUNCH_PER_TASK, without the
 * host's per-launch cost.  This is the pages' CUDA-Graphs comparison point for
 * the megakernel (MPK blog, the overhead of kernel launches that graphs do
 * not remove; survey page on MPK, section 5).
 *   mk_capture_lpt_graph: records one step's launches (the graph's
 *     per_task_launch setting) with the given device buffers baked in; the
 *     caller rewrites d_tokens / d_positions between replays.  Needs a graph
 *     built without trace (its trace clears counters with a memset).
 *     *out receives the handle, owned by the caller.
 *   mk_lpt_graph_launch: one step, asynchronous on `stream`.  Replays use a
 *     data tag reserved for them, and count as steps for the graph's event
 *     epochs, so persistent steps may follow.
 *   mk_lpt_graph_destroy: frees the handle; the mk_graph must outlive it.
 * Errors: MK_ERR_STATE (not loaded), MK_ERR_ARG (bad argument, trace on),
 * MK_ERR_HIP. */
typedef struct mk_lpt_graph mk_lpt_graph;
mk_status mk_capture_lpt_graph(mk_graph* g, const int32_t* d_tokens, const int32_t* d_positions,
                               const mk_kv_cache* kv, float* d_logits, mk_lpt_graph** out);
mk_status mk_lpt_graph_launch(mk_lpt_graph* lg, void* stream);
void mk_lpt_graph_destroy(mk_lpt_graph* lg);

/* Switch the execution mode of a loaded graph (same tables and arena):
 * MK_PERSISTENT or MK_LAUNCH_PER_TASK (per_task_launch = 1: one launch per
 * task), the two timelines of the survey page on MPK, section 3.2.
 * Errors: MK_ERR_ARG (null graph, unknown mode). */
mk_status mk_set_mode(mk_graph* g, int32_t mode, int32_t per_task_launch);

/* After the caller synchronised the stream: read the device status word.
 * MK_OK, MK_ERR_ARG (a position outside the cache or a page-table entry
 * outside the pool was clamped and reported), or MK_ERR_TIMEOUT (watchdog
 * fired; the task, event and counter values are in the message), after which
 * the event state is reset so that the next step can run.  The pages' runtime
 * has no such check (a stuck event there hangs the kernel); the bounded waits
 * behind it are this design's addition. */
mk_status mk_check(mk_graph* g);

/* After sync: copy the trace of the last step (up to cap records) to host
 * memory; *n receives the number of records written by the device.  The
 * counterpart of the pages' profiling trace (survey page on MPK, section 7.2:
 * the profiling flag writes a per-task timeline).  Errors: MK_ERR_ARG,
 * MK_ERR_STATE (graph built without trace). */
mk_status mk_read_trace(mk_graph* g, mk_trace_rec* host_buf, int64_t cap, int64_t* n);

/* After sync: verify a trace against the graph: every task exactly once, no
 * task started before all triggers of its dependency event ended, observed
 * counters at or above their targets, and (if counters != NULL, from
 * mk_read_counters) every event counter equal to need * steps.
 * MK_OK or MK_ERR_TRACE (first violation in the message). */
mk_status mk_check_trace(const mk_graph* g, const mk_trace_rec* recs, int64_t n, uint32_t step,
                         const uint32_t* counters);

/* After sync: the expert choice of step `step` (0-based, within the last
 * launch; one of its last 64 steps) of a routed-expert graph, as recorded by
 * the routing task: experts[L][B][top_k] (int32) and their weights (float,
 * softmax over all experts renormalised over the chosen ones), in the order
 * chosen.  router_logits (nullable; only for the last step of the launch)
 * receives the router logits [L][B][n_experts] the choice was made from.
 * This is the just-in-time, data-dependent part of the step (review page of
 * arXiv 2512.22219, attack 3: routing needs its own balancing), exposed so
 * that a caller can check a choice made in fp32 near a tie.  cap: elements
 * of each buffer.  Errors: MK_ERR_STATE (no routed experts), MK_ERR_ARG. */
mk_status mk_read_routing(mk_graph* g, int32_t step, int32_t* experts, float* weights, float* router_logits,
                          int64_t cap);

/* After sync: host copy of the per-event counter totals (events entries),
 * the counters of the event protocol (review page of arXiv 2512.22219, section
 * 2.4: a task waits on one event counter and increments one).  With
 * mk_check_trace, every counter must equal need x steps.  Errors: MK_ERR_ARG. */
mk_status mk_read_counters(mk_graph* g, uint32_t* host_counters, int64_t cap);

/* Execute the graph's protocol on the host with `threads` threads standing in
 * for the workers and no-op task bodies, writing a trace (recs, cap >= tasks)
 * for mk_check_trace (the event protocol of the review page of arXiv
 * 2512.22219, section 2.4, run without a GPU).  `fault` plants a protocol fault for checker tests:
 * 0 none, 1 drop one trigger (expect MK_ERR_TIMEOUT), 2 duplicate one trigger,
 * 3 start one task without waiting.  Host only, no device. */
mk_status mk_simulate(const mk_graph* g, int32_t threads, int32_t steps, int32_t fault, int32_t timeout_ms,
                      mk_trace_rec* recs, int64_t cap, int64_t* n, uint32_t* counters);

/* Task, event, empty-task and per-worker counts and the workspace sizes of a
 * compiled graph (the "deep, not wide" shape the review page of arXiv
 * 2512.22219 discusses in its attack notes).  Errors: MK_ERR_ARG. */
mk_status mk_graph_stats(const mk_graph* g, mk_stats* out);

/* Write the graph (tasks, events, worker lists) as JSON, the counterpart of
 * the task-graph file the pages' profiling run writes (survey page on MPK,
 * section 7.2).  Host only.  Errors: MK_ERR_ARG (null graph or path). */
mk_status mk_dump_graph(const mk_graph* g, const char* json_path);

/* Host copies of the graph tables for inspection and tests.
 * task rows: {op_kind, layer, dep_event, trig_event, a0, a1, a2, a3} (int32 x 8)
 * event rows: {need, first, last, producers} (int32 x 4)
 * worker lists: CSR (offsets[workers+1], ids[tasks]) */
mk_status mk_get_tasks(const mk_graph* g, int32_t* rows, int64_t cap);
mk_status mk_get_events(const mk_graph* g, int32_t* rows, int64_t cap);
mk_status mk_get_worker_lists(const mk_graph* g, int32_t* offsets, int32_t* ids, int64_t cap);

/* Raw dependency edges (producer, consumer) the compiler derived from the
 * tasks' read/write footprints before any reduction (brute-force check of
 * edge preservation).  *n receives the count; pass rows = NULL to query. */
mk_status mk_get_raw_edges(const mk_graph* g, int32_t* rows, int64_t cap, int64_t* n);

/* Free a graph and its internal stream (the caller's device memory is not
 * touched).  NULL is accepted. */
void mk_destroy_graph(mk_graph* g);
/* Message of the calling thread's last failed call ("" if none); valid until
 * that thread's next call. */
const char* mk_last_error(void);

/* Measurement helper: read `bytes` bytes of device memory once (16-byte
 * loads, `blocks` workgroups of 512 threads, grid-stride), leaving one word
 * per workgroup in d_sink[blocks].  The streaming-read rate of the box, timed
 * by the caller, is the practical ceiling the weight roofline is reported
 * against (survey page on MPK, section 9.3: the step is bounded by the
 * weight-read roofline).  d_buf 16-byte aligned, bytes a multiple of 16.
 * Errors: MK_ERR_ARG, MK_ERR_HIP. */
mk_status mk_stream_read(const void* d_buf, uint64_t bytes, uint32_t* d_sink, int32_t blocks, void* stream);

/* Path of the loaded HIP runtime library (diagnostic: it must be the same one
 * the caller's framework uses). */
const char* mk_hip_runtime_path(void);

#ifdef __cplusplus
}
#endif

#endif /* MK_H */
