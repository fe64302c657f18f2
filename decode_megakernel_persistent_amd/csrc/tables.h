// tables.h - the task-graph tables the host compiler produces and the device
// runtime consumes.  Plain structs only (no HIP types), so the host compiler,
// the CPU protocol simulator and the HIP kernels all read the same layout.
#pragma once
#include <stdint.h>

namespace mk {

// Kinds of operator instance.  One decode step of the decoder is EMBED, then
// per layer QKV -> ATTN -> MERGE -> OPROJ -> (GATEUP -> DOWN | ROUTER -> ROUTE
// -> MOE_GU -> MOE_DOWN -> COMBINE), then LMHEAD.
enum OpKind : int32_t {
  OP_EMPTY = 0,   // inserted by normalisation: waits, then triggers
  OP_EMBED = 1,   // x0[b] = embed[token_b]
  OP_QKV = 2,     // rmsnorm(x) then the q/k/v rows of one head group
  OP_ATTN = 3,    // q/k-norm + RoPE (+ KV append) + attention over one chunk of positions
  OP_MERGE = 4,   // combine the chunk partials of one (sequence, kv head)
  OP_OPROJ = 5,   // x += Wo . attn
  OP_GATEUP = 6,  // a = silu(Wg h) * (Wu h), h = rmsnorm(x)
  OP_DOWN = 7,    // x += Wd . a
  OP_LMHEAD = 8,  // logits = Wlm . rmsnorm(x)
  OP_ROUTER = 9,  // router logits = Wr . rmsnorm(x)
  OP_ROUTE = 10,  // softmax, top-k, work list (run by the dispatch wavefront)
  OP_MOE_GU = 11, // expert gate/up tiles pulled from the work list
  OP_MOE_DOWN = 12,
  OP_COMBINE = 13,// x += sum_k w_k y_k
  OP_KINDS = 14
};

// One task: 32 bytes.  `op` indexes the operator table; dep/trig are event
// indices or -1; a0..a4 are per-kind tile arguments:
//   EMBED  a0 = sequence b
//   GEMV   a0 = tile, a1 = first output row, a2 = rows, a3 = weight element
//          offset of the tile inside the op's weight block
//   ATTN   a0 = b, a1 = kv head g, a2 = chunk
//   MERGE  a0 = b, a1 = g
//   MOE_*  a0 = slot
//   COMBINE a0 = tile, a1 = first row, a2 = rows
struct Task {
  int32_t op;
  int32_t dep;
  int32_t trig;
  int32_t a0, a1, a2, a3, a4;
};

// One event: counter target per step is `need`; its dependents are tasks
// first..last (inclusive), or first = last + 1 (= 0, -1) when it has none.
struct Event {
  int32_t need;
  int32_t first;
  int32_t last;
  int32_t producers;
};

// Operator instance as the device sees it.  Offsets are resolved to device
// pointers when the weights are loaded.
struct OpDesc {
  int32_t kind, layer;
  int32_t K;         // GEMV input length per sequence
  int32_t N;         // GEMV output length per sequence
  int32_t norm_in;   // 1: input is rmsnorm(in) * g
  int32_t ntasks;
  int32_t pre;       // GEMV: weight loads per lane issued before the dependency wait
  int32_t pad;       // bit 0: control wavefront issues no pre-wait loads; bit 1: early trigger;
                     // bit 2: batch-1 tile fed through the LDS weight ring
  const uint16_t* w; // weight block (bf16)
  const float* g;    // input-norm gain [K] (or q-norm gain [D])
  const float* g2;   // k-norm gain [D]
  uint64_t* in;      // tagged input activations [B][K]
  uint64_t* res;     // tagged residual input [B][N]
  uint64_t* out;     // tagged output [B][N]
  uint64_t* aux;     // attention partials / routing tables
  uint64_t* aux2;
};

// Per-graph geometry, uploaded once.
struct Geom {
  int32_t B, H, Hq, Hkv, D, G, I, V, L, C, cap;
  int32_t E, topk, Ie;
  int32_t qkv_stride;   // per-sequence row length of the qkv buffer = Hkv*(G+2)*D
  int32_t part_stride;  // floats of one head partial = D + 2
  int32_t n_events, n_tasks, n_workers, n_ops;
  float eps;
  float attn_scale;     // 1/sqrt(D)
  uint32_t magic;       // configuration hash checked by every worker at entry
  int32_t mfma;         // 1: GEMV tiles use the MFMA path (swizzled weight fragments)
  int32_t lm_event;     // terminal event of the lm_head tiles (-1: none)
  int32_t lm_tiles;     // lm_head tiles (producers of lm_event)
  int32_t ring_u;       // KB per LDS-ring segment of batch-1 GEMV tiles (4, 2 or 1), 0 = no ring tiles
  const double* inv_freq;  // RoPE inverse frequencies [D/2]
};

// Scratch layout: event counters first, 8 sub-counters per event, each on its
// own 128-byte line; then the status block; then activations.
constexpr int kSubCounters = 8;
constexpr int kCounterStride = 32;  // uint32 per 128 B line
constexpr int kEventBytes = kSubCounters * kCounterStride * 4;

enum StatusWord : int32_t {
  ST_ERROR = 0,     // first error code (ErrCode)
  ST_TASK = 1,
  ST_EVENT = 2,
  ST_SEEN = 3,
  ST_TARGET = 4,
  ST_ABORT = 5,     // nonzero: every wait gives up
  ST_DONE = 6,      // workers finished (cumulative over steps)
  ST_TICKET = 7,    // trace ticket (cumulative)
  ST_TRACE_N = 8,   // trace records of the current step
  ST_DISPATCH = 9,  // dispatcher progress (cumulative events seen)
  ST_MIN_TASK = 10, // smallest task id whose wait timed out (0xFFFFFFFF = none)
  ST_ADDR_LO = 11,  // address of a tagged word that never became current
  ST_ADDR_HI = 12,
  ST_ARRIVED = 13,  // worker workgroups that started (cumulative over steps)
  ST_WORDS = 64
};

// LDS budget of one worker (bytes) and the areas the task bodies use.
constexpr int kLdsBytes = 156 * 1024;  // dynamic LDS per worker (gfx950: 160 KB per CU)
constexpr int kStageFloats = 24576;      // GEMV input staging (96 KB)
constexpr int kRowResultFloats = 8192;   // GEMV per-row results (32 KB)
constexpr int kScoreFloats = 8192;       // attention scores of one chunk (32 KB)
// Batch-1 GEMV tiles fed through the LDS weight ring: limits of one tile
// (input length, segments, rows) that the ring's LDS areas hold.
constexpr int kRingMaxK = 12288;
constexpr int kRingMaxSegs = 2048;
constexpr int kRingMaxRows = 1024;

enum ErrCode : uint32_t { ERR_NONE = 0, ERR_TIMEOUT = 1, ERR_CONFIG = 2, ERR_BAD_TASK = 3, ERR_BAD_INPUT = 4, ERR_NOT_RESIDENT = 5 };

// Register hint of the worker kernel.  amdgpu_num_vgpr counts the unified
// VGPR + AGPR file on this architecture, so it does not bind the 256
// architectural registers; what must hold is that two worker wavefronts and
// the dispatch wavefront (about 64 registers: it also routes MoE tokens) fit
// a SIMD's 512, which mk_load_weights checks on the built kernels.
constexpr int kWorkerVgprs = 248;
// The batch-1 variant is held to 216 (its SGPR spill lanes come on top; at
// 232 it would leave the dispatch wavefront less than its 64 registers).
constexpr int kWorkerVgprsB1 = 216;

// Decode steps one persistent launch may run (mk_decode_steps).
constexpr int kMaxStepsPerLaunch = 4096;

// Data tag of captured launch-per-task graphs (never used by other steps).
constexpr uint32_t kGraphTag = 0xFFFFFFFFu;

// Routed-expert graphs keep the expert choice of the last kRouteHistSteps
// steps of a launch (slot = step index within the launch mod this), as
// {int32 expert, float weight} pairs [slot][layer][sequence][top_k], for
// mk_read_routing.
constexpr int kRouteHistSteps = 64;  // a power of two

}  // namespace mk
