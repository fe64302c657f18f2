// device.h - CDNA4 (gfx950) device side: event protocol, tagged activations
// and the task bodies.  Included by runtime.hip only.
//
// Coherence on MI355X: the eight XCD L2 caches are not coherent with each
// other, and whole-L2 write-back/invalidate at every release/acquire costs tens
// of microseconds per event hop.  So no task publishes data through release/
// acquire fences.  Instead every inter-task activation is a 64-bit word
// (fp32 value, 32-bit step tag) written with an agent-scope relaxed atomic
// store; a reader accepts a word only when its tag is the current step's and
// otherwise re-reads it with agent-scope loads.  A single 64-bit atomic word
// cannot be torn, so value and tag always travel together, and the event
// counters (relaxed agent-scope atomics, eight sub-counters per event on
// separate 128-byte lines) only tell a task when its inputs are ready to read.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk.h"
#include "tables.h"

namespace mk {

#define DEV __device__ __forceinline__

typedef uint32_t u32;
typedef uint64_t u64;
typedef u32 u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef u32 u32x2 __attribute__((ext_vector_type(2)));

constexpr int NT = 512;       // threads per worker workgroup (8 wavefronts)
constexpr int NWAVE = NT / 64;
constexpr int kRingVariant = 17;  // kernel template value of the batch-1 LDS-ring variant
constexpr u32 OOB = 0x80000000u;  // buffer offset beyond every tile: the load returns zeros
constexpr int AUX_NT = 2;         // non-temporal hint for streamed weights

// Arguments of one step, identical for every launch of the step.
struct StepArgs {
  const Geom* geom;
  const OpDesc* ops;
  const Task* tasks;
  const Event* events;
  const int32_t* wl_off;
  const int32_t* wl_ids;
  u32* counters;
  u32* status;
  u32* progress;   // per agent: 1 + id of the current task, 0xFFFFFFFF when done
  const int32_t* tokens;
  const int32_t* positions;
  uint16_t* kv_k;     // contiguous [L][B][Hkv][cap][D], or paged pools [L][n_pages][Hkv][page][D]
  uint16_t* kv_v;
  const int32_t* page_table;  // paged: physical page of each logical page, [B][cap >> page_shift]
  int32_t page_shift;         // log2(page size), or -1 for the contiguous layout
  int32_t n_pages;            // paged: pages per pool
  float* logits;
  mk_trace_rec* trace;
  u64 budget;       // wall-clock ticks any single wait may take
  u32 epoch;        // counted steps since the last reset: targets are need * (epoch + 1)
  u32 tag;          // data tag of this step (never 0)
  u32 magic;
  int32_t trace_on;
  int32_t lpt_first;  // launch-per-task: first task id of the launch
  int32_t n_workers;
  int32_t n_steps;    // decode steps of this launch (persistent mode); epoch and tag advance by one per step
  u32 run_base;       // persistent steps before this launch: workers count one arrival / completion per step
  int32_t step;       // this step's index within the launch
  int32_t* tokens_out;  // [n_steps][B] greedy tokens, or null
  u64* cand;          // lm_head tile candidates [tile][B] x (value, id), tagged
  u64* route_hist;    // routed experts: {expert, weight} [kRouteHistSteps][L][B][top_k], or null
};

// Thread index behind an empty asm: index math derived from it stays inside
// the task body instead of being hoisted out of the worker's task loop, where
// it would hold registers through every other body.
DEV int task_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// ---------------------------------------------------------------- scalars
DEV float bf_lo(u32 v) { return __uint_as_float(v << 16); }
DEV float bf_hi(u32 v) { return __uint_as_float(v & 0xffff0000u); }
DEV float bf2f(uint16_t b) { return __uint_as_float((u32)b << 16); }
DEV uint16_t f2bf(float f) {
  u32 x = __float_as_uint(f);
  if ((x & 0x7f800000u) == 0x7f800000u) return (uint16_t)((x >> 16) | ((x & 0xffffu) ? 0x40u : 0u));
  x += 0x7fffu + ((x >> 16) & 1u);
  return (uint16_t)(x >> 16);
}
DEV float silu(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------- global pointers
// Table entries hold generic pointers; casting them to the global address
// space makes the compiler emit global_* instead of flat_* memory operations
// (flat operations also occupy the LDS/scalar wait counter).
typedef __attribute__((address_space(1))) u64 g_u64;
typedef __attribute__((address_space(1))) u32 g_u32;
DEV g_u64* gp(u64* p) { return (g_u64*)p; }
DEV const g_u64* gp(const u64* p) { return (const g_u64*)p; }
DEV g_u32* gp(u32* p) { return (g_u32*)p; }
typedef __attribute__((address_space(1))) const float g_cf32;
DEV float ldg(const float* p) { return *(g_cf32*)p; }

// Buffer resource over [p, p + bytes).  Every resource here is built from
// per-task values, the same in every lane; readfirstlane states that to the
// compiler, which otherwise may keep the descriptor in vector registers and
// wrap each buffer load in a loop over distinct descriptor values.
DEV __amdgpu_buffer_rsrc_t rsrc_u(const void* p, u32 bytes) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const u32 lo = (u32)__builtin_amdgcn_readfirstlane((int)(u32)v);
  const u32 hi = (u32)__builtin_amdgcn_readfirstlane((int)(u32)(v >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)(((uint64_t)hi << 32) | lo), (short)0, n, 0x00020000);
}

// ---------------------------------------------------------------- tagged words
DEV u64 pack(float v, u32 tag) { return ((u64)tag << 32) | (u64)__float_as_uint(v); }
DEV void st_t(u64* p, float v, u32 tag) {
  __hip_atomic_store(gp(p), pack(v, tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Slow path of a tagged read: re-read at agent scope until the word carries
// this step's tag (agent-scope loads observe other XCDs' agent-scope stores).
__device__ __noinline__ u64 ld_t_slow(const u64* p, u32 tag, u64 budget, u32* status) {
  const u64 t0 = wall_clock64();
  for (int i = 0;; ++i) {
    u64 w = __hip_atomic_load(gp(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((u32)(w >> 32) == tag) return w;
    if ((i & 7) == 7) {
      if (__hip_atomic_load(status + ST_ABORT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ||
          wall_clock64() - t0 > budget) {
        u32 z = 0;
        if (__hip_atomic_compare_exchange_strong(status + ST_ERROR, &z, (u32)ERR_TIMEOUT, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
          __hip_atomic_store(status + ST_TASK, 0xFFFFFFFFu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(status + ST_SEEN, (u32)(w >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(status + ST_TARGET, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __hip_atomic_store(status + ST_ADDR_LO, (u32)(uintptr_t)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(status + ST_ADDR_HI, (u32)((uintptr_t)p >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(status + ST_ABORT, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return pack(0.0f, tag);
      }
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// Fast path: a workgroup-scope relaxed load (a plain cached load: one fetch
// per XCD, shared through its L2); fall back when the tag is stale.  Callers
// that read several words issue every ld_raw first and check the tags after,
// so a batch costs one memory round trip.
DEV u64 ld_raw(const u64* p) { return __hip_atomic_load(gp(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); }
DEV float fix_t(u64 w, const u64* p, const StepArgs& a) {
  if ((u32)(w >> 32) != a.tag) w = ld_t_slow(p, a.tag, a.budget, a.status);
  return __uint_as_float((u32)w);
}
DEV float ld_t(const u64* p, const StepArgs& a) { return fix_t(ld_raw(p), p, a); }

// ---------------------------------------------------------------- reductions
DEV float dpp_f(float v, int ctrl);
template <int CTRL>
DEV float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// Sum over each 16-lane row (result in every lane of the row).
DEV float row16_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x124>(v);  // row_ror:4
  v += dpp<0x128>(v);  // row_ror:8
  return v;
}
// Sum over each 8-lane half row (result in every lane of the half row).
DEV float row8_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp<0x141>(v);  // row_half_mirror
  return v;
}
DEV float row16_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x124>(v));
  v = fmaxf(v, dpp<0x128>(v));
  return v;
}
DEV float readlane_f(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }
// Whole-wavefront sum / max, uniform result.  Call with all 64 lanes active.
DEV float wave_sum(float v) {
  v = row16_sum(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
DEV float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

// Slots of the small static LDS block `flags` (int[64]) besides 0..7 (abort,
// seen, tickets, clocks, trigger state) and 8..44 (GEMV reduction slots).
constexpr int kFlagEntryClock = 60;  // timing trace: clock at task entry
constexpr int kFlagWaitClock = 61;   // timing trace: clock when the dependency wait began
constexpr int kFlagWords = 128;      // size of the static flags block (64.. : the LDS weight ring)

// ---------------------------------------------------------------- task context
struct Ctx {
  const StepArgs* a;
  Task t;
  int id;
  int agent;     // worker index, or -1 in launch-per-task mode
  bool lpt;
  char* lds;     // dynamic LDS (kLdsBytes)
  int* flags;    // small static LDS block: [0] abort, [1] seen, [2] start ticket, [3] start clock
  const int* pos;  // this step's positions, copied to LDS at kernel entry
  int next;        // the worker's next task id in this step, or -1 (launch-per-task: -1)
};

// One poll of an event: lane i < kSubCounters loads sub-counter i
// (agent scope); poll_total sums them (uniform result).
DEV u32 poll_issue(const StepArgs& a, int ev, int lane) {
  u32 v = 0;
  if (lane < kSubCounters)
    v = __hip_atomic_load(gp(a.counters + ((size_t)ev * kSubCounters + lane) * kCounterStride), __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT);
  return v;
}
DEV u32 poll_total(u32 v) {
#pragma unroll
  for (int o = 1; o < kSubCounters; o <<= 1) v += __shfl_xor(v, o);
  return (u32)__builtin_amdgcn_readlane((int)v, 0);
}
DEV u32 event_total(const StepArgs& a, int ev, int lane) { return poll_total(poll_issue(a, ev, lane)); }

DEV void report_timeout(const StepArgs& a, int task, int ev, u32 seen, u32 target) {
  u32 z = 0;
  if (__hip_atomic_compare_exchange_strong(a.status + ST_ERROR, &z, (u32)ERR_TIMEOUT, __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
    __hip_atomic_store(a.status + ST_TASK, (u32)task, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.status + ST_EVENT, (u32)ev, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.status + ST_SEEN, seen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.status + ST_TARGET, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // the most upstream (smallest id) task that timed out
  if (task >= 0) __hip_atomic_fetch_min(a.status + ST_MIN_TASK, (u32)task, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(a.status + ST_ABORT, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wavefront 0 only: poll the task's dependency event until it reaches its
// target (bounded by the watchdog budget), then take the trace start ticket.
constexpr int kPolls = 2;         // polls in flight
constexpr int kPollStagger = 4;   // s_sleep units between the first polls
DEV void poll_dep(Ctx& c) {
  const StepArgs& a = *c.a;
  const int lane = threadIdx.x & 63;
  const int ev = c.t.dep;
  // timing trace: the clock when the wait begins (the pre-wait loads issued)
  if (a.trace_on == 2 && lane == 0) c.flags[kFlagWaitClock] = (int)(u32)wall_clock64();
  {
    u32 seen = 0;
    int bad = 0;
    if (ev >= 0) {
      const u32 target = (u32)a.events[ev].need * (a.epoch + 1u);
      seen = event_total(a, ev, lane);
      if (!c.lpt && seen < target) {
        // kPolls polls in flight, staggered, each re-issued as soon as it is
        // consumed: the event is seen about a round trip / kPolls after it lands
        const u64 t0 = wall_clock64();
        u32 p[kPolls];
#pragma unroll
        for (int i = 0; i < kPolls; ++i) {
          p[i] = poll_issue(a, ev, lane);
          if (i + 1 < kPolls) __builtin_amdgcn_s_sleep(kPollStagger);
        }
        for (int polls = 0;; ++polls) {
          bool hit = false;
#pragma unroll
          for (int i = 0; i < kPolls; ++i) {
            if (!hit) {
              seen = poll_total(p[i]);
              if (seen >= target) hit = true;
              else p[i] = poll_issue(a, ev, lane);
            }
          }
          if (hit) break;
          if ((polls & 7) == 7) {
            if (__hip_atomic_load(a.status + ST_ABORT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ||
                wall_clock64() - t0 > a.budget) {
              if (lane == 0) report_timeout(a, c.id, ev, seen, target);
              bad = 1;
              break;
            }
          }
        }
      }
    }
    if (lane == 0) {
      c.flags[1] = (int)seen;
      if (bad) c.flags[0] = 1;
      if (a.trace_on) {
        c.flags[2] = a.trace_on == 1
                         ? (int)__hip_atomic_fetch_add(a.status + ST_TICKET, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : 0;
        c.flags[3] = (int)(u32)wall_clock64();
      }
    }
  }
}

// Wait for the task's dependency event (wavefront 0 polls, the others wait at
// the barrier).  All threads call this.
DEV void wait_dep(Ctx& c) {
  if (threadIdx.x < 64) poll_dep(c);
  __syncthreads();
}

// All threads: once every thread has issued its output stores, one thread
// records the trace and triggers the task's event.  The trigger does not wait
// for the stores to be acknowledged: a consumer that reads a word before it
// lands sees the old tag and re-reads it.
// Thread 0 only: take the trace end ticket and clock, then add to the task's
// trigger event.  Called once per task, by finish or earlier by a body whose
// outputs are about to be stored (flags[5] records that it happened).
DEV void trigger_event(Ctx& c) {
  const StepArgs& a = *c.a;
  if (c.flags[5]) return;
  c.flags[5] = 1;
  c.flags[6] = (a.trace_on == 1 && !c.flags[0])
                   ? (int)__hip_atomic_fetch_add(a.status + ST_TICKET, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                   : 0;
  c.flags[7] = (int)(u32)wall_clock64();
  if (c.t.trig >= 0 && !c.flags[0]) {
    const int sub = (c.agent >= 0 ? c.agent : (int)blockIdx.x) & (kSubCounters - 1);
    __hip_atomic_fetch_add(gp(a.counters + ((size_t)c.t.trig * kSubCounters + sub) * kCounterStride), 1u,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

DEV void finish(Ctx& c) {
  const StepArgs& a = *c.a;
  __syncthreads();
  if (threadIdx.x == 0) {
    trigger_event(c);
    if (a.trace_on && !c.flags[0]) {
      // ticketed trace: global tickets and append order; timing trace: clocks
      // only, one slot per task id (no returning atomics on the task's path).
      // The end ticket and clock are the trigger's.
      const bool tk = a.trace_on == 1;
      u32 slot = tk ? __hip_atomic_fetch_add(a.status + ST_TRACE_N, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                    : (u32)c.id;
      if (slot < (u32)a.geom->n_tasks) {
        mk_trace_rec r;
        r.task = c.id;
        r.worker = (int16_t)c.agent;
        r.xcc = (int16_t)(__builtin_amdgcn_s_getreg(6164) & 0xF);  // HW_REG_XCC_ID[3:0]
        // timing trace: the clocks of task entry and of the start of the wait
        r.t_start = (u32)c.flags[tk ? 2 : kFlagEntryClock];
        r.t_end = (u32)c.flags[tk ? 6 : kFlagWaitClock];
        r.dep_seen = (u32)c.flags[1];
        r.step = a.epoch;
        r.clk_start = (u32)c.flags[3];
        r.clk_end = (u32)c.flags[7];
        a.trace[slot] = r;
      }
    }
  }
}

// Block-wide sum of one value per thread for NB independent values.
template <int NB>
DEV void block_sum(float (&v)[NB], float* red) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float s = wave_sum(v[b]);
    if (lane == 0) red[b * NWAVE + wave] = s;
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) s += red[b * NWAVE + w];
    v[b] = s;
  }
  __syncthreads();
}

// ---------------------------------------------------------------- embedding
// Greedy tokens from the lm_head candidates of an earlier step of this
// launch: wavefront 0 waits until the lm_head event has counted need *
// done_epoch triggers (that step's tiles), then all threads reduce the tiles'
// candidates, tagged `tag`, to one id per sequence b in [b0, b1) (ties to the
// lower id).  Results in tok[b] (LDS), valid after the final barrier.
DEV void lm_argmax(Ctx& c, u32 done_epoch, u32 tag, int b0, int b1, int* tok) {
  const StepArgs& a = *c.a;
  const Geom& G = *a.geom;
  const int ev = G.lm_event, T = G.lm_tiles, B = G.B;
  const int tid = task_tid(), wave = tid >> 6, lane = tid & 63;
  if (tid < 64) {
    const u32 target = (u32)a.events[ev].need * done_epoch;
    const u64 t0 = wall_clock64();
    for (int it = 0;; ++it) {
      const u32 seen = event_total(a, ev, lane);
      if (seen >= target) break;
      if ((it & 7) == 7 && (__hip_atomic_load(a.status + ST_ABORT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ||
                            wall_clock64() - t0 > a.budget)) {
        if (lane == 0) {
          report_timeout(a, c.id, ev, seen, target);
          c.flags[0] = 1;
        }
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
  float* sv = (float*)c.lds + 256;  // [NWAVE][16] values (tok[] may sit below)
  int* si = (int*)(sv + NWAVE * 16);
  for (int b = b0; b < b1; ++b) {
    float best = -INFINITY;
    int id = 0x7fffffff;
    if (!c.flags[0]) {
      for (int j = tid; j < T; j += NT) {
        const u64* p = a.cand + ((size_t)j * B + b) * 2;
        u64 wv = ld_raw(p), wi = ld_raw(p + 1);
        if ((u32)(wv >> 32) != tag) wv = ld_t_slow(p, tag, a.budget, a.status);
        if ((u32)(wi >> 32) != tag) wi = ld_t_slow(p + 1, tag, a.budget, a.status);
        const float v = __uint_as_float((u32)wv);
        const int i = (int)(u32)wi;
        if (v > best || (v == best && i < id)) {
          best = v;
          id = i;
        }
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(best, o);
      const int oi = __shfl_xor(id, o);
      if (ov > best || (ov == best && oi < id)) {
        best = ov;
        id = oi;
      }
    }
    if (lane == 0) {
      sv[wave * 16 + (b - b0)] = best;
      si[wave * 16 + (b - b0)] = id;
    }
  }
  __syncthreads();
  if (tid >= b0 && tid < b1) {
    float best = sv[tid - b0];
    int id = si[tid - b0];
    for (int w = 1; w < NWAVE; ++w) {
      const float v = sv[w * 16 + tid - b0];
      const int i = si[w * 16 + tid - b0];
      if (v > best || (v == best && i < id)) {
        best = v;
        id = i;
      }
    }
    tok[tid] = id;
  }
  __syncthreads();
}

DEV void body_embed(Ctx& c, const OpDesc& op) {
  const StepArgs& a = *c.a;
  const Geom& G = *a.geom;
  const int b = c.t.a0, H = G.H;
  int tok;
  if (a.step > 0) {
    // token feedback: the previous step's greedy token, recorded for the caller
    int* tk = (int*)c.lds;
    lm_argmax(c, a.epoch, a.tag - 1u, b, b + 1, tk);
    tok = tk[b];
    if (threadIdx.x == 0 && a.tokens_out) a.tokens_out[(size_t)(a.step - 1) * G.B + b] = tok;
  } else {
    tok = a.tokens[b];
  }
  if (tok < 0 || tok >= G.V) {
    if (threadIdx.x == 0) {
      u32 z = 0;
      __hip_atomic_compare_exchange_strong(a.status + ST_ERROR, &z, (u32)ERR_BAD_INPUT, __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    tok = 0;
  }
  const uint16_t* row = op.w + (size_t)tok * H;
  for (int k = threadIdx.x; k < H; k += NT) st_t(op.out + (size_t)b * H + k, bf2f(row[k]), a.tag);
}

// ---------------------------------------------------------------- GEMV input staging
// xs[b][k] = in[b][k] * g[k] (g = 1 when the op does not normalise its input),
// ss[b] = this thread's part of sum_k in[b][k]^2.  The RMSNorm scale
// rsqrt(mean(in^2) + eps) is a per-sequence scalar, so it is applied to the
// dot products in the epilogue instead of rescaling xs.
// Staging runs in two parts so that the first batch of input words can be
// issued ahead of the rest of the weight ring: in-order load completion would
// otherwise make the input wait behind the whole ring.
constexpr int kStageCH = 8;  // tagged words in flight per thread

// Words p[k0 + i*stride] (i < N, index < K) loaded as w[i]: while any of them
// still carries an older step's tag (its producer may trigger before storing,
// see gemv_valu), re-read the whole batch at agent scope, one round trip per
// retry, bounded by the watchdog budget.
template <int N>
DEV void refresh_batch(u64 (&w)[N], const u64* p, int k0, int stride, int K, const StepArgs& a) {
  auto stale = [&]() {
    bool st = false;
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (k0 + i * stride < K && (u32)(w[i] >> 32) != a.tag) st = true;
    return st;
  };
  if (!stale()) return;
  const u64 t0 = wall_clock64();
  for (int it = 0;; ++it) {
#pragma unroll
    for (int i = 0; i < N; ++i)
      w[i] = __hip_atomic_load(gp(p + min(k0 + i * stride, K - 1)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!stale()) return;
    if ((it & 7) == 7 && (__hip_atomic_load(a.status + ST_ABORT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ||
                          wall_clock64() - t0 > a.budget)) {
      // report through the word-level slow path (records the address, aborts)
#pragma unroll
      for (int i = 0; i < N; ++i)
        if (k0 + i * stride < K && (u32)(w[i] >> 32) != a.tag) w[i] = ld_t_slow(p + k0 + i * stride, a.tag, a.budget, a.status);
      return;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}
struct StageFirst {
  u64 w[kStageCH];
  float g[kStageCH];
};

DEV void stage_issue(const OpDesc& op, int tid, StageFirst& f) {
  const int K = op.K;
#pragma unroll
  for (int i = 0; i < kStageCH; ++i) f.w[i] = ld_raw(op.in + min(tid + i * NT, K - 1));
#pragma unroll
  for (int i = 0; i < kStageCH; ++i) f.g[i] = op.norm_in ? ldg(op.g + min(tid + i * NT, K - 1)) : 1.0f;
}

template <int NB>
DEV void stage_finish(Ctx& c, const OpDesc& op, int tid, const StageFirst& f, float* xs, float (&ss)[NB]) {
  const StepArgs& a = *c.a;
  const int K = op.K;
  constexpr int CH = kStageCH;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    ss[b] = 0.f;
    const u64* in = op.in + (size_t)b * K;
    for (int k0 = 0; k0 < K; k0 += NT * CH) {
      u64 w[CH];
      float gv[CH];
      if (b == 0 && k0 == 0) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          w[i] = f.w[i];
          gv[i] = f.g[i];
        }
      } else {
        // unconditional loads (clamped index): all in flight before the first tag check
#pragma unroll
        for (int i = 0; i < CH; ++i) w[i] = ld_raw(in + min(k0 + tid + i * NT, K - 1));
#pragma unroll
        for (int i = 0; i < CH; ++i) gv[i] = op.norm_in ? ldg(op.g + min(k0 + tid + i * NT, K - 1)) : 1.0f;
      }
      refresh_batch<CH>(w, in, k0 + tid, NT, K, a);
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int k = k0 + tid + i * NT;
        if (k < K) {
          const float v = __uint_as_float((u32)w[i]);
          xs[b * K + k] = v * gv[i];
          ss[b] += v * v;
        }
      }
    }
  }
}

DEV float a_eps(const Ctx& c) { return c.a->geom->eps; }

// Old-path norm: block reduction of the per-thread sums into rn (its barriers
// also publish xs).
template <int NB>
DEV void stage_norm(Ctx& c, const OpDesc& op, int tid, float (&ss)[NB], float* red, float* rn) {
  if (op.norm_in) {
    block_sum<NB>(ss, red);
    if (tid < NB) {
      float v = ss[0];
#pragma unroll
      for (int b = 1; b < NB; ++b)
        if (tid == b) v = ss[b];
      rn[tid] = rsqrtf(v / (float)op.K + a_eps(c));
    }
  } else {
    if (tid < NB) rn[tid] = 1.0f;
  }
}

// ---------------------------------------------------------------- GEMV epilogue
// Residual words of this thread's first epilogue output, loaded right after
// the wait so that the load overlaps the weight stream.
DEV u64 gemv_residual_prefetch(const Ctx& c, const OpDesc& op, int NB) {
  const int nr = c.t.a2, j = task_tid();
  if ((op.kind != OP_OPROJ && op.kind != OP_DOWN) || j >= NB * nr) return 0ull;
  const int b = j / nr, row = c.t.a1 + (j - b * nr);
  return ld_raw(op.res + (size_t)b * op.N + row);
}

// Where a finished GEMV tile leaves its per-row results and per-sequence
// norm scales in LDS (VALU path, batch NB; MFMA path).
DEV const float* valu_rows(const Ctx& c) { return (const float*)c.lds + kStageFloats; }
DEV const float* valu_scales(const Ctx& c, int NB) { return (const float*)(c.flags + 8) + NB * NWAVE; }

// Greedy candidates of one lm_head tile: per sequence, the largest logit of
// the tile's rows and its vocabulary id (ties to the lower id), taken from the
// same fp32 values the epilogue stores, kept as two tagged words.  All
// threads, after the barrier that ends the dot products (the input staging
// area at the start of LDS is dead by then and holds the per-wave results).
DEV void lm_candidates(Ctx& c, const float* rsl, int NR, const float* rn, int NB) {
  const StepArgs& a = *c.a;
  const int nr = c.t.a2, r0 = c.t.a1, tile = c.t.a0, B = a.geom->B;
  const int tid = task_tid(), wave = tid >> 6, lane = tid & 63;
  float* sv = (float*)c.lds;          // [NWAVE][16] values
  int* si = (int*)(sv + NWAVE * 16);  // [NWAVE][16] ids
  for (int b = 0; b < NB; ++b) {
    float best = -INFINITY;
    int id = 0x7fffffff;
    for (int r = tid; r < nr; r += NT) {
      const float v = rsl[b * NR + r] * rn[b];
      if (v > best) {  // rows ascend per thread: the first maximum is kept
        best = v;
        id = r0 + r;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(best, o);
      const int oi = __shfl_xor(id, o);
      if (ov > best || (ov == best && oi < id)) {
        best = ov;
        id = oi;
      }
    }
    if (lane == 0) {
      sv[wave * 16 + b] = best;
      si[wave * 16 + b] = id;
    }
  }
  __syncthreads();
  if (tid < NB) {
    float best = sv[tid];
    int id = si[tid];
    for (int w = 1; w < NWAVE; ++w) {
      const float v = sv[w * 16 + tid];
      const int i = si[w * 16 + tid];
      if (v > best || (v == best && i < id)) {
        best = v;
        id = i;
      }
    }
    u64* p = a.cand + ((size_t)tile * B + tid) * 2;
    st_t(p, best, a.tag);
    st_t(p + 1, __int_as_float(id), a.tag);
  }
}

DEV void gemv_epilogue(Ctx& c, const OpDesc& op, const float* rsl, int NR, u64 res0, const float* rn, int NB) {
  const StepArgs& a = *c.a;
  const int nr = c.t.a2, r0 = c.t.a1, N = op.N;
  for (int j = threadIdx.x; j < NB * nr; j += NT) {
    const int b = j / nr, r = j - b * nr, row = r0 + r;
    const float scale = rn[b];
    const float v = rsl[b * NR + r] * scale;
    switch (op.kind) {
      case OP_QKV:
      case OP_ROUTER:
        st_t(op.out + (size_t)b * N + row, v, a.tag);
        break;
      case OP_OPROJ:
      case OP_DOWN: {
        const u64* rp = op.res + (size_t)b * N + row;
        const float rv = j == (int)threadIdx.x ? fix_t(res0, rp, a) : ld_t(rp, a);
        st_t(op.out + (size_t)b * N + row, rv + v, a.tag);
        break;
      }
      case OP_GATEUP:
        st_t(op.out + (size_t)b * N + row, silu(v) * (rsl[b * NR + nr + r] * scale), a.tag);
        break;
      case OP_LMHEAD:
        a.logits[(size_t)b * N + row] = v;
        break;
      default:
        break;
    }
  }
}

// ---------------------------------------------------------------- GEMV (VALU, batch <= 4)
// Tile = NR contiguous bf16 rows of length K.  Wavefront w owns rows w, w+8, ...;
// in each row lane l reads 16-byte chunks l, l+64, ... (1 KB coalesced per
// wavefront load).  A row is cut into segments of S chunks per lane; a ring of
// DEPTH segments keeps LOADS loads per lane in flight.  Before the dependency
// wait only the first op.pre loads are issued; after it the first batch of
// input words goes out, then the rest of the ring, then the input is staged
// while the ring streams.  Loads go through a buffer resource so that
// out-of-range segments return zeros without touching memory.
constexpr int kEarlySegments = 4;  // segments of wavefront 0 still to consume when an early trigger fires
template <int NB, int S, int LOADS>
DEV void gemv_valu(Ctx& c, const OpDesc& op) {
  constexpr int DEPTH = LOADS / S > 1 ? LOADS / S : 2;
  const Task& t = c.t;
  const int K = op.K, CPR = K >> 3, NCH = (CPR + 63) >> 6, SPR = NCH / S;
  const bool gu = op.kind == OP_GATEUP;
  const int NR = gu ? 2 * t.a2 : t.a2;
  const int tid = task_tid(), wave = tid >> 6, lane = tid & 63;
  const int nrw = NR > wave ? (NR - wave + NWAVE - 1) / NWAVE : 0;
  const int NSEG = nrw * SPR;
  // ring segments issued before the wait; a control wavefront (op.pad & 1)
  // issues none, so that its event polls do not complete behind weight data
  const int PRE = ((op.pad & 1) && wave == 0) ? 0 : min(DEPTH, (op.pre + S - 1) / S);
  const bool early = (op.pad & 2) != 0;  // trigger before the epilogue (tagged outputs)
  const uint16_t* Wt = op.w + (size_t)(u32)t.a3;
  const __amdgpu_buffer_rsrc_t rs =
      rsrc_u(Wt, (u32)NR * (u32)K * 2u);

  u32x4 buf[DEPTH][S];
  // segment (fi, fq) of the refill cursor
  int fi = 0, fq = 0;
  auto voff = [&](int i, int q, int u) -> u32 {
    const int cc = (q * S + u) * 64 + lane;
    if (i >= nrw || cc >= CPR) return OOB;
    return (u32)((wave + NWAVE * i) * K + cc * 8) * 2u;
  };
  float* xs = (float*)c.lds;
  float* rsl = xs + kStageFloats;
  float* red = (float*)(c.flags + 8);
  // per-sequence RMSNorm scale of the input (1 when the op has no input
  // norm), kept in LDS next to the reduction slots for the epilogue
  float* rn = red + NB * NWAVE;
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    if (d < PRE) {
#pragma unroll
      for (int u = 0; u < S; ++u) buf[d][u] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff(fi, fq, u), 0, AUX_NT);
      if (++fq == SPR) { fq = 0; ++fi; }
    }
  }
  wait_dep(c);
  StageFirst sf;
  stage_issue(op, tid, sf);
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    if (d >= PRE) {
#pragma unroll
      for (int u = 0; u < S; ++u) buf[d][u] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff(fi, fq, u), 0, AUX_NT);
      if (++fq == SPR) { fq = 0; ++fi; }
    }
  }
  float ss[NB];
  stage_finish<NB>(c, op, tid, sf, xs, ss);
  stage_norm<NB>(c, op, tid, ss, red, rn);
  __syncthreads();
  const u64 res0 = gemv_residual_prefetch(c, op, NB);

  float acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = 0.f;
  int ci = 0, cq = 0;  // consume cursor
  for (int s0 = 0; s0 < NSEG; s0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      if (s0 + d < NSEG) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
          const int cc = (cq * S + u) * 64 + lane;
          if (cc < CPR) {
            const u32x4 w = buf[d][u];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
              const f32x4 x0 = *(const f32x4*)(xs + b * K + cc * 8);
              const f32x4 x1 = *(const f32x4*)(xs + b * K + cc * 8 + 4);
              float s = acc[b];
              s = fmaf(bf_lo(w.x), x0.x, s);
              s = fmaf(bf_hi(w.x), x0.y, s);
              s = fmaf(bf_lo(w.y), x0.z, s);
              s = fmaf(bf_hi(w.y), x0.w, s);
              s = fmaf(bf_lo(w.z), x1.x, s);
              s = fmaf(bf_hi(w.z), x1.y, s);
              s = fmaf(bf_lo(w.w), x1.z, s);
              s = fmaf(bf_hi(w.w), x1.w, s);
              acc[b] = s;
            }
          }
        }
        if (cq == SPR - 1) {
          const int r = wave + NWAVE * ci;
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const float v = wave_sum(acc[b]);
            if (lane == 0) rsl[b * NR + r] = v;
            acc[b] = 0.f;
          }
        }
        if (++cq == SPR) { cq = 0; ++ci; }
      }
#pragma unroll
      for (int u = 0; u < S; ++u) buf[d][u] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff(fi, fq, u), 0, AUX_NT);
      if (++fq == SPR) { fq = 0; ++fi; }
      // early trigger: once wavefront 0 has kEarlySegments segments left to
      // consume, the outputs are about an event hop away; consumers that
      // read first find older tags and re-read (refresh_batch / fix_t)
      if (early && wave == 0 && s0 + d + kEarlySegments >= NSEG && threadIdx.x == 0) trigger_event(c);
    }
  }
  __syncthreads();
  gemv_epilogue(c, op, rsl, NR, res0, rn, NB);
}

// Ring depth (loads per lane).  Deeper rings, also for the O projection that
// waits through attention and the merge, measured slower: the extra traffic
// lengthens the latency-bound attention -> merge -> O chain more than the
// prefetch saves.
constexpr int kRingDeep = 8, kRingShallow = 8;
template <int NB, int LOADS>
DEV void gemv_valu_s(Ctx& c, const OpDesc& op) {
  const int nch = ((op.K >> 3) + 63) >> 6;
  if (nch % 4 == 0) gemv_valu<NB, 4, LOADS>(c, op);
  else if (nch % 6 == 0) gemv_valu<NB, 6, LOADS>(c, op);
  else if (nch % 3 == 0) gemv_valu<NB, 3, LOADS>(c, op);
  else if (nch % 2 == 0) gemv_valu<NB, 2, LOADS>(c, op);
  else gemv_valu<NB, 1, LOADS>(c, op);
}
template <int NB>
DEV void gemv_valu_any(Ctx& c, const OpDesc& op) {
  if (op.kind == OP_OPROJ) gemv_valu_s<NB, kRingDeep>(c, op);
  else gemv_valu_s<NB, kRingShallow>(c, op);
}

// ---------------------------------------------------------------- GEMV (batch 1, LDS weight ring)
// Batch-1 tiles whose rows are whole kilobytes.  Wavefronts 4..7 are
// loaders: they stream the tile's weights into a ring of 4 KB LDS slots with
// LDS-DMA loads (global_load_lds_dwordx4: the data lands in LDS, no register
// holds it in flight; one wavefront alone issues them at only ~60% of the HBM
// rate, and the loaders also spend time on the ring's flags), and once the tile's last segment is issued they go on
// into the next GEMV tile of the worker's list, so the compute unit keeps
// weight bytes in flight through this tile's tail, epilogue and trigger and
// through the next tile's dependency wait and input staging.  Wavefronts
// 0..3 stage the input (their loads queue behind no weight loads), take ring
// segments round-robin and leave one partial dot product per segment; the
// epilogue sums each row's partials in a fixed order, so results do not
// depend on timing.
//   segment = U KB of the tile (U = Geom::ring_u: 4, 2 or 1, dividing every
//     ring op's row bytes), i.e. part of one row;
//   ring sequence numbers q count segments over the worker's run; segment q
//     goes to slot q mod kRingSlots and is loaded by loader q mod 4 (the slot
//     count is a multiple of 4, so each loader owns the slots q = j mod 4);
//   flags[kFrFill + s] = the sequence number that last landed in slot s
//     (published by its loader after a vmcnt wait), flags[kFrSlot + s] = the
//     sequence number slot s may take next (a consumer sets q + kRingSlots
//     when done with q).
constexpr int kRingSlots = 24;     // 4 KB slots
constexpr int kRingLoaders = 4;
constexpr int kRingInflight = 4;   // segments in flight per loader (4 loads each at most: vmcnt <= 16);
                                   // fewer than its slots, so landed segments wait in free slots
                                   // instead of stalling the loader until they are consumed
constexpr int kRingCons = NWAVE - kRingLoaders;  // consumer wavefronts
constexpr int kRingThreads = kRingCons * 64;
constexpr int kRingXs = 0;         // LDS byte offsets: staged input [K]
constexpr int kRingPart = 49152;   // per-segment partial sums
constexpr int kRingRows = 57344;   // row sums (lm_head candidates)
constexpr int kRingBase = 61440;   // the ring
constexpr int kRingStageCH = 24;   // input words per consumer thread in flight
static_assert(kRingBase + kRingSlots * 4096 <= kLdsBytes, "ring fits the worker's LDS");
static_assert(kRingSlots % kRingLoaders == 0 && kRingInflight * kRingLoaders < kRingSlots, "ring slots");
static_assert(kRingMaxK * 4 <= kRingPart, "input staging");
static_assert(kRingMaxSegs * 4 <= kRingRows - kRingPart && kRingMaxRows * 4 <= kRingBase - kRingRows, "LDS areas");
// flags[] slots of the ring (the static block has kFlagWords entries)
constexpr int kFrQi = 64;      // [kRingLoaders] loader j: next sequence number to issue
constexpr int kFrQp = 68;      // [kRingLoaders] loader j: next sequence number to publish
constexpr int kFrAhead = 72;   // task id the loaders ran ahead into, or -1
constexpr int kFrAheadQ0 = 73; // its first sequence number
constexpr int kFrGo = 74;      // dependency met (wavefront 0 -> consumers)
constexpr int kFrStaged = 75;  // consumer wavefronts done staging
constexpr int kFrSlot = 76;    // [kRingSlots]
constexpr int kFrDone = 124;   // consumer wavefronts done with this tile's segments
constexpr int kFrFill = kFrSlot + kRingSlots;  // [kRingSlots]
static_assert(kFrFill + kRingSlots <= kFrDone && kFrDone < kFlagWords, "ring flags fit");

// s_waitcnt vmcnt(N), other counters not waited on (gfx9 encoding)
template <int N>
DEV void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// wait until at most k segments of U loads are still in flight (0 <= k < kRingInflight)
template <int U>
DEV void ring_wait_segs(int k) {
  static_assert(kRingInflight <= 11, "one case per segment count");
  switch (k) {
    case 0: vm_wait<0>(); break;
    case 1: vm_wait<U * 1>(); break;
    case 2: vm_wait<U * 2>(); break;
    case 3: vm_wait<U * 3>(); break;
    case 4: vm_wait<U * 4>(); break;
    case 5: vm_wait<U * 5>(); break;
    case 6: vm_wait<U * 6>(); break;
    case 7: vm_wait<U * 7>(); break;
    case 8: vm_wait<U * 8>(); break;
    case 9: vm_wait<U * 9>(); break;
    default: vm_wait<U * 10>(); break;
  }
}

typedef __attribute__((address_space(1))) const void g_cvoid;
typedef __attribute__((address_space(3))) void l_void;
// LDS word access for the loader wavefronts.  The compiler cannot tell the
// ring's LDS-DMA destinations from other LDS words, so before any LDS access
// it can see it waits for every LDS-DMA load in flight (vmcnt(0)), which would
// leave one segment in flight.  These two are invisible to that analysis;
// each waits for its own LDS operation inside the asm block.
DEV u32 lds_addr(const void* p) { return (u32)(uintptr_t)(const __attribute__((address_space(3))) char*)p; }
DEV int lds_rd(const int* p) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return __builtin_amdgcn_readfirstlane(v);
}
DEV void lds_wr(int* p, int v) {
  asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(lds_addr(p)), "v"(v) : "memory");
}

// segment `seg` of the tile at w (U KB at byte offset seg * U KB) into one slot
template <int U>
DEV void ring_issue(const uint16_t* w, int seg, char* slot, int lane) {
  const char* src = (const char*)w + (size_t)seg * (U * 1024) + lane * 16;
#pragma unroll
  for (int u = 0; u < U; ++u)
    __builtin_amdgcn_global_load_lds((g_cvoid*)(src + u * 1024), (l_void*)(slot + u * 1024), 16, 0, AUX_NT);
}

DEV int ring_nr(const Task& t, const OpDesc& op) { return op.kind == OP_GATEUP ? 2 * t.a2 : t.a2; }

// Spin budget check of the ring's LDS waits (they end by construction; the
// budget only turns a protocol bug into a reported error instead of a hang).
DEV bool ring_spin_over(Ctx& c, u64 t0, int it) {
  if ((it & 63) != 63) return false;
  if (lds_rd(c.flags)) return true;
  if (wall_clock64() - t0 > c.a->budget) {
    if ((threadIdx.x & 63) == 0) report_timeout(*c.a, c.id, -1, 0, 0);
    lds_wr(c.flags, 1);
    return true;
  }
  return false;
}

// Loader j (wavefront 4 + j): issues this tile's remaining segments q = j
// mod 4, publishes each one as it lands, then runs ahead into the next tile when
// it is a ring tile too.  Returns once every segment of this tile that it
// loads has landed.
template <int U>
DEV void ring_loader(Ctx& c, const OpDesc& op, int q0, int nseg, int j) {
  int* F = c.flags;
  const int lane = threadIdx.x & 63;
  char* ring = c.lds + kRingBase;
  int qi = lds_rd(F + kFrQi + j), qp = lds_rd(F + kFrQp + j);
  const uint16_t* W = op.w + (size_t)(u32)c.t.a3;
  // the next task of this worker, when it is a ring tile (persistent mode)
  const uint16_t* W2 = nullptr;
  int nseg2 = 0;
  if (c.next >= 0) {
    const Task t2 = c.a->tasks[c.next];
    const OpDesc& o2 = c.a->ops[t2.op];
    if (o2.pad & 4) {
      W2 = o2.w + (size_t)(u32)t2.a3;
      nseg2 = ring_nr(t2, o2) * ((o2.K * 2) / (U * 1024));
    }
  }
  auto publish = [&]() {  // the oldest segment of this loader in flight has landed
    // the vmcnt wait orders the slot's LDS-DMA writes before the flag store
    ring_wait_segs<U>((qi - qp) / kRingLoaders - 1);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    lds_wr(F + kFrFill + qp % kRingSlots, qp);
    qp += kRingLoaders;
  };
  auto slot_free = [&](int q) { return lds_rd(F + kFrSlot + q % kRingSlots) == q; };
  const int qend = q0 + nseg;
  const u64 t0 = wall_clock64();
  int it = 0;
  while (qi < qend) {
    if ((qi - qp) / kRingLoaders == kRingInflight) {
      publish();
    } else if (slot_free(qi)) {
      ring_issue<U>(W, qi - q0, ring + (qi % kRingSlots) * 4096, lane);
      qi += kRingLoaders;
    } else if (qi > qp) {
      publish();
    } else {
      __builtin_amdgcn_s_sleep(1);
      if (ring_spin_over(c, t0, ++it)) break;
    }
  }
  if (W2 && !lds_rd(F)) {
    if (j == 0) {
      lds_wr(F + kFrAhead, c.next);
      lds_wr(F + kFrAheadQ0, qend);
    }
    // publish this tile's segments as they land and keep issuing the next
    // tile's until the consumers are done with this one; then return with up
    // to kRingInflight loads in flight (the next task publishes them)
    for (int it2 = 0;;) {
      if (qp >= qend && lds_rd(F + kFrDone) == kRingCons) break;
      if (qi < qend + nseg2 && (qi - qp) / kRingLoaders < kRingInflight && slot_free(qi)) {
        ring_issue<U>(W2, qi - qend, ring + (qi % kRingSlots) * 4096, lane);
        qi += kRingLoaders;
      } else if (qp < qend) {
        publish();
      } else {
        __builtin_amdgcn_s_sleep(1);
        if (ring_spin_over(c, t0, ++it2)) break;
      }
    }
  } else {
    while (qp < qi) publish();
  }
  lds_wr(F + kFrQi + j, qi);
  lds_wr(F + kFrQp + j, qp);
}

// Consumer wavefronts 0..3: segments s = wave, wave + 4, ... of this tile.
template <int U>
DEV void ring_consume(Ctx& c, const OpDesc& op, int q0, int nseg, int spr, const float* xs, float* part, int wave,
                      int lane) {
  int* F = c.flags;
  char* ring = c.lds + kRingBase;
  const bool early = (op.pad & 2) != 0;
  const u64 t0 = wall_clock64();
  int it = 0;
  for (int s = wave; s < nseg; s += kRingCons) {
    const int q = q0 + s, slot = q % kRingSlots;
    while (__hip_atomic_load(F + kFrFill + slot, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != q) {
      __builtin_amdgcn_s_sleep(1);
      if (ring_spin_over(c, t0, ++it)) return;
    }
    const int col0 = (s % spr) * (U * 512);
    const char* sp = ring + slot * 4096 + lane * 16;
    const float* xp = xs + col0 + lane * 8;
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u32x4 w = *(const u32x4*)(sp + u * 1024);
      const f32x4 x0 = *(const f32x4*)(xp + u * 512);
      const f32x4 x1 = *(const f32x4*)(xp + u * 512 + 4);
      acc = fmaf(bf_lo(w.x), x0.x, acc);
      acc = fmaf(bf_hi(w.x), x0.y, acc);
      acc = fmaf(bf_lo(w.y), x0.z, acc);
      acc = fmaf(bf_hi(w.y), x0.w, acc);
      acc = fmaf(bf_lo(w.z), x1.x, acc);
      acc = fmaf(bf_hi(w.z), x1.y, acc);
      acc = fmaf(bf_lo(w.w), x1.z, acc);
      acc = fmaf(bf_hi(w.w), x1.w, acc);
    }
    const float v = wave_sum(acc);  // every lane's slot reads are complete here
    if (lane == 0) {
      part[s] = v;
      __hip_atomic_store(F + kFrSlot + slot, q + kRingSlots, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    // early trigger once about kEarlySegments segments per wavefront remain
    if (early && wave == 0 && s + kRingCons * kEarlySegments >= nseg && lane == 0) trigger_event(c);
  }
}

// Input staging by the consumer wavefronts: xs[k] = in[k] * g[k]; returns this
// thread's sum of in[k]^2.
DEV float ring_stage(Ctx& c, const OpDesc& op, int tid, float* xs) {
  const StepArgs& a = *c.a;
  const int K = op.K;
  constexpr int CH = kRingStageCH, T = kRingThreads;
  float ss = 0.f;
  // buffer loads: one resource and one register offset for all words (words
  // past K read as zero and are not used)
  const __amdgpu_buffer_rsrc_t rin = rsrc_u(op.in, (u32)K * 8u);
  const __amdgpu_buffer_rsrc_t rg =
      rsrc_u(op.g, op.norm_in ? (u32)K * 4u : 0u);
  for (int base = 0; base < K; base += CH * T) {  // base: the same in every lane (scalar offsets)
    const int k0 = base + tid;
    u64 w[CH];
    float gv[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rin, (u32)tid * 8u, (base + i * T) * 8, 0);
      w[i] = ((u64)v.y << 32) | v.x;
    }
#pragma unroll
    for (int i = 0; i < CH; ++i)
      gv[i] = op.norm_in ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, (u32)tid * 4u, (base + i * T) * 4, 0))
                         : 1.0f;
    refresh_batch<CH>(w, op.in, k0, T, K, a);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int k = k0 + i * T;
      if (k < K) {
        const float v = __uint_as_float((u32)w[i]);
        xs[k] = v * gv[i];
        ss += v * v;
      }
    }
  }
  return ss;
}

DEV const float* ring_rows(const Ctx& c) { return (const float*)(c.lds + kRingRows); }

template <int U>
DEV void gemv_ring(Ctx& c, const OpDesc& op) {
  const StepArgs& a = *c.a;
  int* F = c.flags;
  const int tid = task_tid(), wave = tid >> 6, lane = tid & 63;
  const int nr = c.t.a2, NR = ring_nr(c.t, op);
  const int spr = (op.K * 2) / (U * 1024), nseg = NR * spr;
  float* xs = (float*)(c.lds + kRingXs);
  float* part = (float*)(c.lds + kRingPart);
  float* red = (float*)(F + 8);      // per consumer wavefront: sum of squares
  float* rnp = red + NWAVE;          // the norm scale (where lm_candidates reads it for NB = 1)
  // ring state: continue a run-ahead into this tile, or start an empty ring
  int q0 = 0;
  const bool ahead = lds_rd(F + kFrAhead) == c.id;  // (loaders may have LDS-DMA loads in flight)
  if (ahead) q0 = lds_rd(F + kFrAheadQ0);
  __syncthreads();  // every wavefront has read the state above
  if (!ahead) {
    if (tid < kRingLoaders) {
      F[kFrQi + tid] = tid;
      F[kFrQp + tid] = tid;
    }
    if (tid < kRingSlots) {
      F[kFrSlot + tid] = tid;
      F[kFrFill + tid] = -1;
    }
  }
  if (tid == 0) {
    F[kFrAhead] = -1;
    F[kFrGo] = 0;
    F[kFrStaged] = 0;
    F[kFrDone] = 0;
  }
  __syncthreads();
  u64 res0 = 0;
  if (wave >= kRingCons) {
    ring_loader<U>(c, op, q0, nseg, wave - kRingCons);
  } else {
    // dependency: wavefront 0 polls, the other consumers wait for its flag
    if (wave == 0) {
      poll_dep(c);
      if (lane == 0) __hip_atomic_store(F + kFrGo, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    } else {
      const u64 t0 = wall_clock64();
      int it = 0;
      while (!__hip_atomic_load(F + kFrGo, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP)) {
        __builtin_amdgcn_s_sleep(1);
        if ((++it & 1023) == 0 && wall_clock64() - t0 > (u64)2 * a.budget) break;  // wavefront 0 has its own watchdog
      }
    }
    const float ss = wave_sum(ring_stage(c, op, tid, xs));
    res0 = gemv_residual_prefetch(c, op, 1);
    if (lane == 0) {
      red[wave] = ss;
      __hip_atomic_fetch_add(F + kFrStaged, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    {
      const u64 t0 = wall_clock64();
      int it = 0;
      while (__hip_atomic_load(F + kFrStaged, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < kRingCons) {
        __builtin_amdgcn_s_sleep(1);
        if (ring_spin_over(c, t0, ++it)) break;
      }
    }
    if (tid == 0) {
      float s = 0.f;
      for (int w = 0; w < kRingCons; ++w) s += red[w];
      *rnp = op.norm_in ? rsqrtf(s / (float)op.K + a_eps(c)) : 1.0f;
    }
    ring_consume<U>(c, op, q0, nseg, spr, xs, part, wave, lane);
    // the consumers' own barrier: the loaders keep streaming meanwhile
    if (lane == 0) __hip_atomic_fetch_add(F + kFrDone, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    {
      const u64 t0 = wall_clock64();
      int it = 0;
      while (__hip_atomic_load(F + kFrDone, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < kRingCons) {
        __builtin_amdgcn_s_sleep(1);
        if (ring_spin_over(c, t0, ++it)) break;
      }
    }
  }
  // epilogue (consumer threads only: the loader wavefronts may still have
  // run-ahead loads in flight and issue no other memory operations); the
  // task's closing barrier in finish() joins the loaders
  if (tid < kRingThreads) {
    const float rn = *rnp;
    float* rows = (float*)(c.lds + kRingRows);
    const int r0 = c.t.a1;
    for (int j = tid; j < nr; j += kRingThreads) {
      float sv = 0.f;
      for (int i = 0; i < spr; ++i) sv += part[j * spr + i];
      const float v = sv * rn;
      const int row = r0 + j;
      switch (op.kind) {
        case OP_QKV:
          st_t(op.out + row, v, a.tag);
          break;
        case OP_OPROJ:
        case OP_DOWN: {
          const u64* rp = op.res + row;
          const float rv = j == tid ? fix_t(res0, rp, a) : ld_t(rp, a);
          st_t(op.out + row, rv + v, a.tag);
          break;
        }
        case OP_GATEUP: {
          float su = 0.f;
          for (int i = 0; i < spr; ++i) su += part[(nr + j) * spr + i];
          st_t(op.out + row, silu(v) * (su * rn), a.tag);
          break;
        }
        case OP_LMHEAD:
          a.logits[row] = v;
          rows[j] = sv;
          break;
        default:
          break;
      }
    }
  }
}

DEV void gemv_ring_any(Ctx& c, const OpDesc& op) {
  const int u = c.a->geom->ring_u;
  if (u == 4) gemv_ring<4>(c, op);
  else if (u == 2) gemv_ring<2>(c, op);
  else gemv_ring<1>(c, op);
}

// ---------------------------------------------------------------- GEMV (MFMA, batch 5..16)
// A skinny GEMM on the matrix cores: D[16 rows][16 sequences] += W[16][32] x
// X[32][16] per v_mfma_f32_16x16x32_bf16, sequences past the batch padded
// with zeros.  Still bound by the weight stream (16 flop per weight byte at
// batch 16); the VALU dot products would be LDS-bound here.
//   weights: 1 KB fragments, fragment (group g of 16 rows, k-block kb of 32
//     columns) at ((g * K/32 + kb) * 64 + lane) * 16 bytes, lane l holding
//     row l%16, columns 8*(l/16) .. +8 (laid out at load time);
//   inputs: staged per chunk of KC columns in LDS as bf16 rows, sequence b
//     at b * kMfmaRS elements (row stride padded by 8 so that the 16 lanes of
//     a fragment read fall in distinct banks); the input fragment of k-block
//     kb is read from there, lane l holding sequence l%16, columns
//     kb*32 + 8*(l/16) .. +8.  Each value x is split as hi = bf16(x),
//     lo = bf16(x - hi) and both parts are multiplied (two MFMAs per weight
//     fragment), so the input keeps about 16 significant bits instead of
//     bf16's 8 (a plain bf16 input cost ~2% logits error over 36 layers at
//     batch 16).
// Work items are (row group, K part) pairs: tiles with fewer than eight row
// groups split K across wavefronts (parts interleaved by k-block) and sum the
// parts through LDS.  Each wavefront streams its items' fragments through a
// ring of kMfmaDepth loads; every (chunk, item) segment is padded to whole
// ring turns so that ring slots stay compile-time indices.
constexpr int kMfmaKC = 1536;     // input columns staged per chunk
constexpr int kMfmaRS = kMfmaKC + 8;                // staged row stride (bf16 elements)
constexpr int kMfmaXBytes = 16 * kMfmaRS * 2;       // one staged part (hi or lo), 16 sequences
constexpr int kMfmaDepth = 8;     // weight fragments in flight per wavefront
constexpr int kMfmaMaxItems = 4;  // items per wavefront (row groups per tile <= 32)
constexpr int kMfmaEarlyTurns = 2;  // ring turns of wavefront 0 left when an early trigger fires
constexpr int kMfmaVariant = 16;  // kernel template value of the MFMA variant
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
static_assert(NWAVE == 8, "the MFMA stager gives wavefront w sequences w and w + 8");
static_assert(kMfmaXBytes % 16 == 0, "staged parts stay 16-byte aligned");

// Stage input columns [c0, c0 + ncols) of every sequence (x * g for
// normalising ops) as bf16 hi and lo rows.  Wavefront w stages sequences w
// and w + 8 (rows past the batch are written as zeros): lane l reads words
// c0 + l + 64 i of both sequences, so every load instruction covers 64
// consecutive tagged words (512 bytes, whole cache lines), and kStageMfma
// columns of both sequences (with their gains) are in flight per lane before
// the first tag check.  ss[h] accumulates the sum of squares of the lane's
// values of sequence w + 8 h.
constexpr int kStageMfma = 8;  // columns per lane in flight (x 2 sequences)
DEV void mfma_stage(Ctx& c, const OpDesc& op, int tid, int c0, int ncols, uint16_t* xh, uint16_t* xo, float (&ss)[2]) {
  const StepArgs& a = *c.a;
  const int B = a.geom->B, K = op.K;
  const int wave = tid >> 6, lane = tid & 63;
  bool live[2];
  const u64* src[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int b = wave + 8 * h;
    live[h] = b < B;
    src[h] = op.in + (size_t)(live[h] ? b : 0) * K + c0;
  }
  for (int j0 = 0; j0 * 64 < ncols; j0 += kStageMfma) {
    u64 w[2][kStageMfma];
    float g[kStageMfma];
#pragma unroll
    for (int i = 0; i < kStageMfma; ++i) {
      const int col = min(lane + 64 * (j0 + i), ncols - 1);
#pragma unroll
      for (int h = 0; h < 2; ++h) w[h][i] = ld_raw(src[h] + col);
      g[i] = op.norm_in ? ldg(op.g + c0 + col) : 1.0f;
    }
#pragma unroll
    for (int i = 0; i < kStageMfma; ++i) {
      const int col = lane + 64 * (j0 + i);
      if (col < ncols) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint16_t hi = 0, lo = 0;
          if (live[h]) {
            const float v = fix_t(w[h][i], src[h] + col, a);
            ss[h] += v * v;
            const float x = v * g[i];
            hi = f2bf(x);
            lo = f2bf(x - bf2f(hi));
          }
          const int e = (wave + 8 * h) * kMfmaRS + col;
          xh[e] = hi;
          xo[e] = lo;
        }
      }
    }
  }
}

// LDS locations of the MFMA path's per-row results [B][NR] and norm scales [16].
DEV const float* mfma_rows(const Ctx& c) { return (const float*)(c.lds + 2 * kMfmaXBytes); }
DEV const float* mfma_scales(const Ctx& c) { return mfma_rows(c) + kRowResultFloats + NWAVE * 256 + 16 * NWAVE; }

DEV void gemv_mfma(Ctx& c, const OpDesc& op) {
  const StepArgs& a = *c.a;
  const Task& t = c.t;
  const int B = a.geom->B, K = op.K, KB = K >> 5;
  const bool gu = op.kind == OP_GATEUP;
  const int NR = gu ? 2 * t.a2 : t.a2;
  const int ngroups = NR >> 4;
  const int kparts = ngroups >= NWAVE ? 1 : NWAVE / ngroups;
  const int nitems = ngroups * kparts;
  const int tid = task_tid(), wave = tid >> 6, lane = tid & 63;
  const int nit = nitems > wave ? (nitems - wave + NWAVE - 1) / NWAVE : 0;
  const int KC = min(kMfmaKC, K), KBc = KC >> 5, nchunks = (K + KC - 1) / KC;
  const bool early = (op.pad & 2) != 0;  // trigger before the epilogue (tagged outputs)
  constexpr int DEPTH = kMfmaDepth;
  const int NJ = (KBc + kparts - 1) / kparts;
  const int NJp = (NJ + DEPTH - 1) / DEPTH * DEPTH;
  const uint16_t* Wt = op.w + (size_t)(u32)t.a3;
  const __amdgpu_buffer_rsrc_t rs =
      rsrc_u(Wt, (u32)NR * (u32)K * 2u);

  // fill cursor: chunk fc, item slot fit (its group fg and part fqp), step fj
  int fc = 0, fit = 0, fj = 0;
  int fg = wave % max(ngroups, 1), fqp = wave / max(ngroups, 1);
  auto fill = [&]() -> u32 {
    u32 off = OOB;
    if (fc < nchunks && fit < nit) {
      const int kbl = fqp + fj * kparts, kb = fc * KBc + kbl;
      if (fj < NJ && kbl < KBc && kb < KB) off = (u32)(((fg * KB + kb) << 6) + lane) << 4;
    }
    if (++fj == NJp) {
      fj = 0;
      if (++fit >= nit) {
        fit = 0;
        ++fc;
      }
      const int item = wave + NWAVE * fit;
      fg = item % max(ngroups, 1);
      fqp = item / max(ngroups, 1);
    }
    return off;
  };
  u32x4 buf[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) buf[d] = __builtin_amdgcn_raw_buffer_load_b128(rs, fill(), 0, AUX_NT);

  wait_dep(c);
  uint16_t* xh = (uint16_t*)c.lds;                   // [16][kMfmaRS] bf16, hi parts
  uint16_t* xo = xh + 16 * kMfmaRS;                   // lo parts
  float* rsl = (float*)(c.lds + 2 * kMfmaXBytes);    // [B][NR]
  float* part = rsl + kRowResultFloats;              // [item][16 seq][16 rows]
  float* red = part + NWAVE * 256;                   // [16 seq][NWAVE]
  float* rn = red + 16 * NWAVE;                      // [16]
  const u64 res0 = gemv_residual_prefetch(c, op, B);
  float ss[2] = {0.f, 0.f};
  mfma_stage(c, op, tid, 0, min(KBc, KB) * 32, xh, xo, ss);
  __syncthreads();

  f32x4 acc[kMfmaMaxItems];
#pragma unroll
  for (int i = 0; i < kMfmaMaxItems; ++i) acc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // input fragment of this lane: sequence lane % 16, columns 8 * (lane / 16) .. +8 of a k-block
  const int xrow = (lane & 15) * kMfmaRS + (lane >> 4) * 8;
  for (int cc = 0; cc < nchunks; ++cc) {
    const int kbc = min(KBc, KB - cc * KBc);  // k-blocks in this chunk
    if (cc > 0) {
      __syncthreads();
      mfma_stage(c, op, tid, cc * KC, kbc * 32, xh, xo, ss);
      __syncthreads();
    }
#pragma unroll
    for (int it = 0; it < kMfmaMaxItems; ++it) {
      if (it < nit) {
        const int q = (wave + NWAVE * it) / ngroups;
        for (int j0 = 0; j0 < NJp; j0 += DEPTH) {
#pragma unroll
          for (int d = 0; d < DEPTH; ++d) {
            const int j = j0 + d, kbl = q + j * kparts;
            if (j < NJ && kbl < kbc) {
              const u32x4 xv = *(const u32x4*)(xh + xrow + kbl * 32);
              const u32x4 xw = *(const u32x4*)(xo + xrow + kbl * 32);
              const bf16x8 wv = __builtin_bit_cast(bf16x8, buf[d]);
              acc[it] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv, __builtin_bit_cast(bf16x8, xv), acc[it], 0, 0, 0);
              acc[it] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv, __builtin_bit_cast(bf16x8, xw), acc[it], 0, 0, 0);
            }
            buf[d] = __builtin_amdgcn_raw_buffer_load_b128(rs, fill(), 0, AUX_NT);
          }
          // early trigger: wavefront 0 in its last item of the last chunk with
          // kMfmaEarlyTurns ring turns left; consumers that read first find
          // older tags and re-read (as for the VALU tiles)
          if (early && wave == 0 && cc == nchunks - 1 && it == nit - 1 && j0 + kMfmaEarlyTurns * DEPTH >= NJp &&
              lane == 0)
            trigger_event(c);
        }
      }
    }
  }
  // D layout: lane l holds rows 4*(l/16) + r of sequence l%16
  const int n = lane & 15, r4 = (lane >> 4) * 4;
  if (kparts == 1) {
#pragma unroll
    for (int it = 0; it < kMfmaMaxItems; ++it) {
      if (it < nit && n < B) {
        const int g = (wave + NWAVE * it) % ngroups;
#pragma unroll
        for (int r = 0; r < 4; ++r) rsl[n * NR + g * 16 + r4 + r] = acc[it][r];
      }
    }
  } else if (nit > 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) part[wave * 256 + n * 16 + r4 + r] = acc[0][r];
  }
  // sum of squares per sequence: wavefront w staged sequences w and w + 8
  const float s0 = wave_sum(ss[0]), s1 = wave_sum(ss[1]);
  if (lane < 16) red[lane * NWAVE + wave] = lane == wave ? s0 : (lane == wave + 8 ? s1 : 0.f);
  __syncthreads();
  if (kparts > 1) {
    for (int j = tid; j < B * NR; j += NT) {
      const int nn = j / NR, row = j - nn * NR, g = row >> 4, i = row & 15;
      float sum = 0.f;
      for (int q = 0; q < kparts; ++q) sum += part[(q * ngroups + g) * 256 + nn * 16 + i];
      rsl[nn * NR + row] = sum;
    }
  }
  if (tid < B) {
    float r = 1.0f;
    if (op.norm_in) {
      float tt = 0.f;
#pragma unroll
      for (int w8 = 0; w8 < NWAVE; ++w8) tt += red[tid * NWAVE + w8];
      r = rsqrtf(tt / (float)K + a_eps(c));
    }
    rn[tid] = r;
  }
  __syncthreads();
  gemv_epilogue(c, op, rsl, NR, res0, rn, B);
}

// ---------------------------------------------------------------- group reductions
// Reduction over aligned groups of Lc lanes (Lc a power of two <= 64, uniform
// across the wavefront; every lane of the group receives the result).  Steps
// inside a 16-lane row use DPP; the 32- and 64-lane steps use the CDNA4
// permlane swaps, which exchange rows between two registers.
template <bool MAX>
DEV float grp_op(float x, float y) { return MAX ? fmaxf(x, y) : x + y; }
template <bool MAX>
DEV float group_reduce(float v, int Lc) {
  if (Lc >= 2) v = grp_op<MAX>(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
  if (Lc >= 4) v = grp_op<MAX>(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
  if (Lc >= 8) v = grp_op<MAX>(v, dpp<0x141>(v));  // row_half_mirror
  if (Lc >= 16) v = grp_op<MAX>(v, dpp<0x140>(v)); // row_mirror
  if (Lc >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = grp_op<MAX>(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  if (Lc >= 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = grp_op<MAX>(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return v;
}

// ---------------------------------------------------------------- merge
// Combine the C chunk partials of (sequence b, kv head group gi) for outputs
// k in [k0, k0 + n) of the group (k = h * D + d).  Each chunk left, per head,
// its normalised output o_c = (sum_r e^{s_r - m_c} v_r) / l_c and
// lse_c = m_c + log l_c; the merged output is
//   sum_c e^{lse_c - M} o_c / sum_c e^{lse_c - M},  M = max_c lse_c
// (the split-KV combine of flash decoding).  Lc lanes (C rounded up to a power
// of two) share one output, one chunk per lane: one batch of loads, then three
// group reductions.
DEV void merge_slice(Ctx& c, const u64* parts, u64* out, int b, int gi, int k0, int n, bool early = false) {
  const StepArgs& a = *c.a;
  const Geom& G = *a.geom;
  const int D = G.D, NG = G.G, C = G.C;
  const int tid = task_tid(), wave = tid >> 6, lane = tid & 63;
  int Lc = 1;
  while (Lc < C) Lc <<= 1;
  const int opw = 64 / Lc, per_pass = NWAVE * opw;
  const int cl = lane & (Lc - 1);
  const int cc = cl < C ? cl : C - 1;
  const size_t cstride = (size_t)NG * (D + 2);
  const u64* base = parts + (((size_t)b * G.Hkv + gi) * C + cc) * cstride;
  u64* dst = out + (size_t)b * G.Hq * D + (size_t)gi * NG * D + k0;
  for (int p = 0; p * per_pass < n; ++p) {
    const int kk = p * per_pass + wave * opw + lane / Lc;
    const bool valid = kk < n && cl < C;
    const int k = k0 + (kk < n ? kk : n - 1);
    const int h = k / D, d = k - h * D;
    const u64* pl = base + (size_t)h * (D + 2);
    const u64 wl = ld_raw(pl), wo = ld_raw(pl + 2 + d);
    float lse = -INFINITY, o = 0.f;
    if (valid) {
      lse = fix_t(wl, pl, a);
      o = fix_t(wo, pl + 2 + d, a);
    }
    // inputs of the last pass are current: the outputs are a few instructions away
    if (early && (p + 1) * per_pass >= n && tid == 0) trigger_event(c);
    const float M = group_reduce<true>(lse, Lc);
    const float w = lse == -INFINITY ? 0.f : expf(lse - M);
    const float num = group_reduce<false>(w * o, Lc);
    const float den = group_reduce<false>(w, Lc);
    if (valid && cl == 0) st_t(dst + kk, den > 0.f ? num / den : 0.f, a.tag);
  }
}

DEV void body_merge(Ctx& c, const OpDesc& op) {
  merge_slice(c, op.in, op.out, c.t.a0, c.t.a1, c.t.a2, c.t.a3, (op.pad & 2) != 0);
}

// ---------------------------------------------------------------- KV append
// One wavefront writes a new bf16 cache row (D values staged in LDS by the
// same wavefront) as D/2 packed 32-bit words with agent-scope stores, then
// waits until every store of the wavefront has completed.
//
// Why: in a multi-step launch the chunk bounds follow len = p + 1, so a row
// appended at step s is read at a later step of the same launch by another
// chunk task, which may run on another XCD.  XCD L2 caches are not coherent
// and write back plain stores only at the end of the kernel, so a plain store
// could stay invisible to that reader.  An agent-scope store writes through to
// memory, and the wait makes the row globally visible before the task's
// trigger (issued after the barrier that ends the prologue).  Every later
// reader of the row orders its loads after that trigger through the event
// graph: its worker finished an lm_head tile of the writing step, and every
// lm_head tile depends transitively on every attention chunk of the step.
// The reader's own L2 cannot hold a stale copy of the row: no task reads a
// row before the step that appends it.
template <int D>
DEV void kv_append(const uint16_t* row, uint16_t* dst, int lane, bool ok) {
  // the wavefront's own LDS writes above complete before the reads below
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
  if (ok && lane < D / 2)
    __hip_atomic_store(gp((u32*)dst) + lane, ((const u32*)row)[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);
}

// ---------------------------------------------------------------- attention
// One (sequence b, kv head group gi, chunk ch) task over cache rows
// [t0, t1) of positions 0..p (p = this step's position of sequence b):
// q-norm + RoPE for the NG query heads of the group; in the last chunk also
// k-norm + RoPE of the new key, bf16 rounding and the KV-cache append at p
// (the new row is used from LDS, not re-read); then scores, the chunk-local
// softmax (max m, sum l) and the normalised chunk output o / l with
// lse = m + log l per head.
// Keys are read 16 bytes per lane (D/8 lanes per row, row sums by DPP);
// values 4 bytes per lane (D/2 lanes per row), so each lane accumulates its
// two output columns over whole rows and the only reduction is one pass over
// the eight wavefronts through LDS.  Both rings are issued before the
// dependency wait.
template <int NG, int D>
DEV void attn_chunk(Ctx& c, const OpDesc& op) {
  const StepArgs& a = *c.a;
  const Geom& G = *a.geom;
  const int b = c.t.a0, gi = c.t.a1, ch = c.t.a2;
  const int C = G.C, Hkv = G.Hkv, cap = G.cap;
  const int tid = task_tid(), wave = tid >> 6, lane = tid & 63;
  constexpr int KL = D / 8, KR = 64 / KL, KP = NWAVE * KR;  // keys: lanes per row, rows per wave, rows per pass
  constexpr int VL = D / 2, VR = 64 / VL, VP = NWAVE * VR;  // values
  constexpr int RK = 4, RV = 16;                            // ring depths (passes)
  int pos = c.pos[b];
  // a position outside the cache is reported; the step still runs on a
  // clamped position so that every wait ends, but appends nothing
  bool pos_ok = pos >= 0 && pos < cap;
  if (!pos_ok) {
    if (tid == 0) {
      u32 z = 0;
      __hip_atomic_compare_exchange_strong(a.status + ST_ERROR, &z, (u32)ERR_BAD_INPUT, __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    pos = pos < 0 ? 0 : cap - 1;
  }
  const int len = pos + 1;
  const int t0 = (int)((long)ch * len / C), t1 = (int)((long)(ch + 1) * len / C);
  const bool last = ch == C - 1;
  const int T = t1 - t0;
  const int Told = last ? T - 1 : T;  // rows read from the cache (the newest comes from LDS)

  constexpr int SMAX = kScoreFloats / NG;
  float* qs = (float*)c.lds;                  // [NG][D], pre-scaled by 1/sqrt(D)
  uint16_t* knew = (uint16_t*)(qs + NG * D);  // [D] new key (bf16 bits)
  uint16_t* vnew = knew + D;                  // [D] new value
  float* sc = (float*)(vnew + D);             // [NG][SMAX] raw scores
  float* pt = sc + kScoreFloats;              // [row][NG] softmax numerators e^{s - m}
  float* red = pt + kScoreFloats;             // [NWAVE][NG][D] per-wavefront outputs
  float* ml = red + NWAVE * NG * D;           // [NG][2] m, l
  int* pgl = (int*)(ml + 2 * NG);             // paged: physical pages of the chunk's rows

  // Cache rows.  Contiguous: the buffer resource starts at row t0 of (layer,
  // b, gi).  Paged (the serving layout of paged attention): row t of sequence
  // b lives at row t mod page of physical page table[b][t / page], the pools
  // being [L][n_pages][Hkv][page][D]; the resource spans the layer's pool and
  // the chunk's page numbers are staged in LDS (read again by every ring
  // refill).  A page number outside the pool is reported and read as page 0.
  const bool paged = a.page_shift >= 0;
  const int sh = paged ? a.page_shift : 0, pmask = (1 << sh) - 1;
  uint16_t* Kc;
  uint16_t* Vc;
  u32 span;
  int lp0 = 0;
  size_t new_row = (size_t)pos;  // element row of the appended entry (relative to Kc / Vc)
  if (!paged) {
    const size_t base = ((((size_t)op.layer * G.B + b) * Hkv + gi) * (size_t)cap) * D;
    Kc = a.kv_k + base;
    Vc = a.kv_v + base;
    span = (u32)(Told > 0 ? Told : 0) * (u32)D * 2u;
  } else {
    const size_t pool = (size_t)op.layer * (size_t)a.n_pages * Hkv * ((size_t)1 << sh) * D;
    Kc = a.kv_k + pool;
    Vc = a.kv_v + pool;
    span = (u32)a.n_pages * (u32)Hkv * ((u32)1 << sh) * (u32)D * 2u;
    const int32_t* tbl = a.page_table + (size_t)b * (cap >> sh);
    lp0 = t0 >> sh;
    const int np = Told > 0 ? ((t0 + Told - 1) >> sh) - lp0 + 1 : 0;
    for (int i = tid; i < np; i += NT) {
      int ph = tbl[lp0 + i];
      if (ph < 0 || ph >= a.n_pages) {
        u32 z = 0;
        __hip_atomic_compare_exchange_strong(a.status + ST_ERROR, &z, (u32)ERR_BAD_INPUT, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ph = 0;
      }
      pgl[i] = ph;
    }
    if (last) {
      const int ph = tbl[pos >> sh];
      if (ph < 0 || ph >= a.n_pages) {
        pos_ok = false;  // nothing is appended; the error is reported below
        if (tid == 0) {
          u32 z = 0;
          __hip_atomic_compare_exchange_strong(a.status + ST_ERROR, &z, (u32)ERR_BAD_INPUT, __ATOMIC_RELAXED,
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      } else {
        new_row = ((size_t)(ph * Hkv + gi) << sh) + (size_t)(pos & pmask);
      }
    }
    __syncthreads();
  }
  // element offset of cache row t (t0 <= t < t0 + Told) within the resource
  auto row_off = [&](int t) -> u32 {
    if (!paged) return (u32)(t - t0) * (u32)D;
    return ((u32)((pgl[(t >> sh) - lp0] * Hkv + gi) << sh) + (u32)(t & pmask)) * (u32)D;
  };
  const __amdgpu_buffer_rsrc_t rk =
      rsrc_u(paged ? Kc : Kc + (size_t)t0 * D, (u32)span);
  const __amdgpu_buffer_rsrc_t rv =
      rsrc_u(paged ? Vc : Vc + (size_t)t0 * D, (u32)span);
  const int krow = wave * KR + lane / KL, kc = lane % KL;  // key row within a pass, 16-byte column
  const int vrow = wave * VR + lane / VL, vc = lane % VL;  // value row within a pass, 4-byte column
  auto koff = [&](int p) -> u32 {
    const int r = p * KP + krow;
    return r < Told ? (row_off(t0 + r) + (u32)(kc * 8)) * 2u : OOB;
  };
  auto voff = [&](int p) -> u32 {
    const int r = p * VP + vrow;
    return r < Told ? (row_off(t0 + r) + (u32)(vc * 2)) * 2u : OOB;
  };
  const int nk = (T + KP - 1) / KP, nv = (T + VP - 1) / VP;
  u32x4 kr[RK];
  u32 vr[RV];
#pragma unroll
  for (int p = 0; p < RK; ++p) kr[p] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff(p), 0, AUX_NT);
#pragma unroll
  for (int p = 0; p < RV; ++p) vr[p] = __builtin_amdgcn_raw_buffer_load_b32(rv, voff(p), 0, AUX_NT);

  // inputs that do not depend on this step: gains and RoPE frequencies
  constexpr int half = D / 2;
  float gq0 = 0.f, gq1 = 0.f, gk0 = 0.f, gk1 = 0.f;
  double ifreq = 0.0;
  if (lane < half) {
    gq0 = ldg(op.g + lane);
    gq1 = ldg(op.g + lane + half);
    gk0 = ldg(op.g2 + lane);
    gk1 = ldg(op.g2 + lane + half);
    ifreq = G.inv_freq[lane];
  }

  wait_dep(c);

  // q / k / v prologue: wavefront h handles head h (then k at NG, v at NG+1)
  const u64* qkv = op.in + (size_t)b * G.qkv_stride + (size_t)gi * (NG + 2) * D;
  for (int h = wave; h < NG + 2; h += NWAVE) {
    if (h >= NG && !last) continue;
    float x0 = 0.f, x1 = 0.f;
    {
      const u64* p0 = qkv + (size_t)h * D + (lane < half ? lane : 0);
      const u64 w0 = ld_raw(p0), w1 = ld_raw(p0 + half);
      if (lane < half) {
        x0 = fix_t(w0, p0, a);
        x1 = fix_t(w1, p0 + half, a);
      }
    }
    if (h == NG + 1) {
      if (lane < half) {
        vnew[lane] = f2bf(x0);
        vnew[lane + half] = f2bf(x1);
      }
      kv_append<D>(vnew, Vc + new_row * D, lane, pos_ok);
      continue;
    }
    const float ss = wave_sum(x0 * x0 + x1 * x1);
    const float r = rsqrtf(ss / (float)D + G.eps);
    if (lane < half) {
      x0 *= r * (h < NG ? gq0 : gk0);
      x1 *= r * (h < NG ? gq1 : gk1);
      // angle pos * theta^(-2i/D) in double, reduced to [-pi, pi] in double,
      // then cos/sin in single precision
      const double ang = (double)pos * ifreq;
      const double red2 = ang - 6.283185307179586476925286766559 * rint(ang * 0.15915494309189533576888376337251);
      float sf, cf;
      sincosf((float)red2, &sf, &cf);
      const float y0 = x0 * cf - x1 * sf, y1 = x1 * cf + x0 * sf;
      if (h < NG) {
        qs[h * D + lane] = y0 * G.attn_scale;
        qs[h * D + lane + half] = y1 * G.attn_scale;
      } else {
        knew[lane] = f2bf(y0);
        knew[lane + half] = f2bf(y1);
      }
    }
    if (h == NG) kv_append<D>(knew, Kc + new_row * D, lane, pos_ok);
  }
  __syncthreads();

  // scores s[h][r] = q_h . K_r (q already scaled); this lane's q columns live in registers
  float q[NG][8];
#pragma unroll
  for (int h = 0; h < NG; ++h) {
    const f32x4 q0 = *(const f32x4*)(qs + h * D + kc * 8);
    const f32x4 q1 = *(const f32x4*)(qs + h * D + kc * 8 + 4);
    q[h][0] = q0.x; q[h][1] = q0.y; q[h][2] = q0.z; q[h][3] = q0.w;
    q[h][4] = q1.x; q[h][5] = q1.y; q[h][6] = q1.z; q[h][7] = q1.w;
  }
  for (int p0 = 0; p0 < nk; p0 += RK) {
#pragma unroll
    for (int d = 0; d < RK; ++d) {
      const int p = p0 + d;
      if (p < nk) {
        const int r = p * KP + krow;
        u32x4 k = kr[d];
        if (last && r == T - 1) k = *(const u32x4*)(knew + kc * 8);
        const float kf[8] = {bf_lo(k.x), bf_hi(k.x), bf_lo(k.y), bf_hi(k.y),
                             bf_lo(k.z), bf_hi(k.z), bf_lo(k.w), bf_hi(k.w)};
        float s[NG];
#pragma unroll
        for (int h = 0; h < NG; ++h) {
          float t = kf[0] * q[h][0];
#pragma unroll
          for (int j = 1; j < 8; ++j) t = fmaf(kf[j], q[h][j], t);
          s[h] = KL == 16 ? row16_sum(t) : row8_sum(t);
        }
        if (kc == 0 && r < T) {
#pragma unroll
          for (int h = 0; h < NG; ++h) sc[h * SMAX + r] = s[h];
        }
        if (p + RK < nk) kr[d] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff(p + RK), 0, AUX_NT);
      }
    }
  }
  __syncthreads();

  // chunk-local softmax per head; numerators to pt[row][h], zero-padded to whole value passes
  const int Tp = nv * VP;
  for (int h = wave; h < NG; h += NWAVE) {
    float m = -INFINITY;
    for (int r = lane; r < T; r += 64) m = fmaxf(m, sc[h * SMAX + r]);
    m = wave_max(m);
    float l = 0.f;
    for (int r = lane; r < Tp; r += 64) {
      const float e = r < T ? expf(sc[h * SMAX + r] - m) : 0.f;
      pt[r * NG + h] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) {
      ml[2 * h] = m;
      ml[2 * h + 1] = l;
    }
  }
  __syncthreads();

  // early trigger (separate merge tasks only): the partials are the output
  // pass and the stores away; merge tasks that read first re-read stale words
  if ((op.pad & 2) && !op.aux && tid == 0) trigger_event(c);
  // o[h][2 columns] = sum over this lane's rows of p[r][h] V_r
  float o[NG][2];
#pragma unroll
  for (int h = 0; h < NG; ++h) o[h][0] = o[h][1] = 0.f;
  for (int p0 = 0; p0 < nv; p0 += RV) {
#pragma unroll
    for (int d = 0; d < RV; ++d) {
      const int p = p0 + d;
      if (p < nv) {
        const int r = p * VP + vrow;
        u32 v = vr[d];
        if (last && r == T - 1) v = *(const u32*)(vnew + vc * 2);
        const float v0 = bf_lo(v), v1 = bf_hi(v);
#pragma unroll
        for (int h = 0; h < NG; ++h) {
          const float w = pt[r * NG + h];
          o[h][0] = fmaf(w, v0, o[h][0]);
          o[h][1] = fmaf(w, v1, o[h][1]);
        }
        if (p + RV < nv) vr[d] = __builtin_amdgcn_raw_buffer_load_b32(rv, voff(p + RV), 0, AUX_NT);
      }
    }
  }
  if (VR == 2) {
    // two rows per wavefront instruction: add the upper half's columns to the lower half
#pragma unroll
    for (int h = 0; h < NG; ++h)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(o[h][j]), __float_as_uint(o[h][j]), false, false);
        o[h][j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      }
  }
  if (lane < VL) {
#pragma unroll
    for (int h = 0; h < NG; ++h) {
      float* dstp = red + (wave * NG + h) * D + vc * 2;
      dstp[0] = o[h][0];
      dstp[1] = o[h][1];
    }
  }
  __syncthreads();
  u64* part = op.out + ((((size_t)b * Hkv + gi) * C + ch) * NG) * (size_t)(D + 2);
  for (int j = tid; j < NG * D; j += NT) {
    const int h = j / D, dd = j - h * D;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) s += red[(w * NG + h) * D + dd];
    const float l = ml[2 * h + 1];
    st_t(part + (size_t)h * (D + 2) + 2 + dd, l > 0.f ? s / l : 0.f, a.tag);
  }
  if (tid < NG) {
    const float m = ml[2 * tid], l = ml[2 * tid + 1];
    st_t(part + (size_t)tid * (D + 2), l > 0.f ? m + logf(l) : -INFINITY, a.tag);
  }
  if (op.aux) {
    // fused merge: count this chunk's arrival; the last of the C chunks of
    // (b, gi) combines all partials (their words are tagged, so it can read
    // them as soon as they land)
    __syncthreads();
    if (tid == 0) {
      u32* arr = (u32*)op.aux + ((size_t)b * Hkv + gi) * kCounterStride;
      // the counter grows by C per step and a step's chunks all arrive before
      // the next step's (its O projection waits on every chunk), so the C-th
      // arrival of a step is the one that completes a multiple of C; this
      // holds for replayed graphs too, whose recorded epoch never advances
      const u32 old = __hip_atomic_fetch_add(gp(arr), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      c.flags[4] = (old + 1u) % (u32)C == 0u ? 1 : 0;
    }
    __syncthreads();
    if (c.flags[4]) merge_slice(c, op.out, (u64*)op.aux2, b, gi, 0, NG * D);
  }
}

// ---------------------------------------------------------------- routed experts
// Routing table of one layer (tagged words; ids and counts as exact floats):
//   [b*K*2 + 2j], [+1]      expert and weight of sequence b's j-th choice
//   TB = B*K*2: expert e at TB + e*(B+1): token count, then the count slots
//                (slot = b*K + j, in increasing b)
//   TA = TB + E*(B+1): number of active experts, then the active experts in
//                increasing id order
// The router (a GEMV over the normalised residual) leaves logits [B][E]; the
// dispatch wavefront turns them into this table, the pages' just-in-time
// expert scheduling ([Review], MoE notes).  Expert gate-up and down tasks
// are static per-worker slots that split the active experts' work between
// them; inactive experts cost nothing, and the task counts stay static.
DEV int route_tb(const Geom& G) { return G.B * G.topk * 2; }
DEV int route_ta(const Geom& G) { return route_tb(G) + G.E * (G.B + 1); }

// One wavefront (lanes 0..63): softmax over E <= 256 experts, top-K (ties to
// the lower id), renormalised weights, expert token lists, active list.
DEV void route_wave(const StepArgs& a, const OpDesc& op, int lane) {
  const Geom& G = *a.geom;
  const int B = G.B, E = G.E, K = G.topk;
  __shared__ int s_e[16 * 8];
  __shared__ float s_w[16 * 8];
  u64* route = op.out;
  for (int b = 0; b < B; ++b) {
    const u64* lg = op.in + (size_t)b * E;
    u64 w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = ld_raw(lg + min(lane + 64 * i, E - 1));
    float p[4];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      p[i] = e < E ? fix_t(w[i], lg + e, a) : -INFINITY;
      m = fmaxf(m, p[i]);
    }
    m = wave_max(m);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = lane + 64 * i < E ? expf(p[i] - m) : 0.f;
      sum += p[i];
    }
    sum = wave_sum(sum);
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = lane + 64 * i < E ? p[i] / sum : -1.f;
    float tot = 0.f, wj = 0.f;
    int ej = 0;
    for (int j = 0; j < K; ++j) {
      // this lane's best remaining (lower id wins ties), then the wavefront's
      float bv = -1.f;
      int be = 1 << 30;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (p[i] > bv) {
          bv = p[i];
          be = lane + 64 * i;
        }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oe = __shfl_xor(be, o);
        if (ov > bv || (ov == bv && oe < be)) {
          bv = ov;
          be = oe;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i == be) p[i] = -1.f;
      if (lane == j) {
        ej = be;
        wj = bv;
      }
      tot += bv;
    }
    if (lane < K) {
      s_e[b * K + lane] = ej;
      s_w[b * K + lane] = wj / tot;
      st_t(route + (size_t)(b * K + lane) * 2, (float)ej, a.tag);
      st_t(route + (size_t)(b * K + lane) * 2 + 1, wj / tot, a.tag);
    }
  }
  // one wavefront: its LDS writes above complete before the reads below
  // (no hardware barrier: in a launch-per-task workgroup only wave 0 is here)
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
  // the choice of this step for the host (mk_read_routing), B*K <= 64 records
  if (a.route_hist && lane < B * K) {
    const int rec = (((a.step & (kRouteHistSteps - 1)) * G.L + op.layer) * (B * K) + lane) * 2;
    g_u32* h = (g_u32*)a.route_hist;
    h[rec] = (u32)s_e[lane];
    h[rec + 1] = __float_as_uint(s_w[lane]);
  }
  u64* table = route + route_tb(G);
  u64* act = route + route_ta(G);
  int base = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    int cnt = 0;
    if (e < E) {
      for (int sl = 0; sl < B * K; ++sl)
        if (s_e[sl] == e) {
          st_t(table + (size_t)e * (B + 1) + 1 + cnt, (float)sl, a.tag);
          ++cnt;
        }
      st_t(table + (size_t)e * (B + 1), (float)cnt, a.tag);
    }
    const u64 mask = __ballot(cnt > 0);
    const int before = __builtin_popcountll(mask & ((1ull << lane) - 1ull));
    if (cnt > 0) st_t(act + 1 + base + before, (float)e, a.tag);
    base += __builtin_popcountll(mask);
  }
  if (lane == 0) st_t(act, (float)base, a.tag);
}

// All threads: xs[b][k] = rmsnorm(in[b]) * g for every sequence (fp32 in LDS).
DEV void moe_stage_norm(Ctx& c, const OpDesc& op, int tid, float* xs, float* red) {
  const StepArgs& a = *c.a;
  const int B = a.geom->B, H = op.K;
  const int wave = tid >> 6, lane = tid & 63;
  for (int b = 0; b < B; ++b) {
    const u64* in = op.in + (size_t)b * H;
    float ss = 0.f;
    for (int k0 = 0; k0 < H; k0 += NT * 8) {
      u64 w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = ld_raw(in + min(k0 + tid + i * NT, H - 1));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = k0 + tid + i * NT;
        if (k < H) {
          const float v = fix_t(w[i], in + k, a);
          xs[b * H + k] = v * ldg(op.g + k);
          ss += v * v;
        }
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) red[b * NWAVE + wave] = ss;
  }
  __syncthreads();
  for (int b = 0; b < B; ++b) {
    float t = 0.f;
#pragma unroll
    for (int w8 = 0; w8 < NWAVE; ++w8) t += red[b * NWAVE + w8];
    const float r = rsqrtf(t / (float)H + a.geom->eps);
    for (int k = tid; k < H; k += NT) xs[b * H + k] *= r;
  }
  __syncthreads();
}

// Items [i0, i1) of this slot task: item = (active expert act[item / U],
// unit item % U).  Loads the active list into LDS (ids as ints).
DEV int moe_load_active(Ctx& c, const u64* act, int* s_act, int tid) {
  const StepArgs& a = *c.a;
  const int n = (int)ld_t(act, a);
  for (int i = tid; i < n; i += NT) s_act[i] = (int)ld_t(act + 1 + i, a);
  __syncthreads();
  return n;
}
// Token list of expert e into LDS: s_tok[t] = slot (b*K + j); returns the count.
DEV int moe_load_tokens(Ctx& c, const u64* table, int e, int* s_tok, int tid) {
  const StepArgs& a = *c.a;
  const int B = a.geom->B;
  const u64* te = table + (size_t)e * (B + 1);
  __syncthreads();
  if (tid == 0) s_tok[16] = (int)ld_t(te, a);
  __syncthreads();
  const int n = s_tok[16];
  if (tid < n) s_tok[tid] = (int)ld_t(te + 1 + tid, a);
  __syncthreads();
  return n;
}

// The expert slots stream their items' weights through a ring whose slot of
// every load is a compile-time index: an item is NL loads per lane in a fixed
// order, NL a multiple of the ring depth, so the load DEPTH ahead of load l
// of an item is load l + DEPTH of the same item or load l + DEPTH - NL of the
// next one.  Items past the slot's share load out of range (zeros).
template <int NL>
struct MoeRing {
  static constexpr int DEPTH = NL % 8 == 0 ? 8 : 4;
  static_assert(NL % DEPTH == 0, "items are whole ring turns");
};

// Expert gate-up slot: for each item (expert e, 16-row unit u) and each token
// of e: act[slot][16u + r] = silu(gate_r . h) * (up_r . h).  Weights of one
// unit: 16 gate rows then 16 up rows, rows of H contiguous bf16.  Wavefront w
// computes outputs r = w and w + 8 (gate and up rows in the same wavefront);
// an item is NL = 4 * NCH loads per lane in the order (output, gate/up,
// 1 KB chunk of the row), NCH = H / 512 chunks per row.
template <int NCH>
DEV void moe_gu_items(Ctx& c, const OpDesc& op, const float* xs, const int* s_act, int* s_tok, int i0, int i1) {
  const StepArgs& a = *c.a;
  const Geom& G = *a.geom;
  const int K = G.topk, Ie = G.Ie, H = op.K;
  const int tid = task_tid(), wave = tid >> 6, lane = tid & 63;
  const int U = Ie / 16;
  constexpr int NL = 4 * NCH, DEPTH = MoeRing<NL>::DEPTH;
  // weights of every expert: [E][2*Ie][H]; unit u of e starts at row e*2*Ie + 32u
  const __amdgpu_buffer_rsrc_t rs = rsrc_u(op.w, (u32)G.E * 2u * (u32)Ie * (u32)H * 2u);
  auto rowbase = [&](int it) -> int {  // this wavefront's first row of item it (-1 past the share)
    if (it >= i1) return -1;
    const int e = s_act[it / U];
    return e * 2 * Ie + (it - (it / U) * U) * 32 + wave;
  };
  auto off = [&](int rb, int l) -> u32 {
    const int o = l / (2 * NCH), gu = (l / NCH) & 1, q = l % NCH;
    const int cc = q * 64 + lane;
    if (rb < 0 || cc * 8 >= H) return OOB;
    return (u32)(((rb + gu * 16 + 8 * o) * H + cc * 8) * 2);
  };
  int rb = rowbase(i0), rb_next = rowbase(i0 + 1);
  u32x4 buf[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) buf[d] = __builtin_amdgcn_raw_buffer_load_b128(rs, off(rb, d), 0, AUX_NT);
  int cur_e = -1, ntok = 0;
  int xoff[8], slot[8];
  const u64* table = op.aux + route_tb(G);
  for (int it = i0; it < i1; ++it) {
    const int e = s_act[it / U], u = it - (it / U) * U;
    if (e != cur_e) {
      ntok = moe_load_tokens(c, table, e, s_tok, tid);
      // uniform per workgroup: kept in scalar registers
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        slot[t] = __builtin_amdgcn_readfirstlane(s_tok[t < ntok ? t : 0]);
        xoff[t] = __builtin_amdgcn_readfirstlane((slot[t] / K) * H);  // the token's sequence row of xs
      }
      cur_e = e;
    }
    float acc[2][2][8];  // [output][gate/up][token]
#pragma unroll
    for (int o = 0; o < 2; ++o)
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[o][g2][t] = 0.f;
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      const int o = l / (2 * NCH), gu = (l / NCH) & 1, q = l % NCH, d = l % DEPTH;
      const int cc = q * 64 + lane;
      const u32x4 wv = buf[d];
      if (cc * 8 < H) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          if (t < ntok) {
            const f32x4 x0 = *(const f32x4*)(xs + xoff[t] + cc * 8);
            const f32x4 x1 = *(const f32x4*)(xs + xoff[t] + cc * 8 + 4);
            float sacc = bf_lo(wv.x) * x0.x;
            sacc = fmaf(bf_hi(wv.x), x0.y, sacc);
            sacc = fmaf(bf_lo(wv.y), x0.z, sacc);
            sacc = fmaf(bf_hi(wv.y), x0.w, sacc);
            sacc = fmaf(bf_lo(wv.z), x1.x, sacc);
            sacc = fmaf(bf_hi(wv.z), x1.y, sacc);
            sacc = fmaf(bf_lo(wv.w), x1.z, sacc);
            sacc = fmaf(bf_hi(wv.w), x1.w, sacc);
            acc[o][gu][t] += sacc;
          }
        }
      }
      buf[d] = __builtin_amdgcn_raw_buffer_load_b128(rs, l + DEPTH < NL ? off(rb, l + DEPTH) : off(rb_next, l + DEPTH - NL),
                                                     0, AUX_NT);
    }
    rb = rb_next;
    rb_next = rowbase(it + 2);
#pragma unroll
    for (int o = 0; o < 2; ++o)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (t < ntok) {
          const float gsum = wave_sum(acc[o][0][t]), usum = wave_sum(acc[o][1][t]);
          if (lane == 0) st_t(op.out + (size_t)slot[t] * Ie + u * 16 + wave + 8 * o, silu(gsum) * usum, a.tag);
        }
      }
  }
}

DEV void body_moe_gu(Ctx& c, const OpDesc& op) {
  const StepArgs& a = *c.a;
  const Geom& G = *a.geom;
  const int Ie = G.Ie, H = op.K;
  const int tid = task_tid();
  const int U = Ie / 16;
  float* xs = (float*)c.lds;                                   // [B][H]
  int* s_act = (int*)(c.lds + (size_t)kStageFloats * 4);       // [E]
  int* s_tok = s_act + 256;                                    // [16 + 1]
  float* red = (float*)(s_tok + 32);
  const u64* route = op.aux;
  wait_dep(c);
  const int n_act = moe_load_active(c, route + route_ta(G), s_act, tid);
  const int total = n_act * U, ns = op.ntasks, s = c.t.a0;
  const int i0 = (int)((long)s * total / ns), i1 = (int)((long)(s + 1) * total / ns);
  if (i1 <= i0) return;  // uniform across the workgroup
  moe_stage_norm(c, op, tid, xs, red);
  switch ((H / 8 + 63) / 64) {  // 1 KB chunks per row (the graph admits H <= 4096)
    case 1: moe_gu_items<1>(c, op, xs, s_act, s_tok, i0, i1); break;
    case 2: moe_gu_items<2>(c, op, xs, s_act, s_tok, i0, i1); break;
    case 3: moe_gu_items<3>(c, op, xs, s_act, s_tok, i0, i1); break;
    case 4: moe_gu_items<4>(c, op, xs, s_act, s_tok, i0, i1); break;
    case 5: moe_gu_items<5>(c, op, xs, s_act, s_tok, i0, i1); break;
    case 6: moe_gu_items<6>(c, op, xs, s_act, s_tok, i0, i1); break;
    case 7: moe_gu_items<7>(c, op, xs, s_act, s_tok, i0, i1); break;
    default: moe_gu_items<8>(c, op, xs, s_act, s_tok, i0, i1); break;
  }
}

// Expert down slot: for each item (expert e, 64-row unit u) and token of e:
// y[slot][64u + row] = W_down[e][64u + row] . act[slot].  Wavefront w takes
// rows w, w+8, ..., w+56; lanes read 16-byte chunks of the Ie-long rows.
DEV void body_moe_down(Ctx& c, const OpDesc& op) {
  const StepArgs& a = *c.a;
  const Geom& G = *a.geom;
  const int Ie = op.K, H = op.N;
  const int tid = task_tid(), wave = tid >> 6, lane = tid & 63;
  const int U = H / 64;
  float* xin = (float*)c.lds;                                  // [16 tokens][Ie]
  int* s_act = (int*)(c.lds + (size_t)kStageFloats * 4);
  int* s_tok = s_act + 256;
  const u64* route = op.aux;
  wait_dep(c);
  const int n_act = moe_load_active(c, route + route_ta(G), s_act, tid);
  const int total = n_act * U, ns = op.ntasks, s = c.t.a0;
  const int i0 = (int)((long)s * total / ns), i1 = (int)((long)(s + 1) * total / ns);
  if (i1 <= i0) return;
  const int nchunk = (Ie / 8 + 63) / 64;  // Ie = 768: 2
  const __amdgpu_buffer_rsrc_t rs = rsrc_u(op.w, (u32)G.E * (u32)H * (u32)Ie * 2u);
  constexpr int DEPTH = 8;
  const int NL = 8 * nchunk;  // loads per item per lane: 8 rows x nchunk chunks (a multiple of DEPTH)
  auto rowbase = [&](int it) -> int {  // this wavefront's first row of item it (-1 past the share)
    if (it >= i1) return -1;
    const int e = s_act[it / U];
    return e * H + (it - (it / U) * U) * 64 + wave;
  };
  // fill cursor: item fi (first row f_rb), row fr, chunk fq; no division per load
  int fi = i0, fr = 0, fq = 0, f_rb = rowbase(i0);
  auto fill = [&]() -> u32 {
    const int cc = fq * 64 + lane;
    const u32 off = (f_rb >= 0 && cc * 8 < Ie) ? (u32)(((f_rb + 8 * fr) * Ie + cc * 8) * 2) : OOB;
    if (++fq == nchunk) {
      fq = 0;
      if (++fr == 8) {
        fr = 0;
        f_rb = rowbase(++fi);
      }
    }
    return off;
  };
  u32x4 buf[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) buf[d] = __builtin_amdgcn_raw_buffer_load_b128(rs, fill(), 0, AUX_NT);
  int cur_e = -1, ntok = 0;
  int slot[8];  // the expert's token slots (uniform: scalar registers)
  const u64* table = route + route_tb(G);
  for (int it = i0; it < i1; ++it) {
    const int e = s_act[it / U], u = it - (it / U) * U;
    if (e != cur_e) {
      ntok = moe_load_tokens(c, table, e, s_tok, tid);
      // the expert's token inputs, all loads in flight before the tag checks
      constexpr int PT = 8 * 1024 / NT;  // words per thread for up to 8 tokens of Ie <= 1024
      u64 wv[PT];
      const int n = ntok * Ie;
#pragma unroll
      for (int i = 0; i < PT; ++i) {
        const int j = min(tid + i * NT, max(n - 1, 0));
        const int t = j / Ie, k = j - t * Ie;
        wv[i] = ld_raw(op.in + (size_t)s_tok[t] * Ie + k);
      }
#pragma unroll
      for (int i = 0; i < PT; ++i) {
        const int j = tid + i * NT;
        if (j < n) {
          const int t = j / Ie, k = j - t * Ie;
          xin[t * Ie + k] = fix_t(wv[i], op.in + (size_t)s_tok[t] * Ie + k, a);
        }
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) slot[t] = __builtin_amdgcn_readfirstlane(s_tok[t < ntok ? t : 0]);
      __syncthreads();
      cur_e = e;
    }
    float acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = 0.f;
    int r = 0, q = 0;  // consume cursor: row, chunk
    for (int l0 = 0; l0 < NL; l0 += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        {
          const int cc = q * 64 + lane;
          if (cc * 8 < Ie) {
            const u32x4 wv = buf[d];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              if (t < ntok) {
                const f32x4 x0 = *(const f32x4*)(xin + t * Ie + cc * 8);
                const f32x4 x1 = *(const f32x4*)(xin + t * Ie + cc * 8 + 4);
                float sacc = bf_lo(wv.x) * x0.x;
                sacc = fmaf(bf_hi(wv.x), x0.y, sacc);
                sacc = fmaf(bf_lo(wv.y), x0.z, sacc);
                sacc = fmaf(bf_hi(wv.y), x0.w, sacc);
                sacc = fmaf(bf_lo(wv.z), x1.x, sacc);
                sacc = fmaf(bf_hi(wv.z), x1.y, sacc);
                sacc = fmaf(bf_lo(wv.w), x1.z, sacc);
                sacc = fmaf(bf_hi(wv.w), x1.w, sacc);
                acc[t] += sacc;
              }
            }
          }
          if (q == nchunk - 1) {
            // row r complete: reduce and store per token
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              if (t < ntok) {
                const float v = wave_sum(acc[t]);
                if (lane == 0) st_t(op.out + (size_t)slot[t] * H + u * 64 + wave + 8 * r, v, a.tag);
              }
              acc[t] = 0.f;
            }
          }
          if (++q == nchunk) {
            q = 0;
            ++r;
          }
        }
        buf[d] = __builtin_amdgcn_raw_buffer_load_b128(rs, fill(), 0, AUX_NT);
      }
    }
  }
}

// x_out[b][h] = x_res[b][h] + sum_j w[b][j] * y[b*K + j][h] for the tile's rows.
DEV void body_combine(Ctx& c, const OpDesc& op) {
  const StepArgs& a = *c.a;
  const Geom& G = *a.geom;
  const int B = G.B, K = G.topk, H = op.N;
  const int r0 = c.t.a1, nr = c.t.a2;
  wait_dep(c);
  for (int j = task_tid(); j < B * nr; j += NT) {
    const int b = j / nr, h = r0 + (j - b * nr);
    // residual, K weights and K expert outputs: one batch of loads
    const u64* rp = op.res + (size_t)b * H + h;
    const u64 wr = ld_raw(rp);
    u64 ww[8], wy[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int kk = min(k, K - 1);
      ww[k] = ld_raw(op.aux + (size_t)(b * K + kk) * 2 + 1);
      wy[k] = ld_raw(op.in + (size_t)(b * K + kk) * H + h);
    }
    float v = fix_t(wr, rp, a);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < K) {
        const float wk = fix_t(ww[k], op.aux + (size_t)(b * K + k) * 2 + 1, a);
        v = fmaf(wk, fix_t(wy[k], op.in + (size_t)(b * K + k) * H + h, a), v);
      }
    }
    st_t(op.out + (size_t)b * H + h, v, a.tag);
  }
}

DEV void body_attn(Ctx& c, const OpDesc& op) {
  const Geom& G = *c.a->geom;
  const bool d128 = G.D == 128;
  switch (G.G) {
    case 1: d128 ? attn_chunk<1, 128>(c, op) : attn_chunk<1, 64>(c, op); break;
    case 2: d128 ? attn_chunk<2, 128>(c, op) : attn_chunk<2, 64>(c, op); break;
    case 4: d128 ? attn_chunk<4, 128>(c, op) : attn_chunk<4, 64>(c, op); break;
    default: d128 ? attn_chunk<8, 128>(c, op) : attn_chunk<8, 64>(c, op); break;
  }
}

}  // namespace mk
