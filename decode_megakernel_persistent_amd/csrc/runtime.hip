// runtime.hip - kernels and the host side of the C ABI (include/mk.h).
//
// Persistent mode: one cooperative launch of mk_worker with one 512-thread
// workgroup per compute unit (the 140 KB LDS request leaves room for only one
// per CU) plus a one-wavefront mk_dispatch kernel on an internal second
// stream, as the MPK pages split worker and scheduler kernels onto two
// streams (page "Mirage Persistent Kernel (MPK)", section 5.1).  Each worker
// walks its statically assigned task list in increasing id order; every task
// issues its first weight loads, waits on its dependency event, runs its body
// and triggers its event (MPK abstract: decentralised in-kernel scheduling;
// review page 2512.22219, section 2.4).
//
// Launch-per-task mode: the same bodies, one launch of mk_lpt per
// (event range, operator) run in BFS order; stream order replaces the waits.
#include <dlfcn.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "device.h"
#include "graph.h"

// Translation units.  The library is compiled from this one file several
// times in parallel: with MK_UNIT_NB=v, the kernels of batch variant v (and,
// for v = 1, the dispatch kernel); with MK_UNIT_HOST, the host side, which
// only declares the kernels.  Without either macro the file is one unit.
#if !defined(MK_UNIT_NB) && !defined(MK_UNIT_HOST)
#define MK_UNIT_ALL 1
#endif

namespace mk {

// ---------------------------------------------------------------- kernels
template <int NB, bool MULTI>
DEV void run_task(const StepArgs& a, int id, int agent, bool lpt, char* lds, int* flags, const int* pos, int next) {
  Ctx c;
  c.a = &a;
  c.t = a.tasks[id];
  c.id = id;
  c.agent = agent;
  c.lpt = lpt;
  c.lds = lds;
  c.flags = flags;
  c.pos = pos;
  c.next = next;
  if (threadIdx.x == 0) {
    flags[5] = 0;  // not triggered yet (read after the body's barriers)
    if (a.trace_on == 2) flags[kFlagEntryClock] = (int)(u32)wall_clock64();
  }
  const OpDesc& op = a.ops[c.t.op];
  switch (op.kind) {
    case OP_QKV:
    case OP_OPROJ:
    case OP_GATEUP:
    case OP_DOWN:
    case OP_LMHEAD:
    case OP_ROUTER:
      if constexpr (NB == kMfmaVariant) gemv_mfma(c, op);
      else if constexpr (NB == kRingVariant) {
        if (op.pad & 4) gemv_ring_any(c, op);
        else gemv_valu_any<1>(c, op);
      } else gemv_valu_any<NB>(c, op);
      break;
    case OP_ATTN:
      body_attn(c, op);
      break;
    case OP_MERGE:
      wait_dep(c);
      body_merge(c, op);
      break;
    case OP_ROUTE:
      // normally on the dispatch wavefront; in a launch-per-task workgroup wave 0 routes
      wait_dep(c);
      if (threadIdx.x < 64) route_wave(a, op, threadIdx.x);
      break;
    case OP_MOE_GU:
      body_moe_gu(c, op);
      break;
    case OP_MOE_DOWN:
      body_moe_down(c, op);
      break;
    case OP_COMBINE:
      body_combine(c, op);
      break;
    case OP_EMBED:
      wait_dep(c);
      body_embed(c, op);
      break;
    default:
      wait_dep(c);
      break;
  }
  // greedy candidates of an lm_head tile, from the row results still in LDS
  // (one copy of this code per kernel, not one per GEMV shape)
  if constexpr (MULTI) {
    if (op.kind == OP_LMHEAD && a.cand) {
      if constexpr (NB == kMfmaVariant) lm_candidates(c, mfma_rows(c), c.t.a2, mfma_scales(c), a.geom->B);
      else if constexpr (NB == kRingVariant) {
        if (op.pad & 4) {
          __syncthreads();  // the ring epilogue's row sums, written by other threads
          lm_candidates(c, ring_rows(c), c.t.a2, valu_scales(c, 1), 1);
        } else {
          lm_candidates(c, valu_rows(c), c.t.a2, valu_scales(c, 1), 1);
        }
      } else lm_candidates(c, valu_rows(c), c.t.a2, valu_scales(c, NB), NB);
    }
  }
  finish(c);
}

// Entry checks of every worker / launch; also copies the step's positions
// (at most 16) into LDS, so that no task pays a memory round trip for them.
DEV bool entry_ok(const StepArgs& a, int* flags, int* pos) {
  if ((int)threadIdx.x < a.geom->B) pos[threadIdx.x] = a.positions[threadIdx.x];
  if (threadIdx.x == 0) {
    int ok = 1;
    if (a.geom->magic != a.magic) {
      u32 z = 0;
      __hip_atomic_compare_exchange_strong(a.status + ST_ERROR, &z, (u32)ERR_CONFIG, __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      ok = 0;
    }
    // a failed step leaves the error word set until mk_check clears it
    if (__hip_atomic_load(a.status + ST_ERROR, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) ok = 0;
    flags[0] = ok ? 0 : 1;
    flags[kFrAhead] = -1;  // no LDS-ring run-ahead pending
  }
  __syncthreads();
  return flags[0] == 0;
}

// Register cap: two worker wavefronts per SIMD must leave room for the
// dispatch wavefront (8 VGPRs) on whichever CU it runs, or the worker
// workgroup of that CU could not become resident.
// Two variants: MULTI = false runs one step (the plain task loop); MULTI =
// true runs a.n_steps greedy steps, with the lm_head argmax candidates and the
// token feedback.  Separate instantiations keep the outer step loop and the
// candidate code out of the one-step kernel, where they measurably slowed the
// bodies (register and instruction-cache pressure, ~1.3% of a step).
// (the attribute takes a literal constant, so the unit macro picks the cap)
#if defined(MK_UNIT_NB) && (MK_UNIT_NB == 1 || MK_UNIT_NB == 17)
#define MK_WORKER_VGPRS kWorkerVgprsB1
#else
#define MK_WORKER_VGPRS kWorkerVgprs
#endif
template <int NB, bool MULTI>
__global__ void __launch_bounds__(NT, 1) __attribute__((amdgpu_num_vgpr(MK_WORKER_VGPRS))) mk_worker(StepArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int flags[kFlagWords];
  __shared__ int pos[16];
  // arrival and completion count one per step, so that the dispatch
  // wavefront's targets (workers x persistent steps so far) hold for any mix
  // of launch lengths
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(a.status + ST_ARRIVED, (u32)a.n_steps, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (entry_ok(a, flags, pos)) {
    const int w = blockIdx.x;
    if constexpr (!MULTI) {
      const int kend = a.wl_off[w + 1];
      for (int k = a.wl_off[w]; k < kend; ++k) {
        if (threadIdx.x == 0)
          __hip_atomic_store(a.progress + w, (u32)a.wl_ids[k] + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        run_task<NB, false>(a, a.wl_ids[k], w, false, lds, flags, pos, k + 1 < kend ? a.wl_ids[k + 1] : -1);
        __syncthreads();
        if (lds_rd(flags)) break;  // (not ordered behind the LDS-ring loader's loads in flight)
      }
    } else {
      // Multi-step decode: the same task list once per step, with the step's
      // epoch (event targets), data tag and positions, advanced in the
      // kernel's own argument copy.  A step's embedding waits on the previous
      // step's lm_head event, so a worker may run ahead into the next step
      // only as far as the events allow.
      const int n = a.n_steps;
      for (int s = 0; s < n; ++s) {
        if (s > 0) {
          if ((int)threadIdx.x < a.geom->B) pos[threadIdx.x] = a.positions[threadIdx.x] + s;
          __syncthreads();
        }
        const int kend = a.wl_off[w + 1];
        for (int k = a.wl_off[w]; k < kend; ++k) {
          if (threadIdx.x == 0)
            __hip_atomic_store(a.progress + w, (u32)a.wl_ids[k] + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          run_task<NB, true>(a, a.wl_ids[k], w, false, lds, flags, pos, k + 1 < kend ? a.wl_ids[k + 1] : -1);
          __syncthreads();
          if (lds_rd(flags)) break;
        }
        if (flags[0]) break;
        if (s + 1 < n) {
          a.epoch += 1u;
          a.tag += 1u;
          a.step += 1;
        }
      }
      // the last step's greedy tokens
      if (a.tokens_out && w == 0 && !flags[0] && a.geom->lm_event >= 0) {
        Ctx c;
        c.a = &a;
        c.id = -1;
        c.agent = w;
        c.lpt = false;
        c.lds = lds;
        c.flags = flags;
        c.pos = pos;
        c.next = -1;
        int* tk = (int*)lds;
        lm_argmax(c, a.epoch + 1u, a.tag, 0, a.geom->B, tk);
        if ((int)threadIdx.x < a.geom->B && !flags[0])
          a.tokens_out[(size_t)(n - 1) * a.geom->B + threadIdx.x] = tk[threadIdx.x];
      }
    }
    if (threadIdx.x == 0 && !flags[0])
      __hip_atomic_store(a.progress + w, 0xFFFFFFFFu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(a.status + ST_DONE, (u32)a.n_steps, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int NB>
__global__ void __launch_bounds__(NT, 1) mk_lpt(StepArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int flags[kFlagWords];
  __shared__ int pos[16];
  if (entry_ok(a, flags, pos)) run_task<NB, false>(a, a.lpt_first + (int)blockIdx.x, -1, true, lds, flags, pos, -1);
}

#if defined(MK_UNIT_ALL) || (defined(MK_UNIT_NB) && MK_UNIT_NB == 1)
// The dispatch wavefront: runs the dispatcher's own task list (work-list
// routing of routed-expert layers), then watches the workers until every one
// has finished the step, raising the abort flag if that takes longer than the
// watchdog budget.  Bounded to 64 VGPRs (8 waves per SIMD): two worker
// wavefronts of up to 224 registers and this one must share a SIMD's 512.
// Graphs without dispatcher tasks (dense models) launch mk_dispatch_dense,
// the same wavefront without the routing code, bounded to 32 VGPRs, which
// leaves two worker wavefronts 240 registers each.
template <bool ROUTED>
DEV void dispatch_body(StepArgs& a) {
  const int W = a.n_workers;
  // launch-per-task steps advance the epoch but not the workers' arrival and
  // completion counts, so the targets count persistent steps only
  const u32 target = (u32)W * (a.run_base + (u32)a.n_steps);
  u64 t0 = wall_clock64();
  // entry handshake: every worker workgroup must become resident while the
  // others wait for it; give it a short budget, then report and abort
  const u64 resident_budget = a.budget / 8 + 1;
  for (;;) {
    u32 arrived = __hip_atomic_load(a.status + ST_ARRIVED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (arrived >= target) break;
    if (__hip_atomic_load(a.status + ST_ABORT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;
    if (wall_clock64() - t0 > resident_budget) {
      if (threadIdx.x == 0) {
        u32 z = 0;
        if (__hip_atomic_compare_exchange_strong(a.status + ST_ERROR, &z, (u32)ERR_NOT_RESIDENT, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
          __hip_atomic_store(a.status + ST_SEEN, arrived, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(a.status + ST_TARGET, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __hip_atomic_store(a.status + ST_ABORT, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      return;
    }
    __builtin_amdgcn_s_sleep(16);
  }
  // the dispatcher's own tasks (routing of routed-expert layers), in id order
  if constexpr (ROUTED) {
    __shared__ int flags[64];
    if (threadIdx.x < 64) flags[threadIdx.x] = 0;
    __syncthreads();
    const u32 epoch0 = a.epoch, tag0 = a.tag;
    for (int s = 0; s < a.n_steps; ++s) {
      StepArgs& as = a;
      as.epoch = epoch0 + (u32)s;
      as.tag = tag0 + (u32)s;
      as.step = s;
      for (int k = a.wl_off[W]; k < a.wl_off[W + 1]; ++k) {
        const int id = a.wl_ids[k];
        if (threadIdx.x == 0)
          __hip_atomic_store(a.progress + W, (u32)id + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        Ctx c;
        c.a = &as;
        c.t = a.tasks[id];
        c.id = id;
        c.agent = W;
        c.lpt = false;
        c.lds = nullptr;
        c.flags = flags;
        c.pos = nullptr;
        c.next = -1;
        if (threadIdx.x == 0) {
          flags[5] = 0;
          if (a.trace_on == 2) flags[kFlagEntryClock] = (int)(u32)wall_clock64();
        }
        wait_dep(c);
        if (flags[0]) return;
        route_wave(as, a.ops[c.t.op], threadIdx.x);
        finish(c);
        __syncthreads();
      }
    }
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(a.progress + W, 0xFFFFFFFFu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  t0 = wall_clock64();
  for (;;) {
    u32 done = __hip_atomic_load(a.status + ST_DONE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done >= target) break;
    if (__hip_atomic_load(a.status + ST_ABORT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
    if (wall_clock64() - t0 > (u64)(3 + a.n_steps) * a.budget) {
      if (threadIdx.x == 0) report_timeout(a, -1, -1, done, target);
      break;
    }
    __builtin_amdgcn_s_sleep(127);
  }
}
__global__ void __launch_bounds__(64, 8) mk_dispatch(StepArgs a) { dispatch_body<true>(a); }
__global__ void __launch_bounds__(64, 16) mk_dispatch_dense(StepArgs a) { dispatch_body<false>(a); }
#else
__global__ void __launch_bounds__(64, 8) mk_dispatch(StepArgs a);
__global__ void __launch_bounds__(64, 16) mk_dispatch_dense(StepArgs a);
#endif

#if defined(MK_UNIT_NB)
// this unit's kernels
template __global__ void mk_worker<MK_UNIT_NB, false>(StepArgs);
template __global__ void mk_worker<MK_UNIT_NB, true>(StepArgs);
template __global__ void mk_lpt<MK_UNIT_NB>(StepArgs);
#endif
#if defined(MK_UNIT_HOST)
// defined in the kernel units
extern template __global__ void mk_worker<1, false>(StepArgs);
extern template __global__ void mk_worker<2, false>(StepArgs);
extern template __global__ void mk_worker<3, false>(StepArgs);
extern template __global__ void mk_worker<4, false>(StepArgs);
extern template __global__ void mk_worker<kMfmaVariant, false>(StepArgs);
extern template __global__ void mk_worker<kRingVariant, false>(StepArgs);
extern template __global__ void mk_worker<1, true>(StepArgs);
extern template __global__ void mk_worker<2, true>(StepArgs);
extern template __global__ void mk_worker<3, true>(StepArgs);
extern template __global__ void mk_worker<4, true>(StepArgs);
extern template __global__ void mk_worker<kMfmaVariant, true>(StepArgs);
extern template __global__ void mk_worker<kRingVariant, true>(StepArgs);
extern template __global__ void mk_lpt<1>(StepArgs);
extern template __global__ void mk_lpt<2>(StepArgs);
extern template __global__ void mk_lpt<3>(StepArgs);
extern template __global__ void mk_lpt<4>(StepArgs);
extern template __global__ void mk_lpt<kMfmaVariant>(StepArgs);
extern template __global__ void mk_lpt<kRingVariant>(StepArgs);
#endif

}  // namespace mk

// ==================================================================== host
#if defined(MK_UNIT_ALL) || defined(MK_UNIT_HOST)
namespace mk {
// Kernel variants: 1..4 = VALU GEMV for that batch, kMfmaVariant = MFMA GEMV
// (any batch up to 16), kRingVariant = batch 1 with the LDS weight ring.
// Separate instantiations keep each one's register allocation to the GEMV it
// actually runs (compiling the ring into the batch-1 worker cost ~3% of its
// step even with the ring unused).
typedef void (*kernel_fn)(StepArgs);
static const void* worker_fn(int v, bool multi) {
  if (multi) {
    switch (v) {
      case 1: return (const void*)mk_worker<1, true>;
      case 2: return (const void*)mk_worker<2, true>;
      case 3: return (const void*)mk_worker<3, true>;
      case 4: return (const void*)mk_worker<4, true>;
      case kRingVariant: return (const void*)mk_worker<kRingVariant, true>;
      default: return (const void*)mk_worker<kMfmaVariant, true>;
    }
  }
  switch (v) {
    case 1: return (const void*)mk_worker<1, false>;
    case 2: return (const void*)mk_worker<2, false>;
    case 3: return (const void*)mk_worker<3, false>;
    case 4: return (const void*)mk_worker<4, false>;
    case kRingVariant: return (const void*)mk_worker<kRingVariant, false>;
    default: return (const void*)mk_worker<kMfmaVariant, false>;
  }
}
static const void* lpt_fn(int v) {
  switch (v) {
    case 1: return (const void*)mk_lpt<1>;
    case 2: return (const void*)mk_lpt<2>;
    case 3: return (const void*)mk_lpt<3>;
    case 4: return (const void*)mk_lpt<4>;
    case kRingVariant: return (const void*)mk_lpt<kRingVariant>;
    default: return (const void*)mk_lpt<kMfmaVariant>;
  }
}
static int kernel_variant(const Graph& G) {
  return G.gemv == MK_GEMV_MFMA ? kMfmaVariant : G.geom.ring_u > 0 ? kRingVariant : G.B;
}

}  // namespace mk

using namespace mk;

// ---------------------------------------------------------------- static scratch
// The scratch of mk_decode_step_noalloc: a file-scope device array, one copy
// on every GPU the library runs on, held until the process ends.  Host code
// never uses its name as an address: static_scratch() looks the device copy
// up once per device with hipGetSymbolAddress (at weight loading, the device
// current) and keeps the pointer.
static constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// Clear n_words words of a scratch state region (counters, status, progress,
// arrival counters), the status word `none_word` set to 0xFFFFFFFF.  A kernel
// rather than a memset, so that a caller may capture the call in a graph.
__global__ void __launch_bounds__(256) mk_clear_state(uint32_t* p, uint32_t n_words, uint32_t none_word) {
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n_words; i += gridDim.x * 256u)
    p[i] = i == none_word ? 0xFFFFFFFFu : 0u;
}

// A plain streaming read of `bytes` bytes (16-byte loads, grid-stride): the
// rate a simple kernel reaches on this machine, reported beside the roofline.
// Each workgroup leaves the XOR of what it read in sink[block].
__global__ void __launch_bounds__(512) mk_stream_read_kernel(const mk::u32x4* p, uint64_t n16, uint32_t* sink) {
  uint32_t acc = 0;
  for (uint64_t i = blockIdx.x * 512ull + threadIdx.x; i < n16; i += (uint64_t)gridDim.x * 512ull) {
    const mk::u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[512];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 256; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] ^= red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

namespace {

#define HIPCHK(x)                                                                   \
  do {                                                                              \
    hipError_t e_ = (x);                                                            \
    if (e_ != hipSuccess) {                                                         \
      set_error(std::string(#x) + " failed: " + hipGetErrorString(e_));             \
      return MK_ERR_HIP;                                                            \
    }                                                                               \
  } while (0)

std::string tensor_name_list(const mk_model_shape& s, std::vector<std::pair<std::string, std::pair<int64_t, int64_t>>>* out) {
  const int64_t H = s.hidden, D = s.head_dim, Hq = s.n_q_heads, Hkv = s.n_kv_heads;
  auto add = [&](const std::string& n, int64_t r, int64_t c) { out->push_back({n, {r, c}}); };
  add("embed", s.vocab, H);
  for (int l = 0; l < s.n_layers; ++l) {
    std::string p = "layers." + std::to_string(l) + ".";
    add(p + "in_norm", H, 1);
    add(p + "wq", Hq * D, H);
    add(p + "wk", Hkv * D, H);
    add(p + "wv", Hkv * D, H);
    add(p + "q_norm", D, 1);
    add(p + "k_norm", D, 1);
    add(p + "wo", H, Hq * D);
    add(p + "post_norm", H, 1);
    if (s.n_experts == 0) {
      add(p + "w_gate", s.intermediate, H);
      add(p + "w_up", s.intermediate, H);
      add(p + "w_down", H, s.intermediate);
    } else {
      add(p + "router", s.n_experts, H);
      for (int e = 0; e < s.n_experts; ++e) {
        std::string q = p + "experts." + std::to_string(e) + ".";
        add(q + "w_gate", s.expert_intermediate, H);
        add(q + "w_up", s.expert_intermediate, H);
        add(q + "w_down", H, s.expert_intermediate);
      }
    }
  }
  add("final_norm", H, 1);
  if (!s.tied_embeddings) add("lm_head", s.vocab, H);
  return "";
}

constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices] = {};
uint32_t g_static_tag[kMaxDevices] = {};  // next data tag on each device's static scratch (0: never used)

// Device address of the static scratch on device `dev` (the current device).
mk_status static_scratch(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("static scratch: device index out of range");
    return MK_ERR_ARG;
  }
  std::lock_guard<std::mutex> lk(g_static_mu);
  if (!g_static_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      set_error(std::string("static scratch: hipGetSymbolAddress failed: ") + hipGetErrorString(e));
      return MK_ERR_HIP;
    }
    g_static_ptr[dev] = p;
  }
  *out = g_static_ptr[dev];
  return MK_OK;
}

// The scratch the graph's last step ran on (what mk_check and the readers read).
char* active_scratch(const mk_graph* g) { return (char*)(g->last_static ? g->static_scr : g->scratch); }

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) return 0;
  return p.multiProcessorCount;
}

// Kernel arguments of one launch (epoch and tag taken from the graph handle).
// With on_static, the step runs on the library's static scratch and the
// operator table whose buffers point into it (mk_decode_step_noalloc).
StepArgs step_args(mk_graph* g, const int32_t* d_tokens, const int32_t* d_positions, const mk_kv_cache* kv,
                   float* d_logits, int32_t* d_tokens_out, int32_t n_steps, bool on_static = false) {
  Graph& G = *g->G;
  char* arena = (char*)g->arena;
  char* scr = (char*)(on_static ? g->static_scr : g->scratch);
  StepArgs a;
  std::memset(&a, 0, sizeof a);
  a.geom = (const Geom*)(arena + G.off_geom);
  a.ops = (const OpDesc*)(arena + (on_static ? G.off_ops_static : G.off_ops));
  a.tasks = (const Task*)(arena + G.off_tasks);
  a.events = (const Event*)(arena + G.off_events);
  a.wl_off = (const int32_t*)(arena + G.off_wloff);
  a.wl_ids = (const int32_t*)(arena + G.off_wlids);
  a.counters = (u32*)(scr + G.off_counters);
  a.status = (u32*)(scr + G.off_status);
  a.progress = (u32*)(scr + G.off_progress);
  a.tokens = d_tokens;
  a.positions = d_positions;
  a.kv_k = (uint16_t*)kv->k;
  a.kv_v = (uint16_t*)kv->v;
  a.page_table = kv->page_table;
  a.page_shift = -1;
  for (int s = 0; kv->page_size > 0 && s < 31; ++s)
    if ((1 << s) == kv->page_size) a.page_shift = s;
  a.n_pages = kv->n_pages;
  a.logits = d_logits;
  a.trace = (mk_trace_rec*)g->trace;
  a.budget = g->budget_ticks;
  a.epoch = g->epoch;
  a.tag = g->tag;
  a.magic = G.geom.magic;
  a.trace_on = G.opts.trace;
  a.n_workers = G.W;
  a.n_steps = n_steps;
  a.run_base = g->persistent_steps;
  a.step = 0;
  a.tokens_out = d_tokens_out;
  a.cand = (u64*)(scr + G.off_cand);
  a.route_hist = G.off_route_hist >= 0 ? (u64*)(scr + G.off_route_hist) : nullptr;
  return a;
}

// Checks of a caller's cache description against the graph (see mk_kv_cache).
bool kv_ok(const Graph& G, const mk_kv_cache* kv, const char* who) {
  if (!kv || !kv->k || !kv->v) {
    set_error(std::string(who) + ": null KV cache");
    return false;
  }
  if (kv->capacity != G.cap) {
    set_error(std::string(who) + ": kv capacity " + std::to_string(kv->capacity) + " differs from the graph's max_ctx " +
              std::to_string(G.cap));
    return false;
  }
  if (kv->reserved != 0 || kv->page_size < 0) {
    set_error(std::string(who) + ": bad KV cache description (reserved field or page size)");
    return false;
  }
  if (kv->page_size == 0) return true;
  const int64_t P = kv->page_size;
  if (P < 16 || (P & (P - 1)) || G.cap % P) {
    set_error(std::string(who) + ": page_size must be a power of two >= 16 dividing the capacity");
    return false;
  }
  if (!kv->page_table || kv->n_pages <= 0) {
    set_error(std::string(who) + ": paged KV cache needs a page table and n_pages > 0");
    return false;
  }
  const int64_t pool = (int64_t)kv->n_pages * G.shape.n_kv_heads * P * G.shape.head_dim * 2;
  if (pool >= (1LL << 32)) {
    set_error(std::string(who) + ": one layer's KV pool must stay below 4 GiB");
    return false;
  }
  return true;
}

// The launch-per-task sequence of one step on `stream`: one mk_lpt launch per
// (event range, operator) in BFS order, or one per task.
mk_status launch_lpt(mk_graph* g, StepArgs a, hipStream_t stream) {
  Graph& G = *g->G;
  const void* fn = lpt_fn(kernel_variant(G));
  for (size_t i = 0; i < G.launch_first.size(); ++i) {
    const int32_t first = G.launch_first[i], count = G.launch_count[i];
    if (g->per_task_launch) {
      for (int32_t k = 0; k < count; ++k) {
        a.lpt_first = first + k;
        void* kargs[] = {&a};
        HIPCHK(hipLaunchKernel(fn, dim3(1), dim3(NT), kargs, kLdsBytes, stream));
      }
    } else {
      a.lpt_first = first;
      void* kargs[] = {&a};
      HIPCHK(hipLaunchKernel(fn, dim3(count), dim3(NT), kargs, kLdsBytes, stream));
    }
  }
  return MK_OK;
}

// Enqueue one launch (persistent: the worker grid and the dispatch wavefront;
// launch-per-task: its launch sequence) with the given arguments.
mk_status launch_step(mk_graph* g, StepArgs& a, bool multi, hipStream_t stream) {
  Graph& G = *g->G;
  const int nb = kernel_variant(G);
  if (g->mode == MK_PERSISTENT) {
    hipStream_t side = (hipStream_t)g->side_stream;
    const bool watch = !G.opts.no_watchdog;
    // The worker grid is submitted before the dispatch wavefront, which
    // still runs beside it (its stream waits only on ev_a, recorded ahead of
    // the workers).  Submitted the other way round, the step measured ~0.8%
    // slower.
    if (watch) HIPCHK(hipEventRecord((hipEvent_t)g->ev_a, stream));
    void* kargs[] = {&a};
    hipError_t e = hipLaunchCooperativeKernel(worker_fn(nb, multi), dim3(G.W), dim3(NT), kargs, kLdsBytes, stream);
    if (e == hipErrorCooperativeLaunchTooLarge) {
      (void)hipGetLastError();
      set_error("mk_decode_step: " + std::to_string(G.W) + " workers cannot be co-resident on this device");
      return MK_ERR_NOT_RESIDENT;
    }
    if (e != hipSuccess) {
      set_error(std::string("mk_decode_step: cooperative launch failed: ") + hipGetErrorString(e));
      return MK_ERR_HIP;
    }
    if (watch) {
      HIPCHK(hipStreamWaitEvent(side, (hipEvent_t)g->ev_a, 0));
      if (G.wl_off[G.W + 1] > G.wl_off[G.W]) hipLaunchKernelGGL(mk_dispatch, dim3(1), dim3(64), 0, side, a);
      else hipLaunchKernelGGL(mk_dispatch_dense, dim3(1), dim3(64), 0, side, a);
      HIPCHK(hipGetLastError());
      HIPCHK(hipEventRecord((hipEvent_t)g->ev_b, side));
      HIPCHK(hipStreamWaitEvent(stream, (hipEvent_t)g->ev_b, 0));
    }
    return MK_OK;
  }
  return launch_lpt(g, a, stream);
}

}  // namespace

extern "C" {

mk_status mk_build_graph(const mk_model_shape* shape, int32_t batch, int32_t max_ctx, const mk_build_opts* opts,
                         mk_graph** out) {
  if (!shape || !out) {
    set_error("mk_build_graph: null argument");
    return MK_ERR_ARG;
  }
  *out = nullptr;
  mk_build_opts o{};
  if (opts) o = *opts;
  if (o.mode != MK_PERSISTENT && o.mode != MK_LAUNCH_PER_TASK) {
    set_error("mk_build_graph: unknown mode");
    return MK_ERR_ARG;
  }
  int32_t W = o.num_workers;
  if (W <= 0) {
    W = device_cu_count();
    if (W <= 0) W = 256;  // gfx950 compute units, when no device is visible
  }
  std::string err;
  Graph* G = compile_decoder(*shape, batch, max_ctx, o, W, o.no_fusion == 0, &err);
  if (!G) {
    set_error("mk_build_graph: " + err);
    return MK_ERR_SHAPE;
  }
  mk_graph* g = new mk_graph();
  g->G = G;
  g->mode = o.mode;
  g->per_task_launch = o.per_task_launch;
  *out = g;
  return MK_OK;
}

mk_status mk_workspace_size(const mk_graph* g, size_t* arena_bytes, size_t* scratch_bytes, size_t* trace_bytes) {
  if (!g || !g->G) {
    set_error("mk_workspace_size: null graph");
    return MK_ERR_ARG;
  }
  if (arena_bytes) *arena_bytes = (size_t)g->G->arena_bytes;
  if (scratch_bytes) *scratch_bytes = (size_t)g->G->scratch_bytes;
  if (trace_bytes) *trace_bytes = (size_t)g->G->trace_bytes;
  return MK_OK;
}

// MFMA weight fragments: rows [row0, row0 + nrows) of a [rows, K] bf16 tensor
// become 1 KB fragments of 16 rows x 32 columns, fragment (g, kb) at
// ((g * K/32 + kb) * 64 + lane) * 16 bytes, lane l holding row 16g + l%16,
// columns 32kb + 8(l/16) .. +8 (the A-operand layout of
// v_mfma_f32_16x16x32_bf16).  Done on the host in batches of 1024 rows.
static bool swizzle16(const CopyJob& cj, const mk_tensor* t, const char* src, char* arena, hipStream_t stream) {
  const int64_t K = t->cols, KB = K / 32, ngroups = cj.nrows / 16;
  if (cj.nrows % 16 || K % 32) {
    set_error("mk_load_weights: MFMA fragments need rows in multiples of 16 and K in multiples of 32");
    return false;
  }
  const int64_t GB = 64;  // groups per batch
  std::vector<uint16_t> in((size_t)(GB * 16 * K)), out(in.size());
  const unsigned nth = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  for (int64_t g0 = 0; g0 < ngroups; g0 += GB) {
    const int64_t ng = std::min(GB, ngroups - g0);
    const size_t bytes = (size_t)(ng * 16 * K * 2);
    const char* s = src + (size_t)(g0 * 16 * K * 2);
    if (t->on_device) {
      if (hipMemcpy(in.data(), s, bytes, hipMemcpyDeviceToHost) != hipSuccess) return false;
    } else {
      std::memcpy(in.data(), s, bytes);
    }
    std::vector<std::thread> pool;
    for (unsigned w = 0; w < nth; ++w)
      pool.emplace_back([&, w] {
        for (int64_t g = w; g < ng; g += nth)
          for (int64_t kb = 0; kb < KB; ++kb)
            for (int l = 0; l < 64; ++l)
              std::memcpy(&out[(size_t)(((g * KB + kb) * 64 + l) * 8)],
                          &in[(size_t)((g * 16 + (l & 15)) * K + kb * 32 + (l >> 4) * 8)], 16);
      });
    for (auto& th : pool) th.join();
    if (hipMemcpy(arena + cj.dst + (size_t)(g0 * 16 * K * 2), out.data(), bytes, hipMemcpyHostToDevice) != hipSuccess)
      return false;
  }
  (void)stream;
  return true;
}

// GEMV weight loads per lane issued before the dependency wait.  A load
// issue blocks once the compute unit's outstanding-miss capacity is full, so
// a deep pre-wait burst delays the wait and the input staging behind data
// that then sits in registers; a short burst lets staging overlap the stream.
// Producers whose tasks trigger before their outputs are stored (GEMV tiles
// once their last weight loads are issued, attention chunks after their
// softmax, merge slices once their inputs are current): consumers read tagged
// words and re-read stale ones, so an early trigger overlaps the event hop
// with the tail of the producing task.
static bool early_trigger_kinds(int32_t kind) {
  return kind == OP_QKV || kind == OP_OPROJ || kind == OP_GATEUP || kind == OP_DOWN || kind == OP_ROUTER ||
         kind == OP_ATTN || kind == OP_MERGE;
}
static bool ctrl_wave_kinds(int32_t kind) {
  (void)kind;
  return false;
}
static int32_t default_prefetch_loads(int32_t kind) {
  (void)kind;
  return 64;  // the whole ring
}

mk_status mk_load_weights(mk_graph* g, const mk_tensor* tensors, int32_t n, void* d_arena, void* d_scratch,
                          void* d_trace, void* stream_) {
  if (!g || !g->G || (!tensors && n > 0) || !d_arena || !d_scratch) {
    set_error("mk_load_weights: null argument");
    return MK_ERR_ARG;
  }
  Graph& G = *g->G;
  if (G.trace_bytes > 0 && !d_trace) {
    set_error("mk_load_weights: trace buffer required (graph built with trace on)");
    return MK_ERR_ARG;
  }
  hipStream_t stream = (hipStream_t)stream_;
  // ---- the tensor set
  std::vector<std::pair<std::string, std::pair<int64_t, int64_t>>> want;
  tensor_name_list(G.shape, &want);
  std::map<std::string, const mk_tensor*> have;
  for (int32_t i = 0; i < n; ++i) {
    if (!tensors[i].name || !tensors[i].data) {
      set_error("mk_load_weights: tensor with null name or data");
      return MK_ERR_ARG;
    }
    if (!have.emplace(tensors[i].name, &tensors[i]).second) {
      set_error(std::string("mk_load_weights: duplicate tensor ") + tensors[i].name);
      return MK_ERR_ARG;
    }
  }
  for (auto& w : want) {
    auto it = have.find(w.first);
    if (it == have.end()) {
      set_error("mk_load_weights: missing tensor " + w.first);
      return MK_ERR_ARG;
    }
    if (it->second->rows != w.second.first || it->second->cols != w.second.second) {
      set_error("mk_load_weights: tensor " + w.first + " has shape [" + std::to_string(it->second->rows) + "," +
                std::to_string(it->second->cols) + "], expected [" + std::to_string(w.second.first) + "," +
                std::to_string(w.second.second) + "]");
      return MK_ERR_ARG;
    }
  }
  if ((int32_t)have.size() != (int32_t)want.size()) {
    set_error("mk_load_weights: unexpected extra tensors");
    return MK_ERR_ARG;
  }
  int dev = 0;
  HIPCHK(hipGetDevice(&dev));
  g->device = dev;
  if (!g->side_stream) {
    hipStream_t s2;
    HIPCHK(hipStreamCreateWithFlags(&s2, hipStreamNonBlocking));
    g->side_stream = s2;
    hipEvent_t ea, eb;
    HIPCHK(hipEventCreateWithFlags(&ea, hipEventDisableTiming));
    HIPCHK(hipEventCreateWithFlags(&eb, hipEventDisableTiming));
    g->ev_a = ea;
    g->ev_b = eb;
  }
  char* arena = (char*)d_arena;
  char* scr = (char*)d_scratch;
  // ---- weights
  for (const CopyJob& cj : G.copies) {
    const mk_tensor* t = have[cj.tensor];
    const char* src = (const char*)t->data + (size_t)cj.row0 * (size_t)t->cols * 2;
    const size_t bytes = (size_t)cj.nrows * (size_t)t->cols * 2;
    if (cj.kind == CopyJob::ROWS) {
      HIPCHK(hipMemcpyAsync(arena + cj.dst, src, bytes, t->on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice,
                            stream));
    } else if (cj.kind == CopyJob::GAIN_F32) {
      std::vector<uint16_t> hb((size_t)cj.nrows);
      if (t->on_device) {
        HIPCHK(hipMemcpy(hb.data(), src, bytes, hipMemcpyDeviceToHost));
      } else {
        std::memcpy(hb.data(), src, bytes);
      }
      std::vector<float> hf(hb.size());
      for (size_t i = 0; i < hb.size(); ++i) {
        uint32_t u = (uint32_t)hb[i] << 16;
        std::memcpy(&hf[i], &u, 4);
      }
      HIPCHK(hipMemcpy(arena + cj.dst, hf.data(), hf.size() * 4, hipMemcpyHostToDevice));
    } else if (cj.kind == CopyJob::SWZ16) {
      if (!swizzle16(cj, t, src, arena, stream)) return MK_ERR_HIP;
    } else {
      set_error("mk_load_weights: unsupported copy kind");
      return MK_ERR_SHAPE;
    }
  }
  // ---- tables
  std::vector<double> inv((size_t)G.shape.head_dim / 2);
  for (size_t i = 0; i < inv.size(); ++i)
    inv[i] = std::pow(G.shape.rope_theta, -2.0 * (double)i / (double)G.shape.head_dim);
  HIPCHK(hipMemcpy(arena + G.off_invfreq, inv.data(), inv.size() * 8, hipMemcpyHostToDevice));
  Geom ge = G.geom;
  ge.inv_freq = (const double*)(arena + G.off_invfreq);
  HIPCHK(hipMemcpy(arena + G.off_geom, &ge, sizeof ge, hipMemcpyHostToDevice));
  // the operator table, its buffers in `base` (the caller's scratch, or the
  // library's static scratch for mk_decode_step_noalloc)
  std::vector<OpDesc> od(G.ops.size());
  auto op_table = [&](char* base) {
  auto bufp = [&](int32_t id) -> uint64_t* {
    if (id < 0 || G.bufs[id].off < 0) return nullptr;
    return (uint64_t*)(base + G.bufs[id].off);
  };
  for (size_t i = 0; i < G.ops.size(); ++i) {
    const OpInst& o = G.ops[i];
    OpDesc& d = od[i];
    std::memset(&d, 0, sizeof d);
    d.kind = o.kind;
    d.layer = o.layer;
    d.K = o.K;
    d.N = o.N;
    d.norm_in = o.norm_in;
    d.ntasks = o.ntasks;
    d.pre = G.opts.prefetch_loads > 0 ? G.opts.prefetch_loads : default_prefetch_loads(o.kind);
    d.pad = (ctrl_wave_kinds(o.kind) ? 1 : 0) | (early_trigger_kinds(o.kind) && !G.opts.late_trigger ? 2 : 0) |
            (o.ring ? 4 : 0);
    d.w = o.w_off >= 0 ? (const uint16_t*)(arena + o.w_off) : nullptr;
    d.g = o.g_off >= 0 ? (const float*)(arena + o.g_off) : nullptr;
    d.g2 = o.g2_off >= 0 ? (const float*)(arena + o.g2_off) : nullptr;
    d.in = bufp(o.in_buf);
    d.res = bufp(o.res_buf);
    d.out = bufp(o.out_buf);
    d.aux = bufp(o.aux_buf);
    d.aux2 = bufp(o.aux2_buf);
    if (o.aux_buf == -3)  // attention arrival counters of layer o.layer
      d.aux = (uint64_t*)(base + G.off_arrive +
                          (int64_t)o.layer * G.B * G.shape.n_kv_heads * kCounterStride * 4);
  }
  };
  op_table(scr);
  HIPCHK(hipMemcpy(arena + G.off_ops, od.data(), od.size() * sizeof(OpDesc), hipMemcpyHostToDevice));
  // the same table over the static scratch, when the graph fits it
  g->static_scr = nullptr;
  if (G.scratch_bytes <= (int64_t)kStaticScratchBytes) {
    void* sp = nullptr;
    const mk_status rs = static_scratch(dev, &sp);
    if (rs != MK_OK) return rs;
    op_table((char*)sp);
    HIPCHK(hipMemcpy(arena + G.off_ops_static, od.data(), od.size() * sizeof(OpDesc), hipMemcpyHostToDevice));
    g->static_scr = sp;
  }
  HIPCHK(hipMemcpy(arena + G.off_tasks, G.tasks.data(), G.tasks.size() * sizeof(Task), hipMemcpyHostToDevice));
  if (!G.events.empty())
    HIPCHK(hipMemcpy(arena + G.off_events, G.events.data(), G.events.size() * sizeof(Event), hipMemcpyHostToDevice));
  HIPCHK(hipMemcpy(arena + G.off_wloff, G.wl_off.data(), G.wl_off.size() * 4, hipMemcpyHostToDevice));
  if (!G.wl_ids.empty())
    HIPCHK(hipMemcpy(arena + G.off_wlids, G.wl_ids.data(), G.wl_ids.size() * 4, hipMemcpyHostToDevice));
  HIPCHK(hipMemsetAsync(scr, 0, (size_t)G.scratch_bytes, stream));
  if (G.trace_bytes > 0) HIPCHK(hipMemsetAsync(d_trace, 0, (size_t)G.trace_bytes, stream));
  HIPCHK(hipStreamSynchronize(stream));
  const u32 none = 0xFFFFFFFFu;
  HIPCHK(hipMemcpy(scr + G.off_status + ST_MIN_TASK * 4, &none, 4, hipMemcpyHostToDevice));
  int wcr = 0;
  HIPCHK(hipDeviceGetAttribute(&wcr, hipDeviceAttributeWallClockRate, dev));
  const int64_t us = G.opts.spin_timeout_us > 0 ? G.opts.spin_timeout_us : 2000000;
  g->budget_ticks = (uint64_t)us * (uint64_t)(wcr > 0 ? wcr : 100000) / 1000ull;
  for (int v : {1, 2, 3, 4, (int)kMfmaVariant, (int)kRingVariant}) {
    (void)hipFuncSetAttribute(worker_fn(v, false), hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    (void)hipFuncSetAttribute(worker_fn(v, true), hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    (void)hipFuncSetAttribute(lpt_fn(v), hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  }
  (void)hipGetLastError();
  // co-residency: two worker wavefronts per SIMD plus the dispatch wavefront
  // (both the one-step and the multi-step worker kernel)
  for (bool multi : {false, true}) {
    hipFuncAttributes fw, fd;
    HIPCHK(hipFuncGetAttributes(&fw, worker_fn(kernel_variant(G), multi)));
    const bool routed = G.wl_off[G.W + 1] > G.wl_off[G.W];
    HIPCHK(hipFuncGetAttributes(&fd, routed ? (const void*)mk_dispatch : (const void*)mk_dispatch_dense));
    auto gran = [](int v) { return (v + 7) / 8 * 8; };
    if (2 * gran(fw.numRegs) + gran(fd.numRegs) > 512 || fw.localSizeBytes > 0) {
      set_error("mk_load_weights: worker kernel uses " + std::to_string(fw.numRegs) + " VGPRs and " +
                std::to_string(fw.localSizeBytes) + " B scratch; the dispatch wavefront would not fit beside it" +
                (routed ? " (routed experts at batch 1 need gemv = MK_GEMV_MFMA)" : ""));
      return MK_ERR_NOT_RESIDENT;
    }
  }
  g->arena = d_arena;
  g->scratch = d_scratch;
  g->trace = d_trace;
  g->loaded = true;
  g->last_static = false;
  g->epoch = 0;
  g->persistent_steps = 0;
  g->tag = 1;
  return MK_OK;
}

mk_status mk_set_mode(mk_graph* g, int32_t mode, int32_t per_task_launch) {
  if (!g || (mode != MK_PERSISTENT && mode != MK_LAUNCH_PER_TASK)) {
    set_error("mk_set_mode: bad argument");
    return MK_ERR_ARG;
  }
  g->mode = mode;
  g->per_task_launch = per_task_launch;
  return MK_OK;
}

mk_status mk_decode_step(mk_graph* g, const int32_t* d_tokens, const int32_t* d_positions, const mk_kv_cache* kv,
                         float* d_logits, void* stream_) {
  return mk_decode_steps(g, d_tokens, d_positions, kv, d_logits, nullptr, 1, stream_);
}

mk_status mk_decode_steps(mk_graph* g, const int32_t* d_tokens, const int32_t* d_positions, const mk_kv_cache* kv,
                          float* d_logits, int32_t* d_tokens_out, int32_t n_steps, void* stream_) {
  if (!g || !g->G) {
    set_error("mk_decode_step: null graph");
    return MK_ERR_ARG;
  }
  if (!g->loaded) {
    set_error("mk_decode_step: weights not loaded");
    return MK_ERR_STATE;
  }
  if (!d_tokens || !d_positions || !kv || !d_logits) {
    set_error("mk_decode_step: null argument");
    return MK_ERR_ARG;
  }
  Graph& G = *g->G;
  if (n_steps < 1 || n_steps > kMaxStepsPerLaunch) {
    set_error("mk_decode_steps: n_steps must be in 1.." + std::to_string(kMaxStepsPerLaunch));
    return MK_ERR_ARG;
  }
  if ((n_steps > 1 || d_tokens_out) && g->mode != MK_PERSISTENT) {
    set_error("mk_decode_steps: several steps per launch and token output need the persistent mode");
    return MK_ERR_ARG;
  }
  if (n_steps > 1 && G.opts.trace) {
    set_error("mk_decode_steps: the task trace holds one step; build without trace for several steps per launch");
    return MK_ERR_ARG;
  }
  // tags of this launch stay nonzero and below kGraphTag (reserved for graph replays)
  if (g->tag > kGraphTag - 1u - (uint32_t)n_steps) g->tag = 1;
  if (!kv_ok(G, kv, "mk_decode_step")) return MK_ERR_ARG;
  hipStream_t stream = (hipStream_t)stream_;
  StepArgs a = step_args(g, d_tokens, d_positions, kv, d_logits, d_tokens_out, n_steps);
  if (a.trace_on == 1) HIPCHK(hipMemsetAsync(a.status + ST_TICKET, 0, 2 * sizeof(u32), stream));
  const mk_status rc = launch_step(g, a, n_steps > 1 || d_tokens_out != nullptr, stream);
  if (rc != MK_OK) return rc;
  g->last_static = false;
  g->last_steps = n_steps;
  g->last_tag0 = a.tag;
  g->epoch += (uint32_t)n_steps;
  if (g->mode == MK_PERSISTENT) g->persistent_steps += (uint32_t)n_steps;
  g->tag += (uint32_t)n_steps;
  if (g->tag == 0) g->tag = 1;
  return MK_OK;
}

mk_status mk_decode_step_noalloc(mk_graph* g, const int32_t* d_tokens, const int32_t* d_positions,
                                 const mk_kv_cache* kv, float* d_logits, void* stream_) {
  if (!g || !g->G) {
    set_error("mk_decode_step_noalloc: null graph");
    return MK_ERR_ARG;
  }
  Graph& G = *g->G;
  if (G.scratch_bytes > (int64_t)kStaticScratchBytes) {
    set_error("mk_decode_step_noalloc: the graph needs " + std::to_string(G.scratch_bytes) +
              " bytes of scratch; the static scratch holds " + std::to_string(kStaticScratchBytes));
    return MK_ERR_ARG;
  }
  if (!g->loaded || !g->static_scr) {
    set_error("mk_decode_step_noalloc: weights not loaded");
    return MK_ERR_STATE;
  }
  if (!d_tokens || !d_positions || !kv || !d_logits) {
    set_error("mk_decode_step_noalloc: null argument");
    return MK_ERR_ARG;
  }
  if (!kv_ok(G, kv, "mk_decode_step_noalloc")) return MK_ERR_ARG;
  hipStream_t stream = (hipStream_t)stream_;
  // this call's data tag on the device's static scratch: never one that a
  // word left there by an earlier call carries (tags only grow; when they
  // would reach the reserved graph tag, the whole array is cleared first)
  uint32_t tag;
  bool clear_all = false;
  {
    std::lock_guard<std::mutex> lk(g_static_mu);
    uint32_t& next = g_static_tag[g->device];
    if (next == 0 || next >= kGraphTag - 1u) {
      clear_all = next != 0;
      next = 1;
    }
    tag = next++;
  }
  const uint32_t none_word = (uint32_t)((G.off_status + ST_MIN_TASK * 4) / 4);
  const uint64_t words = (clear_all ? (uint64_t)kStaticScratchBytes : (uint64_t)G.off_state_end) / 4;
  hipLaunchKernelGGL(mk_clear_state, dim3((unsigned)std::min<uint64_t>(1024, (words + 255) / 256)), dim3(256), 0,
                     stream, (uint32_t*)g->static_scr, (uint32_t)words, none_word);
  HIPCHK(hipGetLastError());
  StepArgs a = step_args(g, d_tokens, d_positions, kv, d_logits, nullptr, 1, true);
  a.epoch = 0;
  a.run_base = 0;
  a.tag = tag;
  const mk_status rc = launch_step(g, a, false, stream);
  if (rc != MK_OK) return rc;
  g->last_static = true;
  g->last_steps = 1;
  g->last_tag0 = tag;
  return MK_OK;
}

struct mk_lpt_graph {
  mk_graph* g = nullptr;
  hipGraphExec_t exec = nullptr;
};

mk_status mk_capture_lpt_graph(mk_graph* g, const int32_t* d_tokens, const int32_t* d_positions,
                               const mk_kv_cache* kv, float* d_logits, mk_lpt_graph** out) {
  if (!out) {
    set_error("mk_capture_lpt_graph: null output");
    return MK_ERR_ARG;
  }
  *out = nullptr;
  if (!g || !g->G || !g->loaded) {
    set_error("mk_capture_lpt_graph: weights not loaded");
    return MK_ERR_STATE;
  }
  if (!d_tokens || !d_positions || !d_logits) {
    set_error("mk_capture_lpt_graph: bad argument");
    return MK_ERR_ARG;
  }
  if (!kv_ok(*g->G, kv, "mk_capture_lpt_graph")) return MK_ERR_ARG;
  if (g->G->opts.trace) {
    // the ticketed trace clears its counters with a memset, which a captured graph must not hold
    set_error("mk_capture_lpt_graph: build the graph without trace");
    return MK_ERR_ARG;
  }
  StepArgs a = step_args(g, d_tokens, d_positions, kv, d_logits, nullptr, 1);
  a.tag = kGraphTag;  // replays write and accept only this tag; stream order makes it safe
  hipStream_t cs;
  HIPCHK(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  mk_status rc = MK_OK;
  if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    set_error("mk_capture_lpt_graph: hipStreamBeginCapture failed");
    rc = MK_ERR_HIP;
  } else {
    rc = launch_lpt(g, a, cs);
    const hipError_t e = hipStreamEndCapture(cs, &graph);
    if (rc == MK_OK && e != hipSuccess) {
      set_error(std::string("mk_capture_lpt_graph: hipStreamEndCapture: ") + hipGetErrorString(e));
      rc = MK_ERR_HIP;
    }
  }
  if (rc == MK_OK && hipGraphInstantiateWithFlags(&exec, graph, 0) != hipSuccess) {
    set_error("mk_capture_lpt_graph: hipGraphInstantiate failed");
    rc = MK_ERR_HIP;
  }
  if (graph) (void)hipGraphDestroy(graph);
  (void)hipStreamDestroy(cs);
  if (rc != MK_OK) return rc;
  mk_lpt_graph* lg = new mk_lpt_graph();
  lg->g = g;
  lg->exec = exec;
  *out = lg;
  return MK_OK;
}

mk_status mk_lpt_graph_launch(mk_lpt_graph* lg, void* stream) {
  if (!lg || !lg->exec || !lg->g || !lg->g->loaded) {
    set_error("mk_lpt_graph_launch: bad graph");
    return MK_ERR_ARG;
  }
  HIPCHK(hipGraphLaunch(lg->exec, (hipStream_t)stream));
  // the replayed tasks trigger their events like any launch-per-task step
  lg->g->epoch += 1;
  lg->g->last_steps = 1;
  lg->g->last_tag0 = kGraphTag;
  lg->g->last_static = false;
  return MK_OK;
}

void mk_lpt_graph_destroy(mk_lpt_graph* lg) {
  if (!lg) return;
  if (lg->exec) (void)hipGraphExecDestroy(lg->exec);
  delete lg;
}

mk_status mk_check(mk_graph* g) {
  if (!g || !g->G || !g->loaded) {
    set_error("mk_check: graph not loaded");
    return MK_ERR_STATE;
  }
  Graph& G = *g->G;
  char* scr = active_scratch(g);
  u32 st[ST_WORDS];
  HIPCHK(hipMemcpy(st, scr + G.off_status, sizeof st, hipMemcpyDeviceToHost));
  if (st[ST_ERROR] == ERR_NONE) return MK_OK;
  std::string msg;
  mk_status rc = MK_ERR_TIMEOUT;
  if (st[ST_ERROR] == ERR_TIMEOUT) {
    int32_t task = (int32_t)st[ST_TASK];
    msg = "device wait timed out";
    if (task >= 0 && task < (int32_t)G.tasks.size()) {
      const Task& t = G.tasks[task];
      msg += ": task " + std::to_string(task) + " (" + op_kind_name(G.ops[t.op].kind) + ", layer " +
             std::to_string(G.ops[t.op].layer) + ") waiting on event " + std::to_string((int32_t)st[ST_EVENT]) +
             " saw " + std::to_string(st[ST_SEEN]) + " of " + std::to_string(st[ST_TARGET]);
    } else if (task == -1) {
      msg += ": the dispatcher saw " + std::to_string(st[ST_SEEN]) + " of " + std::to_string(st[ST_TARGET]) +
             " workers finish";
    } else {
      const uint64_t addr = ((uint64_t)st[ST_ADDR_HI] << 32) | st[ST_ADDR_LO];
      const uint64_t base = (uint64_t)(uintptr_t)scr;
      std::string where = "?";
      for (const Buffer& b : G.bufs)
        if (b.off >= 0 && addr >= base + b.off && addr < base + b.off + b.words * 8)
          where = b.name + "[" + std::to_string((addr - base - b.off) / 8) + "]";
      msg += ": activation word " + where + " kept tag " + std::to_string(st[ST_SEEN]) + " (want " +
             std::to_string(st[ST_TARGET]) + ")";
    }
    if (st[ST_ADDR_LO] | st[ST_ADDR_HI]) {
      const uint64_t addr = ((uint64_t)st[ST_ADDR_HI] << 32) | st[ST_ADDR_LO];
      const uint64_t base = (uint64_t)(uintptr_t)scr;
      for (const Buffer& b : G.bufs)
        if (b.off >= 0 && addr >= base + b.off && addr < base + b.off + b.words * 8)
          msg += "; stale word " + b.name + "[" + std::to_string((addr - base - b.off) / 8) + "]";
    }
    {
      std::vector<u32> prog((size_t)G.W + 1);
      if (hipMemcpy(prog.data(), scr + G.off_progress, prog.size() * 4, hipMemcpyDeviceToHost) ==
          hipSuccess) {
        std::vector<std::pair<u32, int>> stuck;
        for (int w = 0; w < G.W; ++w)
          if (prog[w] != 0xFFFFFFFFu && prog[w] != 0) stuck.push_back({prog[w] - 1, w});
        std::sort(stuck.begin(), stuck.end());
        msg += "; " + std::to_string(stuck.size()) + " workers unfinished";
        for (size_t i = 0; i < stuck.size() && i < 4; ++i) {
          const u32 id = stuck[i].first;
          msg += ", worker " + std::to_string(stuck[i].second) + " in task " + std::to_string(id);
          if (id < G.tasks.size())
            msg += std::string(" (") + op_kind_name(G.ops[G.tasks[id].op].kind) + ")";
        }
      }
    }
    const u32 mt = st[ST_MIN_TASK];
    if (mt < (u32)G.tasks.size())
      msg += "; most upstream timed-out task " + std::to_string(mt) + " (" + op_kind_name(G.ops[G.tasks[mt].op].kind) +
             ", layer " + std::to_string(G.ops[G.tasks[mt].op].layer) + ")";
  } else if (st[ST_ERROR] == ERR_NOT_RESIDENT) {
    msg = "only " + std::to_string(st[ST_SEEN] % (u32)G.W) + " of " + std::to_string(G.W) +
          " worker workgroups became resident (the dispatcher gave up waiting)";
    rc = MK_ERR_NOT_RESIDENT;
  } else if (st[ST_ERROR] == ERR_CONFIG) {
    msg = "device tables do not match the graph (reload the weights)";
    rc = MK_ERR_STATE;
  } else if (st[ST_ERROR] == ERR_BAD_INPUT) {
    msg = "token id or position out of range";
    rc = MK_ERR_ARG;
  } else {
    msg = "device error " + std::to_string(st[ST_ERROR]);
    rc = MK_ERR_STATE;
  }
  // reset the event state so that the next step can run (a step on the
  // static scratch starts from a cleared state anyway; the graph's own
  // scratch keeps its epoch otherwise)
  HIPCHK(hipMemset(scr + G.off_counters, 0, (size_t)(G.off_state_end - G.off_counters)));
  HIPCHK(hipDeviceSynchronize());
  const u32 none = 0xFFFFFFFFu;
  HIPCHK(hipMemcpy(scr + G.off_status + ST_MIN_TASK * 4, &none, 4, hipMemcpyHostToDevice));
  if (!g->last_static) {
    g->epoch = 0;
    g->persistent_steps = 0;
  }
  set_error("mk_check: " + msg);
  return rc;
}

mk_status mk_read_trace(mk_graph* g, mk_trace_rec* host_buf, int64_t cap, int64_t* n) {
  if (!g || !g->G || !g->loaded || !n) {
    set_error("mk_read_trace: bad argument");
    return MK_ERR_ARG;
  }
  Graph& G = *g->G;
  if (!g->trace) {
    set_error("mk_read_trace: graph built without trace");
    return MK_ERR_STATE;
  }
  u32 cnt = (u32)G.tasks.size();  // timing trace: one slot per task
  if (G.opts.trace == 1)
    HIPCHK(hipMemcpy(&cnt, active_scratch(g) + G.off_status + ST_TRACE_N * 4, 4, hipMemcpyDeviceToHost));
  int64_t m = std::min<int64_t>({(int64_t)cnt, cap, (int64_t)G.tasks.size()});
  if (m > 0 && host_buf) HIPCHK(hipMemcpy(host_buf, g->trace, (size_t)m * sizeof(mk_trace_rec), hipMemcpyDeviceToHost));
  *n = (int64_t)cnt;
  return MK_OK;
}

mk_status mk_read_routing(mk_graph* g, int32_t step, int32_t* experts, float* weights, float* router_logits,
                          int64_t cap) {
  if (!g || !g->G || !g->loaded || !experts || !weights) {
    set_error("mk_read_routing: bad argument");
    return MK_ERR_ARG;
  }
  Graph& G = *g->G;
  const mk_model_shape& s = G.shape;
  if (s.n_experts == 0 || G.off_route_hist < 0) {
    set_error("mk_read_routing: the graph has no routed experts");
    return MK_ERR_STATE;
  }
  const int64_t n = (int64_t)s.n_layers * G.B * s.top_k;
  if (cap < n || (router_logits && cap < (int64_t)s.n_layers * G.B * s.n_experts)) {
    set_error("mk_read_routing: buffers smaller than layers x batch x top_k (x experts for router logits)");
    return MK_ERR_ARG;
  }
  if (step < 0 || step >= g->last_steps || step < g->last_steps - kRouteHistSteps) {
    set_error("mk_read_routing: step " + std::to_string(step) + " is not one of the last " +
              std::to_string(kRouteHistSteps) + " steps of the last launch (" + std::to_string(g->last_steps) +
              " steps)");
    return MK_ERR_ARG;
  }
  if (router_logits && step != g->last_steps - 1) {
    set_error("mk_read_routing: router logits are kept for the last step of the launch only");
    return MK_ERR_ARG;
  }
  const size_t slot = (size_t)(step % kRouteHistSteps);
  std::vector<u64> rec((size_t)n);
  HIPCHK(hipMemcpy(rec.data(), active_scratch(g) + G.off_route_hist + slot * (size_t)n * 8, (size_t)n * 8,
                   hipMemcpyDeviceToHost));
  for (int64_t i = 0; i < n; ++i) {
    experts[i] = (int32_t)(uint32_t)rec[(size_t)i];
    const uint32_t wb = (uint32_t)(rec[(size_t)i] >> 32);
    std::memcpy(&weights[i], &wb, 4);
  }
  if (router_logits) {
    // tagged words [B][E] of each layer's router buffer, tagged with the last step's tag
    const uint32_t want = g->last_tag0 + (uint32_t)step;
    const int64_t be = (int64_t)G.B * s.n_experts;
    std::vector<u64> w((size_t)be);
    for (int32_t l = 0; l < s.n_layers; ++l) {
      const std::string name = "rlog." + std::to_string(l);
      const Buffer* buf = nullptr;
      for (const Buffer& b : G.bufs)
        if (b.name == name) buf = &b;
      if (!buf || buf->off < 0 || buf->words != be) {
        set_error("mk_read_routing: router buffer of layer " + std::to_string(l) + " not found");
        return MK_ERR_STATE;
      }
      HIPCHK(hipMemcpy(w.data(), active_scratch(g) + buf->off, (size_t)be * 8, hipMemcpyDeviceToHost));
      for (int64_t i = 0; i < be; ++i) {
        if ((uint32_t)(w[(size_t)i] >> 32) != want) {
          set_error("mk_read_routing: router logits of layer " + std::to_string(l) + " are not the last step's");
          return MK_ERR_STATE;
        }
        const uint32_t vb = (uint32_t)w[(size_t)i];
        std::memcpy(&router_logits[(size_t)l * be + i], &vb, 4);
      }
    }
  }
  return MK_OK;
}

mk_status mk_read_counters(mk_graph* g, uint32_t* host_counters, int64_t cap) {
  if (!g || !g->G || !g->loaded || !host_counters) {
    set_error("mk_read_counters: bad argument");
    return MK_ERR_ARG;
  }
  Graph& G = *g->G;
  const int64_t ne = (int64_t)G.events.size();
  if (cap < ne) {
    set_error("mk_read_counters: buffer too small");
    return MK_ERR_ARG;
  }
  std::vector<u32> raw((size_t)ne * kSubCounters * kCounterStride);
  if (ne > 0)
    HIPCHK(hipMemcpy(raw.data(), active_scratch(g) + G.off_counters, raw.size() * 4, hipMemcpyDeviceToHost));
  for (int64_t e = 0; e < ne; ++e) {
    u32 s = 0;
    for (int k = 0; k < kSubCounters; ++k) s += raw[((size_t)e * kSubCounters + k) * kCounterStride];
    host_counters[e] = s;
  }
  return MK_OK;
}

mk_status mk_graph_stats(const mk_graph* g, mk_stats* out) {
  if (!g || !g->G || !out) {
    set_error("mk_graph_stats: null argument");
    return MK_ERR_ARG;
  }
  const Graph& G = *g->G;
  std::memset(out, 0, sizeof *out);
  out->tasks = (int64_t)G.tasks.size();
  out->empty_tasks = G.n_empty;
  out->events = (int64_t)G.events.size();
  out->ops = (int64_t)G.ops.size();
  out->workers = G.W;
  out->launches_per_step = (int64_t)G.launch_first.size();
  out->raw_edges = (int64_t)G.raw_edges.size();
  out->reduced_edges = G.n_reduced_edges;
  for (int32_t w = 0; w < G.W; ++w)
    out->max_tasks_per_worker = std::max<int64_t>(out->max_tasks_per_worker, G.wl_off[w + 1] - G.wl_off[w]);
  out->weight_bytes = G.weight_bytes_step;
  out->arena_bytes = G.arena_bytes;
  out->scratch_bytes = G.scratch_bytes;
  out->trace_bytes = G.trace_bytes;
  out->batch = G.B;
  out->max_ctx = G.cap;
  out->attn_chunks = G.C;
  out->gemv = G.gemv;
  out->ring_kb = G.geom.ring_u;
  out->ring_ops = 0;
  for (const OpInst& o : G.ops) out->ring_ops += o.ring ? 1 : 0;
  return MK_OK;
}

mk_status mk_dump_graph(const mk_graph* g, const char* json_path) {
  if (!g || !g->G || !json_path) {
    set_error("mk_dump_graph: null argument");
    return MK_ERR_ARG;
  }
  dump_json(*g->G, json_path);
  return MK_OK;
}

mk_status mk_get_tasks(const mk_graph* g, int32_t* rows, int64_t cap) {
  if (!g || !g->G || !rows || cap < (int64_t)g->G->tasks.size()) {
    set_error("mk_get_tasks: bad argument");
    return MK_ERR_ARG;
  }
  const Graph& G = *g->G;
  for (size_t i = 0; i < G.tasks.size(); ++i) {
    const Task& t = G.tasks[i];
    int32_t* r = rows + 8 * i;
    r[0] = G.ops[t.op].kind;
    r[1] = G.ops[t.op].layer;
    r[2] = t.dep;
    r[3] = t.trig;
    r[4] = t.a0;
    r[5] = t.a1;
    r[6] = t.a2;
    r[7] = t.a3;
  }
  return MK_OK;
}

mk_status mk_get_events(const mk_graph* g, int32_t* rows, int64_t cap) {
  if (!g || !g->G || !rows || cap < (int64_t)g->G->events.size()) {
    set_error("mk_get_events: bad argument");
    return MK_ERR_ARG;
  }
  const Graph& G = *g->G;
  for (size_t i = 0; i < G.events.size(); ++i) {
    rows[4 * i] = G.events[i].need;
    rows[4 * i + 1] = G.events[i].first;
    rows[4 * i + 2] = G.events[i].last;
    rows[4 * i + 3] = G.events[i].producers;
  }
  return MK_OK;
}

mk_status mk_get_worker_lists(const mk_graph* g, int32_t* offsets, int32_t* ids, int64_t cap) {
  if (!g || !g->G || !offsets || !ids || cap < (int64_t)g->G->wl_ids.size()) {
    set_error("mk_get_worker_lists: bad argument");
    return MK_ERR_ARG;
  }
  const Graph& G = *g->G;
  std::memcpy(offsets, G.wl_off.data(), G.wl_off.size() * 4);
  std::memcpy(ids, G.wl_ids.data(), G.wl_ids.size() * 4);
  return MK_OK;
}

mk_status mk_get_raw_edges(const mk_graph* g, int32_t* rows, int64_t cap, int64_t* n) {
  if (!g || !g->G || !n) {
    set_error("mk_get_raw_edges: bad argument");
    return MK_ERR_ARG;
  }
  const Graph& G = *g->G;
  *n = (int64_t)G.raw_edges.size();
  if (!rows) return MK_OK;
  if (cap < *n) {
    set_error("mk_get_raw_edges: buffer too small");
    return MK_ERR_ARG;
  }
  for (size_t i = 0; i < G.raw_edges.size(); ++i) {
    rows[2 * i] = G.raw_edges[i].first;
    rows[2 * i + 1] = G.raw_edges[i].second;
  }
  return MK_OK;
}

void mk_destroy_graph(mk_graph* g) {
  if (!g) return;
  if (g->side_stream) (void)hipStreamDestroy((hipStream_t)g->side_stream);
  if (g->ev_a) (void)hipEventDestroy((hipEvent_t)g->ev_a);
  if (g->ev_b) (void)hipEventDestroy((hipEvent_t)g->ev_b);
  delete g->G;
  delete g;
}

mk_status mk_stream_read(const void* d_buf, uint64_t bytes, uint32_t* d_sink, int32_t blocks, void* stream) {
  if (!d_buf || !d_sink || blocks <= 0 || bytes % 16 || ((uintptr_t)d_buf & 15)) {
    set_error("mk_stream_read: bad argument (16-byte aligned buffer, size a multiple of 16, blocks > 0)");
    return MK_ERR_ARG;
  }
  hipLaunchKernelGGL(mk_stream_read_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream, (const mk::u32x4*)d_buf,
                     bytes / 16, d_sink);
  HIPCHK(hipGetLastError());
  return MK_OK;
}

const char* mk_hip_runtime_path(void) {
  static std::string path;
  Dl_info info;
  if (dladdr((void*)&hipGetDeviceCount, &info) && info.dli_fname) path = info.dli_fname;
  return path.c_str();
}

}  // extern "C"
#endif  // host section
