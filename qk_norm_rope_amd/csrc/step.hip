// Single-launch mixed step (nest "models/qwen3-8b/files": Entries table, step_paged;
// src/attention.linnet step_paged: one QK-norm + RoPE pass over the prompt tokens
// and the decode rows, every k/v write before any attention read, then prefill
// attention for the prompt tokens and paged decode attention for the rows).
//
// One persistent kernel, one workgroup of 8 waves per CU, running the work protocol
// of step_protocol.h: phase 1 takes the plan (ticket 0: sorts the prefill tiles by
// cost) and the append chunks (at least 16 tokens each and at most one per
// workgroup, one token per 256-thread half);
// after every phase-1 item has published, phase 2 takes prefill work items in plan
// order, then decode slices, so the two kernels' tails overlap.
// Visibility across XCDs (each has its own L2): the phase-1 items write with
// agent-scope relaxed atomic stores (written through to the level every XCD
// reads), every wave drains them (s_waitcnt), the workgroup meets at a barrier,
// and one relaxed add publishes the item; the wait ends with an agent-scope
// acquire (an L2 invalidate, once per workgroup), so phase 2's plain loads miss
// any stale copy. A release add per item would write back the XCD's whole L2
// each time: with 264 append items that alone took about 250 us of the step.
// The wait polls with relaxed loads (an acquire on every poll would invalidate
// the XCD's L2 each time, for every waiting workgroup) and is bounded in
// wall-clock time.
#include <algorithm>

#include "decode_body.h"
#include "prefill_body.h"
#include "append_body.h"
#include "kernels.h"
#include "step_protocol.h"

namespace qknr {
namespace {

constexpr int kStepThreads = 512;
constexpr int kAppendMinPerItem = 16;       // tokens per append item at least
constexpr int kPlanCap = kTabCache / 2;     // tiles the in-kernel plan sorts (keys in the page-id cache)
constexpr int kStepMaxRows = 8192;          // decode rows (LDS prefix table)
constexpr uint64_t kWaitTicks = 100000000;  // wait bound: 1 s of the 100 MHz real-time counter

struct StepParams {
  int n_tokens, n_prefill, n_q_heads, n_kv_heads;
  const uint16_t *q, *k, *v;
  const float *q_gain, *k_gain;
  float eps;
  const float *rope_cos, *rope_sin;
  int rope_rows;
  const int *positions, *step_positions, *slots, *decode_table;
  int pages_per_row;
  int64_t num_pages;
  uint16_t *q_out, *k_pool, *v_pool;
  StepWork work;
  int append_per_item;   // tokens per append item (even)
  PrefillParams pre;
  int n_tiles;
  int* order;   // plan output (null: tiles in pack order)
  DecodeParams dec;
  int* ctl;
};

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// The protocol's environment on the GPU. Every single-thread step (take a ticket,
// publish, wait, leave) runs in wave 0 under a scalar branch: all 64 lanes execute
// the atomic with lane 0 adding 1 and the others 0, and lane 0's result goes to the
// workgroup through LDS and readfirstlane. No per-lane branch surrounds an atomic,
// a wait or a barrier: an earlier form with per-lane `tid == 0` branches was
// compiled into a loop nest that only thread 0 could leave (a hang).
struct DeviceEnv {
  const StepParams& S;
  int* ctl;
  int* s_word;     // LDS word for broadcasts
  int* s_prefix;   // LDS prefix table of the decode slices
  int tid, lane;
  bool wave0;

  __device__ int broadcast_from_wave0(int v) {   // v: wave 0's uniform value
    if (wave0) *s_word = v;
    __syncthreads();
    const int r = __builtin_amdgcn_readfirstlane(*s_word);
    __syncthreads();   // s_word is rewritten by the next broadcast
    return r;
  }

  __device__ int take(int word) {
    __syncthreads();   // the previous item's LDS use is over
    int old = 0;
    if (wave0)
      old = __builtin_amdgcn_readfirstlane(__hip_atomic_fetch_add(&ctl[word], lane == 0 ? 1 : 0, __ATOMIC_RELAXED,
                                                                  __HIP_MEMORY_SCOPE_AGENT));
    return broadcast_from_wave0(old);
  }

  __device__ void publish(int word) {
    __builtin_amdgcn_s_waitcnt(0);   // this wave's agent-coherent stores are complete
    __syncthreads();                 // ... and every other wave's
    if (wave0) {
      const int at = word == kAppendDone ? kShardBase + kShardStride * (int)(blockIdx.x % kAppendShards) : word;
      __hip_atomic_fetch_add(&ctl[at], lane == 0 ? 1 : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  __device__ bool wait_ready(int n_append, int n_plan) {
    int ready = 0;
    if (wave0) {
      const uint64_t t_end = __builtin_amdgcn_s_memrealtime() + kWaitTicks;
      int seen_a = 0, seen_p = 0;
      for (;;) {
        seen_a = 0;
#pragma unroll
        for (int k = 0; k < kAppendShards; ++k)
          seen_a += __builtin_amdgcn_readfirstlane(__hip_atomic_load(&ctl[kShardBase + kShardStride * k],
                                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        seen_p = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(&ctl[kPlanDone], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        if (seen_a >= n_append && seen_p >= n_plan) {
          ready = 1;
          break;
        }
        if (__builtin_amdgcn_s_memrealtime() > t_end) break;
        __builtin_amdgcn_s_sleep(32);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // pairs with the items' release adds
      if (!ready) {
        __hip_atomic_store(&ctl[kFault], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ctl[kSeenAppend], seen_a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&ctl[kSeenPlan], seen_p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    return broadcast_from_wave0(ready) != 0;
  }

  __device__ int leave() {
    int old = 0;
    if (wave0)
      // relaxed: the words the last one clears are only touched by atomics, every
      // one of which a leaving workgroup has completed (its results were used)
      old = __builtin_amdgcn_readfirstlane(__hip_atomic_fetch_add(&ctl[kExited], lane == 0 ? 1 : 0,
                                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    return broadcast_from_wave0(old);
  }

  __device__ void clear() {
    if (wave0 && lane < kFault) __hip_atomic_store(&ctl[lane], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (wave0 && lane < kAppendShards)
      __hip_atomic_store(&ctl[kShardBase + kShardStride * lane], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  __device__ void plan() {
    if (S.order)
      plan_tiles<true>(S.n_prefill, S.positions, nullptr, S.n_tiles, S.order,
                 reinterpret_cast<unsigned long long*>(sTab), tid, kStepThreads);
  }

  __device__ void append(int chunk) {
    const int t0 = chunk * S.append_per_item;
    for (int i = tid >> 8; i < S.append_per_item; i += 2) {
      const int t = t0 + i;
      if (t >= S.n_tokens) break;
      append_token<uint16_t, uint16_t, false, false, true>(
          t, tid & 255, S.n_q_heads, S.n_kv_heads, S.q, S.k, S.v, S.q_gain, S.k_gain, S.eps, S.rope_cos,
          S.rope_sin, S.rope_rows, kHeadDim, S.positions, S.step_positions, S.n_prefill, S.slots,
          S.n_prefill, S.decode_table, S.pages_per_row, S.num_pages, S.q_out, S.k_pool, S.v_pool);
    }
  }

  // an opaque copy of the thread index: what the items derive from it is
  // recomputed per item instead of being hoisted out of the loop, where it would
  // stay live through the other kind of item
  __device__ int opaque_tid() {
    int t = tid;
    asm volatile("" : "+v"(t));
    return t;
  }

  __device__ void prefill(int item) { prefill_item<false>(S.pre, item, opaque_tid()); }

  __device__ void decode(int slice) {
    decode_slice<8>(S.dec, slice, S.work.n_decode_items, s_prefix, opaque_tid());
  }
};

__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void step_paged_kernel(StepParams S) {
  extern __shared__ int s_prefix[];   // decode: [n_rows + 1]
  __shared__ int s_word;
  const int tid = threadIdx.x;
  DeviceEnv e{S, S.ctl, &s_word, s_prefix, tid, tid & 63, wave_id() == 0};
  run_step_protocol(e, S.work);
}

int step_grid(int n_rows) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, step_paged_kernel, kStepThreads,
                                                   (size_t)(n_rows + 1) * sizeof(int)) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  return cus * per_cu;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

bool step_enabled() { return true; }

int step_max_rows() { return kStepMaxRows; }

size_t step_workspace_bytes(int n_prefill, int n_decode, int n_kv_heads, int pages_per_row) {
  const size_t tiles = (size_t)(n_prefill + kTile - 1) / kTile;
  size_t bytes = kCtlInts * sizeof(int) + align256(tiles * sizeof(int));
  if (n_decode > 0) bytes += decode_workspace_bytes(n_decode, n_kv_heads, pages_per_row);
  return bytes;
}

hipError_t launch_step(hipStream_t stream, const StepArgs& a) {
  const int P = a.n_prefill, R = a.n_decode;
  const int n_q = a.n_q_heads;
  char* ws = static_cast<char*>(a.workspace);
  const int n_tiles = (P + kTile - 1) / kTile;
  StepParams S;
  S.n_tokens = P + R;
  S.n_prefill = P;
  S.n_q_heads = a.n_q_heads;
  S.n_kv_heads = a.n_kv_heads;
  S.q = (const uint16_t*)a.q;
  S.k = (const uint16_t*)a.k;
  S.v = (const uint16_t*)a.v;
  S.q_gain = a.q_gain;
  S.k_gain = a.k_gain;
  S.eps = a.eps;
  S.rope_cos = a.rope_cos;
  S.rope_sin = a.rope_sin;
  S.rope_rows = a.rope_rows;
  S.positions = a.positions;
  S.step_positions = a.step_positions;
  S.slots = a.slots;
  S.decode_table = a.table + (int64_t)a.decode_row0 * a.pages_per_row;
  S.pages_per_row = a.pages_per_row;
  S.num_pages = a.num_pages;
  S.q_out = (uint16_t*)a.q_out;
  S.k_pool = (uint16_t*)a.k_pool;
  S.v_pool = (uint16_t*)a.v_pool;
  // Append items: at least 16 tokens, and at most one per workgroup besides the
  // one that takes the plan, so that no workgroup runs two while others wait for
  // them (a workgroup runs an item's tokens two at a time, one per 256-thread half).
  const int grid = step_grid(R);
  {
    const int per = std::max(kAppendMinPerItem, (S.n_tokens + std::max(grid - 1, 1) - 1) / std::max(grid - 1, 1));
    S.append_per_item = (per + 1) & ~1;
  }
  S.work.n_append_items = (S.n_tokens + S.append_per_item - 1) / S.append_per_item;
  S.ctl = reinterpret_cast<int*>(ws);
  S.order = (n_tiles > 0 && n_tiles <= kPlanCap) ? reinterpret_cast<int*>(ws + kCtlInts * sizeof(int)) : nullptr;
  S.n_tiles = n_tiles;
  S.work.n_prefill_items = n_tiles * a.n_kv_heads;

  PrefillParams& Pp = S.pre;
  Pp.n_tokens = P;
  Pp.n_kv = a.n_kv_heads;
  Pp.q = (const uint16_t*)a.q_out;
  Pp.k_pool = (const uint16_t*)a.k_pool;
  Pp.v_pool = (const uint16_t*)a.v_pool;
  Pp.num_pages = a.num_pages;
  Pp.table = a.table;
  Pp.n_table_rows = a.n_table_rows;
  Pp.pages_per_row = a.pages_per_row;
  Pp.rows = a.rows;
  Pp.positions = a.positions;
  Pp.scale_log2 = a.scale * kLog2e;
  Pp.out = a.prefill_out;
  Pp.order = S.order;
  Pp.lo = nullptr;
  Pp.gate = nullptr;
  Pp.pairs = nullptr;   // one item per tile and KV head, in plan order
  Pp.n_pairs = nullptr;
  Pp.tickets = nullptr;
  Pp.partials = nullptr;
  Pp.partial_ml = nullptr;

  DecodeParams& D = S.dec;
  const size_t dec_off = kCtlInts * sizeof(int) + align256((size_t)n_tiles * sizeof(int));
  const size_t pairs = (size_t)R * a.n_kv_heads;
  D.n_rows = R;
  D.n_kv = a.n_kv_heads;
  D.q = (const uint16_t*)a.q_out + (int64_t)P * n_q * kHeadDim;
  D.k_pool = (const uint16_t*)a.k_pool;
  D.v_pool = (const uint16_t*)a.v_pool;
  D.num_pages = a.num_pages;
  D.table = S.decode_table;
  D.pages_per_row = a.pages_per_row;
  D.positions = a.step_positions;
  D.scale_log2 = a.scale * kLog2e;
  D.out = a.decode_out;
  D.gate = nullptr;
  D.counters = R > 0 ? reinterpret_cast<int*>(ws + dec_off) : nullptr;
  D.partials = R > 0 ? reinterpret_cast<float*>(ws + dec_off + align256(pairs * sizeof(int))) : nullptr;
  S.work.n_decode_items =
      R > 0 ? std::min(kMaxGrid, std::max(1, a.decode_slices > 0 ? a.decode_slices : grid)) : 0;
  S.work.grid = grid;

  hipLaunchKernelGGL(step_paged_kernel, dim3(grid), dim3(kStepThreads), (size_t)(R + 1) * sizeof(int), stream, S);
  return hipGetLastError();
}

}  // namespace qknr
