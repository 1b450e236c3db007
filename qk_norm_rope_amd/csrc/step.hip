// Single-launch mixed step (nest "models/qwen3-8b/files": Entries table, step_paged;
// src/attention.linnet step_paged: one QK-norm + RoPE pass over the prompt tokens
// and the decode rows, every k/v write before any attention read, then prefill
// attention for the prompt tokens and paged decode attention for the rows).
//
// One persistent kernel, one workgroup of 8 waves per CU, taking work items from
// tickets in the workspace:
//   phase 1  item 0 sorts the prefill tiles by cost (the plan); items 1.. run the
//            QK-norm + RoPE + append of 16 tokens each (two tokens at a time, one
//            per 256-thread half). None of these waits for anything.
//   phase 2  after every phase-1 item has published its writes: prefill work items
//            (64-token tile, KV head) in plan order, then decode slices. Workgroups
//            that run out of prefill items start decode slices while the last
//            tiles finish, so the two kernels' tails overlap.
// A workgroup only waits for phase-1 items, and every phase-1 item is held by a
// workgroup that is running and never waits, so the wait ends whatever the number
// of resident workgroups. The wait polls with relaxed loads (an acquire on every
// poll would invalidate the XCD's L2 each time, for every waiting workgroup) and
// is bounded in wall-clock time: a workgroup that gives up sets the fault word,
// records the counts it saw, and skips phase 2.
// Visibility across XCDs (each has its own L2): every wave drains its stores, the
// workgroup meets at a barrier, and one agent-scope release add publishes the
// item; the waiter's agent-scope acquire load pairs with it.
// The last workgroup to leave clears the control words, so a call leaves the
// workspace as it found it (zero), with no memset on the stream.
#include <algorithm>

#include "decode_body.h"
#include "prefill_body.h"
#include "append_body.h"
#include "kernels.h"

namespace qknr {
namespace {

constexpr int kStepThreads = 512;
constexpr int kAppendPerItem = 16;          // tokens per append item
constexpr int kPlanCap = kTabCache / 2;     // tiles the in-kernel plan sorts (keys in the page-id cache)
constexpr int kStepMaxRows = 8192;          // decode rows (LDS prefix table)
constexpr uint64_t kWaitTicks = 100000000;  // wait bound: 1 s of the 100 MHz real-time counter

// control words at the start of the workspace
// (kFault and the two words after it are written only when a wait gives up)
enum : int { kTicketA = 0, kAppendDone, kPlanDone, kTicketB, kExited, kFault, kSeenAppend, kSeenPlan,
             kCtlInts = 64 };

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
  int n_append_items;
  PrefillParams pre;
  int n_tiles, n_prefill_items;
  int* order;   // plan output (null: tiles in pack order)
  DecodeParams dec;
  int n_decode_items;
  int* ctl;
};

// The single-thread steps of the loops (take a ticket, publish an item, wait, leave)
// run in wave 0 under a scalar branch, with lane 0's value taken by readfirstlane,
// never under a per-lane `tid == 0` branch: an earlier form with per-lane
// branches was compiled into a loop nest in which only thread 0 left the inner
// loop to take tickets, while the other threads of its wave went around again on
// the old item and the wave never let thread 0 run (a hang). A barrier also
// separates the publish step of one item from the ticket step of the next.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ int take_ticket(int* ctr, int* s_item) {
  __syncthreads();
  if (wave_id() == 0) {
    const int old = __hip_atomic_fetch_add(ctr, (threadIdx.x & 63) == 0 ? 1 : 0, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    *s_item = __builtin_amdgcn_readfirstlane(old);   // lane 0's ticket, stored by every lane
  }
  __syncthreads();
  const int it = __builtin_amdgcn_readfirstlane(*s_item);
  __syncthreads();   // s_item is rewritten by the next take
  return it;
}

__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void step_paged_kernel(StepParams S) {
  extern __shared__ int s_prefix[];   // decode: [n_rows + 1]
  __shared__ int s_item;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const bool wave0 = wave_id() == 0;
  int* ctl = S.ctl;

  // ---- phase 1: the plan and the append items
  for (;;) {
    const int it = take_ticket(&ctl[kTicketA], &s_item);
    if (it > S.n_append_items) break;
    if (it == 0) {
      if (S.order)
        plan_tiles(S.n_prefill, S.positions, nullptr, S.n_tiles, S.order,
                   reinterpret_cast<unsigned long long*>(sTab), tid, kStepThreads);
    } else {
      const int t0 = (it - 1) * kAppendPerItem;
      for (int i = tid >> 8; i < kAppendPerItem; i += 2) {
        const int t = t0 + i;
        if (t >= S.n_tokens) break;
        append_token<uint16_t, uint16_t, false, false>(
            t, tid & 255, S.n_q_heads, S.n_kv_heads, S.q, S.k, S.v, S.q_gain, S.k_gain, S.eps, S.rope_cos,
            S.rope_sin, S.rope_rows, kHeadDim, S.positions, S.step_positions, S.n_prefill, S.slots,
            S.n_prefill, S.decode_table, S.pages_per_row, S.num_pages, S.q_out, S.k_pool, S.v_pool);
      }
    }
    // publish: each wave's stores are complete, then one release by the workgroup
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (wave0)
      __hip_atomic_fetch_add(&ctl[it == 0 ? kPlanDone : kAppendDone], lane == 0 ? 1 : 0, __ATOMIC_RELEASE,
                             __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- wait until every phase-1 item has published
  if (wave0) {
    const uint64_t t_end = __builtin_amdgcn_s_memrealtime() + kWaitTicks;
    int ready = 0, seen_a = 0, seen_p = 0;
    for (;;) {
      seen_a = __builtin_amdgcn_readfirstlane(
          __hip_atomic_load(&ctl[kAppendDone], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      seen_p = __builtin_amdgcn_readfirstlane(
          __hip_atomic_load(&ctl[kPlanDone], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      if (seen_a >= S.n_append_items && seen_p >= 1) {
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
    s_item = ready;
  }
  __syncthreads();
  const bool ready = __builtin_amdgcn_readfirstlane(s_item) != 0;
  __syncthreads();

  // ---- phase 2: prefill items, then decode slices
  if (ready) {
    for (;;) {
      const int it = take_ticket(&ctl[kTicketB], &s_item);
      // an opaque copy of the thread index: what the items derive from it is
      // recomputed per item instead of being hoisted out of the loop, where it
      // would stay live through the other kind of item
      int t = tid;
      asm volatile("" : "+v"(t));
      if (it < S.n_prefill_items) {
        prefill_item<false>(S.pre, it, t);
      } else if (it - S.n_prefill_items < S.n_decode_items) {
        decode_slice<8>(S.dec, it - S.n_prefill_items, S.n_decode_items, s_prefix, t);
      } else {
        break;
      }
      __syncthreads();   // LDS reuse by the next item
    }
  }

  // ---- the last workgroup out clears the tickets (the fault words stay)
  if (wave0) {
    const int out = __builtin_amdgcn_readfirstlane(__hip_atomic_fetch_add(
        &ctl[kExited], lane == 0 ? 1 : 0, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT));
    if (out == (int)gridDim.x - 1 && lane < kFault)   // lane i clears word i
      __hip_atomic_store(&ctl[lane], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
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

// The kernel is built but not launched: an earlier form of it hung on the GPU (the
// ticket loop nest described at take_ticket), and the corrected form has not yet
// run on a GPU.
bool step_enabled() { return false; }

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
  S.n_append_items = (S.n_tokens + kAppendPerItem - 1) / kAppendPerItem;
  S.ctl = reinterpret_cast<int*>(ws);
  S.order = (n_tiles > 0 && n_tiles <= kPlanCap) ? reinterpret_cast<int*>(ws + kCtlInts * sizeof(int)) : nullptr;
  S.n_tiles = n_tiles;
  S.n_prefill_items = n_tiles * a.n_kv_heads;

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

  const int grid = step_grid(R);
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
  S.n_decode_items = R > 0 ? std::min(kMaxGrid, std::max(1, a.decode_slices > 0 ? a.decode_slices : 2 * grid)) : 0;

  hipLaunchKernelGGL(step_paged_kernel, dim3(grid), dim3(kStepThreads), (size_t)(R + 1) * sizeof(int), stream, S);
  return hipGetLastError();
}

}  // namespace qknr
