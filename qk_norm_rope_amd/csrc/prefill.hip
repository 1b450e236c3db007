// K3 kernels and launchers: the tile plan, the first visible positions of a packed
// form, and one workgroup per (64-token tile, KV head) work item. The device code
// of a work item (and its design) is in prefill_body.h.
#include "prefill_body.h"
#include "kernels.h"

namespace qknr {
namespace {

__global__ __launch_bounds__(1024) void prefill_plan_kernel(int n_tokens, const int* __restrict__ positions,
                                                            const int* __restrict__ lo, int n_tiles,
                                                            int* __restrict__ order) {
  __shared__ unsigned long long keys[kPlanMaxTiles];
  plan_tiles(n_tokens, positions, lo, n_tiles, order, keys, threadIdx.x, blockDim.x);
}

// First visible position of every token of a pack whose prompts attend only among
// themselves (nest "models/qwen3-8b/files", src/attention.linnet prefill_packed:
// token i sees token j when segments agree and positions[j] <= positions[i]). Each
// segment is one run of the pack with positions rising by one, so the first visible
// position is the position of the run's first token. One workgroup of 1024 threads:
// a chunk of tokens per thread, run starts carried across chunks by a prefix max
// (s_last: 1024 ints of LDS).
__device__ __forceinline__ void segment_starts(int n_tokens, const int* __restrict__ positions,
                                               const int* __restrict__ segments, int* __restrict__ lo,
                                               int* s_last, int tid) {
  const int per = (n_tokens + 1023) / 1024;
  const int c0 = min(tid * per, n_tokens), c1 = min(c0 + per, n_tokens);
  int last = -1;   // index of the last run start inside this chunk
  for (int i = c0; i < c1; ++i)
    if (i == 0 || segments[i] != segments[i - 1]) last = i;
  s_last[tid] = last;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {   // inclusive prefix max (Hillis-Steele)
    const int x = tid >= d ? s_last[tid - d] : -1;
    __syncthreads();
    s_last[tid] = max(s_last[tid], x);
    __syncthreads();
  }
  int start = tid > 0 ? s_last[tid - 1] : -1;
  for (int i = c0; i < c1; ++i) {
    if (i == 0 || segments[i] != segments[i - 1]) start = i;
    lo[i] = min(positions[start], positions[i]);
  }
}

__global__ __launch_bounds__(1024) void segment_start_kernel(int n_tokens, const int* __restrict__ positions,
                                                             const int* __restrict__ segments,
                                                             int* __restrict__ lo) {
  __shared__ int s_last[1024];
  segment_starts(n_tokens, positions, segments, lo, s_last, threadIdx.x);
}

// The packed form's two set-up steps in one launch: first visible positions, then
// the tile order by cost (the workgroup's own lo writes are visible to it after
// the barrier).
__global__ __launch_bounds__(1024) void packed_plan_kernel(int n_tokens, const int* __restrict__ positions,
                                                           const int* __restrict__ segments, int* __restrict__ lo,
                                                           int n_tiles, int* __restrict__ order) {
  __shared__ int s_last[1024];
  __shared__ unsigned long long keys[kPlanMaxTiles];
  segment_starts(n_tokens, positions, segments, lo, s_last, threadIdx.x);
  __syncthreads();
  plan_tiles(n_tokens, positions, lo, n_tiles, order, keys, threadIdx.x, blockDim.x);
}

__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void paged_prefill_bf16_kernel(PrefillParams P) {
  prefill_item(P, blockIdx.x, threadIdx.x);
}

}  // namespace

int prefill_max_pages_per_row() { return kTabCache; }

size_t prefill_workspace_bytes(int n_tokens, int /*n_kv_heads*/) {
  const size_t tiles = (size_t)(n_tokens + kTile - 1) / kTile;
  return (tiles * sizeof(int) + 255) / 256 * 256;
}

size_t segment_start_bytes(int n_tokens) { return ((size_t)n_tokens * sizeof(int) + 255) / 256 * 256; }

hipError_t launch_segment_start(hipStream_t stream, int n_tokens, const int32_t* positions,
                                const int32_t* segments, int32_t* lo) {
  hipLaunchKernelGGL(segment_start_kernel, dim3(1), dim3(1024), 0, stream, n_tokens, positions, segments, lo);
  return hipGetLastError();
}

hipError_t launch_prefill_bf16(hipStream_t stream, const AttnArgs& a) {
  const int n_tiles = (a.n_queries + kTile - 1) / kTile;
  int* order = nullptr;
  int* lo = nullptr;
  if (a.segments)   // packed form: first visible positions after the tile order
    lo = reinterpret_cast<int*>(static_cast<char*>(a.workspace) + prefill_workspace_bytes(a.n_queries, a.n_kv_heads));
  if (n_tiles <= kPlanMaxTiles) {
    order = static_cast<int*>(a.workspace);
    if (lo)
      hipLaunchKernelGGL(packed_plan_kernel, dim3(1), dim3(1024), 0, stream, a.n_queries, a.positions,
                         a.segments, lo, n_tiles, order);
    else
      hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(1024), 0, stream, a.n_queries, a.positions,
                         nullptr, n_tiles, order);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else if (lo) {
    hipError_t e = launch_segment_start(stream, a.n_queries, a.positions, a.segments, lo);
    if (e != hipSuccess) return e;
  }
  PrefillParams P;
  P.n_tokens = a.n_queries;
  P.n_kv = a.n_kv_heads;
  P.q = (const uint16_t*)a.q;
  P.k_pool = (const uint16_t*)a.k_pool;
  P.v_pool = (const uint16_t*)a.v_pool;
  P.num_pages = a.num_pages;
  P.table = a.table;
  P.n_table_rows = a.n_table_rows;
  P.pages_per_row = a.pages_per_row;
  P.rows = a.rows;
  P.positions = a.positions;
  P.scale_log2 = a.scale * kLog2e;
  P.out = a.out;
  P.order = order;
  P.lo = lo;
  P.gate = (const uint16_t*)a.gate;
  hipLaunchKernelGGL(paged_prefill_bf16_kernel, dim3(n_tiles * a.n_kv_heads), dim3(512), 0, stream, P);
  return hipGetLastError();
}

}  // namespace qknr
