// K3 kernels and launchers: the tile plan, the first visible positions of a packed
// form, and one workgroup per (64-token tile, KV head) work item. The device code
// of a work item (and its design) is in prefill_body.h.
#include <algorithm>
#include <climits>

#include "prefill_body.h"
#include "kernels.h"

namespace qknr {
namespace {

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

// Exclusive prefix sum of v over the 1024 threads of the workgroup (.x) and the
// total (.y). s_scan: 16 ints of LDS; every thread calls it.
__device__ int2 block_scan(int v, int* s_scan, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  __syncthreads();   // s_scan is free (a previous call's readers are done)
  if (lane == 63) s_scan[wave] = x;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const int c = s_scan[w];
    before += w < wave ? c : 0;
    total += c;
  }
  return make_int2(before + x - v, total);
}

// The same over the 64 lanes of one wave, with DPP row shifts and row broadcasts
// (no barriers, no LDS round trips).
__device__ int2 wave_scan_dpp(int v) {
  int x = v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return make_int2(x - v, __builtin_amdgcn_readlane(x, 63));
}

constexpr int kSplitPlanMaxTiles = 512;   // tiles for which the plan considers key splits
constexpr int kMinChunkPages = 4;          // pages of a chunk at least (a chunk's set-up is ~2 pages)

// The work list of one prefill call (one workgroup of 1024 threads):
//  1. the packed form's first visible positions (segments given);
//  2. per tile: its key pages (from the smallest first visible position to the
//     largest position), and whether its tokens form one run (one row, every
//     index in range);
//  3. tiles sorted by decreasing cost (largest visible span first);
//  4. key splits (tiles <= kSplitPlanMaxTiles and a partial-state budget): with
//     T = total item pages / CUs, a one-run tile of p > 1.5 T pages asks for
//     min(8, ceil(p / T)) chunks; in the sorted order, a tile gets its chunks if
//     the extra chunks asked for up to and including it fit the grid's spare
//     workgroups; the chunks take the tile's place in the order. Every step is
//     a sum or scan, one tile per thread.
// Up to 64 tiles, steps 3-5 run in one wave, one tile per lane: a rank sort
// through LDS (each lane counts the keys below its own) and DPP scans.
//     (A split costs a merge: partial states through memory, a release and an
//     acquire that write back and invalidate the XCD's L2; below 1.5 T it loses.)
//  5. the tickets of the split tiles' merges are zeroed.
// Without splits the list is the sorted tiles, one pair each.
// Steps 4-5 for the tile of sorted rank i (in: i < n_tiles) whose sorted key is
// key; scan is block_scan or wave_scan_dpp over the threads taking part, stride their
// count. Splits only when max_extra_pairs > 0.
template <class Scan>
__device__ void assign_pairs(int i, bool in, unsigned long long key, const int* s_aux, int n_tiles, int n_kv,
                             int n_cus, int max_extra_pairs, int* n_pairs, int4* pairs, int* tickets, int stride,
                             Scan scan) {
  const int t = in ? (int)(key & 0xffffffffu) : 0;
  const int aux = in ? s_aux[t] : 0;
  const int pages = aux >> 1;
  const long long total = (long long)scan(pages).y * n_kv;
  const int target = max(kMinChunkPages, (int)((total + n_cus - 1) / n_cus));
  int S = 1;
  if (max_extra_pairs > 0 && (aux & 1) && 2 * pages > 3 * target)
    S = min(kMaxChunks, min(pages, (pages + target - 1) / target));
  const int2 asked = scan(S - 1);   // exclusive prefix, total
  if (asked.x + S - 1 > max_extra_pairs) S = 1;
  const int2 extra = scan(S - 1);
  const int2 slot = scan(S > 1 ? S : 0);
  const int2 split = scan(S > 1 ? 1 : 0);
  if (in)
    for (int c = 0; c < S; ++c) pairs[i + extra.x + c] = make_int4(t, c | (S << 8), slot.x, split.x);
  if (i == 0) *n_pairs = n_tiles + extra.y;
  for (int j = i; j < split.y * n_kv; j += stride) tickets[j] = 0;
}

__global__ __launch_bounds__(1024) void prefill_plan_kernel(
    int n_tokens, const int* __restrict__ positions, const int* __restrict__ segments, int* __restrict__ lo,
    const int* __restrict__ rows, int n_table_rows, int max_pos, int n_tiles, int n_kv, int n_cus,
    int max_extra_pairs, int* __restrict__ n_pairs, int4* __restrict__ pairs, int* __restrict__ tickets) {
  __shared__ unsigned long long keys[kPlanMaxTiles];
  __shared__ int s_aux[kPlanMaxTiles];   // pages << 1 | one-run flag
  __shared__ int s_last[1024];
  __shared__ int s_scan[16];
  const int tid = threadIdx.x;
  if (segments) {
    segment_starts(n_tokens, positions, segments, lo, s_last, tid);
    __syncthreads();   // the workgroup's own lo writes are visible to it after the barrier
  }
  int npow2 = 1;
  while (npow2 < n_tiles) npow2 <<= 1;
  constexpr int kBatch = 8;
  const int wave = tid >> 6, lane = tid & 63;
  const int* lsrc = lo ? lo : positions;
  for (int i0 = wave; i0 < npow2; i0 += kBatch * 16) {
    int pos[kBatch], fst[kBatch], row[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {   // every load of the batch first
      const int i = i0 + u * 16;
      const int t = i * kTile + lane;
      const int tc = (i < n_tiles && t < n_tokens) ? t : 0;
      pos[u] = positions[tc];
      fst[u] = lsrc[tc];
      row[u] = rows[tc];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = i0 + u * 16;
      if (i >= npow2) break;
      const int t = i * kTile + lane;
      const bool ok = i < n_tiles && t < n_tokens;
      int hi = ok ? max(pos[u] + 1, 0) : 0;
      int f = lo ? (ok ? max(fst[u], 0) : 0x7fffffff) : 0;
      const bool valid = !ok || (row[u] >= 0 && row[u] < n_table_rows && pos[u] >= 0 && pos[u] < max_pos);
      int rmin = ok ? row[u] : 0x7fffffff, rmax = ok ? row[u] : -1;
      const bool all_valid = __all(valid);
      hi = wave_reduce_dpp<true>(hi);
      f = wave_reduce_dpp<false>(f);
      rmin = wave_reduce_dpp<false>(rmin);
      rmax = wave_reduce_dpp<true>(rmax);
      if (lane == 0 && i < npow2) {
        const int cost = max(hi - f, 0);
        keys[i] = i < n_tiles ? ((unsigned long long)(0xffffffffu - (unsigned)cost) << 32) | (unsigned)i : ~0ull;
        const int pages = hi > f ? (hi - 1) / kPageSize - f / kPageSize + 1 : 0;
        s_aux[i] = (pages << 1) | ((all_valid && rmin == rmax) ? 1 : 0);
      }
    }
  }
  __syncthreads();
  if (n_tiles <= 64) {
    if (wave != 0) return;
    const bool in = lane < n_tiles;
    unsigned long long key = in ? keys[lane] : ~0ull;
    {
      // rank sort: keys are distinct (the tile index is in the low word); each lane
      // counts the keys below its own and places it there
      int rank = 0;
      for (int k = 0; k < n_tiles; ++k) rank += keys[k] < key ? 1 : 0;
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_wave_barrier();
      static_assert(kPlanMaxTiles >= 128, "the ranked keys go to keys[64..127]");
      if (in) keys[64 + rank] = key;
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_wave_barrier();
      key = in ? keys[64 + lane] : ~0ull;
    }
    assign_pairs(lane, in, key, s_aux, n_tiles, n_kv, n_cus, n_tiles <= kSplitPlanMaxTiles ? max_extra_pairs : 0,
                 n_pairs, pairs, tickets, 64, [&](int v) { return wave_scan_dpp(v); });
    return;
  }
  for (int k = 2; k <= npow2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < npow2; i += 1024) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long a = keys[i], b = keys[ixj];
          const bool up = (i & k) == 0;
          if ((a > b) == up) { keys[i] = b; keys[ixj] = a; }
        }
      }
      __syncthreads();
    }
  }
  if (max_extra_pairs > 0) {   // one sorted tile per thread (n_tiles <= kSplitPlanMaxTiles <= 1024)
    assign_pairs(tid, tid < n_tiles, tid < n_tiles ? keys[tid] : 0ull, s_aux, n_tiles, n_kv, n_cus, max_extra_pairs,
                 n_pairs, pairs, tickets, 1024, [&](int v) { return block_scan(v, s_scan, tid); });
  } else {
    for (int i = tid; i < n_tiles; i += 1024) pairs[i] = make_int4((int)(keys[i] & 0xffffffffu), 1 << 8, 0, 0);
    if (tid == 0) *n_pairs = n_tiles;
  }
}

__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void paged_prefill_bf16_kernel(PrefillParams P) {
  prefill_item(P, blockIdx.x, threadIdx.x);
}

}  // namespace

int prefill_max_pages_per_row() { return kTabCache; }

namespace {

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace of the bfloat16 prefill: [pair count][pairs][merge tickets][partial
// states of split chunks]. Extra chunks: up to one spare workgroup per CU (as
// pairs: CUs / KV heads), for plans of at most kSplitPlanMaxTiles tiles.
struct PrefillLayout {
  int n_tiles, max_extra_pairs;
  size_t pairs, tickets, partials, total;
};

PrefillLayout prefill_layout(int n_tokens, int n_kv) {
  PrefillLayout L;
  L.n_tiles = (n_tokens + kTile - 1) / kTile;
  const int cus = device_cus(), kv = std::max(n_kv, 1);
  L.max_extra_pairs = L.n_tiles <= kSplitPlanMaxTiles
                          ? std::min(std::max(1, cus / kv), L.n_tiles * (kMaxChunks - 1))
                          : 0;
  size_t off = 256;   // the pair count
  L.pairs = off;
  off += align256((size_t)(L.n_tiles + L.max_extra_pairs) * sizeof(int4));
  L.tickets = off;
  off += align256((size_t)L.max_extra_pairs * n_kv * sizeof(int));
  L.partials = off;
  // a split tile of S chunks adds S - 1 pairs and needs S <= 2 (S - 1) chunk states
  off += (size_t)2 * L.max_extra_pairs * n_kv * kTile * kGroup * kPartialFloats * sizeof(float);
  L.total = align256(off);
  return L;
}

}  // namespace

size_t prefill_workspace_bytes(int n_tokens, int n_kv_heads) {
  return prefill_layout(n_tokens, n_kv_heads).total;
}

size_t segment_start_bytes(int n_tokens) { return ((size_t)n_tokens * sizeof(int) + 255) / 256 * 256; }

hipError_t launch_segment_start(hipStream_t stream, int n_tokens, const int32_t* positions,
                                const int32_t* segments, int32_t* lo) {
  hipLaunchKernelGGL(segment_start_kernel, dim3(1), dim3(1024), 0, stream, n_tokens, positions, segments, lo);
  return hipGetLastError();
}

hipError_t launch_prefill_bf16(hipStream_t stream, const AttnArgs& a) {
  const PrefillLayout L = prefill_layout(a.n_queries, a.n_kv_heads);
  char* ws = static_cast<char*>(a.workspace);
  int* lo = nullptr;
  if (a.segments)   // packed form: first visible positions after the prefill workspace
    lo = reinterpret_cast<int*>(ws + L.total);
  PrefillParams P;
  P.order = nullptr;
  P.pairs = nullptr;
  P.n_pairs = nullptr;
  P.tickets = nullptr;
  P.partials = nullptr;
  P.partial_ml = nullptr;
  int grid = L.n_tiles * a.n_kv_heads;
  if (L.n_tiles <= kPlanMaxTiles) {
    int* n_pairs = reinterpret_cast<int*>(ws);
    int4* pairs = reinterpret_cast<int4*>(ws + L.pairs);
    P.n_pairs = n_pairs;
    P.pairs = pairs;
    P.tickets = reinterpret_cast<int*>(ws + L.tickets);
    P.partials = reinterpret_cast<float*>(ws + L.partials);
    P.partial_ml = P.partials + (size_t)2 * L.max_extra_pairs * a.n_kv_heads * kTile * kGroup * kHeadDim;
    hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(1024), 0, stream, a.n_queries, a.positions,
                       a.segments, lo, a.rows, a.n_table_rows, a.pages_per_row * kPageSize, L.n_tiles,
                       a.n_kv_heads, device_cus(), L.max_extra_pairs, n_pairs, pairs, P.tickets);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    grid = (L.n_tiles + L.max_extra_pairs) * a.n_kv_heads;
  } else if (lo) {
    hipError_t e = launch_segment_start(stream, a.n_queries, a.positions, a.segments, lo);
    if (e != hipSuccess) return e;
  }
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
  P.lo = lo;
  P.gate = (const uint16_t*)a.gate;
  hipLaunchKernelGGL(paged_prefill_bf16_kernel, dim3(grid), dim3(512), 0, stream, P);
  return hipGetLastError();
}

}  // namespace qknr
