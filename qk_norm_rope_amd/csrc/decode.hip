// K2 kernel and launcher: workgroups of 4 waves, one per resident slot of the GPU,
// each streaming an equal share of the (row, KV head, page) units on a cost scale
// that also charges each segment's set-up. The device
// code (and its design) is in decode_body.h.
#include <algorithm>
#include <mutex>

#include "decode_body.h"
#include "kernels.h"
#include "qknr.h"

namespace qknr {
namespace {

__global__ __launch_bounds__(256) void paged_decode_bf16_kernel(DecodeParams P) {
  extern __shared__ int s_prefix[];   // [n_rows + 1]: slice cost before row b
  decode_slice<4>(P, blockIdx.x, gridDim.x, s_prefix, threadIdx.x);
}

// Small batches (few rows x short tables): one workgroup of 4 waves per (row b, KV
// head g, chunk c of CP pages), the grid fixed by the host as rows x KV heads x
// ceil(pages_per_row / CP). A workgroup knows its row before it reads anything,
// so the row's position, the query operand and the chunk's page ids travel in one
// memory round trip, and then all CP pages of the chunk are in flight at once
// (the stream-K kernel needs a round trip for the positions, one for the prefix
// over the rows and then fetches two pages per wave at a time). A chunk past the
// row's last page leaves at once; a row of one chunk is written directly; the
// chunks of a longer row leave partial states that the last one to finish merges
// in chunk order (deterministic). Wave w takes keys 16w..16w+15 of every page,
// with the same per-page arithmetic as decode_slice.
template <int CP>
__device__ __forceinline__ void decode_chunk(const DecodeParams& P, const int blk, const int C, const int tid) {
  __shared__ __attribute__((aligned(16))) float s_p[4][16][kGroup];
  __shared__ float s_m[4][kGroup], s_l[4][kGroup];
  __shared__ __attribute__((aligned(16))) float s_acc[4][kGroup][kHeadDim];
  __shared__ int s_last;
  constexpr int TPH = 256 / kGroup;     // threads per head in the merge
  constexpr int DPT = kHeadDim / TPH;   // dimensions per thread in the merge (2)
  const int w = tid >> 6, l = tid & 63, hr = l & 15, G4 = l >> 4;
  const int c = blk % C;
  const int bg = blk / C;   // (row, KV head) segment
  const int g = bg % P.n_kv, b = bg / P.n_kv;
  const int n_q = P.n_kv * kGroup;
  const int64_t pool_slots = P.num_pages * kPageSize;

  // ---- one round trip: position, query operand, the chunk's page ids
  const int pos = P.positions[b];
  bf16x8 qa[4];
  if (hr < kGroup) {
    // rows 0..3 = heads 4g..4g+3; k-slot 8*G4+i of step st = dim 8*(4*st+G4)+i
    const uint16_t* qp = P.q + ((int64_t)b * n_q + g * kGroup + hr) * kHeadDim;
#pragma unroll
    for (int st = 0; st < 4; ++st) qa[st] = *reinterpret_cast<const bf16x8*>(qp + 8 * (4 * st + G4));
  } else {
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int i = 0; i < 8; ++i) qa[st][i] = (__bf16)0.0f;
  }
  const int p0 = c * CP;
  const int tbl = (l < CP && p0 + l < P.pages_per_row) ? P.table[(int64_t)b * P.pages_per_row + p0 + l] : -1;
  if (pos < 0 || pos >= P.pages_per_row * kPageSize) {
    // no keys: NaN outputs (as the float32 kernel gives them), written by chunk 0
    if (c == 0) {
      float* orow = P.out + ((int64_t)b * n_q + g * kGroup) * kHeadDim;
      for (int e = tid; e < kGroup * kHeadDim; e += 256) orow[e] = __builtin_nanf("");
    }
    return;
  }
  const int np = pos / kPageSize + 1;
  if (p0 >= np) return;
  const int n_pg = min(np - p0, CP);       // pages of this chunk
  const int nc = (np + CP - 1) / CP;       // chunks of the row

  // ---- all the chunk's pages in flight
  PageRegs r[CP];
#pragma unroll
  for (int i = 0; i < CP; ++i) {
    r[i].ok = false;
    if (i < n_pg) {
      const int64_t page = __builtin_amdgcn_readlane(tbl, i);
      r[i].ok = page >= 0 && page < P.num_pages;
      const int64_t pg = r[i].ok ? page : 0;
      const uint16_t* krow = P.k_pool + ((int64_t)g * pool_slots + pg * kPageSize + 16 * w + hr) * kHeadDim + 8 * G4;
      const uint16_t* vrow =
          P.v_pool + ((int64_t)g * pool_slots + pg * kPageSize + 16 * w + 4 * G4) * kHeadDim + 8 * hr;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(krow + 32 * st));
        r[i].k[st] = __builtin_bit_cast(bf16x8, x);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vrow + jj * kHeadDim));
        r[i].v[jj] = make_uint4(x[0], x[1], x[2], x[3]);
      }
    }
  }

  // ---- per page: scores (MFMA), online softmax per head, P.V
  float m[kGroup], lsum[kGroup], acc[kGroup][8];
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    m[i] = -INFINITY;
    lsum[i] = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[i][d] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < CP; ++i) {
    if (i >= n_pg) break;
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[st], r[i].k[st], sc, 0, 0, 0);
    const int key0 = (p0 + i) * kPageSize + 16 * w;
    const bool kvalid = r[i].ok && key0 + hr <= pos;
    float pr[kGroup], corr[kGroup];
    bool any_change = false;
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      const float x = kvalid ? sc[h] * P.scale_log2 : -INFINITY;
      const float pm = lane0(row_max16(x));
      const float mn = fmaxf(m[h], pm);
      corr[h] = (m[h] == mn) ? 1.f : __builtin_amdgcn_exp2f(m[h] - mn);
      any_change |= (m[h] != mn);
      const float ms = (mn == -INFINITY) ? 0.f : mn;
      pr[h] = __builtin_amdgcn_exp2f(x - ms);
      lsum[h] = lsum[h] * corr[h] + pr[h];
      m[h] = mn;
    }
    if (l < 16) *reinterpret_cast<float4*>(&s_p[w][l][0]) = make_float4(pr[0], pr[1], pr[2], pr[3]);
    __builtin_amdgcn_wave_barrier();
    if (any_change) {
#pragma unroll
      for (int h = 0; h < kGroup; ++h)
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[h][d] *= corr[h];
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int kk = 4 * G4 + jj;
      const bool vok = r[i].ok && key0 + kk <= pos;
      const float4 ph = *reinterpret_cast<const float4*>(&s_p[w][kk][0]);
      float vf[8];
      vf[0] = bf16_lo(r[i].v[jj].x); vf[1] = bf16_hi(r[i].v[jj].x);
      vf[2] = bf16_lo(r[i].v[jj].y); vf[3] = bf16_hi(r[i].v[jj].y);
      vf[4] = bf16_lo(r[i].v[jj].z); vf[5] = bf16_hi(r[i].v[jj].z);
      vf[6] = bf16_lo(r[i].v[jj].w); vf[7] = bf16_hi(r[i].v[jj].w);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const float x = vok ? vf[d] : 0.f;
        acc[0][d] += ph.x * x;
        acc[1][d] += ph.y * x;
        acc[2][d] += ph.z * x;
        acc[3][d] += ph.w * x;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- the four waves' states merged through LDS
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    lsum[h] = row_sum16(lsum[h]);
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[h][d] = group_sum4(acc[h][d]);
  }
  if (l < 16) {
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      float4* dst = reinterpret_cast<float4*>(&s_acc[w][h][8 * l]);
      dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
  }
  if (l == 0) {
#pragma unroll
    for (int h = 0; h < kGroup; ++h) { s_m[w][h] = m[h]; s_l[w][h] = lsum[h]; }
  }
  __syncthreads();
  const int hi = tid / TPH;
  const int dd = DPT * (tid % TPH);
  float M = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, s_m[ww][hi]);
  float L = 0.f, A[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) A[e] = 0.f;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    const float mw = s_m[ww][hi];
    const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
    L += f * s_l[ww][hi];
#pragma unroll
    for (int e = 0; e < DPT; ++e) A[e] += f * s_acc[ww][hi][dd + e];
  }
  float* orow = P.out + ((int64_t)b * n_q + g * kGroup + hi) * kHeadDim + dd;
  float gt[DPT] = {1.f, 1.f};
  if (P.gate) {   // output gate: out *= sigmoid(gate) at the same element
    const uint32_t gw =
        *reinterpret_cast<const uint32_t*>(P.gate + ((int64_t)b * n_q + g * kGroup + hi) * kHeadDim + dd);
    gt[0] = sigmoidf(bf16_lo(gw));
    gt[1] = sigmoidf(bf16_hi(gw));
  }
  if (nc == 1) {
#pragma unroll
    for (int e = 0; e < DPT; ++e) orow[e] = (A[e] / L) * gt[e];
    return;
  }
  // ---- partial state of chunk c; the last chunk of the row to finish merges them
  float* part = P.partials + ((int64_t)bg * C + c) * kPartial + hi * (kHeadDim + 2);
  if ((tid % TPH) == 0) { store_sc1(part, M); store_sc1(part + 1, L); }
#pragma unroll
  for (int e = 0; e < DPT; ++e) store_sc1(part + 2 + dd + e, A[e]);
  __builtin_amdgcn_s_waitcnt(0);   // the partial is at the coherence point before the ticket
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(&P.counters[bg], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old == nc - 1);
  }
  __syncthreads();
  if (!s_last) return;
  float Mx = -INFINITY, Lt = 0.f, B[DPT] = {0.f, 0.f};
  for (int c0 = 0; c0 < nc; c0 += 8) {
    float mv[8], lv[8], x[8][DPT];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const bool ok = c0 + k < nc;
      const float* ps = P.partials + ((int64_t)bg * C + (ok ? c0 + k : 0)) * kPartial + hi * (kHeadDim + 2);
      mv[k] = ok ? load_sc1(ps) : -INFINITY;
      lv[k] = ok ? load_sc1(ps + 1) : 0.f;
#pragma unroll
      for (int e = 0; e < DPT; ++e) x[k][e] = ok ? load_sc1(ps + 2 + dd + e) : 0.f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (mv[k] == -INFINITY) continue;
      const float mn = fmaxf(Mx, mv[k]);
      const float fo = (Mx == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(Mx - mn);
      const float fi = __builtin_amdgcn_exp2f(mv[k] - mn);
      Lt = Lt * fo + lv[k] * fi;
#pragma unroll
      for (int e = 0; e < DPT; ++e) B[e] = B[e] * fo + x[k][e] * fi;
      Mx = mn;
    }
  }
#pragma unroll
  for (int e = 0; e < DPT; ++e) orow[e] = (B[e] / Lt) * gt[e];
  if (tid == 0) __hip_atomic_store(&P.counters[bg], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kChunkPages = 2;

__global__ __launch_bounds__(256) void paged_decode_small_kernel(DecodeParams P, int chunks_per_row) {
  decode_chunk<kChunkPages>(P, blockIdx.x, chunks_per_row, threadIdx.x);
}

int grid_for_device() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    // occupancy with a 1024-row prefix table (larger tables only lower the
    // occupancy; the result stays correct when not every workgroup is resident)
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, paged_decode_bf16_kernel, 256,
                                                     4096) != hipSuccess ||
        per_cu <= 0)
      per_cu = 2;
    cached[dev] = std::min(kMaxGrid, cus * per_cu);
  }
  return cached[dev];
}

// Scratch of the allocation-free entry point: the merge counters of at most
// kNoAllocMaxPairs (row, KV head) segments, then the partial states of kMaxGrid
// workgroups, laid out as launch_decode_bf16 expects a workspace. Each GPU the
// library runs on holds one copy until the process ends; every call on that GPU
// shares it.
constexpr size_t kNoAllocCounterBytes = (size_t)kNoAllocMaxPairs * sizeof(int);
constexpr size_t kNoAllocScratchBytes = kNoAllocCounterBytes + (size_t)kMaxGrid * 2 * kPartial * sizeof(float);
static_assert(kNoAllocCounterBytes % 256 == 0, "partials start on a 256-byte boundary");
static_assert(kNoAllocMaxPairs == QKR_NOALLOC_MAX_ROW_HEADS, "limit stated in the header");
static_assert(kNoAllocScratchBytes == QKR_NOALLOC_SCRATCH_BYTES, "size stated in the header");
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// Device address of `scratch` on each device, looked up once per device with that
// device current. In host code the array's name is only a stand-in for the symbol,
// never a device address: kernels and copies take this pointer.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// The merge counters must start at zero: a fill kernel (not a memset node, so the
// call can sit inside a captured graph) clears the ones a call uses.
__global__ __launch_bounds__(256) void zero_ints_kernel(int* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

int decode_noalloc_max_pairs() { return kNoAllocMaxPairs; }

hipError_t launch_decode_bf16_noalloc(hipStream_t stream, const AttnArgs& a) {
  const int pairs = a.n_queries * a.n_kv_heads;   // <= kNoAllocMaxPairs, checked by the caller
  if (pairs <= 0 || pairs > kNoAllocMaxPairs) return hipErrorInvalidValue;
  void* ptr = nullptr;
  hipError_t e = scratch_of_current_device(&ptr);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(zero_ints_kernel, dim3((pairs + 255) / 256), dim3(256), 0, stream, static_cast<int*>(ptr),
                     pairs);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  AttnArgs b = a;
  b.workspace = ptr;
  b.workspace_bytes = kNoAllocScratchBytes;
  return launch_decode_bf16(stream, b);
}

size_t decode_workspace_bytes(int n_rows, int n_kv_heads, int /*pages_per_row*/) {
  const size_t pairs = (size_t)n_rows * n_kv_heads;
  const size_t counters = (pairs * sizeof(int) + 255) / 256 * 256;
  return counters + (size_t)kMaxGrid * 2 * kPartial * sizeof(float);
}

int decode_max_rows() { return kMaxRows; }

bool decode_cost_fits(int n_rows, int n_kv_heads, int pages_per_row) {
  return (int64_t)n_rows * n_kv_heads * ((int64_t)kCostA * pages_per_row + kCostB) < ((int64_t)1 << 31);
}

// Small batches take the fixed (row, KV head, chunk) grid: when the bound rows x KV
// heads x pages per row is at most 16 pages per resident workgroup and the chunks'
// partial states fit the workspace's partial area.
bool decode_uses_small_kernel(int n_rows, int n_kv_heads, int pages_per_row) {
  const int64_t bound_units = (int64_t)n_rows * n_kv_heads * pages_per_row;
  const int chunks = (pages_per_row + kChunkPages - 1) / kChunkPages;
  const int64_t small_grid = (int64_t)n_rows * n_kv_heads * chunks;
  return bound_units <= 16LL * grid_for_device() && small_grid <= 2LL * kMaxGrid;
}

hipError_t launch_decode_bf16(hipStream_t stream, const AttnArgs& a) {
  const size_t pairs = (size_t)a.n_queries * a.n_kv_heads;
  const size_t counter_bytes = (pairs * sizeof(int) + 255) / 256 * 256;
  DecodeParams P;
  P.n_rows = a.n_queries;
  P.n_kv = a.n_kv_heads;
  P.q = (const uint16_t*)a.q;
  P.k_pool = (const uint16_t*)a.k_pool;
  P.v_pool = (const uint16_t*)a.v_pool;
  P.num_pages = a.num_pages;
  P.table = a.table;
  P.pages_per_row = a.pages_per_row;
  P.positions = a.positions;
  P.scale_log2 = a.scale * kLog2e;
  P.out = a.out;
  P.gate = (const uint16_t*)a.gate;
  P.counters = static_cast<int*>(a.workspace);
  P.partials = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + counter_bytes);
  // One workgroup per resident slot, each with an equal share of the cost scale
  // (pages plus a per-segment charge), so slices with many short segments take
  // fewer pages. With slices cut by pages alone, two rounds of workgroups had evened
  // out their different segment counts on ragged batches; cost-cut slices in one
  // round are faster still (64 ragged rows 244 against 259 µs, the mixed step's 128
  // rows 628 against 645 µs), and each workgroup's set-up and merge come once.
  const int grid = grid_for_device();
  if (decode_uses_small_kernel(a.n_queries, a.n_kv_heads, a.pages_per_row)) {
    const int chunks = (a.pages_per_row + kChunkPages - 1) / kChunkPages;
    const int64_t small_grid = (int64_t)a.n_queries * a.n_kv_heads * chunks;
    hipLaunchKernelGGL(paged_decode_small_kernel, dim3((unsigned)small_grid), dim3(256), 0, stream, P, chunks);
    return hipGetLastError();
  }
  const size_t lds = (size_t)(a.n_queries + 1) * sizeof(int);
  hipLaunchKernelGGL(paged_decode_bf16_kernel, dim3(grid), dim3(256), lds, stream, P);
  return hipGetLastError();
}

}  // namespace qknr
