// K2 kernel and launcher: workgroups of 4 waves, one or two per resident slot of the GPU,
// each streaming an equal slice of the (row, KV head, page) units. The device
// code (and its design) is in decode_body.h.
#include <algorithm>
#include <mutex>

#include "decode_body.h"
#include "kernels.h"
#include "qknr.h"

namespace qknr {
namespace {

__global__ __launch_bounds__(256) void paged_decode_bf16_kernel(DecodeParams P) {
  extern __shared__ int s_prefix[];   // [n_rows + 1]: units before row b
  decode_slice<4>(P, blockIdx.x, gridDim.x, s_prefix, threadIdx.x);
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
  // Large batches take two workgroups per resident slot: slices halve and the
  // workgroups that finish first take the rest, which evens out the slices'
  // different segment counts (64 ragged rows: 5.4 TB/s instead of 5.1). Smaller
  // ones keep one: each workgroup pays a fixed set-up and merge, which a second
  // round of workgroups with half the units each only repeats (128 rows at 1 KV
  // head: 5.2 TB/s with one round, 4.4 with two; 8 rows: a chain of memory round
  // trips that a second round lengthens). The host knows only the bound
  // rows x KV heads x pages per row on the units; two rounds from 300 units per
  // resident workgroup.
  int grid = grid_for_device();
  if ((int64_t)a.n_queries * a.n_kv_heads * a.pages_per_row >= 300LL * grid) grid = std::min(kMaxGrid, 2 * grid);
  const size_t lds = (size_t)(a.n_queries + 1) * sizeof(int);
  hipLaunchKernelGGL(paged_decode_bf16_kernel, dim3(grid), dim3(256), lds, stream, P);
  return hipGetLastError();
}

}  // namespace qknr
