// HBM read-rate reference: a plain streaming read with nothing of the attention
// path in it (no paging, masking or arithmetic beyond a sum), so that a measured
// bandwidth can be set beside what the same GPU reaches on the simplest possible
// read, as well as beside the published peak.
#include "common.h"
#include "kernels.h"

namespace qknr {
namespace {

// Grid-stride over 16-byte elements, four loads in flight per thread per step;
// the sum is stored only if it equals a value no sum of the buffer takes in
// practice, which keeps the loads without writing anything.
__global__ __launch_bounds__(256) void read_probe_kernel(const float4* __restrict__ a, size_t n, float* __restrict__ out) {
  float s = 0.f;
  const size_t stride = (size_t)gridDim.x * 256 * 4;
  for (size_t i = (size_t)blockIdx.x * 256 * 4 + threadIdx.x; i < n; i += stride) {
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t j = i + (size_t)u * 256;
      v[u] = j < n ? a[j] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) s += (v[u].x + v[u].y) + (v[u].z + v[u].w);
  }
  if (s == -1.2345678e-30f) out[0] = s;
}

}  // namespace

hipError_t launch_read_probe(hipStream_t stream, const void* buf, size_t bytes, float* out) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  // two workgroups per CU: the fastest of 2..32 per CU on a 4 GiB read
  hipLaunchKernelGGL(read_probe_kernel, dim3(2 * cus), dim3(256), 0, stream, static_cast<const float4*>(buf),
                     bytes / 16, out);
  return hipGetLastError();
}

}  // namespace qknr
