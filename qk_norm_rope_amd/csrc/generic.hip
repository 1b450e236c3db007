// Attention for pools of any dtype, one workgroup per (query, KV head).
//
// Used for float32 pools, where the bfloat16 MFMA kernels do not apply. Each of
// the 4 waves is one query head of the group; lane l owns dimensions 2l, 2l+1.
// Keys are visited in position order with an online softmax (fantasma
// "src/inference/model.zig", fullAttentionForward: scaled dot product with every
// cached key of KV head h / 4, max-subtracted exponentials, weighted sum of V;
// nest "models/qwen3-8b/files", src/attention.linnet decode: keys up to and
// including the query's position).
#include "common.h"
#include "kernels.h"

namespace qknr {
namespace {

template <typename T> __device__ inline void load2(const T* p, float& a, float& b);
template <> __device__ inline void load2<float>(const float* p, float& a, float& b) {
  float2 v = *reinterpret_cast<const float2*>(p);
  a = v.x; b = v.y;
}
template <> __device__ inline void load2<uint16_t>(const uint16_t* p, float& a, float& b) {
  uint32_t w = *reinterpret_cast<const uint32_t*>(p);
  a = bf16_lo(w); b = bf16_hi(w);
}

template <typename T>
__global__ __launch_bounds__(256) void attention_generic_kernel(
    int n_q_heads, const T* __restrict__ q, const T* __restrict__ k_pool,
    const T* __restrict__ v_pool, int64_t num_pages, const int* __restrict__ table,
    int n_table_rows, int pages_per_row, const int* __restrict__ rows,
    const int* __restrict__ positions, const int* __restrict__ lo, const T* __restrict__ gate,
    float scale, float* __restrict__ out) {
  const int t = blockIdx.x;
  const int g = blockIdx.y;
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = g * kGroup + w;
  const int row = rows ? rows[t] : t;
  const int pos = positions[t];
  float* o = out + ((int64_t)t * n_q_heads + h) * kHeadDim + 2 * lane;
  if (row < 0 || row >= n_table_rows || pos < 0 || pos >= pages_per_row * kPageSize) {
    o[0] = __builtin_nanf("");
    o[1] = __builtin_nanf("");
    return;
  }
  float q0, q1;
  load2<T>(q + ((int64_t)t * n_q_heads + h) * kHeadDim + 2 * lane, q0, q1);
  const int64_t pool_slots = num_pages * kPageSize;
  const T* kb = k_pool + (int64_t)g * pool_slots * kHeadDim + 2 * lane;
  const T* vb = v_pool + (int64_t)g * pool_slots * kHeadDim + 2 * lane;
  const int* trow = table + (int64_t)row * pages_per_row;
  float m = -INFINITY, l = 0.f, a0 = 0.f, a1 = 0.f;
  const int first = lo ? min(max(lo[t], 0), pos) : 0;   // packed form: own segment only
  for (int j = first; j <= pos; ++j) {
    const int64_t page = trow[j / kPageSize];
    if (page < 0 || page >= num_pages) continue;
    const int64_t slot = page * kPageSize + j % kPageSize;
    float k0, k1, v0, v1;
    load2<T>(kb + slot * kHeadDim, k0, k1);
    load2<T>(vb + slot * kHeadDim, v0, v1);
    const float s = wave_sum(q0 * k0 + q1 * k1) * scale;
    const float mn = fmaxf(m, s);
    const float corr = expf(m - mn);
    const float p = expf(s - mn);
    l = l * corr + p;
    a0 = a0 * corr + p * v0;
    a1 = a1 * corr + p * v1;
    m = mn;
  }
  float g0 = 1.f, g1 = 1.f;
  if (gate) {   // output gate: out *= sigmoid(gate) at the same element
    load2<T>(gate + ((int64_t)t * n_q_heads + h) * kHeadDim + 2 * lane, g0, g1);
    g0 = sigmoidf(g0);
    g1 = sigmoidf(g1);
  }
  o[0] = (a0 / l) * g0;
  o[1] = (a1 / l) * g1;
}

}  // namespace

hipError_t launch_attention_generic(hipStream_t stream, const AttnArgs& a) {
  const dim3 grid(a.n_queries, a.n_kv_heads), block(256);
  int32_t* lo = nullptr;
  if (a.segments) {
    lo = static_cast<int32_t*>(a.workspace);
    const hipError_t e = launch_segment_start(stream, a.n_queries, a.positions, a.segments, lo);
    if (e != hipSuccess) return e;
  }
  if (a.bf16) {
    hipLaunchKernelGGL(attention_generic_kernel<uint16_t>, grid, block, 0, stream, a.n_q_heads,
                       (const uint16_t*)a.q, (const uint16_t*)a.k_pool, (const uint16_t*)a.v_pool,
                       a.num_pages, a.table, a.n_table_rows, a.pages_per_row, a.rows,
                       a.positions, lo, (const uint16_t*)a.gate, a.scale, a.out);
  } else {
    hipLaunchKernelGGL(attention_generic_kernel<float>, grid, block, 0, stream, a.n_q_heads,
                       (const float*)a.q, (const float*)a.k_pool, (const float*)a.v_pool,
                       a.num_pages, a.table, a.n_table_rows, a.pages_per_row, a.rows,
                       a.positions, lo, (const float*)a.gate, a.scale, a.out);
  }
  return hipGetLastError();
}

}  // namespace qknr
