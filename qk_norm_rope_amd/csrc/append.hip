// K1 kernel and launcher: one workgroup of 256 threads per token. The device code
// (and the float32 order it fixes) is in append_body.h.
#include "append_body.h"
#include "kernels.h"

#pragma clang fp contract(off)

namespace qknr {
namespace {

template <typename TIn, typename TOut, bool WHOLE, bool PARTIAL>
__global__ __launch_bounds__(256) void qknorm_rope_append_kernel(
    int n_tokens, int n_q_heads, int n_kv_heads,
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ q_gain, const float* __restrict__ k_gain, float eps,
    const float* __restrict__ rope_cos, const float* __restrict__ rope_sin, int rope_rows,
    int rotary_dim,
    const int* __restrict__ positions, const int* __restrict__ slots, int n_slotted,
    const int* __restrict__ table, int pages_per_row, int64_t num_pages,
    TOut* __restrict__ q_out, TOut* __restrict__ k_pool, TOut* __restrict__ v_pool) {
  append_token<TIn, TOut, WHOLE, PARTIAL>(blockIdx.x, threadIdx.x, n_q_heads, n_kv_heads, q, k, v, q_gain,
                                          k_gain, eps, rope_cos, rope_sin, rope_rows, rotary_dim, positions,
                                          positions, n_tokens, slots, n_slotted, table, pages_per_row,
                                          num_pages, q_out, k_pool, v_pool);
}

}  // namespace

template <typename TI, typename TO>
static void launch_typed(hipStream_t stream, const AppendArgs& a) {
  const dim3 grid(a.n_tokens), block(256);
  const int rd = a.rotary_dim;
  const bool partial = rd != kHeadDim;
#define QKNR_APPEND(W, PT)                                                                 \
  hipLaunchKernelGGL((qknorm_rope_append_kernel<TI, TO, W, PT>), grid, block, 0, stream,     \
                     a.n_tokens, a.n_q_heads, a.n_kv_heads, (const TI*)a.q, (const TI*)a.k,             \
                     (const TI*)a.v, a.q_gain, a.k_gain, a.eps, a.rope_cos, a.rope_sin,     \
                     a.rope_rows, rd, a.positions, a.slots, a.n_slotted, a.table,           \
                     a.pages_per_row, a.num_pages, (TO*)a.q_out, (TO*)a.k_pool, (TO*)a.v_pool)
  if (a.norm_whole) {
    if (partial) QKNR_APPEND(true, true); else QKNR_APPEND(true, false);
  } else {
    if (partial) QKNR_APPEND(false, true); else QKNR_APPEND(false, false);
  }
#undef QKNR_APPEND
}

int append_max_whole_heads() { return kMaxWholeHeads; }

hipError_t launch_append(hipStream_t stream, const AppendArgs& a) {
  if (a.in_bf16 && a.out_bf16) launch_typed<uint16_t, uint16_t>(stream, a);
  else if (a.in_bf16) launch_typed<uint16_t, float>(stream, a);
  else if (a.out_bf16) launch_typed<float, uint16_t>(stream, a);
  else launch_typed<float, float>(stream, a);
  return hipGetLastError();
}

}  // namespace qknr
