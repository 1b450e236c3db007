// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qknr {

struct AppendArgs {
  int n_tokens, n_q_heads, n_kv_heads;
  const void *q, *k, *v;
  bool in_bf16, out_bf16;
  const float *q_gain, *k_gain;
  float eps;
  const float *rope_cos, *rope_sin;
  int rope_rows;
  const int32_t *positions, *slots;
  int n_slotted;
  const int32_t* table;
  int pages_per_row;
  int64_t num_pages;
  void *q_out, *k_pool, *v_pool;
  bool norm_whole = false;   // one RMS norm over all heads (gains heads*head_dim wide)
  int rotary_dim = 128;      // elements of each head that rotate (pairs (i, i + rotary_dim/2))
};

struct AttnArgs {
  int n_queries;          // decode rows, or prefill tokens
  int n_q_heads, n_kv_heads;
  bool bf16;              // pool / q dtype
  const void* q;
  const void *k_pool, *v_pool;
  int64_t num_pages;
  const int32_t* table;
  int n_table_rows, pages_per_row;
  const int32_t* rows;    // prefill: row of each token; decode: nullptr (row = index)
  const int32_t* positions;
  const int32_t* segments = nullptr;   // packed prefill: prompt of each token, else nullptr
  const void* gate = nullptr;          // optional output gate (pool dtype), out *= sigmoid(gate)
  float scale;
  float* out;
  void* workspace;
  size_t workspace_bytes;
};

hipError_t launch_append(hipStream_t stream, const AppendArgs& a);
int append_max_whole_heads();

// Decode: split-K over page ranges with a fused last-arriver merge.
size_t decode_workspace_bytes(int n_rows, int n_kv_heads, int pages_per_row);
int decode_max_rows();
// true when rows x KV heads x pages per row stay within the split's 32-bit cost scale
bool decode_cost_fits(int n_rows, int n_kv_heads, int pages_per_row);
hipError_t launch_decode_bf16(hipStream_t stream, const AttnArgs& a);
// true when launch_decode_bf16 takes the (row, KV head, chunk) kernel on the current device
bool decode_uses_small_kernel(int n_rows, int n_kv_heads, int pages_per_row);
// The same kernel on the library's own per-device scratch (no workspace argument,
// no allocation); rows x KV heads at most decode_noalloc_max_pairs().
int decode_noalloc_max_pairs();
hipError_t launch_decode_bf16_noalloc(hipStream_t stream, const AttnArgs& a);

// Prefill: MFMA flash attention over 64-token tiles of the pack.
size_t prefill_workspace_bytes(int n_tokens, int n_kv_heads);
int prefill_max_pages_per_row();
// With a.segments set, the workspace continues after prefill_workspace_bytes with
// segment_start_bytes of first visible positions.
hipError_t launch_prefill_bf16(hipStream_t stream, const AttnArgs& a);

// Packed form: first visible position of every token (its segment's first position).
size_t segment_start_bytes(int n_tokens);
hipError_t launch_segment_start(hipStream_t stream, int n_tokens, const int32_t* positions,
                                const int32_t* segments, int32_t* lo);

// One workgroup per (query, KV head); any pool dtype. Used for float32 pools. With
// a.segments set, the first segment_start_bytes of the workspace take the first
// visible positions.
hipError_t launch_attention_generic(hipStream_t stream, const AttnArgs& a);

// Single-launch mixed step: append over the prompt tokens and the decode rows,
// then prefill attention over the prompt tokens and decode attention over the rows,
// in one persistent kernel (bfloat16 inputs and pool).
struct StepArgs {
  int n_prefill, n_decode, n_q_heads, n_kv_heads;
  const void *q, *k, *v;
  const float *q_gain, *k_gain;
  float eps;
  const float *rope_cos, *rope_sin;
  int rope_rows;
  const int32_t *positions, *step_positions, *rows, *slots, *table;
  int n_table_rows, pages_per_row, decode_row0;
  int64_t num_pages;
  float scale;
  void *q_out, *k_pool, *v_pool;
  float *prefill_out, *decode_out;
  void* workspace;
  int decode_slices = 0;   // decode work items (0: one per resident workgroup)
};
// Device-data validation: counts of index violations, kCheckCounts ints in device
// memory (the order of QKR_CHECK_* in qknr.h).
enum : int { kCheckRow = 0, kCheckPosition, kCheckPage, kCheckSlotRange, kCheckSlotMismatch, kCheckCounts = 8 };
struct CheckArgs {
  const int32_t* table;
  int n_table_rows, pages_per_row;
  int64_t num_pages;
  int n_tokens;
  const int32_t *rows, *positions, *slots;
  int n_decode;
  const int32_t* step_positions;
  int decode_row0;
  int rope_rows;   // 0: no rotation-table limit
  int32_t* counts;
};
// plain streaming read of bytes (a multiple of 16) at buf, 16-byte aligned
hipError_t launch_read_probe(hipStream_t stream, const void* buf, size_t bytes, float* out);
// `iters` rounds of 8 bf16 32x32x16 MFMAs per wave, 8 waves per CU; *flops: the FLOPs enqueued
hipError_t launch_mfma_probe(hipStream_t stream, int iters, float* out, long long* flops);

hipError_t launch_check_indices(hipStream_t stream, const CheckArgs& a);

size_t step_workspace_bytes(int n_prefill, int n_decode, int n_kv_heads, int pages_per_row);
// Whether step_paged launches its kernel (off until the kernel has passed its GPU tests).
bool step_enabled();
int step_max_rows();
hipError_t launch_step(hipStream_t stream, const StepArgs& a);

}  // namespace qknr
