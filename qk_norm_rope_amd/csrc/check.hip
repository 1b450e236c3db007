// Device-data validation: counts the index violations that the append and the
// attention kernels would otherwise only range-check (they skip or mask what is out
// of range, so bad indices pass silently there). nest "models/qwen3-8b/files",
// README: every name, shape and dtype is checked before anything runs; Entries
// table: a row's positions lie in the pages its table row lists, pages of 64.
//
// One wave per query (prompt token or decode row): lane 0 checks the row, the
// position and the slot, and the 64 lanes walk the table entries of the pages the
// query sees (0 .. position / 64), so a long row is read 64 entries at a time. Each
// kind of violation is counted once per query with one agent-scope atomic add per
// wave; the counters are zeroed by a fill kernel launched first on the same stream.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace qknr {
namespace {

struct CheckParams {
  const int* table;
  int n_table_rows, pages_per_row;
  int64_t num_pages;
  int n_tokens;                 // prompt tokens (rows, positions, slots)
  const int *rows, *positions, *slots;
  int n_decode;                 // decode rows (step_positions, table row decode_row0 + b)
  const int* step_positions;
  int decode_row0;
  int rope_rows;
  int* counts;                  // kCheckCounts ints
};

__global__ __launch_bounds__(256) void zero_counts_kernel(int* counts) {
  if (threadIdx.x < kCheckCounts) counts[threadIdx.x] = 0;
}

__global__ __launch_bounds__(256) void check_indices_kernel(CheckParams P) {
  const int lane = threadIdx.x & 63;
  const int q = blockIdx.x * 4 + (threadIdx.x >> 6);   // query index: prompt tokens, then decode rows
  if (q >= P.n_tokens + P.n_decode) return;
  // positions the page table reaches, and the rotation table when one is given
  int64_t max_pos = (int64_t)P.pages_per_row * kPageSize;
  if (P.rope_rows > 0 && P.rope_rows < max_pos) max_pos = P.rope_rows;
  int row, pos, slot = -1;
  if (q < P.n_tokens) {
    row = P.rows[q];
    pos = P.positions[q];
    if (P.slots) slot = P.slots[q];
  } else {
    row = P.decode_row0 + (q - P.n_tokens);
    pos = P.step_positions[q - P.n_tokens];
  }
  const bool row_bad = row < 0 || row >= P.n_table_rows;
  const bool pos_bad = pos < 0 || pos >= max_pos;
  // pages the query sees: table entries 0 .. pos / 64 of its row
  bool page_bad = false;
  if (!row_bad && !pos_bad) {
    const int* trow = P.table + (int64_t)row * P.pages_per_row;
    const int n_pages = pos / kPageSize + 1;
    for (int i = lane; i < n_pages; i += 64) {
      const int id = trow[i];
      page_bad |= id < 0 || id >= P.num_pages;
    }
  }
  page_bad = __any(page_bad);
  bool slot_range = false, slot_mismatch = false;
  if (q < P.n_tokens && P.slots && slot >= 0) {
    const int64_t pool_slots = P.num_pages * kPageSize;
    slot_range = slot >= pool_slots;
    if (!row_bad && !pos_bad) {
      const int64_t page = P.table[(int64_t)row * P.pages_per_row + pos / kPageSize];
      slot_mismatch = (int64_t)slot != page * kPageSize + pos % kPageSize;
    }
  }
  if (lane == 0) {
    if (q < P.n_tokens && row_bad) atomicAdd(&P.counts[kCheckRow], 1);
    if (pos_bad) atomicAdd(&P.counts[kCheckPosition], 1);
    if (page_bad) atomicAdd(&P.counts[kCheckPage], 1);
    if (slot_range) atomicAdd(&P.counts[kCheckSlotRange], 1);
    if (slot_mismatch) atomicAdd(&P.counts[kCheckSlotMismatch], 1);
  }
}

}  // namespace

hipError_t launch_check_indices(hipStream_t stream, const CheckArgs& a) {
  CheckParams P;
  P.table = a.table;
  P.n_table_rows = a.n_table_rows;
  P.pages_per_row = a.pages_per_row;
  P.num_pages = a.num_pages;
  P.n_tokens = a.n_tokens;
  P.rows = a.rows;
  P.positions = a.positions;
  P.slots = a.slots;
  P.n_decode = a.n_decode;
  P.step_positions = a.step_positions;
  P.decode_row0 = a.decode_row0;
  P.rope_rows = a.rope_rows;
  P.counts = a.counts;
  hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(256), 0, stream, a.counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = a.n_tokens + a.n_decode;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(check_indices_kernel, dim3((n + 3) / 4), dim3(256), 0, stream, P);
  return hipGetLastError();
}

}  // namespace qknr
