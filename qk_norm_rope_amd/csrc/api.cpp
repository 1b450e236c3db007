// Host side of the C ABI declared in include/qknr.h: argument checks, workspace
// sizing, kernel selection and launches on the caller's stream.
//
// Every check runs before anything is enqueued (nest "models/qwen3-8b/files",
// README: names, shapes and dtypes are checked before anything runs;
// src/attention.linnet where-clause: Heads % KvHeads == 0, HeadDim even,
// PageSize > 0).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdint>

#include "qknr.h"
#include "kernels.h"

namespace {

constexpr int kHeadDimC = 128;
constexpr int kPageSizeC = 64;


int check_pool(const qkr_pool* pool) {
  if (!pool) return QKR_EINVAL;
  if (pool->num_q_heads <= 0 || pool->num_kv_heads <= 0 || pool->num_pages <= 0) return QKR_EINVAL;
  if (pool->num_q_heads % pool->num_kv_heads != 0) return QKR_EINVAL;
  if (pool->reserved != 0) return QKR_EINVAL;
  if (pool->dtype != QKR_F32 && pool->dtype != QKR_BF16) return QKR_EUNSUPPORTED;
  if (pool->head_dim != kHeadDimC || pool->page_size != kPageSizeC) return QKR_EUNSUPPORTED;
  if (pool->num_q_heads / pool->num_kv_heads != 4) return QKR_EUNSUPPORTED;
  // slot indices are formed in 64-bit; keep the element count of one pool addressable
  if (pool->num_pages > (int64_t(1) << 40) / (64 * 128)) return QKR_EUNSUPPORTED;
  return QKR_OK;
}

thread_local char g_last_error[256] = "";

int launch_status(hipError_t e) {
  if (e == hipSuccess) return QKR_OK;
  snprintf(g_last_error, sizeof(g_last_error), "%s (hipError %d)", hipGetErrorString(e), (int)e);
  return QKR_ELAUNCH;
}

// Attention options: the optional output gate; reserved fields must be zero.
int attn_opts(const qkr_attn_opts* opts, const void** gate) {
  *gate = nullptr;
  if (!opts) return QKR_OK;
  for (int i = 0; i < 6; ++i)
    if (opts->reserved[i] != 0) return QKR_EINVAL;
  *gate = opts->gate;
  return QKR_OK;
}

// Workspace of the packed form: the bfloat16 kernel's tile schedule, then the
// first visible position of every token.
size_t packed_workspace(const qkr_pool* pool, int32_t n_tokens) {
  const size_t lo = qknr::segment_start_bytes(n_tokens);
  if (pool->dtype != QKR_BF16) return lo;
  return qknr::prefill_workspace_bytes(n_tokens, pool->num_kv_heads) + lo;
}

int prefill_common(void* stream, const qkr_pool* pool, int32_t n_tokens,
                   const void* q, const void* k_pool, const void* v_pool,
                   const int32_t* table, int32_t n_table_rows, int32_t pages_per_row,
                   const int32_t* rows, const int32_t* positions, const int32_t* segments,
                   float scale, float* out, void* workspace, size_t workspace_bytes,
                   const qkr_attn_opts* opts) {
  const void* gate = nullptr;
  if (int os = attn_opts(opts, &gate)) return os;
  int st = check_pool(pool);
  if (st != QKR_OK) return st;
  if (n_tokens < 0) return QKR_EINVAL;
  if (n_tokens == 0) return QKR_OK;
  if (!q || !k_pool || !v_pool || !table || !rows || !positions || !out || n_table_rows <= 0 ||
      pages_per_row <= 0)
    return QKR_EINVAL;
  if (!std::isfinite(scale)) return QKR_EINVAL;
  qknr::AttnArgs a;
  a.n_queries = n_tokens;
  a.n_q_heads = pool->num_q_heads;
  a.n_kv_heads = pool->num_kv_heads;
  a.bf16 = pool->dtype == QKR_BF16;
  a.q = q; a.k_pool = k_pool; a.v_pool = v_pool;
  a.num_pages = pool->num_pages;
  a.table = table; a.n_table_rows = n_table_rows; a.pages_per_row = pages_per_row;
  a.rows = rows; a.positions = positions; a.segments = segments;
  a.scale = scale; a.out = out;
  a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  a.gate = gate;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t need = segments ? packed_workspace(pool, n_tokens)
                               : (a.bf16 ? qknr::prefill_workspace_bytes(n_tokens, pool->num_kv_heads) : 0);
  if (need > 0 && (!workspace || workspace_bytes < need)) return QKR_EWORKSPACE;
  if (!a.bf16) return launch_status(qknr::launch_attention_generic(s, a));
  if (pages_per_row > qknr::prefill_max_pages_per_row()) return QKR_EUNSUPPORTED;
  return launch_status(qknr::launch_prefill_bf16(s, a));
}

}  // namespace

extern "C" {

int qkr_version(void) { return 100; }

int qkr_mfma_probe(void* stream, int32_t iters, float* out, int64_t* flops) {
  if (!out || !flops || iters < 0) return QKR_EINVAL;
  long long f = 0;
  const int st = launch_status(qknr::launch_mfma_probe(static_cast<hipStream_t>(stream), iters, out, &f));
  *flops = st == QKR_OK ? (int64_t)f : 0;
  return st;
}

int qkr_read_probe(void* stream, const void* buf, size_t bytes, float* out) {
  if (!buf || !out || (reinterpret_cast<uintptr_t>(buf) & 15) != 0 || bytes % 16 != 0) return QKR_EINVAL;
  if (bytes == 0) return QKR_OK;
  return launch_status(qknr::launch_read_probe(static_cast<hipStream_t>(stream), buf, bytes, out));
}

const char* qkr_last_error(void) { return g_last_error; }

const char* qkr_status_str(int s) {
  switch (s) {
    case QKR_OK: return "ok";
    case QKR_EINVAL: return "invalid argument";
    case QKR_EUNSUPPORTED: return "unsupported shape or dtype";
    case QKR_EWORKSPACE: return "workspace missing or too small";
    case QKR_ELAUNCH: return "kernel launch failed";
    case QKR_EDATA: return "device data out of range";
    default: return "unknown status";
  }
}

int qkr_rope_table(double theta, int32_t rope_rows, int32_t head_dim, float* cos_out, float* sin_out) {
  if (!cos_out || !sin_out || rope_rows < 0 || head_dim <= 0 || head_dim % 2 != 0 || !(theta > 0.0))
    return QKR_EINVAL;
  const int half = head_dim / 2;
  for (int i = 0; i < half; ++i) {
    const double inv = 1.0 / std::pow(theta, (2.0 * i) / head_dim);
    for (int32_t pos = 0; pos < rope_rows; ++pos) {
      const double a = pos * inv;
      cos_out[(int64_t)pos * half + i] = (float)std::cos(a);
    }
    for (int32_t pos = 0; pos < rope_rows; ++pos) {
      const double a = pos * inv;
      sin_out[(int64_t)pos * half + i] = (float)std::sin(a);
    }
  }
  return QKR_OK;
}

int qknorm_rope_append_ex(void* stream, const qkr_pool* pool, int32_t n_tokens,
                          const void* q, const void* k, const void* v, int32_t in_dtype,
                          const float* q_gain, const float* k_gain, float eps,
                          const float* rope_cos, const float* rope_sin, int32_t rope_rows,
                          const int32_t* positions, const int32_t* slots, int32_t n_slotted,
                          const int32_t* table, int32_t pages_per_row,
                          void* q_out, void* k_pool, void* v_pool, const qkr_append_opts* opts) {
  int st = check_pool(pool);
  if (st != QKR_OK) return st;
  if (n_tokens < 0 || n_slotted < 0 || n_slotted > n_tokens) return QKR_EINVAL;
  if (in_dtype != QKR_F32 && in_dtype != QKR_BF16) return QKR_EUNSUPPORTED;
  bool whole = false;
  int rotary_dim = kHeadDimC;
  if (opts) {
    for (int i = 0; i < 6; ++i)
      if (opts->reserved[i] != 0) return QKR_EINVAL;
    if (opts->qk_norm_whole != 0 && opts->qk_norm_whole != 1) return QKR_EINVAL;
    whole = opts->qk_norm_whole == 1;
    if (opts->rotary_dim != 0) {
      if (opts->rotary_dim < 2 || opts->rotary_dim > kHeadDimC || opts->rotary_dim % 2 != 0) return QKR_EINVAL;
      rotary_dim = opts->rotary_dim;
    }
    if (whole && pool->num_q_heads + pool->num_kv_heads > qknr::append_max_whole_heads()) return QKR_EUNSUPPORTED;
  }
  if (n_tokens == 0) return QKR_OK;
  if (!q || !k || !v || !q_gain || !k_gain || !rope_cos || !rope_sin || !positions || !q_out ||
      !k_pool || !v_pool)
    return QKR_EINVAL;
  if (rope_rows <= 0) return QKR_EINVAL;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return QKR_EINVAL;
  if (n_slotted > 0 && !slots) return QKR_EINVAL;
  if (n_slotted < n_tokens && (!table || pages_per_row <= 0)) return QKR_EINVAL;
  qknr::AppendArgs a;
  a.n_tokens = n_tokens;
  a.n_q_heads = pool->num_q_heads;
  a.n_kv_heads = pool->num_kv_heads;
  a.q = q; a.k = k; a.v = v;
  a.in_bf16 = in_dtype == QKR_BF16;
  a.out_bf16 = pool->dtype == QKR_BF16;
  a.q_gain = q_gain; a.k_gain = k_gain; a.eps = eps;
  a.rope_cos = rope_cos; a.rope_sin = rope_sin; a.rope_rows = rope_rows;
  a.positions = positions; a.slots = slots; a.n_slotted = n_slotted;
  a.table = table; a.pages_per_row = pages_per_row; a.num_pages = pool->num_pages;
  a.q_out = q_out; a.k_pool = k_pool; a.v_pool = v_pool;
  a.norm_whole = whole;
  a.rotary_dim = rotary_dim;
  return launch_status(qknr::launch_append(static_cast<hipStream_t>(stream), a));
}

int qknorm_rope_append(void* stream, const qkr_pool* pool, int32_t n_tokens,
                       const void* q, const void* k, const void* v, int32_t in_dtype,
                       const float* q_gain, const float* k_gain, float eps,
                       const float* rope_cos, const float* rope_sin, int32_t rope_rows,
                       const int32_t* positions, const int32_t* slots, int32_t n_slotted,
                       const int32_t* table, int32_t pages_per_row,
                       void* q_out, void* k_pool, void* v_pool) {
  return qknorm_rope_append_ex(stream, pool, n_tokens, q, k, v, in_dtype, q_gain, k_gain, eps,
                               rope_cos, rope_sin, rope_rows, positions, slots, n_slotted, table,
                               pages_per_row, q_out, k_pool, v_pool, nullptr);
}

size_t paged_decode_attn_workspace(const qkr_pool* pool, int32_t n_rows, int32_t pages_per_row) {
  if (check_pool(pool) != QKR_OK || n_rows <= 0 || pages_per_row <= 0) return 0;
  if (pool->dtype != QKR_BF16) return 0;
  return qknr::decode_workspace_bytes(n_rows, pool->num_kv_heads, pages_per_row);
}

const char* paged_decode_attn_kernel(const qkr_pool* pool, int32_t n_rows, int32_t pages_per_row) {
  if (check_pool(pool) != QKR_OK || n_rows <= 0 || pages_per_row <= 0) return "";
  if (pool->dtype != QKR_BF16) return "attention_generic_kernel";
  return qknr::decode_uses_small_kernel(n_rows, pool->num_kv_heads, pages_per_row) ? "paged_decode_small_kernel"
                                                                                   : "paged_decode_bf16_kernel";
}

int paged_decode_attn_ex(void* stream, const qkr_pool* pool, int32_t n_rows,
                         const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* table, int32_t pages_per_row,
                         const int32_t* positions, float scale, float* out,
                         void* workspace, size_t workspace_bytes, const qkr_attn_opts* opts) {
  const void* gate = nullptr;
  if (int os = attn_opts(opts, &gate)) return os;
  int st = check_pool(pool);
  if (st != QKR_OK) return st;
  if (n_rows < 0) return QKR_EINVAL;
  if (n_rows == 0) return QKR_OK;
  if (!q || !k_pool || !v_pool || !table || !positions || !out || pages_per_row <= 0) return QKR_EINVAL;
  if (!std::isfinite(scale)) return QKR_EINVAL;
  qknr::AttnArgs a;
  a.n_queries = n_rows;
  a.n_q_heads = pool->num_q_heads;
  a.n_kv_heads = pool->num_kv_heads;
  a.bf16 = pool->dtype == QKR_BF16;
  a.q = q; a.k_pool = k_pool; a.v_pool = v_pool;
  a.num_pages = pool->num_pages;
  a.table = table; a.n_table_rows = n_rows; a.pages_per_row = pages_per_row;
  a.rows = nullptr; a.positions = positions; a.scale = scale; a.out = out;
  a.workspace = workspace; a.workspace_bytes = workspace_bytes;
  a.gate = gate;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!a.bf16) return launch_status(qknr::launch_attention_generic(s, a));
  if (n_rows > qknr::decode_max_rows()) return QKR_EUNSUPPORTED;
  if (!qknr::decode_cost_fits(n_rows, pool->num_kv_heads, pages_per_row)) return QKR_EUNSUPPORTED;
  const size_t need = qknr::decode_workspace_bytes(n_rows, pool->num_kv_heads, pages_per_row);
  if (!workspace || workspace_bytes < need) return QKR_EWORKSPACE;
  return launch_status(qknr::launch_decode_bf16(s, a));
}

int paged_decode_attn(void* stream, const qkr_pool* pool, int32_t n_rows,
                      const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* table, int32_t pages_per_row,
                      const int32_t* positions, float scale, float* out,
                      void* workspace, size_t workspace_bytes) {
  return paged_decode_attn_ex(stream, pool, n_rows, q, k_pool, v_pool, table, pages_per_row,
                              positions, scale, out, workspace, workspace_bytes, nullptr);
}

int paged_decode_attn_noalloc(void* stream, const qkr_pool* pool, int32_t n_rows,
                              const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* table, int32_t pages_per_row,
                              const int32_t* positions, float scale, float* out) {
  int st = check_pool(pool);
  if (st != QKR_OK) return st;
  if (n_rows < 0) return QKR_EINVAL;
  if (n_rows == 0) return QKR_OK;
  if (!q || !k_pool || !v_pool || !table || !positions || !out || pages_per_row <= 0) return QKR_EINVAL;
  if (!std::isfinite(scale)) return QKR_EINVAL;
  const bool bf16 = pool->dtype == QKR_BF16;
  if (bf16 && n_rows > qknr::decode_max_rows()) return QKR_EUNSUPPORTED;
  if (bf16 && !qknr::decode_cost_fits(n_rows, pool->num_kv_heads, pages_per_row)) return QKR_EUNSUPPORTED;
  if (bf16 && (int64_t)n_rows * pool->num_kv_heads > qknr::decode_noalloc_max_pairs()) {
    snprintf(g_last_error, sizeof(g_last_error),
             "paged_decode_attn_noalloc: %d rows x %d KV heads exceed the scratch limit of %d (row, KV head) "
             "pairs; use paged_decode_attn with a workspace",
             (int)n_rows, (int)pool->num_kv_heads, qknr::decode_noalloc_max_pairs());
    return QKR_EUNSUPPORTED;
  }
  qknr::AttnArgs a;
  a.n_queries = n_rows;
  a.n_q_heads = pool->num_q_heads;
  a.n_kv_heads = pool->num_kv_heads;
  a.bf16 = bf16;
  a.q = q; a.k_pool = k_pool; a.v_pool = v_pool;
  a.num_pages = pool->num_pages;
  a.table = table; a.n_table_rows = n_rows; a.pages_per_row = pages_per_row;
  a.rows = nullptr; a.positions = positions; a.scale = scale; a.out = out;
  a.workspace = nullptr; a.workspace_bytes = 0;
  a.gate = nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!bf16) return launch_status(qknr::launch_attention_generic(s, a));   // needs no scratch
  return launch_status(qknr::launch_decode_bf16_noalloc(s, a));
}

size_t paged_prefill_attn_workspace(const qkr_pool* pool, int32_t n_tokens) {
  if (check_pool(pool) != QKR_OK || n_tokens <= 0) return 0;
  if (pool->dtype != QKR_BF16) return 0;
  return qknr::prefill_workspace_bytes(n_tokens, pool->num_kv_heads);
}

int paged_prefill_attn_ex(void* stream, const qkr_pool* pool, int32_t n_tokens,
                          const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* table, int32_t n_table_rows, int32_t pages_per_row,
                          const int32_t* rows, const int32_t* positions,
                          float scale, float* out, void* workspace, size_t workspace_bytes,
                          const qkr_attn_opts* opts) {
  return prefill_common(stream, pool, n_tokens, q, k_pool, v_pool, table, n_table_rows,
                        pages_per_row, rows, positions, nullptr, scale, out, workspace,
                        workspace_bytes, opts);
}

int paged_prefill_attn(void* stream, const qkr_pool* pool, int32_t n_tokens,
                       const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* table, int32_t n_table_rows, int32_t pages_per_row,
                       const int32_t* rows, const int32_t* positions,
                       float scale, float* out, void* workspace, size_t workspace_bytes) {
  return paged_prefill_attn_ex(stream, pool, n_tokens, q, k_pool, v_pool, table, n_table_rows,
                               pages_per_row, rows, positions, scale, out, workspace,
                               workspace_bytes, nullptr);
}

size_t packed_prefill_attn_workspace(const qkr_pool* pool, int32_t n_tokens) {
  if (check_pool(pool) != QKR_OK || n_tokens <= 0) return 0;
  return packed_workspace(pool, n_tokens);
}

int packed_prefill_attn_ex(void* stream, const qkr_pool* pool, int32_t n_tokens,
                           const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* table, int32_t n_table_rows, int32_t pages_per_row,
                           const int32_t* rows, const int32_t* positions, const int32_t* segments,
                           float scale, float* out, void* workspace, size_t workspace_bytes,
                           const qkr_attn_opts* opts) {
  if (!segments && n_tokens > 0) return QKR_EINVAL;
  return prefill_common(stream, pool, n_tokens, q, k_pool, v_pool, table, n_table_rows,
                        pages_per_row, rows, positions, segments, scale, out, workspace,
                        workspace_bytes, opts);
}

int packed_prefill_attn(void* stream, const qkr_pool* pool, int32_t n_tokens,
                        const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* table, int32_t n_table_rows, int32_t pages_per_row,
                        const int32_t* rows, const int32_t* positions, const int32_t* segments,
                        float scale, float* out, void* workspace, size_t workspace_bytes) {
  return packed_prefill_attn_ex(stream, pool, n_tokens, q, k_pool, v_pool, table, n_table_rows,
                                pages_per_row, rows, positions, segments, scale, out, workspace,
                                workspace_bytes, nullptr);
}

int qkr_check_indices(void* stream, const qkr_pool* pool,
                      const int32_t* table, int32_t n_table_rows, int32_t pages_per_row,
                      int32_t n_tokens, const int32_t* rows, const int32_t* positions, const int32_t* slots,
                      int32_t n_decode, const int32_t* step_positions, int32_t decode_row0,
                      int32_t rope_rows, int32_t* counts, int32_t wait) {
  static_assert(QKR_CHECK_ROW == qknr::kCheckRow && QKR_CHECK_POSITION == qknr::kCheckPosition &&
                    QKR_CHECK_PAGE == qknr::kCheckPage && QKR_CHECK_SLOT_RANGE == qknr::kCheckSlotRange &&
                    QKR_CHECK_SLOT_MISMATCH == qknr::kCheckSlotMismatch && QKR_CHECK_COUNTS == qknr::kCheckCounts,
                "count layout");
  int st = check_pool(pool);
  if (st != QKR_OK) return st;
  if (n_tokens < 0 || n_decode < 0 || rope_rows < 0) return QKR_EINVAL;
  if (!counts || !table || n_table_rows <= 0 || pages_per_row <= 0) return QKR_EINVAL;
  if (n_tokens > 0 && (!rows || !positions)) return QKR_EINVAL;
  if (n_decode > 0) {
    if (!step_positions) return QKR_EINVAL;
    if (decode_row0 < 0 || (int64_t)decode_row0 + n_decode > n_table_rows) return QKR_EINVAL;
  }
  if ((int64_t)n_tokens + n_decode > (int64_t)1 << 30) return QKR_EUNSUPPORTED;
  qknr::CheckArgs a;
  a.table = table;
  a.n_table_rows = n_table_rows;
  a.pages_per_row = pages_per_row;
  a.num_pages = pool->num_pages;
  a.n_tokens = n_tokens;
  a.rows = rows;
  a.positions = positions;
  a.slots = slots;
  a.n_decode = n_decode;
  a.step_positions = step_positions;
  a.decode_row0 = decode_row0;
  a.rope_rows = rope_rows;
  a.counts = counts;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = launch_status(qknr::launch_check_indices(s, a));
  if (st != QKR_OK || !wait) return st;
  int32_t host[QKR_CHECK_COUNTS];
  st = launch_status(hipMemcpyAsync(host, counts, sizeof(host), hipMemcpyDeviceToHost, s));
  if (st != QKR_OK) return st;
  st = launch_status(hipStreamSynchronize(s));
  if (st != QKR_OK) return st;
  for (int i = 0; i < QKR_CHECK_COUNTS; ++i)
    if (host[i] != 0) {
      snprintf(g_last_error, sizeof(g_last_error),
               "qkr_check_indices: %d bad rows, %d bad positions, %d queries with a page outside the pool, "
               "%d slots outside the pool, %d slots that differ from their row's page table",
               host[QKR_CHECK_ROW], host[QKR_CHECK_POSITION], host[QKR_CHECK_PAGE], host[QKR_CHECK_SLOT_RANGE],
               host[QKR_CHECK_SLOT_MISMATCH]);
      return QKR_EDATA;
    }
  return QKR_OK;
}

size_t step_paged_workspace(const qkr_pool* pool, int32_t n_prefill, int32_t n_decode, int32_t pages_per_row) {
  if (check_pool(pool) != QKR_OK || n_prefill < 0 || n_decode < 0 || pages_per_row <= 0) return 0;
  if (pool->dtype != QKR_BF16) return 0;
  return qknr::step_workspace_bytes(n_prefill, n_decode, pool->num_kv_heads, pages_per_row);
}

int step_paged(void* stream, const qkr_pool* pool, int32_t n_prefill, int32_t n_decode,
               const void* q, const void* k, const void* v, int32_t in_dtype,
               const float* q_gain, const float* k_gain, float eps,
               const float* rope_cos, const float* rope_sin, int32_t rope_rows,
               const int32_t* positions, const int32_t* rows, const int32_t* slots,
               const int32_t* step_positions,
               const int32_t* table, int32_t n_table_rows, int32_t pages_per_row, int32_t decode_row0,
               float scale, void* q_out, void* k_pool, void* v_pool,
               float* prefill_out, float* decode_out, void* workspace, size_t workspace_bytes) {
  int st = check_pool(pool);
  if (st != QKR_OK) return st;
  if (n_prefill < 0 || n_decode < 0) return QKR_EINVAL;
  if (in_dtype != QKR_F32 && in_dtype != QKR_BF16) return QKR_EUNSUPPORTED;
  if (pool->dtype != QKR_BF16 || in_dtype != QKR_BF16) return QKR_EUNSUPPORTED;
  if (n_prefill == 0 && n_decode == 0) return QKR_OK;
  if ((int64_t)n_prefill + n_decode > (int64_t)1 << 30) return QKR_EUNSUPPORTED;
  if (!q || !k || !v || !q_gain || !k_gain || !rope_cos || !rope_sin || !table || !q_out || !k_pool ||
      !v_pool)
    return QKR_EINVAL;
  if (rope_rows <= 0 || n_table_rows <= 0 || pages_per_row <= 0) return QKR_EINVAL;
  if (!(eps >= 0.0f) || !std::isfinite(eps) || !std::isfinite(scale)) return QKR_EINVAL;
  if (n_prefill > 0 && (!positions || !rows || !slots || !prefill_out)) return QKR_EINVAL;
  if (n_decode > 0) {
    if (!step_positions || !decode_out) return QKR_EINVAL;
    if (decode_row0 < 0 || (int64_t)decode_row0 + n_decode > n_table_rows) return QKR_EINVAL;
    if (n_decode > qknr::step_max_rows()) return QKR_EUNSUPPORTED;
    if (!qknr::decode_cost_fits(n_decode, pool->num_kv_heads, pages_per_row)) return QKR_EUNSUPPORTED;
  }
  if (pages_per_row > qknr::prefill_max_pages_per_row()) return QKR_EUNSUPPORTED;
  const size_t need = qknr::step_workspace_bytes(n_prefill, n_decode, pool->num_kv_heads, pages_per_row);
  if (!workspace || workspace_bytes < need) return QKR_EWORKSPACE;
  if (!qknr::step_enabled()) {
    snprintf(g_last_error, sizeof(g_last_error),
             "step_paged: the single-launch kernel is switched off in this version of the library; "
             "call qknorm_rope_append, paged_prefill_attn and paged_decode_attn");
    return QKR_EUNSUPPORTED;
  }
  qknr::StepArgs a;
  a.n_prefill = n_prefill;
  a.n_decode = n_decode;
  a.n_q_heads = pool->num_q_heads;
  a.n_kv_heads = pool->num_kv_heads;
  a.q = q; a.k = k; a.v = v;
  a.q_gain = q_gain; a.k_gain = k_gain; a.eps = eps;
  a.rope_cos = rope_cos; a.rope_sin = rope_sin; a.rope_rows = rope_rows;
  a.positions = positions; a.step_positions = step_positions; a.rows = rows; a.slots = slots;
  a.table = table; a.n_table_rows = n_table_rows; a.pages_per_row = pages_per_row;
  a.decode_row0 = n_decode > 0 ? decode_row0 : 0;
  a.num_pages = pool->num_pages;
  a.scale = scale;
  a.q_out = q_out; a.k_pool = k_pool; a.v_pool = v_pool;
  a.prefill_out = prefill_out; a.decode_out = decode_out;
  a.workspace = workspace;
  return launch_status(qknr::launch_step(static_cast<hipStream_t>(stream), a));
}

}  // extern "C"
