/*
 * qknr.h -- C ABI of libqknr: paged QK-norm + RoPE + grouped-query attention
 * for AMD Instinct MI355X (gfx950).
 *
 * The operations are the attention step of a Qwen3-style decoder serving from a
 * paged KV cache, as the nest "models/qwen3-8b/files" page states them
 * (README: architecture paragraph and Entries table; src/attention.linnet:
 * decode_paged, prefill_paged, step_paged, split_heads; src/norm.linnet;
 * src/rope.linnet), with the loop form of fantasma "src/inference/model.zig"
 * (fullAttentionForward, applyRope).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Streams: `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   Every call only enqueues work on that stream; nothing synchronises, nothing
 *   allocates device memory, and the library keeps no state between calls, so
 *   calls are thread-safe. Ordering (append before attention) comes from the
 *   stream. The one exception is paged_decode_attn_noalloc, which works in a
 *   library-owned scratch array per GPU (see there).
 * - Ownership: the caller owns every buffer. Device pointers must stay valid
 *   until the enqueued work has finished.
 * - Activations are token-major: q is [n][num_q_heads*head_dim] and k, v are
 *   [n][num_kv_heads*head_dim]; head h occupies columns h*head_dim ..
 *   h*head_dim+head_dim-1 (attention.linnet, split_heads / merge_heads).
 * - Pools: k_pool and v_pool are [num_kv_heads][num_pages*page_size][head_dim]
 *   in the pool dtype (cache_k / cache_v of attention.linnet with Batch = 1:
 *   one row that is a pool of pages). Position p of a row whose page list is
 *   table[r][0..pages_per_row) lives in slot table[r][p / page_size]*page_size
 *   + p % page_size (Entries table, decode_paged).
 * - Tables are int32 [n_table_rows][pages_per_row], row-major.
 * - Positions are 0-based. A query at position p sees positions 0..p of its
 *   row, its own included (attention.linnet, decode: keys up to and including
 *   the query's position).
 * - Query head h reads KV head h / (num_q_heads / num_kv_heads) (model.zig,
 *   fullAttentionForward).
 * - Errors: a negative qkr_status is returned before anything is enqueued when
 *   an argument is invalid; QKR_ELAUNCH when the runtime refuses a launch.
 *   Device-side data (page ids, positions, slots, rows) is not validated
 *   against the caller's intent, but every index the kernels form is range
 *   checked, so bad data never causes an out-of-bounds access: a query whose
 *   position or row is out of range gets NaN outputs; a page id outside the pool
 *   makes the keys of that page invisible (the output is then unspecified but
 *   finite); an out-of-range slot skips the write.
 * - The kernels are built for head_dim 128 and page_size 64; other values
 *   return QKR_EUNSUPPORTED.
 */
#ifndef QKNR_H
#define QKNR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { QKR_F32 = 0, QKR_BF16 = 1 } qkr_dtype;

typedef enum {
  QKR_OK = 0,
  QKR_EINVAL = -1,          /* null pointer, negative count, bad divisibility  */
  QKR_EUNSUPPORTED = -2,    /* head_dim != 128, page_size != 64, dtype combo    */
  QKR_EWORKSPACE = -3,      /* workspace missing or smaller than required       */
  QKR_ELAUNCH = -4,         /* the HIP runtime reported an error on launch      */
  QKR_EDATA = -5            /* qkr_check_indices found out-of-range device data */
} qkr_status;

/* Shape of the paged pool. num_q_heads % num_kv_heads == 0 and the group size
 * num_q_heads / num_kv_heads must be 4 for the bfloat16 attention kernels
 * (attention.linnet where-clause: Heads % KvHeads == 0). */
typedef struct qkr_pool {
  int32_t num_q_heads;   /* 32 for Qwen3-8B                                   */
  int32_t num_kv_heads;  /* 8 for Qwen3-8B                                    */
  int32_t head_dim;      /* 128                                               */
  int32_t page_size;     /* 64                                                */
  int64_t num_pages;     /* pool capacity in pages                            */
  int32_t dtype;         /* qkr_dtype of k_pool, v_pool and q_out             */
  int32_t reserved;      /* must be 0                                         */
} qkr_pool;

/*
 * qknorm_rope_append -- QK-norm, RoPE and the cache write for n_tokens tokens.
 *
 * For every token t and every query head / KV head slice x (head_dim wide):
 *   y = x * (mean(x^2) + eps)^(-1/2) * gain   (gain = q_gain or k_gain, shared
 *                                              by all heads; norm.linnet with
 *                                              eps 1e-6, applied after the
 *                                              split into heads, README)
 *   then RoPE at positions[t]: element i and i + head_dim/2 rotate by the angle
 *   whose cosine/sine are rope_cos/rope_sin[positions[t]][i] (model.zig,
 *   applyRope; rope.linnet, tables).
 * Rotated q goes to q_out[t] (pool dtype). Rotated k and raw v (only cast to the
 * pool dtype) go to slot s of every KV head of k_pool / v_pool, where
 *   s = slots[t]                                   for t <  n_slotted
 *     (prefill_paged: the caller gives each prompt token its slot), and
 *   s = table[b][p / 64]*64 + p % 64, b = t - n_slotted, p = positions[t]
 *                                                  for t >= n_slotted
 *     (decode_paged: row b's slot from its page table).
 * A negative slot skips the write (padding). This covers step_paged's single
 * norm + rope + write over prompt tokens followed by decode rows.
 *
 * The float32 arithmetic is fixed so that q_out and the written pool bytes are
 * reproducible bit for bit: squares summed in pairs (i, i+64), then a pairwise
 * tree over i, mean by an exact /128, r = 1/sqrt(ms + eps) correctly rounded,
 * y = (x*r)*g, rotation without fused multiply-add, round-to-nearest-even store.
 *
 * q, k, v      : device, in_dtype, shapes above.
 * q_gain/k_gain: device float32 [head_dim].
 * rope_cos/sin : device float32 [rope_rows][head_dim/2] (see qkr_rope_table).
 * positions    : device int32 [n_tokens], each in [0, rope_rows).
 * slots        : device int32 [n_slotted] (may be NULL when n_slotted == 0).
 * table        : device int32 [n_tokens - n_slotted][pages_per_row] (may be NULL
 *                when n_slotted == n_tokens).
 * q_out        : device, pool dtype, [n_tokens][num_q_heads*head_dim].
 * n_tokens == 0 is a no-op.
 */
int qknorm_rope_append(void* stream, const qkr_pool* pool, int32_t n_tokens,
                       const void* q, const void* k, const void* v, int32_t in_dtype,
                       const float* q_gain, const float* k_gain, float eps,
                       const float* rope_cos, const float* rope_sin, int32_t rope_rows,
                       const int32_t* positions,
                       const int32_t* slots, int32_t n_slotted,
                       const int32_t* table, int32_t pages_per_row,
                       void* q_out, void* k_pool, void* v_pool);

/* Options of qknorm_rope_append_ex. A null pointer, or all fields 0, gives
 * qknorm_rope_append. */
typedef struct qkr_append_opts {
  int32_t qk_norm_whole;  /* 1: one RMS norm over all heads of q and one over all
                             heads of k (logicaffeine author.rs, qk_norm_segments
                             with qk_norm_whole); q_gain then has
                             num_q_heads*head_dim entries and k_gain
                             num_kv_heads*head_dim (head h at h*head_dim..).
                             num_q_heads + num_kv_heads <= 256 (else
                             QKR_EUNSUPPORTED). 0: per head (default).          */
  int32_t rotary_dim;     /* R: only elements 0..R-1 of each head rotate, pairs
                             (i, i + R/2), with rope_cos/rope_sin of width R/2
                             (qkr_rope_table with head_dim = R); elements R.. pass
                             unchanged (model.zig applyRope, rotary_dim). Even,
                             2..head_dim; 0 means head_dim (default).           */
  int32_t reserved[6];    /* must be 0                                          */
} qkr_append_opts;

/*
 * qknorm_rope_append_ex -- qknorm_rope_append with the options above (the
 * attention variants of the pages: whole-vector QK-norm, partial rotary). The
 * float32 order of the whole-vector norm: each head's sum of squares as in the
 * per-head norm, then the head sums added pairwise (neighbours first, an odd last
 * one carried up), ms = total / (heads*head_dim), r = 1/sqrt(ms + eps).
 * Invalid options return QKR_EINVAL before anything is enqueued.
 */
int qknorm_rope_append_ex(void* stream, const qkr_pool* pool, int32_t n_tokens,
                          const void* q, const void* k, const void* v, int32_t in_dtype,
                          const float* q_gain, const float* k_gain, float eps,
                          const float* rope_cos, const float* rope_sin, int32_t rope_rows,
                          const int32_t* positions,
                          const int32_t* slots, int32_t n_slotted,
                          const int32_t* table, int32_t pages_per_row,
                          void* q_out, void* k_pool, void* v_pool,
                          const qkr_append_opts* opts);

/* Options of the *_ex attention calls. A null pointer, or all fields 0, gives the
 * plain call. */
typedef struct qkr_attn_opts {
  const void* gate;       /* optional, device, pool dtype, [n][num_q_heads*head_dim]
                             in the layout of out: every output element is
                             multiplied by sigmoid(gate) (model.zig,
                             fullAttentionForward, output gate). null: no gate. */
  int32_t reserved[6];    /* must be 0                                          */
} qkr_attn_opts;

/*
 * paged_decode_attn -- one query token per row over that row's pages
 * (attention.linnet, decode_paged / paged_attention).
 *
 * Row b's query q[b] (pool dtype, [n_rows][num_q_heads*head_dim], normally the
 * q_out of qknorm_rope_append) attends with each query head over positions
 * 0..positions[b] of table row b:
 *   out[b][h] = sum_j softmax_j(scale * <q_bh, K_j>) V_j
 * out is float32 [n_rows][num_q_heads*head_dim]. The work is split over page
 * ranges (flash decoding) and the partial softmax states are merged exactly;
 * the split depends only on positions, so the result does not depend on where
 * the pages sit in the pool.
 *
 * A bfloat16 pool takes at most 12288 rows per call, and n_rows * num_kv_heads *
 * (5 * pages_per_row + 12) must stay below 2^31 (the split's cost scale; 12288
 * rows of 8 KV heads allow 4366 pages per row); beyond either, QKR_EUNSUPPORTED.
 * workspace: device memory of at least paged_decode_attn_workspace() bytes. It
 * must be zero-filled before its first use; every call leaves it ready for the
 * next (its counters return to zero). Calls that share a workspace must be
 * ordered on one stream.
 */
int paged_decode_attn(void* stream, const qkr_pool* pool, int32_t n_rows,
                      const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* table, int32_t pages_per_row,
                      const int32_t* positions, float scale, float* out,
                      void* workspace, size_t workspace_bytes);

size_t paged_decode_attn_workspace(const qkr_pool* pool, int32_t n_rows, int32_t pages_per_row);

/* The name of the kernel paged_decode_attn launches for n_rows rows and tables of
 * pages_per_row pages on the current device, as profilers list it:
 * "paged_decode_small_kernel" (one workgroup per row, KV head and chunk of 2 pages,
 * for small batches), "paged_decode_bf16_kernel" (the split-K grid) or
 * "attention_generic_kernel" (a float32 pool). "" for an invalid pool or size.
 * The string is static; nothing is launched. */
const char* paged_decode_attn_kernel(const qkr_pool* pool, int32_t n_rows, int32_t pages_per_row);

/* paged_decode_attn with qkr_attn_opts (output gate). */
int paged_decode_attn_ex(void* stream, const qkr_pool* pool, int32_t n_rows,
                         const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* table, int32_t pages_per_row,
                         const int32_t* positions, float scale, float* out,
                         void* workspace, size_t workspace_bytes, const qkr_attn_opts* opts);

/*
 * paged_decode_attn_noalloc -- paged_decode_attn with no workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation. It computes exactly what
 * paged_decode_attn computes (the same kernel and the same split, so the same
 * bits) and calls no allocating routine.
 *
 * Scratch: instead of a caller's workspace, the call uses a library-owned device
 * array of QKR_NOALLOC_SCRATCH_BYTES (8.5 MiB) per GPU, held from the first call on
 * that GPU until the process ends (its address is looked up once per device, on
 * the first call with that device current). Each call clears the merge counters it
 * uses with a small fill kernel on `stream`, then launches the decode kernel.
 * Every call on one GPU shares that GPU's array and the array keeps the last
 * call's contents, so calls that may overlap on one GPU (different streams,
 * different threads without ordering) race and give wrong results: order them on
 * one stream.
 *
 * Limit: n_rows * num_kv_heads <= QKR_NOALLOC_MAX_ROW_HEADS (12288 rows at 8 KV
 * heads) for a bfloat16 pool, besides paged_decode_attn's own 12288 rows; larger
 * batches return QKR_EUNSUPPORTED before anything is enqueued (qkr_last_error
 * names the scratch limit). A float32 pool needs no
 * scratch. The other arguments, errors and layouts are those of paged_decode_attn.
 */
#define QKR_NOALLOC_MAX_ROW_HEADS 98304
#define QKR_NOALLOC_SCRATCH_BYTES (98304 * 4 + 2048 * 2 * 520 * 4)
int paged_decode_attn_noalloc(void* stream, const qkr_pool* pool, int32_t n_rows,
                              const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* table, int32_t pages_per_row,
                              const int32_t* positions, float scale, float* out);

/*
 * paged_prefill_attn -- packed prompt tokens over their rows' pages
 * (attention.linnet, prefill_paged / paged_prefill_attention).
 *
 * Token p (query q[p], row rows[p], position positions[p]) attends with each
 * query head over positions 0..positions[p] of table row rows[p]; the keys of
 * the pass itself are already in the pool (the append runs first), so a chunk
 * sees its own earlier tokens and any history or shared pages before it.
 * Prompts are packed end to end; the kernel tiles the pack in blocks of 64
 * tokens and handles blocks that span several rows.
 *
 * rows, positions: device int32 [n_tokens]; rows[p] in [0, n_table_rows).
 * A bfloat16 pool takes tables of at most 2048 pages per row (131072 positions;
 * QKR_EUNSUPPORTED above).
 * out: float32 [n_tokens][num_q_heads*head_dim].
 * workspace: at least paged_prefill_attn_workspace() bytes, sized for the
 * current device (its CU count sets how many workgroups a long block's keys may
 * be split over). It holds the block schedule and, for blocks whose keys are
 * split, the partial softmax states and merge counters; contents need no
 * initialisation (the call resets its counters). Calls that may overlap need
 * workspaces of their own.
 */
int paged_prefill_attn(void* stream, const qkr_pool* pool, int32_t n_tokens,
                       const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* table, int32_t n_table_rows, int32_t pages_per_row,
                       const int32_t* rows, const int32_t* positions,
                       float scale, float* out, void* workspace, size_t workspace_bytes);

size_t paged_prefill_attn_workspace(const qkr_pool* pool, int32_t n_tokens);

/* paged_prefill_attn with qkr_attn_opts (output gate). */
int paged_prefill_attn_ex(void* stream, const qkr_pool* pool, int32_t n_tokens,
                          const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* table, int32_t n_table_rows, int32_t pages_per_row,
                          const int32_t* rows, const int32_t* positions,
                          float scale, float* out, void* workspace, size_t workspace_bytes,
                          const qkr_attn_opts* opts);

/*
 * packed_prefill_attn -- prompts packed end to end that attend only among
 * themselves (attention.linnet, prefill_packed; on a scratch pool also the
 * training form packed, which keeps no cache).
 *
 * Token p (query q[p], prompt segments[p], row rows[p], position positions[p])
 * attends with each query head over the tokens j of its own prompt with
 * positions[j] <= positions[p]. Their keys and values are read from the pool,
 * where qknorm_rope_append wrote them; history in the row before the prompt's
 * first position is not seen.
 * Preconditions (not checked on the device): every prompt is one contiguous run
 * of the pack whose positions rise by one, and all its tokens use one row.
 * segments: device int32 [n_tokens]; the other arguments as for
 * paged_prefill_attn (same row-length limit for a bfloat16 pool).
 * workspace: at least packed_prefill_attn_workspace() bytes; as for
 * paged_prefill_attn, plus the tokens' first visible positions.
 */
int packed_prefill_attn(void* stream, const qkr_pool* pool, int32_t n_tokens,
                        const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* table, int32_t n_table_rows, int32_t pages_per_row,
                        const int32_t* rows, const int32_t* positions, const int32_t* segments,
                        float scale, float* out, void* workspace, size_t workspace_bytes);

size_t packed_prefill_attn_workspace(const qkr_pool* pool, int32_t n_tokens);

/* packed_prefill_attn with qkr_attn_opts (output gate). */
int packed_prefill_attn_ex(void* stream, const qkr_pool* pool, int32_t n_tokens,
                           const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* table, int32_t n_table_rows, int32_t pages_per_row,
                           const int32_t* rows, const int32_t* positions, const int32_t* segments,
                           float scale, float* out, void* workspace, size_t workspace_bytes,
                           const qkr_attn_opts* opts);

/*
 * step_paged -- one mixed serving step in a single launch (nest
 * "models/qwen3-8b/files": Entries table, step_paged; attention.linnet,
 * step_paged): QK-norm + RoPE of the n_prefill prompt tokens and the n_decode
 * decode rows, their k/v written into the pool, then prefill attention for the
 * prompt tokens and decode attention for the rows, with every write before any
 * read. The result is the one of
 *   qknorm_rope_append over all n_prefill + n_decode tokens (slots for the
 *     prompt tokens, table rows decode_row0 + b for decode row b), then
 *   paged_prefill_attn over the prompt tokens and
 *   paged_decode_attn over the rows (table + decode_row0 * pages_per_row):
 * q_out and the pool bytes are identical to that sequence, prefill_out is
 * identical to paged_prefill_attn's, and decode_out equals paged_decode_attn's
 * up to float32 rounding (the page ranges are split differently).
 *
 * q, k, v: bfloat16 [n_prefill + n_decode][heads*head_dim], prompt tokens first
 *   (in_dtype must be QKR_BF16, the pool bfloat16; else QKR_EUNSUPPORTED).
 * positions, rows, slots: device int32 [n_prefill] (the prompt tokens);
 * step_positions: device int32 [n_decode] (the decode rows).
 * table: device int32 [n_table_rows][pages_per_row]; prompt token p uses row
 *   rows[p], decode row b uses row decode_row0 + b (decode_row0 + n_decode <=
 *   n_table_rows). At most 2048 pages per row and 8192 decode rows
 *   (QKR_EUNSUPPORTED above).
 * q_out: [n_prefill + n_decode][num_q_heads*head_dim] bfloat16;
 * prefill_out: float32 [n_prefill][num_q_heads*head_dim];
 * decode_out: float32 [n_decode][num_q_heads*head_dim].
 * workspace: at least step_paged_workspace() bytes, zero-filled before its first
 *   use; every call leaves it zero again (calls sharing it must be ordered on one
 *   stream). Its int32 word 5 becomes 1 if a workgroup ever gave up waiting for
 *   the writes (a wait bounded at one second that a correct launch never
 *   exhausts; words 6 and 7 then hold the counts it saw); the library never
 *   clears those words.
 * Device indices are range-checked as in the three calls above.
 */
int step_paged(void* stream, const qkr_pool* pool, int32_t n_prefill, int32_t n_decode,
               const void* q, const void* k, const void* v, int32_t in_dtype,
               const float* q_gain, const float* k_gain, float eps,
               const float* rope_cos, const float* rope_sin, int32_t rope_rows,
               const int32_t* positions, const int32_t* rows, const int32_t* slots,
               const int32_t* step_positions,
               const int32_t* table, int32_t n_table_rows, int32_t pages_per_row, int32_t decode_row0,
               float scale, void* q_out, void* k_pool, void* v_pool,
               float* prefill_out, float* decode_out, void* workspace, size_t workspace_bytes);

size_t step_paged_workspace(const qkr_pool* pool, int32_t n_prefill, int32_t n_decode, int32_t pages_per_row);

/*
 * qkr_check_indices -- validate the device-side indices of a step before it runs
 * (nest "models/qwen3-8b/files", README: every name, shape and dtype is checked
 * before anything runs; Entries table: a row's positions lie in the pages its
 * table row lists). The append and attention calls range-check every index they
 * form and skip or mask what is out of range, so bad data passes there without a
 * diagnosis; this call counts it.
 *
 * Queries: n_tokens prompt tokens (rows, positions, and optionally slots: device
 * int32 [n_tokens]) and n_decode decode rows (step_positions: device int32
 * [n_decode]; decode row b uses table row decode_row0 + b). For each query it
 * counts, into counts[QKR_CHECK_*] (device int32 [QKR_CHECK_COUNTS]):
 *   QKR_CHECK_ROW           prompt tokens with rows[p] outside [0, n_table_rows);
 *   QKR_CHECK_POSITION      queries with a position outside [0, pages_per_row*64)
 *                           or, when rope_rows > 0, outside [0, rope_rows);
 *   QKR_CHECK_PAGE          queries with a valid row and position one of whose
 *                           visible pages (table entries 0 .. position / 64 of
 *                           its row) is outside [0, num_pages);
 *   QKR_CHECK_SLOT_RANGE    prompt tokens with slots[p] >= num_pages*64
 *                           (negative slots are padding and not counted);
 *   QKR_CHECK_SLOT_MISMATCH prompt tokens with a valid row and position whose
 *                           slots[p] >= 0 differs from table[rows[p]][pos / 64]*64
 *                           + pos % 64.
 * Two real tokens writing one slot are not detected. decode_row0 + n_decode <=
 * n_table_rows is checked on the host (QKR_EINVAL).
 *
 * wait == 0: the counts are zeroed and filled on `stream` (a fill kernel and one
 * check kernel); nothing allocates and nothing synchronises; the counts are valid
 * once the stream reaches them. wait != 0: the call then waits for `stream`,
 * reads the counts and returns QKR_EDATA if any is non-zero (QKR_OK otherwise).
 * counts must not be shared by calls that may overlap.
 */
#define QKR_CHECK_ROW 0
#define QKR_CHECK_POSITION 1
#define QKR_CHECK_PAGE 2
#define QKR_CHECK_SLOT_RANGE 3
#define QKR_CHECK_SLOT_MISMATCH 4
#define QKR_CHECK_COUNTS 8
int qkr_check_indices(void* stream, const qkr_pool* pool,
                      const int32_t* table, int32_t n_table_rows, int32_t pages_per_row,
                      int32_t n_tokens, const int32_t* rows, const int32_t* positions, const int32_t* slots,
                      int32_t n_decode, const int32_t* step_positions, int32_t decode_row0,
                      int32_t rope_rows, int32_t* counts, int32_t wait);

/*
 * qkr_rope_table -- host helper: the RoPE cos/sin table (host memory).
 * For pos < rope_rows and i < head_dim/2:
 *   inv = 1 / theta^(2i/head_dim), a = pos*inv (double precision),
 *   cos_out[pos][i] = (float)cos(a), sin_out[pos][i] = (float)sin(a)
 * (model.zig, loadWeights; rope.linnet, tables with THETA = 1e6). Only half the
 * width is stored because both halves of a head use the same frequencies.
 */
int qkr_rope_table(double theta, int32_t rope_rows, int32_t head_dim,
                   float* cos_out, float* sin_out);

/*
 * qkr_read_probe -- measurement helper, not part of the attention path: one
 * streaming read (non-temporal 16-byte loads, as the decode kernel's K/V loads) of
 * `bytes` bytes of device memory at `buf` (16-byte aligned,
 * bytes a multiple of 16), enqueued on `stream`. Timing it gives the read rate a
 * kernel with no paging, masking or attention arithmetic reaches on this GPU, a
 * practical ceiling to set beside the published HBM peak. `out` (device, 1 float)
 * is written only in the practically impossible case that the buffer sums to a
 * fixed sentinel; its content is not meaningful. Returns QKR_EINVAL for a null
 * pointer, a misaligned buffer or a size that is not a multiple of 16.
 */
int qkr_read_probe(void* stream, const void* buf, size_t bytes, float* out);

/*
 * qkr_mfma_probe -- measurement helper, not part of the attention path: one kernel
 * of `iters` rounds of eight independent bf16 32x32x16 MFMAs per wave, eight waves
 * on every CU, with no memory traffic in the loop, enqueued on `stream`. Timing it
 * gives the dense bf16 rate the matrix cores sustain on this GPU, a practical
 * ceiling to set beside the published MFMA peak. *flops (host) receives the FLOPs
 * the kernel performs; `out` (device, 1 float) is written only in the practically
 * impossible case that the accumulators sum to a fixed sentinel. QKR_EINVAL for a
 * null pointer or a negative count.
 */
int qkr_mfma_probe(void* stream, int32_t iters, float* out, int64_t* flops);

/* Human-readable name of a qkr_status value. */
const char* qkr_status_str(int status);

/* Text of the HIP runtime error behind the calling thread's last QKR_ELAUNCH
 * ("" if none). The pointer stays valid until the thread's next failing call. */
const char* qkr_last_error(void);

/* Library version, as MAJOR*10000 + MINOR*100 + PATCH. */
int qkr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QKNR_H */
