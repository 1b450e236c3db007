// K3: paged prefill attention with bfloat16 MFMA, float32 accumulation. Device
// code shared by the prefill kernels and the single-launch step.
//
// nest "models/qwen3-8b/files": Entries table (prefill_paged: prompts packed end to
// end, each token attending over its row's pages up to its position, for chunks
// and shared prefixes) and src/attention.linnet (prefill_paged writes k/v into the
// pool, then paged_prefill_attention reads table[rows[p]]; scale rsqrt(head_dim)).
// fantasma "src/inference/model.zig", fullAttentionForward: query head h reads KV
// head h / 4; max-subtracted softmax; weighted sum of V.
//
// Work item = (64-token tile of the pack, KV head g), one workgroup of 8 waves:
// wave w is query head 4g + (w & 3) for the queries 32*(w >> 2) .. +31 of the
// tile, so one K/V page staged in LDS feeds all 256 query rows. Per 64-key page
// and wave:
//   S^T (64 keys x 32 queries) = K . Q^T   : 16 x v_mfma_f32_32x32x16_bf16,
//       K from LDS (16-byte reads), Q kept in registers;
//   online softmax along the lane's own keys (each lane holds one query's keys,
//       the other half sits in lane l ^ 32); the running max only moves when the
//       page's max exceeds it by more than 2^8 (exact after the final division);
//   O^T (128 dims x 32 queries) += V^T . P^T : 16 MFMAs, V^T read from the
//       row-major V page with ds_read_b64_tr_b16, P^T straight from the S^T
//       accumulators (keys permuted the same way on both operands).
// Pages reach three LDS buffers through 16-byte LDS-direct buffer loads with an
// XOR-swizzled layout, issued by waves 4..7 in the phases where they run the
// softmax. Waves w and w + 4 share a SIMD and run half a page apart: in each phase
// one issues the MFMAs of PV(j-1) and S(j) while the other runs the softmax. The
// page loop is compiled once per group of four waves. A tile that holds tokens of
// several rows runs once per row ("run"); masking uses each token's position. A
// plan kernel orders tiles by decreasing cost (largest visible position) so the
// long ones start first; item i maps to KV head i % 8, which keeps one KV head's
// pages on one XCD's L2.
#pragma once
#include "common.h"

namespace qknr {
namespace {

constexpr int kTile = 64;
constexpr int kPlanMaxTiles = 8192;
constexpr int kMaxChunks = 8;          // key chunks of one split tile at most
constexpr float kRescaleThreshold = 8.0f;  // log2 units

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ---------------------------------------------------------------- planning
// Tile order by decreasing cost, sorted in LDS (keys: at least n_tiles rounded up
// to a power of two entries) by the nthreads threads of one workgroup.
template <bool kAgentStores = false>
__device__ __forceinline__ void plan_tiles(int n_tokens, const int* __restrict__ positions,
                                           const int* __restrict__ lo, int n_tiles, int* __restrict__ order,
                                           unsigned long long* keys, int tid, int nthreads) {
  int npow2 = 1;
  while (npow2 < n_tiles) npow2 <<= 1;
  // cost of a tile: keys from its smallest first visible position to its largest
  // position; one wave per tile, one lane per token. A wave takes kBatch tiles at a
  // time and issues all their loads before reducing, so a batch costs one memory
  // round trip instead of one per tile.
  constexpr int kBatch = 8;
  const int wave = tid >> 6, lane = tid & 63, n_waves = nthreads >> 6;
  const int* lsrc = lo ? lo : positions;   // read either way (no branch around the load)
  for (int i0 = wave; i0 < npow2; i0 += kBatch * n_waves) {
    int hi[kBatch], first[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {   // unconditional loads (clamped index), then selects
      const int i = i0 + u * n_waves;
      const int t = i * kTile + lane;
      const bool ok = i < n_tiles && t < n_tokens;
      const int tc = ok ? t : 0;   // n_tokens >= 1
      hi[u] = positions[tc];
      first[u] = lsrc[tc];
      hi[u] = ok ? max(hi[u] + 1, 0) : 0;
      first[u] = lo ? (ok ? max(first[u], 0) : 0x7fffffff) : 0;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = i0 + u * n_waves;
      if (i >= npow2) break;
      int h = hi[u], f = first[u];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        h = max(h, __shfl_xor(h, m));
        f = min(f, __shfl_xor(f, m));
      }
      const int cost = max(h - f, 0);
      if (lane == 0)
        keys[i] = i < n_tiles ? ((unsigned long long)(0xffffffffu - (unsigned)cost) << 32) | (unsigned)i : ~0ull;
    }
  }
  __syncthreads();
  for (int k = 2; k <= npow2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < npow2; i += nthreads) {
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
  for (int i = tid; i < n_tiles; i += nthreads) {
    const int v = (int)(keys[i] & 0xffffffffu);
    if (kAgentStores) __hip_atomic_store(&order[i], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else order[i] = v;
  }
}

// ---------------------------------------------------------------- attention
struct PrefillParams {
  int n_tokens, n_kv;
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  int64_t num_pages;
  const int* table;
  int n_table_rows, pages_per_row;
  const int* rows;
  const int* positions;
  float scale_log2;
  float* out;
  const int* order;   // tile order (used when pairs is null)
  const int* lo;   // first visible position per token (packed form), or null (0)
  const uint16_t* gate;   // optional output gate [n_tokens][n_q*128], bf16
  // Key-split work list from the split plan (null: one item per tile and KV head):
  // pair k = (tile, chunk s | chunks S << 8, first partial slot, split index);
  // item = k * n_kv + g. A chunk of a split tile covers pages [s*len/S, (s+1)*len/S)
  // of its run's len visible pages and leaves a partial state; the last chunk of
  // (tile, g) to finish merges them.
  const int4* pairs;
  const int* n_pairs;
  int* tickets;        // [split tiles][n_kv], zeroed by the plan
  float* partials;     // O: [slot][n_kv][64 tokens][4 heads][128]
  float* partial_ml;   // (m, l): [slot][n_kv][64 tokens][4 heads][2]
};

constexpr int kPartialFloats = kHeadDim + 2;   // m, l, O[128] of one (token, head)

__device__ __forceinline__ bf16x8 join(i16x4 a, i16x4 b) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Marks x as produced at this point. The page loop's barriers order memory only,
// so without this the compiler may sink a phase's register-only work (softmax,
// MFMAs) past the barrier to its consumer and undo the two-group interleave.
template <typename T>
__device__ __forceinline__ void pin(T& x) { asm volatile("" : "+v"(x)); }

// Raw buffer descriptor over one K or V page of one KV head (64 rows x 256 bytes).
// Word 3 selects 32-bit data format, as the LDS-direct dword loads need; reads past
// the page return zero instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint16_t* page_base) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)page_base, 0, kPageSize * kHeadDim * 2, 0x00020000);
}

// s_waitcnt vmcnt(n) (gfx9 encoding), leaving the other counters alone
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

typedef __attribute__((address_space(3))) void lds_void;

// Instruction order for the fused MFMA stream (scheduler groups): the LDS reads of
// the first A operands, then every MFMA followed by the reads of the operand A
// places later. Operands 0..15 take two transposed reads, 16..31 one 16-byte read.
template <int A, int I = 0>
__device__ __forceinline__ void fused_order() {
  if constexpr (I < A) {
    __builtin_amdgcn_sched_group_barrier(0x100, I < 16 ? 2 : 1, 0);
    fused_order<A, I + 1>();
  } else if constexpr (I < A + 32) {
    constexpr int m = I - A;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (m + A < 32) __builtin_amdgcn_sched_group_barrier(0x100, m + A < 16 ? 2 : 1, 0);
    fused_order<A, I + 1>();
  }
}

// LDS page layout: 64 rows of 256 bytes (16 chunks of 16 bytes) with the chunks
// of each row permuted by an XOR swizzle, so that the MFMA operand reads hit
// every bank once per cycle:
//   K: chunk c of row r sits at chunk c ^ (r & 15). A 16-byte read of one chunk
//      by 16 consecutive rows touches 16 distinct chunk positions.
//   V: chunk c of row r sits at chunk c ^ 4(r & 3). The transposed 8-byte reads
//      take 64 bytes (4 chunks) from each of 4 consecutive rows; the swizzle puts
//      the 4 rows in the 4 different 64-byte quarters of the bank space.
// A page is copied with 16-byte LDS-direct loads: one wave instruction fills 1 KB
// (4 rows) linearly, each lane fetching the global chunk that belongs at its slot.
constexpr int kRowBytes = kHeadDim * 2;
constexpr int kKPageBytes = kTile * kRowBytes;
constexpr int kVPageBytes = kTile * kRowBytes;
__device__ __forceinline__ int k_swz(int r) { return r & 15; }
__device__ __forceinline__ int v_swz(int r) { return 4 * (r & 3); }

constexpr int kTabCache = 2048;   // page ids of a run kept in LDS (pages_per_row at most)

// Three K/V page buffers as separate LDS objects: every buffer index below is a
// compile-time constant, so the compiler can tell a page being copied in from the
// page being read and does not wait for the copy before the reads.
__shared__ __attribute__((aligned(1024))) uint8_t sK0[kKPageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t sK1[kKPageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t sK2[kKPageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t sV0[kVPageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t sV1[kVPageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t sV2[kVPageBytes];

// token rows, positions and first visible positions of the tile, and the page ids
// of the current run
__shared__ int sRow[kTile], sPos[kTile], sLo[kTile];
__shared__ __attribute__((aligned(16))) int sTab[kTabCache];

template <int B> __device__ __forceinline__ uint8_t* kbuf() { return B == 0 ? sK0 : (B == 1 ? sK1 : sK2); }
template <int B> __device__ __forceinline__ uint8_t* vbuf() { return B == 0 ? sV0 : (B == 1 ? sV1 : sV2); }
template <int B> struct Buf { static constexpr int value = B; };

// Workgroup barrier for the page loop. The only LDS writes in flight are the
// page copies, which the caller has already waited for (vmcnt), so no fence on
// global memory is needed; the signal fences keep the compiler from moving LDS
// reads across the barrier.
__device__ __forceinline__ void page_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Eight waves: wave w is query head 4g + (w & 3) for the 32 queries
// 32*(w >> 2) .. +31 of the tile, two waves per SIMD. Pages are copied straight
// from HBM into LDS (global_load_lds) one page ahead of the computation.
// Partial state of one chunk of a split tile, then, in the last chunk of (tile, g)
// to finish, the exact merge of all chunks' states into the output:
//   M = max_s m_s,  out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s
// (m in the softmax's scaled log2 units; O and l relative to 2^m). The states are
// written with plain vector stores; each wave drains them, the workgroup meets at
// a barrier, and one agent-scope release precedes the ticket (per tile and KV
// head); the last chunk takes one agent-scope acquire before reading them. No
// workgroup waits for another.
__device__ __forceinline__ void split_epilogue(const PrefillParams& P, const f32x16 (&o)[4], float m, float lt,
                                               bool active, int qn, int hq, int lh, int g, int chunk, int n_chunks,
                                               int slot0, int split, int t0, int tid) {
  __shared__ int s_last;
  const int n_q = P.n_kv * kGroup;
  // opaque copies: the addresses below are formed here, not hoisted to the item's
  // start, where they would stay live (and spill) through the page loop
  asm volatile("" : "+v"(qn), "+v"(lh), "+v"(tid));
  // (chunk s, token q, head h) -> row of 128 floats of O, 2 floats of (m, l)
  auto row = [&](int s, int q, int h) -> int64_t {
    return (((int64_t)(slot0 + s) * P.n_kv + g) * kTile + q) * kGroup + h;
  };
  if (active) {
    const int64_t r = row(chunk, qn, hq);
    float* op = P.partials + r * kHeadDim + 4 * lh;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4*>(op + 32 * dt + 8 * j) =
            f32x4{o[dt][4 * j], o[dt][4 * j + 1], o[dt][4 * j + 2], o[dt][4 * j + 3]};
    if (lh == 0) *reinterpret_cast<float2*>(P.partial_ml + 2 * r) = make_float2(m, lt);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int old = __hip_atomic_fetch_add(&P.tickets[split * P.n_kv + g], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == n_chunks - 1;
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  // weights 2^(m_s - M) / L per (token, head, chunk), in the free K page buffer
  float* wts = reinterpret_cast<float*>(sK0);   // [64][4][kMaxChunks]
  if (tid < kTile * kGroup) {
    const int q = tid >> 2, h = tid & 3;
    if (sRow[q] >= 0) {
      float2 ml[kMaxChunks];
#pragma unroll
      for (int s = 0; s < kMaxChunks; ++s)
        ml[s] = s < n_chunks ? *reinterpret_cast<const float2*>(P.partial_ml + 2 * row(s, q, h))
                             : make_float2(-INFINITY, 0.f);
      float M = -INFINITY;
#pragma unroll
      for (int s = 0; s < kMaxChunks; ++s) M = fmaxf(M, ml[s].x);
      float L = 0.f, f[kMaxChunks];
#pragma unroll
      for (int s = 0; s < kMaxChunks; ++s) {
        f[s] = ml[s].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml[s].x - M);
        L += f[s] * ml[s].y;
      }
      const float inv = 1.0f / L;
#pragma unroll
      for (int s = 0; s < kMaxChunks; ++s) wts[(q * kGroup + h) * kMaxChunks + s] = f[s] * inv;
    }
  }
  __syncthreads();
  // rows (token, head) = 256, 32 per wave; a row is 128 floats, 2 per lane; 4 rows
  // x every chunk loaded per batch
  const int wv = tid >> 6, ln = tid & 63;
  constexpr int kRows = 4;
  for (int r0 = wv * 32; r0 < wv * 32 + 32; r0 += kRows) {
    float2 x[kRows][kMaxChunks];
#pragma unroll
    for (int u = 0; u < kRows; ++u)
#pragma unroll
      for (int s = 0; s < kMaxChunks; ++s)
        x[u][s] = s < n_chunks ? *reinterpret_cast<const float2*>(
                                     P.partials + row(s, (r0 + u) >> 2, (r0 + u) & 3) * kHeadDim + 2 * ln)
                               : make_float2(0.f, 0.f);
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const int q = (r0 + u) >> 2, h = (r0 + u) & 3;
      if (sRow[q] < 0) continue;
      float2 acc = make_float2(0.f, 0.f);
#pragma unroll
      for (int s = 0; s < kMaxChunks; ++s) {
        const float wgt = wts[(q * kGroup + h) * kMaxChunks + s];   // 0 past n_chunks
        acc.x += wgt * x[u][s].x;
        acc.y += wgt * x[u][s].y;
      }
      const int64_t oi = ((int64_t)(t0 + q) * n_q + g * kGroup + h) * kHeadDim + 2 * ln;
      if (P.gate) {   // output gate: out *= sigmoid(gate) at the same element
        const uint32_t gw = *reinterpret_cast<const uint32_t*>(P.gate + oi);
        acc.x *= sigmoidf(bf16_lo(gw));
        acc.y *= sigmoidf(bf16_hi(gw));
      }
      *reinterpret_cast<float2*>(P.out + oi) = acc;
    }
  }
  __syncthreads();   // the weights' LDS is the next item's page buffer
}

// One work item (64-token tile, KV head) by a workgroup of 512 threads; tid is the
// thread's index in the workgroup.
// kSplits: the item may be a chunk of a split tile (P.pairs from the split plan).
template <bool kSplits = true>
__device__ __forceinline__ void prefill_item(const PrefillParams& P, const int item, const int tid) {
  const int n_q = P.n_kv * kGroup;
  const int g = item % P.n_kv;
  int tile, chunk = 0, n_chunks = 1, slot0 = 0, split = 0;
  if (kSplits && P.pairs) {
    const int k = item / P.n_kv;
    // both loads in one round trip: pairs has a slot for every workgroup of the grid
    const int n_pairs = *P.n_pairs;
    const int4 pr = P.pairs[k];
    asm volatile("" : : "s"(n_pairs), "s"(pr.x), "s"(pr.y), "s"(pr.z), "s"(pr.w));   // not sunk past the test
    if (k >= n_pairs) return;   // a spare workgroup: fewer chunks than the grid allows
    tile = pr.x;
    chunk = pr.y & 0xff;
    n_chunks = pr.y >> 8;
    slot0 = pr.z;
    split = pr.w;
  } else {
    tile = P.order ? P.order[item / P.n_kv] : item / P.n_kv;
  }
  const int w = tid >> 6;
  const int l = tid & 63;
  const int lq = l & 31;        // query index within the wave's 32 queries
  const int lh = l >> 5;        // half of the wave
  const int head = g * kGroup + (w & 3);
  const int qn = 32 * (w >> 2) + lq;   // the lane's query within the tile
  const int t0 = tile * kTile;
  const int max_pos = P.pages_per_row * kPageSize;

  // Q^T operand: lane holds query qn, dims 16*ks + 8*lh .. +7. Loaded first: the
  // addresses depend only on the tile, so the loads overlap those of the tile's
  // rows and positions instead of following them.
  bf16x8 qb[8];
  {
    const int t = t0 + qn;
    if (t < P.n_tokens) {
      const uint16_t* qp = P.q + ((int64_t)t * n_q + head) * kHeadDim + 8 * lh;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qb[ks] = *reinterpret_cast<const bf16x8*>(qp + 16 * ks);
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int i = 0; i < 8; ++i) qb[ks][i] = (__bf16)0.0f;
    }
  }
  if (tid < kTile) {
    const int t = t0 + tid;
    int r = -1, p = -1, f = 0;
    if (t < P.n_tokens) {
      r = P.rows[t];
      p = P.positions[t];
      if (r < 0 || r >= P.n_table_rows || p < 0 || p >= max_pos) r = -1;
      if (P.lo) f = min(max(P.lo[t], 0), max(p, 0));
    }
    sRow[tid] = r;
    sPos[tid] = p;
    sLo[tid] = f;
  }
  __syncthreads();

  const int qpos = sPos[qn];
  const int qlo = sLo[qn];   // first visible position of the lane's query

  const int64_t pool_slots = P.num_pages * kPageSize;
  const uint16_t* kbase = P.k_pool + (int64_t)g * pool_slots * kHeadDim;
  const uint16_t* vbase = P.v_pool + (int64_t)g * pool_slots * kHeadDim;
  const float sc = P.scale_log2;
  // K operand (S^T = K . Q^T): lane reads row kt*32 + lq, chunk 2*ks + lh;
  // byte offset of ks's chunk in rows kt*32 + lq (kt adds 32 rows)
  int kofs[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kofs[ks] = lq * kRowBytes + (((2 * ks + lh) ^ k_swz(lq)) << 4);
  // V^T operand (transposed reads): lane reads 8 bytes of row 16c + 8h + 4lh + jj/4,
  // dims 32dt + 16(G4 & 1) + 4(jj & 3) .. +3, i.e. chunk 4dt + 2(G4 & 1) + (jj & 3)/2
  const int jj = l & 15;
  const int vrow = 4 * lh + (jj >> 2);
  int vofs[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
    vofs[dt] = vrow * kRowBytes + (((4 * dt + 2 * ((l >> 4) & 1) + ((jj & 3) >> 1)) ^ v_swz(vrow)) << 4) + 8 * (jj & 1);
  // page copy, by waves 4..7 only (they issue it in the phases where they run the
  // softmax, so the MFMA stream of waves 0..3 carries no copy instructions):
  // instruction q of wave w fills rows 16(w - 4) + 4q .. +3; lane i takes row
  // 16(w - 4) + 4q + i/16 and the global chunk that belongs at slot i % 16
  const int crow0 = 16 * (w - 4) + (l >> 4);
  const int cslot = l & 15;

  // lane l holds token l of the tile; runs are found with ballots and a wave max
  const int my_row = sRow[l];
  const int my_pos = sPos[l];
  const int my_lo = sLo[l];
  int a = 0;
  while (a < kTile) {
    const int r = __builtin_amdgcn_readlane(my_row, a);
    const unsigned long long other = __ballot(l > a && my_row != r);
    const int e = other ? (int)__builtin_ctzll(other) : kTile;
    if (r < 0) {
      // tokens with a row or position out of range: NaN outputs, as the float32
      // kernel gives them (the tile's tail past the pack is left alone)
      if (qn >= a && qn < e && t0 + qn < P.n_tokens) {
        float* op = P.out + ((int64_t)(t0 + qn) * n_q + head) * kHeadDim + 64 * lh;
        const float nan = __builtin_nanf("");
#pragma unroll
        for (int i = 0; i < 64; i += 4) *reinterpret_cast<f32x4*>(op + i) = f32x4{nan, nan, nan, nan};
      }
      a = e;
      continue;
    }
    int mp = (l >= a && l < e) ? my_pos : 0;
    int mf = (l >= a && l < e) ? my_lo : 0x7fffffff;
#pragma unroll
    for (int mm = 32; mm >= 1; mm >>= 1) {
      mp = max(mp, __shfl_xor(mp, mm));
      mf = min(mf, __shfl_xor(mf, mm));
    }
    const int maxp = uniform(mp);
    const int runlo = uniform(mf);   // smallest first visible position of the run
    // pages [j0, npages) of the run: from the first page any query of the run sees
    // to the page of its last position; a chunk of a split tile takes its share
    int j0 = runlo / kPageSize;
    int npages = maxp / kPageSize + 1;
    if (n_chunks > 1) {
      const int len = npages - j0;
      const int b = j0;
      j0 = b + chunk * len / n_chunks;
      npages = b + (chunk + 1) * len / n_chunks;
    }
    const int* trow = P.table + (int64_t)r * P.pages_per_row;
    bool bad = false;
    for (int i = j0 + tid; i < npages; i += 512) {
      const int id = trow[i];
      sTab[i] = id;
      bad |= id < 0 || id >= P.num_pages;
    }
    // every position <= maxp of the row holds finite data; masked keys past maxp
    // are fetched from this slot instead (their probability is exactly 0)
    const int64_t last_page = trow[maxp / kPageSize];
    const bool last_ok = last_page >= 0 && last_page < P.num_pages;
    const int64_t fill_page = uniform64(last_ok ? last_page : 0);
    const int fill_row = uniform(last_ok ? maxp % kPageSize : 0);
    // some page of the run is outside the pool: only then does the softmax look pages up
    const bool any_bad = __syncthreads_or(bad);
    // the LDS read is unconditional (clamped index), so its wait falls at the first
    // use of the id instead of right after the read
    auto page_of = [&](int p) -> int64_t {
      const int v = sTab[min(max(p, j0), npages - 1)];
      return (p >= j0 && p < npages) ? v : -1;
    };
    auto page_ok = [&](int64_t page) { return page >= 0 && page < P.num_pages; };

    const bool active = qn >= a && qn < e;
    // smallest position among the wave's queries; -1 when some query is not in this run
    int wmin = active ? qpos : -1;
    // largest first visible position among the wave's queries of this run
    int wlo = active ? qlo : 0;
#pragma unroll
    for (int mm = 32; mm >= 1; mm >>= 1) {
      wmin = min(wmin, __shfl_xor(wmin, mm));
      wlo = max(wlo, __shfl_xor(wlo, mm));
    }
    wmin = uniform(wmin);
    wlo = uniform(wlo);

    float m = -INFINITY;
    float lsum = 0.f;
    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;

    // copy page p into buffer B: wave w >= 4 moves rows 16(w - 4)..+15 of K and of V
    // with four 1 KB instructions each. Rows past the run's last position, and
    // pages past the run or outside the pool, copy the run's last valid row instead;
    // rows before the run's first visible position (history a packed prompt does
    // not see, which need not be finite: a NaN V row would turn its zero weight
    // into NaN) copy the first visible row of the same page. Both hold finite data
    // and those keys are masked, so every step issues the same copies and the
    // compiler tracks which buffer each copy targets. The page is addressed
    // through a buffer descriptor (reads past the page return zero).
    auto fetch = [&](auto Bc, int p, int64_t page) {
      constexpr int B = decltype(Bc)::value;
      page = uniform64(page);
      const bool ok = page_ok(page);
      const int64_t src = ok ? page : fill_page;
      const int lim = ok ? maxp - p * kPageSize : -1;   // rows <= lim hold real keys
      const int low = runlo - p * kPageSize;             // rows >= low are visible to the run (low <= lim)
      const __amdgpu_buffer_rsrc_t rk = page_rsrc(kbase + src * kPageSize * kHeadDim);
      const __amdgpu_buffer_rsrc_t rv = page_rsrc(vbase + src * kPageSize * kHeadDim);
      if (w >= 4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = crow0 + 4 * q;
          const int srow = row > lim ? fill_row : (row < low ? low : row);
          const int ko = srow * kRowBytes + ((cslot ^ k_swz(row)) << 4);
          const int vo = srow * kRowBytes + ((cslot ^ v_swz(row)) << 4);
          const int dst = (16 * (uniform(w) - 4) + 4 * q) * kRowBytes;   // scalar LDS offset
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kbuf<B>() + dst), 16, ko, 0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vbuf<B>() + dst), 16, vo, 0, 0, 0);
        }
      }
    };

    f32x16 st[2];   // S^T of the page: keys x queries
    // ---- mask + online softmax of st (page j) into pb
    bf16x8 pb[4];
    auto softmax = [&](int j) {
      const bool pok = !any_bad || page_ok(uniform64(page_of(j)));
      const int kpos0 = j * kPageSize;
      if (!pok || wmin < kpos0 + kPageSize - 1 || wlo > kpos0) {
        // key index = kt*32 + 8*(rg>>2) + 4*lh + (rg&3); compare the constant part
        const int lim = ((active && pok) ? qpos - kpos0 : -1) - 4 * lh;
        const int low = qlo - kpos0 - 4 * lh;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int rg = 0; rg < 16; ++rg) {
            const int kk = kt * 32 + 8 * (rg >> 2) + (rg & 3);
            st[kt][rg] = (kk <= lim && kk >= low) ? st[kt][rg] : -INFINITY;
          }
      }
      // exp2 of the page's scaled scores against the shift ms into pb (bf16);
      // returns the lane's sum of them (four chains keep the additions independent)
      auto exp_page = [&](float ms) {
        float ps4[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
          for (int ii = 0; ii < 8; ++ii) {
            const int rg = 4 * (2 * (c & 1) + (ii >> 2)) + (ii & 3);
            const float ev = __builtin_amdgcn_exp2f(__builtin_fmaf(st[c >> 1][rg], sc, -ms));
            if (c == 0 && ii < 4) ps4[ii] = ev;
            else ps4[ii & 3] += ev;
            pb[c][ii] = (__bf16)ev;
          }
        }
        return (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]);
      };
      // The page against the running max as it stands. A lane whose sum stays at
      // most 2^7 has no score above m + 7, so its query's max cannot have risen past
      // m + kRescaleThreshold and the page max is not needed. Only when some lane's
      // sum is larger, or from the start while a query of the wave has no finite max
      // yet, does the wave take the page max and compute the page against the max
      // that results. Either way the result is the one taking the max first gives,
      // bit for bit.
      float ps = 0.f;
      bool slow = __any(m == -INFINITY);
      if (!slow) {
        ps = exp_page(m);
        slow = __any(!(ps <= 128.f));
      }
      float mn = m, corr = 1.f;
      bool need = false;
      if (slow) {
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int rg = 0; rg < 16; ++rg) mx = fmaxf(mx, st[kt][rg]);
        {
          // the other half of the query's keys sits in lane l ^ 32. The swap's two
          // results are read by value (__uint_as_float): a __builtin_bit_cast of an
          // element of the returned vector reads element 0 for either index (seen in
          // the front end's IR), which dropped the other half from the page max.
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
          mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sc;
        }
        need = mx > m + kRescaleThreshold;
        mn = need ? mx : m;
        corr = need ? __builtin_amdgcn_exp2f(m - mn) : 1.f;
        ps = exp_page(mn == -INFINITY ? 0.f : mn);
      }
      lsum = lsum * corr + ps;
      m = mn;
      if (__any(need)) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
          for (int i = 0; i < 16; ++i) o[dt][i] *= corr;
          pin(o[dt]);
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) pin(pb[c]);
      pin(m);
      pin(lsum);
    };
    // Ping-pong: waves w and w+4 share a SIMD; group 0 (w < 4) and group 1 run
    // one phase apart, so in every phase one of them issues MFMAs while the
    // other runs the softmax. For page j0 + j (j counted from the run's first
    // visible page j0; LDS buffer j % 3):
    //   phase 2j  : group 0 PV(j-1) + S(j)   | group 1 softmax(j-1)
    //   phase 2j+1: group 0 softmax(j)       | group 1 PV(j-1) + S(j)
    // Page j+1 is copied in during phases 2j..2j+1 into the buffer page j-2 used.
    const int nrel = npages - j0;   // pages of the run from its first visible one
    int64_t next_page = 0;   // table entry of the page the next even phase copies
    // PV(j-1) then S(j) as one stream of 32 MFMAs whose LDS operands are read
    // kAhead MFMAs early, so the reads overlap the matrix core instead of stalling it
    auto fused = [&](auto KBc, auto VBc) {
      constexpr int KB = decltype(KBc)::value;
      constexpr int VB = decltype(VBc)::value;
      const uint8_t* kl = kbuf<KB>();
      const uint8_t* vl = vbuf<VB>();
      constexpr int kAhead = 4;
      // opaque per phase: keeps the compiler from hoisting one address register per
      // (buffer, read) out of the loop; the reads use immediate offsets instead
#pragma unroll
      for (int i = 0; i < 4; ++i) pin(vofs[i]);
#pragma unroll
      for (int i = 0; i < 8; ++i) pin(kofs[i]);
      auto ld = [&](int i) -> bf16x8 {
        if (i < 16) {   // V^T, keys 16c .. 16c+15 (c = i / 4), dims 32dt .. (dt = i % 4)
          const uint8_t* pa = vl + vofs[i & 3] + (16 * (i >> 2)) * kRowBytes;
          const i16x4 ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)pa);
          const i16x4 rb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa + 8 * kRowBytes));
          return join(ra, rb);
        }
        const int ks = (i - 16) >> 1, kt = i & 1;   // K, dims 16ks .., keys 32kt ..
        return *reinterpret_cast<const bf16x8*>(kl + kofs[ks] + kt * 32 * kRowBytes);
      };
      bf16x8 buf[kAhead];
#pragma unroll
      for (int i = 0; i < kAhead; ++i) buf[i] = ld(i);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) st[kt][i] = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const bf16x8 av = buf[i % kAhead];
        if (i + kAhead < 32) buf[i % kAhead] = ld(i + kAhead);
        if (i < 16) o[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[i >> 2], o[i & 3], 0, 0, 0);
        else st[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qb[(i - 16) >> 1], st[i & 1], 0, 0, 0);
      }
      fused_order<kAhead>();
    };
    // j == 0 multiplies the zero weights pb by finite V rows (buffer filled before
    // the loop); j == nrel computes scores of copied fill rows that are never used
    auto mfma_phase = [&](auto KBc, auto VBc, int j) {
      if (j <= nrel) {
        fused(KBc, VBc);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) pin(o[dt]);
        pin(st[0]);
        pin(st[1]);
      }
    };
    // The page loop is compiled once per group (waves 0-3 and waves 4-7 take
    // different branches of a wave-uniform test), so values one group keeps across
    // a phase do not occupy registers in the other group's code. Both copies meet
    // the same barriers in the same order.
    auto page_loop = [&](auto Gc) {
      constexpr int G = decltype(Gc)::value;
      auto phase_even = [&](auto KBc, auto VBc, auto NBc, int j) {
        wait_vmcnt<0>();        // page j's copies (issued two phases ago) are in LDS
        page_barrier();
        if constexpr (G == 1) {
          fetch(NBc, j0 + j + 1, next_page);
          next_page = page_of(j0 + j + 2);   // read now, used by the next even phase
          if (j >= 1 && j - 1 < nrel) softmax(j0 + j - 1);
        } else {
          mfma_phase(KBc, VBc, j);
        }
      };
      auto phase_odd = [&](auto KBc, auto VBc, int j) {
        page_barrier();
        if constexpr (G == 0) {
          if (j < nrel) softmax(j0 + j);
        } else {
          mfma_phase(KBc, VBc, j);
        }
      };
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[c][i] = (__bf16)0.0f;
      if constexpr (G == 1) {
        fetch(Buf<0>{}, j0, page_of(j0));
        fetch(Buf<2>{}, npages, -1);   // finite rows for the zero-weight PV of the first phase
        next_page = page_of(j0 + 1);
      }
      // page steps j = 0 .. nrel (the last one only finishes PV(nrel - 1)); the
      // buffer rotation is unrolled by three and left as soon as step nrel is done
      for (int j = 0;; j += 3) {
        phase_even(Buf<0>{}, Buf<2>{}, Buf<1>{}, j);
        phase_odd(Buf<0>{}, Buf<2>{}, j);
        if (j >= nrel) break;
        phase_even(Buf<1>{}, Buf<0>{}, Buf<2>{}, j + 1);
        phase_odd(Buf<1>{}, Buf<0>{}, j + 1);
        if (j + 1 >= nrel) break;
        phase_even(Buf<2>{}, Buf<1>{}, Buf<0>{}, j + 2);
        phase_odd(Buf<2>{}, Buf<1>{}, j + 2);
        if (j + 2 >= nrel) break;
      }
    };
    if (uniform(w) < 4) page_loop(Buf<0>{});
    else page_loop(Buf<1>{});
    wait_vmcnt<0>();
    __syncthreads();   // all reads of the page buffers and sTab are done before the next run

    // ---- normalise and store: lane holds dims 32dt + 8j + 4lh + i of its query
    const float lt = lsum + __shfl_xor(lsum, 32);
    if (kSplits && n_chunks > 1) {   // a chunk of a split tile: its one run is done; partial state, merge
      split_epilogue(P, o, m, lt, active, qn, w & 3, lh, g, chunk, n_chunks, slot0, split, t0, tid);
      return;
    }
    if (active) {
      const int t = t0 + qn;
      const float inv = 1.0f / lt;
      float* op = P.out + ((int64_t)t * n_q + head) * kHeadDim + 4 * lh;
      const uint16_t* gp = P.gate ? P.gate + ((int64_t)t * n_q + head) * kHeadDim + 4 * lh : nullptr;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 v4 = {o[dt][4 * j] * inv, o[dt][4 * j + 1] * inv, o[dt][4 * j + 2] * inv,
                      o[dt][4 * j + 3] * inv};
          if (gp) {   // output gate: out *= sigmoid(gate) at the same element
            const uint2 gw = *reinterpret_cast<const uint2*>(gp + 32 * dt + 8 * j);
            v4[0] *= sigmoidf(bf16_lo(gw.x));
            v4[1] *= sigmoidf(bf16_hi(gw.x));
            v4[2] *= sigmoidf(bf16_lo(gw.y));
            v4[3] *= sigmoidf(bf16_hi(gw.y));
          }
          *reinterpret_cast<f32x4*>(op + 32 * dt + 8 * j) = v4;
        }
    }
    a = e;
  }
}

}  // namespace
}  // namespace qknr
