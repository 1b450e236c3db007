// K3: paged prefill attention with bfloat16 MFMA, float32 accumulation.
//
// nest "models/qwen3-8b/files": Entries table (prefill_paged: prompts packed end to
// end, each token attending over its row's pages up to its position, for chunks
// and shared prefixes) and src/attention.linnet (prefill_paged writes k/v into the
// pool, then paged_prefill_attention reads table[rows[p]]; scale rsqrt(head_dim)).
// fantasma "src/inference/model.zig", fullAttentionForward: query head h reads KV
// head h / 4; max-subtracted softmax; weighted sum of V.
//
// Work item = (64-token tile of the pack, KV head g); wave w is query head 4g+w,
// so the 4 waves share every K/V page staged in LDS. Per 64-key page and wave:
//   S^T (64 keys x 64 queries) = K . Q^T   : 32 x v_mfma_f32_32x32x16_bf16,
//       K from LDS (16-byte reads), Q kept in registers;
//   online softmax along the lane's own keys (each lane holds one query's keys,
//       the other half sits in lane l^32), the running max only moves when the
//       page's max exceeds it by more than 2^8 (exact after the final division);
//   O^T (128 dims x 64 queries) += V^T . P^T : 32 MFMAs, V^T read from the
//       row-major V page with ds_read_b64_tr_b16, P^T straight from the S^T
//       accumulators (keys permuted the same way on both operands).
// Pages stream through a double-buffered LDS stage. A tile that holds tokens of
// several rows runs once per row ("run"); masking uses each token's position.
// A plan kernel orders tiles by decreasing cost (largest visible position) so
// the long ones start first; item i maps to KV head i % 8, which keeps one KV
// head's pages on one XCD's L2.
#include "common.h"
#include "kernels.h"

namespace qknr {
namespace {

constexpr int kTile = 64;
constexpr int kKStride = kHeadDim + 8;    // bf16 per K row in LDS (16-byte reads, no conflicts)
constexpr int kVStride = kHeadDim + 16;   // bf16 per V row in LDS (transposed 8-byte reads)
constexpr int kPlanMaxTiles = 8192;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ---------------------------------------------------------------- planning
__global__ __launch_bounds__(1024) void prefill_plan_kernel(int n_tokens, const int* __restrict__ positions,
                                                            int n_tiles, int* __restrict__ order) {
  __shared__ unsigned long long keys[kPlanMaxTiles];
  int npow2 = 1;
  while (npow2 < n_tiles) npow2 <<= 1;
  // cost of a tile: its largest visible position + 1; one wave per tile, one lane per token
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n_waves = blockDim.x >> 6;
  for (int i = wave; i < npow2; i += n_waves) {
    int cost = 0;
    if (i < n_tiles) {
      const int t = i * kTile + lane;
      cost = t < n_tokens ? max(positions[t] + 1, 0) : 0;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) cost = max(cost, __shfl_xor(cost, m));
    }
    if (lane == 0)
      keys[i] = i < n_tiles ? ((unsigned long long)(0xffffffffu - (unsigned)cost) << 32) | (unsigned)i : ~0ull;
  }
  __syncthreads();
  for (int k = 2; k <= npow2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < npow2; i += blockDim.x) {
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
  for (int i = threadIdx.x; i < n_tiles; i += blockDim.x) order[i] = (int)(keys[i] & 0xffffffffu);
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
  const int* order;
};

__device__ __forceinline__ bf16x8 join(i16x4 a, i16x4 b) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Waves w and w+4 share a SIMD: w < 4 is group A (queries 0..31 of the tile),
// w >= 4 group B (queries 32..63), both for query head 4g + (w & 3). Between two
// workgroup barriers ("phases") one group issues MFMAs while the other runs the
// softmax, so each SIMD's matrix core and vector ALU work at the same time:
//   group A, phase 2j  : O += V(j-1).P(j-1);  S(j) = K(j).Q   (MFMA)
//   group A, phase 2j+1: mask + softmax of S(j) -> P(j)      (VALU)
//   group B runs the same sequence one phase later.
// Page j's K is read in phases 2j..2j+1 and its V in 2j+2..2j+3, so three LDS
// page buffers suffice; page j+1 is fetched in phase 2j and stored in 2j+1.
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void paged_prefill_bf16_kernel(PrefillParams P) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[3][kTile * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t sV[3][kTile * kVStride];
  __shared__ int sRow[kTile], sPos[kTile];

  const int n_q = P.n_kv * kGroup;
  const int item = blockIdx.x;
  const int tile = P.order ? P.order[item / P.n_kv] : item / P.n_kv;
  const int g = item % P.n_kv;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int lq = l & 31;        // query index within the wave's 32 queries
  const int lh = l >> 5;        // half of the wave
  const int grp = w >> 2;       // 0: group A, 1: group B (one phase later)
  const int head = g * kGroup + (w & 3);
  const int qn = 32 * grp + lq; // the lane's query within the tile
  const int t0 = tile * kTile;
  const int max_pos = P.pages_per_row * kPageSize;

  if (tid < kTile) {
    const int t = t0 + tid;
    int r = -1, p = -1;
    if (t < P.n_tokens) {
      r = P.rows[t];
      p = P.positions[t];
      if (r < 0 || r >= P.n_table_rows || p < 0 || p >= max_pos) r = -1;
    }
    sRow[tid] = r;
    sPos[tid] = p;
  }
  __syncthreads();

  // Q^T operand: lane holds query qn, dims 16*ks + 8*lh .. +7
  const int qpos = sPos[qn];
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

  const int64_t pool_slots = P.num_pages * kPageSize;
  const uint16_t* kbase = P.k_pool + (int64_t)g * pool_slots * kHeadDim;
  const uint16_t* vbase = P.v_pool + (int64_t)g * pool_slots * kHeadDim;
  const float sc = P.scale_log2;
  const int G4 = l >> 4;
  const int jj = l & 15;

  int a = 0;
  while (a < kTile) {
    const int r = uniform(sRow[a]);
    int e = a + 1;
    while (e < kTile && sRow[e] == r) ++e;
    e = uniform(e);
    if (r < 0) { a = e; continue; }
    int maxp = 0;
    for (int i = a; i < e; ++i) maxp = max(maxp, sPos[i]);
    maxp = uniform(maxp);
    const int npages = maxp / kPageSize + 1;
    const int* trow = P.table + (int64_t)r * P.pages_per_row;

    const bool active = qn >= a && qn < e;
    // smallest position among the wave's queries; -1 when some query is not in this run
    int wmin = active ? qpos : -1;
#pragma unroll
    for (int mm = 32; mm >= 1; mm >>= 1) wmin = min(wmin, __shfl_xor(wmin, mm));
    wmin = uniform(wmin);

    float m = -INFINITY;     // running max of scale*log2(e)*score, per query
    float lsum = 0.f;        // this lane's share of the softmax denominator
    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
    f32x16 st[2];
    bf16x8 pb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[c][i] = (__bf16)0.0f;

    // staging: 1024 chunks of 16 bytes for K and for V, 2 per thread
    uint4 kr[2], vr[2];
    auto fetch = [&](int p) {
      const int64_t page = trow[p];
      const bool ok = page >= 0 && page < P.num_pages;
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int c = tid + 512 * rr;
        const int key = c >> 4;
        const int c16 = c & 15;
        if (ok && p * kPageSize + key <= maxp) {
          const int64_t off = (page * kPageSize + key) * kHeadDim + c16 * 8;
          kr[rr] = *reinterpret_cast<const uint4*>(kbase + off);
          vr[rr] = *reinterpret_cast<const uint4*>(vbase + off);
        } else {
          kr[rr] = make_uint4(0, 0, 0, 0);
          vr[rr] = make_uint4(0, 0, 0, 0);
        }
      }
    };
    auto stage = [&](int buf) {
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int c = tid + 512 * rr;
        const int key = c >> 4;
        const int c16 = c & 15;
        *reinterpret_cast<uint4*>(&sK[buf][key * kKStride + c16 * 8]) = kr[rr];
        *reinterpret_cast<uint4*>(&sV[buf][key * kVStride + c16 * 8]) = vr[rr];
      }
    };

    fetch(0);
    stage(0);
    __syncthreads();

    const int n_phases = 2 * npages + 2;
    for (int ph = 0; ph < n_phases; ++ph) {
      const int jn = ph >> 1;                  // page staged during this phase pair: jn + 1
      if (!(ph & 1) && jn + 1 < npages) fetch(jn + 1);
      const int my = ph - grp;                 // this group's own phase
      if (my >= 0) {
        const int j = my >> 1;
        if (!(my & 1)) {
          // ---- MFMA phase: O += V(j-1) . P(j-1), then S(j) = K(j) . Q
          if (j >= 1) {
            const uint16_t* vl = &sV[(j - 1) % 3][0];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const int keyA = 16 * c + 4 * lh;
#pragma unroll
              for (int dt = 0; dt < 4; ++dt) {
                const int dim0 = 32 * dt + 16 * (G4 & 1);
                const uint16_t* pa = vl + (keyA + (jj >> 2)) * kVStride + dim0 + 4 * (jj & 3);
                const i16x4 ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)pa);
                const i16x4 rb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa + 8 * kVStride));
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join(ra, rb), pb[c], o[dt], 0, 0, 0);
              }
            }
          }
          if (j < npages) {
            const uint16_t* kl = &sK[j % 3][0];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
              for (int i = 0; i < 16; ++i) st[kt][i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
              for (int kt = 0; kt < 2; ++kt) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kl + (kt * 32 + lq) * kKStride + 16 * ks + 8 * lh);
                st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[ks], st[kt], 0, 0, 0);
              }
            }
          }
        } else if (j < npages) {
          // ---- VALU phase: mask, online softmax of S(j) -> P(j)
          const int kpos0 = j * kPageSize;
          const int64_t page = trow[j];
          const bool pok = page >= 0 && page < P.num_pages;
          if (!pok || wmin < kpos0 + kPageSize - 1) {
            const int lim = (active && pok) ? qpos - kpos0 : -1;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
              for (int rg = 0; rg < 16; ++rg) {
                const int key = kt * 32 + 8 * (rg >> 2) + 4 * lh + (rg & 3);
                st[kt][rg] = (key <= lim) ? st[kt][rg] : -INFINITY;
              }
          }
          float mx = -INFINITY;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int rg = 0; rg < 16; ++rg) mx = fmaxf(mx, st[kt][rg]);
          mx = fmaxf(mx, __shfl_xor(mx, 32)) * sc;
          const bool need = mx > m + kRescaleThreshold;
          const float mn = need ? mx : m;
          const float corr = need ? __builtin_amdgcn_exp2f(m - mn) : 1.f;
          const float ms = (mn == -INFINITY) ? 0.f : mn;
          float ps = 0.f;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) {
              const int rg = 4 * (2 * (c & 1) + (ii >> 2)) + (ii & 3);
              const float ev = __builtin_amdgcn_exp2f(__builtin_fmaf(st[c >> 1][rg], sc, -ms));
              ps += ev;
              pb[c][ii] = (__bf16)ev;
            }
          }
          lsum = lsum * corr + ps;
          m = mn;
          if (__any(need)) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
              for (int i = 0; i < 16; ++i) o[dt][i] *= corr;
          }
        }
      }
      if ((ph & 1) && jn + 1 < npages) stage((jn + 1) % 3);
      __syncthreads();
    }

    // ---- normalise and store: lane holds dims 32dt + 8j + 4lh + i of its query
    const float lt = lsum + __shfl_xor(lsum, 32);
    if (active) {
      const int t = t0 + qn;
      const float inv = 1.0f / lt;
      float* op = P.out + ((int64_t)t * n_q + head) * kHeadDim + 4 * lh;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 v4 = {o[dt][4 * j] * inv, o[dt][4 * j + 1] * inv, o[dt][4 * j + 2] * inv,
                            o[dt][4 * j + 3] * inv};
          *reinterpret_cast<f32x4*>(op + 32 * dt + 8 * j) = v4;
        }
    }
    a = e;
  }
}

}  // namespace

size_t prefill_workspace_bytes(int n_tokens, int /*n_kv_heads*/) {
  const size_t tiles = (size_t)(n_tokens + kTile - 1) / kTile;
  return (tiles * sizeof(int) + 255) / 256 * 256;
}

hipError_t launch_prefill_bf16(hipStream_t stream, const AttnArgs& a) {
  const int n_tiles = (a.n_queries + kTile - 1) / kTile;
  int* order = nullptr;
  if (n_tiles <= kPlanMaxTiles) {
    order = static_cast<int*>(a.workspace);
    hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(1024), 0, stream, a.n_queries,
                       a.positions, n_tiles, order);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  PrefillParams P;
  P.n_tokens = a.n_queries;
  P.n_kv = a.n_kv_heads;
  P.q = (const uint16_t*)a.q;
  P.k_pool = (const uint16_t*)a.k_pool;
  P.v_pool = (const uint16_t*)a.v_pool;
  P.num_pages = a.num_pages;
  P.table = a.table;
  P.n_table_rows = a.n_table_rows;
  P.pages_per_row = a.pages_per_row;
  P.rows = a.rows;
  P.positions = a.positions;
  P.scale_log2 = a.scale * kLog2e;
  P.out = a.out;
  P.order = order;
  hipLaunchKernelGGL(paged_prefill_bf16_kernel, dim3(n_tiles * a.n_kv_heads), dim3(512), 0, stream, P);
  return hipGetLastError();
}

}  // namespace qknr
