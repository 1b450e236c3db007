// K2: paged decode attention, split over page ranges (flash decoding), bfloat16.
//
// nest "models/qwen3-8b/files": Entries table (decode_paged: row b's positions lie
// in the pages table[b] lists, pages of 64) and src/attention.linnet (decode_paged
// calls paged_attention with scale rsqrt(head_dim); decode: every position up to
// and including the query's is visible). fantasma "src/inference/model.zig",
// fullAttentionForward: query head h reads KV head h / 4; scores scaled by
// 1/sqrt(head_dim); max-subtracted softmax; weighted sum of V.
//
// Work item = (row b, KV head g, range of the row's pages). One workgroup of 4
// waves runs an item; wave w takes keys 16w..16w+15 of every page, so each 16 KB
// K chunk and 16 KB V chunk of a (page, KV head) is read once for all 4 query
// heads of the group:
//   * scores of the 4 heads x 16 keys on one v_mfma_f32_16x16x32_bf16 chain
//     (query rows 4..15 are zero);
//   * an online softmax per head with wave-level max/sum reductions;
//   * P.V on the vector ALU, lane l holding 8 dimensions of 4 keys.
// The 4 waves merge through LDS; when a row has several items, each writes its
// (max, sum, acc) state to the workspace and the last one to finish (a ticket
// counter per (row, KV head)) merges them in split order, so the result does not
// depend on timing. The split size depends only on the positions.
//
// Every workgroup plans the same split from the positions (sum and max of the
// rows' page counts), then walks the item list with a grid stride.
#include "common.h"
#include "kernels.h"

namespace qknr {
namespace {

constexpr int kMaxSplits = 64;        // items per (row, KV head) at most
constexpr int kMinSplitPages = 2;     // pages per item at least
constexpr int kTargetItems = 2048;    // items the plan aims for
constexpr int kGridCap = 2048;        // workgroups launched at most
constexpr int kPartial = kGroup * (kHeadDim + 2);  // floats per item: per head (m, l, acc[128])
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = max(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float max16(float x) {
  x = fmaxf(x, __shfl_xor(x, 8, 16));
  x = fmaxf(x, __shfl_xor(x, 4, 16));
  x = fmaxf(x, __shfl_xor(x, 2, 16));
  x = fmaxf(x, __shfl_xor(x, 1, 16));
  return x;
}
__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 8, 16);
  x += __shfl_xor(x, 4, 16);
  x += __shfl_xor(x, 2, 16);
  x += __shfl_xor(x, 1, 16);
  return x;
}

__global__ __launch_bounds__(256) void paged_decode_bf16_kernel(
    int n_rows, int n_kv, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, int64_t num_pages, const int* __restrict__ table,
    int pages_per_row, const int* __restrict__ positions, float scale_log2, float* __restrict__ out,
    int* __restrict__ counters, float* __restrict__ partials) {
  __shared__ int s_red[8];
  __shared__ int s_last;
  __shared__ float s_m[4][kGroup], s_l[4][kGroup];
  __shared__ __attribute__((aligned(16))) float s_acc[4][kGroup][kHeadDim];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int l = tid & 63;
  const int hr = l & 15;   // MFMA row/column index within a 16-lane group
  const int G = l >> 4;    // 16-lane group
  const int n_q = n_kv * kGroup;
  const int max_pos = pages_per_row * kPageSize;

  // ---- plan: the same in every workgroup
  int sum = 0, mx = 0;
  for (int b = tid; b < n_rows; b += 256) {
    const int p = positions[b];
    const int np = (p >= 0 && p < max_pos) ? p / kPageSize + 1 : 0;
    sum += np;
    mx = max(mx, np);
  }
  sum = wave_sum_i(sum);
  mx = wave_max_i(mx);
  if (l == 0) { s_red[w] = sum; s_red[4 + w] = mx; }
  __syncthreads();
  sum = s_red[0] + s_red[1] + s_red[2] + s_red[3];
  mx = max(max(s_red[4], s_red[5]), max(s_red[6], s_red[7]));
  const long long chunks = (long long)sum * n_kv;
  int split = (int)((chunks + kTargetItems - 1) / kTargetItems);
  split = max(split, kMinSplitPages);
  split = max(split, (mx + kMaxSplits - 1) / kMaxSplits);
  const int s_max = (mx + split - 1) / split;
  const long long n_items = (long long)n_rows * s_max * n_kv;

  const int64_t pool_slots = num_pages * kPageSize;

  for (long long it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int g = (int)(it % n_kv);
    const long long r2 = it / n_kv;
    const int s = (int)(r2 % s_max);
    const int b = (int)(r2 / s_max);
    const int pos = positions[b];
    if (pos < 0 || pos >= max_pos) continue;
    const int np = pos / kPageSize + 1;
    const int pb = s * split;
    if (pb >= np) continue;
    const int pe = min(pb + split, np);
    const int nsplit = (np + split - 1) / split;

    // query operand: rows 0..3 = heads 4g..4g+3, 8 dims per MFMA step
    bf16x8 qa[4];
    if (hr < kGroup) {
      const uint16_t* qp = q + ((int64_t)b * n_q + g * kGroup + hr) * kHeadDim + 32 * G;
#pragma unroll
      for (int st = 0; st < 4; ++st) qa[st] = *reinterpret_cast<const bf16x8*>(qp + 8 * st);
    } else {
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < 8; ++i) qa[st][i] = (__bf16)0.0f;
    }

    float m[kGroup], lsum[kGroup], acc[kGroup][8];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      m[i] = -INFINITY;
      lsum[i] = 0.f;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[i][d] = 0.f;
    }
    const uint16_t* kbase = k_pool + (int64_t)g * pool_slots * kHeadDim;
    const uint16_t* vbase = v_pool + (int64_t)g * pool_slots * kHeadDim;
    const int* trow = table + (int64_t)b * pages_per_row;

    for (int p = pb; p < pe; ++p) {
      const int64_t page = trow[p];
      if (page < 0 || page >= num_pages) continue;
      const int key0 = p * kPageSize + 16 * w;  // position of this wave's first key
      const uint16_t* krow = kbase + (page * kPageSize + 16 * w + hr) * kHeadDim + 32 * G;
      bf16x8 kb[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) kb[st] = *reinterpret_cast<const bf16x8*>(krow + 8 * st);
      const uint16_t* vrow = vbase + (page * kPageSize + 16 * w + 4 * G) * kHeadDim + 8 * hr;
      uint4 vv[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) vv[jj] = *reinterpret_cast<const uint4*>(vrow + jj * kHeadDim);

      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[st], kb[st], sc, 0, 0, 0);

      // lanes 0..15: sc[i] = score of head i with key key0 + l
      const bool kvalid = key0 + hr <= pos;
      float x[kGroup], mn[kGroup], corr[kGroup], pr[kGroup];
      bool any_change = false;
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        x[i] = kvalid ? sc[i] * scale_log2 : -INFINITY;
        const float pm = lane0(max16(x[i]));
        mn[i] = fmaxf(m[i], pm);
        corr[i] = (m[i] == mn[i]) ? 1.f : __builtin_amdgcn_exp2f(m[i] - mn[i]);
        any_change |= (m[i] != mn[i]);
        const float ms = (mn[i] == -INFINITY) ? 0.f : mn[i];
        pr[i] = __builtin_amdgcn_exp2f(x[i] - ms);
        lsum[i] = lsum[i] * corr[i] + pr[i];
        m[i] = mn[i];
      }
      if (any_change) {
#pragma unroll
        for (int i = 0; i < kGroup; ++i)
#pragma unroll
          for (int d = 0; d < 8; ++d) acc[i][d] *= corr[i];
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int src = 4 * G + jj;  // lane holding this key's probabilities
        const bool vok = key0 + src <= pos;
        float ph[kGroup];
#pragma unroll
        for (int i = 0; i < kGroup; ++i) ph[i] = __shfl(pr[i], src);
        float vf[8];
        vf[0] = bf16_lo(vv[jj].x); vf[1] = bf16_hi(vv[jj].x);
        vf[2] = bf16_lo(vv[jj].y); vf[3] = bf16_hi(vv[jj].y);
        vf[4] = bf16_lo(vv[jj].z); vf[5] = bf16_hi(vv[jj].z);
        vf[6] = bf16_lo(vv[jj].w); vf[7] = bf16_hi(vv[jj].w);
#pragma unroll
        for (int d = 0; d < 8; ++d) vf[d] = vok ? vf[d] : 0.f;
#pragma unroll
        for (int i = 0; i < kGroup; ++i)
#pragma unroll
          for (int d = 0; d < 8; ++d) acc[i][d] += ph[i] * vf[d];
      }
    }

    // ---- merge the wave's lanes, then the 4 waves
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      lsum[i] = sum16(lsum[i]);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        acc[i][d] += __shfl_xor(acc[i][d], 16);
        acc[i][d] += __shfl_xor(acc[i][d], 32);
      }
    }
    if (l < 16) {
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        float4* dst = reinterpret_cast<float4*>(&s_acc[w][i][8 * l]);
        dst[0] = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
        dst[1] = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
      }
    }
    if (l == 0) {
#pragma unroll
      for (int i = 0; i < kGroup; ++i) { s_m[w][i] = m[i]; s_l[w][i] = lsum[i]; }
    }
    __syncthreads();
    const int hi = tid >> 6;          // head within the group
    const int dd = 2 * (tid & 63);    // two dimensions per thread
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, s_m[ww][hi]);
    float L = 0.f, A0 = 0.f, A1 = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float mw = s_m[ww][hi];
      const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L += f * s_l[ww][hi];
      A0 += f * s_acc[ww][hi][dd];
      A1 += f * s_acc[ww][hi][dd + 1];
    }
    float* orow = out + ((int64_t)b * n_q + g * kGroup + hi) * kHeadDim + dd;
    if (nsplit == 1) {
      orow[0] = A0 / L;
      orow[1] = A1 / L;
    } else {
      const int64_t rg = (int64_t)b * n_kv + g;
      float* part = partials + (rg * kMaxSplits + s) * kPartial + hi * (kHeadDim + 2);
      if ((tid & 63) == 0) { part[0] = M; part[1] = L; }
      part[2 + dd] = A0;
      part[3 + dd] = A1;
      __threadfence();
      __syncthreads();
      if (tid == 0) s_last = (atomicAdd(&counters[rg], 1) == nsplit - 1);
      __syncthreads();
      if (s_last) {
        __threadfence();
        const float* base = partials + rg * kMaxSplits * kPartial + hi * (kHeadDim + 2);
        float Mx = -INFINITY;
        for (int sp = 0; sp < nsplit; ++sp) Mx = fmaxf(Mx, base[sp * kPartial]);
        float Lt = 0.f, B0 = 0.f, B1 = 0.f;
        for (int sp = 0; sp < nsplit; ++sp) {
          const float* ps = base + sp * kPartial;
          const float f = (ps[0] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ps[0] - Mx);
          Lt += f * ps[1];
          B0 += f * ps[2 + dd];
          B1 += f * ps[3 + dd];
        }
        orow[0] = B0 / Lt;
        orow[1] = B1 / Lt;
        if (tid == 0) counters[rg] = 0;
      }
    }
    __syncthreads();
  }
}

}  // namespace

size_t decode_workspace_bytes(int n_rows, int n_kv_heads, int /*pages_per_row*/) {
  const size_t pairs = (size_t)n_rows * n_kv_heads;
  const size_t counters = (pairs * sizeof(int) + 255) / 256 * 256;
  return counters + pairs * kMaxSplits * kPartial * sizeof(float);
}

hipError_t launch_decode_bf16(hipStream_t stream, const AttnArgs& a) {
  const size_t pairs = (size_t)a.n_queries * a.n_kv_heads;
  const size_t counter_bytes = (pairs * sizeof(int) + 255) / 256 * 256;
  int* counters = static_cast<int*>(a.workspace);
  float* partials = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + counter_bytes);
  long long max_splits = (long long)(a.pages_per_row + kMinSplitPages - 1) / kMinSplitPages;
  if (max_splits > kMaxSplits) max_splits = kMaxSplits;
  const long long items = (long long)pairs * max_splits;
  const int grid = (int)(items < kGridCap ? items : kGridCap);
  hipLaunchKernelGGL(paged_decode_bf16_kernel, dim3(grid), dim3(256), 0, stream, a.n_queries,
                     a.n_kv_heads, (const uint16_t*)a.q, (const uint16_t*)a.k_pool,
                     (const uint16_t*)a.v_pool, a.num_pages, a.table, a.pages_per_row,
                     a.positions, a.scale * kLog2e, a.out, counters, partials);
  return hipGetLastError();
}

}  // namespace qknr
