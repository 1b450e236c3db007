// K1: fused QK-norm + RoPE + paged cache append. Device code shared by the append
// kernel and the single-launch step.
//
// nest "models/qwen3-8b/files": README (QK-norm: RMS normalisation of every head's
// head_dim slice, after the split into heads and before rope; eps 1e-6),
// src/attention.linnet (decode_paged / prefill_paged / step_paged: q and k are
// normed and rotated, then k and v are written into the pool at the token's slot),
// src/norm.linnet, src/rope.linnet. fantasma "src/inference/model.zig":
// fullAttentionForward and applyRope (rotate_half pairing of i with i + 64).
//
// One workgroup per token; 8 lanes per head vector, lane j holding elements
// 8j..8j+7 of each half (16-byte accesses for bfloat16). The float32 arithmetic is fixed (no contraction into
// fused multiply-adds, pairwise sums in a fixed tree, correctly rounded sqrt and
// division) so the stored bytes are reproducible bit for bit:
//   p_i  = x_i*x_i + x_{i+64}*x_{i+64}                      (i < 64)
//   ss   = pairwise tree over i (neighbours first)
//   r    = 1 / sqrt(ss/128 + eps)
//   y_d  = (x_d * r) * g_d
//   y'_i = y_i*c_i - y_{i+64}*s_i,  y'_{i+64} = y_{i+64}*c_i + y_i*s_i
// The stored value rounds to the pool dtype (bfloat16: nearest even).
#pragma once
#include "common.h"

namespace qknr {
namespace {

template <typename T> struct Vec8;
template <> struct Vec8<float> {
  struct Raw { float4 u, v; };
  __device__ static Raw load_raw(const float* p) {
    return Raw{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
  }
  __device__ static void unpack(const Raw& r, float (&o)[8]) {
    o[0] = r.u.x; o[1] = r.u.y; o[2] = r.u.z; o[3] = r.u.w; o[4] = r.v.x; o[5] = r.v.y; o[6] = r.v.z; o[7] = r.v.w;
  }
  __device__ static void load(const float* p, float (&o)[8]) { unpack(load_raw(p), o); }
  __device__ static void store_agent(float* p, const float (&o)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) __hip_atomic_store(p + i, o[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ static void store(float* p, const float (&o)[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(o[4], o[5], o[6], o[7]);
  }
};
template <> struct Vec8<uint16_t> {
  typedef uint4 Raw;
  __device__ static Raw load_raw(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ static void unpack(const Raw& v, float (&o)[8]) {
    o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
    o[4] = bf16_lo(v.z); o[5] = bf16_hi(v.z); o[6] = bf16_lo(v.w); o[7] = bf16_hi(v.w);
  }
  __device__ static void load(const uint16_t* p, float (&o)[8]) { unpack(load_raw(p), o); }
  __device__ static void store_agent(uint16_t* p, const float (&o)[8]) {
    uint64_t* q = reinterpret_cast<uint64_t*>(p);
    const uint64_t a = (uint64_t)(f32_to_bf16(o[0]) | (f32_to_bf16(o[1]) << 16)) |
                       ((uint64_t)(f32_to_bf16(o[2]) | (f32_to_bf16(o[3]) << 16)) << 32);
    const uint64_t b = (uint64_t)(f32_to_bf16(o[4]) | (f32_to_bf16(o[5]) << 16)) |
                       ((uint64_t)(f32_to_bf16(o[6]) | (f32_to_bf16(o[7]) << 16)) << 32);
    __hip_atomic_store(q, a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ static void store(uint16_t* p, const float (&o)[8]) {
    uint4 v;
    v.x = f32_to_bf16(o[0]) | (f32_to_bf16(o[1]) << 16);
    v.y = f32_to_bf16(o[2]) | (f32_to_bf16(o[3]) << 16);
    v.z = f32_to_bf16(o[4]) | (f32_to_bf16(o[5]) << 16);
    v.w = f32_to_bf16(o[6]) | (f32_to_bf16(o[7]) << 16);
    *reinterpret_cast<uint4*>(p) = v;
  }
};

// Pairwise float32 sum of the n <= 256 non-negative values v[0..n), neighbours
// first, an odd last one carried up a level (the order the whole-vector norm
// pins), by one wave; the result is in lane 0. The values are padded with zeros
// to a power of two: adding +0 leaves a non-negative partial sum unchanged, so the
// balanced tree over the padded values adds exactly what the carried-up order
// adds. Lane l holds the padded values [l*per, (l+1)*per) and adds them pairwise
// in-lane (the first levels); xor shuffles do the rest.
__device__ __forceinline__ float pair_sums_wave(const float* v, int n, int lane) {
  int np2 = 1;
  while (np2 < n) np2 <<= 1;
  const int per = np2 > 64 ? np2 / 64 : 1;   // 1, 2 or 4
  const int lanes = np2 / per;
  float x[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = lane * per + u;
    x[u] = (u < per && i < n) ? v[i] : 0.f;
  }
  float t = per == 4 ? (x[0] + x[1]) + (x[2] + x[3]) : (per == 2 ? x[0] + x[1] : x[0]);
  for (int m = 1; m < lanes; m <<= 1) t = t + __shfl_xor(t, m);
  return t;
}

constexpr int kMaxWholeHeads = 256;   // q heads + kv heads for the whole-vector norm

// WHOLE: one RMS norm over all heads of q and over all heads of k (gains of width
// heads*head_dim). PARTIAL: only the first rotary_dim elements of a head rotate.
// AGENT: every store is an agent-scope relaxed atomic store (written through to
// the level all XCDs share), for readers in other workgroups of the same launch
// that synchronise without a cache write-back.
// Token t by 256 threads (tid 0..255). Positions: token t < n_first reads
// positions[t], a later one positions2[t - n_first]. WHOLE uses workgroup barriers
// (the workgroup is the 256 threads).
template <typename TIn, typename TOut, bool WHOLE, bool PARTIAL, bool AGENT = false>
__device__ __forceinline__ void append_token(
    const int t, const int tid, int n_q_heads, int n_kv_heads,
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ q_gain, const float* __restrict__ k_gain, float eps,
    const float* __restrict__ rope_cos, const float* __restrict__ rope_sin, int rope_rows,
    int rotary_dim,
    const int* __restrict__ positions, const int* __restrict__ positions2, int n_first,
    const int* __restrict__ slots, int n_slotted,
    const int* __restrict__ table, int pages_per_row, int64_t num_pages,
    TOut* __restrict__ q_out, TOut* __restrict__ k_pool, TOut* __restrict__ v_pool) {
#pragma clang fp contract(off)
  __shared__ float s_ss[WHOLE ? 2 : 1][WHOLE ? kMaxWholeHeads : 1];
  __shared__ float s_r[2];
  __shared__ float s_y[PARTIAL ? 32 : 1][PARTIAL ? kHeadDim : 1];
  typedef Vec8<TIn> VIn;
  typedef typename VIn::Raw RawIn;
  const int j = tid & 7;     // lane within the head vector's 8
  const int grp = tid >> 3;  // 32 head vectors in flight
  const int n_norm = n_q_heads + n_kv_heads;
  const int n_v8 = n_kv_heads * (kHeadDim / 8);   // 8-element pieces of the token's v
  auto source = [&](int hv) -> const TIn* {
    return hv < n_q_heads ? q + ((int64_t)t * n_q_heads + hv) * kHeadDim
                          : k + ((int64_t)t * n_kv_heads + (hv - n_q_heads)) * kHeadDim;
  };

  // Every load the position does not decide goes out with the position's: the
  // first two head vectors of the lane's group (hv = grp, grp + 32), its first
  // piece of v and a caller-given slot. Only the page table and the rotation's
  // cos/sin wait for the position. The whole-vector norm leaves its head vectors
  // to the cache instead: it reads them in two passes around a barrier, and
  // holding them in registers costs it a workgroup per CU (36.5 -> 40.8 us on
  // 4224 tokens).
  const int pos = t < n_first ? positions[t] : positions2[t - n_first];
  constexpr int kHeld = WHOLE ? 0 : 2;   // head vectors held from the start
  RawIn ra[2] = {}, rb[2] = {}, rv = {};
#pragma unroll
  for (int u = 0; u < kHeld; ++u) {
    const int hv = grp + 32 * u;
    if (hv < n_norm) {
      ra[u] = VIn::load_raw(source(hv) + 8 * j);
      rb[u] = VIn::load_raw(source(hv) + kHeadDim / 2 + 8 * j);
    }
  }
  if (tid < n_v8) rv = VIn::load_raw(v + (int64_t)t * n_kv_heads * kHeadDim + 8 * tid);
  int64_t slot = -1;
  if (t < n_slotted) slot = slots[t];
  if (pos < 0 || pos >= rope_rows) return;  // no rotation exists for it: skip the token

  const int64_t pool_slots = num_pages * kPageSize;
  if (t >= n_slotted) {
    const int b = t - n_slotted;
    const int pg = pos / kPageSize;
    if (pg < pages_per_row) {
      const int64_t page = table[(int64_t)b * pages_per_row + pg];
      if (page >= 0 && page < num_pages) slot = page * kPageSize + pos % kPageSize;
    }
  }
  if (slot >= pool_slots) slot = -1;

  const int half_r = PARTIAL ? rotary_dim / 2 : kHeadDim / 2;
  float c[8], s[8];
  if (!PARTIAL) {
    Vec8<float>::load(rope_cos + (int64_t)pos * (kHeadDim / 2) + 8 * j, c);
    Vec8<float>::load(rope_sin + (int64_t)pos * (kHeadDim / 2) + 8 * j, s);
  }
  const float* cs_row = rope_cos + (int64_t)pos * half_r;
  const float* sn_row = rope_sin + (int64_t)pos * half_r;
  // partial rotary: cos/sin of the lane's first-half elements 8j + i, read once per
  // token (element e < R/2 uses entry e, R/2 <= e < R entry e - R/2)
  float pc[8], pz[8];
  if (PARTIAL) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = 8 * j + i;
      const int idx = e < half_r ? e : e - half_r;
      pc[i] = e < rotary_dim ? cs_row[idx] : 0.f;
      pz[i] = e < rotary_dim ? sn_row[idx] : 0.f;
    }
  }

  // per-head sum of squares: lane j holds elements 8j..8j+7 of each half; its
  // in-lane adds are the first three levels of the pairwise tree over the 64
  // p_i, the three xor-shuffles the rest
  auto head_ss = [&](const float (&a)[8], const float (&b)[8]) {
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = a[i] * a[i] + b[i] * b[i];
    float ss = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    ss = ss + __shfl_xor(ss, 1, 8);
    ss = ss + __shfl_xor(ss, 2, 8);
    ss = ss + __shfl_xor(ss, 4, 8);
    return ss;
  };

  // the two halves of head vector hv (iteration (hv - grp) / 32 of the group):
  // the first two iterations' were loaded at the start
  auto fetch = [&](int hv, float (&a)[8], float (&b)[8]) {
    const int it = (hv - grp) >> 5;
    if (kHeld > 0 && it == 0) {
      VIn::unpack(ra[0], a);
      VIn::unpack(rb[0], b);
    } else if (kHeld > 1 && it == 1) {
      VIn::unpack(ra[1], a);
      VIn::unpack(rb[1], b);
    } else {
      VIn::load(source(hv) + 8 * j, a);
      VIn::load(source(hv) + kHeadDim / 2 + 8 * j, b);
    }
  };

  if (WHOLE) {
    for (int hv = grp; hv < n_norm; hv += 32) {
      float a[8], b[8];
      fetch(hv, a, b);
      const float ss = head_ss(a, b);
      if (j == 0) {
        if (hv < n_q_heads) s_ss[0][hv] = ss;
        else s_ss[1][hv - n_q_heads] = ss;
      }
    }
    __syncthreads();
    if (tid < 128) {   // wave 0: the q heads' sums, wave 1: the k heads'
      const int which = tid >> 6;
      const int nh = which == 0 ? n_q_heads : n_kv_heads;
      const float total = pair_sums_wave(s_ss[which], nh, tid & 63);
      if ((tid & 63) == 0) {
        const float ms = total / (float)(nh * kHeadDim);
        s_r[which] = 1.0f / __builtin_sqrtf(ms + eps);
      }
    }
    __syncthreads();
  }

  for (int hv = grp; hv < n_norm; hv += 32) {
    const float* g;
    TOut* dst;
    bool write = true;
    int hl;   // head index within q or k
    if (hv < n_q_heads) {
      hl = hv;
      g = q_gain;
      dst = q_out + ((int64_t)t * n_q_heads + hv) * kHeadDim;
    } else {
      hl = hv - n_q_heads;
      g = k_gain;
      write = slot >= 0;
      dst = k_pool + ((int64_t)hl * pool_slots + (write ? slot : 0)) * kHeadDim;
    }
    if (WHOLE) g += (int64_t)hl * kHeadDim;
    float a[8], b[8];
    fetch(hv, a, b);

    float r;
    if (WHOLE) {
      r = s_r[hv < n_q_heads ? 0 : 1];
    } else {
      const float ms = head_ss(a, b) * (1.0f / kHeadDim);
      r = 1.0f / __builtin_sqrtf(ms + eps);
    }

    float ga[8], gb[8];
    Vec8<float>::load(g + 8 * j, ga);
    Vec8<float>::load(g + kHeadDim / 2 + 8 * j, gb);
    float ya[8], yb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ya[i] = (a[i] * r) * ga[i];
      yb[i] = (b[i] * r) * gb[i];
    }
    float oa[8], ob[8];
    if (!PARTIAL) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float ac = ya[i] * c[i];
        const float bs = yb[i] * s[i];
        const float bc = yb[i] * c[i];
        const float as = ya[i] * s[i];
        oa[i] = ac - bs;
        ob[i] = bc + as;
      }
    } else {
      // pairs (e, e + R/2) for e < R/2 may sit in other lanes of the 8: go through LDS
      // (the 8 lanes of a head are one wave, so program order orders the accesses)
      float* yrow = s_y[grp];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        yrow[8 * j + i] = ya[i];
        yrow[kHeadDim / 2 + 8 * j + i] = yb[i];
      }
      __builtin_amdgcn_wave_barrier();
      // cv, sv: cos and sin of the element's rotation angle
      auto rot = [&](int e, float y, float cv, float sv) -> float {
        if (e < half_r) {
          const float ye = y * cv;
          const float ps = yrow[e + half_r] * sv;
          return ye - ps;
        }
        if (e < rotary_dim) {
          const float ye = y * cv;
          const float ps = yrow[e - half_r] * sv;
          return ye + ps;
        }
        return y;
      };
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        oa[i] = rot(8 * j + i, ya[i], pc[i], pz[i]);
        // second-half elements rotate only when R > 64 (entry e - R/2)
        const int e = kHeadDim / 2 + 8 * j + i;
        const bool r2 = e < rotary_dim;
        ob[i] = rot(e, yb[i], r2 ? cs_row[e - half_r] : 0.f, r2 ? sn_row[e - half_r] : 0.f);
      }
      __builtin_amdgcn_wave_barrier();   // the row is rewritten by the group's next head
    }
    if (write) {
      if (AGENT) {
        Vec8<TOut>::store_agent(dst + 8 * j, oa);
        Vec8<TOut>::store_agent(dst + kHeadDim / 2 + 8 * j, ob);
      } else {
        Vec8<TOut>::store(dst + 8 * j, oa);
        Vec8<TOut>::store(dst + kHeadDim / 2 + 8 * j, ob);
      }
    }
  }

  if (slot >= 0) {
    // v: cast only, 8 elements per thread per pass (the first pass loaded at the start)
    for (int e = tid; e < n_v8; e += 256) {
      const int kh = e / (kHeadDim / 8);
      const int c8 = e % (kHeadDim / 8);
      float x[8];
      if (e == tid) VIn::unpack(rv, x);
      else VIn::load(v + ((int64_t)t * n_kv_heads + kh) * kHeadDim + 8 * c8, x);
      TOut* vd = v_pool + ((int64_t)kh * pool_slots + slot) * kHeadDim + 8 * c8;
      if (AGENT) Vec8<TOut>::store_agent(vd, x);
      else Vec8<TOut>::store(vd, x);
    }
  }
}

}  // namespace
}  // namespace qknr
