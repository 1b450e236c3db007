// K2: paged decode attention, bfloat16, split evenly over the GPU (stream-K
// flash decoding). Device code shared by the decode kernel and the single-launch
// step.
//
// nest "models/qwen3-8b/files": Entries table (decode_paged: row b's positions lie
// in the pages table[b] lists, pages of 64) and src/attention.linnet (decode_paged
// calls paged_attention with scale rsqrt(head_dim); decode: every position up to
// and including the query's is visible). fantasma "src/inference/model.zig",
// fullAttentionForward: query head h reads KV head h / 4; scores scaled by
// 1/sqrt(head_dim); max-subtracted softmax; weighted sum of V.
//
// Work list: unit = (row b, KV head g, page p of the row), ordered by row, then KV
// head, then page; a "segment" is the run of units of one (b, g). The grid G is
// the number of workgroups the GPU holds at once, and workgroup i takes an equal
// share [i*C/G, (i+1)*C/G) of a cost scale on which a segment of np pages costs
// kCostA * np + kCostB: every workgroup streams about the same number of 32 KB K/V
// page chunks plus segment set-ups, whatever the rows' lengths. A segment that lies
// inside one workgroup's range is finished there; a segment cut by range ends yields
// one partial softmax state (max, sum, acc) per workgroup touching it, and the last
// of them to finish (ticket counter per segment) merges them in workgroup order, so
// the result depends only on the positions, never on timing or on where pages sit.
//
// Inside a workgroup, wave w takes keys 16w..16w+15 of each page, so each page's
// K and V are read once for the 4 query heads of the group:
//   * scores of 4 heads x 16 keys: 4 x v_mfma_f32_16x16x32_bf16 (query rows 4..15
//     are zero);
//   * online softmax per head, row max by DPP rotations inside 16-lane rows;
//   * P.V on the vector ALU, lane l holding 8 dimensions of 4 keys, the
//     probabilities passed through LDS;
//   * the next page's K/V loads (non-temporal: each byte is read once) are in
//     flight while the current page computes, across segment boundaries too.
// Partial states travel through agent-coherent (sc1) stores and loads with an
// explicit wait before the ticket, so no cache-wide write-back is needed.
#pragma once
#include "common.h"

namespace qknr {
namespace {

constexpr int kPartial = kGroup * (kHeadDim + 2);  // floats per partial: per head (m, l, acc[128])
constexpr int kMaxGrid = 2048;                     // workgroups launched at most
constexpr int kMaxRows = 12288;                    // rows per call (LDS prefix table)
constexpr int kNoAllocMaxPairs = kMaxRows * 8;     // rows x KV heads of the allocation-free call

struct DecodeParams {
  int n_rows, n_kv;
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  int64_t num_pages;
  const int* table;
  int pages_per_row;
  const int* positions;
  float scale_log2;
  float* out;
  int* counters;      // [n_rows * n_kv], zero between calls
  float* partials;    // [grid][2][kPartial]
  const uint16_t* gate;   // optional output gate [n_rows][n_q*128], bf16
};

// max over the 16 lanes of a DPP row, result in every lane of the row
#define QKNR_ROR(v, n) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + (n), 0xf, 0xf, false))

// Sum over the 16 lanes of a row (every lane gets it): DPP rotations by 8, 4, 2, 1.
__device__ __forceinline__ float row_sum16(float x) {
  x += QKNR_ROR(x, 8);
  x += QKNR_ROR(x, 4);
  x += QKNR_ROR(x, 2);
  x += QKNR_ROR(x, 1);
  return x;
}

// Sum of a lane's value over the four 16-lane groups (lanes l, l^16, l^32, l^48):
// v_permlane16_swap pairs row 0 with row 1 and row 2 with row 3, v_permlane32_swap
// the two halves.
__device__ __forceinline__ float group_sum4(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, QKNR_ROR(x, 8));
  x = fmaxf(x, QKNR_ROR(x, 4));
  x = fmaxf(x, QKNR_ROR(x, 2));
  x = fmaxf(x, QKNR_ROR(x, 1));
#undef QKNR_ROR
  return x;
}

// Slices are cut on a cost scale, not on units: a (row, KV head) segment of np pages
// costs kCostA * np + kCostB, so that a slice holding many short segments gets fewer
// pages (a segment's set-up, q and page-id loads and finish cost about as much as
// 2.4 pages' streaming). A row whose position is outside its table has np = 0 but
// keeps its kCostB per KV head, which makes a row's unit offset follow from its cost
// offset and its index alone.
constexpr int kCostA = 5;
constexpr int kCostB = 12;

__device__ __forceinline__ long long range_begin(int i, long long U, int G) { return (long long)i * U / G; }

// workgroup whose range holds point u of a range [0, U) cut into G slices
__device__ __forceinline__ int owner(long long u, long long U, int G) {
  int i = (int)((u * G) / U);
  while (i + 1 < G && range_begin(i + 1, U, G) <= u) ++i;
  while (i > 0 && range_begin(i, U, G) > u) --i;
  return i;
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// One (row, KV head) segment of a workgroup's slice: pages p0..pe-1 of row b's
// pos / 64 + 1 pages for KV head g; whole when the slice holds all of them.
struct DecodeSeg {
  int b, pos, g, p0, pe, win, tbl;
  long long seg_begin, seg_end, stop;
  long long cost_begin;   // the segment's first point on the slices' cost scale
  bool whole;
  bf16x8 qa[4];
};

struct PageRegs {
  bf16x8 k[4];
  uint4 v[4];
  bool ok;
};

// Slice gi of Gd by a workgroup of NW waves (4 or 8): wave w takes keys
// 16(w % 4)..+15 of pages p0 + w / 4, p0 + w / 4 + NW / 4, ... of the slice.
// s_prefix: LDS for n_rows + 1 ints; tid: the thread's index in the workgroup.
template <int NW>
__device__ __forceinline__ void decode_slice(const DecodeParams& P, const int gi, const int Gd, int* s_prefix,
                                             const int tid) {
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  constexpr int NT = 64 * NW;        // threads
  constexpr int kStride = NW / 4;    // pages between a wave's pages
  constexpr int TPH = NT / kGroup;   // threads per head in the merge
  constexpr int DPT = kHeadDim / TPH;   // dimensions per thread in the merge
  __shared__ __attribute__((aligned(16))) float s_p[NW][16][kGroup];
  __shared__ float s_m[NW][kGroup], s_l[NW][kGroup];
  __shared__ __attribute__((aligned(16))) float s_acc[NW][kGroup][kHeadDim];
  __shared__ int s_scan[NW];
  __shared__ int s_last;

  const int w = tid >> 6;
  const int kw = NW == 4 ? w : (w & 3);   // 16-key quarter of a page
  const int l = tid & 63;
  const int hr = l & 15;   // MFMA row/column index within a 16-lane group
  const int G4 = l >> 4;   // 16-lane group
  const int n_q = P.n_kv * kGroup;
  const int max_pos = P.pages_per_row * kPageSize;
  const int n_rows = P.n_rows;

  // ---- cost per row, exclusive prefix over rows (blocked scan); the host keeps the
  // total below 2^31
  auto row_cost = [&](int p) {
    const int np = (p >= 0 && p < max_pos) ? p / kPageSize + 1 : 0;
    return (kCostA * np + kCostB) * P.n_kv;
  };
  {
    const int per = (n_rows + NT - 1) / NT;
    const int b0 = tid * per;
    int local = 0;
    for (int b = b0; b < min(b0 + per, n_rows); ++b) local += row_cost(P.positions[b]);
    int incl = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (l >= d) incl += y;
    }
    if (l == 63) s_scan[w] = incl;
    __syncthreads();
    int off = 0;
    for (int ww = 0; ww < w; ++ww) off += s_scan[ww];
    int run = off + incl - local;
    for (int b = b0; b < min(b0 + per, n_rows); ++b) {
      s_prefix[b] = run;
      run += row_cost(P.positions[b]);
    }
    if (tid == NT - 1) s_prefix[n_rows] = off + incl;
    __syncthreads();
  }
  // units (row, KV head, page) before row b (each row's cost holds kCostB per KV
  // head besides its pages, so the difference is a multiple of kCostA below 2^31)
  auto units_before = [&](int b) -> long long {
    return (long long)((unsigned)(s_prefix[b] - kCostB * P.n_kv * b) / (unsigned)kCostA);
  };
  const int C = s_prefix[n_rows];
  const long long U = units_before(n_rows);
  // the unit at point c < C of the cost scale, lo the last row whose prefix is <= c:
  // in segment g of that row the first kCostB points lead to its first page, then
  // each page takes kCostA points
  auto unit_in_row = [&](int c, int lo) -> long long {
    const int sc = (s_prefix[lo + 1] - s_prefix[lo]) / P.n_kv;   // a segment's cost
    const int np = (sc - kCostB) / kCostA;
    const int r = c - s_prefix[lo];
    const int g = r / sc;
    const int q = r - g * sc - kCostB;
    return units_before(lo) + (long long)g * np + (q <= 0 ? 0 : min(np, (q + kCostA - 1) / kCostA));
  };
  const int top = 1 << (31 - __builtin_clz(n_rows));   // n_rows >= 1

  // a row without units (position outside its table) gets NaN outputs, as the
  // float32 kernel gives it: row b is written by slice b % Gd
  for (int bb = gi; bb < n_rows; bb += Gd) {
    if (s_prefix[bb + 1] - s_prefix[bb] == kCostB * P.n_kv) {
      float* orow = P.out + (int64_t)bb * n_q * kHeadDim;
      for (int e = tid; e < n_q * kHeadDim; e += NT) orow[e] = __builtin_nanf("");
    }
  }
  // the slice's ends on the cost scale, both rows searched in one pass
  const int c0 = (int)range_begin(gi, C, Gd), c1 = (int)range_begin(gi + 1, C, Gd);
  int lo0 = 0, lo1 = 0;
  for (int st = top; st > 0; st >>= 1) {
    if (lo0 + st < n_rows && s_prefix[lo0 + st] <= c0) lo0 += st;
    if (lo1 + st < n_rows && s_prefix[lo1 + st] <= c1) lo1 += st;
  }
  const long long u0 = c0 >= C ? U : unit_in_row(c0, lo0);
  const long long u1 = c1 >= C ? U : unit_in_row(c1, lo1);
  if (u0 >= u1) return;

  const int64_t pool_slots = P.num_pages * kPageSize;
  const int b = lo0;   // u0 lies in this row or a later one (rows without units between)

  // Open the segment holding unit u (row cursor bb moves forward to its row): its
  // page range in this slice, and the loads of its query operand and of the ids of
  // its first 64 pages are issued.
  auto open = [&](long long u, int& bb, DecodeSeg& sg) {
    while (units_before(bb + 1) <= u) ++bb;   // skip rows without units
    sg.b = bb;
    sg.pos = P.positions[bb];
    const int np = sg.pos / kPageSize + 1;
    const long long base = units_before(bb);
    sg.g = (int)((u - base) / np);
    sg.p0 = (int)((u - base) % np);
    sg.cost_begin = s_prefix[bb] + (long long)sg.g * (kCostA * np + kCostB);
    sg.seg_begin = base + (long long)sg.g * np;
    sg.seg_end = sg.seg_begin + np;
    sg.stop = min(u1, sg.seg_end);
    sg.pe = sg.p0 + (int)(sg.stop - u);
    sg.whole = (sg.p0 == 0) && (sg.pe == np);
    // query operand: rows 0..3 = heads 4g..4g+3; k-slot 8*G4+i of step st = dim 8*(4*st+G4)+i,
    // so each K load of a step reads 64 contiguous bytes of every row
    if (hr < kGroup) {
      const uint16_t* qp = P.q + ((int64_t)bb * n_q + sg.g * kGroup + hr) * kHeadDim;
#pragma unroll
      for (int st = 0; st < 4; ++st) sg.qa[st] = *reinterpret_cast<const bf16x8*>(qp + 8 * (4 * st + G4));
    } else {
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int i = 0; i < 8; ++i) sg.qa[st][i] = (__bf16)0.0f;
    }
    // page ids of the segment's pages, 64 at a time: lane i holds the id of page
    // win + i (loaded with q, so no page's K/V load waits on a table load); a
    // wave moves its window when it reaches a page past it (pages rise)
    const int* trow = P.table + (int64_t)bb * P.pages_per_row;
    sg.win = sg.p0;
    sg.tbl = sg.p0 + l < sg.pe ? trow[sg.p0 + l] : -1;
  };

  float m[kGroup], lsum[kGroup], acc[kGroup][8];
  auto reset = [&]() {
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      m[i] = -INFINITY;
      lsum[i] = 0.f;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[i][d] = 0.f;
    }
  };

  auto fetch = [&](DecodeSeg& sg, int p, PageRegs& r) {
    if (p - sg.win >= 64) {
      const int* trow = P.table + (int64_t)sg.b * P.pages_per_row;
      sg.win = p;
      sg.tbl = p + l < sg.pe ? trow[p + l] : -1;
    }
    const int64_t page = __builtin_amdgcn_readlane(sg.tbl, p - sg.win);
    r.ok = page >= 0 && page < P.num_pages;
    const int64_t pg = r.ok ? page : 0;
    const uint16_t* kbase = P.k_pool + (int64_t)sg.g * pool_slots * kHeadDim;
    const uint16_t* vbase = P.v_pool + (int64_t)sg.g * pool_slots * kHeadDim;
    const uint16_t* krow = kbase + (pg * kPageSize + 16 * kw + hr) * kHeadDim + 8 * G4;
    const uint16_t* vrow = vbase + (pg * kPageSize + 16 * kw + 4 * G4) * kHeadDim + 8 * hr;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      // K and V rows are read once per call: streaming (non-temporal) loads
      const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(krow + 32 * st));
      r.k[st] = __builtin_bit_cast(bf16x8, x);
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      // each V row is read whole, once
      const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vrow + jj * kHeadDim));
      r.v[jj] = make_uint4(x[0], x[1], x[2], x[3]);
    }
  };

auto compute = [&](const DecodeSeg& sg, int p, const PageRegs& r) {
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sg.qa[st], r.k[st], sc, 0, 0, 0);
    // lanes 0..15: sc[i] = score of head i with key p*64 + 16w + lane
    const int key0 = p * kPageSize + 16 * kw;
    const bool kvalid = r.ok && key0 + hr <= sg.pos;
    float pr[kGroup];
    bool any_change = false;
    float corr[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      const float x = kvalid ? sc[i] * P.scale_log2 : -INFINITY;
      const float pm = lane0(row_max16(x));
      const float mn = fmaxf(m[i], pm);
      corr[i] = (m[i] == mn) ? 1.f : __builtin_amdgcn_exp2f(m[i] - mn);
      any_change |= (m[i] != mn);
      const float ms = (mn == -INFINITY) ? 0.f : mn;
      pr[i] = __builtin_amdgcn_exp2f(x - ms);
      lsum[i] = lsum[i] * corr[i] + pr[i];
      m[i] = mn;
    }
    if (l < 16) *reinterpret_cast<float4*>(&s_p[w][l][0]) = make_float4(pr[0], pr[1], pr[2], pr[3]);
    __builtin_amdgcn_wave_barrier();
    if (any_change) {
#pragma unroll
      for (int i = 0; i < kGroup; ++i)
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[i][d] *= corr[i];
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int kk = 4 * G4 + jj;
      const bool vok = r.ok && key0 + kk <= sg.pos;
      const float4 ph = *reinterpret_cast<const float4*>(&s_p[w][kk][0]);
      float vf[8];
      vf[0] = bf16_lo(r.v[jj].x); vf[1] = bf16_hi(r.v[jj].x);
      vf[2] = bf16_lo(r.v[jj].y); vf[3] = bf16_hi(r.v[jj].y);
      vf[4] = bf16_lo(r.v[jj].z); vf[5] = bf16_hi(r.v[jj].z);
      vf[6] = bf16_lo(r.v[jj].w); vf[7] = bf16_hi(r.v[jj].w);
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const float x = vok ? vf[d] : 0.f;
        acc[0][d] += ph.x * x;
        acc[1][d] += ph.y * x;
        acc[2][d] += ph.z * x;
        acc[3][d] += ph.w * x;
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  auto finish = [&](const DecodeSeg& sg) {
    // Finish a segment: merge the wave's lanes (DPP rotations within 16 lanes,
    // permlane swaps across the 16-lane groups: no LDS round trips), then the NW
    // waves; store the output, or the partial state and, in the last workgroup of
    // a cut segment, merge the partials
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      lsum[i] = row_sum16(lsum[i]);
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[i][d] = group_sum4(acc[i][d]);
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
    const int hi = tid / TPH;              // head within the group
    const int dd = DPT * (tid % TPH);      // DPT dimensions per thread
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, s_m[ww][hi]);
    float L = 0.f, A[DPT];
#pragma unroll
    for (int c = 0; c < DPT; ++c) A[c] = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float mw = s_m[ww][hi];
      const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L += f * s_l[ww][hi];
#pragma unroll
      for (int c = 0; c < DPT; ++c) A[c] += f * s_acc[ww][hi][dd + c];
    }
    float* orow = P.out + ((int64_t)sg.b * n_q + sg.g * kGroup + hi) * kHeadDim + dd;
    // output gate: out *= sigmoid(gate) at the same element
    float gt[DPT];
#pragma unroll
    for (int c = 0; c < DPT; ++c) gt[c] = 1.f;
    if (P.gate) {
      const uint16_t* gp = P.gate + ((int64_t)sg.b * n_q + sg.g * kGroup + hi) * kHeadDim + dd;
      if constexpr (DPT == 2) {
        const uint32_t gw = *reinterpret_cast<const uint32_t*>(gp);
        gt[0] = sigmoidf(bf16_lo(gw));
        gt[1] = sigmoidf(bf16_hi(gw));
      } else {
#pragma unroll
        for (int c = 0; c < DPT; ++c) gt[c] = sigmoidf(bf16_lo(gp[c]));
      }
    }
    if (sg.whole) {
#pragma unroll
      for (int c = 0; c < DPT; ++c) orow[c] = (A[c] / L) * gt[c];
    } else {
      // slot 1: the segment goes on past this slice (the slice's last segment); slot
      // 0: it began before the slice (its first). A slice has at most one of each.
      const int slot = sg.stop < sg.seg_end ? 1 : 0;
      float* part = P.partials + ((int64_t)gi * 2 + slot) * kPartial + hi * (kHeadDim + 2);
      if ((tid % TPH) == 0) { store_sc1(part, M); store_sc1(part + 1, L); }
#pragma unroll
      for (int c = 0; c < DPT; ++c) store_sc1(part + 2 + dd + c, A[c]);
      __builtin_amdgcn_s_waitcnt(0);   // the partial is at the coherence point before the ticket
      __syncthreads();
      const int rg = sg.b * P.n_kv + sg.g;
      // the workgroups whose slices hold the segment's units: the owners of the
      // cost points of its first and last page, and those between, whose slice ends
      // both fall inside the segment (page index of a point there: seg_page)
      const int np = (int)(sg.seg_end - sg.seg_begin);
      const int i0 = owner(sg.cost_begin + kCostB, C, Gd);
      const int i1 = owner(sg.cost_begin + kCostB + (long long)kCostA * (np - 1), C, Gd);
      auto seg_page = [&](long long c) {
        const long long q = c - sg.cost_begin - kCostB;
        return q <= 0 ? 0 : (int)min((long long)np, (q + kCostA - 1) / kCostA);
      };
      // workgroups with an empty range (a slice inside one page's cost) add no partial
      auto holds = [&](int i) {
        return i == i0 || i == i1 || seg_page(range_begin(i, C, Gd)) < seg_page(range_begin(i + 1, C, Gd));
      };
      int count = 0;
      for (int i = i0; i <= i1; ++i) count += holds(i);
      if (tid == 0) {
        const int old = __hip_atomic_fetch_add(&P.counters[rg], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old == count - 1);
      }
      __syncthreads();
      if (s_last) {
        // one pass over the partials in workgroup order, 8 partials' loads in flight at a time
        float Mx = -INFINITY, Lt = 0.f, B[DPT];
#pragma unroll
        for (int c = 0; c < DPT; ++c) B[c] = 0.f;
        for (int ib = i0; ib <= i1; ib += 8) {
          float mv[8], lv[8], x[8][DPT];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int i = ib + k;
            const bool ok = i <= i1 && holds(i);
            const int slot = i == i1 ? 0 : 1;   // only the last holder's slice ends in the segment
            const float* ps = P.partials + ((int64_t)(ok ? i : i0) * 2 + slot) * kPartial + hi * (kHeadDim + 2);
            mv[k] = ok ? load_sc1(ps) : -INFINITY;
            lv[k] = ok ? load_sc1(ps + 1) : 0.f;
#pragma unroll
            for (int c = 0; c < DPT; ++c) x[k][c] = ok ? load_sc1(ps + 2 + dd + c) : 0.f;
          }
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            if (mv[k] == -INFINITY) continue;
            const float mn = fmaxf(Mx, mv[k]);
            const float fo = (Mx == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(Mx - mn);
            const float fi = __builtin_amdgcn_exp2f(mv[k] - mn);
            Lt = Lt * fo + lv[k] * fi;
#pragma unroll
            for (int c = 0; c < DPT; ++c) B[c] = B[c] * fo + x[k][c] * fi;
            Mx = mn;
          }
        }
#pragma unroll
        for (int c = 0; c < DPT; ++c) orow[c] = (B[c] / Lt) * gt[c];
        if (tid == 0) __hip_atomic_store(&P.counters[rg], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();   // LDS reuse by the next segment
  };

  int bb = b;
  if constexpr (NW == 4) {
    // One stream of pages over the slice's segments: while a segment runs, the
    // next one is already open (row, q, page ids loaded), and its first page is
    // fetched into the free buffer during the current segment's last page, so a
    // segment boundary restarts no memory round trip.
    DecodeSeg cur, nxt;
    open(u0, bb, cur);
    bool more = cur.stop < u1;
    if (more) open(cur.stop, bb, nxt);
    PageRegs ra, rb;
    fetch(cur, cur.p0, ra);
    while (true) {
      reset();
      for (int p = cur.p0; p < cur.pe; p += 2) {
        if (p + 1 < cur.pe) fetch(cur, p + 1, rb);
        else if (more) fetch(nxt, nxt.p0, rb);
        compute(cur, p, ra);
        if (p + 2 < cur.pe) fetch(cur, p + 2, ra);
        else if (p + 2 == cur.pe && more) fetch(nxt, nxt.p0, ra);
        if (p + 1 < cur.pe) compute(cur, p + 1, rb);
      }
      finish(cur);
      if (!more) break;
      if ((cur.pe - cur.p0) & 1) ra = rb;   // an odd page count left the next first page in rb
      cur = nxt;
      more = cur.stop < u1;
      if (more) open(cur.stop, bb, nxt);
    }
  } else {
    // wave w takes pages p0 + w / 4, p0 + w / 4 + 2, ... of each segment
    long long u = u0;
    while (u < u1) {
      DecodeSeg cur;
      open(u, bb, cur);
      reset();
      const int q0 = cur.p0 + (w >> 2);
      PageRegs ra, rb;
      if (q0 < cur.pe) fetch(cur, q0, ra);
      for (int p = q0; p < cur.pe; p += 2 * kStride) {
        if (p + kStride < cur.pe) fetch(cur, p + kStride, rb);
        compute(cur, p, ra);
        if (p + 2 * kStride < cur.pe) fetch(cur, p + 2 * kStride, ra);
        if (p + kStride < cur.pe) compute(cur, p + kStride, rb);
      }
      finish(cur);
      u = cur.stop;
    }
  }
}

}  // namespace
}  // namespace qknr
