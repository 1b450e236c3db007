// Shared device helpers for the libqknr kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <climits>

namespace qknr {

constexpr int kHeadDim = 128;   // nest qwen3-8b README: head dimension 128
constexpr int kPageSize = 64;   // nest qwen3-8b Entries table: PageSize 64
constexpr int kGroup = 4;       // query heads per KV head (32 / 8)

constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// float32 -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// low / high bfloat16 of a packed pair as float32
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// Agent-coherent float stores and loads (partial softmax states exchanged between
// workgroups: visible across XCDs without a cache-wide write-back).
__device__ __forceinline__ void store_sc1(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_sc1(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Logistic function 1 / (1 + e^-x): the attention output gate (fantasma
// "src/inference/model.zig", fullAttentionForward: attn_out *= sigmoid(gate)).
__device__ __forceinline__ float sigmoidf(float x) { return 1.0f / (1.0f + __expf(-x)); }

// Maximum or minimum of an int over the 64 lanes of a wave, returned to every lane:
// DPP row shifts within each 16-lane row, then row broadcasts across rows, then lane
// 63's value (lanes a shift leaves without a source keep the identity given as the
// old value). No LDS round trips, unlike lane shuffles.
template <bool MAX>
__device__ __forceinline__ int wave_reduce_dpp(int v) {
  constexpr int id = MAX ? INT_MIN : INT_MAX;
  auto op = [](int a, int b) { return MAX ? max(a, b) : min(a, b); };
  int x = v;
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x111, 0xf, 0xf, false));   // row_shr:1
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x112, 0xf, 0xf, false));   // row_shr:2
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x114, 0xf, 0xf, false));   // row_shr:4
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x118, 0xf, 0xf, false));   // row_shr:8
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x142, 0xa, 0xf, false));   // row_bcast:15 into rows 1, 3
  x = op(x, __builtin_amdgcn_update_dpp(id, x, 0x143, 0xc, 0xf, false));   // row_bcast:31 into rows 2, 3
  return __builtin_amdgcn_readlane(x, 63);
}

// Broadcast lane 0's value to the whole wave (result lives in a scalar register).
__device__ __forceinline__ float lane0(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

}  // namespace qknr
