// Shared device and host helpers of liblsi (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/lsi.h"

namespace lsi {

// ---------------------------------------------------------------------------
// Vector types for the MFMA builtins
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) int i32x8;

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Order-preserving float -> uint32 key.  Larger key == larger float.
// -0 is folded onto +0 and NaN sorts below -inf (key 0).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exact fp8 E4M3FN -> bf16 conversion of the four codes in a dword
// (every E4M3FN value is representable in bf16; scale 1.0 keeps it exact).
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t d) {
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d, 1.0f, true);
  u32x2 r;
  r.x = __builtin_bit_cast(uint32_t, lo);
  r.y = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// 8 fp8 codes (two dwords) -> 8 bf16 in the same element order.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t d0, uint32_t d1) {
  u32x2 a = fp8x4_to_bf16x4(d0);
  u32x2 b = fp8x4_to_bf16x4(d1);
  u32x4 v = {a.x, a.y, b.x, b.y};
  return __builtin_bit_cast(bf16x8, v);
}

// Sum of a value across the two 32-lane halves of a wave; every lane gets
// the total.
__device__ __forceinline__ float half_swap_sum(float x) {
  uint32_t u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Inclusive sum over the 64 lanes of a wave by DPP: four row shifts sum each
// row of 16 lanes, then lane 15 of each row is added to the next row and
// lane 31 to the upper two (row_bcast), six VALU steps where a shuffle loop
// makes six LDS-crossbar round trips.
__device__ __forceinline__ uint32_t wave_incl_sum(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// ---------------------------------------------------------------------------
// Host side: error detail and launch checking
// ---------------------------------------------------------------------------
void set_error(const std::string& msg);
int32_t fail(int32_t status, const std::string& msg);
int32_t check_launch(const char* what);
// Kernel timing (lsi_profile_events): with profiling on for the calling
// thread, hands out the next pair of caller events for a kernel named `name`
// (false when off or when the caller's events are used up).
bool prof_next(const char* name, hipEvent_t* start, hipEvent_t* stop);

// Every kernel of the library is launched through this: with timing on, the
// start and stop events travel with the dispatch itself (no extra packets on
// the stream, so the timed kernel runs as it would untimed).
template <class K, class... Args>
inline void launch(K kernel, dim3 grid, dim3 block, uint32_t smem, hipStream_t s, const char* name,
                   Args... args) {
  hipEvent_t e0, e1;
  if (prof_next(name, &e0, &e1))
    hipExtLaunchKernelGGL(kernel, grid, block, smem, s, e0, e1, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, smem, s, args...);
}

inline int ilog2(int v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}
inline bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int num_cus();

}  // namespace lsi
