// Device-side helpers shared by the gfx950 kernels of libpkv: storage-format
// conversions and cross-lane reductions on a 64-lane wavefront.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;
constexpr int kBlockSize = 16;   // tokens per KV block (the only size built)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Storage-format tags.
struct F32  { static constexpr int kBytes = 4; };
struct BF16 { static constexpr int kBytes = 2; };
struct FP8  { static constexpr int kBytes = 1; };   // OCP e4m3fn

// bfloat16 halves of a 32-bit word -> float (exact: a bf16 is the top half of a float).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Four e4m3 bytes of a 32-bit word -> floats.  gfx950's conversion reads the
// OCP e4m3fn encoding.
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float& a, float& b, float& c, float& d) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  a = lo.x; b = lo.y; c = hi.x; d = hi.y;
}

// Two bf16 x two bf16 products summed into an fp32 accumulator.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, a), __builtin_bit_cast(bf2, b),
                                         acc, false);
}

// DPP controls (within rows of 16 lanes).
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;    // lane i <- lane 7-i within each 8 lanes
constexpr int kDppRowRor8 = 0x128;       // lane i <- lane (i+8)%16 within each 16 lanes

template <int Ctrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_amdgcn_update_dpp(0.0f, x, Ctrl, 0xF, 0xF, false);
}

// Sum over each aligned group of 8 lanes; every lane of the group gets the sum.
__device__ __forceinline__ float sum8(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  return x;
}

// Combine the 8 lane-groups of 8 (lanes l, l^8, l^16, ... l^56): sum / max.
__device__ __forceinline__ float sum_over_groups8(float x) {
  x += dpp<kDppRowRor8>(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}
__device__ __forceinline__ float max_over_groups8(float x) {
  x = fmaxf(x, dpp<kDppRowRor8>(x));
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

// Integer sum over the wave, returned uniform: rows of 16 lanes by DPP, then
// the four row totals read as scalars.
template <int Ctrl>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, Ctrl, 0xF, 0xF, false);
}
__device__ __forceinline__ int wave_sum_uniform(int x) {
  x += dpp_i<kDppQuadXor1>(x);
  x += dpp_i<kDppQuadXor2>(x);
  x += dpp_i<kDppHalfMirror>(x);
  x += dpp_i<kDppRowRor8>(x);
  return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) +
         __builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48);
}
__device__ __forceinline__ int wave_max_uniform(int x) {
  x = max(x, dpp_i<kDppQuadXor1>(x));
  x = max(x, dpp_i<kDppQuadXor2>(x));
  x = max(x, dpp_i<kDppHalfMirror>(x));
  x = max(x, dpp_i<kDppRowRor8>(x));
  return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

// Inclusive prefix sum over the wave's 64 lanes: DPP shifts within rows of
// 16 lanes, then the totals of the earlier rows read as scalars.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_i<0x111>(x);                  // row_shr:1 (lanes shifted in from outside the row read 0)
  x += dpp_i<0x112>(x);                  // row_shr:2
  x += dpp_i<0x114>(x);                  // row_shr:4
  x += dpp_i<0x118>(x);                  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// 8- and 16-byte loads of streamed K/V data.  With PKV_NT_LOADS (the default)
// they carry the nontemporal hint: each slice is read once per step, so it
// should not displace reusable lines from the caches.  kNT = false gives plain
// loads, for data that other workgroups read again soon through the same L2.
#ifndef PKV_NT_LOADS
#define PKV_NT_LOADS 1
#endif
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename T> struct VecOf;
template <> struct VecOf<uint4> { using type = u32x4; };
template <> struct VecOf<uint2> { using type = u32x2; };

template <typename T, bool kNT = bool(PKV_NT_LOADS)>
__device__ __forceinline__ T load_streamed(const char* p) {
  using V = typename VecOf<T>::type;
  V v;
  if constexpr (kNT) v = __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
  else v = *reinterpret_cast<const V*>(p);
  return __builtin_bit_cast(T, v);
}

}  // namespace pkv
