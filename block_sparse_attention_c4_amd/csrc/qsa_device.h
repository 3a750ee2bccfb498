// Device-side helpers shared by the QSA c4 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

constexpr int kBlock = 4;        // tokens per compressed block
constexpr int kTopK = 512;       // blocks kept per query
constexpr int kMaxSel = 2051;    // 4 * 512 + 3
constexpr int kIdxHeads = 4;
constexpr int kIdxDim = 128;
constexpr int kQHeads = 16;
constexpr int kKVHeads = 2;
constexpr int kGroup = kQHeads / kKVHeads;   // 8 query heads per KV head
constexpr int kHeadDim = 256;
constexpr int kMaxContext = 262144;
constexpr int kMaxBlocks = kMaxContext / kBlock;   // 65536
constexpr int kScoreGroup = 16;  // blocks per group maximum written by the scorer

// Device-side contents (page tables, positions, counts) are trusted.  A build with
// -DQSA_DEBUG checks the documented ranges where the kernels read them and traps on
// a violation; the release build compiles the checks away.
#ifdef QSA_DEBUG
#define QSA_CHECK(cond) \
  do {                  \
    if (!(cond)) __builtin_trap(); \
  } while (0)
#else
#define QSA_CHECK(cond) \
  do {                  \
  } while (0)
#endif

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// double -> bf16 bits, round to nearest even, without double rounding: the value
// is first cut to float toward zero with a sticky last bit (round to odd), which
// keeps 16 guard bits below bf16's last place.
__device__ __forceinline__ uint32_t f64_to_bf16(double x) {
  float f = __double2float_rz(x);
  uint32_t u = __float_as_uint(f);
  if ((double)f != x) u |= 1u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Order-preserving unsigned key of a float (larger float -> larger key).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Cross-lane moves within a row of 16 lanes (DPP).
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}
// Sum over the 16 lanes of a row; every lane of the row receives the sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xb1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f<0x4e>(v);    // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);   // row_half_mirror
  v += dpp_f<0x140>(v);   // row_mirror
  return v;
}

// Max over the 16 lanes of a row; every lane of the row receives it.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xb1>(v));
  v = fmaxf(v, dpp_f<0x4e>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return v;
}

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// Value of lane ^ 16 / lane ^ 32, on the VALU (gfx950 v_permlane16/32_swap): swapping
// a register with itself leaves the partner row (half) in one of the two results.
__device__ __forceinline__ uint32_t lane_xor16_u32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return ((threadIdx.x >> 4) & 1) ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t lane_xor32_u32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return ((threadIdx.x >> 5) & 1) ? r[0] : r[1];
}
__device__ __forceinline__ float lane_xor16(float v) {
  return __uint_as_float(lane_xor16_u32(__float_as_uint(v)));
}
__device__ __forceinline__ float lane_xor32(float v) {
  return __uint_as_float(lane_xor32_u32(__float_as_uint(v)));
}

template <int kCtrl, int kRowMask>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, kRowMask, 0xf, false);
}
// Inclusive prefix sum over the 64 lanes (DPP: row shifts, then row broadcasts).
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += dpp_i<0x111, 0xf>(x);   // row_shr:1
  x += dpp_i<0x112, 0xf>(x);   // row_shr:2
  x += dpp_i<0x114, 0xf>(x);   // row_shr:4
  x += dpp_i<0x118, 0xf>(x);   // row_shr:8
  x += dpp_i<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
  x += dpp_i<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}
// Max / min of a 32-bit unsigned over the 64 lanes; every lane gets the result.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)dpp_i<0xb1, 0xf>((int)v));
  v = max(v, (uint32_t)dpp_i<0x4e, 0xf>((int)v));
  v = max(v, (uint32_t)dpp_i<0x141, 0xf>((int)v));
  v = max(v, (uint32_t)dpp_i<0x140, 0xf>((int)v));
  v = max(v, lane_xor16_u32(v));
  return max(v, lane_xor32_u32(v));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)dpp_i<0xb1, 0xf>((int)v));
  v = min(v, (uint32_t)dpp_i<0x4e, 0xf>((int)v));
  v = min(v, (uint32_t)dpp_i<0x141, 0xf>((int)v));
  v = min(v, (uint32_t)dpp_i<0x140, 0xf>((int)v));
  v = min(v, lane_xor16_u32(v));
  return min(v, lane_xor32_u32(v));
}

// max(0, x) as an integer max on the bits: negative values and -0 become +0.
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// Block score from the 4 head dots: sum_h w_h * max(0, d_h), in a fixed order.  The
// sum starts from +0 and every term adds a product onto it, so a zero score is +0
// and equal scores have equal keys.  Every MFMA scorer uses this function, so equal
// operands give bit-identical scores.
__device__ __forceinline__ float head_mix(f32x4_t d, const float (&w)[kIdxHeads]) {
  float s = fmaf(w[0], relu_bits(d[0]), 0.f);   // +0 addend: a zero product gives +0
  s = fmaf(w[1], relu_bits(d[1]), s);
  s = fmaf(w[2], relu_bits(d[2]), s);
  s = fmaf(w[3], relu_bits(d[3]), s);
  return s;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

}  // namespace qsa
