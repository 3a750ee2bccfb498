// Arithmetic of one compressed index key, on the 16 lanes of a row.
//
// [SGLang day-0 post on Qwen3.8-Flash-Next, section "Qwen Sparse Attention:
// Retrieve Coarsely, Attend Precisely"]: a block's 4 raw indexer keys are averaged
// in FP32, the mean is normalised and turned by the rotary phase of the block's
// first token, and the result is kept in bf16.
//
// Lane j (0..15) of a row owns rotary pairs i = 4j .. 4j+3, i.e. dims 4j..4j+3 and
// 64+4j..64+4j+3, so every rotation is lane local.  The mean is taken in FP32 in
// token order; the norm, the rotation and the rounding are done in FP64, which
// keeps the phase exact to well below a bf16 step even at position 262140 (an FP32
// angle would be off by up to ~0.016 rad there).  The angle is reduced to
// [-pi, pi] with a two-constant Cody-Waite step before sincos.
//
// The builder and the decode scorer that ingests a step's token itself both use
// these functions, so they produce the same bits.
#pragma once

#include "qsa_device.h"

namespace qsa {

constexpr double kTwoPiHi = 6.283185307179586;          // 2*pi rounded to double
constexpr double kTwoPiLo = 2.4492935982947064e-16;     // 2*pi - kTwoPiHi
constexpr double kInvTwoPi = 0.15915494309189535;

// FP32 mean of the block's 4 raw keys (src[tok] = token tok's 128 bf16 dims, 8-byte
// aligned): m[0..3] = dims 4j..4j+3, m[4..7] = dims 64+4j..64+4j+3.  The sum runs in
// token order, then is scaled by 1/4.
__device__ __forceinline__ void key_block_mean(const uint16_t* const (&src)[kBlock], int j,
                                               float (&m)[8]) {
#pragma unroll
  for (int tok = 0; tok < kBlock; ++tok) {
    const u32x2_t a = *reinterpret_cast<const u32x2_t*>(src[tok] + 4 * j);
    const u32x2_t bb = *reinterpret_cast<const u32x2_t*>(src[tok] + 64 + 4 * j);
    const float v[8] = {bf16lo(a.x), bf16hi(a.x), bf16lo(a.y), bf16hi(a.y),
                        bf16lo(bb.x), bf16hi(bb.x), bf16lo(bb.y), bf16hi(bb.y)};
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = (tok == 0) ? v[e] : (m[e] + v[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] = m[e] * 0.25f;
}

// Normalise the mean over the 16 lanes of the row (FP64), turn pair 4j+e by the
// angle ppos[e] * inv_freq[4j+e], round to bf16 (nearest even).  lo packs dims
// 4j..4j+3, hi dims 64+4j..64+4j+3, ready to store at the key's row.
__device__ __forceinline__ void key_rotate(const float (&m)[8], const double (&ppos)[4],
                                           const double* inv_freq, int j, u32x2_t& lo,
                                           u32x2_t& hi) {
  double md[8];
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    md[e] = (double)m[e];
    ss += md[e] * md[e];
  }
#pragma unroll
  for (int sh = 1; sh < 16; sh <<= 1) ss += __shfl_xor(ss, sh, 64);
  const double nrm = fmax(sqrt(ss), 1e-12);

  uint32_t outw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double x = ppos[e] * inv_freq[4 * j + e];
    const double k = rint(x * kInvTwoPi);
    double red = fma(-k, kTwoPiHi, x);
    red = fma(-k, kTwoPiLo, red);
    double s, co;
    sincos(red, &s, &co);
    const double a = md[e] / nrm;
    const double bv = md[4 + e] / nrm;
    const double y0 = a * co - bv * s;
    const double y1 = bv * co + a * s;
    outw[e] = f64_to_bf16(y0) | (f64_to_bf16(y1) << 16);
  }
  // outw[e] packs (dim 4j+e, dim 64+4j+e)
  lo.x = (outw[0] & 0xffffu) | (outw[1] << 16);
  lo.y = (outw[2] & 0xffffu) | (outw[3] << 16);
  hi.x = (outw[0] >> 16) | (outw[1] & 0xffff0000u);
  hi.y = (outw[2] >> 16) | (outw[3] & 0xffff0000u);
}

}  // namespace qsa
