// Stage 1: compressed index-key builder.
//
// [SGLang day-0 post on Qwen3.8-Flash-Next, section "Qwen Sparse Attention:
// Retrieve Coarsely, Attend Precisely"]: the 4 raw indexer keys of a block are
// averaged in FP32, normalised and turned by the rotary phase of the block's first
// token; the result is one bf16 key stored at the block's first slot / 4.  The raw
// keys of the unfinished block wait in a 4-slot ring per request.
//
// One wave per work group handles 4 blocks, 16 lanes per block; the key arithmetic
// (FP32 mean in token order, FP64 norm and rotation, bf16 rounding) is in
// qsa_keymath.h.  The inverse frequencies theta^(-2i/128) come from the host's libm.
//
// MRoPE [same section: a block's key is rotated by the multimodal rotary position of
// its first token, and the indexer shares the attention layers' MRoPE code]: with 3-D
// token positions (temporal, height, width), pair i turns by
// pos[axis(i)] * theta^(-2i/128), the per-pair axis map coming from the host.  The
// positions of the unfinished block's tokens wait in a position ring beside the key
// ring.
#include "qsa_device.h"
#include "qsa_keymath.h"
#include "qsa_launch.h"

#include <cmath>

namespace qsa {

namespace {

constexpr int kUnits = 4;   // blocks per work group

__global__ void __launch_bounds__(64)
build_kernel(const uint16_t* __restrict__ new_k, const int32_t* __restrict__ cu_new,
             const int32_t* __restrict__ len_before, const int32_t* __restrict__ page_table,
             int pt_stride, int page_size, uint16_t* __restrict__ ring,
             uint16_t* __restrict__ comp, const int32_t* __restrict__ new_mpos,
             int32_t* __restrict__ ring_mpos, RopeTable rope) {
  const int b = blockIdx.y;
  const int off = cu_new[b];
  const int n = cu_new[b + 1] - off;
  if (n <= 0) return;
  const int lb = len_before[b];
  const int le = lb + n;
  const int c0 = lb / kBlock;
  const int unit = threadIdx.x >> 4;
  const int j = threadIdx.x & 15;
  const int c = c0 + blockIdx.x * kUnits + unit;
  const bool complete = (kBlock * c + kBlock - 1) < le;
  const int bpp = page_size / kBlock;   // compressed rows per page
  int64_t row = 0;
  QSA_CHECK(lb >= 0 && (le - 1) / page_size < pt_stride);
  if (complete) {
    QSA_CHECK(page_table[(size_t)b * pt_stride + c / bpp] >= 0);
    row = (int64_t)page_table[(size_t)b * pt_stride + c / bpp] * bpp + (c % bpp);
  }

  // read phase: FP32 mean in token order
  float m[8];
  if (complete) {
    const uint16_t* src[kBlock];
#pragma unroll
    for (int tok = 0; tok < kBlock; ++tok) {
      const int t = kBlock * c + tok;
      src[tok] = (t < lb) ? ring + ((size_t)b * kBlock + (t & 3)) * kIdxDim
                          : new_k + (size_t)(off + t - lb) * kIdxDim;
    }
    key_block_mean(src, j, m);
  }
  // 3-D position of the block's first token (slot 0 of the ring when it is older
  // than this call)
  int p3[3] = {0, 0, 0};
  if (complete && new_mpos) {
    const int t = kBlock * c;
    const int32_t* src = (t < lb) ? ring_mpos + (size_t)b * kBlock * 3 : new_mpos + (size_t)(off + t - lb) * 3;
#pragma unroll
    for (int k = 0; k < 3; ++k) p3[k] = src[k];
  }
  // Every ring read of this launch happens above, in work group 0 (only block
  // c0 can hold tokens older than this call).  Work group 0 writes the ring
  // only after its reads.
  __syncthreads();
  if (blockIdx.x == 0 && (le % kBlock) != 0) {
    const int first = max(kBlock * (le / kBlock), lb);
    for (int t = first; t < le; ++t) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(new_k + (size_t)(off + t - lb) * kIdxDim);
      uint32_t* dst = reinterpret_cast<uint32_t*>(ring + ((size_t)b * kBlock + (t & 3)) * kIdxDim);
      dst[threadIdx.x] = src[threadIdx.x];   // 64 lanes x 2 bf16 = 128 dims
      if (new_mpos && threadIdx.x < 3)
        ring_mpos[((size_t)b * kBlock + (t & 3)) * 3 + threadIdx.x] =
            new_mpos[(size_t)(off + t - lb) * 3 + threadIdx.x];
    }
  }
  if (!complete) return;

  double ppos[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    ppos[e] = new_mpos ? (double)p3[rope.axis[4 * j + e]] : (double)(kBlock * c);
  u32x2_t lo, hi;
  key_rotate(m, ppos, rope.inv_freq, j, lo, hi);
  uint16_t* dst = comp + row * kIdxDim;
  *reinterpret_cast<u32x2_t*>(dst + 4 * j) = lo;
  *reinterpret_cast<u32x2_t*>(dst + 64 + 4 * j) = hi;
}

}  // namespace

hipError_t launch_build(const BuildArgs& a, hipStream_t stream) {
  RopeTable rope;
  for (int i = 0; i < kIdxDim / 2; ++i) {
    rope.inv_freq[i] = std::pow((double)a.theta, -(2.0 * i) / (double)kIdxDim);
    rope.axis[i] = a.pair_axis ? a.pair_axis[i] : 0;
  }
  // blocks touched by n new tokens starting anywhere: at most n/4 + 2
  const int units = a.max_new / kBlock + 2;
  dim3 grid((units + kUnits - 1) / kUnits, a.batch);
  QSA_LAUNCH(build_kernel, grid, dim3(64), 0, stream, a.new_k, a.cu_new, a.len_before,
                     a.page_table, a.pt_stride, a.page_size, a.ring, a.comp, a.new_mpos,
                     a.ring_mpos, rope);
  return hipGetLastError();
}

}  // namespace qsa
