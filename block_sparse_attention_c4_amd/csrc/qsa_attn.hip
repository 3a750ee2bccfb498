// Stage 3: sparse GQA over the selected positions, read from the raw paged K/V.
//
// [SGLang day-0 post on Qwen3.8-Flash-Next, section "Qwen Sparse Attention:
// Retrieve Coarsely, Attend Precisely"]: attention weights and the weighted sum
// of values are computed from the full-resolution K/V rows of the selected logical
// positions, not from the compressed keys.
// [Same post, section "IndexShare MTP: Reusing the QSA Selection Across Draft
// Steps"]: a draft step attends to the captured selection plus the positions
// drafted since, passed here as extra positions.
//
// Work: one work group (4 waves) per (query, KV head, split of the position
// list).  A wave takes 32 positions per step, gathering K and V rows straight
// through the page table (a block's 4 positions are 4 adjacent slots).  Both
// products run on MFMA v_mfma_f32_16x16x32_bf16 with the 8 query heads of the
// KV group in the 16-wide N dimension:
//    S^T[pos, head] = K[pos, :] . Q^T[:, head]       (A = K rows, B = Q^T)
//    O^T[dim, head] += V^T[dim, pos] . P^T[pos, head] (A = V^T, B = P^T)
// The S^T accumulator layout (lane = head column, 4 positions per lane) is
// exactly the B operand layout of the second product, so P never leaves the
// lane.  V^T fragments come from each lane loading 16 B (8 dims) of its 8
// positions and transposing the 8x8 bf16 tile in registers (v_perm_b32).
// Softmax is online (running max and sum per head, log2 domain).  The 4 waves
// merge through LDS; with several splits, a combine kernel merges the split
// partials.
//
// FP8 K/V [ailone.io model page on Qwen3.8-Flash-Next, comparison of vLLM builds:
// a K/V cache in FP8]: the pools hold OCP E4M3 codes with one scale per pool.  The
// rows are loaded as codes (half the bytes and registers) and turned into bf16
// fragments just before use by v_cvt_scalef32_pk_bf16_fp8 with scale 1, which is
// exact (every E4M3 value is a bf16 value).  k_scale is folded into the softmax
// scale and v_scale into the output.  The K dims are permuted so that a lane reads
// 16 contiguous bytes per row; the query fragments follow the same permutation.
#include "qsa_device.h"
#include "qsa_launch.h"

#include <atomic>

namespace qsa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kChunk = 32;                      // positions per wave step
constexpr int kPartFloats = 2 * kGroup + kGroup * kHeadDim;   // m[8], l[8], acc[8][256]
constexpr int kAccPad = kHeadDim + 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Registers of one 32-position step: K rows of the two 16-position tiles and the
// lane's 8 V rows (both 128-dim halves), plus which of those V rows are real.
struct KV {
  u32x4_t k0[8], k1[8];
  u32x4_t v[2][8];
  uint32_t okmask;
};

// The same step as FP8 codes: K fragment pairs (16 codes = 2 fragments) and V rows
// of 8 codes.
struct KV8 {
  u32x4_t k0[4], k1[4];
  u32x2_t v[2][8];
  uint32_t okmask;
};

template <bool kFp8> struct KVRegs { typedef KV type; };
template <> struct KVRegs<true> { typedef KV8 type; };

// Dims held by lane (r, j) in query/key fragment kc.  bf16: 32 kc + 8 j + (0..7).
// FP8: 64 (kc/2) + 16 j + 8 (kc%2) + (0..7), so fragments 2kk and 2kk+1 of a row are
// 16 contiguous codes.
template <bool kFp8>
__device__ __forceinline__ int frag_dim(int kc, int j) {
  return kFp8 ? 64 * (kc >> 1) + 16 * j + 8 * (kc & 1) : 32 * kc + 8 * j;
}

// ok bit e: V row e of the lane is a real position; slot -1 = no position, whose
// loads read slot 0 and are discarded
__device__ __forceinline__ void step_slots(const int32_t* s_slot, int cb, int end_local, int r,
                                           int j, int& s0, int& s1, int (&sv)[8],
                                           uint32_t& ok) {
  const int li0 = cb + r, li1 = cb + 16 + r;
  s0 = li0 < end_local ? s_slot[li0] : -1;
  s1 = li1 < end_local ? s_slot[li1] : -1;
  ok = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int li = cb + (e < 4 ? 0 : 16) + 4 * j + (e & 3);
    sv[e] = li < end_local ? s_slot[li] : -1;
    ok |= (sv[e] >= 0 ? 1u : 0u) << e;
  }
}

__device__ __forceinline__ void load_kv(KV& x, const int32_t* s_slot, int cb, int end_local,
                                        const void* k_pool_v, const void* v_pool_v, int g, int r,
                                        int j) {
  const uint16_t* __restrict__ k_pool = static_cast<const uint16_t*>(k_pool_v);
  const uint16_t* __restrict__ v_pool = static_cast<const uint16_t*>(v_pool_v);
  int s0, s1, sv[8];
  step_slots(s_slot, cb, end_local, r, j, s0, s1, sv, x.okmask);
  const uint16_t* k0 = k_pool + ((size_t)max(s0, 0) * kKVHeads + g) * kHeadDim;
  const uint16_t* k1 = k_pool + ((size_t)max(s1, 0) * kKVHeads + g) * kHeadDim;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    x.k0[k] = ld16(k0 + frag_dim<false>(k, j));
    x.k1[k] = ld16(k1 + frag_dim<false>(k, j));
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint16_t* vp = v_pool + ((size_t)max(sv[e], 0) * kKVHeads + g) * kHeadDim + 8 * r;
    x.v[0][e] = ld16(vp);
    x.v[1][e] = ld16(vp + 128);
  }
}

__device__ __forceinline__ void load_kv(KV8& x, const int32_t* s_slot, int cb, int end_local,
                                        const void* k_pool_v, const void* v_pool_v, int g, int r,
                                        int j) {
  const uint8_t* __restrict__ k_pool = static_cast<const uint8_t*>(k_pool_v);
  const uint8_t* __restrict__ v_pool = static_cast<const uint8_t*>(v_pool_v);
  int s0, s1, sv[8];
  step_slots(s_slot, cb, end_local, r, j, s0, s1, sv, x.okmask);
  const uint8_t* k0 = k_pool + ((size_t)max(s0, 0) * kKVHeads + g) * kHeadDim;
  const uint8_t* k1 = k_pool + ((size_t)max(s1, 0) * kKVHeads + g) * kHeadDim;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    x.k0[kk] = ld16(k0 + frag_dim<true>(2 * kk, j));
    x.k1[kk] = ld16(k1 + frag_dim<true>(2 * kk, j));
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint8_t* vp = v_pool + ((size_t)max(sv[e], 0) * kKVHeads + g) * kHeadDim + 8 * r;
    x.v[0][e] = *reinterpret_cast<const u32x2_t*>(vp);
    x.v[1][e] = *reinterpret_cast<const u32x2_t*>(vp + 128);
  }
}

// 4 E4M3 codes -> 4 bf16 (2 dwords), exact.
__device__ __forceinline__ u32x2_t fp8x4_to_bf16(uint32_t w) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return u32x2_t{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

__device__ __forceinline__ u32x4_t fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const u32x2_t a = fp8x4_to_bf16(w0), b = fp8x4_to_bf16(w1);
  return u32x4_t{a.x, a.y, b.x, b.y};
}

// bf16 fragments of a step, for either register layout: K fragment k of tile 0/1,
// V row e of half gm.  FP8 codes are converted where they are used.
__device__ __forceinline__ u32x4_t kfrag(const KV& x, int tile, int k) {
  return tile ? x.k1[k] : x.k0[k];
}
__device__ __forceinline__ u32x4_t kfrag(const KV8& x, int tile, int k) {
  const u32x4_t c = tile ? x.k1[k >> 1] : x.k0[k >> 1];
  return (k & 1) ? fp8x8_to_bf16(c.z, c.w) : fp8x8_to_bf16(c.x, c.y);
}
__device__ __forceinline__ u32x4_t vrow(const KV& x, int gm, int e) { return x.v[gm][e]; }
__device__ __forceinline__ u32x4_t vrow(const KV8& x, int gm, int e) {
  return fp8x8_to_bf16(x.v[gm][e].x, x.v[gm][e].y);
}

struct SoftmaxState {
  float m, l;
  f32x4_t acc[2][8];
};

template <class KVR>
__device__ __forceinline__ void attend_step(SoftmaxState& st, const KVR& x, const u32x4_t (&qf)[8],
                                            float scale_log2) {
  f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    s0 = mfma16(kfrag(x, 0, k), qf[k], s0);
    s1 = mfma16(kfrag(x, 1, k), qf[k], s1);
  }
  float xs[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xs[i] = (x.okmask >> i) & 1u ? s0[i] * scale_log2 : -INFINITY;
    xs[4 + i] = (x.okmask >> (4 + i)) & 1u ? s1[i] * scale_log2 : -INFINITY;
  }
  float mx = xs[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) mx = fmaxf(mx, xs[e]);
  mx = fmaxf(mx, lane_xor16(mx));
  mx = fmaxf(mx, lane_xor32(mx));
  const float m_new = fmaxf(st.m, mx);
  float pr[8];
  float alpha = 1.f;
  if (m_new == -INFINITY) {
#pragma unroll
    for (int e = 0; e < 8; ++e) pr[e] = 0.f;
  } else {
    alpha = exp2f(st.m - m_new);   // m = -inf gives 0
#pragma unroll
    for (int e = 0; e < 8; ++e) pr[e] = exp2f(xs[e] - m_new);
  }
  float rs = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) rs += pr[e];
  rs += lane_xor16(rs);
  rs += lane_xor32(rs);
  st.l = st.l * alpha + rs;
  st.m = m_new;
  // rows of V that are not real positions are zeroed (their weight is 0, and the
  // pool may hold anything there)
  const u32x4_t pf = {pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                      pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
#pragma unroll
  for (int gm = 0; gm < 2; ++gm) {
    u32x4_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool ok = (x.okmask >> e) & 1u;
      v[e] = ok ? vrow(x, gm, e) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int tau = 0; tau < 8; ++tau) {
      const uint32_t sel = (tau & 1) ? 0x07060302u : 0x05040100u;
      const int dw = tau >> 1;
      u32x4_t a;
      a.x = __builtin_amdgcn_perm(v[1][dw], v[0][dw], sel);
      a.y = __builtin_amdgcn_perm(v[3][dw], v[2][dw], sel);
      a.z = __builtin_amdgcn_perm(v[5][dw], v[4][dw], sel);
      a.w = __builtin_amdgcn_perm(v[7][dw], v[6][dw], sel);
      const f32x4_t c = st.acc[gm][tau] * alpha;
      st.acc[gm][tau] = mfma16(a, pf, c);
    }
  }
}

constexpr int kMaxSplitLen = 2176;   // >= kMaxSel + QSA_MAX_EXTRA, a multiple of 128
constexpr int kSlotsPer = (kMaxSplitLen + kThreads - 1) / kThreads;   // list entries per thread

template <bool kFp8, int kDepth>
__global__ void __launch_bounds__(kThreads)
attn_kernel(const uint16_t* __restrict__ q, const int32_t* __restrict__ q_req,
            const void* __restrict__ k_pool, const void* __restrict__ v_pool,
            const int32_t* __restrict__ page_table, int pt_stride, int page_size,
            const int32_t* __restrict__ sel_pos, const int32_t* __restrict__ sel_count,
            int sel_stride, const int32_t* __restrict__ extra_pos, int n_extra, float scale_log2,
            float v_scale, int splits, float* __restrict__ part, uint16_t* __restrict__ out,
            float* __restrict__ lse) {
  typedef typename KVRegs<kFp8>::type KVR;
  __shared__ float s_m[kWaves][kGroup];
  __shared__ float s_l[kWaves][kGroup];
  __shared__ float s_acc[kWaves][kGroup][kAccPad];
  __shared__ int32_t s_slot[kMaxSplitLen];

  const int bid = blockIdx.x;
  const int sp = bid % splits;
  const int tg = bid / splits;
  const int g = tg % kKVHeads;
  const int t = tg / kKVHeads;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 15;
  const int j = lane >> 4;

  // Q^T operand: head r of the group (zero for the 8 padding columns)
  u32x4_t qf[8];
  {
    const uint16_t* qrow = q + ((size_t)t * kQHeads + g * kGroup + (r & 7)) * kHeadDim;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      qf[k] = (r < kGroup) ? ld16(qrow + frag_dim<kFp8>(k, j)) : u32x4_t{0u, 0u, 0u, 0u};
  }

  // This split's share of the position list: the list's bound (2051 + extras)
  // in 32-position chunks, dealt out evenly, so that every work group streams
  // about the same bytes.
  const int bound = kMaxSel + n_extra;
  const int nchunk = (bound + kChunk - 1) / kChunk;
  const int start = (sp * nchunk / splits) * kChunk;
  const int span = min(((sp + 1) * nchunk / splits) * kChunk, bound) - start;
  const int req = q_req ? q_req[t] : t;
  const int cnt = sel_count[t];
  QSA_CHECK(cnt >= 0 && cnt <= sel_stride && cnt <= kMaxSel);   // the splits cover kMaxSel + n_extra
  const int total = cnt + n_extra;
  const int len = max(0, min(span, total - start));
  // Translate the positions to pool slots (-1 = no position).  All list loads
  // go out before the count is needed, and all page-table loads go out
  // together, so the translation costs two memory round trips.
  {
    const int32_t* pt_row = page_table + (size_t)req * pt_stride;
    const int32_t* lst = sel_pos + (size_t)t * sel_stride;
    int p[kSlotsPer];
#pragma unroll
    for (int u = 0; u < kSlotsPer; ++u) {
      const int i = tid + u * kThreads;
      p[u] = (i < span && start + i < sel_stride) ? lst[start + i] : -1;
    }
#pragma unroll
    for (int u = 0; u < kSlotsPer; ++u) {
      const int li = start + tid + u * kThreads;
      if (tid + u * kThreads >= len) p[u] = -1;
      else if (li >= cnt) p[u] = extra_pos[(size_t)t * n_extra + (li - cnt)];
    }
    int pg[kSlotsPer];
#pragma unroll
    for (int u = 0; u < kSlotsPer; ++u) {
      QSA_CHECK(p[u] < pt_stride * page_size);
      pg[u] = p[u] >= 0 ? pt_row[p[u] / page_size] : 0;
      QSA_CHECK(pg[u] >= 0);
    }
#pragma unroll
    for (int u = 0; u < kSlotsPer; ++u) {
      const int i = tid + u * kThreads;
      if (i < span) s_slot[i] = p[u] >= 0 ? pg[u] * page_size + p[u] % page_size : -1;
    }
  }
  __syncthreads();

  SoftmaxState st;
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int gm = 0; gm < 2; ++gm)
#pragma unroll
    for (int tau = 0; tau < 8; ++tau) st.acc[gm][tau] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // this wave's 32-position steps: w, w + 4, ...; kDepth steps' loads in flight
  const int stride = kWaves * kChunk;
  const int cb0 = w * kChunk;
  if constexpr (kDepth == 1) {
    // A list that ends inside a chunk (the 0..3 tokens of the unfinished block, or
    // drafted positions) leaves a last chunk of a few rows.  Its wave would pay one
    // more full round trip for them, and its work group would finish last; so that
    // chunk is requested with the wave's first chunk and attended right after it.
    const int last = ((len + kChunk - 1) / kChunk - 1) * kChunk;
    const bool early_tail = (len % kChunk) != 0 && last >= stride && last % stride == cb0;
    KVR x, tail;
    if (early_tail) load_kv(tail, s_slot, last, len, k_pool, v_pool, g, r, j);
    const int end = early_tail ? last : len;
    for (int cb = cb0; cb < end; cb += stride) {
      load_kv(x, s_slot, cb, len, k_pool, v_pool, g, r, j);
      attend_step(st, x, qf, scale_log2);
      if (early_tail && cb == cb0) attend_step(st, tail, qf, scale_log2);
    }
  } else {
    KVR buf[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
      if (cb0 + d * stride < len) load_kv(buf[d], s_slot, cb0 + d * stride, len, k_pool, v_pool, g, r, j);
    for (int cb = cb0; cb < len; cb += kDepth * stride) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        const int c = cb + d * stride;
        if (c < len) {
          attend_step(st, buf[d], qf, scale_log2);
          if (c + kDepth * stride < len)
            load_kv(buf[d], s_slot, c + kDepth * stride, len, k_pool, v_pool, g, r, j);
        }
      }
    }
  }
  const float m_run = st.m, l_run = st.l;

  // merge the 4 waves.  Lane (r, j) holds head r, dims 128*gm + 32*j + 8*i + tau.
  if (r < kGroup) {
    if (j == 0) {
      s_m[w][r] = m_run;
      s_l[w][r] = l_run;
    }
#pragma unroll
    for (int gm = 0; gm < 2; ++gm)
#pragma unroll
      for (int tau = 0; tau < 8; ++tau)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_acc[w][r][128 * gm + 32 * j + 8 * i + tau] = st.acc[gm][tau][i];
  }
  __syncthreads();

  const int h = tid >> 5;              // 0..7
  const int d0 = (tid & 31) * 8;       // 8 dims per thread
  float M = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, s_m[ww][h]);
  float L = 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float mw = s_m[ww][h];
      const float sc = mw == -INFINITY ? 0.f : exp2f(mw - M);
      L += sc * s_l[ww][h];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += sc * s_acc[ww][h][d0 + e];
    }
  }

  if (splits == 1) {
    const float inv = L > 0.f ? (kFp8 ? v_scale : 1.f) / L : 0.f;
    uint16_t* orow = out + ((size_t)t * kQHeads + g * kGroup + h) * kHeadDim + d0;
    u32x4_t ov = {pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
                  pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv)};
    *reinterpret_cast<u32x4_t*>(orow) = ov;
    if (lse && (tid & 31) == 0)
      lse[(size_t)t * kQHeads + g * kGroup + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  } else {
    float* pp = part + ((size_t)tg * splits + sp) * kPartFloats;
    if ((tid & 31) == 0) {
      pp[h] = M;
      pp[kGroup + h] = L;
    }
    float* pa = pp + 2 * kGroup + h * kHeadDim + d0;
    *reinterpret_cast<f32x4_t*>(pa) = f32x4_t{o[0], o[1], o[2], o[3]};
    *reinterpret_cast<f32x4_t*>(pa + 4) = f32x4_t{o[4], o[5], o[6], o[7]};
  }
}

// Merge the split partials of one (query, KV head): 256 threads, thread = (head, 8 dims).
// Every split's partial is requested before any is used (one memory round trip).
constexpr int kMaxCombine = 8;         // splits merged from registers; more loop over memory

__global__ void __launch_bounds__(256)
combine_kernel(const float* __restrict__ part, int splits, float v_scale, uint16_t* __restrict__ out,
               float* __restrict__ lse) {
  const int tg = blockIdx.x;
  const int g = tg % kKVHeads;
  const int t = tg / kKVHeads;
  const int tid = threadIdx.x;
  const int h = tid >> 5;
  const int d0 = (tid & 31) * 8;
  const float* base = part + (size_t)tg * splits * kPartFloats;
  float M = -INFINITY, L = 0.f;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += kMaxCombine) {
    const int ns = min(kMaxCombine, splits - s0);
    float ms[kMaxCombine], ls[kMaxCombine];
    f32x4_t a0[kMaxCombine], a1[kMaxCombine];
#pragma unroll
    for (int i = 0; i < kMaxCombine; ++i) {
      if (i < ns) {
        const float* pp = base + (size_t)(s0 + i) * kPartFloats;
        ms[i] = pp[h];
        ls[i] = pp[kGroup + h];
        a0[i] = *reinterpret_cast<const f32x4_t*>(pp + 2 * kGroup + h * kHeadDim + d0);
        a1[i] = *reinterpret_cast<const f32x4_t*>(pp + 2 * kGroup + h * kHeadDim + d0 + 4);
      }
    }
    // an empty split wrote l = 0 and zero accumulators: its weight is 0
    float Mn = M;
#pragma unroll
    for (int i = 0; i < kMaxCombine; ++i)
      if (i < ns && ls[i] > 0.f) Mn = fmaxf(Mn, ms[i]);
    if (Mn == -INFINITY) continue;
    const float rescale = M == -INFINITY ? 0.f : exp2f(M - Mn);
    L *= rescale;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= rescale;
#pragma unroll
    for (int i = 0; i < kMaxCombine; ++i) {
      if (i < ns && ls[i] > 0.f) {
        const float sc = exp2f(ms[i] - Mn);
        L += sc * ls[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] += sc * a0[i][e];
          o[4 + e] += sc * a1[i][e];
        }
      }
    }
    M = Mn;
  }
  const float inv = L > 0.f ? v_scale / L : 0.f;   // v_scale is 1 for bf16 pools
  uint16_t* orow = out + ((size_t)t * kQHeads + g * kGroup + h) * kHeadDim + d0;
  u32x4_t ov = {pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
                pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv)};
  *reinterpret_cast<u32x4_t*>(orow) = ov;
  if (lse && (tid & 31) == 0)
    lse[(size_t)t * kQHeads + g * kGroup + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

}  // namespace

void attn_plan(int total_q, int n_extra, int* splits, int* split_len) {
  const int nchunk = (kMaxSel + n_extra + kChunk - 1) / kChunk;   // 32-position chunks
  const int pairs = total_q * kKVHeads;
  int s = (256 + pairs - 1) / pairs;     // about one 4-wave work group per CU
  s = std::max(1, std::min(s, nchunk / kWaves));   // at least a chunk per wave
  *splits = s;
  *split_len = ((nchunk + s - 1) / s) * kChunk;   // the longest split
}

size_t attn_workspace_bytes(int total_q, int n_extra) {
  int splits, len;
  attn_plan(total_q, n_extra, &splits, &len);
  if (splits == 1) return 0;
  return (size_t)total_q * kKVHeads * splits * kPartFloats * sizeof(float);
}

// Scratch of the allocation-free decode call (qsa_sparse_gqa_decode_noalloc): the
// split partials live in this file-scope device array instead of a caller
// workspace.  Every GPU that runs the library holds its own copy until the process
// ends.  In host code `scratch` names only a host-side stand-in; its device address
// on the current GPU comes from hipGetSymbolAddress, taken once per device and kept
// in scratch_ptr[].  Calls that overlap on one GPU share (and race on) the array.
static __device__ __align__(256) float scratch[kAttnScratchBytes / sizeof(float)];

constexpr int kScratchDevices = 64;
static std::atomic<void*> scratch_ptr[kScratchDevices];

hipError_t attn_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
    scratch_ptr[dev].store(p, std::memory_order_release);   // racing threads store the same address
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  // FP8 codes stand for code * scale: k_scale goes into the logits' scale, v_scale
  // onto the normalised output
  const float scale_log2 = a.sm_scale * (a.fp8 ? a.k_scale : 1.f) * kLog2e;
  const float v_scale = a.fp8 ? a.v_scale : 1.f;
  const int nblk = a.total_q * kKVHeads * a.splits;
  // Steps in flight per wave.  Launches of at most one work group per CU (decode's
  // split lists; target verification's 128 queries) run fastest with one: more only
  // lengthens the gathers' queues in the memory system (decode FP8 22.0 / 22.5 /
  // 24.2 / 25.7 us and bf16 30.7 / 32.0 us for depth 1 / 2 / 3 / 4; verification
  // 92.2 against 94.4 us for depth 1 / 2).  Prefill chunks (many work groups per CU)
  // gain a little from two (2160 against 2198 us).
  const bool one_step = a.splits > 1 || nblk <= 256;
  auto kern = a.fp8 ? (one_step ? attn_kernel<true, 1> : attn_kernel<true, 2>)
                    : (one_step ? attn_kernel<false, 1> : attn_kernel<false, 2>);
  QSA_LAUNCH(kern, dim3(nblk), dim3(kThreads), 0, stream, a.q, a.q_req, a.k_pool,
                     a.v_pool, a.page_table, a.pt_stride, a.page_size, a.sel_pos, a.sel_count,
                     a.sel_stride, a.extra_pos, a.n_extra, scale_log2, v_scale, a.splits, a.part,
                     a.out, a.lse);
  if (a.splits > 1) {
    QSA_LAUNCH(combine_kernel, dim3(a.total_q * kKVHeads), dim3(256), 0, stream, a.part,
                       a.splits, v_scale, a.out, a.lse);
  }
  return hipGetLastError();
}

}  // namespace qsa
