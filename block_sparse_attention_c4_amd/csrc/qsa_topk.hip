// Stage 2b: top-512 block selection and expansion to token positions.
//
// [SGLang day-0 post on Qwen3.8-Flash-Next, section "Qwen Sparse Attention:
// Retrieve Coarsely, Attend Precisely"]: the best 512 blocks are kept, expanded to
// their 2048 token positions, and the 0..3 tokens of the unfinished block are
// appended.  Ties go to the lower block index; kept blocks are listed ascending.
//
// Two selects, both on an order-preserving 32-bit key of each FP32 score and one
// 1024-thread work group per query row:
//   - topk_kernel (decode, verification, the indexer's general path): the
//     latency-bound select described before it below.  It starts from the scorer's
//     16-block group maxima and reads only the candidate groups of a long row.
//   - topk_row, used by topk_queued_kernel for the rows that the code-based prefill
//     select of qsa_prefill.hip hands over (heavy ties): every score of the row is read
//     once, as float4 quads kept in registers (at most 16 quads per thread for 65536
//     blocks).
//      1. n <= 512: every block is kept.
//      2. Lower bound: the 512th largest quad maximum t0 (found to 16 bits below the
//         keys' common prefix, rounded down) has at least 512 quads, hence 512 scores,
//         at or above it.  (Skipped when n <= 4096: t0 = 0.)
//      3. Scores >= t0 go to LDS as candidates (a block-wide prefix count gives their
//         slots); typically a thousand or fewer.
//      4. Exact radix select over the candidates: the threshold key and how many keys
//         equal to it are kept (ties go to the lowest block indices).
//      5. Kept blocks are marked in an LDS bitmap and written in index order from a
//         per-word prefix count.
//     Radix passes use 8-bit digits that start at the first bit where the keys' max
//     and min differ; one wave scans the 256-bin histogram while the other waves
//     clear the next one.  More than kCap candidates falls back to a select over the
//     score row in global memory.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

namespace {

constexpr int kT = 1024;               // threads per work group
constexpr int kW = kT / 64;
constexpr int kCap = 4096;             // LDS candidates
constexpr int kWords = kMaxBlocks / 32;   // 2048 bitmap words, 2 per thread
constexpr int kRankCap = 256;          // keys ranked directly after the first select pass

struct __attribute__((aligned(16))) Smem {
  uint32_t red[2 * kW];
  int wsum[kW];
  uint32_t hist[2][256];
  uint32_t key[kCap];
  uint16_t idx[kCap];
  uint32_t bits[kWords];
  uint32_t eqbits[kWords];
  uint16_t wpre[kWords];               // kept bits in the words before each word
  uint32_t rank_key[kRankCap];
  int misc[8];
};

__shared__ Smem sm;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Exclusive scan of one int per thread; .x = prefix, .y = total.
__device__ __forceinline__ int2 block_scan(int v) {
  const int w = threadIdx.x >> 6;
  const int inc = wave_inclusive_sum(v);
  if (lane_id() == 63) sm.wsum[w] = inc;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kW / 4; ++i) {
    const int4 x = reinterpret_cast<const int4*>(sm.wsum)[i];
    const int xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      before += 4 * i + j < w ? xs[j] : 0;
      all += xs[j];
    }
  }
  __syncthreads();
  return make_int2(before + inc - v, all);
}

// One radix-select pass over a histogram that has been filled: wave 0 finds the
// bin of the kk-th largest (lane l owns bins 4l..4l+3, read as one 16-byte load),
// the other waves clear the other histogram.
__device__ __forceinline__ void radix_find(int buf, int kk) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    const uint4 h = reinterpret_cast<const uint4*>(sm.hist[buf])[tid];
    const int mine = (int)(h.x + h.y + h.z + h.w);
    const int inc = wave_inclusive_sum(mine);
    const int above = __builtin_amdgcn_readlane(inc, 63) - inc;   // keys in higher lanes' bins
    if (above < kk && kk <= above + mine) {
      const int a3 = above + (int)h.w;
      const int a2 = a3 + (int)h.z;
      const int a1 = a2 + (int)h.y;
      int d, r;
      if (kk <= a3) { d = 3; r = kk - above; }
      else if (kk <= a2) { d = 2; r = kk - a3; }
      else if (kk <= a1) { d = 1; r = kk - a2; }
      else { d = 0; r = kk - a1; }
      sm.misc[0] = 4 * tid + d;
      sm.misc[1] = r;
    }
  } else if (tid < 64 + 256) {
    sm.hist[buf ^ 1][tid - 64] = 0u;
  }
}

// Count one key into the histogram.
__device__ __forceinline__ void hist_add(uint32_t* hist, bool ok, uint32_t d) {
  if (ok) atomicAdd(&hist[d], 1u);
}

__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// k-th largest among the register-held keys (0 = empty).  Returns (key, number of
// keys equal to it that are kept).  With lower_bound, returns instead a key that at
// least k keys reach (the lower edge of the first pass's bin).
//
// Pass 1 bins the values linearly over [min, max] (256 bins), which spreads any
// score distribution over the histogram (bins of the key's high bits would pile
// the bulk of the scores into a few exponent bins and serialize the LDS atomics).
// The keys in the chosen bin lie between conservative key bounds one bin wider on
// each side; the exact key is then found by 8-bit radix passes over key - (lower
// bound) among them.
template <int E>
__device__ __forceinline__ uint2 select_keys(const uint32_t (&key)[E], int kk, bool lower_bound) {
  const int tid = threadIdx.x, w = tid >> 6;
  uint32_t mx = 0u, mn = 0xffffffffu;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    mx = max(mx, key[e]);
    mn = min(mn, key[e] ? key[e] : 0xffffffffu);
  }
  mx = wave_max_u32(mx);
  mn = wave_min_u32(mn);
  if (lane_id() == 0) {
    sm.red[w] = mx;
    sm.red[kW + w] = mn;
  }
  if (tid < 256) sm.hist[0][tid] = 0u;
  if (tid == 0) sm.misc[4] = 0;        // keys gathered for ranking
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kW / 4; ++i) {
    const uint4 a = reinterpret_cast<const uint4*>(sm.red)[i];
    const uint4 b = reinterpret_cast<const uint4*>(sm.red + kW)[i];
    mx = max(max(mx, max(a.x, a.y)), max(a.z, a.w));
    mn = min(min(mn, min(b.x, b.y)), min(b.z, b.w));
  }
  if (mx == mn) return make_uint2(mx, (uint32_t)kk);   // all equal: every kept key ties

  // pass 1: linear bins of the value
  const float fmn = key_float(mn), fmx = key_float(mx);
  const float scale = 256.f / (fmx - fmn);
  uint32_t lo_key = mn, hi_key = mx;
  int bin = -1;                        // keys in play: bin == -1 (all) or linear bin == bin
  int buf = 0;
  if (scale > 0.f && scale < 3.0e38f && fmx - fmn < 3.0e38f) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int d = min(255, (int)((key_float(key[e]) - fmn) * scale));
      hist_add(sm.hist[0], key[e] != 0u, (uint32_t)d);
    }
    __syncthreads();
    radix_find(0, kk);
    __syncthreads();
    bin = sm.misc[0];
    kk = sm.misc[1];
    buf = 1;
    if (bin > 0) lo_key = max(mn, float_key(fmn + (float)(bin - 1) / scale));
    if (bin < 255) hi_key = min(mx, float_key(fmn + (float)(bin + 2) / scale));
    if (lower_bound) return make_uint2(lo_key, 0u);
    // Few keys in the chosen bin (the usual case): gather them and rank each against
    // the others, instead of radix passes with two barriers each.
    const int m = (int)sm.hist[0][bin];
    if (m <= kRankCap) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const uint32_t k = key[e];
        if (k != 0u && min(255, (int)((key_float(k) - fmn) * scale)) == bin)
          sm.rank_key[atomicAdd(&sm.misc[4], 1)] = k;
      }
      __syncthreads();
      for (int i = tid; i < m; i += kT) {
        const uint32_t ki = sm.rank_key[i];
        int gt = 0, ge = 0;
        for (int j = 0; j < m; ++j) {
          const uint32_t kj = sm.rank_key[j];
          gt += kj > ki ? 1 : 0;
          ge += kj >= ki ? 1 : 0;
        }
        if (gt < kk && kk <= ge) {     // ki is the kk-th largest of the bin
          sm.misc[5] = (int)ki;
          sm.misc[6] = kk - gt;
        }
      }
      __syncthreads();
      return make_uint2((uint32_t)sm.misc[5], (uint32_t)sm.misc[6]);
    }
  }
  // radix passes over r = key - lo_key among the keys in play
  const uint32_t range = hi_key - lo_key;
  int hi = range ? 31 - __clz(range) : -1;
  uint32_t prefix = 0u;
  while (hi >= 0) {
    const int lo = max(hi - 7, 0);
    const uint32_t pmask = hi == 31 ? 0u : ~((2u << hi) - 1u);
    const uint32_t dmask = (1u << (hi - lo + 1)) - 1u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t k = key[e];
      bool ok = k != 0u;
      if (bin >= 0) ok = ok && min(255, (int)((key_float(k) - fmn) * scale)) == bin;
      const uint32_t r = k - lo_key;
      hist_add(sm.hist[buf], ok && (r & pmask) == prefix, (r >> lo) & dmask);
    }
    __syncthreads();
    radix_find(buf, kk);
    __syncthreads();
    prefix |= (uint32_t)sm.misc[0] << lo;
    kk = sm.misc[1];
    buf ^= 1;
    hi = lo - 1;
    if (lower_bound) break;
  }
  return make_uint2(lo_key + prefix, (uint32_t)kk);
}

// Slow path for heavy ties: exact k-th largest over the score row in global memory.
__device__ uint2 select_row(const float* srow, int n, int kk) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t pmask = pass == 0 ? 0u : (0xffffffffu << (shift + 8));
    if (tid < 256) sm.hist[0][tid] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += kT) {
      const uint32_t key = float_key(srow[i]);
      if ((key & pmask) == prefix) atomicAdd(&sm.hist[0][(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    radix_find(0, kk);
    __syncthreads();
    prefix |= (uint32_t)sm.misc[0] << shift;
    kk = sm.misc[1];
  }
  return make_uint2(prefix, (uint32_t)kk);
}

// Quads q = tid + kT*e of the row (coalesced: a wave reads 1 KB per load).  kHold
// keeps their keys in registers (up to 8 quads per thread); otherwise only the
// maxima are kept and the row is read again (from L2) for the count and the write.
// The lower bound ranks the maxima of single quads when n <= 8192, else of 16-block
// groups, whose 4 quads sit in 4 adjacent lanes.
template <int E, bool kHold>
__device__ __forceinline__ void topk_quads(const float* srow, int n) {
  const int tid = threadIdx.x;
  const int nq = (n + 3) / 4;
  auto quad_keys = [&](int e, uint32_t (&k)[4]) {
    const int q = tid + kT * e;
    const f32x4_t v = q < nq ? *reinterpret_cast<const f32x4_t*>(srow + 4 * q)
                             : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) k[i] = (4 * q + i < n) ? float_key(v[i]) : 0u;   // 0: past n
  };
  uint32_t k4[kHold ? E : 1][4];
  uint32_t qm[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    uint32_t k[4];
    quad_keys(e, k);
    qm[e] = max(max(k[0], k[1]), max(k[2], k[3]));
    if (kHold)
#pragma unroll
      for (int i = 0; i < 4; ++i) k4[kHold ? e : 0][i] = k[i];
  }
  uint32_t t0 = 1u;                    // any score qualifies when n <= 4096
  if (n > 8192) {
    uint32_t gm[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      uint32_t m = max(qm[e], (uint32_t)dpp_i<0xb1, 0xf>((int)qm[e]));   // quad_perm [1,0,3,2]
      m = max(m, (uint32_t)dpp_i<0x4e, 0xf>((int)m));                   // quad_perm [2,3,0,1]
      gm[e] = (tid & 3) == 0 ? m : 0u;
    }
    t0 = max(select_keys<E>(gm, kTopK, true).x, 1u);
  } else if (n > 4096) {
    t0 = max(select_keys<E>(qm, kTopK, true).x, 1u);
  }

  int cnt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (qm[e] < t0) continue;
    uint32_t k[4];
    if (kHold) {
#pragma unroll
      for (int i = 0; i < 4; ++i) k[i] = k4[kHold ? e : 0][i];
    } else {
      quad_keys(e, k);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) cnt += k[i] >= t0 ? 1 : 0;
  }
  const int2 sc = block_scan(cnt);
  int off = sc.x;
  if (sc.y <= kCap) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (qm[e] < t0) continue;
      uint32_t k[4];
      if (kHold) {
#pragma unroll
        for (int i = 0; i < 4; ++i) k[i] = k4[kHold ? e : 0][i];
      } else {
        quad_keys(e, k);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (k[i] >= t0) {
          sm.key[off] = k[i];
          sm.idx[off] = (uint16_t)(4 * (tid + kT * e) + i);
          ++off;
        }
    }
  }
  if (tid == 0) sm.misc[2] = sc.y;
  __syncthreads();
}

// Candidates from the scorer's 16-block group maxima (EG per thread): the 512th
// largest maximum (found to a lower bound) has at least 512 groups, hence 512
// scores, at or above it, so only the groups whose maximum reaches it are read.
// Candidates take LDS slots (a wave prefix sum, one atomic per wave); misc[2] =
// their count.
template <int EG>
__device__ __forceinline__ void topk_groups(const float* srow, const float* grow, int n) {
  const int tid = threadIdx.x;
  const int ng = (n + kScoreGroup - 1) / kScoreGroup;
  uint32_t gk[EG];
#pragma unroll
  for (int e = 0; e < EG; ++e) {
    const int g = tid + kT * e;
    gk[e] = g < ng ? float_key(grow[g]) : 0u;
  }
  if (tid == 0) sm.misc[2] = 0;
  const uint32_t t0 = max(select_keys<EG>(gk, kTopK, true).x, 1u);   // (its barriers order misc[2])
  // one pass per e, wave-uniform: a lane reads its group only if it is a candidate;
  // slots come from a wave prefix sum and one LDS atomic per wave
  f32x4_t vals[EG][4];                 // every pass's loads are issued before any is used
#pragma unroll
  for (int e = 0; e < EG; ++e) {
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(srow + kScoreGroup * (tid + kT * e));
#pragma unroll
    for (int q = 0; q < 4; ++q) vals[e][q] = gk[e] >= t0 ? src[q] : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int e = 0; e < EG; ++e) {
    const int g = tid + kT * e;
    const bool cand = gk[e] >= t0;
    uint32_t k[16];
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4_t v = vals[e][q];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = kScoreGroup * g + 4 * q + i;
        const uint32_t key = float_key(v[i]);
        k[4 * q + i] = (cand && c < n && key >= t0) ? key : 0u;
        cnt += k[4 * q + i] ? 1 : 0;
      }
    }
    const int incl = wave_inclusive_sum(cnt);
    const int wtot = __builtin_amdgcn_readlane(incl, 63);
    int base = 0;
    if ((tid & 63) == 63 && wtot > 0) base = atomicAdd(&sm.misc[2], wtot);
    base = __builtin_amdgcn_readlane(base, 63);
    int slot = base + incl - cnt;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (k[i]) {
        if (slot < kCap) {
          sm.key[slot] = k[i];
          sm.idx[slot] = (uint16_t)(kScoreGroup * g + i);
        }
        ++slot;
      }
  }
  __syncthreads();
}

__device__ __forceinline__ void topk_row(int t, const float* __restrict__ scores, int score_stride,
                                         const float* __restrict__ gmax,
                                         const int32_t* __restrict__ q_pos,
                                         int32_t* __restrict__ sel_blocks, int32_t* __restrict__ sel_pos,
                                         int sel_stride, int32_t* __restrict__ sel_count) {
  const int tid = threadIdx.x;
  const int p = q_pos[t];
  const int n = (p + 1) / kBlock;
  QSA_CHECK(p >= 0 && n <= score_stride);
  const int pend = (p + 1) % kBlock;
  int32_t* row_b = sel_blocks + (size_t)t * kTopK;
  int32_t* row_p = sel_pos + (size_t)t * sel_stride;

  if (n <= kTopK) {
    for (int i = tid; i < kTopK; i += kT) row_b[i] = i < n ? i : -1;
    for (int i = tid; i < sel_stride; i += kT) row_p[i] = i <= p ? i : -1;
    if (tid == 0) sel_count[t] = p + 1;
    return;
  }

  const float* srow = scores + (size_t)t * score_stride;
  const int nwords = (n + 31) / 32;
  const int w0 = 2 * tid;              // this thread's two bitmap words
  if (w0 < nwords) {
    sm.bits[w0] = 0u;
    sm.eqbits[w0] = 0u;
  }
  if (w0 + 1 < nwords) {
    sm.bits[w0 + 1] = 0u;
    sm.eqbits[w0 + 1] = 0u;
  }

  // candidates (scores >= a lower bound of the 512th) -> sm.key / sm.idx
  const int nq = (n + 3) / 4;
  const float* grow = gmax ? gmax + (size_t)t * (score_stride / kScoreGroup) : nullptr;
  if (nq <= 4 * kT) topk_quads<4, true>(srow, n);
  else if (grow && n <= 2 * kT * kScoreGroup) topk_groups<2>(srow, grow, n);
  else if (grow) topk_groups<4>(srow, grow, n);
  else if (nq <= 8 * kT) topk_quads<8, true>(srow, n);
  else topk_quads<16, false>(srow, n);

  // exact select over the candidates, mark kept (bits) and tied (eqbits) blocks
  if (tid == 0) sm.misc[3] = 0;        // keys equal to the threshold
  const int ncand = sm.misc[2];
  uint2 thr;
  if (ncand <= kCap) {
    constexpr int EC = kCap / kT;
    uint32_t ck[EC];
#pragma unroll
    for (int e = 0; e < EC; ++e) {
      const int i = tid + kT * e;
      ck[e] = i < ncand ? sm.key[i] : 0u;
    }
    thr = select_keys<EC>(ck, kTopK, false);
#pragma unroll
    for (int e = 0; e < EC; ++e) {
      const int i = tid + kT * e;
      if (i < ncand && ck[e] >= thr.x) {
        const int c = sm.idx[i];
        if (ck[e] == thr.x) atomicAdd(&sm.misc[3], 1);
        atomicOr(ck[e] > thr.x ? &sm.bits[c >> 5] : &sm.eqbits[c >> 5], 1u << (c & 31));
      }
    }
  } else {
    thr = select_row(srow, n, kTopK);
    for (int c = tid; c < n; c += kT) {
      const uint32_t k = float_key(srow[c]);
      if (k >= thr.x) {
        if (k == thr.x) atomicAdd(&sm.misc[3], 1);
        atomicOr(k > thr.x ? &sm.bits[c >> 5] : &sm.eqbits[c >> 5], 1u << (c & 31));
      }
    }
  }
  __syncthreads();

  // ties: keep the need_eq lowest indices of eqbits (all of them in the usual case)
  {
    const int need_eq = (int)thr.y;
    const uint32_t e0 = w0 < nwords ? sm.eqbits[w0] : 0u;
    const uint32_t e1 = w0 + 1 < nwords ? sm.eqbits[w0 + 1] : 0u;
    if (sm.misc[3] == need_eq) {
      if (e0) sm.bits[w0] |= e0;
      if (e1) sm.bits[w0 + 1] |= e1;
    } else {
      int r = block_scan(__popc(e0) + __popc(e1)).x;
      uint32_t keep0 = 0, keep1 = 0;
      for (uint32_t e = e0; e; e &= e - 1) keep0 |= (r++ < need_eq) ? (e & (~e + 1u)) : 0u;
      for (uint32_t e = e1; e; e &= e - 1) keep1 |= (r++ < need_eq) ? (e & (~e + 1u)) : 0u;
      if (keep0) sm.bits[w0] |= keep0;
      if (keep1) sm.bits[w0 + 1] |= keep1;
    }
  }

  // emit the kept blocks in index order, each expanded to its 4 positions
  {
    const uint32_t b0 = w0 < nwords ? sm.bits[w0] : 0u;
    const uint32_t b1 = w0 + 1 < nwords ? sm.bits[w0 + 1] : 0u;
    const int idx0 = block_scan(__popc(b0) + __popc(b1)).x;
    if (n <= 8 * kT) {
      // dense rows: per-word prefix in LDS, then one block per thread per step
      if (w0 < nwords) sm.wpre[w0] = (uint16_t)idx0;
      if (w0 + 1 < nwords) sm.wpre[w0 + 1] = (uint16_t)(idx0 + __popc(b0));
      __syncthreads();
      for (int c = tid; c < n; c += kT) {
        const uint32_t wv = sm.bits[c >> 5];
        const int b = c & 31;
        if ((wv >> b) & 1u) {
          const int idx = sm.wpre[c >> 5] + __popc(wv & ((1u << b) - 1u));
          if (idx < kTopK) {   // exactly kTopK bits are set; the guard only bounds the row
            row_b[idx] = c;
            *reinterpret_cast<int4*>(row_p + kBlock * idx) = make_int4(4 * c, 4 * c + 1, 4 * c + 2, 4 * c + 3);
          }
        }
      }
    } else {
      int idx = idx0;
      const uint32_t word[2] = {b0, b1};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        for (uint32_t e = word[h]; e; e &= e - 1) {
          const int c = 32 * (w0 + h) + __ffs(e) - 1;
          if (idx < kTopK) {
            row_b[idx] = c;
            *reinterpret_cast<int4*>(row_p + kBlock * idx) = make_int4(4 * c, 4 * c + 1, 4 * c + 2, 4 * c + 3);
          }
          ++idx;
        }
      }
    }
  }
  const int base = kBlock * kTopK;
  for (int i = base + tid; i < sel_stride; i += kT) {
    const int k = i - base;
    row_p[i] = k < pend ? kBlock * n + k : -1;
  }
  if (tid == 0) sel_count[t] = base + pend;
}

// ------------------------------------------------------------------ latency-bound select

// The select of topk_kernel: one work group of kFT = 1024 threads per row.  A row's
// time is a chain of dependent steps (two memory round trips, then LDS work with a
// barrier after each step).  With 16 waves, 4 per SIMD, each wave holds only a few of
// the row's units per step and the waves of a SIMD hide each other's LDS and memory
// latency (batch 32: 9.6 us per launch against 11.2 with 512 threads and 15.0 with
// 256).  The work on the row's scores is done four scores at a time.
//   - The row's position and its 16-block group maxima (written by the scorer) are
//     requested together at kernel start, the maxima before the row's length is known
//     (the workspace row of maxima is score_stride / 16 long), so the first memory
//     round trip brings both.  Thread i holds groups kGPT i .. kGPT i + kGPT - 1.
//   - Lower bound t0: the 512th largest group maximum, from one linear-bin histogram
//     pass (256 bins between the smallest and largest maximum), rounded down by one
//     bin.  At least 512 groups reach it, hence at least 512 scores.
//   - The candidate groups (maximum >= t0, about 520-600) are gathered in LDS, and
//     each thread loads the scores of up to kCGT of them (the second and last round
//     trip; the scorer writes a row's last group whole, -inf past the row's end).
//   - Every float4 of those scores that holds a score >= t0 goes to an LDS list as it
//     is (about 650 per row), with the index of its first block.
//   - The exact 512th largest key T and how many keys equal to T are kept come from
//     radix passes of 8 bits over key - t0 by the whole group, one barrier each (the
//     list's keys >= t0 lie between t0 and the row's largest maximum); a pass whose
//     chosen bin holds one key stops there and uses the bin as the threshold.
//   - The kept blocks (keys above T) and the blocks whose key equals T are marked in
//     two LDS bitmaps.  One block scan of the words' (greater, equal) counts gives
//     each word the kept blocks before it, and each kept block is written to its slot
//     by the thread that holds its key (so the stores are spread over all threads),
//     the need_eq lowest-indexed equal blocks included.
// Rows of fewer than 1024 groups load their whole score row instead and take the
// bound from 4-block quad maxima (or keep every score when the row has fewer than
// 512 quads): with so few groups the 512th group maximum keeps most groups, and their
// float4s above it can overflow the list.  Rows with too many candidates (heavy ties,
// such as a row of equal scores) take an exact select over the row in memory.
constexpr int kFT = 1024;                         // threads per row
constexpr int kFW = kFT / 64;
constexpr int kGPT = kMaxBlocks / kScoreGroup / kFT;   // group maxima per thread: 4
constexpr int kFCG = 1024;                        // candidate groups
constexpr int kCGT = kFCG / kFT;                  // candidate groups per thread: 1
constexpr int kShort = 2 * kTopK * kScoreGroup;   // rows below this many blocks are short
constexpr int kSPT = kShort / kFT;                // short-row scores per thread: 16
constexpr int kF4 = 1024;                         // listed float4s
constexpr int kF4T = kF4 / kFT;                   // listed float4s per thread: 1
constexpr int kBWords = kMaxBlocks / 32;          // bitmap words: 2048
constexpr int kBWT = kBWords / kFT;               // bitmap words per thread: 2
static_assert(kGPT % 4 == 0 && kSPT % 4 == 0, "whole 16-byte accesses");
static_assert(kFT >= 256 && kFT <= 1024 && kBWT >= 1, "256-bin histograms, one bin per thread");
static_assert(4 * kF4 < 65536, "bitmap counts packed in 16 bits");

struct __attribute__((aligned(16))) SmemF {
  f32x4_t lv[kF4];                   // listed float4s of scores
  int lc[kF4];                       // the block of each one's first score
  uint32_t gtb[kBWords];             // blocks with key > T
  uint32_t eqb[kBWords];             // blocks with key == T
  uint32_t pre[kBWords];             // per bitmap word: (equal before it) << 16 | (above before it)
  uint32_t hist[256];                // lower-bound histogram
  uint32_t rhist[3][256];            // the select's radix histograms (one per pass, cycled)
  uint16_t cg[kFCG];                 // candidate groups
  uint32_t red[2 * kFW];             // per-wave max / min
  uint32_t wsum[kFW];                // block-scan wave totals
  int misc[4];                       // [0] candidate groups, [1] listed float4s, [2] a published key
};

__shared__ SmemF sf;

// Exclusive block-wide scan of one value per thread; .x = prefix, .y = total.
__device__ __forceinline__ uint2 fscan(uint32_t v) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint32_t inc = (uint32_t)wave_inclusive_sum((int)v);
  if (lane == 63) sf.wsum[w] = inc;
  __syncthreads();
  uint32_t before = 0u, total = 0u;
#pragma unroll
  for (int i = 0; i < kFW; ++i) {
    const uint32_t x = sf.wsum[i];
    before += i < w ? x : 0u;
    total += x;
  }
  return make_uint2(before + inc - v, total);
}

// Slot base of this lane's `cnt` items in a shared counter (one LDS atomic per wave).
__device__ __forceinline__ int wave_slots(int cnt, int* counter) {
  const int lane = threadIdx.x & 63;
  const int incl = wave_inclusive_sum(cnt);
  const int wtot = __builtin_amdgcn_readlane(incl, 63);
  int base = 0;
  if (lane == 63 && wtot > 0) base = atomicAdd(counter, wtot);
  return __builtin_amdgcn_readlane(base, 63) + incl - cnt;
}

// Block-wide max and min of one key per thread (min over non-zero keys); one barrier.
__device__ __forceinline__ uint2 block_max_min(uint32_t mx, uint32_t mn) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  mx = wave_max_u32(mx);
  mn = wave_min_u32(mn);
  if (lane == 0) {
    sf.red[w] = mx;
    sf.red[kFW + w] = mn;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kFW; ++i) {
    mx = max(mx, sf.red[i]);
    mn = min(mn, sf.red[kFW + i]);
  }
  return make_uint2(mx, mn);
}

// The bin of a 256-bin histogram that holds the kk-th largest entry, found by every
// wave at once (lane l reads bins 4l..4l+3): .x = bin, .y = rank of the entry inside
// the bin (1 = its largest), .z = the bin's count.
__device__ __forceinline__ int3 hist_find(const uint32_t* H, int kk) {
  const int lane = threadIdx.x & 63;
  const uint4 h = reinterpret_cast<const uint4*>(H)[lane];
  const int mine = (int)(h.x + h.y + h.z + h.w);
  const int inc = wave_inclusive_sum(mine);
  const int above = __builtin_amdgcn_readlane(inc, 63) - inc;   // entries in higher lanes' bins
  int d = 0, r = 0, cnt = 0;
  const bool here = above < kk && kk <= above + mine;
  if (here) {
    const int a3 = above + (int)h.w, a2 = a3 + (int)h.z, a1 = a2 + (int)h.y;
    if (kk <= a3) { d = 3; r = kk - above; cnt = (int)h.w; }
    else if (kk <= a2) { d = 2; r = kk - a3; cnt = (int)h.z; }
    else if (kk <= a1) { d = 1; r = kk - a2; cnt = (int)h.y; }
    else { d = 0; r = kk - a1; cnt = (int)h.x; }
    d += 4 * lane;
  }
  const int src = (int)__ffsll((unsigned long long)__ballot(here)) - 1;
  return make_int3(__shfl(d, src, 64), __shfl(r, src, 64), __shfl(cnt, src, 64));
}

// Lower bound of the kk-th largest of the units' keys (0 = no unit): a key that at
// least kk units reach, and the largest unit.  Every thread returns the same pair.
// Two barriers.
template <int U>
__device__ __forceinline__ uint2 units_lower_bound(const uint32_t (&uk)[U], int kk) {
  const int tid = threadIdx.x;
  uint32_t mx = 0u, mn = 0xffffffffu;
#pragma unroll
  for (int e = 0; e < U; ++e) {
    mx = max(mx, uk[e]);
    mn = min(mn, uk[e] ? uk[e] : 0xffffffffu);
  }
  if (tid < 256) sf.hist[tid] = 0u;
  const uint2 mm = block_max_min(mx, mn);
  mx = mm.x;
  mn = mm.y;
  if (mx == mn) return make_uint2(mx, mx);   // every unit equal (block-uniform)
  const float fmn = key_float(mn), fmx = key_float(mx);
  const float scale = 256.f / (fmx - fmn);
  if (!(scale > 0.f && scale < 3.0e38f && fmx - fmn < 3.0e38f)) return make_uint2(mn, mx);
#pragma unroll
  for (int e = 0; e < U; ++e)
    if (uk[e]) atomicAdd(&sf.hist[min(255, (int)((key_float(uk[e]) - fmn) * scale))], 1u);
  __syncthreads();
  const int bin = hist_find(sf.hist, kk).x;
  // every unit of the bins from `bin` up lies at or above the edge of bin - 1
  return make_uint2(bin > 0 ? max(mn, float_key(fmn + (float)(bin - 1) / scale)) : mn, mx);
}

// The threshold of a select: a listed key k (nonzero, >= lo_key) is above it when
// (k - lo_key) >> shift > q, equal to it when (k - lo_key) >> shift == q, and the
// need_eq lowest-indexed keys equal to it are kept.
struct Thresh {
  uint32_t lo_key, q;
  int shift, need_eq;
};

// 0 = below the threshold (or no key), 1 = equal, 2 = above.
__device__ __forceinline__ int classify(uint32_t k, const Thresh& th) {
  if (k == 0u) return 0;
  const uint32_t d = (k - th.lo_key) >> th.shift;
  return d > th.q ? 2 : (d == th.q ? 1 : 0);
}

// The kk-th largest of the keys held by the block (E per thread, 0 = none), all in
// [lo_key, hi_key].  Radix passes of 8 bits over key - lo_key from the top of the
// range, one barrier each: the histogram a pass fills was cleared during the
// previous pass, and it clears the one the next pass fills (rhist[0] is cleared by
// the caller before an earlier barrier).  A pass whose chosen bin holds a single key
// ends the search there: that key is the kk-th largest and the only one of its value,
// so the threshold is its bin (no barrier to publish the key itself).  The same
// Thresh in every thread.
template <int E>
__device__ __forceinline__ Thresh block_select(const uint32_t (&key)[E], uint32_t lo_key,
                                               uint32_t hi_key, int kk) {
  const int tid = threadIdx.x;
  if (hi_key <= lo_key) return Thresh{lo_key, 0u, 0, kk};   // every key equal
  int hi = 31 - __clz(hi_key - lo_key);
  uint32_t prefix = 0u;              // digits of key - lo_key found so far
  for (int pass = 0;; ++pass) {
    uint32_t* H = sf.rhist[pass % 3];
    const int lo = max(hi - 7, 0);
    const uint32_t pmask = hi == 31 ? 0u : ~((2u << hi) - 1u);
    const uint32_t dmask = (1u << (hi - lo + 1)) - 1u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t r = key[e] - lo_key;
      if (key[e] && (r & pmask) == prefix) atomicAdd(&H[(r >> lo) & dmask], 1u);
    }
    if (tid < 256) sf.rhist[(pass + 1) % 3][tid] = 0u;
    __syncthreads();
    const int3 f = hist_find(H, kk);
    kk = f.y;
    prefix |= (uint32_t)f.x << lo;
    if (lo == 0) return Thresh{lo_key, prefix, 0, kk};   // every key of the bin is equal
    if (f.z == 1) return Thresh{lo_key, prefix >> lo, lo, 1};
    hi = lo - 1;
  }
}

// Kept blocks of a row from its scores in memory, for rows the latency-bound select
// does not cover (heavy ties, such as a row of equal scores; n > 512): four radix
// passes of 8 bits over the whole row find T and need_eq exactly, then thread i emits
// the kept blocks of its contiguous slice of the row at the slots given by a block
// scan.  Slow but exact for any row; out of line, so that its registers do not add
// to the latency-bound select's.
__device__ __attribute__((noinline)) void topk_row_general(
    int t, const float* __restrict__ scores, int score_stride, const int32_t* __restrict__ q_pos,
    int32_t* __restrict__ sel_blocks, int32_t* __restrict__ sel_pos, int sel_stride,
    int32_t* __restrict__ sel_count) {
  const int tid = threadIdx.x;
  const float* srow = scores + (size_t)t * score_stride;
  const int p = q_pos[t];
  const int n = (p + 1) / kBlock;
  const int pend = (p + 1) % kBlock;
  int32_t* row_b = sel_blocks + (size_t)t * kTopK;
  int32_t* row_p = sel_pos + (size_t)t * sel_stride;
  uint32_t prefix = 0u;
  int kk = kTopK;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t pmask = pass == 0 ? 0u : (0xffffffffu << (shift + 8));
    __syncthreads();                   // the previous pass has read the histogram
    if (tid < 256) sf.hist[tid] = 0u;
    __syncthreads();
    for (int c = tid; c < n; c += kFT) {
      const uint32_t key = float_key(srow[c]);
      if ((key & pmask) == prefix) atomicAdd(&sf.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    const int3 f = hist_find(sf.hist, kk);
    prefix |= (uint32_t)f.x << shift;
    kk = f.y;
  }
  const uint32_t T = prefix;
  const int need_eq = kk;
  const int per = (n + kFT - 1) / kFT;
  const int cb = min(n, per * tid), ce = min(n, cb + per);
  int gt = 0, eq = 0;
  for (int c = cb; c < ce; ++c) {
    const uint32_t key = float_key(srow[c]);
    gt += key > T ? 1 : 0;
    eq += key == T ? 1 : 0;
  }
  // (equal counts clamped at 512 keep min(prefix, need_eq) exact and the sums in 17 bits)
  const uint2 sc = fscan(((uint32_t)min(eq, kTopK) << 10) | (uint32_t)gt);
  int bgt = (int)(sc.x & 1023u), beq = (int)(sc.x >> 10);
  for (int c = cb; c < ce; ++c) {
    const uint32_t key = float_key(srow[c]);
    int out = -1;
    if (key > T) {
      out = bgt + min(beq, need_eq);
      ++bgt;
    } else if (key == T) {
      if (beq < need_eq) out = bgt + beq;
      ++beq;
    }
    if (out >= 0 && out < kTopK) {
      row_b[out] = c;
      *reinterpret_cast<int4*>(row_p + kBlock * out) = make_int4(4 * c, 4 * c + 1, 4 * c + 2, 4 * c + 3);
    }
  }
  const int base = kBlock * kTopK;
  for (int i = base + tid; i < sel_stride; i += kFT) {
    const int kq = i - base;
    row_p[i] = kq < pend ? kBlock * n + kq : -1;
  }
  if (tid == 0) sel_count[t] = base + pend;
}

// This thread's float4s of scores (E of them, the first block of each in c[]; -inf
// or a block past the row = no score) that hold a score >= t0f go to the list.
template <int E>
__device__ __forceinline__ void list_float4s(const f32x4_t (&v)[E], const int (&c)[E], float t0f) {
  bool in[E];
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    in[e] = fmaxf(fmaxf(v[e][0], v[e][1]), fmaxf(v[e][2], v[e][3])) >= t0f;
    cnt += in[e] ? 1 : 0;
  }
  int slot = wave_slots(cnt, &sf.misc[1]);
  if (cnt > 0) {
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (in[e]) {
        if (slot < kF4) {
          sf.lv[slot] = v[e];
          sf.lc[slot] = c[e];
        }
        ++slot;
      }
  }
}

__device__ __forceinline__ void topk_row_fast(int t, const float* __restrict__ scores,
                                              const float* __restrict__ gmax, int score_stride,
                                              const int32_t* __restrict__ q_pos,
                                              int32_t* __restrict__ sel_blocks,
                                              int32_t* __restrict__ sel_pos, int sel_stride,
                                              int32_t* __restrict__ sel_count) {
  const int tid = threadIdx.x;
  const float* srow = scores + (size_t)t * score_stride;
  const int gstride = score_stride / kScoreGroup;      // a multiple of 8
  // this thread's group maxima, requested with the row's position (a thread past the
  // workspace row reads its last ones)
  f32x4_t gm4[kGPT / 4];
  {
    const float* grow = gmax + (size_t)t * gstride;
#pragma unroll
    for (int i = 0; i < kGPT / 4; ++i)
      gm4[i] = *reinterpret_cast<const f32x4_t*>(grow + min(kGPT * tid + 4 * i, gstride - 4));
  }
  const int p = q_pos[t];
  const int n = (p + 1) / kBlock;
  QSA_CHECK(p >= 0 && n <= score_stride);
  const int pend = (p + 1) % kBlock;
  int32_t* row_b = sel_blocks + (size_t)t * kTopK;
  int32_t* row_p = sel_pos + (size_t)t * sel_stride;
  if (n <= kTopK) {
    for (int i = tid; i < kTopK; i += kFT) row_b[i] = i < n ? i : -1;
    for (int i = tid; i < sel_stride; i += kFT) row_p[i] = i <= p ? i : -1;
    if (tid == 0) sel_count[t] = p + 1;
    return;
  }
  // cleared before the first barrier: the select's first histogram, the bitmaps, the
  // counters
  if (tid < 256) sf.rhist[0][tid] = 0u;
#pragma unroll
  for (int i = 0; i < kBWT; ++i) {
    sf.gtb[kBWT * tid + i] = 0u;
    sf.eqb[kBWT * tid + i] = 0u;
  }
  if (tid == 0) {
    sf.misc[0] = 0;
    sf.misc[1] = 0;
  }
  uint32_t t_low, row_max;           // every listed key >= t_low lies in [t_low, row_max]
  if (n >= kShort) {
    const int G = (n + kScoreGroup - 1) / kScoreGroup;
    // ---- lower bound from the group maxima
    uint32_t uk[kGPT];
#pragma unroll
    for (int e = 0; e < kGPT; ++e) uk[e] = kGPT * tid + e < G ? float_key(gm4[e >> 2][e & 3]) : 0u;
    const uint2 lb = units_lower_bound<kGPT>(uk, kTopK);
    t_low = max(lb.x, 1u);
    row_max = lb.y;
    // ---- candidate groups into LDS (any order)
    int nc = 0;
#pragma unroll
    for (int e = 0; e < kGPT; ++e) nc += uk[e] >= t_low ? 1 : 0;
    int slot = wave_slots(nc, &sf.misc[0]);
    if (nc > 0) {
#pragma unroll
      for (int e = 0; e < kGPT; ++e)
        if (uk[e] >= t_low) {
          if (slot < kFCG) sf.cg[slot] = (uint16_t)(kGPT * tid + e);
          ++slot;
        }
    }
    __syncthreads();
    const int ncg = sf.misc[0];
    if (ncg > kFCG) {                  // heavy ties
      __syncthreads();
      topk_row_general(t, scores, score_stride, q_pos, sel_blocks, sel_pos, sel_stride, sel_count);
      return;
    }
    // ---- candidate groups tid, tid + kFT, ..: their scores, as 4 float4s each
    // (unconditional loads; past the last candidate a thread reads group 0, masked)
    f32x4_t v[kCGT * 4];
    int c[kCGT * 4];
#pragma unroll
    for (int e = 0; e < kCGT; ++e) {
      const int i = tid + kFT * e;
      const int g = i < ncg ? (int)sf.cg[i] : -1;
      const f32x4_t* src = reinterpret_cast<const f32x4_t*>(srow + kScoreGroup * max(g, 0));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[4 * e + q] = src[q];
        c[4 * e + q] = g < 0 ? kMaxBlocks : kScoreGroup * g + 4 * q;
      }
    }
#pragma unroll
    for (int e = 0; e < kCGT * 4; ++e)
      if (c[e] >= kMaxBlocks) v[e] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    list_float4s<kCGT * 4>(v, c, key_float(t_low));
  } else {
    // ---- short row: the whole row, kSPT blocks per thread in index order
    const int cs0 = kSPT * tid;
    f32x4_t v[kSPT / 4];
    int c[kSPT / 4];
    uint32_t uk[kSPT / 4];             // quad maxima
#pragma unroll
    for (int q = 0; q < kSPT / 4; ++q) {
      c[q] = cs0 + 4 * q;
      v[q] = *reinterpret_cast<const f32x4_t*>(srow + min(c[q], score_stride - 4));
    }
#pragma unroll
    for (int q = 0; q < kSPT / 4; ++q) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (c[q] + j >= n) v[q][j] = -INFINITY;
      const float m = fmaxf(fmaxf(v[q][0], v[q][1]), fmaxf(v[q][2], v[q][3]));
      uk[q] = c[q] < n ? float_key(m) : 0u;
    }
    if ((n + 3) / 4 >= kTopK) {        // at least 512 quads: the 512th largest quad maximum
      const uint2 lb = units_lower_bound<kSPT / 4>(uk, kTopK);
      t_low = max(lb.x, 1u);
      row_max = lb.y;
    } else {                           // every score is a candidate: the row's range
      uint32_t mx = 0u, mn = 0xffffffffu;
#pragma unroll
      for (int q = 0; q < kSPT / 4; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (c[q] + j < n) {
            const uint32_t k = float_key(v[q][j]);
            mx = max(mx, k);
            mn = min(mn, k);
          }
      const uint2 mm = block_max_min(mx, mn);
      t_low = max(mm.y, 1u);
      row_max = mm.x;
    }
    list_float4s<kSPT / 4>(v, c, key_float(t_low));
  }
  __syncthreads();
  const int n4 = sf.misc[1];
  if (n4 > kF4) {                      // heavy ties
    __syncthreads();
    topk_row_general(t, scores, score_stride, q_pos, sel_blocks, sel_pos, sel_stride, sel_count);
    return;
  }

  // ---- the exact threshold over the listed keys >= t_low; thread i holds float4s
  // kF4T i .. kF4T i + kF4T - 1
  uint32_t lk[kF4T * 4];
  int lc[kF4T];
#pragma unroll
  for (int e = 0; e < kF4T; ++e) {
    const int i = kF4T * tid + e;
    const f32x4_t x = sf.lv[min(i, kF4 - 1)];
    lc[e] = sf.lc[min(i, kF4 - 1)];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t k = float_key(x[j]);
      lk[4 * e + j] = (i < n4 && k >= t_low) ? k : 0u;
    }
  }
  const Thresh th = block_select<kF4T * 4>(lk, t_low, row_max, kTopK);
  const int need_eq = th.need_eq;

  // ---- mark the blocks above T and those equal to T
#pragma unroll
  for (int e = 0; e < kF4T; ++e)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cl = classify(lk[4 * e + j], th);
      if (cl > 0) {
        const int cc = lc[e] + j;
        atomicOr(cl == 2 ? &sf.gtb[cc >> 5] : &sf.eqb[cc >> 5], 1u << (cc & 31));
      }
    }
  __syncthreads();

  // ---- per bitmap word, the blocks above T and equal to T before it within its wave
  // (thread i owns words kBWT i .. kBWT i + kBWT - 1), and per wave its totals; the
  // emit adds the totals of the waves before.  Counts are packed (equal << 16 | above):
  // a set bit is a listed key, at most 4 kF4 of them, so neither half carries.
  {
    uint32_t gc[kBWT], ec[kBWT];
#pragma unroll
    for (int i = 0; i < kBWT; ++i) {
      gc[i] = __popc(sf.gtb[kBWT * tid + i]);
      ec[i] = __popc(sf.eqb[kBWT * tid + i]);
    }
    uint32_t v = 0u;
#pragma unroll
    for (int i = 0; i < kBWT; ++i) v += (ec[i] << 16) | gc[i];
    const uint32_t inc = (uint32_t)wave_inclusive_sum((int)v);
    if ((tid & 63) == 63) sf.wsum[tid >> 6] = inc;
    uint32_t run = inc - v;
#pragma unroll
    for (int i = 0; i < kBWT; ++i) {
      sf.pre[kBWT * tid + i] = run;
      run += (ec[i] << 16) | gc[i];
    }
  }
  __syncthreads();
  // ---- emit: each kept block goes from the thread that holds its key to slot (above
  // before it) + min(equal before it, need_eq); a block equal to the threshold is kept
  // while fewer than need_eq equal blocks precede it
#pragma unroll
  for (int e = 0; e < kF4T; ++e) {
    // a float4's 4 blocks lie in one bitmap word (its first block is a multiple of 4);
    // an entry past the list holds no key, and its word index is only kept in range
    const int w = min(max(lc[e] >> 5, 0), kBWords - 1);
    const int ow = (w / kBWT) >> 6;    // the wave of the word's owner
    uint32_t pw = sf.pre[w];
#pragma unroll
    for (int i = 0; i < kFW; ++i) pw += i < ow ? sf.wsum[i] : 0u;
    const uint32_t gw = sf.gtb[w], ew = sf.eqb[w];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cl = classify(lk[4 * e + j], th);
      if (cl > 0) {
        const int cc = lc[e] + j;
        const uint32_t below = (1u << (cc & 31)) - 1u;
        const int g_below = (int)(pw & 0xffffu) + __popc(gw & below);
        const int e_below = (int)(pw >> 16) + __popc(ew & below);
        int out = -1;
        if (cl == 2) out = g_below + min(e_below, need_eq);
        else if (e_below < need_eq) out = g_below + e_below;
        if (out >= 0 && out < kTopK) {   // exactly kTopK are kept; the guard bounds the row
          row_b[out] = cc;
          *reinterpret_cast<int4*>(row_p + kBlock * out) =
              make_int4(4 * cc, 4 * cc + 1, 4 * cc + 2, 4 * cc + 3);
        }
      }
    }
  }
  const int base = kBlock * kTopK;
  for (int i = base + tid; i < sel_stride; i += kFT) {
    const int kq = i - base;
    row_p[i] = kq < pend ? kBlock * n + kq : -1;
  }
  if (tid == 0) sel_count[t] = base + pend;
}

__global__ void __launch_bounds__(kFT)
topk_kernel(const float* __restrict__ scores, const float* __restrict__ gmax, int score_stride,
            const int32_t* __restrict__ q_pos, int32_t* __restrict__ sel_blocks,
            int32_t* __restrict__ sel_pos, int sel_stride, int32_t* __restrict__ sel_count) {
  topk_row_fast(blockIdx.x, scores, gmax, score_stride, q_pos, sel_blocks, sel_pos, sel_stride,
                sel_count);
}

// The rows listed in queue[1 .. queue[0]] (rows the code-based select hands over).
__global__ void __launch_bounds__(kT)
topk_queued_kernel(const int* __restrict__ queue, const float* __restrict__ scores,
                   int score_stride, const int32_t* __restrict__ q_pos,
                   int32_t* __restrict__ sel_blocks, int32_t* __restrict__ sel_pos, int sel_stride,
                   int32_t* __restrict__ sel_count) {
  const int nq = queue[0];
  for (int k = blockIdx.x; k < nq; k += gridDim.x) {
    __syncthreads();                   // LDS of the previous row is free
    topk_row(queue[1 + k], scores, score_stride, nullptr, q_pos, sel_blocks, sel_pos, sel_stride,
             sel_count);
  }
}

}  // namespace

void launch_topk(const IndexArgs& a, hipStream_t stream) {
  QSA_LAUNCH(topk_kernel, dim3(a.total_q), dim3(kFT), 0, stream, a.scores, a.gmax_f, a.score_stride,
             a.q_pos, a.sel_blocks, a.sel_pos, a.sel_stride, a.sel_count);
}

void launch_topk_queued(const IndexArgs& a, hipStream_t stream) {
  QSA_LAUNCH(topk_queued_kernel, dim3(std::min(a.total_q, 256)), dim3(kT), 0, stream, a.queue,
                     a.scores, a.score_stride, a.q_pos, a.sel_blocks, a.sel_pos, a.sel_stride,
                     a.sel_count);
}

}  // namespace qsa
