// Stage 2: indexer - block scores, top-512 selection and expansion.
//
// [SGLang day-0 post on Qwen3.8-Flash-Next, section "Qwen Sparse Attention:
// Retrieve Coarsely, Attend Precisely"]: a query scores every visible compressed
// block, the best 512 blocks are kept and expanded to their 2048 token
// positions, and the 0..3 tokens of the unfinished block are appended (at most
// 2051 positions).  The scoring formula is cut off on the page; the kernels
// compute s_c = sum_h w_h * max(0, q_h . k_c) over the 4 indexer heads.
//
// Kernels:
//  * score_kernel: paged GEMV.  One wave streams one group of 16 consecutive
//    blocks (one 4 KB compressed page when page_size = 64) per step: 4 loads of
//    16 B per lane, each load covering 4 blocks x 256 B contiguous.  Lane l
//    owns dims (l%16)*8 .. +8 of block (l/16); dot products use v_dot2_f32_bf16
//    (bf16 pairs, FP32 accumulation) and are summed over the 16 lanes of a row
//    with DPP.  Besides every score it writes each group's maximum.
//  * topk_kernel: one 1024-thread work group per query.  The 512th largest
//    group maximum t0 is a lower bound of the 512th largest score, so only
//    scores >= t0 (typically under a thousand) are gathered into LDS; an exact
//    4 x 8-bit radix select over them finds the threshold key, ties at the
//    threshold go to the lowest block indices, and the kept blocks are emitted
//    in ascending order through an LDS bitmap and a block-wide prefix count.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

namespace {

constexpr int kScoreThreads = 256;
constexpr int kScoreMaxQ = 4096;       // queries per scorer launch (LDS prefix table)
constexpr int kTopkThreads = 1024;
constexpr int kCandCap = 4096;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ int groups_of(int p) {
  const int n = (p + 1) / kBlock;
  return (n + kScoreGroup - 1) / kScoreGroup;
}

// ------------------------------------------------------------------ scorer

__global__ void __launch_bounds__(kScoreThreads)
score_kernel(int nq, const uint16_t* __restrict__ idx_q, const float* __restrict__ idx_w,
             const int32_t* __restrict__ q_req, const int32_t* __restrict__ q_pos,
             const int32_t* __restrict__ page_table, int pt_stride, int page_size,
             const uint16_t* __restrict__ comp, float* __restrict__ scores,
             float* __restrict__ gmax, int score_stride) {
  __shared__ int s_pre[kScoreMaxQ + 1];
  __shared__ int s_part[kScoreThreads];
  const int tid = threadIdx.x;

  // exclusive prefix of groups per query: s_pre[t] = first group of query t
  const int per = (nq + kScoreThreads - 1) / kScoreThreads;
  const int q0 = min(tid * per, nq), q1 = min(q0 + per, nq);
  int sum = 0;
  for (int t = q0; t < q1; ++t) sum += groups_of(q_pos[t]);
  s_part[tid] = sum;
  __syncthreads();
  for (int d = 1; d < kScoreThreads; d <<= 1) {
    const int v = (tid >= d) ? s_part[tid - d] : 0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  int run = s_part[tid] - sum;
  for (int t = q0; t < q1; ++t) {
    s_pre[t] = run;
    run += groups_of(q_pos[t]);
  }
  if (tid == kScoreThreads - 1) s_pre[nq] = s_part[tid];
  __syncthreads();
  const int total = s_pre[nq];

  const int lane = tid & 63;
  const int nwaves = gridDim.x * (kScoreThreads / 64);
  const int wave = blockIdx.x * (kScoreThreads / 64) + (tid >> 6);
  const int g_begin = (int)(((int64_t)total * wave) / nwaves);
  const int g_end = (int)(((int64_t)total * (wave + 1)) / nwaves);
  if (g_begin >= g_end) return;

  // query owning g_begin: last t with s_pre[t] <= g_begin (skipping empty queries)
  int lo = 0, hi = nq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_pre[mid] <= g_begin) lo = mid; else hi = mid - 1;
  }
  int t = lo;
  while (s_pre[t + 1] <= g_begin) ++t;

  const int d0 = (lane & 15) * 8;
  const int row_in_step = lane >> 4;
  const int bpp = page_size / kBlock;
  int cur_t = -1;
  u32x4_t qf[kIdxHeads];
  float w[kIdxHeads];
  int req = 0, n_c = 0;
  for (int gi = g_begin; gi < g_end; ++gi) {
    while (s_pre[t + 1] <= gi) ++t;
    if (t != cur_t) {
      cur_t = t;
      req = q_req[t];
      n_c = (q_pos[t] + 1) / kBlock;
#pragma unroll
      for (int h = 0; h < kIdxHeads; ++h) {
        qf[h] = ld16(idx_q + ((size_t)t * kIdxHeads + h) * kIdxDim + d0);
        w[h] = idx_w[(size_t)t * kIdxHeads + h];
      }
    }
    const int g = gi - s_pre[t];
    const int32_t* pt_row = page_table + (size_t)req * pt_stride;
    u32x4_t kv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = g * kScoreGroup + 4 * r + row_in_step;
      const int cc = min(c, n_c - 1);
      const int64_t row = (int64_t)pt_row[cc / bpp] * bpp + (cc % bpp);
      kv[r] = ld16(comp + row * kIdxDim + d0);
    }
    float best = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float s = 0.f;
#pragma unroll
      for (int h = 0; h < kIdxHeads; ++h) {
        float a = dot2(kv[r].x, qf[h].x, 0.f);
        a = dot2(kv[r].y, qf[h].y, a);
        a = dot2(kv[r].z, qf[h].z, a);
        a = dot2(kv[r].w, qf[h].w, a);
        a = row16_sum(a);
        s += w[h] * fmaxf(a, 0.f);
      }
      const int c = g * kScoreGroup + 4 * r + row_in_step;
      if (c < n_c) {
        if ((lane & 15) == 0) scores[(size_t)t * score_stride + c] = s;
        best = fmaxf(best, s);
      }
    }
    best = fmaxf(best, shfl_xor_f(best, 16));
    best = fmaxf(best, shfl_xor_f(best, 32));
    if (lane == 0) gmax[(size_t)t * (score_stride / kScoreGroup) + g] = best;
  }
}

// ------------------------------------------------------------------ top-512

struct TopkSmem {
  uint32_t hist[256];
  uint32_t cand_key[kCandCap];
  uint32_t cand_idx[kCandCap];
  uint32_t bits[kMaxBlocks / 32];
  uint32_t eqbits[kMaxBlocks / 32];
  int wsum[kTopkThreads / 64];
  int misc[8];
};

// k-th largest key (k >= 1) among n elements given by key_at(i), i < n; returns the
// key and sets *rank_in_eq to how many elements equal to it are needed (1..).
template <typename KeyAt>
__device__ uint32_t kth_largest(TopkSmem& sm, int n, int k, KeyAt key_at, int* rank_in_eq) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0;
  int kk = k;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const uint32_t mask = pass == 0 ? 0u : (0xffffffffu << (shift + 8));
    if (tid < 256) sm.hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kTopkThreads) {
      const uint32_t key = key_at(i);
      if ((key & mask) == prefix) atomicAdd(&sm.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      const uint32_t h0 = sm.hist[4 * tid], h1 = sm.hist[4 * tid + 1];
      const uint32_t h2 = sm.hist[4 * tid + 2], h3 = sm.hist[4 * tid + 3];
      const int mine = (int)(h0 + h1 + h2 + h3);
      // suffix sum over lanes >= tid
      int suf = mine;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_down(suf, d, 64);
        if (tid + d < 64) suf += v;
      }
      int above = suf - mine;   // elements whose digit lies in higher lanes
      if (above < kk && kk <= suf) {
        const uint32_t hh[4] = {h0, h1, h2, h3};
        int dsel = 4 * tid;
        for (int q = 3; q >= 0; --q) {
          if (kk <= above + (int)hh[q]) { dsel = 4 * tid + q; break; }
          above += (int)hh[q];
        }
        sm.misc[0] = dsel;
        sm.misc[1] = kk - above;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sm.misc[0] << shift;
    kk = sm.misc[1];
    __syncthreads();
  }
  *rank_in_eq = kk;
  return prefix;
}

// Block-wide exclusive scan of one int per thread; returns the exclusive prefix,
// total in *tot.
__device__ int block_exclusive_scan(TopkSmem& sm, int v, int* tot) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(inc, d, 64);
    if (lane >= d) inc += u;
  }
  if (lane == 63) sm.wsum[wv] = inc;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < kTopkThreads / 64; ++i) {
      const int x = sm.wsum[i];
      sm.wsum[i] = run;
      run += x;
    }
    sm.misc[2] = run;
  }
  __syncthreads();
  const int res = sm.wsum[wv] + inc - v;
  *tot = sm.misc[2];
  __syncthreads();
  return res;
}

__global__ void __launch_bounds__(kTopkThreads)
topk_kernel(const float* __restrict__ scores, const float* __restrict__ gmax, int score_stride,
            const int32_t* __restrict__ q_pos, int32_t* __restrict__ sel_blocks,
            int32_t* __restrict__ sel_pos, int sel_stride, int32_t* __restrict__ sel_count) {
  __shared__ TopkSmem sm;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int p = q_pos[t];
  const int n = (p + 1) / kBlock;
  const int pend = (p + 1) % kBlock;
  int32_t* row_b = sel_blocks + (size_t)t * kTopK;
  int32_t* row_p = sel_pos + (size_t)t * sel_stride;

  if (n <= kTopK) {
    // every block is kept: the positions are simply 0..p
    for (int i = tid; i < kTopK; i += kTopkThreads) row_b[i] = i < n ? i : -1;
    for (int i = tid; i < sel_stride; i += kTopkThreads) row_p[i] = i <= p ? i : -1;
    if (tid == 0) sel_count[t] = p + 1;
    return;
  }

  const float* srow = scores + (size_t)t * score_stride;
  const float* grow = gmax + (size_t)t * (score_stride / kScoreGroup);
  const int ng = (n + kScoreGroup - 1) / kScoreGroup;
  const int nwords = (n + 31) / 32;

  // candidates: scores >= t0, t0 = 512th largest group maximum
  bool overflow = true;
  int ncand = 0;
  if (ng >= kTopK) {
    int dummy;
    const uint32_t t0 = kth_largest(sm, ng, kTopK,
                                    [&](int i) { return float_key(grow[i]); }, &dummy);
    if (tid == 0) sm.misc[3] = 0;
    __syncthreads();
    for (int g = tid; g < ng; g += kTopkThreads) {
      if (float_key(grow[g]) < t0) continue;
      const int cbase = g * kScoreGroup;
      const int cend = min(cbase + kScoreGroup, n);
      for (int c = cbase; c < cend; ++c) {
        const uint32_t key = float_key(srow[c]);
        if (key >= t0) {
          const int slot = atomicAdd(&sm.misc[3], 1);
          if (slot < kCandCap) {
            sm.cand_key[slot] = key;
            sm.cand_idx[slot] = (uint32_t)c;
          }
        }
      }
    }
    __syncthreads();
    ncand = sm.misc[3];
    overflow = ncand > kCandCap;
    __syncthreads();
  }

  for (int i = tid; i < nwords; i += kTopkThreads) {
    sm.bits[i] = 0;
    sm.eqbits[i] = 0;
  }
  int need_eq;
  uint32_t thr;
  if (!overflow) {
    thr = kth_largest(sm, ncand, kTopK, [&](int i) { return sm.cand_key[i]; }, &need_eq);
    __syncthreads();
    for (int i = tid; i < ncand; i += kTopkThreads) {
      const uint32_t key = sm.cand_key[i];
      const uint32_t c = sm.cand_idx[i];
      if (key > thr) atomicOr(&sm.bits[c >> 5], 1u << (c & 31));
      else if (key == thr) atomicOr(&sm.eqbits[c >> 5], 1u << (c & 31));
    }
  } else {
    thr = kth_largest(sm, n, kTopK, [&](int i) { return float_key(srow[i]); }, &need_eq);
    __syncthreads();
    for (int c = tid; c < n; c += kTopkThreads) {
      const uint32_t key = float_key(srow[c]);
      if (key > thr) atomicOr(&sm.bits[c >> 5], 1u << (c & 31));
      else if (key == thr) atomicOr(&sm.eqbits[c >> 5], 1u << (c & 31));
    }
  }
  __syncthreads();

  // ties at the threshold: keep the need_eq lowest block indices
  {
    const int w0 = 2 * tid, w1 = 2 * tid + 1;
    const uint32_t e0 = w0 < nwords ? sm.eqbits[w0] : 0u;
    const uint32_t e1 = w1 < nwords ? sm.eqbits[w1] : 0u;
    int tot;
    int rank = block_exclusive_scan(sm, __popc(e0) + __popc(e1), &tot);
    uint32_t keep0 = 0, keep1 = 0;
    for (uint32_t e = e0; e; e &= e - 1) {
      if (rank < need_eq) keep0 |= e & (~e + 1);
      ++rank;
    }
    for (uint32_t e = e1; e; e &= e - 1) {
      if (rank < need_eq) keep1 |= e & (~e + 1);
      ++rank;
    }
    if (keep0) sm.bits[w0] |= keep0;
    if (keep1) sm.bits[w1] |= keep1;
  }
  __syncthreads();

  // emit kept blocks in ascending order, each expanded to its 4 positions
  {
    const int w0 = 2 * tid, w1 = 2 * tid + 1;
    const uint32_t b0 = w0 < nwords ? sm.bits[w0] : 0u;
    const uint32_t b1 = w1 < nwords ? sm.bits[w1] : 0u;
    int tot;
    int idx = block_exclusive_scan(sm, __popc(b0) + __popc(b1), &tot);
    const uint32_t word[2] = {b0, b1};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      for (uint32_t e = word[q]; e; e &= e - 1) {
        const int c = 32 * (w0 + q) + __ffs(e) - 1;
        if (idx < kTopK) {   // exactly kTopK bits are set; the guard only bounds the row
          row_b[idx] = c;
#pragma unroll
          for (int k = 0; k < kBlock; ++k) row_p[kBlock * idx + k] = kBlock * c + k;
        }
        ++idx;
      }
    }
  }
  const int base = kBlock * kTopK;
  for (int i = base + tid; i < sel_stride; i += kTopkThreads) {
    const int k = i - base;
    row_p[i] = k < pend ? kBlock * n + k : -1;
  }
  if (tid == 0) sel_count[t] = base + pend;
}

}  // namespace

size_t index_workspace_bytes(int total_q, int max_pos) {
  const int nb = (max_pos + kBlock - 1) / kBlock;
  const size_t stride = (size_t)((nb + 63) / 64) * 64;
  const size_t s = (size_t)total_q * stride * sizeof(float);
  const size_t g = (size_t)total_q * (stride / kScoreGroup) * sizeof(float);
  return ((s + 255) / 256) * 256 + ((g + 255) / 256) * 256;
}

void index_workspace_carve(IndexArgs& a, void* ws) {
  const int nb = (a.max_pos + kBlock - 1) / kBlock;
  a.score_stride = ((nb + 63) / 64) * 64;
  const size_t s = (size_t)a.total_q * a.score_stride * sizeof(float);
  a.scores = reinterpret_cast<float*>(ws);
  a.gmax = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + ((s + 255) / 256) * 256);
}

hipError_t launch_index(const IndexArgs& a, hipStream_t stream) {
  for (int q0 = 0; q0 < a.total_q; q0 += kScoreMaxQ) {
    const int nq = std::min(kScoreMaxQ, a.total_q - q0);
    // blocks to score are only known on the device; size the grid by the bound
    const int64_t groups_bound =
        (int64_t)nq * ((a.max_pos / kBlock + kScoreGroup - 1) / kScoreGroup);
    const int waves_wanted = (int)std::min<int64_t>(groups_bound / 2 + 1, 16384);
    const int grid = std::max(1, waves_wanted / (kScoreThreads / 64));
    hipLaunchKernelGGL(score_kernel, dim3(grid), dim3(kScoreThreads), 0, stream, nq,
                       a.idx_q + (size_t)q0 * kIdxHeads * kIdxDim, a.idx_w + (size_t)q0 * kIdxHeads,
                       a.q_req + q0, a.q_pos + q0, a.page_table, a.pt_stride, a.page_size, a.comp,
                       a.scores + (size_t)q0 * a.score_stride,
                       a.gmax + (size_t)q0 * (a.score_stride / kScoreGroup), a.score_stride);
  }
  hipLaunchKernelGGL(topk_kernel, dim3(a.total_q), dim3(kTopkThreads), 0, stream, a.scores, a.gmax,
                     a.score_stride, a.q_pos, a.sel_blocks, a.sel_pos, a.sel_stride, a.sel_count);
  return hipGetLastError();
}

}  // namespace qsa
