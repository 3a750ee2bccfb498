// Stage 2a: indexer block scores for decode-like batches (paged GEMV) and for a
// few queries per request (multi-query MFMA scorer).
//
// [SGLang day-0 post on Qwen3.8-Flash-Next, section "Qwen Sparse Attention:
// Retrieve Coarsely, Attend Precisely"]: a query scores every visible compressed
// block.  The scoring formula is cut off on the page; the kernels compute
// s_c = sum_h w_h * max(0, q_h . k_c) over the 4 indexer heads.
//
// score_kernel is a paged GEMV.  A wave streams groups of 16 consecutive blocks
// (one 4 KB compressed page when page_size = 64): 4 loads of 16 B per lane.  The
// dot products run on v_mfma_f32_16x16x32_bf16 with the group's keys as the B
// operand (lane l holds block l%16, dims 8(l/16) + 32kc of K-chunk kc, so a load
// covers 64 contiguous bytes of each of the 16 rows) and the query's 4 heads as rows
// 0..3 of the A operand (rows 4..15 zero): four MFMAs leave the 4 head dots of block
// l in lane l < 16, which mixes them with head_mix, the arithmetic of every MFMA
// scorer.  The MFMA's idle rows cost nothing that matters here; against the
// v_dot2_f32_bf16 form with DPP row sums it replaces about 160 VALU instructions per
// group by 4 MFMAs and 8 VALU, and the batch-32 decode scorer went from 20.2 to
// 17.7 us.
//
// score_multi_kernel serves batches with a few queries per request, such as the
// verification pass over drafted tokens [same post, section "IndexShare MTP:
// Reusing the QSA Selection Across Draft Steps": the target model checks N+1
// tokens per request]: the queries of a request share each key load.  Top-512
// selection and expansion live in qsa_topk.hip.
#include "qsa_device.h"
#include "qsa_keymath.h"
#include "qsa_launch.h"

#include <cmath>

namespace qsa {

namespace {


__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ int groups_of(int p) {
  const int n = (p + 1) / kBlock;
  return (n + kScoreGroup - 1) / kScoreGroup;
}

// ------------------------------------------------------------------ scorer

// One wave per work group.  The (at most 64) queries of a launch are laid out one
// per lane: each lane holds its query's group count, first group, request and
// block count, and a group index is mapped to its query with one ballot.  The
// wave takes a contiguous range of at most kWaveGroups groups.
//
// The loop over the range issues loads only: page-table entries two groups ahead,
// keys (and the query's rows when the query changes) one group ahead, each into a
// ping-pong register set; scores stay in LDS until the range is done.  With no
// store in flight the in-order load counter lets each wait cover exactly the loads
// it needs, so three groups' loads overlap.
//
// A decode step can also ingest each request's new token in the same launch
// (score_build_kernel).  The first nq work groups then belong one to each query:
// query t's group writes the token to its ring slot or, when the token completes a
// block, builds that block's key with the builder's arithmetic (qsa_keymath.h),
// stores it, and scores the query's last 16-block group, which holds the new block,
// with the key taken from LDS.  The other work groups score every group but the
// last of each query.  No work group reads memory that another one writes.
constexpr int kWaveGroups = 64;
// Waves of a scorer launch (at most): 3 per SIMD, all resident at once (batch-32
// decode 17.8 us against 18.1 us with 4096 waves and 18.2 us with 2048; the
// multi-query scorer of batch-32 verification 22.1 against 22.6 us with 4096).
constexpr int kScorerWaves = 3072;

struct GroupMeta {
  int t, g, n_c;
  const int32_t* pt_row;
};

struct QueryRows {
  u32x4_t af[4];         // A operand: head l%16 (rows 4..15 zero), dims 8(l/16) + 32kc
  float w[kIdxHeads];
};

// The step's new tokens (score_build_kernel): query t of the launch is request
// req0 + t, and its own token, at position q_pos[t], is the one ingested.
struct Ingest {
  const uint16_t* new_k;   // [nq, 128] raw indexer keys of those tokens
  uint16_t* ring;          // [batch, 4, 128] pending-token ring
  uint16_t* comp;          // the compressed key cache (the new blocks' rows are written)
  const int32_t* new_mpos; // [nq, 3] MRoPE positions of those tokens, or NULL (1-D RoPE)
  int32_t* ring_mpos;      // [batch, 4, 3] positions of the ring's tokens (MRoPE only)
  int req0;
  RopeTable rope;
};

template <bool kIngest>
__device__ __forceinline__ void score_body(
    int nq, const uint16_t* __restrict__ idx_q, const float* __restrict__ idx_w,
    const int32_t* __restrict__ q_req, const int32_t* __restrict__ q_pos,
    const int32_t* __restrict__ page_table, int pt_stride, int page_size,
    const uint16_t* __restrict__ comp, float* __restrict__ scores, int score_stride,
    float* __restrict__ gmax, const Ingest* ing) {
  __shared__ float s_out[kWaveGroups * kScoreGroup];
  __shared__ int s_tg[kWaveGroups];    // query << 16 | group, per group of the range
  const int lane = threadIdx.x;
  const int my_nc = lane < nq ? (q_pos[lane] + 1) / kBlock : 0;
  QSA_CHECK(lane >= nq || (q_pos[lane] >= 0 && my_nc <= score_stride));
  const int my_req = lane < nq ? (kIngest ? ing->req0 + lane : q_req[lane]) : 0;
  const int all_groups = (my_nc + kScoreGroup - 1) / kScoreGroup;
  // with kIngest the last group of a query is left to the query's own work group
  const int my_groups = kIngest ? max(all_groups - 1, 0) : all_groups;
  int incl = my_groups;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(incl, d, 64);
    if (lane >= d) incl += u;
  }
  const int excl = incl - my_groups;
  const int total = __shfl(incl, 63, 64);

  const int bpp = page_size / kBlock;
  int g_begin = 0;
  int ng = 0;

  auto meta = [&](int i) {             // group g_begin + i: i wave-uniform, every lane active
    GroupMeta m;
    const int gi = g_begin + i;
    m.t = __popcll(__ballot(incl <= gi));   // first query whose groups reach gi
    m.g = gi - __shfl(excl, m.t, 64);
    m.n_c = __shfl(my_nc, m.t, 64);
    m.pt_row = page_table + (size_t)__shfl(my_req, m.t, 64) * pt_stride;
    return m;
  };
  // lane l holds block l%16 of a group as the B operand, dims 8(l/16) + 32kc
  auto block_of = [&](const GroupMeta& m) { return min(m.g * kScoreGroup + (lane & 15), m.n_c - 1); };
  auto pt_load = [&](int i) {
    const GroupMeta m = meta(i);
    const int pg = m.pt_row[block_of(m) / bpp];
    QSA_CHECK(pg >= 0);
    return pg;
  };
  auto key_load = [&](int i, int pg, u32x4_t (&kv)[4]) {
    const GroupMeta m = meta(i);
    if (lane == 0) s_tg[i] = (m.t << 16) | m.g;
    const int c = block_of(m);
    const uint16_t* krow = comp + ((int64_t)pg * bpp + (c % bpp)) * kIdxDim + 8 * (lane >> 4);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) kv[kc] = ld16(krow + 32 * kc);
  };
  auto query_load = [&](int t, QueryRows& q) {
    const int h = lane & 15;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
      q.af[kc] = h < kIdxHeads
                     ? ld16(idx_q + ((size_t)t * kIdxHeads + h) * kIdxDim + 32 * kc + 8 * (lane >> 4))
                     : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < kIdxHeads; ++j) q.w[j] = idx_w[(size_t)t * kIdxHeads + j];
  };
  // the group's 16 block scores on MFMA: lanes 0..15 receive the 4 head dots of block l
  auto compute = [&](int i, const u32x4_t (&kv)[4], const QueryRows& q) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) acc = mfma16(q.af[kc], kv[kc], acc);
    const float s = head_mix(acc, q.w);
    if (lane < kScoreGroup) s_out[i * kScoreGroup + lane] = s;
  };

  if (kIngest && (int)blockIdx.x < nq) {
    // ---- query t's own work group: its token, then its last group
    const int t = blockIdx.x;
    const int b = ing->req0 + t;
    const int p = q_pos[t];
    const int n_c = (p + 1) / kBlock;
    const bool fresh = ((p + 1) % kBlock) == 0;   // the token completes block n_c - 1
    const uint16_t* nk = ing->new_k + (size_t)t * kIdxDim;
    uint16_t* rb = ing->ring + (size_t)b * kBlock * kIdxDim;
    QSA_CHECK(p >= 0 && p / page_size < pt_stride);
    if (!fresh) {   // the token waits in ring slot p % 4 until its block completes
      reinterpret_cast<uint32_t*>(rb + (p % kBlock) * kIdxDim)[lane] =
          reinterpret_cast<const uint32_t*>(nk)[lane];   // 64 lanes x 2 bf16
      if (ing->new_mpos && lane < 3)
        ing->ring_mpos[((size_t)b * kBlock + (p % kBlock)) * 3 + lane] =
            ing->new_mpos[(size_t)t * 3 + lane];
    }
    if (n_c == 0) return;
    GroupMeta m;
    m.t = t;
    m.g = (n_c - 1) / kScoreGroup;
    m.n_c = n_c;
    m.pt_row = page_table + (size_t)b * pt_stride;
    const int pg = m.pt_row[block_of(m) / bpp];
    QSA_CHECK(pg >= 0);
    QueryRows q;
    query_load(t, q);
    const int j = lane & 15;
    float mean[8];
    if (fresh) {   // tokens 4c..4c+2 wait in ring slots 0..2, token 4c+3 is the new one
      const uint16_t* src[kBlock] = {rb, rb + kIdxDim, rb + 2 * kIdxDim, nk};
      key_block_mean(src, j, mean);
    }
    u32x4_t kv[4];
    {   // the new block's row is stale here; it is replaced below
      const int c = block_of(m);
      const uint16_t* krow = ing->comp + ((int64_t)pg * bpp + (c % bpp)) * kIdxDim + 8 * (lane >> 4);
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) kv[kc] = ld16(krow + 32 * kc);
    }
    if (fresh) {
      __shared__ __attribute__((aligned(16))) u32x2_t s_key[kIdxDim / 4];
      const int c = n_c - 1;
      double ppos[4];
      if (ing->new_mpos) {   // 3-D position of token 4c, which waits in ring slot 0
        const int32_t* p3 = ing->ring_mpos + (size_t)b * kBlock * 3;
#pragma unroll
        for (int e = 0; e < 4; ++e) ppos[e] = (double)p3[ing->rope.axis[4 * j + e]];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) ppos[e] = (double)(kBlock * c);
      }
      u32x2_t lo, hi;
      key_rotate(mean, ppos, ing->rope.inv_freq, j, lo, hi);
      if (lane < 16) {
        const int64_t row = (int64_t)m.pt_row[c / bpp] * bpp + (c % bpp);
        uint16_t* dst = ing->comp + row * kIdxDim;
        *reinterpret_cast<u32x2_t*>(dst + 4 * j) = lo;
        *reinterpret_cast<u32x2_t*>(dst + 64 + 4 * j) = hi;
        s_key[j] = lo;          // dims 4j..4j+3
        s_key[16 + j] = hi;     // dims 64+4j..64+4j+3
      }
      __syncthreads();
      if (block_of(m) == c) {
        const uint16_t* nkey = reinterpret_cast<const uint16_t*>(s_key) + 8 * (lane >> 4);
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) kv[kc] = *reinterpret_cast<const u32x4_t*>(nkey + 32 * kc);
      }
    }
    if (lane == 0) s_tg[0] = (t << 16) | m.g;
    compute(0, kv, q);
    ng = 1;
  } else {
    const int wave = blockIdx.x - (kIngest ? nq : 0);
    const int nwaves = gridDim.x - (kIngest ? nq : 0);
    g_begin = (int)(((int64_t)total * wave) / nwaves);
    const int g_end = (int)(((int64_t)total * (wave + 1)) / nwaves);
    ng = g_end - g_begin;              // <= kWaveGroups (the launch sizes the grid for it)
    if (ng <= 0) return;

    // pipeline: at step i the page entries of group i+2 and the keys of group i+1
    // are requested, then group i is scored
    int pg0, pg1 = 0;
    u32x4_t kv0[4], kv1[4];
    QueryRows q0, q1;
    int t0 = meta(0).t;
    query_load(t0, q0);
    pg0 = pt_load(0);
    if (ng > 1) pg1 = pt_load(1);
    key_load(0, pg0, kv0);
    int tq1 = t0;
    for (int i = 0; i < ng; i += 2) {
      // even step: group i in kv0 / q0
      if (i + 2 < ng) pg0 = pt_load(i + 2);
      if (i + 1 < ng) {
        tq1 = meta(i + 1).t;
        if (tq1 != t0) query_load(tq1, q1); else q1 = q0;
        key_load(i + 1, pg1, kv1);
      }
      compute(i, kv0, q0);
      if (i + 1 >= ng) break;
      // odd step: group i+1 in kv1 / q1
      if (i + 3 < ng) pg1 = pt_load(i + 3);
      if (i + 2 < ng) {
        t0 = meta(i + 2).t;
        if (t0 != tq1) query_load(t0, q0); else q0 = q1;
        key_load(i + 2, pg0, kv0);
      }
      compute(i + 1, kv1, q1);
    }
  }

  // write the range's scores and each group's maximum: lane l covers group l / 4,
  // blocks 4 (l % 4) .. +3.  Past the last block the computed scores repeat the last
  // block's (the loads were clamped), so the maximum is that of the visible blocks.
  const int gstride = score_stride / kScoreGroup;
  for (int i0 = 0; i0 < ng; i0 += 16) {
    const int i = min(i0 + (lane >> 2), ng - 1);
    const int tg = s_tg[i];
    const int t = tg >> 16;
    const int n_c = __shfl(my_nc, t, 64);     // every lane active: its own query's count
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(&s_out[i * kScoreGroup + 4 * (lane & 3)]);
    float m = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
    m = fmaxf(m, dpp_f<0xb1>(m));            // quad_perm [1,0,3,2]
    m = fmaxf(m, dpp_f<0x4e>(m));            // quad_perm [2,3,0,1]
    if (i0 + (lane >> 2) < ng) {
      if ((lane & 3) == 0) gmax[(size_t)t * gstride + (tg & 0xffff)] = m;
      // the group's whole 16 scores, -inf past the last block (the select reads
      // groups whole)
      const int c = (tg & 0xffff) * kScoreGroup + 4 * (lane & 3);
      f32x4_t o = v;
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = c + k < n_c ? v[k] : -INFINITY;
      *reinterpret_cast<f32x4_t*>(scores + (size_t)t * score_stride + c) = o;
    }
  }
}

__global__ void __launch_bounds__(64)
score_kernel(int nq, const uint16_t* __restrict__ idx_q, const float* __restrict__ idx_w,
             const int32_t* __restrict__ q_req, const int32_t* __restrict__ q_pos,
             const int32_t* __restrict__ page_table, int pt_stride, int page_size,
             const uint16_t* __restrict__ comp, float* __restrict__ scores, int score_stride,
             float* __restrict__ gmax) {
  score_body<false>(nq, idx_q, idx_w, q_req, q_pos, page_table, pt_stride, page_size, comp,
                    scores, score_stride, gmax, nullptr);
}

__global__ void __launch_bounds__(64)
score_build_kernel(int nq, const uint16_t* __restrict__ idx_q, const float* __restrict__ idx_w,
                   const int32_t* __restrict__ q_pos, const int32_t* __restrict__ page_table,
                   int pt_stride, int page_size, const uint16_t* __restrict__ comp,
                   float* __restrict__ scores, int score_stride, float* __restrict__ gmax,
                   Ingest ing) {
  score_body<true>(nq, idx_q, idx_w, nullptr, q_pos, page_table, pt_stride, page_size, comp,
                   scores, score_stride, gmax, &ing);
}

// ------------------------------------------------------------------ multi-query scorer

// A few queries per request: target verification of drafted tokens, small chunks.
// Queries are taken in windows of 4 consecutive ones.  The queries of a window that
// share a request form a pass, and a pass scores each 16-block group of its request
// once for all its queries, on MFMA: A = 4 queries x 4 heads (16 rows; rows of
// queries outside the pass are zero), B = the group's 16 keys (k = dims).  Lane l
// of the result holds the 4 head dots of query l/16 and block l%16.
//
// One wave per work group; a launch covers up to 64 windows, one per lane.  Units
// (window, pass, group) are flattened and each wave takes a contiguous range.  The
// loop requests page-table entries two units ahead and keys (plus the pass's query
// rows when the pass changes) one unit ahead.  A unit's scores are stored after the
// next unit's loads have been issued, so a wait never covers a store issued less
// than a unit earlier.
constexpr int kWin = 4;
constexpr int kMultiWindows = 64;

struct Unit {
  int win, j, g;        // window (lane), leader query of the pass, group
  int mask;             // the pass's queries in the window (4 bits)
  int nc_max;           // visible blocks of the pass's longest query
  const int32_t* pt_row;
};

struct PassRows {
  u32x4_t af[4];        // A operand: query (l%16)/4, head l%4, dims 8(l/16) + 32kc
  float w[kIdxHeads];   // weights of this lane's result query l/16
  int nc;               // its visible blocks (0 when it is not in the pass)
  int t;                // its query index in the launch
};

__global__ void __launch_bounds__(64, 4)   // 4 waves per SIMD
score_multi_kernel(int nq, const uint16_t* __restrict__ idx_q, const float* __restrict__ idx_w,
                   const int32_t* __restrict__ q_req, const int32_t* __restrict__ q_pos,
                   const int32_t* __restrict__ page_table, int pt_stride, int page_size,
                   const uint16_t* __restrict__ comp, float* __restrict__ scores, int score_stride,
                   float* __restrict__ gmax) {
  // per window: requests, visible blocks, and per pass leader j its queries (4 bits)
  // and visible blocks of its longest query (0: j leads no pass)
  __shared__ int s_req[kMultiWindows][kWin], s_nc[kMultiWindows][kWin];
  __shared__ int s_pnc[kMultiWindows][kWin], s_pmask[kMultiWindows];
  const int lane = threadIdx.x;
  int mine = 0;
  {
    int wreq[kWin], wnc[kWin];
#pragma unroll
    for (int j = 0; j < kWin; ++j) {
      const int t = kWin * lane + j;
      wreq[j] = t < nq ? q_req[t] : -1;
      wnc[j] = t < nq ? (q_pos[t] + 1) / kBlock : 0;
      QSA_CHECK(t >= nq || (q_pos[t] >= 0 && wnc[j] <= score_stride));
      s_req[lane][j] = wreq[j];
      s_nc[lane][j] = wnc[j];
    }
    int pmask = 0;
#pragma unroll
    for (int j = 0; j < kWin; ++j) {
      bool leader = wreq[j] >= 0;
#pragma unroll
      for (int i = 0; i < j; ++i) leader = leader && wreq[i] != wreq[j];
      int m = 0, ncm = 0;
#pragma unroll
      for (int i = j; i < kWin; ++i)
        if (wreq[i] == wreq[j]) {
          m |= 1 << i;
          ncm = max(ncm, wnc[i]);
        }
      pmask |= (leader ? m : 0) << (4 * j);
      s_pnc[lane][j] = leader ? ncm : 0;
      mine += leader ? (ncm + kScoreGroup - 1) / kScoreGroup : 0;
    }
    s_pmask[lane] = pmask;
  }
  __syncthreads();
  const int incl = wave_inclusive_sum(mine);
  const int excl = incl - mine;
  const int total = __shfl(incl, 63, 64);
  const int wave = blockIdx.x, nwaves = gridDim.x;
  const int g_begin = (int)(((int64_t)total * wave) / nwaves);
  const int ng = (int)(((int64_t)total * (wave + 1)) / nwaves) - g_begin;
  if (ng <= 0) return;
  const int bpp = page_size / kBlock;
  const int gstride = score_stride / kScoreGroup;

  auto groups = [](int nc) { return (nc + kScoreGroup - 1) / kScoreGroup; };
  auto unit = [&](int i) {             // unit g_begin + i: i wave-uniform, every lane active;
    Unit u;                            // every field is wave-uniform (scalar registers)
    const int gi = g_begin + i;
    u.win = __builtin_amdgcn_readfirstlane(__popcll(__ballot(incl <= gi)));
    int local = __builtin_amdgcn_readfirstlane(gi - __shfl(excl, u.win, 64));
    const int G0 = groups(s_pnc[u.win][0]), G1 = groups(s_pnc[u.win][1]), G2 = groups(s_pnc[u.win][2]);
    int j = 0;
    if (local >= G0) {
      local -= G0;
      j = 1;
      if (local >= G1) {
        local -= G1;
        j = 2;
        if (local >= G2) {
          local -= G2;
          j = 3;
        }
      }
    }
    u.j = __builtin_amdgcn_readfirstlane(j);
    u.g = __builtin_amdgcn_readfirstlane(local);
    u.mask = __builtin_amdgcn_readfirstlane((s_pmask[u.win] >> (4 * u.j)) & 15);
    u.nc_max = __builtin_amdgcn_readfirstlane(s_pnc[u.win][u.j]);
    u.pt_row = page_table + (size_t)__builtin_amdgcn_readfirstlane(s_req[u.win][u.j]) * pt_stride;
    return u;
  };
  auto block_of = [&](const Unit& u) { return min(u.g * kScoreGroup + (lane & 15), u.nc_max - 1); };
  auto pt_load = [&](const Unit& u) {
    const int pg = u.pt_row[block_of(u) / bpp];
    QSA_CHECK(pg >= 0);
    return pg;
  };
  auto key_load = [&](const Unit& u, int pg, u32x4_t (&kf)[4]) {
    const int c = block_of(u);
    const uint16_t* krow = comp + ((int64_t)pg * bpp + (c % bpp)) * kIdxDim + 8 * (lane >> 4);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) kf[kc] = ld16(krow + 32 * kc);
  };
  auto pass_load = [&](const Unit& u, PassRows& r) {
    const int qa = (lane & 15) >> 2;   // A row query
    const int ta = kWin * u.win + qa;
    const bool ina = (u.mask >> qa) & 1;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
      r.af[kc] = ina ? ld16(idx_q + ((size_t)ta * kIdxHeads + (lane & 3)) * kIdxDim + 32 * kc +
                            8 * (lane >> 4))
                     : u32x4_t{0u, 0u, 0u, 0u};
    const int qd = lane >> 4;          // result query
    r.t = kWin * u.win + qd;
    const bool ind = (u.mask >> qd) & 1;
    r.nc = ind ? s_nc[u.win][qd] : 0;
#pragma unroll
    for (int h = 0; h < kIdxHeads; ++h) r.w[h] = ind ? idx_w[(size_t)r.t * kIdxHeads + h] : 0.f;
  };
  auto same_pass = [](const Unit& a, const Unit& b) { return a.win == b.win && a.j == b.j; };
  auto compute_store = [&](const Unit& u, const u32x4_t (&kf)[4], const PassRows& r) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) acc = mfma16(r.af[kc], kf[kc], acc);
    const float s = head_mix(acc, r.w);
    const int c = u.g * kScoreGroup + (lane & 15);
    const bool ok = c < r.nc;
    const float m = row16_max(ok ? s : -INFINITY);
    // the query's groups whole, -inf past its last block (the select reads groups whole)
    if (c < ((r.nc + kScoreGroup - 1) & ~(kScoreGroup - 1)))
      scores[(size_t)r.t * score_stride + c] = ok ? s : -INFINITY;
    if ((lane & 15) == 0 && u.g * kScoreGroup < r.nc) gmax[(size_t)r.t * gstride + u.g] = m;
  };

  // units i (even) and i+1 (odd) alternate between two register sets
  Unit ua = unit(0), ub = ua, uc = ua, ud = ua;
  PassRows r0, r1;
  u32x4_t k0[4], k1[4];
  int pg0 = pt_load(ua), pg1 = 0;
  pass_load(ua, r0);
  if (ng > 1) {
    ub = unit(1);
    pg1 = pt_load(ub);
  }
  key_load(ua, pg0, k0);
  for (int i = 0; i < ng; i += 2) {
    if (i + 2 < ng) {
      uc = unit(i + 2);
      pg0 = pt_load(uc);
    }
    if (i + 1 < ng) {
      if (same_pass(ub, ua)) r1 = r0; else pass_load(ub, r1);
      key_load(ub, pg1, k1);
    }
    compute_store(ua, k0, r0);
    if (i + 1 >= ng) break;
    if (i + 3 < ng) {
      ud = unit(i + 3);
      pg1 = pt_load(ud);
    }
    if (i + 2 < ng) {
      if (same_pass(uc, ub)) r0 = r1; else pass_load(uc, r0);
      key_load(uc, pg0, k0);
    }
    compute_store(ub, k1, r1);
    ua = uc;
    ub = ud;
  }
}

}  // namespace

// Workspace: FP32 score rows [total_q, stride], then FP32 group maxima
// [total_q, stride / 16] (decode scorer); the code rows and 16-bit group maxima of
// the MFMA path live in the score rows' bytes (the FP32 rows are written only after
// every code has been read).  Then the queue of rows handed to the FP32 select.
static size_t score_rows_bytes(int total_q, int max_pos, int* stride) {
  const int nb = (max_pos + kBlock - 1) / kBlock;
  *stride = ((nb + 127) / 128) * 128;
  const size_t floats = (size_t)total_q * *stride + (size_t)total_q * (*stride / kScoreGroup);
  return (floats * sizeof(float) + 255) / 256 * 256;
}

size_t index_workspace_bytes(int total_q, int max_pos) {
  int stride;
  const size_t rows = score_rows_bytes(total_q, max_pos, &stride);
  return rows + ((size_t)(total_q + 1) * sizeof(int) + 255) / 256 * 256;
}

void index_workspace_carve(IndexArgs& a, void* ws) {
  const size_t rows = score_rows_bytes(a.total_q, a.max_pos, &a.score_stride);
  char* base = static_cast<char*>(ws);
  a.scores = reinterpret_cast<float*>(base);
  a.gmax_f = a.scores + (size_t)a.total_q * a.score_stride;
  a.codes = reinterpret_cast<uint16_t*>(base);
  a.gmax = a.codes + (size_t)a.total_q * a.score_stride;
  a.queue = reinterpret_cast<int*>(base + rows);
}

// Decode-like batches (about one query per request) take the paged GEMV scorer;
// a few queries per request (2 to 15 on average) take the multi-query MFMA scorer;
// both feed the FP32 select.  Chunks of many queries per request share their keys
// over 64-query tiles and take the MFMA scorer with the code-based select.
static bool use_mfma(const IndexArgs& a) {
  return a.total_q >= 64 && a.total_q >= 16 * a.batch;
}
static bool use_multi(const IndexArgs& a) { return a.total_q >= 2 * a.batch; }

hipError_t launch_index(const IndexArgs& a, hipStream_t stream) {
  if (use_mfma(a)) return launch_index_mfma(a, stream);
  const int64_t gpq = (a.max_pos / kBlock + kScoreGroup - 1) / kScoreGroup;   // groups per query, bound
  if (use_multi(a)) {
    constexpr int kQPerLaunch = kWin * kMultiWindows;
    for (int q0 = 0; q0 < a.total_q; q0 += kQPerLaunch) {
      const int nq = std::min(kQPerLaunch, a.total_q - q0);
      // passes: one per window, plus one per request boundary inside a window
      const int64_t passes = std::min<int64_t>(nq, (nq + kWin - 1) / kWin + a.batch - 1);
      const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(passes * gpq / 2, kScorerWaves));
      QSA_LAUNCH(score_multi_kernel, dim3(grid), dim3(64), 0, stream, nq,
                         a.idx_q + (size_t)q0 * kIdxHeads * kIdxDim,
                         a.idx_w + (size_t)q0 * kIdxHeads, a.q_req + q0, a.q_pos + q0,
                         a.page_table, a.pt_stride, a.page_size, a.comp,
                         a.scores + (size_t)q0 * a.score_stride, a.score_stride,
                         a.gmax_f + (size_t)q0 * (a.score_stride / kScoreGroup));
    }
    launch_topk(a, stream);
    return hipGetLastError();
  }
  constexpr int kQPerLaunch = 64;
  for (int q0 = 0; q0 < a.total_q; q0 += kQPerLaunch) {
    const int nq = std::min(kQPerLaunch, a.total_q - q0);
    // the block counts are only known on the device: size the grid by the bound,
    // at most kScorerWaves waves
    const int64_t groups_bound = (int64_t)nq * gpq;
    // at most kWaveGroups groups per wave; otherwise one group per wave, at most
    // kScorerWaves waves (small batches: batch 1 at 4099 positions 25.8 against 26.5 us
    // per step with two groups per wave)
    const int64_t want = std::min<int64_t>(groups_bound, kScorerWaves);
    const int grid = (int)std::max<int64_t>(
        1, std::max<int64_t>(want, (groups_bound + kWaveGroups - 1) / kWaveGroups));
    QSA_LAUNCH(score_kernel, dim3(grid), dim3(64), 0, stream, nq,
                       a.idx_q + (size_t)q0 * kIdxHeads * kIdxDim, a.idx_w + (size_t)q0 * kIdxHeads,
                       a.q_req + q0, a.q_pos + q0, a.page_table, a.pt_stride, a.page_size, a.comp,
                       a.scores + (size_t)q0 * a.score_stride, a.score_stride,
                       a.gmax_f + (size_t)q0 * (a.score_stride / kScoreGroup));
  }
  launch_topk(a, stream);
  return hipGetLastError();
}

// A decode step with its builder folded in: query t is request t and its own token
// (position q_pos[t]) is ingested by the scorer launch (score_build_kernel).
hipError_t launch_index_ingest(const IndexArgs& a, const IngestArgs& f, hipStream_t stream) {
  Ingest ing;
  for (int i = 0; i < kIdxDim / 2; ++i) {
    ing.rope.inv_freq[i] = std::pow((double)f.theta, -(2.0 * i) / (double)kIdxDim);
    ing.rope.axis[i] = f.pair_axis ? f.pair_axis[i] : 0;
  }
  ing.ring = f.ring;
  ing.comp = f.comp;
  ing.ring_mpos = f.ring_mpos;
  const int64_t gpq = (a.max_pos / kBlock + kScoreGroup - 1) / kScoreGroup;
  constexpr int kQPerLaunch = 64;
  for (int q0 = 0; q0 < a.total_q; q0 += kQPerLaunch) {
    const int nq = std::min(kQPerLaunch, a.total_q - q0);
    const int64_t groups_bound = (int64_t)nq * gpq;
    // the queries' own work groups take nq of the kScorerWaves
    const int64_t want = std::min<int64_t>(groups_bound, kScorerWaves - nq);
    const int grid = (int)std::max<int64_t>(
        1, std::max<int64_t>(want, (groups_bound + kWaveGroups - 1) / kWaveGroups));
    ing.new_k = f.new_k + (size_t)q0 * kIdxDim;
    ing.new_mpos = f.new_mpos ? f.new_mpos + (size_t)q0 * 3 : nullptr;
    ing.req0 = q0;
    // nq work groups of the queries' own, then the scorer's
    QSA_LAUNCH(score_build_kernel, dim3(nq + grid), dim3(64), 0, stream, nq,
                       a.idx_q + (size_t)q0 * kIdxHeads * kIdxDim, a.idx_w + (size_t)q0 * kIdxHeads,
                       a.q_pos + q0, a.page_table, a.pt_stride, a.page_size, a.comp,
                       a.scores + (size_t)q0 * a.score_stride, a.score_stride,
                       a.gmax_f + (size_t)q0 * (a.score_stride / kScoreGroup), ing);
  }
  launch_topk(a, stream);
  return hipGetLastError();
}

}  // namespace qsa
