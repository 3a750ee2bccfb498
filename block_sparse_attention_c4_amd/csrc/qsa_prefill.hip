// Stage 2, many queries per request (chunked prefill): block scores on MFMA and a
// throughput-oriented top-512.
//
// [SGLang day-0 post on Qwen3.8-Flash-Next, section "Qwen Sparse Attention:
// Retrieve Coarsely, Attend Precisely"]: every query scores each visible compressed
// block, keeps the best 512 blocks and attends to their tokens plus the tokens of
// the unfinished block.  The score of a block is s_c = sum_h w_h * max(0, q_h . k_c)
// over the 4 indexer heads (the page's formula is cut off; this is the reading
// the library implements).
//
// With thousands of queries on the same keys the scores are a dense contraction:
// [T*4 query-head rows x 128] x [128 x blocks].  score_mfma_kernel computes it with
// v_mfma_f32_16x16x32_bf16, one 64-query x 2048-block tile per work group.  The A
// operand holds 4 queries x 4 heads per 16 rows, so each lane of the result holds
// the 4 head dots of one (query, block) pair and mixes them in registers.
//
// A float score matrix for a 4096-query chunk at 128K context would be 528 MB
// written and read again.  Instead the scorer writes, per (query, block), the top
// 16 bits of the score's order-preserving key (a "code") and, per 16-block group,
// the largest code.  topk_codes_kernel finds the 512th largest code T from the
// groups whose maximum can reach it, keeps every block whose code exceeds T, and
// ranks the blocks whose code equals T by their exact FP32 scores, recomputed with
// the same MFMA arithmetic (an MFMA result element depends only on its own row and
// column operands, so the recomputed values are bit-identical).  Rows that exceed
// the kernel's candidate capacities (heavy ties) are queued; rescore_kernel writes
// their exact scores and the general FP32 top-k handles them.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

namespace {

constexpr int kPfQ = 64;         // queries per scorer work group (4 waves x 16)
constexpr int kPfRange = 2048;   // blocks per scorer work group
constexpr int kLdsRow = 136;     // bf16 per staged key row: 128 + 8 to spread LDS banks

__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Top 16 bits of the order-preserving key of a score.
__device__ __forceinline__ uint32_t score_code(float s) {
  const uint32_t u = __float_as_uint(s);
  return (u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u)) >> 16;
}

__device__ __forceinline__ int64_t comp_row(const int32_t* pt_row, int c, int bpp) {
  QSA_CHECK(pt_row[c / bpp] >= 0);
  return (int64_t)pt_row[c / bpp] * bpp + (c % bpp);
}

// A operand of one query for a recompute: its 4 heads in rows 0..3, zeros elsewhere.
__device__ __forceinline__ void query_rows(const uint16_t* idx_q, int t, u32x4_t (&af)[4]) {
  const int lane = threadIdx.x & 63;
  const int h = lane & 15;
#pragma unroll
  for (int kc = 0; kc < 4; ++kc)
    af[kc] = h < kIdxHeads
                 ? ld16(idx_q + ((size_t)t * kIdxHeads + h) * kIdxDim + 32 * kc + 8 * (lane >> 4))
                 : u32x4_t{0u, 0u, 0u, 0u};
}

// Scores of one query against 16 blocks (lane l & 15 gives the block); the result
// is valid in lanes 0..15.
__device__ __forceinline__ float score16(const u32x4_t (&af)[4], const uint16_t* krow,
                                         const float (&w)[kIdxHeads]) {
  const int lane = threadIdx.x & 63;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) acc = mfma16(af[kc], ld16(krow + 32 * kc + 8 * (lane >> 4)), acc);
  return head_mix(acc, w);
}

// ------------------------------------------------------------------ scorer

// A work group is 4 waves over a 64-query x 2048-block tile; a wave owns 16 queries
// (4 A tiles of 4 queries x 4 heads).  The block range is walked in phases of
// kPhase groups of 16 blocks.  One phase: its keys (loaded into registers during
// the previous phase) go to LDS; the next phase's keys are requested; the previous
// phase's codes are written out from LDS (128-byte row segments, one thread per
// (query, group), which also takes the group's maximum); the phase's groups are
// scored into the LDS code buffer.  Loads and stores issued in one phase are
// complete by the next phase's wait.
constexpr int kSW = 4;                               // waves per work group
constexpr int kST = 64 * kSW;                        // threads
constexpr int kATiles = kPfQ / (4 * kSW);            // A tiles per wave: 4
constexpr int kQW = 4 * kATiles;                     // queries per wave
constexpr int kPhase = 8;
constexpr int kStage = kPhase * 256 / kST;           // 16-byte key chunks per thread per phase
constexpr int kCodeRow = kPhase * kScoreGroup + 16;  // u16 per staged code row (+16: the 4 query rows of
                                                     // an epilogue store fall in distinct banks)
static_assert(kPhase % 4 == 0 && kST >= 4 * kPfQ, "the flush covers 64 queries x kPhase groups");

__global__ void __launch_bounds__(kST, 2)
score_mfma_kernel(int total_q, const uint16_t* __restrict__ idx_q, const float* __restrict__ idx_w,
                  const int32_t* __restrict__ q_req, const int32_t* __restrict__ q_pos,
                  const int32_t* __restrict__ page_table, int pt_stride, int page_size,
                  const uint16_t* __restrict__ comp, uint16_t* __restrict__ codes,
                  uint16_t* __restrict__ gmax, int stride, int n_ranges, int n_tiles,
                  int* __restrict__ queue) {
  __shared__ __attribute__((aligned(16))) uint16_t kv[kPhase][16 * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t cbuf[2][kPfQ * kCodeRow];
  __shared__ uint32_t rows[kPfRange];  // compressed-cache row of each block of the range
  // Work groups are dealt to the 8 XCDs round-robin; give each XCD a contiguous run
  // of (range, tile) pairs, range-major, so that the tiles of a key range meet in
  // one L2.
  const int hw = blockIdx.x;
  const int total = n_ranges * n_tiles;
  const int lin = (total % 8 == 0) ? (hw % 8) * (total / 8) + hw / 8 : hw;
  const int range = lin / n_tiles, tile = lin % n_tiles;
  if (hw == 0 && threadIdx.x == 0) queue[0] = 0;   // rows sent to the FP32 fallback

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int t0 = tile * kPfQ;
  const int c_begin = range * kPfRange;
  const int gstride = stride / kScoreGroup;
  const int bpp = page_size / kBlock;

  // lane l describes query t0 + l (the same in every wave)
  const int tq = t0 + lane;
  const bool qv = tq < total_q;
  const int req = qv ? q_req[tq] : -1;
  const int nc = qv ? (q_pos[tq] + 1) / kBlock : 0;
  QSA_CHECK(!qv || (q_pos[tq] >= 0 && nc <= stride));
  uint64_t remaining = __ballot(qv && nc > c_begin);
  const int fq = tid >> 2, fg = tid & 3;          // flush (tid < 256): query t0 + fq, groups fg + 4k

  while (remaining) {                  // one pass per request present in the tile
    const int r = __shfl(req, __ffsll((unsigned long long)remaining) - 1, 64);
    const uint64_t mask = __ballot(qv && req == r);
    remaining &= ~mask;
    const bool mine = (mask >> lane) & 1;
    const int nc_max = __builtin_amdgcn_readfirstlane((int)wave_max_u32(mine ? (uint32_t)nc : 0u));
    const int c_end = min(c_begin + kPfRange, nc_max);
    if (c_end <= c_begin) continue;
    const int n_here = c_end - c_begin;

    const int32_t* pt_row = page_table + (size_t)r * pt_stride;
    for (int i = tid; i < n_here; i += kST) {
      const int c = c_begin + i;
      QSA_CHECK(pt_row[c / bpp] >= 0);
      rows[i] = (uint32_t)pt_row[c / bpp] * (uint32_t)bpp + (uint32_t)(c % bpp);
    }

    u32x4_t af[kATiles][4];            // [A tile][k chunk]: row l%16 = query (l%16)/4, head l%4
    float wt[kATiles][kIdxHeads];      // weights of the query this lane's results belong to
    int st_nc[kATiles];
#pragma unroll
    for (int a = 0; a < kATiles; ++a) {
      const int qa = kQW * w + 4 * a + ((lane & 15) >> 2);
      const bool in = (mask >> qa) & 1;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
        af[a][kc] = in ? ld16(idx_q + ((size_t)(t0 + qa) * kIdxHeads + (lane & 3)) * kIdxDim +
                              32 * kc + 8 * (lane >> 4))
                       : u32x4_t{0u, 0u, 0u, 0u};
      const int qs = kQW * w + 4 * a + (lane >> 4);
      const bool ok = (mask >> qs) & 1;
      const int nc_q = __shfl(nc, qs, 64);   // every lane takes part: an idle source lane reads 0
      st_nc[a] = ok ? nc_q : 0;
#pragma unroll
      for (int h = 0; h < kIdxHeads; ++h) wt[a][h] = ok ? idx_w[(size_t)(t0 + qs) * kIdxHeads + h] : 0.f;
    }
    // groups below every visible count of the wave's queries need no masking
    const uint64_t wbits = (1ull << kQW) - 1ull;
    const uint64_t wmask = (mask >> (kQW * w)) & wbits;
    const uint32_t ncw = (uint32_t)__shfl(nc, kQW * w + (lane & (kQW - 1)), 64);
    const uint32_t wmin = wave_min_u32(lane < kQW ? ncw : 0xffffffffu);
    const int wave_min_nc = __builtin_amdgcn_readfirstlane(wmask == wbits ? (int)wmin : 0);
    // flush side: this thread's query
    const bool f_ok = tid < 256 && ((mask >> fq) & 1);
    uint16_t* f_codes = codes + (size_t)(t0 + fq) * stride + kScoreGroup * fg;
    uint16_t* f_gmax = gmax + (size_t)(t0 + fq) * gstride + fg;
    __syncthreads();                   // rows[] ready

    // staging: chunk i = tid + kST * k is group i / 256, block row (i / 16) % 16, dims (i % 16) * 8
    auto gload = [&](int c0, int k) {  // clamped past the end: always kStage loads in flight
      const int i = tid + kST * k;
      const int j = min(c0 - c_begin + kScoreGroup * (i >> 8) + ((i >> 4) & 15), n_here - 1);
      return ld16(comp + (size_t)rows[j] * kIdxDim + (i & 15) * 8);
    };
    auto flush = [&](int c0, int b) {  // codes of the phase at c0, staged in cbuf[b]
#pragma unroll
      for (int gg = 0; gg < kPhase; gg += 4) {   // groups fg, fg + 4, ... of the phase
        const int g = fg + gg;
        if (f_ok && c0 + kScoreGroup * g < c_end) {
          const u32x4_t x = *reinterpret_cast<const u32x4_t*>(&cbuf[b][fq * kCodeRow + kScoreGroup * g]);
          const u32x4_t y = *reinterpret_cast<const u32x4_t*>(&cbuf[b][fq * kCodeRow + kScoreGroup * g + 8]);
          *reinterpret_cast<u32x4_t*>(f_codes + c0 + kScoreGroup * gg) = x;
          *reinterpret_cast<u32x4_t*>(f_codes + c0 + kScoreGroup * gg + 8) = y;
          uint32_t m = 0u;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            m = max(m, max(x[i] & 0xffffu, x[i] >> 16));
            m = max(m, max(y[i] & 0xffffu, y[i] >> 16));
          }
          f_gmax[c0 / kScoreGroup + gg] = (uint16_t)m;
        }
      }
    };
    auto frag = [&](int d, u32x4_t (&bf)[4]) {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
        bf[kc] = *reinterpret_cast<const u32x4_t*>(&kv[d][(lane & 15) * kLdsRow + 32 * kc + 8 * (lane >> 4)]);
    };
    auto mma_with = [&](const u32x4_t (&bf)[4], f32x4_t (&acc)[kATiles]) {
#pragma unroll
      for (int a = 0; a < kATiles; ++a) acc[a] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
#pragma unroll
        for (int a = 0; a < kATiles; ++a) acc[a] = mfma16(af[a][kc], bf[kc], acc[a]);
    };
    auto mma = [&](int d, f32x4_t (&acc)[kATiles]) {
      u32x4_t bf[4];
      frag(d, bf);
      mma_with(bf, acc);
    };

    u32x4_t cur[kStage];
#pragma unroll
    for (int k = 0; k < kStage; ++k) cur[k] = gload(c_begin, k);
    int pb = 0;                        // code buffer of this phase
    for (int c0 = c_begin; c0 < c_end; c0 += kScoreGroup * kPhase) {
      __syncthreads();                 // the previous phase is done with kv[] and cbuf[pb]
#pragma unroll
      for (int k = 0; k < kStage; ++k) {
        const int i = tid + kST * k;
        *reinterpret_cast<u32x4_t*>(&kv[i >> 8][((i >> 4) & 15) * kLdsRow + (i & 15) * 8]) = cur[k];
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kStage; ++k) cur[k] = gload(c0 + kScoreGroup * kPhase, k);
      if (c0 > c_begin) flush(c0 - kScoreGroup * kPhase, pb ^ 1);

      // software pipeline over the phase's groups: the MFMAs of group d+1 are issued
      // before the epilogue of group d, which they do not depend on
      uint16_t* cw0 = &cbuf[pb][(kQW * w + (lane >> 4)) * kCodeRow + (lane & 15)];
      f32x4_t acc0[kATiles], acc1[kATiles];
      if (c0 + kScoreGroup * kPhase <= wave_min_nc) {
        // every block of the phase is visible to every query of the wave: straight-line
        // code, one MFMA interleaved with a few VALU instructions of the previous epilogue
        auto epi = [&](int d, const f32x4_t (&acc)[kATiles]) {
#pragma unroll
          for (int a = 0; a < kATiles; ++a)
            cw0[4 * a * kCodeRow + kScoreGroup * d] = (uint16_t)score_code(head_mix(acc[a], wt[a]));
        };
        auto interleave = [&]() {
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // next group's B fragment reads
#pragma unroll
          for (int i = 0; i < 4 * kATiles; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0); // a few VALU
          }
          __builtin_amdgcn_sched_group_barrier(0x200, kATiles, 0);   // code writes to LDS
        };
        // B fragments are read one group ahead of their MFMAs
        u32x4_t bfa[4], bfb[4];
        frag(0, bfa);
        frag(1, bfb);
        mma_with(bfa, acc0);
#pragma unroll
        for (int d = 0; d < kPhase; d += 2) {
          if (d + 2 < kPhase) frag(d + 2, bfa);
          mma_with(bfb, acc1);
          epi(d, acc0);
          interleave();
          if (d + 3 < kPhase) frag(d + 3, bfb);
          if (d + 2 < kPhase) mma_with(bfa, acc0);
          epi(d + 1, acc1);
          if (d + 2 < kPhase) interleave();
        }
      } else {
        const int ng = min(kPhase, (c_end - c0 + kScoreGroup - 1) / kScoreGroup);
        auto epi = [&](int d, const f32x4_t (&acc)[kATiles]) {
          const int c = c0 + kScoreGroup * d + (lane & 15);
#pragma unroll
          for (int a = 0; a < kATiles; ++a)
            cw0[4 * a * kCodeRow + kScoreGroup * d] =
                c < st_nc[a] ? (uint16_t)score_code(head_mix(acc[a], wt[a])) : (uint16_t)0;
        };
        mma(0, acc0);
#pragma unroll
        for (int d = 0; d < kPhase; d += 2) {
          if (ng > d + 1) mma(d + 1, acc1);
          if (ng > d) epi(d, acc0);
          if (ng > d + 2) mma(d + 2, acc0);
          if (ng > d + 1) epi(d + 1, acc1);
        }
      }
      pb ^= 1;
    }
    __syncthreads();
    flush(c_begin + ((n_here - 1) / (kScoreGroup * kPhase)) * (kScoreGroup * kPhase), pb ^ 1);
    __syncthreads();                   // the next request reuses rows[], kv[] and cbuf[]
  }
}

// ------------------------------------------------------------------ top-512 over codes

constexpr int kTT = 256;               // threads per row
constexpr int kTW = kTT / 64;
constexpr int kEnt = 32;               // entries per thread (register-held)
constexpr int kRowCap = kTT * kEnt;    // rows of at most 8192 blocks are read whole
constexpr int kListCap = 1024;         // LDS candidates of the longer rows (about 600 typical)
static_assert(kListCap % kTT == 0, "the list is read back as kListCap / kTT entries per thread");
constexpr int kTieCap = 256;           // blocks sharing the threshold code (a few dozen typical)
constexpr int kWords = kMaxBlocks / 32;
constexpr int kWordsPerThread = kWords / kTT;   // 8
constexpr int kCandPass = 3;          // candidate groups per thread per load pass

struct __attribute__((aligned(16))) SmemC {
  uint32_t red[2 * kTW];
  int wsum[kTW];
  uint32_t hist[2][256];
  uint32_t list[kListCap];             // (code << 16) | block
  uint32_t tie_key[kTieCap];
  uint16_t tie_idx[kTieCap];
  uint32_t bits[kWords];
  int misc[8];
};

__shared__ SmemC sc;

__device__ __forceinline__ int2 block_scan256(int v) {
  const int w = threadIdx.x >> 6;
  const int inc = wave_inclusive_sum(v);
  if ((threadIdx.x & 63) == 63) sc.wsum[w] = inc;
  __syncthreads();
  const int4 x = *reinterpret_cast<const int4*>(sc.wsum);
  const int xs[4] = {x.x, x.y, x.z, x.w};
  int before = 0;
#pragma unroll
  for (int j = 0; j < kTW; ++j) before += j < w ? xs[j] : 0;
  __syncthreads();
  return make_int2(before + inc - v, x.x + x.y + x.z + x.w);
}

// Wave 0 finds the bin of the kk-th largest in hist[buf]: misc[0] = bin, misc[1] =
// rank inside it, misc[2] = its count.  The other waves clear hist[buf ^ 1].
__device__ __forceinline__ void find_bin(int buf, int kk) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    const uint4 h = reinterpret_cast<const uint4*>(sc.hist[buf])[tid];
    const int mine = (int)(h.x + h.y + h.z + h.w);
    const int inc = wave_inclusive_sum(mine);
    const int above = __builtin_amdgcn_readlane(inc, 63) - inc;
    if (above < kk && kk <= above + mine) {
      const int a3 = above + (int)h.w, a2 = a3 + (int)h.z, a1 = a2 + (int)h.y;
      int d, r, cnt;
      if (kk <= a3) { d = 3; r = kk - above; cnt = h.w; }
      else if (kk <= a2) { d = 2; r = kk - a3; cnt = h.z; }
      else if (kk <= a1) { d = 1; r = kk - a2; cnt = h.y; }
      else { d = 0; r = kk - a1; cnt = h.x; }
      sc.misc[0] = 4 * tid + d;
      sc.misc[1] = r;
      sc.misc[2] = cnt;
    }
  } else {
    sc.hist[buf ^ 1][tid - 64] = 0u;   // 192 threads clear 256 bins
    if (tid < 128) sc.hist[buf ^ 1][tid + 128] = 0u;
  }
}

// kk-th largest 16-bit value among the non-zero values (v[] >> kShift) of the work
// group.  Returns (value T, how many entries equal to T are kept, how many entries
// equal T).  kShift = 16 reads the codes of packed (code << 16 | block) entries.
template <int E, int kShift = 0>
__device__ __forceinline__ int3 select16(const uint32_t (&v)[E], int kk) {
  const int tid = threadIdx.x, w = tid >> 6;
  uint32_t mx = 0u, mn = 0xffffu;
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint32_t x = v[e] >> kShift;
    mx = max(mx, x);
    mn = min(mn, x ? x : 0xffffu);
    cnt += x ? 1 : 0;
  }
  mx = wave_max_u32(mx);
  mn = wave_min_u32(mn);
  if ((tid & 63) == 0) {
    sc.red[w] = mx;
    sc.red[kTW + w] = mn;
  }
  sc.hist[0][tid] = 0u;
  const int total = block_scan256(cnt).y;   // (its barriers also publish red[])
  {
    const uint4 a = *reinterpret_cast<const uint4*>(sc.red);
    const uint4 b = *reinterpret_cast<const uint4*>(sc.red + kTW);
    mx = max(max(a.x, a.y), max(a.z, a.w));
    mn = min(min(b.x, b.y), min(b.z, b.w));
  }
  if (mx == mn) return make_int3((int)mx, kk, total);
  int hi = 31 - __clz(mx ^ mn);
  uint32_t prefix = mx & ~((2u << hi) - 1u);   // bits above hi, shared by all values
  int buf = 0, count = 0;
  while (hi >= 0) {
    const int lo = max(hi - 7, 0);
    const uint32_t pmask = ~((2u << hi) - 1u);
    const uint32_t dmask = (1u << (hi - lo + 1)) - 1u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t x = v[e] >> kShift;
      if (x && (x & pmask) == prefix) atomicAdd(&sc.hist[buf][(x >> lo) & dmask], 1u);
    }
    __syncthreads();
    find_bin(buf, kk);
    __syncthreads();
    prefix |= (uint32_t)sc.misc[0] << lo;
    kk = sc.misc[1];
    count = sc.misc[2];
    buf ^= 1;
    hi = lo - 1;
  }
  return make_int3((int)prefix, kk, count);
}

__device__ __forceinline__ void mark(int c) { atomicOr(&sc.bits[c >> 5], 1u << (c & 31)); }

__device__ __forceinline__ void queue_row(int* queue, int t) {
  if (threadIdx.x == 0) queue[1 + atomicAdd(queue, 1)] = t;
}

// Six rows per CU (16 KB of LDS, at most 80 VGPRs each).  The register cap spills a
// few values that live across the whole row to scratch; that is still faster than
// five or four rows per CU without spills (81 against 88 us on the 4096-row chunk).
__global__ void __launch_bounds__(kTT, 6)
topk_codes_kernel(const uint16_t* __restrict__ codes, const uint16_t* __restrict__ gmax, int stride,
                  const int32_t* __restrict__ q_req, const int32_t* __restrict__ q_pos,
                  const uint16_t* __restrict__ idx_q, const float* __restrict__ idx_w,
                  const int32_t* __restrict__ page_table, int pt_stride, int page_size,
                  const uint16_t* __restrict__ comp, int32_t* __restrict__ sel_blocks,
                  int32_t* __restrict__ sel_pos, int sel_stride, int32_t* __restrict__ sel_count,
                  int* __restrict__ queue) {
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int p = q_pos[t];
  const int n = (p + 1) / kBlock;
  QSA_CHECK(p >= 0 && n <= stride);
  const int pend = (p + 1) % kBlock;
  int32_t* row_b = sel_blocks + (size_t)t * kTopK;
  int32_t* row_p = sel_pos + (size_t)t * sel_stride;

  if (n <= kTopK) {
    for (int i = tid; i < kTopK; i += kTT) row_b[i] = i < n ? i : -1;
    for (int i = tid; i < sel_stride; i += kTT) row_p[i] = i <= p ? i : -1;
    if (tid == 0) sel_count[t] = p + 1;
    return;
  }

  const uint16_t* crow = codes + (size_t)t * stride;
  const int nwords = (n + 31) / 32;
  const int w0 = kWordsPerThread * tid;
  if (tid == 0) {
    sc.misc[4] = 0;                    // list length
    sc.misc[5] = 0;                    // tie count
  }

  // ---- from the entries (code << 16 | block) of this thread, E per thread: the
  // threshold, the kept blocks and the expanded output
  auto finish = [&](auto& ent) {
    constexpr int E = (int)(sizeof(ent) / sizeof(ent[0]));
    // the bitmap (the candidate groups' scratch above) starts empty
#pragma unroll
    for (int i = 0; i < kWordsPerThread; ++i) sc.bits[w0 + i] = 0u;

    // ---- the 512th largest code T: codes above it are kept; of the cnt entries equal
    // to T, `need` are kept, ranked by exact score
    const int3 sel = select16<E, 16>(ent, kTopK);
    const uint32_t T = (uint32_t)sel.x;
    const int need = sel.y, cnt = sel.z;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t cve = ent[e] >> 16;
      if (!ent[e] || cve < T) continue;
      const int c = (int)(ent[e] & 0xffffu);
      if (cve > T || need == cnt) {
        mark(c);
      } else {
        const int slot = atomicAdd(&sc.misc[5], 1);
        if (slot < kTieCap) sc.tie_idx[slot] = (uint16_t)c;
      }
    }
    __syncthreads();
    if (need != cnt) {
      // the tied entries written above number cnt whenever the codes and maxima come
      // from one scorer pass; otherwise (or beyond the tie buffer) the FP32 path takes
      // the row
      if (cnt > kTieCap || sc.misc[5] != cnt) {
        queue_row(queue, t);
        return;
      }
      // exact scores of the tied blocks (same MFMA arithmetic as the scorer)
      const int lane = tid & 63, w = tid >> 6;
      const int bpp = page_size / kBlock;
      const int32_t* pt_row = page_table + (size_t)q_req[t] * pt_stride;
      u32x4_t af[4];
      query_rows(idx_q, t, af);
      float wq[kIdxHeads];
#pragma unroll
      for (int h = 0; h < kIdxHeads; ++h) wq[h] = idx_w[(size_t)t * kIdxHeads + h];
      for (int j0 = 16 * w; j0 < cnt; j0 += 16 * kTW) {
        const int j = j0 + (lane & 15);
        const int c = min((int)sc.tie_idx[min(j, cnt - 1)], n - 1);
        const float s = score16(af, comp + comp_row(pt_row, c, bpp) * kIdxDim, wq);
        if (lane < 16 && j < cnt) sc.tie_key[j] = float_key(s);
      }
      __syncthreads();
      // rank: higher score first, then lower block index
      for (int j = tid; j < cnt; j += kTT) {
        const uint32_t kj = sc.tie_key[j];
        const int ij = sc.tie_idx[j];
        int rank = 0;
        for (int i = 0; i < cnt; ++i) {
          const uint32_t ki = sc.tie_key[i];
          rank += (ki > kj || (ki == kj && sc.tie_idx[i] < ij)) ? 1 : 0;
        }
        if (rank < need) mark(ij);
      }
      __syncthreads();
    }

    // ---- emit the kept blocks in index order, each expanded to its 4 positions
    {
      uint32_t wv[kWordsPerThread];
      int k = 0;
#pragma unroll
      for (int i = 0; i < kWordsPerThread; ++i) {
        wv[i] = w0 + i < nwords ? sc.bits[w0 + i] : 0u;
        k += __popc(wv[i]);
      }
      int idx = block_scan256(k).x;
#pragma unroll
      for (int i = 0; i < kWordsPerThread; ++i)
        for (uint32_t e = wv[i]; e; e &= e - 1) {
          const int c = 32 * (w0 + i) + __ffs(e) - 1;
          if (idx < kTopK) {             // exactly kTopK bits are set; the guard bounds the row
            row_b[idx] = c;
            *reinterpret_cast<int4*>(row_p + kBlock * idx) = make_int4(4 * c, 4 * c + 1, 4 * c + 2, 4 * c + 3);
          }
          ++idx;
        }
    }
    const int base = kBlock * kTopK;
    for (int i = base + tid; i < sel_stride; i += kTT) {
      const int k = i - base;
      row_p[i] = k < pend ? kBlock * n + k : -1;
    }
    if (tid == 0) sel_count[t] = base + pend;
  };

  // ---- entries (code << 16 | block): the whole row, or the blocks of the groups
  // whose maximum reaches the 512th largest group maximum (at least 512 blocks of
  // the row reach that value, so the 512 best are among them)
  if (n <= kRowCap) {
    uint32_t ent[kEnt];
#pragma unroll
    for (int e = 0; e < kEnt / 8; ++e) {
      const int ch = tid + kTT * e;
      const u32x4_t v = 8 * ch < n ? ld16(crow + 8 * ch) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = 8 * ch + i;
        const uint32_t code = (v[i / 2] >> (16 * (i & 1))) & 0xffffu;
        ent[8 * e + i] = c < n ? (code << 16) | (uint32_t)c : 0u;
      }
    }
    finish(ent);
  } else {
    const int ng = (n + kScoreGroup - 1) / kScoreGroup;   // <= 4096
    const uint16_t* grow = gmax + (size_t)t * (stride / kScoreGroup);
    uint32_t gk[16];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int ch = tid + kTT * e;
      const u32x4_t v = 8 * ch < ng ? ld16(grow + 8 * ch) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i)
        gk[8 * e + i] = 8 * ch + i < ng ? (v[i / 2] >> (16 * (i & 1))) & 0xffffu : 0u;
    }
    const uint32_t gstar = (uint32_t)select16<16>(gk, kTopK).x;
    // compact the candidate groups (maximum >= gstar) into the bitmap words, which
    // are cleared only after the list is built
    uint16_t* cand = reinterpret_cast<uint16_t*>(sc.bits);   // room for kWords * 2 >= 4096
    int nmine = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) nmine += gk[j] >= gstar ? 1 : 0;   // gk = 0 is never >= gstar > 0
    const int2 cs = block_scan256(nmine);
    {
      int slot = cs.x;
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (gk[8 * e + i] >= gstar) cand[slot++] = (uint16_t)(8 * (tid + kTT * e) + i);
    }
    __syncthreads();
    const int ncand = cs.y;
    // every candidate's codes are requested before any is used: kCandPass groups per
    // thread per pass; list slots come from a wave prefix count and one atomic per wave
    for (int j0 = 0; j0 < ncand; j0 += kCandPass * kTT) {
      u32x4_t a[kCandPass], b[kCandPass];
      int gg[kCandPass];
#pragma unroll
      for (int r = 0; r < kCandPass; ++r) {
        const int j = j0 + kTT * r + tid;
        gg[r] = j < ncand ? (int)cand[j] : -1;
        const uint16_t* src = crow + kScoreGroup * max(gg[r], 0);
        a[r] = gg[r] >= 0 ? ld16(src) : u32x4_t{0u, 0u, 0u, 0u};
        b[r] = gg[r] >= 0 ? ld16(src + 8) : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int r = 0; r < kCandPass; ++r) {
        uint32_t keep[16];
        int k = 0;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const uint32_t word = jj < 8 ? a[r][jj / 2] : b[r][(jj - 8) / 2];
          const uint32_t code = (word >> (16 * (jj & 1))) & 0xffffu;
          const int c = kScoreGroup * gg[r] + jj;
          keep[jj] = (gg[r] >= 0 && c < n && code >= gstar) ? (code << 16) | (uint32_t)c : 0u;
          k += keep[jj] ? 1 : 0;
        }
        const int incl = wave_inclusive_sum(k);
        const int wtot = __builtin_amdgcn_readlane(incl, 63);
        int base = 0;
        if ((tid & 63) == 63 && wtot > 0) base = atomicAdd(&sc.misc[4], wtot);
        int slot = __builtin_amdgcn_readlane(base, 63) + incl - k;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj)
          if (keep[jj]) {
            if (slot < kListCap) sc.list[slot] = keep[jj];
            ++slot;
          }
      }
    }
    __syncthreads();
    const int len = sc.misc[4];
    // heavy ties (more candidates than the list holds), or fewer than 512 candidates
    // (maxima that do not match the codes): the FP32 path takes the row
    if (len > kListCap || len < kTopK) {
      queue_row(queue, t);
      return;
    }
    uint32_t ent[kListCap / kTT];
#pragma unroll
    for (int e = 0; e < kListCap / kTT; ++e) {
      const int i = tid + kTT * e;
      ent[e] = i < len ? sc.list[i] : 0u;
    }
    finish(ent);
  }
}

// Exact FP32 scores of the queued rows (into the FP32 score rows of the workspace,
// which alias the codes: every code has been read by now).
__global__ void __launch_bounds__(256)
rescore_kernel(const int* __restrict__ queue, const int32_t* __restrict__ q_req,
               const int32_t* __restrict__ q_pos, const uint16_t* __restrict__ idx_q,
               const float* __restrict__ idx_w, const int32_t* __restrict__ page_table,
               int pt_stride, int page_size, const uint16_t* __restrict__ comp,
               float* __restrict__ scores, int stride) {
  const int nq = queue[0];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int bpp = page_size / kBlock;
  for (int k = blockIdx.x; k < nq; k += gridDim.x) {
    const int t = queue[1 + k];
    const int n = (q_pos[t] + 1) / kBlock;
    const int32_t* pt_row = page_table + (size_t)q_req[t] * pt_stride;
    u32x4_t af[4];
    query_rows(idx_q, t, af);
    float wq[kIdxHeads];
#pragma unroll
    for (int h = 0; h < kIdxHeads; ++h) wq[h] = idx_w[(size_t)t * kIdxHeads + h];
    for (int c0 = kScoreGroup * w; c0 < n; c0 += kScoreGroup * 4) {
      const int c = c0 + (lane & 15);
      const float s = score16(af, comp + comp_row(pt_row, min(c, n - 1), bpp) * kIdxDim, wq);
      if (lane < 16 && c < n) scores[(size_t)t * stride + c] = s;
    }
  }
}

}  // namespace

hipError_t launch_index_mfma(const IndexArgs& a, hipStream_t stream) {
  const int n_ranges = (a.max_pos / kBlock + kPfRange - 1) / kPfRange;
  const int n_tiles = (a.total_q + kPfQ - 1) / kPfQ;
  QSA_LAUNCH(score_mfma_kernel, dim3(n_ranges * n_tiles), dim3(kST), 0, stream, a.total_q,
                     a.idx_q, a.idx_w, a.q_req, a.q_pos, a.page_table, a.pt_stride, a.page_size,
                     a.comp, a.codes, a.gmax, a.score_stride, n_ranges, n_tiles, a.queue);
  QSA_LAUNCH(topk_codes_kernel, dim3(a.total_q), dim3(kTT), 0, stream, a.codes, a.gmax,
                     a.score_stride, a.q_req, a.q_pos, a.idx_q, a.idx_w, a.page_table, a.pt_stride,
                     a.page_size, a.comp, a.sel_blocks, a.sel_pos, a.sel_stride, a.sel_count, a.queue);
  const int g = std::min(a.total_q, 256);
  QSA_LAUNCH(rescore_kernel, dim3(g), dim3(256), 0, stream, a.queue, a.q_req, a.q_pos,
                     a.idx_q, a.idx_w, a.page_table, a.pt_stride, a.page_size, a.comp, a.scores,
                     a.score_stride);
  launch_topk_queued(a, stream);
  return hipGetLastError();
}

}  // namespace qsa
