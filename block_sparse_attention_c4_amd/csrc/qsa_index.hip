// Stage 2a: indexer block scores (decode).
//
// [SGLang day-0 post on Qwen3.8-Flash-Next, section "Qwen Sparse Attention:
// Retrieve Coarsely, Attend Precisely"]: a query scores every visible compressed
// block.  The scoring formula is cut off on the page; the kernels compute
// s_c = sum_h w_h * max(0, q_h . k_c) over the 4 indexer heads.
//
// score_kernel is a paged GEMV.  A wave streams groups of 16 consecutive blocks
// (one 4 KB compressed page when page_size = 64): 4 loads of 16 B per lane, each
// load covering 4 blocks x 256 B contiguous.  Lane l owns dims (l%16)*8 .. +8 of
// block (l/16); the dot products use v_dot2_f32_bf16 (bf16 pairs, FP32
// accumulation) and are summed over the 16 lanes of a row with DPP.  Top-512
// selection and expansion live in qsa_topk.hip.
#include "qsa_device.h"
#include "qsa_launch.h"

namespace qsa {

namespace {


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

// One wave per work group.  The (at most 64) queries of a launch are laid out one
// per lane: each lane holds its query's group count, first group, request and
// block count, and a group index is mapped to its query with one ballot.  The
// wave takes a contiguous range of the launch's groups and keeps two groups'
// loads in flight while it computes the previous one.
struct GroupLoad {
  u32x4_t kv[4];
  int t, g;
};

__global__ void __launch_bounds__(64)
score_kernel(int nq, const uint16_t* __restrict__ idx_q, const float* __restrict__ idx_w,
             const int32_t* __restrict__ q_req, const int32_t* __restrict__ q_pos,
             const int32_t* __restrict__ page_table, int pt_stride, int page_size,
             const uint16_t* __restrict__ comp, float* __restrict__ scores, int score_stride) {
  const int lane = threadIdx.x;
  const int my_nc = lane < nq ? (q_pos[lane] + 1) / kBlock : 0;
  const int my_req = lane < nq ? q_req[lane] : 0;
  const int my_groups = (my_nc + kScoreGroup - 1) / kScoreGroup;
  int incl = my_groups;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(incl, d, 64);
    if (lane >= d) incl += u;
  }
  const int excl = incl - my_groups;
  const int total = __shfl(incl, 63, 64);
  const int wave = blockIdx.x, nwaves = gridDim.x;
  const int g_begin = (int)(((int64_t)total * wave) / nwaves);
  const int g_end = (int)(((int64_t)total * (wave + 1)) / nwaves);
  if (g_begin >= g_end) return;

  const int d0 = (lane & 15) * 8;
  const int row_in_step = lane >> 4;
  const int bpp = page_size / kBlock;

  auto issue = [&](GroupLoad& L, int gi) {
    const int t = __popcll(__ballot(incl <= gi));   // first query whose groups reach gi
    L.t = t;
    L.g = gi - __shfl(excl, t, 64);
    const int n_c = __shfl(my_nc, t, 64);
    const int32_t* pt_row = page_table + (size_t)__shfl(my_req, t, 64) * pt_stride;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = min(L.g * kScoreGroup + 4 * r + row_in_step, n_c - 1);
      const int64_t row = (int64_t)pt_row[c / bpp] * bpp + (c % bpp);
      L.kv[r] = ld16(comp + row * kIdxDim + d0);
    }
  };

  int cur_t = -1;
  u32x4_t qf[kIdxHeads];
  float w[kIdxHeads];
  auto compute = [&](const GroupLoad& L) {
    const int t = L.t;
    if (t != cur_t) {
      cur_t = t;
#pragma unroll
      for (int h = 0; h < kIdxHeads; ++h) {
        qf[h] = ld16(idx_q + ((size_t)t * kIdxHeads + h) * kIdxDim + d0);
        w[h] = idx_w[(size_t)t * kIdxHeads + h];
      }
    }
    const int n_c = __shfl(my_nc, t, 64);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float s = 0.f;
#pragma unroll
      for (int h = 0; h < kIdxHeads; ++h) {
        float a = dot2(L.kv[r].x, qf[h].x, 0.f);
        a = dot2(L.kv[r].y, qf[h].y, a);
        a = dot2(L.kv[r].z, qf[h].z, a);
        a = dot2(L.kv[r].w, qf[h].w, a);
        a = row16_sum(a);
        s += w[h] * fmaxf(a, 0.f);
      }
      const int c = L.g * kScoreGroup + 4 * r + row_in_step;
      if (c < n_c && (lane & 15) == 0) scores[(size_t)t * score_stride + c] = s;
    }
  };

  GroupLoad A, B;
  issue(A, g_begin);
  if (g_begin + 1 < g_end) issue(B, g_begin + 1);
  for (int gi = g_begin; gi < g_end; gi += 2) {
    compute(A);
    if (gi + 2 < g_end) issue(A, gi + 2);
    if (gi + 1 < g_end) {
      compute(B);
      if (gi + 3 < g_end) issue(B, gi + 3);
    }
  }
}

}  // namespace

// Workspace: FP32 score rows [total_q, stride]; the code rows and group maxima of
// the MFMA path live in the same bytes (the FP32 rows are written only after every
// code has been read).  Then the queue of rows handed to the FP32 select.
static size_t score_rows_bytes(int total_q, int max_pos, int* stride) {
  const int nb = (max_pos + kBlock - 1) / kBlock;
  *stride = ((nb + 127) / 128) * 128;
  return ((size_t)total_q * *stride * sizeof(float) + 255) / 256 * 256;
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
  a.codes = reinterpret_cast<uint16_t*>(base);
  a.gmax = a.codes + (size_t)a.total_q * a.score_stride;
  a.queue = reinterpret_cast<int*>(base + rows);
}

// Decode-like batches (about one query per request) take the paged GEMV scorer and
// the latency-oriented select; chunks of many queries per request share their keys
// and take the MFMA scorer.
static bool use_mfma(const IndexArgs& a) {
  return a.total_q >= 64 && a.total_q >= 4 * a.batch;
}

hipError_t launch_index(const IndexArgs& a, hipStream_t stream) {
  if (use_mfma(a)) return launch_index_mfma(a, stream);
  constexpr int kQPerLaunch = 64;
  for (int q0 = 0; q0 < a.total_q; q0 += kQPerLaunch) {
    const int nq = std::min(kQPerLaunch, a.total_q - q0);
    // the block counts are only known on the device: size the grid by the bound,
    // at most 16 waves per CU
    const int64_t groups_bound =
        (int64_t)nq * ((a.max_pos / kBlock + kScoreGroup - 1) / kScoreGroup);
    const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(groups_bound / 2, 4096));
    hipLaunchKernelGGL(score_kernel, dim3(grid), dim3(64), 0, stream, nq,
                       a.idx_q + (size_t)q0 * kIdxHeads * kIdxDim, a.idx_w + (size_t)q0 * kIdxHeads,
                       a.q_req + q0, a.q_pos + q0, a.page_table, a.pt_stride, a.page_size, a.comp,
                       a.scores + (size_t)q0 * a.score_stride, a.score_stride);
  }
  launch_topk(a, stream);
  return hipGetLastError();
}

}  // namespace qsa
