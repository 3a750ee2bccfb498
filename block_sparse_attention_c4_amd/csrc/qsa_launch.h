// Internal launch interface between the C ABI (qsa_api.cpp) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// Every kernel launch of the library.  When the calling thread asked for kernel
// timing, the launch takes the next (start, stop) event pair, which the runtime sets
// from the dispatch's own start and end timestamps.
#define QSA_LAUNCH(kernel, grid, block, shmem, stream, ...)                                  \
  do {                                                                                       \
    hipEvent_t qsa_ev0_ = nullptr, qsa_ev1_ = nullptr;                                       \
    ::qsa::launch_events(&qsa_ev0_, &qsa_ev1_);                                              \
    if (qsa_ev0_ != nullptr)                                                                 \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, qsa_ev0_, qsa_ev1_, 0u,      \
                            __VA_ARGS__);                                                    \
    else                                                                                     \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                   \
  } while (0)

namespace qsa {

// Start and stop events for the next kernel launch, when the calling thread asked for
// kernel timing (qsa_profile_kernel_events) and pairs are left; both null otherwise.
void launch_events(hipEvent_t* start, hipEvent_t* stop);

struct RopeTable {
  double inv_freq[64];   // theta^(-2i/128), i < 64
  uint8_t axis[64];      // MRoPE: position component (0 t, 1 h, 2 w) that turns pair i
};

struct BuildArgs {
  int batch, max_new, page_size, pt_stride;
  float theta;
  const uint16_t* new_k;
  const int32_t* cu_new;
  const int32_t* len_before;
  const int32_t* page_table;
  uint16_t* ring;
  uint16_t* comp;
  const int32_t* new_mpos;   // [total_new, 3] 3-D positions, or NULL: 1-D RoPE at 4c
  int32_t* ring_mpos;        // [batch, 4, 3] positions of the ring's tokens (MRoPE only)
  const uint8_t* pair_axis;  // host [64] (MRoPE only)
};
hipError_t launch_build(const BuildArgs& a, hipStream_t stream);

struct IndexArgs {
  int batch, total_q, max_pos, page_size, pt_stride, sel_stride;
  const uint16_t* idx_q;
  const float* idx_w;
  const int32_t* q_req;
  const int32_t* q_pos;
  const int32_t* page_table;
  const uint16_t* comp;
  int32_t* sel_blocks;
  int32_t* sel_pos;
  int32_t* sel_count;
  // workspace
  float* scores;       // [total_q, score_stride] FP32 scores
  float* gmax_f;       // [total_q, score_stride / 16] their 16-block group maxima
  uint16_t* codes;     // [total_q, score_stride] score codes (aliases scores)
  uint16_t* gmax;      // [total_q, score_stride / 16] group maxima of the codes (aliases scores)
  int* queue;          // [1 + total_q]: count, then rows handed to the FP32 select
  int score_stride;    // multiple of 128, >= max_pos / 4
};
size_t index_workspace_bytes(int total_q, int max_pos);
void index_workspace_carve(IndexArgs& a, void* ws);
hipError_t launch_index(const IndexArgs& a, hipStream_t stream);
// Decode step whose queries' own tokens are ingested by the scorer launch: query t
// is request t, its token sits at q_pos[t] (q_req unused).
struct IngestArgs {
  const uint16_t* new_k;     // [total_q, 128] raw indexer keys of the queries' tokens
  uint16_t* ring;            // [total_q, 4, 128]
  uint16_t* comp;            // the compressed key cache (same memory as IndexArgs::comp)
  float theta;
  const int32_t* new_mpos;   // [total_q, 3] MRoPE positions of the tokens, or NULL (1-D RoPE)
  int32_t* ring_mpos;        // [total_q, 4, 3] (MRoPE only)
  const uint8_t* pair_axis;  // host [64] (MRoPE only)
};
hipError_t launch_index_ingest(const IndexArgs& a, const IngestArgs& f, hipStream_t stream);
hipError_t launch_index_mfma(const IndexArgs& a, hipStream_t stream);
void launch_topk(const IndexArgs& a, hipStream_t stream);
void launch_topk_queued(const IndexArgs& a, hipStream_t stream);

struct AttnArgs {
  int total_q, page_size, pt_stride, sel_stride, n_extra;
  float sm_scale;
  const uint16_t* q;
  const int32_t* q_req;      // NULL: query t reads request t
  const void* k_pool;         // bf16, or FP8 E4M3 codes when fp8
  const void* v_pool;
  bool fp8;
  float k_scale, v_scale;     // FP8 pools: a code stands for e4m3(code) * scale
  const int32_t* page_table;
  const int32_t* sel_pos;
  const int32_t* sel_count;
  const int32_t* extra_pos;  // may be NULL
  uint16_t* out;
  float* lse;                // may be NULL
  // workspace (split partials)
  float* part;               // [total_q, kv, splits, 8 + 8 + 8*256]
  int splits;
  int split_len;             // positions of the longest split (multiple of 32)
};
void attn_plan(int total_q, int n_extra, int* splits, int* split_len);
size_t attn_workspace_bytes(int total_q, int n_extra);
// Static scratch of the allocation-free decode call: its size, and its device
// address on the current GPU (looked up once per device).
constexpr size_t kAttnScratchBytes = size_t(8) << 20;
hipError_t attn_scratch(void** ptr);
hipError_t launch_attn(const AttnArgs& a, hipStream_t stream);

}  // namespace qsa
