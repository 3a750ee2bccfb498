// C ABI of the QSA c4 hot path: argument checks, workspace carving, launches.
// The operations themselves are specified in include/qsa.h.
#include <cmath>
#include "qsa.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include "qsa_launch.h"

static_assert(qsa::kAttnScratchBytes == QSA_ATTN_SCRATCH_BYTES, "scratch size as declared in qsa.h");

namespace {

bool dims_supported(const qsa_dims* d) {
  return d->num_q_heads == 16 && d->num_kv_heads == 2 && d->head_dim == 256 &&
         d->idx_heads == 4 && d->idx_dim == 128 && d->page_size >= 16 && d->page_size % 16 == 0 &&
         d->rope_theta > 1.f && d->sm_scale > 0.f;
}

int check_dims(const qsa_dims* d) {
  if (!d) return QSA_E_NULL;
  return dims_supported(d) ? QSA_OK : QSA_E_UNSUPPORTED;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? QSA_OK : QSA_E_HIP; }

// (start, stop) HIP event pairs that the calling thread asked the next call to set
// for its kernels (qsa_profile_kernel_events).  A call's CallScope drops the request
// when the call returns, whether or not every pair was used.
constexpr int kMaxProfileEvents = 16;
struct ProfileEvents {
  hipEvent_t ev[kMaxProfileEvents];
  int n = 0, next = 0;
};
thread_local ProfileEvents t_profile;

struct CallScope {
  ~CallScope() { t_profile.n = t_profile.next = 0; }
};

}  // namespace

namespace qsa {
void launch_events(hipEvent_t* start, hipEvent_t* stop) {
  if (t_profile.next + 1 < t_profile.n) {
    *start = t_profile.ev[t_profile.next];
    *stop = t_profile.ev[t_profile.next + 1];
    t_profile.next += 2;
  } else {
    *start = *stop = nullptr;
  }
}
}  // namespace qsa

extern "C" {

const char* qsa_status_string(int status) {
  switch (status) {
    case QSA_OK: return "QSA_OK";
    case QSA_E_NULL: return "QSA_E_NULL: a required pointer is NULL";
    case QSA_E_SHAPE: return "QSA_E_SHAPE: a size or stride is out of range";
    case QSA_E_UNSUPPORTED: return "QSA_E_UNSUPPORTED: dims other than 16/2/256 heads, 4x128 indexer";
    case QSA_E_WORKSPACE: return "QSA_E_WORKSPACE: workspace missing, misaligned or too small";
    case QSA_E_HIP: return "QSA_E_HIP: a HIP launch failed";
    case QSA_E_SCRATCH:
      return "QSA_E_SCRATCH: the call needs more scratch than the library's static buffer holds";
    default: return "QSA: unknown status";
  }
}

int qsa_profile_kernel_events(void* const* events, int32_t n_events) {
  t_profile.n = t_profile.next = 0;   // a rejected request also cancels an earlier one
  if (n_events < 0 || n_events > kMaxProfileEvents || n_events % 2 != 0) return QSA_E_SHAPE;
  if (n_events > 0 && !events) return QSA_E_NULL;
  for (int i = 0; i < n_events; ++i)
    if (!events[i]) return QSA_E_NULL;
  for (int i = 0; i < n_events; ++i) t_profile.ev[i] = static_cast<hipEvent_t>(events[i]);
  t_profile.n = n_events;
  t_profile.next = 0;
  return QSA_OK;
}

size_t qsa_workspace_bytes(const qsa_dims* dims, int op, int32_t total_q, int32_t max_pos,
                           int32_t n_extra) {
  if (check_dims(dims) != QSA_OK || total_q < 0) return 0;
  switch (op) {
    case QSA_OP_INDEX_TOPK:
      if (max_pos < 1 || max_pos > QSA_MAX_CONTEXT) return 0;
      return qsa::index_workspace_bytes(total_q, max_pos);
    case QSA_OP_GQA_DECODE:
      if (n_extra < 0 || n_extra > QSA_MAX_EXTRA) return 0;
      return qsa::attn_workspace_bytes(total_q, n_extra);
    case QSA_OP_GQA_PREFILL:
      return qsa::attn_workspace_bytes(total_q, 0);
    default:
      return 0;
  }
}

static int build_common(const qsa_dims* dims, int32_t batch, const uint16_t* new_idx_k,
                        const int32_t* new_mpos, const int32_t* cu_new, const int32_t* len_before,
                        int32_t total_new, int32_t max_new, const int32_t* page_table,
                        int32_t pt_stride, const uint8_t* pair_axis, uint16_t* ring,
                        int32_t* ring_mpos, uint16_t* comp_cache, void* stream);

int qsa_build_index_keys(const qsa_dims* dims, int32_t batch, const uint16_t* new_idx_k,
                         const int32_t* cu_new, const int32_t* len_before, int32_t total_new,
                         int32_t max_new, const int32_t* page_table, int32_t pt_stride,
                         uint16_t* ring, uint16_t* comp_cache, void* stream) {
  return build_common(dims, batch, new_idx_k, nullptr, cu_new, len_before, total_new, max_new,
                      page_table, pt_stride, nullptr, ring, nullptr, comp_cache, stream);
}

int qsa_build_index_keys_mrope(const qsa_dims* dims, int32_t batch, const uint16_t* new_idx_k,
                               const int32_t* new_mpos, const int32_t* cu_new,
                               const int32_t* len_before, int32_t total_new, int32_t max_new,
                               const int32_t* page_table, int32_t pt_stride,
                               const uint8_t* pair_axis, uint16_t* ring, int32_t* ring_mpos,
                               uint16_t* comp_cache, void* stream) {
  CallScope scope;
  if (!pair_axis) return QSA_E_NULL;
  for (int i = 0; i < 64; ++i)
    if (pair_axis[i] > 2) return QSA_E_SHAPE;
  if (batch > 0 && total_new > 0 && (!new_mpos || !ring_mpos)) return QSA_E_NULL;
  return build_common(dims, batch, new_idx_k, new_mpos, cu_new, len_before, total_new, max_new,
                      page_table, pt_stride, pair_axis, ring, ring_mpos, comp_cache, stream);
}

static int build_common(const qsa_dims* dims, int32_t batch, const uint16_t* new_idx_k,
                        const int32_t* new_mpos, const int32_t* cu_new, const int32_t* len_before,
                        int32_t total_new, int32_t max_new, const int32_t* page_table,
                        int32_t pt_stride, const uint8_t* pair_axis, uint16_t* ring,
                        int32_t* ring_mpos, uint16_t* comp_cache, void* stream) {
  CallScope scope;
  int st = check_dims(dims);
  if (st != QSA_OK) return st;
  if (batch < 0 || total_new < 0 || max_new < 0 || max_new > total_new || pt_stride < 1 ||
      batch > 65535 || max_new > QSA_MAX_CONTEXT)
    return QSA_E_SHAPE;
  if (batch == 0 || total_new == 0) return QSA_OK;
  if (!new_idx_k || !cu_new || !len_before || !page_table || !ring || !comp_cache) return QSA_E_NULL;
  if (!aligned(new_idx_k, 8) || !aligned(ring, 8) || !aligned(comp_cache, 8)) return QSA_E_SHAPE;
  if (!aligned(new_mpos, 4) || !aligned(ring_mpos, 4)) return QSA_E_SHAPE;   // NULL passes
  qsa::BuildArgs a;
  a.batch = batch;
  a.max_new = max_new;
  a.page_size = dims->page_size;
  a.pt_stride = pt_stride;
  a.theta = dims->rope_theta;
  a.new_k = new_idx_k;
  a.cu_new = cu_new;
  a.len_before = len_before;
  a.page_table = page_table;
  a.ring = ring;
  a.comp = comp_cache;
  a.new_mpos = new_mpos;
  a.ring_mpos = ring_mpos;
  a.pair_axis = pair_axis;
  return hip_status(qsa::launch_build(a, static_cast<hipStream_t>(stream)));
}

int qsa_index_topk(const qsa_dims* dims, int32_t batch, int32_t total_q, const uint16_t* idx_q,
                   const float* idx_w, const int32_t* q_req, const int32_t* q_pos,
                   int32_t max_pos, const int32_t* page_table, int32_t pt_stride,
                   const uint16_t* comp_cache, int32_t* sel_blocks, int32_t* sel_pos,
                   int32_t sel_stride, int32_t* sel_count, void* workspace, size_t ws_bytes,
                   void* stream) {
  CallScope scope;
  int st = check_dims(dims);
  if (st != QSA_OK) return st;
  if (batch < 1 || total_q < 0 || max_pos < 1 || max_pos > QSA_MAX_CONTEXT || pt_stride < 1 ||
      sel_stride < QSA_MAX_SEL)
    return QSA_E_SHAPE;
  if (total_q == 0) return QSA_OK;
  if (!idx_q || !idx_w || !q_req || !q_pos || !page_table || !comp_cache || !sel_blocks ||
      !sel_pos || !sel_count)
    return QSA_E_NULL;
  if (!aligned(idx_q, 16) || !aligned(comp_cache, 16) || !aligned(sel_pos, 16) ||
      sel_stride % 4 != 0)
    return QSA_E_SHAPE;
  const size_t need = qsa::index_workspace_bytes(total_q, max_pos);
  if (!workspace || ws_bytes < need || !aligned(workspace, 256)) return QSA_E_WORKSPACE;
  qsa::IndexArgs a;
  a.batch = batch;
  a.total_q = total_q;
  a.max_pos = max_pos;
  a.page_size = dims->page_size;
  a.pt_stride = pt_stride;
  a.sel_stride = sel_stride;
  a.idx_q = idx_q;
  a.idx_w = idx_w;
  a.q_req = q_req;
  a.q_pos = q_pos;
  a.page_table = page_table;
  a.comp = comp_cache;
  a.sel_blocks = sel_blocks;
  a.sel_pos = sel_pos;
  a.sel_count = sel_count;
  qsa::index_workspace_carve(a, workspace);
  return hip_status(qsa::launch_index(a, static_cast<hipStream_t>(stream)));
}

static int decode_build_index_common(const qsa_dims* dims, int32_t batch,
                                     const uint16_t* new_idx_k, const int32_t* new_mpos,
                                     const int32_t* pos, int32_t max_pos, const int32_t* page_table,
                                     int32_t pt_stride, const uint8_t* pair_axis, uint16_t* ring,
                                     int32_t* ring_mpos, uint16_t* comp_cache, const uint16_t* idx_q,
                                     const float* idx_w, int32_t* sel_blocks, int32_t* sel_pos,
                                     int32_t sel_stride, int32_t* sel_count, void* workspace,
                                     size_t ws_bytes, void* stream) {
  CallScope scope;
  int st = check_dims(dims);
  if (st != QSA_OK) return st;
  if (batch < 1 || batch > 65535 || max_pos < 1 || max_pos > QSA_MAX_CONTEXT || pt_stride < 1 ||
      sel_stride < QSA_MAX_SEL)
    return QSA_E_SHAPE;
  if (!new_idx_k || !pos || !page_table || !ring || !comp_cache || !idx_q || !idx_w ||
      !sel_blocks || !sel_pos || !sel_count)
    return QSA_E_NULL;
  if (!aligned(new_idx_k, 8) || !aligned(ring, 8) || !aligned(idx_q, 16) ||
      !aligned(comp_cache, 16) || !aligned(sel_pos, 16) || sel_stride % 4 != 0 ||
      !aligned(new_mpos, 4) || !aligned(ring_mpos, 4))   // NULL passes
    return QSA_E_SHAPE;
  const size_t need = qsa::index_workspace_bytes(batch, max_pos);
  if (!workspace || ws_bytes < need || !aligned(workspace, 256)) return QSA_E_WORKSPACE;
  qsa::IndexArgs a;
  a.batch = batch;
  a.total_q = batch;
  a.max_pos = max_pos;
  a.page_size = dims->page_size;
  a.pt_stride = pt_stride;
  a.sel_stride = sel_stride;
  a.idx_q = idx_q;
  a.idx_w = idx_w;
  a.q_req = nullptr;
  a.q_pos = pos;
  a.page_table = page_table;
  a.comp = comp_cache;
  a.sel_blocks = sel_blocks;
  a.sel_pos = sel_pos;
  a.sel_count = sel_count;
  qsa::index_workspace_carve(a, workspace);
  qsa::IngestArgs f;
  f.new_k = new_idx_k;
  f.ring = ring;
  f.comp = comp_cache;
  f.theta = dims->rope_theta;
  f.new_mpos = new_mpos;
  f.ring_mpos = ring_mpos;
  f.pair_axis = pair_axis;
  return hip_status(qsa::launch_index_ingest(a, f, static_cast<hipStream_t>(stream)));
}

int qsa_decode_build_index_topk(const qsa_dims* dims, int32_t batch, const uint16_t* new_idx_k,
                                const int32_t* pos, int32_t max_pos, const int32_t* page_table,
                                int32_t pt_stride, uint16_t* ring, uint16_t* comp_cache,
                                const uint16_t* idx_q, const float* idx_w, int32_t* sel_blocks,
                                int32_t* sel_pos, int32_t sel_stride, int32_t* sel_count,
                                void* workspace, size_t ws_bytes, void* stream) {
  return decode_build_index_common(dims, batch, new_idx_k, nullptr, pos, max_pos, page_table,
                                   pt_stride, nullptr, ring, nullptr, comp_cache, idx_q, idx_w,
                                   sel_blocks, sel_pos, sel_stride, sel_count, workspace, ws_bytes,
                                   stream);
}

int qsa_decode_build_index_topk_mrope(const qsa_dims* dims, int32_t batch,
                                      const uint16_t* new_idx_k, const int32_t* new_mpos,
                                      const int32_t* pos, int32_t max_pos,
                                      const int32_t* page_table, int32_t pt_stride,
                                      const uint8_t* pair_axis, uint16_t* ring, int32_t* ring_mpos,
                                      uint16_t* comp_cache, const uint16_t* idx_q,
                                      const float* idx_w, int32_t* sel_blocks, int32_t* sel_pos,
                                      int32_t sel_stride, int32_t* sel_count, void* workspace,
                                      size_t ws_bytes, void* stream) {
  CallScope scope;
  if (!pair_axis || !new_mpos || !ring_mpos) return QSA_E_NULL;
  for (int i = 0; i < 64; ++i)
    if (pair_axis[i] > 2) return QSA_E_SHAPE;
  return decode_build_index_common(dims, batch, new_idx_k, new_mpos, pos, max_pos, page_table,
                                   pt_stride, pair_axis, ring, ring_mpos, comp_cache, idx_q, idx_w,
                                   sel_blocks, sel_pos, sel_stride, sel_count, workspace, ws_bytes,
                                   stream);
}

// fp8: the pools hold E4M3 codes scaled by k_scale / v_scale (finite and > 0).
// static_scratch: the split partials go to the library's static device array instead
// of the caller's workspace (workspace and ws_bytes are ignored).
static int gqa_common(const qsa_dims* dims, int32_t total_q, const uint16_t* q,
                      const int32_t* q_req, const void* k_pool, const void* v_pool, bool fp8,
                      float k_scale, float v_scale, const int32_t* page_table, int32_t pt_stride,
                      const int32_t* sel_pos, const int32_t* sel_count, int32_t sel_stride,
                      const int32_t* extra_pos, int32_t n_extra, uint16_t* out, float* lse,
                      void* workspace, size_t ws_bytes, void* stream,
                      bool static_scratch = false) {
  CallScope scope;
  int st = check_dims(dims);
  if (st != QSA_OK) return st;
  if (fp8 && !(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return QSA_E_SHAPE;
  if (total_q < 0 || pt_stride < 1 || sel_stride < 1 || n_extra < 0 || n_extra > QSA_MAX_EXTRA ||
      total_q > (1 << 24))
    return QSA_E_SHAPE;
  if (total_q == 0) return QSA_OK;
  if (!q || !k_pool || !v_pool || !page_table || !sel_pos || !sel_count || !out) return QSA_E_NULL;
  if (n_extra > 0 && !extra_pos) return QSA_E_NULL;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16))
    return QSA_E_SHAPE;
  const size_t need = qsa::attn_workspace_bytes(total_q, n_extra);
  if (static_scratch) {
    if (need > qsa::kAttnScratchBytes) return QSA_E_SCRATCH;
    workspace = nullptr;
    if (need > 0 && qsa::attn_scratch(&workspace) != hipSuccess) return QSA_E_HIP;
  } else if (need > 0 && (!workspace || ws_bytes < need || !aligned(workspace, 256))) {
    return QSA_E_WORKSPACE;
  }
  qsa::AttnArgs a;
  a.total_q = total_q;
  a.page_size = dims->page_size;
  a.pt_stride = pt_stride;
  a.sel_stride = sel_stride;
  a.n_extra = n_extra;
  a.sm_scale = dims->sm_scale;
  a.q = q;
  a.q_req = q_req;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.fp8 = fp8;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.page_table = page_table;
  a.sel_pos = sel_pos;
  a.sel_count = sel_count;
  a.extra_pos = n_extra > 0 ? extra_pos : nullptr;
  a.out = out;
  a.lse = lse;
  a.part = static_cast<float*>(workspace);
  qsa::attn_plan(total_q, n_extra, &a.splits, &a.split_len);
  return hip_status(qsa::launch_attn(a, static_cast<hipStream_t>(stream)));
}

int qsa_sparse_gqa_decode(const qsa_dims* dims, int32_t batch, const uint16_t* q,
                          const uint16_t* k_pool, const uint16_t* v_pool,
                          const int32_t* page_table, int32_t pt_stride, const int32_t* sel_pos,
                          const int32_t* sel_count, int32_t sel_stride, const int32_t* extra_pos,
                          int32_t n_extra, uint16_t* out, float* lse, void* workspace,
                          size_t ws_bytes, void* stream) {
  return gqa_common(dims, batch, q, nullptr, k_pool, v_pool, false, 1.f, 1.f, page_table,
                    pt_stride, sel_pos, sel_count, sel_stride, extra_pos, n_extra, out, lse,
                    workspace, ws_bytes, stream);
}

int qsa_sparse_gqa_decode_noalloc(const qsa_dims* dims, int32_t batch, const uint16_t* q,
                                  const uint16_t* k_pool, const uint16_t* v_pool,
                                  const int32_t* page_table, int32_t pt_stride,
                                  const int32_t* sel_pos, const int32_t* sel_count,
                                  int32_t sel_stride, const int32_t* extra_pos, int32_t n_extra,
                                  uint16_t* out, float* lse, void* stream) {
  return gqa_common(dims, batch, q, nullptr, k_pool, v_pool, false, 1.f, 1.f, page_table,
                    pt_stride, sel_pos, sel_count, sel_stride, extra_pos, n_extra, out, lse,
                    nullptr, 0, stream, true);
}

int qsa_sparse_gqa_decode_fp8(const qsa_dims* dims, int32_t batch, const uint16_t* q,
                              const uint8_t* k_pool, const uint8_t* v_pool, float k_scale,
                              float v_scale, const int32_t* page_table, int32_t pt_stride,
                              const int32_t* sel_pos, const int32_t* sel_count, int32_t sel_stride,
                              const int32_t* extra_pos, int32_t n_extra, uint16_t* out, float* lse,
                              void* workspace, size_t ws_bytes, void* stream) {
  return gqa_common(dims, batch, q, nullptr, k_pool, v_pool, true, k_scale, v_scale, page_table,
                    pt_stride, sel_pos, sel_count, sel_stride, extra_pos, n_extra, out, lse,
                    workspace, ws_bytes, stream);
}

int qsa_sparse_gqa_prefill(const qsa_dims* dims, int32_t total_q, const uint16_t* q,
                           const int32_t* q_req, const uint16_t* k_pool, const uint16_t* v_pool,
                           const int32_t* page_table, int32_t pt_stride, const int32_t* sel_pos,
                           const int32_t* sel_count, int32_t sel_stride, uint16_t* out,
                           float* lse, void* workspace, size_t ws_bytes, void* stream) {
  if (total_q > 0 && !q_req) return QSA_E_NULL;
  return gqa_common(dims, total_q, q, q_req, k_pool, v_pool, false, 1.f, 1.f, page_table,
                    pt_stride, sel_pos, sel_count, sel_stride, nullptr, 0, out, lse, workspace,
                    ws_bytes, stream);
}

int qsa_sparse_gqa_prefill_fp8(const qsa_dims* dims, int32_t total_q, const uint16_t* q,
                               const int32_t* q_req, const uint8_t* k_pool, const uint8_t* v_pool,
                               float k_scale, float v_scale, const int32_t* page_table,
                               int32_t pt_stride, const int32_t* sel_pos, const int32_t* sel_count,
                               int32_t sel_stride, uint16_t* out, float* lse, void* workspace,
                               size_t ws_bytes, void* stream) {
  if (total_q > 0 && !q_req) return QSA_E_NULL;
  return gqa_common(dims, total_q, q, q_req, k_pool, v_pool, true, k_scale, v_scale, page_table,
                    pt_stride, sel_pos, sel_count, sel_stride, nullptr, 0, out, lse, workspace,
                    ws_bytes, stream);
}

}  // extern "C"
