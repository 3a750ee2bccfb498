/*
 * qsa.h - C ABI of the QSA c4 hot path on MI355X (gfx950).
 *
 * QSA ("Qwen Sparse Attention", compression ratio 4) attends each query to at
 * most 2051 positions of a long context.  A light indexer picks them: every 4
 * tokens' raw indexer keys are compressed into one key, the query scores every
 * visible compressed block, the best 512 blocks are kept and expanded back to
 * token positions, and the 0..3 tokens of the unfinished block are appended.
 * Attention then reads those positions from the raw, uncompressed paged K/V
 * cache.  [SGLang day-0 post on Qwen3.8-Flash-Next, section "Qwen Sparse
 * Attention: Retrieve Coarsely, Attend Precisely"; section "IndexShare MTP:
 * Reusing the QSA Selection Across Draft Steps" for the reuse step.]
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless marked "host".  The caller owns every
 *    buffer; the library never allocates, frees or synchronises, and reads no
 *    device memory back to the host.  Scratch memory comes from the caller's
 *    workspace, sized by qsa_workspace_bytes() (qsa_sparse_gqa_decode_noalloc
 *    uses the library's static device array instead).
 *  - bf16 tensors are passed as uint16_t bit patterns; all are row-major and
 *    densely packed in the shapes given.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    is ordered after earlier work on it.  Calls are graph-capturable: no host
 *    readback and no data-dependent launch shape.
 *  - Host-side arguments are validated before anything is launched; on error a
 *    status other than QSA_OK is returned and nothing is enqueued.  Contents of
 *    device arrays (page tables, positions, counts) are trusted: they must lie
 *    in the ranges stated below.  The library built with -DQSA_DEBUG
 *    (libqsa_debug.so) checks them where the kernels read them and traps the
 *    kernel on a violation.
 *  - Reentrant; no mutable global state, except that qsa_sparse_gqa_decode_noalloc
 *    keeps a static scratch array on each device and caches its address.
 *
 * Supported shapes: num_q_heads = 16, num_kv_heads = 2, head_dim = 256,
 * idx_heads = 4, idx_dim = 128, page_size a multiple of 16 (64 in practice),
 * positions 0 .. QSA_MAX_CONTEXT-1.  Anything else returns QSA_E_UNSUPPORTED.
 *
 * Layouts:
 *  - Raw K/V pool (the ordinary paged cache): k_pool, v_pool [slots, Hkv, D].
 *    Token t of request b lives in slot
 *        page_table[b * pt_stride + t / page_size] * page_size + t % page_size.
 *    Page-table entries are >= 0 where a position is read, and slot indices
 *    are below 2^31 (a pool of 2^31 slots would hold 2 TB of bf16 K).
 *  - Compressed key cache: comp_cache [slots / 4, idx_dim].  Block c (tokens
 *    4c..4c+3) of request b lives at row  slot(4c) / 4  (the block's first
 *    slot over 4, page aligned), so it follows the page's ownership.
 *  - Ring: ring [batch, 4, idx_dim] holds the raw indexer keys of a request's
 *    unfinished block; token t sits in slot t % 4.
 */
#ifndef QSA_H
#define QSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_BLOCK 4            /* tokens per compressed block (c4)            */
#define QSA_TOPK 512           /* blocks kept per query                       */
#define QSA_MAX_SEL 2051       /* 4 * 512 + 3 positions at most per query     */
#define QSA_MAX_CONTEXT 262144 /* positions 0 .. 262143                       */
#define QSA_MAX_EXTRA 8        /* extra (drafted) positions per reuse query   */

typedef struct qsa_dims {
  int32_t num_q_heads;  /* attention query heads              (16)          */
  int32_t num_kv_heads; /* attention K/V heads                (2)           */
  int32_t head_dim;     /* attention head size                (256)         */
  int32_t idx_heads;    /* indexer query heads                (4)           */
  int32_t idx_dim;      /* indexer head size                  (128)         */
  int32_t page_size;    /* tokens per page; multiple of 16    (64)          */
  float rope_theta;     /* rotary base of the indexer keys    (1e7)         */
  float sm_scale;       /* attention logit scale              (1/sqrt(256)) */
} qsa_dims;

enum qsa_status {
  QSA_OK = 0,
  QSA_E_NULL = 1,        /* a required pointer is NULL                       */
  QSA_E_SHAPE = 2,       /* a size or stride is out of range                 */
  QSA_E_UNSUPPORTED = 3, /* dims other than the compiled ones                */
  QSA_E_WORKSPACE = 4,   /* workspace missing or smaller than required       */
  QSA_E_HIP = 5,         /* a HIP launch failed (see hipGetLastError)        */
  QSA_E_SCRATCH = 6      /* more scratch than the static buffer holds        */
};

enum qsa_op {
  QSA_OP_INDEX_TOPK = 1,
  QSA_OP_GQA_DECODE = 2,
  QSA_OP_GQA_PREFILL = 3
};

/* Human-readable name of a status code (static string, never NULL). */
const char* qsa_status_string(int status);

/* Profiling aid: the calling thread's next QSA call (any entry point below)
 * launches its i-th kernel with the start and stop events events[2i] and
 * events[2i+1] (hipExtLaunchKernelGGL: the runtime sets them from the dispatch's own
 * start and end timestamps, so their elapsed time is the kernel's duration), for i <
 * n_events / 2 and as many kernels as the call launches; then the request lapses
 * (also when that call returns an error).  events: n_events hipEvent_t handles created
 * by the caller (host array).  n_events even, 0..16 (0 cancels), else QSA_E_SHAPE; a
 * NULL handle gives QSA_E_NULL; a rejected request also cancels an earlier one.  It
 * changes no result.  The kernels a call launches, in order:
 * qsa_decode_build_index_topk: the scorer (builder folded in), then the select;
 * qsa_index_topk: the scorer (one launch per 64 queries, or per 256 queries of the
 * multi-query scorer, in decode and verification batches), then the select, and for
 * prefill chunks the MFMA scorer, the code select, the exact rescoring and the queued
 * select; the sparse GQA calls: the gather, then the split combine when the list is
 * split; the builders: one kernel. */
int qsa_profile_kernel_events(void* const* events, int32_t n_events);

/* Workspace bytes that `op` needs for `total_q` queries.
 *   INDEX_TOPK:  max_pos = an upper bound on every q_pos + 1 (host).
 *   GQA_DECODE / GQA_PREFILL: n_extra = columns of extra_pos (0 for prefill).
 * Returns 0 for bad arguments.  The workspace must be 256-byte aligned. */
size_t qsa_workspace_bytes(const qsa_dims* dims, int op, int32_t total_q, int32_t max_pos,
                           int32_t n_extra);

/* Stage 1 - compressed index-key builder.  [QSA section: each group of 4 raw
 * indexer keys becomes one BF16 compressed key: their FP32 mean, normalised and
 * rotated by the block's first-token rotary position; a 4-slot per-request ring holds
 * the raw keys of the unfinished block; compressed keys sit at full_slot / 4.]
 *
 * Ingests the raw indexer keys of new tokens len_before[b] .. len_before[b] +
 * n_b - 1 of every request b (n_b = cu_new[b+1] - cu_new[b]).  For each block
 * that becomes complete, its key is
 *     m   = ((k0 + k1) + k2) + k3, times 1/4, in FP32 (token order);
 *     k   = m / max(||m||_2, 1e-12);
 *     key = k with pair (i, i+64) turned by angle 4c * theta^(-2i/128);
 * rounded to bf16 (nearest-even) and stored at comp_cache row slot(4c) / 4.
 * Raw keys of earlier tokens of the block are read from the ring; raw keys of
 * tokens left in an unfinished block are written to ring slots t % 4.
 *
 *   new_idx_k  [total_new, idx_dim] bf16  raw keys, request-major (read)
 *   cu_new     [batch + 1] int32          offsets into new_idx_k (read)
 *   len_before [batch] int32              tokens ingested before this call (read)
 *   total_new, max_new (host)             cu_new[batch] and max n_b
 *   page_table [batch, pt_stride] int32   physical page of each logical page;
 *                                         must cover every written block
 *   ring       [batch, 4, idx_dim] bf16   in/out
 *   comp_cache [rows, idx_dim] bf16       out (rows of completed blocks only)
 */
int qsa_build_index_keys(const qsa_dims* dims, int32_t batch, const uint16_t* new_idx_k,
                         const int32_t* cu_new, const int32_t* len_before, int32_t total_new,
                         int32_t max_new, const int32_t* page_table, int32_t pt_stride,
                         uint16_t* ring, uint16_t* comp_cache, void* stream);

/* Stage 1 with MRoPE positions - as qsa_build_index_keys, for models whose tokens
 * carry 3-D rotary positions (temporal, height, width; image and video tokens).
 * [QSA section: a block's key is rotated by the multimodal rotary position of its
 * first token, and the indexer shares the attention layers' MRoPE code.  The pages
 * give no section layout; the axis map is an argument.]
 *
 * Every step is that of qsa_build_index_keys except the angle: pair (i, i+64) of
 * block c is turned by  P[pair_axis[i]] * theta^(-2i/128),  where P is the 3-D
 * position of the block's first token 4c.  A text token whose position is
 * (p, p, p) at sequence index p gives the same keys as qsa_build_index_keys.
 *
 *   new_mpos   [total_new, 3] int32       3-D positions of the new tokens (read)
 *   pair_axis  [64] uint8 (host)          0 = temporal, 1 = height, 2 = width;
 *                                         other values give QSA_E_SHAPE.  Contiguous
 *                                         sections of 16, 24, 24 pairs are the usual
 *                                         layout; an interleaved map is allowed too
 *   ring_mpos  [batch, 4, 3] int32        in/out: positions of the ring's tokens,
 *                                         slot t % 4, kept like the key ring
 *   every other argument as for qsa_build_index_keys.  The same ring and
 *   compressed cache may not be driven by both calls for one request.
 */
int qsa_build_index_keys_mrope(const qsa_dims* dims, int32_t batch, const uint16_t* new_idx_k,
                               const int32_t* new_mpos, const int32_t* cu_new,
                               const int32_t* len_before, int32_t total_new, int32_t max_new,
                               const int32_t* page_table, int32_t pt_stride,
                               const uint8_t* pair_axis, uint16_t* ring, int32_t* ring_mpos,
                               uint16_t* comp_cache, void* stream);

/* Stage 2 - indexer: score, top-512, expansion.  [QSA section: every complete
 * block a query can see gets a score; the 512 highest-scoring blocks become their
 * 2048 token positions, and the 0..3 tokens of the still-open block are added, for
 * at most 2051 positions.]
 *
 * For query t at position p = q_pos[t] of request b = q_req[t]:
 *   n_c = (p + 1) / 4 complete blocks are visible;
 *   s_c = sum_h w_h * max(0, q_h . key_c)  for c < n_c  (FP32 accumulation);
 *   the 512 best blocks are kept (all if n_c <= 512), higher score first, ties
 *   to the lower block index, and written ascending to sel_blocks (-1 pad);
 *   sel_pos gets 4c..4c+3 of each kept block, ascending, then 4*n_c .. p;
 *   sel_count = 4 * min(n_c, 512) + (p + 1) % 4; the rest of the row is -1.
 *
 *   idx_q      [total_q, idx_heads, idx_dim] bf16  indexer queries (rotary applied)
 *   idx_w      [total_q, idx_heads] float          per-head weights w_h
 *   q_req, q_pos [total_q] int32                   request and position of each query
 *   max_pos (host)                                 > every q_pos; <= QSA_MAX_CONTEXT
 *   comp_cache                                     as written by the builder
 *   sel_blocks [total_q, 512] int32   out
 *   sel_pos    [total_q, sel_stride] int32 out; sel_stride >= 2051 and a multiple
 *              of 4, sel_pos 16-byte aligned
 *   sel_count  [total_q] int32        out
 *   workspace  >= qsa_workspace_bytes(QSA_OP_INDEX_TOPK, total_q, max_pos, 0)
 */
int qsa_index_topk(const qsa_dims* dims, int32_t batch, int32_t total_q, const uint16_t* idx_q,
                   const float* idx_w, const int32_t* q_req, const int32_t* q_pos,
                   int32_t max_pos, const int32_t* page_table, int32_t pt_stride,
                   const uint16_t* comp_cache, int32_t* sel_blocks, int32_t* sel_pos,
                   int32_t sel_stride, int32_t* sel_count, void* workspace, size_t ws_bytes,
                   void* stream);

/* Stages 1 + 2 of one decode step in two launches instead of three.  [QSA section:
 * during decode the new token's indexer key enters the ring, or completes a block
 * whose compressed key is stored, before the query scores the visible blocks; the
 * pages lay this bookkeeping out as separate kernels ahead of the indexer.]
 *
 * Request b has exactly one new token, at position p = pos[b] (the tokens before it:
 * 0 .. p-1 are already ingested), and that token is also the request's query.  The
 * call has the effect of
 *     qsa_build_index_keys(cu_new = 0, 1, .., batch; len_before = pos; total_new =
 *                          batch; max_new = 1)
 * followed by
 *     qsa_index_topk(total_q = batch; q_req[b] = b; q_pos = pos)
 * and writes the same ring, comp_cache, sel_blocks, sel_pos and sel_count bits as
 * those two calls.  The scorer launch ingests the tokens itself: each query's own
 * work group builds the key of a block its token completes and scores the query's
 * last 16 blocks with it.  1-D RoPE (qsa_decode_build_index_topk_mrope takes 3-D
 * positions).
 *
 *   new_idx_k  [batch, idx_dim] bf16  raw indexer key of each request's new token
 *              (8-byte aligned)
 *   pos        [batch] int32          position of that token (>= 0)
 *   max_pos (host)                    > every pos; <= QSA_MAX_CONTEXT
 *   page_table [batch, pt_stride]     must cover position pos[b] of every request
 *   ring, comp_cache                  in/out, as for qsa_build_index_keys; a block
 *                                     row written here must not be read by another
 *                                     request's query of the same call (distinct
 *                                     requests do not share a page being written)
 *   idx_q, idx_w                      [batch, ...] as for qsa_index_topk
 *   sel_blocks, sel_pos, sel_stride, sel_count   out, as for qsa_index_topk
 *   workspace  >= qsa_workspace_bytes(QSA_OP_INDEX_TOPK, batch, max_pos, 0)
 */
int qsa_decode_build_index_topk(const qsa_dims* dims, int32_t batch, const uint16_t* new_idx_k,
                                const int32_t* pos, int32_t max_pos, const int32_t* page_table,
                                int32_t pt_stride, uint16_t* ring, uint16_t* comp_cache,
                                const uint16_t* idx_q, const float* idx_w, int32_t* sel_blocks,
                                int32_t* sel_pos, int32_t sel_stride, int32_t* sel_count,
                                void* workspace, size_t ws_bytes, void* stream);

/* Stages 1 + 2 of one decode step with MRoPE positions - as qsa_decode_build_index_topk,
 * for tokens with 3-D rotary positions.  [QSA section: a block's key is rotated by the
 * multimodal rotary position of its first token.]
 *
 * The call has the effect of qsa_build_index_keys_mrope (same new_mpos, pair_axis and
 * ring_mpos; cu_new = 0, 1, .., batch; len_before = pos) followed by qsa_index_topk,
 * and writes the same bits as those two calls.  A block completed by the new token has
 * its first token in ring slot 0, so its angle comes from ring_mpos slot 0.
 *
 *   new_mpos   [batch, 3] int32   3-D position of each request's new token
 *   pair_axis  [64] uint8 (host)  as for qsa_build_index_keys_mrope
 *   ring_mpos  [batch, 4, 3] int32 in/out, beside ring
 * The other arguments are those of qsa_decode_build_index_topk.  NULL new_mpos,
 * pair_axis or ring_mpos returns QSA_E_NULL; an axis above 2 returns QSA_E_SHAPE.
 */
int qsa_decode_build_index_topk_mrope(const qsa_dims* dims, int32_t batch,
                                      const uint16_t* new_idx_k, const int32_t* new_mpos,
                                      const int32_t* pos, int32_t max_pos,
                                      const int32_t* page_table, int32_t pt_stride,
                                      const uint8_t* pair_axis, uint16_t* ring, int32_t* ring_mpos,
                                      uint16_t* comp_cache, const uint16_t* idx_q,
                                      const float* idx_w, int32_t* sel_blocks, int32_t* sel_pos,
                                      int32_t sel_stride, int32_t* sel_count, void* workspace,
                                      size_t ws_bytes, void* stream);

/* Stage 3 - sparse GQA, decode (one query per request).  [QSA section: attention
 * weights and the weighted value sum come from the full-resolution K/V; IndexShare
 * section: a draft step reuses the captured selection plus the positions drafted
 * since the capture.]
 *
 * For request b, head h (KV head g = h / (Hq / Hkv)) over the position list
 * S = sel_pos[b, 0 .. sel_count[b]-1]  plus every extra_pos[b, j] >= 0:
 *   out[b, h] = sum_t softmax_t(sm_scale * q[b, h] . K[t, g]) * V[t, g],
 *   lse[b, h] = log(sum_t exp(sm_scale * q[b, h] . K[t, g]))   (natural log).
 * Positions must be distinct and their pages mapped; an empty S gives out = 0
 * and lse = -inf.
 *
 *   q          [batch, Hq, D] bf16
 *   k_pool, v_pool [slots, Hkv, D] bf16
 *   sel_pos [batch, sel_stride], sel_count [batch] int32; sel_count <= sel_stride
 *              and sel_count <= QSA_MAX_SEL (the most an indexer row can hold; the
 *              kernels size their per-query work for it, and the QSA_DEBUG build
 *              traps on a larger count)
 *   extra_pos  [batch, n_extra] int32 or NULL (n_extra = 0); n_extra <= QSA_MAX_EXTRA
 *   out        [batch, Hq, D] bf16 out;  lse [batch, Hq] float out or NULL
 *   workspace  >= qsa_workspace_bytes(QSA_OP_GQA_DECODE, batch, 0, n_extra)
 */
int qsa_sparse_gqa_decode(const qsa_dims* dims, int32_t batch, const uint16_t* q,
                          const uint16_t* k_pool, const uint16_t* v_pool,
                          const int32_t* page_table, int32_t pt_stride, const int32_t* sel_pos,
                          const int32_t* sel_count, int32_t sel_stride, const int32_t* extra_pos,
                          int32_t n_extra, uint16_t* out, float* lse, void* workspace,
                          size_t ws_bytes, void* stream);

/* Stage 3, decode, without a workspace: qsa_sparse_gqa_decode for callers that
 * cannot allocate device memory (code under hipGraph capture, tight serving loops
 * such as the IndexShare draft steps, harnesses that forbid hipMalloc).
 *
 * Arguments and results are those of qsa_sparse_gqa_decode (same kernels, same
 * bits), minus the workspace: the split partials go to a device array that the
 * library holds on every GPU it runs on, QSA_ATTN_SCRATCH_BYTES bytes, until the
 * process ends.  The call allocates nothing.  Its device address is looked up on
 * the first call on each device, which must be the current device (the one
 * `stream` belongs to).
 *  - Calls on one GPU share that array: calls that may overlap (on different
 *    streams, or from different threads) race on it and must be ordered by the
 *    caller.  Nothing in it needs clearing: every call writes the partials it reads.
 *  - A call needing more than QSA_ATTN_SCRATCH_BYTES returns QSA_E_SCRATCH and
 *    enqueues nothing.  Every batch size fits today: the partials are largest near
 *    batch 127 (4,194,048 bytes); from batch 128 on the call needs none.
 *  - QSA_E_HIP if the array's address cannot be obtained.
 */
#define QSA_ATTN_SCRATCH_BYTES (8u << 20)
int qsa_sparse_gqa_decode_noalloc(const qsa_dims* dims, int32_t batch, const uint16_t* q,
                                  const uint16_t* k_pool, const uint16_t* v_pool,
                                  const int32_t* page_table, int32_t pt_stride,
                                  const int32_t* sel_pos, const int32_t* sel_count,
                                  int32_t sel_stride, const int32_t* extra_pos, int32_t n_extra,
                                  uint16_t* out, float* lse, void* stream);

/* Stage 3 - sparse GQA over a chunk of prefill queries: as the decode call, with
 * query t reading request q_req[t] and no extra positions.  [QSA section: for
 * prefill the expanded indices feed sparse GQA.]
 *
 *   q [total_q, Hq, D] bf16;  q_req [total_q] int32;  out [total_q, Hq, D] bf16;
 *   sel_count [total_q] <= min(sel_stride, QSA_MAX_SEL), as for the decode call;
 *   lse [total_q, Hq] float or NULL;
 *   workspace >= qsa_workspace_bytes(QSA_OP_GQA_PREFILL, total_q, 0, 0)
 */
int qsa_sparse_gqa_prefill(const qsa_dims* dims, int32_t total_q, const uint16_t* q,
                           const int32_t* q_req, const uint16_t* k_pool, const uint16_t* v_pool,
                           const int32_t* page_table, int32_t pt_stride, const int32_t* sel_pos,
                           const int32_t* sel_count, int32_t sel_stride, uint16_t* out,
                           float* lse, void* workspace, size_t ws_bytes, void* stream);

/* Stage 3 with an FP8 K/V cache - sparse GQA as qsa_sparse_gqa_decode /
 * qsa_sparse_gqa_prefill, over pools of OCP FP8 E4M3 codes with one scale per
 * pool.  [ailone.io model page on Qwen3.8-Flash-Next, comparison of vLLM builds: a
 * K/V cache in FP8 runs at the speed of BF16 and holds a larger token pool.  The
 * page states neither the FP8 format nor the scaling; E4M3 with per-pool scales is
 * the reading implemented.]
 *
 * A code c of k_pool stands for the value e4m3(c) * k_scale, a code of v_pool for
 * e4m3(c) * v_scale, where e4m3(c) = (-1)^s (1 + m/8) 2^(e-7) for exponent e > 0
 * and (-1)^s (m/8) 2^-6 for e = 0 (bias 7, 3 mantissa bits, no infinities; the
 * codes 0x7f and 0xff are NaN and must not appear at attended positions).  With
 * those values the results are defined as for the bf16 calls.
 *
 *   k_pool, v_pool [slots, Hkv, D] uint8 codes, 16-byte aligned (half the bytes of
 *                  the bf16 pools, same slot layout)
 *   k_scale, v_scale (host) finite and > 0, else QSA_E_SHAPE
 *   every other argument, the workspace included, as for the bf16 call
 */
int qsa_sparse_gqa_decode_fp8(const qsa_dims* dims, int32_t batch, const uint16_t* q,
                              const uint8_t* k_pool, const uint8_t* v_pool, float k_scale,
                              float v_scale, const int32_t* page_table, int32_t pt_stride,
                              const int32_t* sel_pos, const int32_t* sel_count, int32_t sel_stride,
                              const int32_t* extra_pos, int32_t n_extra, uint16_t* out, float* lse,
                              void* workspace, size_t ws_bytes, void* stream);

int qsa_sparse_gqa_prefill_fp8(const qsa_dims* dims, int32_t total_q, const uint16_t* q,
                               const int32_t* q_req, const uint8_t* k_pool, const uint8_t* v_pool,
                               float k_scale, float v_scale, const int32_t* page_table,
                               int32_t pt_stride, const int32_t* sel_pos, const int32_t* sel_count,
                               int32_t sel_stride, uint16_t* out, float* lse, void* workspace,
                               size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
