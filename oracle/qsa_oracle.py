"""Plain, slow reference for the QSA c4 hot path (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this module. The library path never does: it shares no code, constants,
tables or helpers with the HIP kernels, and it reads no value they produce.

Everything is computed from the bf16 input bits (or FP8 K/V codes) in float64,
except the one step whose precision the pages fix (the block mean is taken in
FP32).

Sources, cited by title and section:
  [QSA]  SGLang day-0 post on Qwen3.8-Flash-Next, section "Qwen Sparse Attention:
         Retrieve Coarsely, Attend Precisely".
  [IS]   same post, section "IndexShare MTP: Reusing the QSA Selection Across
         Draft Steps"; and its "Model Architecture" list, IndexShare MTP item.
  [AIL]  ailone.io model page on Qwen3.8-Flash-Next, its comparison of vLLM builds:
         a K/V cache in FP8 at the speed of BF16 with a larger token pool.

Readings where the pages are silent or garbled (the plainest reading that the rest of
the pages supports):
  R1  The scoring formula is cut off in [QSA]; the score of block c for a query is
      s_c = sum_h w_h * max(0, q_h . k_c) over the 4 indexer heads, no 1/sqrt(d).
  R2  "normalized" is the L2 norm, floored at 1e-12 (an all-zero mean stays zero).
  R3  The block's rotary phase is 1-D RoPE at the block's first position 4c, with
      rotate-half pairing (i, i+64) over all 128 dims and theta = 1e7; the angle of
      pair i is 4c * theta**(-2i/128).  Normalise first, then rotate.
  R4  The FP32 mean sums the four raw keys in token order, then scales by 1/4.
  R5  Only complete blocks are scored: n_c(p) = (p+1) // 4 for a query at p; a block
      the query's own token completes is visible.  The 0..3 tokens of the unfinished
      block, 4*n_c .. p, are appended directly.
  R6  Top-512 ties: higher score first, then lower block index.  All blocks are
      kept when n_c <= 512.  The kept blocks are reported in ascending order.
  R7  Sparse GQA: query head h reads KV head h // (16/2); logits are scaled by
      1/sqrt(256); no sink, soft-cap or output gate; lse is the natural log.
  R8  IndexShare: reuse step j attends to the captured positions plus p_cap+1 ..
      p_cap+j (the positions drafted since the capture).
  R9  FP8 K/V [AIL] (format and scaling not stated): OCP FP8 E4M3 codes (bias 7, 3
      mantissa bits, no infinities, S.1111.111 is NaN, largest finite 448) with one
      scale per pool; a stored code c stands for e4m3(c) * k_scale (K) or
      e4m3(c) * v_scale (V).  Attention is then as in R7 on those values.
  R10 MRoPE [QSA: each block's key is rotated by the multimodal rotary position of
      the block's first token, and the indexer shares the attention layers' MRoPE]: a token has a 3-D position
      (temporal, height, width); each rotary pair i takes the angle
      pos[axis(i)] * theta**(-2i/128) from one component, chosen by a per-pair axis
      map.  The pages give no sections; the default map is contiguous sections of
      16, 24 and 24 pairs (t, h, w).  A text token at sequence position p has the
      position (p, p, p), which reduces MRoPE to R3.
  parity unpinned: fidelity to the real model's readings R1, R3 (pairing, rotary
      fraction, theta), R10's sections and R2's epsilon cannot be checked against
      the pages.
"""

from __future__ import annotations

import numpy as np

TOPK_BLOCKS = 512
BLOCK = 4                      # compression ratio c4
MAX_SELECTED = TOPK_BLOCKS * BLOCK + BLOCK - 1   # 2051
NORM_FLOOR = 1e-12


# ---------------------------------------------------------------- number formats

def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def e4m3_to_f64(codes) -> np.ndarray:
    """OCP FP8 E4M3 codes -> float64 (exact), reading R9.

    A code is sign s, exponent e (4 bits, bias 7) and mantissa m (3 bits): e > 0
    gives (-1)^s * (1 + m/8) * 2^(e-7); e = 0 gives (-1)^s * (m/8) * 2^-6; the
    all-ones exponent and mantissa (0x7f, 0xff) are NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e > 0, (1.0 + m / 8.0) * np.exp2(e - 7.0), (m / 8.0) * 2.0 ** -6)
    return np.where((c & 0x7F) == 0x7F, np.nan, s * mag)


def round_to_bf16(x) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even), returned as float64.

    bf16 keeps 8 significant bits and float32's exponent range, so the spacing of
    the grid around x is 2**(e-8) where x = m * 2**e, 0.5 <= |m| < 1, and 2**-133
    below the smallest normal.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e, -125) - 8
    y = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    big = np.abs(y) > 3.3895313892515355e38
    return np.where(big, np.copysign(np.inf, x), y)


def f64_to_bf16_bits(x) -> np.ndarray:
    y = round_to_bf16(x).astype(np.float32)     # exact: y is on the bf16 grid
    return (y.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------- paged addressing

def token_slot(page_row, t, page_size: int):
    """Slot of logical token t in the raw K/V pool [QSA]: the raw K/V stays in the
    ordinary paged pool, one token per slot."""
    t = np.asarray(t, dtype=np.int64)
    return np.asarray(page_row, dtype=np.int64)[t // page_size] * page_size + t % page_size


def comp_slot(page_row, c, page_size: int):
    """Slot of compressed block c in the compressed cache: the full slot of the
    block's first token divided by 4, which is page aligned [QSA]."""
    c = np.asarray(c, dtype=np.int64)
    return token_slot(page_row, BLOCK * c, page_size) // BLOCK


# ---------------------------------------------------------------- stage 1: keys

def inv_freqs(d: int, theta: float) -> np.ndarray:
    """theta**(-2i/d) for the d/2 rotary pairs (i, i + d/2)."""
    return theta ** (-(2.0 * np.arange(d // 2)) / d)


def rotate(x, pos, theta: float) -> np.ndarray:
    """Rotary phase of position `pos` on the last axis of x (reading R3)."""
    x = np.asarray(x, dtype=np.float64)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freqs(x.shape[-1], theta)
    return rotate_by(x, ang)


def mrope_angles(pos3, pair_axis, theta: float, d: int = 128) -> np.ndarray:
    """Angles of MRoPE (reading R10): pair i of a token at 3-D position pos3 turns
    by pos3[axis(i)] * theta**(-2i/d).  pos3: [..., 3] -> [..., d/2]."""
    pos3 = np.asarray(pos3, dtype=np.float64)
    return pos3[..., np.asarray(pair_axis, dtype=np.int64)] * inv_freqs(d, theta)


def rotate_by(x, ang) -> np.ndarray:
    """Turn pair (i, i + d/2) of the last axis of x by ang[..., i] (rotate-half)."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def block_mean_fp32(raw4_bits) -> np.ndarray:
    """Mean of the 4 raw keys of a block, taken in FP32 [QSA] (reading R4).

    raw4_bits: [..., 4, d] bf16 bits -> [..., d] float32.
    """
    k = bf16_to_f64(raw4_bits).astype(np.float32)
    s = k[..., 0, :] + k[..., 1, :]
    s = s + k[..., 2, :]
    s = s + k[..., 3, :]
    return s * np.float32(0.25)


def compress_blocks(raw_bits, first_pos, theta: float) -> np.ndarray:
    """Compressed index keys [QSA]: the FP32 mean of each block's 4 raw keys is
    L2-normalised (R2), turned by the rotary phase of the block's first position
    (R3) and stored as bf16.

    raw_bits: [n, 4, d] bf16 bits; first_pos: [n] -> [n, d] bf16 bits.
    """
    return f64_to_bf16_bits(rotate(normalised_means(raw_bits), first_pos, theta))


def compress_blocks_mrope(raw_bits, first_pos3, pair_axis, theta: float) -> np.ndarray:
    """compress_blocks with MRoPE (R10): each block is turned by the angles of its
    first token's 3-D position.  first_pos3: [n, 3]."""
    k = normalised_means(raw_bits)
    return f64_to_bf16_bits(rotate_by(k, mrope_angles(first_pos3, pair_axis, theta, k.shape[-1])))


def normalised_means(raw_bits) -> np.ndarray:
    """FP32 block means (R4), L2-normalised in float64 with the floor of R2."""
    m = block_mean_fp32(raw_bits).astype(np.float64)
    norm = np.sqrt(np.sum(m * m, axis=-1, keepdims=True))
    return m / np.maximum(norm, NORM_FLOOR)


def build_index_state(raw_bits, length: int, theta: float, mpos=None, pair_axis=None):
    """Index state of a request after tokens 0..length-1 are ingested [QSA]:
    one compressed key per complete block, and the raw keys of the unfinished
    block's tokens in ring slots t % 4.  With mpos ([length, 3] 3-D positions) the
    blocks are turned by MRoPE (R10) with the axis map pair_axis.

    Returns (comp [length//4, d] bf16 bits, ring dict {slot: bits [d]}).
    """
    raw = np.asarray(raw_bits)[:length]
    n_c = length // BLOCK
    blocks = raw[:BLOCK * n_c].reshape(n_c, BLOCK, raw.shape[-1])
    if mpos is None:
        comp = compress_blocks(blocks, BLOCK * np.arange(n_c), theta)
    else:
        first = np.asarray(mpos)[:BLOCK * n_c:BLOCK]
        comp = compress_blocks_mrope(blocks, first, pair_axis, theta)
    ring = {t % BLOCK: raw[t].copy() for t in range(BLOCK * n_c, length)}
    return comp, ring


# ---------------------------------------------------------------- stage 2: indexer

def visible_blocks(p: int) -> int:
    """Complete blocks visible to a query at position p (reading R5)."""
    return (p + 1) // BLOCK


def score_blocks(idx_q_bits, idx_w, comp_bits) -> np.ndarray:
    """s_c = sum_h w_h * max(0, q_h . k_c) (reading R1) for every row k_c of comp.

    idx_q_bits: [4, d]; idx_w: [4]; comp_bits: [n, d] -> [n] float64.
    """
    qh = bf16_to_f64(idx_q_bits)
    k = bf16_to_f64(comp_bits)
    w = np.asarray(idx_w, dtype=np.float64)
    dots = k @ qh.T                               # [n, 4]
    return np.maximum(dots, 0.0) @ w


def score_blocks_many(idx_q_bits, idx_w, comp_bits) -> np.ndarray:
    """score_blocks for several queries against the same keys (reading R1):
    row t, column c holds sum_h w[t,h] * max(0, q[t,h] . k_c).

    idx_q_bits: [T, 4, d]; idx_w: [T, 4]; comp_bits: [n, d] -> [T, n] float64.
    """
    qh = bf16_to_f64(idx_q_bits)                  # [T, 4, d]
    k = bf16_to_f64(comp_bits)                    # [n, d]
    w = np.asarray(idx_w, dtype=np.float64)       # [T, 4]
    T, H, d = qh.shape
    dots = (qh.reshape(T * H, d) @ k.T).reshape(T, H, -1)   # [T, 4, n]
    return np.einsum("th,thn->tn", w, np.maximum(dots, 0.0))


def select_blocks(scores, topk: int = TOPK_BLOCKS) -> np.ndarray:
    """The best `topk` blocks [QSA], ties by lower index (R6), in ascending order."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    if n <= topk:
        return np.arange(n, dtype=np.int64)
    order = np.lexsort((np.arange(n), -s))        # primary: -s, secondary: index
    return np.sort(order[:topk]).astype(np.int64)


def expand_positions(sel_blocks, p: int) -> np.ndarray:
    """Logical token positions attended by a query at p [QSA]: the 4 tokens of
    every kept block, then the 0..3 tokens of the unfinished block (R5)."""
    sel = np.asarray(sel_blocks, dtype=np.int64)
    full = (BLOCK * sel[:, None] + np.arange(BLOCK)[None, :]).reshape(-1)
    pending = np.arange(BLOCK * visible_blocks(p), p + 1, dtype=np.int64)
    return np.concatenate([full, pending])


# ---------------------------------------------------------------- stage 3: sparse GQA

def sparse_gqa(q_bits, k_rows_bits, v_rows_bits, sm_scale: float):
    """Softmax attention of every query head over the given K/V rows [QSA]: the
    values come from the raw, uncompressed cache (R7).

    q_bits: [Hq, D]; k_rows_bits, v_rows_bits: [n, Hkv, D] -> (out [Hq, D], lse [Hq]).
    """
    return attention_f64(bf16_to_f64(q_bits), bf16_to_f64(k_rows_bits),
                         bf16_to_f64(v_rows_bits), sm_scale)


def sparse_gqa_fp8(q_bits, k_rows_codes, v_rows_codes, k_scale: float, v_scale: float,
                   sm_scale: float):
    """sparse_gqa over FP8 K/V rows (reading R9): the codes decoded and scaled by
    their pool's scale, then the same attention."""
    return attention_f64(bf16_to_f64(q_bits), e4m3_to_f64(k_rows_codes) * k_scale,
                         e4m3_to_f64(v_rows_codes) * v_scale, sm_scale)


def attention_f64(q, k, v, sm_scale: float):
    """Per-head softmax attention in float64 (R7): q [Hq, D], k and v [n, Hkv, D]."""
    hq, hkv = q.shape[0], k.shape[1]
    group = hq // hkv
    out = np.zeros_like(q)
    lse = np.zeros(hq)
    for h in range(hq):
        g = h // group
        logits = (k[:, g, :] @ q[h]) * sm_scale
        m = logits.max()
        e = np.exp(logits - m)
        out[h] = (e @ v[:, g, :]) / e.sum()
        lse[h] = m + np.log(e.sum())
    return out, lse


# ---------------------------------------------------------------- whole queries

def gather_rows(pool, page_row, positions, page_size: int):
    return np.asarray(pool)[token_slot(page_row, positions, page_size)]


def query(comp_bits, idx_q_bits, idx_w, q_bits, p: int, page_row, k_pool, v_pool,
          page_size: int, sm_scale: float, topk: int = TOPK_BLOCKS, kv_scales=None):
    """One query at position p through indexer and sparse GQA.

    comp_bits: the request's compressed keys in logical block order (at least
    visible_blocks(p) rows).  k_pool / v_pool hold bf16 bits, or FP8 E4M3 codes when
    kv_scales = (k_scale, v_scale) is given.  Returns a dict with scores,
    sel_blocks, positions, out and lse.
    """
    n_c = visible_blocks(p)
    scores = score_blocks(idx_q_bits, idx_w, comp_bits[:n_c])
    sel = select_blocks(scores, topk)
    pos = expand_positions(sel, p)
    out, lse = attend_positions(q_bits, pos, page_row, k_pool, v_pool, page_size, sm_scale,
                                kv_scales)
    return {"scores": scores, "sel_blocks": sel, "positions": pos, "out": out, "lse": lse}


def attend_positions(q_bits, pos, page_row, k_pool, v_pool, page_size: int, sm_scale: float,
                     kv_scales=None):
    """Sparse GQA of one query over logical positions `pos` of its request."""
    k = gather_rows(k_pool, page_row, pos, page_size)
    v = gather_rows(v_pool, page_row, pos, page_size)
    if kv_scales is None:
        return sparse_gqa(q_bits, k, v, sm_scale)
    return sparse_gqa_fp8(q_bits, k, v, kv_scales[0], kv_scales[1], sm_scale)


def indexshare_step(captured_positions, p_cap: int, j: int, q_bits, page_row, k_pool,
                    v_pool, page_size: int, sm_scale: float, kv_scales=None):
    """Reuse step j of the draft loop [IS] (reading R8): the captured selection
    plus the positions drafted since, without running the indexer."""
    pos = np.concatenate([np.asarray(captured_positions, dtype=np.int64),
                          np.arange(p_cap + 1, p_cap + j + 1, dtype=np.int64)])
    out, lse = attend_positions(q_bits, pos, page_row, k_pool, v_pool, page_size, sm_scale,
                                kv_scales)
    return {"positions": pos, "out": out, "lse": lse}


# ---------------------------------------------------------------- workload drivers
# These take any object with the fields of a synthetic workload (lengths,
# page_table, page_size, raw_idx_k, idx_q, idx_w, q, q_req, q_pos, k_pool, v_pool,
# rope_theta, prefix_len, reuse_q, reuse_steps; for kv = "fp8" also k_pool_fp8,
# v_pool_fp8, k_scale, v_scale).

def index_state(wl, b: int, length: int):
    mpos = getattr(wl, "mpos", None)
    if mpos is None:
        return build_index_state(wl.raw_idx_k[b], length, wl.rope_theta)
    return build_index_state(wl.raw_idx_k[b], length, wl.rope_theta, mpos[b], wl.pair_axis)


def kv_pools(wl, kv: str):
    """The workload's K/V pools and scales for kv = "bf16" or "fp8" (R9)."""
    if kv == "fp8":
        return wl.k_pool_fp8, wl.v_pool_fp8, (wl.k_scale, wl.v_scale)
    return wl.k_pool, wl.v_pool, None


def run_queries(wl, rows=None, sm_scale: float = 1.0 / 16.0, topk: int = TOPK_BLOCKS,
                kv: str = "bf16"):
    """Every (or the listed) query row of a decode / prefill / capture workload.

    The compressed keys a query sees are those of the request's complete blocks
    up to and including its own position; a block's key depends only on its own
    four tokens, so one build over the request's tokens serves every row.
    """
    k_pool, v_pool, scales = kv_pools(wl, kv)
    rows = range(wl.total_q) if rows is None else rows
    comp_of = {}
    res = {}
    for t in rows:
        b = int(wl.q_req[t])
        p = int(wl.q_pos[t])
        if b not in comp_of:
            comp_of[b], _ = index_state(wl, b, int(wl.lengths[b]))
        res[t] = query(comp_of[b], wl.idx_q[t], wl.idx_w[t], wl.q[t], p, wl.page_table[b],
                       k_pool, v_pool, wl.page_size, sm_scale, topk, scales)
    return res


def run_selections(wl, rows=None, chunk: int = 256):
    """Indexer results (scores, sel_blocks, positions) of every (or the listed) query
    row, without attention: the rows of a request are scored against its keys in
    batches of `chunk` queries (score_blocks_many), then selected and expanded one
    by one."""
    rows = list(range(wl.total_q)) if rows is None else list(rows)
    res = {}
    by_req = {}
    for t in rows:
        by_req.setdefault(int(wl.q_req[t]), []).append(t)
    for b, ts in by_req.items():
        comp, _ = index_state(wl, b, int(wl.lengths[b]))
        for i in range(0, len(ts), chunk):
            part = ts[i:i + chunk]
            n_max = max(visible_blocks(int(wl.q_pos[t])) for t in part)
            s_all = score_blocks_many(wl.idx_q[part], wl.idx_w[part], comp[:n_max])
            for j, t in enumerate(part):
                p = int(wl.q_pos[t])
                s = s_all[j, :visible_blocks(p)].copy()
                sel = select_blocks(s)
                res[t] = {"scores": s, "sel_blocks": sel, "positions": expand_positions(sel, p)}
    return res


def run_indexshare(wl, captured, sm_scale: float = 1.0 / 16.0, kv: str = "bf16"):
    """Reuse steps 1..reuse_steps for every request, from the capture results
    `captured` (as returned by run_queries)."""
    k_pool, v_pool, scales = kv_pools(wl, kv)
    res = {}
    for b in range(wl.batch):
        p_cap = int(wl.q_pos[b])
        for j in range(1, wl.reuse_steps + 1):
            res[(j, b)] = indexshare_step(captured[b]["positions"], p_cap, j,
                                          wl.reuse_q[j - 1, b], wl.page_table[b], k_pool,
                                          v_pool, wl.page_size, sm_scale, scales)
    return res
