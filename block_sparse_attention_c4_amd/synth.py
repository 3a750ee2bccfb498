"""Seeded synthetic inputs for the QSA c4 hot path.

This module only draws inputs. It computes nothing that the path computes: no
compressed keys, scores, selections or attention. It is the one module that both
the oracle tests and the HIP path read, so that both sides see the same bytes.

Recipe (all values are stored as bf16 bit patterns in ``uint16`` arrays, except
the per-head indexer weights, which are float32):

* values are standard normal float32 draws rounded to bf16 (round to nearest
  even); the indexer head weights w_h are U(0.5, 1.5);
* tensors are drawn in a fixed order: lengths, page permutation, raw index keys,
  index queries, weights, attention queries, K pool, V pool, hot block ids;
* large tensors are drawn in fixed chunks of 2**22 values, chunk i from child i of
  ``numpy.random.SeedSequence(seed)`` spawned for that tensor, so the values do
  not depend on how many threads draw them;
* "hot" blocks (the planted signal of the decode workloads): every raw index key
  of a hot block c is set to 0.8*sqrt(128) times the unit mean direction u of the
  request's index-query heads, turned back by the block's rotary phase, so that
  after the block is compressed at position 4c its key points along u.

Page layout: a page holds ``page_size`` consecutive token slots of one request.
``page_table[b, j]`` is the physical page of the request's j-th logical page
(-1 past the end). Token t of request b lives in slot
``page_table[b, t // page_size] * page_size + t % page_size`` of the K/V pools.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

PAGE_SIZE = 64
NUM_Q_HEADS = 16
NUM_KV_HEADS = 2
HEAD_DIM = 256
IDX_HEADS = 4
IDX_DIM = 128
ROPE_THETA = 1.0e7

_CHUNK = 1 << 22


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).copy()
    r = (b >> 16) & 1
    b += 0x7FFF
    b += r
    b >>= 16
    return b.astype(np.uint16)


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_bf16(seed_seq: np.random.SeedSequence, n: int) -> np.ndarray:
    """n standard-normal values as bf16 bits, drawn chunk by chunk."""
    out = np.empty(n, dtype=np.uint16)
    nch = (n + _CHUNK - 1) // _CHUNK
    kids = seed_seq.spawn(nch)

    def work(i: int) -> None:
        lo = i * _CHUNK
        hi = min(n, lo + _CHUNK)
        g = np.random.default_rng(kids[i])
        out[lo:hi] = f32_to_bf16_bits(g.standard_normal(hi - lo, dtype=np.float32))

    if nch == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nch)))
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    """One batch of synthetic inputs for a QSA layer.

    kind: "decode" (one query per request at p = L_b - 1), "prefill" (a chunk of
    new tokens per request appended to a cached prefix) or "indexshare" (decode at
    the capture token, then reuse steps that append positions).
    """

    name: str
    kind: str
    seed: int
    lengths: np.ndarray            # [B] tokens in each request's cache incl. the query token(s)
    alloc_tokens: np.ndarray       # [B] token slots reserved per request (>= lengths)
    page_size: int
    page_table: np.ndarray         # [B, max_pages] int32, -1 padded
    num_pages: int
    raw_idx_k: list                # B arrays [L_b, 128] uint16: raw indexer keys of tokens 0..L_b-1
    idx_q: np.ndarray              # [T, 4, 128] uint16 (post-rotary indexer queries)
    idx_w: np.ndarray              # [T, 4] float32
    q: np.ndarray                  # [T, 16, 256] uint16 (post-rotary attention queries)
    q_req: np.ndarray              # [T] int32 request of each query
    q_pos: np.ndarray              # [T] int32 position of each query
    k_pool: np.ndarray             # [num_pages*page_size, 2, 256] uint16
    v_pool: np.ndarray             # [num_pages*page_size, 2, 256] uint16
    prefix_len: np.ndarray         # [B] tokens whose indexer keys are ingested before the step
    hot_blocks: list = field(default_factory=list)   # B arrays of planted block ids
    reuse_q: np.ndarray | None = None                # [steps, B, 16, 256] uint16 (indexshare)
    reuse_steps: int = 0
    rope_theta: float = ROPE_THETA
    k_pool_fp8: np.ndarray | None = None             # FP8 E4M3 codes of the pools (uint8), and
    v_pool_fp8: np.ndarray | None = None             # their per-pool scales
    k_scale: float = 1.0
    v_scale: float = 1.0
    mpos: list | None = None                         # B arrays [L_b, 3] int32: 3-D (MRoPE) positions
    pair_axis: np.ndarray | None = None              # [64] uint8: position component of each rotary pair

    @property
    def batch(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.q_pos.shape[0])


def _page_table(rng: np.random.Generator, alloc_tokens: np.ndarray, page_size: int,
                order: str) -> tuple[np.ndarray, int]:
    pages = (alloc_tokens + page_size - 1) // page_size
    total = int(pages.sum())
    if order == "identity":
        perm = np.arange(total, dtype=np.int64)
    elif order == "shuffled":
        perm = rng.permutation(total)
    else:
        raise ValueError(order)
    pt = np.full((len(pages), int(pages.max())), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages):
        pt[b, :n] = perm[off:off + n]
        off += int(n)
    return pt, total


def _turn_back(u: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """u turned by the rotary phase of position -pos (pairs (i, i+64))."""
    half = u.shape[0] // 2
    ang = -float(pos) * theta ** (-np.arange(half, dtype=np.float64) * 2.0 / u.shape[0])
    c, s = np.cos(ang), np.sin(ang)
    a, b = u[:half], u[half:]
    return np.concatenate([a * c - b * s, b * c + a * s])


def make_workload(name: str, kind: str, seed: int, lengths, *, hot_per_req: int = 0,
                  page_order: str = "shuffled", chunk: int = 0, reuse_steps: int = 0,
                  page_size: int = PAGE_SIZE, rope_theta: float = ROPE_THETA,
                  draw_lengths=None) -> Workload:
    """Draw a workload.

    decode:     one query per request at p = L_b - 1; prefix_len = L_b - 1.
    prefill:    ``chunk`` queries per request at positions L_b - chunk .. L_b - 1;
                prefix_len = L_b - chunk.
    indexshare: like decode (the capture query at p = L_b - 1), plus ``reuse_steps``
                fresh attention queries per request for positions L_b .. L_b+steps-1.
    ``draw_lengths(rng)`` (optional) draws the lengths from the workload's own
    generator, so that lengths are the first thing drawn.
    """
    root = np.random.SeedSequence(seed)
    s_len, s_perm, s_rk, s_iq, s_w, s_q, s_k, s_v, s_hot, s_rq = root.spawn(10)
    if draw_lengths is not None:
        lengths = draw_lengths(np.random.default_rng(s_len))
    lengths = np.asarray(lengths, dtype=np.int64)
    B = len(lengths)
    extra = reuse_steps if kind == "indexshare" else 0
    alloc = lengths + extra
    pt, num_pages = _page_table(np.random.default_rng(s_perm), alloc, page_size, page_order)

    if kind in ("decode", "indexshare"):
        prefix = lengths - 1
        q_req = np.arange(B, dtype=np.int32)
        q_pos = (lengths - 1).astype(np.int32)
    elif kind == "prefill":
        assert chunk > 0 and np.all(lengths >= chunk)
        prefix = lengths - chunk
        q_req = np.repeat(np.arange(B, dtype=np.int32), chunk)
        q_pos = np.concatenate([np.arange(L - chunk, L, dtype=np.int32) for L in lengths])
    else:
        raise ValueError(kind)
    T = len(q_pos)

    flat_rk = _normal_bf16(s_rk, int(lengths.sum()) * IDX_DIM).reshape(-1, IDX_DIM)
    offs = np.concatenate([[0], np.cumsum(lengths)])
    raw_idx_k = [flat_rk[offs[b]:offs[b + 1]] for b in range(B)]
    idx_q = _normal_bf16(s_iq, T * IDX_HEADS * IDX_DIM).reshape(T, IDX_HEADS, IDX_DIM)
    idx_w = np.random.default_rng(s_w).uniform(0.5, 1.5, size=(T, IDX_HEADS)).astype(np.float32)
    q = _normal_bf16(s_q, T * NUM_Q_HEADS * HEAD_DIM).reshape(T, NUM_Q_HEADS, HEAD_DIM)
    nslots = num_pages * page_size
    k_pool = _normal_bf16(s_k, nslots * NUM_KV_HEADS * HEAD_DIM).reshape(nslots, NUM_KV_HEADS, HEAD_DIM)
    v_pool = _normal_bf16(s_v, nslots * NUM_KV_HEADS * HEAD_DIM).reshape(nslots, NUM_KV_HEADS, HEAD_DIM)

    hot_blocks = []
    g_hot = np.random.default_rng(s_hot)
    for b in range(B):
        n_c = int(lengths[b]) // 4
        k = min(hot_per_req, n_c)
        ids = np.sort(g_hot.choice(n_c, size=k, replace=False)) if k else np.zeros(0, np.int64)
        hot_blocks.append(ids)
        if k:
            # direction of the request's (first) query's indexer heads
            tq = int(np.nonzero(q_req == b)[0][-1])
            u = bf16_bits_to_f32(idx_q[tq]).astype(np.float64).mean(axis=0)
            u /= np.linalg.norm(u)
            for c in ids:
                v = 0.8 * math.sqrt(IDX_DIM) * _turn_back(u, 4 * int(c), rope_theta)
                raw_idx_k[b][4 * c:4 * c + 4] = f32_to_bf16_bits(v.astype(np.float32))[None, :]

    reuse_q = None
    if kind == "indexshare" and reuse_steps:
        reuse_q = _normal_bf16(s_rq, reuse_steps * B * NUM_Q_HEADS * HEAD_DIM).reshape(
            reuse_steps, B, NUM_Q_HEADS, HEAD_DIM)

    return Workload(name=name, kind=kind, seed=seed, lengths=lengths, alloc_tokens=alloc,
                    page_size=page_size, page_table=pt, num_pages=num_pages,
                    raw_idx_k=raw_idx_k, idx_q=idx_q, idx_w=idx_w, q=q, q_req=q_req,
                    q_pos=q_pos, k_pool=k_pool, v_pool=v_pool,
                    prefix_len=prefix.astype(np.int64), hot_blocks=hot_blocks,
                    reuse_q=reuse_q, reuse_steps=reuse_steps if kind == "indexshare" else 0,
                    rope_theta=rope_theta)


def with_fp8_kv(wl: Workload) -> Workload:
    """Add FP8 E4M3 copies of the K/V pools: each pool's bf16 values divided by one
    scale (its largest magnitude / 448) and rounded to nearest even by torch's
    float8_e4m3fn conversion."""
    import torch

    def quantize(pool_bits):
        x = torch.from_numpy(bf16_bits_to_f32(pool_bits))
        scale = float(x.abs().max()) / 448.0
        if scale == 0.0:
            scale = 1.0
        codes = (x / scale).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        return codes, scale

    wl.k_pool_fp8, wl.k_scale = quantize(wl.k_pool)
    wl.v_pool_fp8, wl.v_scale = quantize(wl.v_pool)
    return wl


def contiguous_pair_axis(sections=(16, 24, 24)) -> np.ndarray:
    """Axis map of contiguous MRoPE sections: the first sections[0] rotary pairs take
    the temporal component, the next sections[1] the height, the rest the width."""
    return np.repeat(np.arange(3), sections).astype(np.uint8)


def mrope_positions(length: int, images) -> np.ndarray:
    """3-D positions [length, 3] of a token stream with vision spans.

    images: (start, T, H, W) tuples, sorted, non-overlapping: T*H*W vision tokens
    from sequence index `start`.  A text token has (p, p, p), p counting on from the
    previous token; a vision token k of a span whose first position is p0 has
    (p0 + k // (H*W), p0 + (k // W) % H, p0 + k % W); text after a span resumes at
    p0 + max(T, H, W)."""
    pos = np.zeros((length, 3), dtype=np.int32)
    nxt, t = 0, 0
    for start, T, H, W in list(images) + [(length, 0, 0, 0)]:
        while t < min(start, length):
            pos[t] = nxt
            nxt += 1
            t += 1
        n = min(T * H * W, length - t)
        if n <= 0:
            continue
        k = np.arange(n)
        pos[t:t + n, 0] = nxt + k // (H * W)
        pos[t:t + n, 1] = nxt + (k // W) % H
        pos[t:t + n, 2] = nxt + k % W
        t += n
        nxt += max(T, H, W)
    return pos


def with_mrope(wl: Workload, images_per_request, pair_axis=None) -> Workload:
    """Give every request of wl 3-D positions with the listed vision spans."""
    wl.mpos = [mrope_positions(int(L), imgs) for L, imgs in zip(wl.lengths, images_per_request)]
    wl.pair_axis = contiguous_pair_axis() if pair_axis is None else np.asarray(pair_axis, np.uint8)
    return wl


# --- the five workloads at full size ------------------------------------------------

def _loguniform_lengths(B: int, lo: int, hi: int):
    def draw(rng):
        return np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=B))).astype(np.int64)
    return draw


def _plus_pending(B: int, base: int):
    def draw(rng):
        return base + rng.integers(0, 4, size=B)
    return draw


def decode_b1_l4099(seed: int = 1001) -> Workload:
    """Batch 1, L = 4099 (1024 complete blocks, 3 pending), 8 hot blocks, identity pages."""
    return make_workload("decode_b1_l4099", "decode", seed, [4099], hot_per_req=8,
                         page_order="identity")


def decode_b8_l32k(seed: int = 1002) -> Workload:
    """Batch 8, L_b = 32768 + U{0..3}, 32 hot blocks per request, shuffled pages."""
    return make_workload("decode_b8_l32k", "decode", seed, None, hot_per_req=32,
                         page_order="shuffled", draw_lengths=_plus_pending(8, 32768))


def decode_b32_mixed(seed: int = 1003) -> Workload:
    """Batch 32, L_b log-uniform in [4096, 131072], one shared pool, interleaved pages."""
    return make_workload("decode_b32_loguniform_4k_128k", "decode", seed, None,
                         page_order="shuffled", draw_lengths=_loguniform_lengths(32, 4096, 131072))


def prefill_4096_on_126976(seed: int = 1004) -> Workload:
    """Batch 1: 4096 new tokens appended to a 126976-token cached prefix."""
    return make_workload("prefill_chunk4096_prefix126976", "prefill", seed, [131072], chunk=4096,
                         page_order="shuffled")


def indexshare_b4_l262140(seed: int = 1005) -> Workload:
    """Batch 4, L = 262140; capture at p = 262139, then 3 reuse steps at 262140..262142."""
    return make_workload("indexshare_b4_l262140", "indexshare", seed, [262140] * 4,
                         page_order="shuffled", reuse_steps=3)


# the MRoPE prefill chunk: a 4 x 32 x 32 video span at index 20000 of the prefix, and
# the 4096-token chunk one 64 x 64 image
PREFILL_MROPE_SPANS = [[(20000, 4, 32, 32), (126976, 1, 64, 64)]]


def prefill_4096_on_126976_mrope(seed: int = 1004) -> Workload:
    """The prefill chunk with MRoPE positions (PREFILL_MROPE_SPANS, contiguous 16/24/24
    axis map)."""
    wl = prefill_4096_on_126976(seed)
    wl.name = "prefill_chunk4096_prefix126976_mrope"
    return with_mrope(wl, PREFILL_MROPE_SPANS)


def decode_b8_l131072(seed: int = 1007) -> Workload:
    """Batch 8 at exactly L = 131072 (32768 complete blocks, no pending token): the
    literal 128K decode point, shuffled pages."""
    return make_workload("decode_b8_l131072", "decode", seed, [131072] * 8, page_order="shuffled")


def verify_b32_loguniform(seed: int = 1006) -> Workload:
    """Target verification of drafted tokens: batch 32, 4 query tokens per request (the
    capture token plus 3 drafts) at the end of a cache of log-uniform length in
    [4096, 131072]; every query has its own selection."""
    return make_workload("verify_b32x4_loguniform_4k_128k", "prefill", seed, None, chunk=4,
                         page_order="shuffled", draw_lengths=_loguniform_lengths(32, 4096, 131072))


FULL_SIZE = {
    "decode_b1_l4099": decode_b1_l4099,
    "decode_b8_l32k": decode_b8_l32k,
    "decode_b32_loguniform_4k_128k": decode_b32_mixed,
    "prefill_chunk4096_prefix126976": prefill_4096_on_126976,
    "indexshare_b4_l262140": indexshare_b4_l262140,
    "verify_b32x4_loguniform_4k_128k": verify_b32_loguniform,
    "decode_b8_l131072": decode_b8_l131072,
    "prefill_chunk4096_prefix126976_mrope": prefill_4096_on_126976_mrope,
}
