"""GPU parity over seeded random shapes.

The other parity cases use pages of 16 and 64 tokens.  Here every case draws its
page size from 32, 48, 80, 128 and 256 tokens (pages that split a 16-block group
at a point that is not a power of two, and pages that hold several groups), its
batch, its context lengths (log-uniform, tiny ones included) and its chunk size,
all from the case's seed.  Each path runs end to end and is checked on every row
against the oracle: decode through the separate builder and indexer calls and
through the folded call, prefill chunks through the MFMA scorer and through the
multi-query scorer, target verification, and IndexShare reuse steps; decode and
prefill also with FP8 K/V pools, and with 3-D MRoPE positions (random vision spans,
random maps of rotary pairs to axes).

An optional wide sweep (QSA_SHAPE_SWEEP=first:last, one case per seed) draws every
page size from 16 to 256 tokens, contexts up to 262144 positions, batches up to 70
requests and chunks up to 199 queries.
"""

import os

import numpy as np
import pytest

from block_sparse_attention_c4_amd import synth
from tests import test_gpu_parity as G

pytestmark = pytest.mark.gpu

PAGE_SIZES = (32, 48, 80, 128, 256)
# the optional wide sweep also draws the pages the other cases use
WIDE_PAGE_SIZES = (16, 32, 48, 64, 80, 128, 256)
KINDS = ("decode", "prefill_mfma", "prefill_multi", "indexshare")


def _lengths(rng, n, lo, hi):
    """n lengths log-uniform in [lo, hi]; one of them at most 6 when lo allows it."""
    x = np.exp(rng.uniform(np.log(lo), np.log(hi), size=n)).astype(np.int64)
    if lo <= 6 and n > 1:
        x[rng.integers(n)] = rng.integers(lo, 7)
    return np.maximum(x, lo)


def _case(kind, seed, wide=False):
    """The workload of the case's seed.  wide: contexts up to 262144 positions,
    batches up to 70 requests, chunks up to 199 queries, every page size."""
    rng = np.random.default_rng(seed)
    ps = int(rng.choice(WIDE_PAGE_SIZES if wide else PAGE_SIZES))
    name = f"{'w' if wide else ''}{kind}_s{seed}_p{ps}"
    if kind == "decode":
        B = int(rng.choice((1, 3, 17, 40, 70))) if wide else int(rng.integers(1, 13))
        return synth.make_workload(name, "decode", seed,
                                   _lengths(rng, B, 1, 262144 if wide else 40000),
                                   hot_per_req=int(rng.integers(0, 9 if wide else 5)), page_size=ps)
    if kind == "prefill_mfma":     # at least 64 queries and 16 per request
        B = int(rng.integers(1, 4))
        chunk = int(rng.integers(max(16, (64 + B - 1) // B), 200 if wide else 81))
        return synth.make_workload(name, "prefill", seed,
                                   _lengths(rng, B, chunk, 140000 if wide else 40000),
                                   chunk=chunk, hot_per_req=int(rng.integers(0, 9 if wide else 5)),
                                   page_size=ps)
    if kind == "prefill_multi":    # 2..8 queries per request
        B = int(rng.integers(2, 40 if wide else 13))
        chunk = int(rng.integers(2, 9))
        return synth.make_workload(name, "prefill", seed,
                                   _lengths(rng, B, chunk, 140000 if wide else 40000),
                                   chunk=chunk, page_size=ps)
    if kind == "indexshare":
        B = int(rng.integers(1, 6 if wide else 5))
        return synth.make_workload(name, "indexshare", seed,
                                   _lengths(rng, B, 1, 262140 if wide else 40000),
                                   reuse_steps=3, page_size=ps)
    raise ValueError(kind)


CASES = ([("decode", s) for s in range(401, 409)]
         + [("prefill_mfma", s) for s in range(411, 416)]
         + [("prefill_multi", s) for s in range(421, 426)]
         + [("indexshare", s) for s in range(431, 434)])

# FP8 E4M3 K/V pools: the same draws, with FP8 copies of the pools
FP8_CASES = [("decode", s) for s in (441, 442)] + [("prefill_mfma", s) for s in (451, 452)]


def _log(wl):
    G.P.log(f"[shape] {wl.name}: B={wl.batch} T={wl.total_q} lengths={wl.lengths.tolist()}")


@pytest.mark.parametrize("kind,seed", CASES)
def test_random_shape_end_to_end(kind, seed):
    wl = _case(kind, seed)
    _log(wl)
    if kind == "indexshare":
        G._check_indexshare(wl)
        return
    G._check_e2e(wl)
    if kind == "decode":
        G._check_fused_equals_separate(wl)
        G._check_e2e_fused(wl)


@pytest.mark.parametrize("kind,seed", FP8_CASES)
def test_random_shape_end_to_end_fp8(kind, seed):
    wl = synth.with_fp8_kv(_case(kind, seed))
    _log(wl)
    G._check_e2e(wl, kv="fp8")


def _spans(rng, L):
    """0-3 sorted, non-overlapping vision spans (start, T, H, W) in a stream of L tokens
    (a span may run past the end, which cuts it)."""
    out, t = [], 0
    for _ in range(int(rng.integers(0, 4))):
        if t >= L:
            break
        T, H, W = int(rng.integers(1, 4)), int(rng.integers(1, 33)), int(rng.integers(1, 33))
        start = int(rng.integers(t, L))
        out.append((start, T, H, W))
        t = start + T * H * W
    return out


def _mrope_case(kind, seed):
    """A case of _case with 3-D positions: random vision spans per request and a
    contiguous, interleaved or random map of rotary pairs to axes."""
    wl = _case(kind, seed)
    rng = np.random.default_rng(seed + 7919)
    pick = int(rng.integers(3))
    axis = None if pick == 0 else (np.arange(64) % 3 if pick == 1 else rng.integers(0, 3, size=64))
    return synth.with_mrope(wl, [_spans(rng, int(L)) for L in wl.lengths], pair_axis=axis)


MROPE_CASES = ([("decode", s) for s in (461, 462, 463)]
               + [("prefill_mfma", s) for s in (471, 472)] + [("prefill_multi", s) for s in (481, 482)])


@pytest.mark.parametrize("kind,seed", MROPE_CASES)
def test_random_shape_end_to_end_mrope(kind, seed):
    wl = _mrope_case(kind, seed)
    _log(wl)
    G._check_e2e(wl)
    if kind == "decode":
        G._check_fused_equals_separate(wl)
        G._check_e2e_fused(wl)


def _sweep_seeds():
    """Seeds of the optional wide sweep, QSA_SHAPE_SWEEP="first:last" (unset: none)."""
    spec = os.environ.get("QSA_SHAPE_SWEEP", "")
    if not spec:
        return []
    first, last = (int(x) for x in spec.split(":"))
    return list(range(first, last))


@pytest.mark.skipif(not _sweep_seeds(), reason="the wide sweep runs with QSA_SHAPE_SWEEP=first:last")
@pytest.mark.parametrize("seed", _sweep_seeds() or [0])
def test_random_shape_sweep(seed):
    """Wide shapes: the path is seed % 4 of KINDS; every fifth seed of the decode and
    MFMA-prefill paths uses FP8 pools.  Prefill chunks through the MFMA scorer check
    the attention of 64 sampled rows (the selection of every row)."""
    kind = KINDS[seed % 4]
    fp8 = seed % 5 == 0 and kind in ("decode", "prefill_mfma")
    wl = _case(kind, seed, wide=True)
    if fp8:
        wl = synth.with_fp8_kv(wl)
    _log(wl)
    try:
        if kind == "indexshare":
            G._check_indexshare(wl)
        else:
            G._check_e2e(wl, sample=64 if kind == "prefill_mfma" else None, kv="fp8" if fp8 else "bf16")
            if kind == "decode" and not fp8:
                G._check_fused_equals_separate(wl)
    finally:
        G._CACHE.clear()

