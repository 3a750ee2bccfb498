"""GPU parity over seeded random shapes.

The other parity cases use pages of 16 and 64 tokens.  Here every case draws its
page size from 32, 48, 80, 128 and 256 tokens (pages that split a 16-block group
at a point that is not a power of two, and pages that hold several groups), its
batch, its context lengths (log-uniform, tiny ones included) and its chunk size,
all from the case's seed.  Each path runs end to end and is checked on every row
against the oracle: decode through the separate builder and indexer calls and
through the folded call, prefill chunks through the MFMA scorer and through the
multi-query scorer, target verification, and IndexShare reuse steps; decode and
prefill also with FP8 K/V pools.
"""

import numpy as np
import pytest

from block_sparse_attention_c4_amd import synth
from tests import test_gpu_parity as G

pytestmark = pytest.mark.gpu

PAGE_SIZES = (32, 48, 80, 128, 256)


def _lengths(rng, n, lo, hi):
    """n lengths log-uniform in [lo, hi]; one of them at most 6 when lo allows it."""
    x = np.exp(rng.uniform(np.log(lo), np.log(hi), size=n)).astype(np.int64)
    if lo <= 6 and n > 1:
        x[rng.integers(n)] = rng.integers(lo, 7)
    return np.maximum(x, lo)


def _case(kind, seed):
    """(workload, description) of the case's seed."""
    rng = np.random.default_rng(seed)
    ps = int(rng.choice(PAGE_SIZES))
    name = f"{kind}_s{seed}_p{ps}"
    if kind == "decode":
        B = int(rng.integers(1, 13))
        return synth.make_workload(name, "decode", seed, _lengths(rng, B, 1, 40000),
                                   hot_per_req=int(rng.integers(0, 5)), page_size=ps)
    if kind == "prefill_mfma":     # at least 64 queries and 16 per request
        B = int(rng.integers(1, 4))
        chunk = int(rng.integers(max(16, (64 + B - 1) // B), 81))
        return synth.make_workload(name, "prefill", seed, _lengths(rng, B, chunk, 40000),
                                   chunk=chunk, hot_per_req=int(rng.integers(0, 5)), page_size=ps)
    if kind == "prefill_multi":    # 2..8 queries per request
        B = int(rng.integers(2, 13))
        chunk = int(rng.integers(2, 9))
        return synth.make_workload(name, "prefill", seed, _lengths(rng, B, chunk, 40000),
                                   chunk=chunk, page_size=ps)
    if kind == "indexshare":
        B = int(rng.integers(1, 5))
        return synth.make_workload(name, "indexshare", seed, _lengths(rng, B, 1, 40000),
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
