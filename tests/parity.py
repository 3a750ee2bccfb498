"""Comparison helpers for the GPU parity tests (HIP path vs the CPU oracle).

Tolerances:
  * compressed keys: within 1 bf16 ulp of the oracle's key;
  * selection: the kept block set equals the oracle's, except that a block may be
    swapped for another only where both lie within 1e-5 (relative) of the
    oracle's 512th score (a boundary tie in float32 vs float64 arithmetic);
  * positions, counts, ring contents: bit exact;
  * attention output (bf16) vs the float64 oracle: max-abs <= 2e-2 and mean-abs
    <= 2e-3 per query; lse within 2e-4 absolute (natural log).
"""

from __future__ import annotations

import sys

import numpy as np

from oracle import qsa_oracle as O

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
LSE_ABS = 2e-4
TIE_REL = 1e-5


def log(*a) -> None:
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 steps between bit patterns (monotone integer mapping)."""
    def ordered(u):
        u = np.asarray(u, dtype=np.uint16).astype(np.int32)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def oracle_index_states(wl, lengths=None):
    """Oracle compressed keys and rings of every request after `lengths` tokens."""
    lengths = wl.lengths if lengths is None else lengths
    out = []
    for b in range(wl.batch):
        out.append(O.index_state(wl, b, int(lengths[b])))
    return out


def check_comp_cache(wl, gpu_comp: np.ndarray, states) -> tuple[int, int]:
    """Every complete block's key in the GPU compressed cache vs the oracle.
    Returns (blocks compared, blocks not bit-identical)."""
    n_all = 0
    n_diff = 0
    for b, (comp, _) in enumerate(states):
        if comp.shape[0] == 0:
            continue
        slots = O.comp_slot(wl.page_table[b], np.arange(comp.shape[0]), wl.page_size)
        got = gpu_comp[slots]
        d = bf16_ulp_distance(got, comp)
        assert d.max() <= 1, f"request {b}: compressed key off by {d.max()} bf16 ulps"
        n_all += comp.shape[0]
        n_diff += int(np.count_nonzero(d.max(axis=1)))
    return n_all, n_diff


def check_ring(gpu_ring: np.ndarray, states) -> None:
    for b, (_, ring) in enumerate(states):
        for slot, key in ring.items():
            np.testing.assert_array_equal(gpu_ring[b, slot], key, err_msg=f"ring of request {b} slot {slot}")


def kth_score(scores: np.ndarray, k: int) -> float:
    return float(np.sort(scores)[::-1][k - 1])


def check_selection(gpu_blocks_row: np.ndarray, res: dict, where: str, exact: bool = False) -> bool:
    """GPU kept blocks vs the oracle's; returns True if identical.

    A difference is allowed only between blocks whose oracle scores lie within
    TIE_REL of the oracle's 512th score (float32 against float64 arithmetic), and
    never across an exact tie: a kept block and a dropped block with equal oracle
    scores must follow the tie rule (lower index kept).  Equal oracle scores come
    from equal inputs (zero keys, a zero query, ReLU's zeros), on which the GPU's
    float32 scores are equal too.  exact=True demands the oracle's set."""
    scores = res["scores"]
    want = res["sel_blocks"]
    n = scores.shape[0]
    k = min(n, O.TOPK_BLOCKS)
    got = gpu_blocks_row[gpu_blocks_row >= 0]
    assert np.all(gpu_blocks_row[k:] == -1), f"{where}: row not padded with -1"
    assert len(got) == k, f"{where}: kept {len(got)} blocks, want {k}"
    assert np.all(np.diff(got) > 0) and (k == 0 or got[-1] < n), f"{where}: not ascending / out of range"
    if np.array_equal(got, want):
        return True
    d_in = np.setdiff1d(got, want)      # kept by the GPU only
    d_out = np.setdiff1d(want, got)     # kept by the oracle only
    assert not exact, (f"{where}: selection differs where it must be exact: GPU-only blocks "
                       f"{d_in[:8]} (scores {scores[d_in[:8]]}), oracle-only {d_out[:8]} "
                       f"(scores {scores[d_out[:8]]})")
    s_k = kth_score(scores, k)
    tol = TIE_REL * max(abs(s_k), 1e-6)
    diff = np.concatenate([d_in, d_out])
    bad = diff[np.abs(scores[diff] - s_k) > tol]
    assert bad.size == 0, (f"{where}: selection differs beyond boundary ties: blocks {bad[:8]} "
                           f"scores {scores[bad[:8]]} vs 512th {s_k}")
    for a in d_in:
        broken = d_out[(scores[d_out] == scores[a]) & (d_out < a)]
        assert broken.size == 0, (f"{where}: exact tie resolved against the lower index: kept {a}, "
                                  f"dropped {broken[:4]} (score {scores[a]})")
    return False


def check_positions(gpu_pos_row: np.ndarray, gpu_count: int, res: dict, where: str) -> None:
    want = res["positions"]
    assert gpu_count == len(want), f"{where}: count {gpu_count} want {len(want)}"
    np.testing.assert_array_equal(gpu_pos_row[:gpu_count], want, err_msg=where)
    assert np.all(gpu_pos_row[gpu_count:] == -1), f"{where}: tail not -1"


def check_positions_valid(gpu_pos_row, gpu_count, gpu_blocks_row, p: int, where: str) -> None:
    """Validity of a row whose kept set legitimately differs from the oracle's."""
    blocks = gpu_blocks_row[gpu_blocks_row >= 0]
    n_c = (p + 1) // 4
    want = np.concatenate([(4 * blocks[:, None] + np.arange(4)).reshape(-1),
                           np.arange(4 * n_c, p + 1)])
    assert gpu_count == len(want), where
    np.testing.assert_array_equal(gpu_pos_row[:gpu_count], want, err_msg=where)


def oracle_on_gpu_positions(wl, t: int, gpu_pos_row, gpu_count: int, kv: str = "bf16",
                            sm_scale: float = 1.0 / 16.0) -> dict:
    """The oracle's attention for query row t over the positions the GPU selected
    (for a row whose kept set legitimately differs from the oracle's at a tie)."""
    k_pool, v_pool, scales = O.kv_pools(wl, kv)
    b = int(wl.q_req[t])
    pos = np.asarray(gpu_pos_row[:gpu_count], dtype=np.int64)
    out, lse = O.attend_positions(wl.q[t], pos, wl.page_table[b], k_pool, v_pool, wl.page_size,
                                  sm_scale, scales)
    return {"positions": pos, "out": out, "lse": lse}


def check_attention(gpu_out: np.ndarray, gpu_lse: np.ndarray, res: dict, where: str):
    err = np.abs(gpu_out - res["out"])
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{where}: max-abs {mx:.3e} mean-abs {mean:.3e}"
    le = float(np.abs(gpu_lse - res["lse"]).max())
    assert le <= LSE_ABS, f"{where}: lse off by {le:.3e}"
    return mx, mean, le
