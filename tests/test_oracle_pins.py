"""Pins for the CPU oracle: closed forms, hand-derived values, invariants, library
special cases and brute force on tiny inputs.  None of these re-types the oracle's
own formula; each is chosen so that a plausible slip in the oracle (a dropped term,
a wrong sign or index, a transposed operand, a wrong tie rule) fails one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from block_sparse_attention_c4_amd import synth
from oracle import qsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits(values):
    return synth.f32_to_bf16_bits(np.asarray(values, dtype=np.float32))


# ------------------------------------------------------------------ bf16 rounding

def test_round_to_bf16_ties_and_grid():
    # spacing of bf16 just above 1 is 2**-7; midpoints go to the even neighbour
    x = np.array([1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-30, -(1 + 2**-8), 0.0, 2**-133, 3 * 2**-134])
    want = np.array([1.0, 1 + 2**-6, 1 + 2**-7, -1.0, 0.0, 2**-133, 2**-132])
    np.testing.assert_array_equal(O.round_to_bf16(x), want)


def test_round_to_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e-39,
                        rng.standard_normal(2000) * 1e30]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_to_bf16(x.astype(np.float64)), ref)
    np.testing.assert_array_equal(O.f64_to_bf16_bits(x.astype(np.float64)),
                                  torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


# ------------------------------------------------------------------ paged addressing

def test_token_and_comp_slots_by_hand():
    row = np.array([5, 2, 9])
    # page size 64: token t -> row[t//64]*64 + t%64
    assert list(O.token_slot(row, [0, 63, 64, 100, 128], 64)) == [320, 383, 128, 164, 576]
    # block c -> full slot of token 4c, divided by 4 (16 blocks per page)
    assert list(O.comp_slot(row, [0, 15, 16, 20, 32], 64)) == [80, 95, 32, 36, 144]


# ------------------------------------------------------------------ stage 1: compressed keys

def _golden_raw():
    g = json.load(open(os.path.join(GOLDEN, "compress_two_blocks.json")))
    raw = np.zeros((8, g["dim"]), dtype=np.float32)
    for t, dims in g["raw_keys"].items():
        for d, v in dims.items():
            raw[int(t), int(d)] = v
    return g, bits(raw)


def test_compress_two_blocks_hand_example():
    g, raw = _golden_raw()
    comp, ring = O.build_index_state(raw, 8, g["theta"])
    assert comp.shape == (2, 128) and ring == {}
    got = O.bf16_to_f64(comp)
    for bi, blk in enumerate(["block0", "block1"]):
        want = np.zeros(128)
        for d, v in g["expected_bf16"][blk].items():
            want[int(d)] = v
        np.testing.assert_array_equal(got[bi], want)


def test_compress_two_blocks_unrounded_closed_form():
    g, raw = _golden_raw()
    m = O.block_mean_fp32(raw.reshape(2, 4, 128)).astype(np.float64)
    kbar = m / np.linalg.norm(m, axis=1, keepdims=True)
    y = O.rotate(kbar, np.array([0, 4]), g["theta"])
    a1 = 4.0 * 1e7 ** (-2.0 / 128)
    closed = {0: (3 * math.cos(4) - 4 * math.sin(4)) / 13, 64: (4 * math.cos(4) + 3 * math.sin(4)) / 13,
              1: 12 / 13 * math.cos(a1), 65: 12 / 13 * math.sin(a1)}
    for d, v in closed.items():
        assert abs(y[1, d] - v) < 1e-14
        assert abs(y[1, d] - g["exact"]["block1"][str(d)]) < 1e-10
    assert abs(y[0, 0] - 2 ** -0.5) < 1e-15 and abs(y[0, 1] - 2 ** -0.5) < 1e-15


def test_compressed_keys_are_unit_norm_and_zero_block_stays_zero():
    rng = np.random.default_rng(11)
    raw = bits(rng.standard_normal((64, 128)))
    raw[8:12] = 0                                  # block 2 all zero
    comp, _ = O.build_index_state(raw, 64, 1e7)
    k = O.bf16_to_f64(comp)
    norms = np.linalg.norm(k, axis=1)
    # each element moves by at most half a bf16 ulp (<= 2**-9 relative)
    assert np.all(np.abs(norms[np.arange(16) != 2] - 1) < 2 ** -8)
    assert np.all(k[2] == 0)


def test_compress_uses_all_four_tokens():
    # keys e0, e0, e0, 5 e1 at position 0: mean (3 e0 + 5 e1)/4, unit (3, 5)/sqrt(34)
    raw = np.zeros((4, 128), np.float32)
    raw[0:3, 0] = 1.0
    raw[3, 1] = 5.0
    comp, _ = O.build_index_state(bits(raw), 4, 1e7)
    k = O.bf16_to_f64(comp[0])
    assert k[0] == O.round_to_bf16(3 / math.sqrt(34)) == 0.515625
    assert k[1] == O.round_to_bf16(5 / math.sqrt(34)) == 0.859375
    assert np.count_nonzero(k) == 2


def test_block_mean_is_fp32_in_token_order():
    # 256 + 2**-20 rounds to 256 in FP32, so the FP32 mean of (256, 2**-20, -256, 0)
    # is 0 while the exact mean is 2**-22 (reading R4)
    raw = np.zeros((4, 128), np.float32)
    raw[:, 0] = [256.0, 2.0**-20, -256.0, 0.0]
    raw[:, 1] = 1.0
    m = O.block_mean_fp32(bits(raw)[None])[0]
    assert m[0] == 0.0 and m[1] == 1.0


def test_rotary_phase_properties():
    rng = np.random.default_rng(5)
    x, y = rng.standard_normal((2, 128))
    th = 1e7
    # phases add
    np.testing.assert_allclose(O.rotate(O.rotate(x, 1000, th), 2345, th), O.rotate(x, 3345, th), atol=1e-12)
    # inner products depend only on the position difference
    a = O.rotate(x, 777, th) @ O.rotate(y, 77, th)
    b = O.rotate(x, 700, th) @ O.rotate(y, 0, th)
    assert abs(a - b) < 1e-10
    # the last pair turns slowest: theta**(-126/128) per position
    e = np.zeros(128)
    e[63] = 1.0
    r = O.rotate(e, 10**6, th)
    ang = 10**6 * th ** (-126 / 128)
    assert abs(r[63] - math.cos(ang)) < 1e-12 and abs(r[127] - math.sin(ang)) < 1e-12


def test_ring_holds_the_unfinished_block():
    rng = np.random.default_rng(2)
    raw = bits(rng.standard_normal((23, 128)))
    for L in range(0, 23):
        comp, ring = O.build_index_state(raw, L, 1e7)
        assert comp.shape[0] == L // 4
        assert sorted(ring) == sorted(t % 4 for t in range(4 * (L // 4), L))
        assert len(ring) == L % 4
        for t in range(4 * (L // 4), L):
            np.testing.assert_array_equal(ring[t % 4], raw[t])


def test_block_keys_do_not_depend_on_later_tokens():
    rng = np.random.default_rng(9)
    raw = bits(rng.standard_normal((200, 128)))
    full, _ = O.build_index_state(raw, 200, 1e7)
    part, _ = O.build_index_state(raw, 77, 1e7)
    np.testing.assert_array_equal(full[:19], part)


# ------------------------------------------------------------------ stage 2: scores, top-512, expansion

def test_scores_on_basis_keys_closed_form():
    rng = np.random.default_rng(4)
    q = bits(rng.standard_normal((4, 128)))
    w = np.array([0.5, 1.0, 1.25, 1.5], np.float32)
    comp = bits(np.eye(128))
    s = O.score_blocks(q, w, comp)
    qf = O.bf16_to_f64(q)
    for i in range(128):
        want = sum(float(w[h]) * max(0.0, qf[h, i]) for h in range(4))
        assert s[i] == pytest.approx(want, rel=0, abs=1e-15)


def test_scores_relu_and_weights():
    k = bits(np.full((1, 128), 0.125))
    qpos = bits(np.full((4, 128), 2.0))
    assert O.score_blocks(qpos, [1, 0, 0, 0], k)[0] == pytest.approx(2.0 * 0.125 * 128)
    assert O.score_blocks(bits(np.full((4, 128), -2.0)), [1, 1, 1, 1], k)[0] == 0.0
    mixed = np.stack([np.full(128, 2.0), np.full(128, -2.0), np.full(128, 1.0), np.full(128, -1.0)])
    assert O.score_blocks(bits(mixed), [0.5, 0.7, 1.5, 0.9], k)[0] == pytest.approx(
        0.5 * 32 + 1.5 * 16)


def test_scores_brute_force_tiny():
    rng = np.random.default_rng(8)
    q = bits(rng.standard_normal((4, 128)))
    k = bits(rng.standard_normal((6, 128)))
    w = rng.uniform(0.5, 1.5, 4).astype(np.float32)
    s = O.score_blocks(q, w, k)
    qf, kf = O.bf16_to_f64(q), O.bf16_to_f64(k)
    for c in range(6):
        tot = 0.0
        for h in range(4):
            dot = math.fsum(qf[h, i] * kf[c, i] for i in range(128))
            tot += float(w[h]) * (dot if dot > 0 else 0.0)
        assert s[c] == pytest.approx(tot, rel=1e-13, abs=1e-13)


def test_scores_many_queries_brute_force_tiny():
    # several queries, each with its own heads and weights, against shared keys: row t
    # must use query t's heads and weights (a swapped or transposed operand fails)
    rng = np.random.default_rng(9)
    T, n = 3, 5
    q = bits(rng.standard_normal((T, 4, 128)))
    k = bits(rng.standard_normal((n, 128)))
    w = rng.uniform(0.5, 1.5, (T, 4)).astype(np.float32)
    w[1] = [1.0, 0.0, 0.0, 0.0]        # one head alone: ReLU of one dot product
    s = O.score_blocks_many(q, w, k)
    assert s.shape == (T, n)
    qf, kf = O.bf16_to_f64(q), O.bf16_to_f64(k)
    for t in range(T):
        for c in range(n):
            tot = 0.0
            for h in range(4):
                dot = math.fsum(qf[t, h, i] * kf[c, i] for i in range(128))
                tot += float(w[t, h]) * (dot if dot > 0 else 0.0)
            assert s[t, c] == pytest.approx(tot, rel=1e-13, abs=1e-13)


def test_selection_driver_matches_whole_queries():
    # the indexer-only driver gives the rows' scores, selections and positions of the
    # full per-query path (rows of two requests, a ragged last batch of rows)
    wl = synth.make_workload("seldrv", "prefill", 26, [2300, 5000], chunk=7)
    rows = [0, 3, 6, 7, 9, 13]
    full = O.run_queries(wl, rows)
    sel = O.run_selections(wl, rows, chunk=4)
    for t in rows:
        np.testing.assert_array_equal(sel[t]["sel_blocks"], full[t]["sel_blocks"])
        np.testing.assert_array_equal(sel[t]["positions"], full[t]["positions"])
        np.testing.assert_allclose(sel[t]["scores"], full[t]["scores"], rtol=1e-13, atol=1e-13)


def test_select_all_when_few_blocks():
    for n in [0, 1, 511, 512]:
        np.testing.assert_array_equal(O.select_blocks(np.random.rand(n)), np.arange(n))


def test_select_planted_ranking():
    rng = np.random.default_rng(1)
    n = 3000
    s = rng.permutation(n).astype(np.float64)
    want = np.nonzero(s >= n - 512)[0]
    np.testing.assert_array_equal(O.select_blocks(s), want)


def test_select_ties_prefer_lower_index():
    n = 2000
    s = np.zeros(n)
    s[1::5] = 2.0          # 400 blocks clearly in
    s[0::5] = 1.0          # 400 tied blocks compete for the last 112 places
    sel = O.select_blocks(s)
    want = np.sort(np.concatenate([np.arange(1, n, 5), np.arange(0, n, 5)[:112]]))
    np.testing.assert_array_equal(sel, want)
    np.testing.assert_array_equal(O.select_blocks(np.ones(n)), np.arange(512))


def test_select_invariants_random():
    rng = np.random.default_rng(6)
    for n in [513, 1000, 40000]:
        s = np.round(rng.standard_normal(n), 2)        # many exact ties
        sel = O.select_blocks(s)
        assert len(sel) == 512 and np.all(np.diff(sel) > 0)
        out = np.setdiff1d(np.arange(n), sel)
        assert s[sel].min() >= s[out].max()
        thr = s[sel].min()
        # among blocks at the threshold, the kept ones are the lowest indices
        at = np.nonzero(s == thr)[0]
        kept = np.intersect1d(at, sel)
        np.testing.assert_array_equal(kept, at[:len(kept)])


def test_expansion_closed_form():
    for p in [0, 2, 3, 4098, 4095, 131071, 262142]:
        n_c = (p + 1) // 4
        sel = np.arange(min(n_c, 512)) * (max(n_c, 1) // max(min(n_c, 512), 1))
        pos = O.expand_positions(sel, p)
        assert len(pos) == 4 * min(n_c, 512) + (p + 1) % 4 <= 2051
        assert np.all(np.diff(pos) > 0) and pos.max(initial=-1) <= p
        pend = np.arange(4 * n_c, p + 1)
        assert np.all(np.isin(pend, pos))
    pos = O.expand_positions(np.array([0, 7]), 4098)
    assert list(pos) == [0, 1, 2, 3, 28, 29, 30, 31, 4096, 4097, 4098]


# ------------------------------------------------------------------ stage 3: sparse GQA

def test_gqa_single_position_returns_its_value():
    rng = np.random.default_rng(12)
    q = bits(rng.standard_normal((16, 256)))
    k = bits(rng.standard_normal((1, 2, 256)))
    v = bits(rng.standard_normal((1, 2, 256)))
    out, lse = O.sparse_gqa(q, k, v, 1 / 16)
    vf, qf, kf = O.bf16_to_f64(v), O.bf16_to_f64(q), O.bf16_to_f64(k)
    for h in range(16):
        np.testing.assert_array_equal(out[h], vf[0, h // 8])
        assert lse[h] == pytest.approx(float(qf[h] @ kf[0, h // 8]) / 16, abs=1e-12)


def test_gqa_zero_query_is_mean_and_two_point_weights():
    rng = np.random.default_rng(13)
    n = 37
    k = bits(rng.standard_normal((n, 2, 256)))
    v = bits(rng.standard_normal((n, 2, 256)))
    out, lse = O.sparse_gqa(np.zeros((16, 256), np.uint16), k, v, 1 / 16)
    vf = O.bf16_to_f64(v)
    for h in range(16):
        np.testing.assert_allclose(out[h], vf[:, h // 8].mean(axis=0), atol=1e-13)
        assert lse[h] == pytest.approx(math.log(n), abs=1e-12)
    # two keys whose logits differ by log(3): weights 3/4 and 1/4
    q = np.zeros((16, 256), np.float32)
    q[:, 0] = 16.0
    k2 = np.zeros((2, 2, 256), np.float32)
    k2[0, :, 0] = math.log(3.0)
    v2 = np.zeros((2, 2, 256), np.float32)
    v2[0, :, 1] = 1.0
    v2[1, :, 1] = 5.0
    out2, _ = O.sparse_gqa(bits(q), bits(k2), bits(v2), 1 / 16)
    lg3 = float(O.bf16_to_f64(bits([math.log(3.0)]))[0])
    w0 = math.exp(lg3) / (math.exp(lg3) + 1)
    assert out2[0, 1] == pytest.approx(w0 * 1 + (1 - w0) * 5, abs=1e-12)


def _torch_sdpa(qf, kf, vf, scale):
    """Dense attention of one query over all rows via torch (CPU, float64)."""
    Q = torch.from_numpy(qf)[None, :, None, :]                   # [1, 16, 1, D]
    K = torch.from_numpy(np.repeat(kf.transpose(1, 0, 2), 8, axis=0))[None]   # [1, 16, n, D]
    V = torch.from_numpy(np.repeat(vf.transpose(1, 0, 2), 8, axis=0))[None]
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=scale)
    return o[0, :, 0, :].numpy()


def test_gqa_matches_torch_sdpa():
    rng = np.random.default_rng(14)
    q = bits(rng.standard_normal((16, 256)))
    k = bits(rng.standard_normal((300, 2, 256)))
    v = bits(rng.standard_normal((300, 2, 256)))
    out, _ = O.sparse_gqa(q, k, v, 1 / 16)
    ref = _torch_sdpa(O.bf16_to_f64(q), O.bf16_to_f64(k), O.bf16_to_f64(v), 1 / 16)
    np.testing.assert_allclose(out, ref, atol=1e-12)


# ------------------------------------------------------------------ MRoPE (reading R10)

def test_mrope_text_positions_reduce_to_1d_rope():
    rng = np.random.default_rng(17)
    raw = bits(rng.standard_normal((203, 128)))
    pos3 = np.repeat(np.arange(203)[:, None], 3, axis=1)
    for axis in (synth.contiguous_pair_axis(), np.arange(64) % 3):
        comp3, ring3 = O.build_index_state(raw, 203, 1e7, pos3, axis)
        comp1, ring1 = O.build_index_state(raw, 203, 1e7)
        np.testing.assert_array_equal(comp3, comp1)
        assert ring3.keys() == ring1.keys()


def _one_block_with_mean(dims):
    # four equal raw keys with ones at `dims`: the mean is that vector exactly
    raw = np.zeros((4, 128), np.float32)
    raw[:, dims] = 1.0
    return bits(raw)[None]


@pytest.mark.parametrize("layout", ["contiguous", "interleaved"])
def test_mrope_block_turned_by_each_pairs_own_axis(layout):
    # mean e0 + e20 + e50, first token at (t, h, w) = (5, 2, 9).  Contiguous
    # sections 16/24/24 put pairs 0, 20, 50 on t, h, w; the interleaved map i % 3 on
    # t, w, w.  Pair i's dims (i, i + 64) become cos(a_i), sin(a_i) over sqrt(3).
    axis = synth.contiguous_pair_axis() if layout == "contiguous" else (np.arange(64) % 3).astype(np.uint8)
    pos = {"contiguous": {0: 5, 20: 2, 50: 9}, "interleaved": {0: 5, 20: 9, 50: 9}}[layout]
    key = O.bf16_to_f64(O.compress_blocks_mrope(_one_block_with_mean([0, 20, 50]),
                                                np.array([[5, 2, 9]]), axis, 1e7))[0]
    for i, p in pos.items():
        a = p * 1e7 ** (-2.0 * i / 128)
        for dim, want in ((i, math.cos(a) / math.sqrt(3)), (i + 64, math.sin(a) / math.sqrt(3))):
            # within half a bf16 step of the exact value
            assert abs(key[dim] - want) <= 2.0 ** (math.floor(math.log2(abs(want))) - 8), (dim, key[dim], want)
    others = np.setdiff1d(np.arange(128), [0, 20, 50, 64, 84, 114])
    assert np.all(key[others] == 0.0)


def test_mrope_positions_of_a_vision_span():
    # text 0..2, a 1 x 2 x 3 image from index 3, text again from position 3 + 3
    pos = synth.mrope_positions(11, [(3, 1, 2, 3)])
    want = [(0, 0, 0), (1, 1, 1), (2, 2, 2),
            (3, 3, 3), (3, 3, 4), (3, 3, 5), (3, 4, 3), (3, 4, 4), (3, 4, 5),
            (6, 6, 6), (7, 7, 7)]
    assert [tuple(r) for r in pos] == want


# ------------------------------------------------------------------ FP8 K/V (reading R9)

def test_e4m3_decode_hand_values():
    # 1.0 = 0.0111.000, 1.5 = 0.0111.100, 448 = 0.1111.110 (largest finite),
    # 2^-6 = 0.0001.000 (smallest normal), 2^-9 = 0.0000.001 (smallest subnormal),
    # 7 * 2^-9 = 0.0000.111, -1.0 = 1.0111.000, -0 = 1.0000.000, 0.1111.111 is NaN
    codes = [0x38, 0x3C, 0x7E, 0x08, 0x01, 0x07, 0xB8, 0x80, 0x00, 0x7F, 0xFF]
    want = [1.0, 1.5, 448.0, 2.0 ** -6, 2.0 ** -9, 7 * 2.0 ** -9, -1.0, -0.0, 0.0,
            float("nan"), float("nan")]
    got = O.e4m3_to_f64(codes)
    for c, g, w in zip(codes, got, want):
        if math.isnan(w):
            assert math.isnan(g), hex(c)
        else:
            assert g == w and math.copysign(1.0, g) == math.copysign(1.0, w), hex(c)


def test_e4m3_decode_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_to_f64(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_fp8_gqa_single_position_and_scales():
    # one position: every head returns v_scale * V and lse = sm_scale * k_scale * q.K
    rng = np.random.default_rng(15)
    q = bits(rng.standard_normal((16, 256)))
    k = rng.integers(0, 0x7E, size=(1, 2, 256), dtype=np.uint8)
    v = rng.integers(0, 0x7E, size=(1, 2, 256), dtype=np.uint8)
    k[..., ::2] |= 0x80                     # negative values too
    out, lse = O.sparse_gqa_fp8(q, k, v, 0.25, 3.0, 1 / 16)
    kv = torch.from_numpy(k).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    vv = torch.from_numpy(v).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    qf = O.bf16_to_f64(q)
    for h in range(16):
        np.testing.assert_array_equal(out[h], 3.0 * vv[0, h // 8])
        assert lse[h] == pytest.approx(float(qf[h] @ kv[0, h // 8]) * 0.25 / 16, abs=1e-12)


def test_fp8_gqa_matches_torch_sdpa_on_decoded_values():
    rng = np.random.default_rng(16)
    q = bits(rng.standard_normal((16, 256)))
    k = rng.integers(0, 256, size=(200, 2, 256), dtype=np.uint8)
    v = rng.integers(0, 256, size=(200, 2, 256), dtype=np.uint8)
    k[(k & 0x7F) == 0x7F] = 0x3F           # no NaN codes in an input
    v[(v & 0x7F) == 0x7F] = 0x3F
    out, _ = O.sparse_gqa_fp8(q, k, v, 0.01, 0.5, 1 / 16)
    kf = torch.from_numpy(k).view(torch.float8_e4m3fn).to(torch.float64).numpy() * 0.01
    vf = torch.from_numpy(v).view(torch.float8_e4m3fn).to(torch.float64).numpy() * 0.5
    ref = _torch_sdpa(O.bf16_to_f64(q), kf, vf, 1 / 16)
    np.testing.assert_allclose(out, ref, atol=1e-12)


# ------------------------------------------------------------------ whole query

def test_pipeline_equals_dense_causal_attention_when_few_blocks():
    # n_c <= 512 everywhere: the selection is every block, so QSA is dense causal
    # attention over 0..p (the dense per-request fallback used as a correctness
    # proof on the pages' L20 run is the same idea)
    wl = synth.make_workload("tiny", "decode", 21, [5, 600, 1403, 2051], page_order="identity")
    res = O.run_queries(wl)
    off = np.concatenate([[0], np.cumsum((wl.alloc_tokens + 63) // 64 * 64)])
    for b in range(wl.batch):
        L = int(wl.lengths[b])
        kf = O.bf16_to_f64(wl.k_pool[off[b]:off[b] + L])
        vf = O.bf16_to_f64(wl.v_pool[off[b]:off[b] + L])
        ref = _torch_sdpa(O.bf16_to_f64(wl.q[b]), kf, vf, 1 / 16)
        np.testing.assert_allclose(res[b]["out"], ref, atol=1e-12)
        assert len(res[b]["positions"]) == L


def test_prefill_rows_equal_decode_queries():
    wl = synth.make_workload("pf", "prefill", 22, [2600], chunk=9)
    res = O.run_queries(wl)
    for t in range(wl.total_q):
        p = int(wl.q_pos[t])
        comp, _ = O.build_index_state(wl.raw_idx_k[0], p + 1, wl.rope_theta)
        r = O.query(comp, wl.idx_q[t], wl.idx_w[t], wl.q[t], p, wl.page_table[0], wl.k_pool,
                    wl.v_pool, 64, 1 / 16)
        np.testing.assert_array_equal(r["positions"], res[t]["positions"])
        np.testing.assert_array_equal(r["out"], res[t]["out"])


def test_planted_hot_blocks_are_selected():
    wl = synth.make_workload("hot", "decode", 23, [4099, 9000], hot_per_req=8)
    res = O.run_queries(wl)
    for b in range(wl.batch):
        assert np.all(np.isin(wl.hot_blocks[b], res[b]["sel_blocks"]))
        # and they are the top scorers
        s = res[b]["scores"]
        assert set(np.argsort(-s)[:8]) == set(wl.hot_blocks[b])


def test_indexshare_reuse_equals_dense_when_selection_is_everything():
    wl = synth.make_workload("is", "indexshare", 24, [1200, 803], reuse_steps=3, page_order="identity")
    cap = O.run_queries(wl)
    res = O.run_indexshare(wl, cap)
    off = np.concatenate([[0], np.cumsum((wl.alloc_tokens + 63) // 64 * 64)])
    for b in range(wl.batch):
        p_cap = int(wl.q_pos[b])
        for j in range(1, 4):
            p = p_cap + j
            r = res[(j, b)]
            assert len(r["positions"]) == len(cap[b]["positions"]) + j
            np.testing.assert_array_equal(r["positions"], np.arange(p + 1))
            kf = O.bf16_to_f64(wl.k_pool[off[b]:off[b] + p + 1])
            vf = O.bf16_to_f64(wl.v_pool[off[b]:off[b] + p + 1])
            ref = _torch_sdpa(O.bf16_to_f64(wl.reuse_q[j - 1, b]), kf, vf, 1 / 16)
            np.testing.assert_allclose(r["out"], ref, atol=1e-12)


def test_indexshare_budget_at_capture_boundary():
    # capture where the query's own token completes a block: 2048 captured
    # positions, then 2048 + j at reuse step j (at most 2051)
    wl = synth.make_workload("isb", "indexshare", 25, [4100], reuse_steps=3)
    cap = O.run_queries(wl)
    assert len(cap[0]["positions"]) == 2048
    res = O.run_indexshare(wl, cap)
    for j in range(1, 4):
        pos = res[(j, 0)]["positions"]
        assert len(pos) == 2048 + j <= O.MAX_SELECTED
        assert len(np.unique(pos)) == len(pos) and pos.max() == 4099 + j
