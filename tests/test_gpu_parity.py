"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Stage-isolated checks feed each stage the oracle's output of the previous stage
(so a legitimate 1-ulp key difference cannot cascade); end-to-end checks run the
three GPU stages back to back.  Small ragged workloads are checked on every
query.  At full size every query row's selection and positions are checked; the
attention output of every decode request, and of a sample of prefill rows plus
every row whose selection was swapped at a tie, in the same launch configuration
the benchmark times.
"""

import numpy as np
import pytest
import torch

from block_sparse_attention_c4_amd import runner, synth
from oracle import qsa_oracle as O
from tests import parity as P

pytestmark = pytest.mark.gpu

_CACHE = {}


def _gpu():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    return "cuda:0"


def full(name):
    if name not in _CACHE:
        P.log(f"[gen] {name}")
        _CACHE[name] = synth.FULL_SIZE[name]()
    return _CACHE[name]


SMALL = {
    # lengths cover: empty selection, dense (n_c <= 512), n_c = 512 / 513, the direct
    # top-k path (n_c < 8192) and the group-filtered path (n_c >= 8192)
    "decode_ragged": lambda: synth.make_workload(
        "decode_ragged", "decode", 301, [1, 2, 5, 600, 2048, 2051, 2052, 2055, 5003, 33001, 40000],
        hot_per_req=8),
    "decode_page16": lambda: synth.make_workload(
        "decode_page16", "decode", 302, [37, 2060, 9000, 35000], hot_per_req=4, page_size=16),
    # many queries per request: the MFMA scorer and the code-based select.  A 64-query
    # tile straddles the two requests; rows of 516..525 blocks take the whole-row
    # select, rows of ~8330 blocks the group-maximum candidates; 74 rows leave a
    # ragged last tile
    "prefill_ragged": lambda: synth.make_workload(
        "prefill_ragged", "prefill", 303, [2101, 33333], chunk=37),
    # page 16 (a 16-block group spans 4 pages), rows with fewer than 512 blocks,
    # three requests in one tile, ~17500-block rows
    "prefill_page16_mixed": lambda: synth.make_workload(
        "prefill_page16_mixed", "prefill", 309, [300, 9000, 70001], chunk=70, page_size=16,
        hot_per_req=6),
    "indexshare_small": lambda: synth.make_workload(
        "indexshare_small", "indexshare", 304, [4100, 33003, 700], reuse_steps=3),
    # more than 64 decode queries: the scorer launches in chunks of 64 queries
    "decode_batch70": lambda: synth.make_workload(
        "decode_batch70", "decode", 305,
        [3, 700, 2051, 40000] + [1 + (i * 7919) % 20000 for i in range(66)], hot_per_req=2),
    # a prefill chunk of fewer than 64 queries: the multi-query scorer (5 windows of
    # 4 queries per request) and the FP32 select
    "prefill_small_chunk": lambda: synth.make_workload(
        "prefill_small_chunk", "prefill", 306, [5000, 40000], chunk=20),
    # target verification, 4 query tokens per request: the multi-query scorer with one
    # pass per window.  Lengths cover queries with no visible block, n_c around 512,
    # the direct and the group-maximum select, page 16
    "verify_ragged": lambda: synth.make_workload(
        "verify_ragged", "prefill", 312,
        [4, 7, 2052, 2055, 4100, 9003, 33001, 40000, 701, 2100, 16, 70001], chunk=4,
        hot_per_req=2),
    "verify_page16": lambda: synth.make_workload(
        "verify_page16", "prefill", 313, [2050, 9000, 35003, 64], chunk=4, page_size=16),
    # 3 queries per request: windows of 4 straddle requests (two passes per window)
    "verify_chunk3": lambda: synth.make_workload(
        "verify_chunk3", "prefill", 314, [3 + (i * 2741) % 12000 for i in range(21)], chunk=3),
    # 70 requests x 4 queries: more than the 256 queries of one multi-query launch
    "verify_batch70": lambda: synth.make_workload(
        "verify_batch70", "prefill", 315, [4 + (i * 7919) % 6000 for i in range(70)], chunk=4),
}


def small(name):
    key = "small:" + name
    if key not in _CACHE:
        _CACHE[key] = SMALL[name]()
    return _CACHE[key]


def _device(wl, kv="bf16"):
    P.log(f"[upload] {wl.name} B={wl.batch} T={wl.total_q} pages={wl.num_pages} kv={kv}")
    return runner.DeviceWorkload(wl, _gpu(), kv=kv)


def fp8(wl):
    """The workload with FP8 E4M3 copies of its K/V pools (made once)."""
    if wl.k_pool_fp8 is None:
        synth.with_fp8_kv(wl)
    return wl


def _rows(wl, sample):
    if sample is None or wl.total_q <= sample:
        return list(range(wl.total_q))
    rng = np.random.default_rng(7)
    head = list(range(8)) + list(range(wl.total_q - 8, wl.total_q))
    mid = rng.choice(np.arange(8, wl.total_q - 8), size=sample - 16, replace=False)
    return sorted(set(head) | set(int(x) for x in mid))


def _upload_oracle_comp(dw, wl, states):
    comp = np.zeros(dw.comp.shape, dtype=np.uint16)
    for b, (keys, _) in enumerate(states):
        if keys.shape[0]:
            comp[O.comp_slot(wl.page_table[b], np.arange(keys.shape[0]), wl.page_size)] = keys
    dw.comp.copy_(torch.from_numpy(comp.view(np.int16)))


# ------------------------------------------------------------------ stage 1

def _check_builder(wl):
    dw = _device(wl)
    dw.build_prefix()
    dw.build_step()
    torch.cuda.synchronize()
    states = P.oracle_index_states(wl)
    n, nd = P.check_comp_cache(wl, dw.comp_numpy(), states)
    P.check_ring(dw.ring_numpy(), states)
    P.log(f"[builder] {wl.name}: {n} keys, {nd} not bit-identical (<= 1 ulp)")
    return dw


@pytest.mark.parametrize("name", list(SMALL))
def test_builder_small(name):
    _check_builder(small(name))


@pytest.mark.parametrize("name", list(synth.FULL_SIZE))
def test_builder_full(name):
    _check_builder(full(name))


def test_builder_incremental_decode_matches_bulk():
    # ingest token by token (decode steps) and compare with one bulk ingest
    wl = synth.make_workload("inc", "decode", 305, [70, 23], page_order="shuffled")
    dw = _device(wl)
    dims = dw.dims
    from block_sparse_attention_c4_amd import binding as B
    for t in range(int(wl.lengths.max())):
        live = [b for b in range(wl.batch) if t < wl.lengths[b]]
        keys = np.stack([wl.raw_idx_k[b][t] for b in range(wl.batch) if t < wl.lengths[b]])
        cu = np.zeros(wl.batch + 1, np.int32)
        for b in range(wl.batch):
            cu[b + 1] = cu[b] + (1 if b in live else 0)
        B.qsa_build_index_keys(dims, wl.batch, runner._u16(keys, dw.dev), runner._i32(cu, dw.dev),
                               runner._i32(np.full(wl.batch, t), dw.dev), len(live), 1,
                               dw.page_table, dw.pt_stride, dw.ring, dw.comp)
    torch.cuda.synchronize()
    states = P.oracle_index_states(wl)
    P.check_comp_cache(wl, dw.comp_numpy(), states)
    P.check_ring(dw.ring_numpy(), states)


# MRoPE positions: vision spans in the cached prefix, inside the step's chunk and under
# the decode token; chunks that start inside a block read the first token's position
# from the position ring
MROPE = {
    "mrope_prefill": lambda: synth.with_mrope(
        synth.make_workload("mrope_prefill", "prefill", 317, [3000, 9000], chunk=37),
        [[(100, 1, 16, 16), (2970, 1, 2, 8)], [(5000, 2, 8, 8)]]),
    # request 4: the decode token 779 completes block 776..779, whose first token (a
    # vision token of the span 700..776) arrived earlier and waits in the position ring
    "mrope_decode": lambda: synth.with_mrope(
        synth.make_workload("mrope_decode", "decode", 318, [4099, 777, 2100, 6, 780]),
        [[(50, 1, 32, 32)], [(700, 1, 7, 11)], [], [(1, 1, 1, 3)], [(700, 1, 7, 11)]]),
    "mrope_interleaved": lambda: synth.with_mrope(
        synth.make_workload("mrope_interleaved", "prefill", 319, [2501, 700], chunk=9),
        [[(1000, 3, 10, 12)], [(690, 1, 3, 3)]], pair_axis=np.arange(64) % 3),
}


def mrope(name):
    key = "mrope:" + name
    if key not in _CACHE:
        _CACHE[key] = MROPE[name]()
    return _CACHE[key]


@pytest.mark.parametrize("name", list(MROPE))
def test_builder_mrope(name):
    wl = mrope(name)
    dw = _check_builder(wl)
    # the position ring holds the unfinished block's tokens, slot t % 4
    ring_pos = dw.ring_mpos.cpu().numpy()
    for b in range(wl.batch):
        L = int(wl.lengths[b])
        for t in range(4 * (L // 4), L):
            np.testing.assert_array_equal(ring_pos[b, t % 4], wl.mpos[b][t], err_msg=f"{name} {b} {t}")


@pytest.mark.parametrize("name", list(MROPE))
def test_end_to_end_mrope(name):
    _check_e2e(mrope(name))


def test_builder_mrope_text_positions_equal_1d_builder():
    # (p, p, p) positions through the MRoPE call give the 1-D call's keys, bit for bit
    wl = synth.make_workload("mrope_text", "prefill", 320, [5000, 2222], chunk=45)
    dw1 = _device(wl)
    dw1.build_prefix()
    dw1.build_step()
    synth.with_mrope(wl, [[], []])
    dw3 = _device(wl)
    dw3.build_prefix()
    dw3.build_step()
    torch.cuda.synchronize()
    assert torch.equal(dw1.comp, dw3.comp)
    assert torch.equal(dw1.ring, dw3.ring)


# ------------------------------------------------------------------ stage 2 (fed oracle keys)

def selections(wl):
    """The oracle's indexer results for every query row of wl (cached per workload)."""
    key = ("sel", wl.name, id(wl))
    if key not in _CACHE:
        _CACHE[key] = O.run_selections(wl)
    return _CACHE[key]


def _check_rows_selection(wl, gb, gp, gc, res, exact=False, tag=""):
    """Selection and positions of every query row; returns the rows whose kept set
    differs from the oracle's at a boundary tie.  exact: a bool, or a function of
    the row that says whether that row's selection must equal the oracle's."""
    swapped = []
    for t in range(wl.total_q):
        where = f"{wl.name} row {t} (p={int(wl.q_pos[t])}){tag}"
        ex = exact(t) if callable(exact) else exact
        if P.check_selection(gb[t], res[t], where, exact=ex):
            P.check_positions(gp[t], int(gc[t]), res[t], where)
        else:
            swapped.append(t)
            P.check_positions_valid(gp[t], int(gc[t]), gb[t], int(wl.q_pos[t]), where)
    assert len(swapped) <= max(1, wl.total_q // 50), f"{len(swapped)} rows with tie-swapped selections"
    return swapped


def _check_index_stage(wl, exact=False):
    dw = _device(wl)
    states = P.oracle_index_states(wl)
    _upload_oracle_comp(dw, wl, states)
    dw.index()
    torch.cuda.synchronize()
    gb = dw.sel_blocks.cpu().numpy()
    gp = dw.sel_pos.cpu().numpy()
    gc = dw.sel_count.cpu().numpy()
    swapped = _check_rows_selection(wl, gb, gp, gc, selections(wl), exact)
    P.log(f"[index] {wl.name}: {wl.total_q} rows (all), {len(swapped)} resolved by boundary ties"
          f"{' (exact)' if exact is True else ''}")


@pytest.mark.parametrize("name", list(SMALL))
def test_index_stage_small(name):
    _check_index_stage(small(name))


@pytest.mark.parametrize("name", list(synth.FULL_SIZE))
def test_index_stage_full(name):
    _check_index_stage(full(name))


def test_index_all_ties():
    # zero indexer queries: every score is 0, so the lowest 512 blocks win
    wl = synth.make_workload("ties", "decode", 306, [9000, 40000, 2100])
    wl.idx_q[:] = 0
    _check_index_stage(wl, exact=True)


def test_index_all_ties_long_rows():
    # every score 0 on rows long enough for the group-maxima path: exactly 1024 groups
    # (every group a candidate, whose float4s overflow the list), 1094 groups (more
    # candidate groups than the list of groups holds) and 2048 groups; each row falls
    # back to the exact select over the row in memory and keeps the 512 lowest blocks
    wl = synth.make_workload("ties_long", "decode", 317, [65539, 70000, 131072])
    wl.idx_q[:] = 0
    _check_index_stage(wl, exact=True)


def test_index_zero_keys_tie_break():
    # all-zero raw keys: every compressed key is zero (the norm floor), every score
    # is 0, and the 512 lowest block indices are kept
    wl = synth.make_workload("dup", "decode", 307, [12000])
    for b in range(wl.batch):
        wl.raw_idx_k[b][:] = 0
    _check_index_stage(wl, exact=True)


def test_index_prefill_all_ties():
    # many queries, every score 0: each row is handed from the code-based select to
    # the FP32 select, which keeps the 512 lowest blocks
    wl = synth.make_workload("ties_prefill", "prefill", 310, [9000, 40000], chunk=48)
    wl.idx_q[:] = 0
    _check_index_stage(wl, exact=True)


def test_index_verify_all_ties():
    # 4 queries per request with zero indexer queries: the multi-query scorer writes
    # +0 for every block, and the FP32 select keeps the 512 lowest blocks
    wl = synth.make_workload("ties_verify", "prefill", 316, [9000, 40000, 2100, 7], chunk=4)
    wl.idx_q[:] = 0
    _check_index_stage(wl, exact=True)


def test_index_prefill_equal_keys():
    # every raw key equal: every compressed key of a request differs only by its
    # rotation, so scores spread over few distinct codes; plus rows with all-zero keys
    wl = synth.make_workload("eq_prefill", "prefill", 311, [20000, 6000], chunk=40)
    wl.raw_idx_k[0][:] = wl.raw_idx_k[0][0]
    wl.raw_idx_k[1][:] = 0
    # request 1's rows tie exactly (every score is 0): the 512 lowest blocks, exactly
    _check_index_stage(wl, exact=lambda t: int(wl.q_req[t]) == 1)


# ------------------------------------------------------------------ stage 3 (fed oracle positions)

def _upload_oracle_positions(dw, res, rows):
    sp = np.full(dw.sel_pos.shape, -1, dtype=np.int32)
    sc = np.zeros(dw.sel_count.shape, dtype=np.int32)
    for t in rows:
        pos = res[t]["positions"]
        sp[t, :len(pos)] = pos
        sc[t] = len(pos)
    dw.sel_pos.copy_(torch.from_numpy(sp))
    dw.sel_count.copy_(torch.from_numpy(sc))


def _check_attention_stage(wl, sample=None, kv="bf16"):
    dw = _device(wl, kv)
    rows = _rows(wl, sample)
    res = O.run_queries(wl, rows, kv=kv)
    _upload_oracle_positions(dw, res, range(wl.total_q) if sample is None else rows)
    dw.attend()
    torch.cuda.synchronize()
    out = dw.out_f64()
    lse = dw.lse.cpu().numpy()
    worst = 0.0
    for t in rows:
        mx, _, _ = P.check_attention(out[t], lse[t], res[t], f"{wl.name} row {t}")
        worst = max(worst, mx)
    P.log(f"[attn] {wl.name} {kv}: {len(rows)} rows, worst max-abs {worst:.2e}")


@pytest.mark.parametrize("name", list(SMALL))
def test_attention_stage_small(name):
    _check_attention_stage(small(name))


@pytest.mark.parametrize("name", [n for n in synth.FULL_SIZE if not n.endswith("_mrope")])
def test_attention_stage_full(name):
    # (the MRoPE prefill chunk attends exactly as the plain one: its positions only
    # change the indexer keys)
    wl = full(name)
    _check_attention_stage(wl, sample=48 if wl.kind == "prefill" else None)


# FP8 E4M3 K/V pools with per-pool scales: the same bar, against the oracle on the
# decoded and scaled codes
FP8_SMALL = ["decode_ragged", "decode_page16", "prefill_ragged", "decode_batch70", "verify_chunk3"]


@pytest.mark.parametrize("name", FP8_SMALL)
def test_attention_stage_fp8_small(name):
    _check_attention_stage(fp8(small(name)), kv="fp8")


@pytest.mark.parametrize("name", ["decode_b32_loguniform_4k_128k", "prefill_chunk4096_prefix126976"])
def test_attention_stage_fp8_full(name):
    wl = fp8(full(name))
    _check_attention_stage(wl, sample=48 if wl.kind == "prefill" else None, kv="fp8")


# ------------------------------------------------------------------ end to end

def _check_outputs(dw, wl, sample=None, kv="bf16", tag=""):
    """Selection and positions of every row; attention and lse of the sampled rows
    and of every row whose selection was swapped at a tie (those against the oracle's
    attention over the GPU's own positions)."""
    gb = dw.sel_blocks.cpu().numpy()
    gp = dw.sel_pos.cpu().numpy()
    gc = dw.sel_count.cpu().numpy()
    out = dw.out_f64()
    lse = dw.lse.cpu().numpy()
    swapped = _check_rows_selection(wl, gb, gp, gc, selections(wl), tag=tag)
    rows = _rows(wl, sample)
    same = [t for t in rows if t not in swapped]
    res = O.run_queries(wl, same, kv=kv)
    for t in same:
        P.check_attention(out[t], lse[t], res[t], f"{wl.name} row {t}{tag}")
    for t in swapped:
        ref = P.oracle_on_gpu_positions(wl, t, gp[t], int(gc[t]), kv=kv)
        P.check_attention(out[t], lse[t], ref, f"{wl.name} row {t}{tag} (tie-swapped selection)")
    P.log(f"[e2e{tag}] {wl.name}: selection of all {wl.total_q} rows; attention of "
          f"{len(same) + len(swapped)} rows ({len(swapped)} tie-swapped, checked on the GPU's positions)")


def _check_e2e(wl, sample=None, kv="bf16"):
    dw = _device(wl, kv)
    dw.build_prefix()
    dw.step()
    torch.cuda.synchronize()
    states = P.oracle_index_states(wl)
    P.check_comp_cache(wl, dw.comp_numpy(), states)
    _check_outputs(dw, wl, sample, kv)
    return dw


@pytest.mark.parametrize("name", list(SMALL))
def test_end_to_end_small(name):
    _check_e2e(small(name))


@pytest.mark.parametrize("name", list(synth.FULL_SIZE))
def test_end_to_end_full(name):
    wl = full(name)
    _check_e2e(wl, sample=48 if wl.kind == "prefill" else None)


def test_end_to_end_fp8_decode_full():
    _check_e2e(fp8(full("decode_b32_loguniform_4k_128k")), kv="fp8")


def test_planted_hot_blocks_selected_on_gpu():
    wl = full("decode_b8_l32k")
    dw = _device(wl)
    dw.build_prefix()
    dw.step()
    torch.cuda.synchronize()
    gb = dw.sel_blocks.cpu().numpy()
    for b in range(wl.batch):
        assert np.all(np.isin(wl.hot_blocks[b], gb[b]))


# ------------------------------------------------------------------ IndexShare

def _check_indexshare(wl, kv="bf16"):
    dw = _device(wl, kv)
    dw.build_prefix()
    dw.step()                     # capture: the indexer runs on the last accepted token
    torch.cuda.synchronize()
    cap = O.run_queries(wl, kv=kv)
    res = O.run_indexshare(wl, cap, kv=kv)
    gb = dw.sel_blocks.cpu().numpy()
    # reuse steps over the oracle's captured selection (stage isolated)
    _upload_oracle_positions(dw, cap, range(wl.batch))
    for j in range(1, wl.reuse_steps + 1):
        dw.set_reuse(j)
        dw.reuse_step(j)
        torch.cuda.synchronize()
        out = dw.out_f64()
        lse = dw.lse.cpu().numpy()
        for b in range(wl.batch):
            P.check_attention(out[b], lse[b], res[(j, b)], f"{wl.name} reuse step {j} request {b}")
    for b in range(wl.batch):
        P.check_selection(gb[b], cap[b], f"{wl.name} capture {b}")
    P.log(f"[indexshare] {wl.name}: {wl.reuse_steps} reuse steps x {wl.batch} requests")


def test_indexshare_small():
    _check_indexshare(small("indexshare_small"))


def test_indexshare_full():
    _check_indexshare(full("indexshare_b4_l262140"))


def test_indexshare_fp8_small():
    _check_indexshare(fp8(small("indexshare_small")), kv="fp8")


# ------------------------------------------------------------------ edge cases

def test_max_context():
    # p = 262143: 65536 visible blocks, the largest the library supports
    wl = synth.make_workload("maxctx", "decode", 308, [262144], hot_per_req=16)
    _check_e2e(wl)


def test_repeat_runs_are_bitwise_identical():
    wl = full("decode_b32_loguniform_4k_128k")
    dw = _device(wl)
    dw.build_prefix()
    dw.step()
    torch.cuda.synchronize()
    first = [x.clone() for x in (dw.comp, dw.sel_blocks, dw.sel_pos, dw.sel_count, dw.out, dw.lse)]
    dw.step()
    torch.cuda.synchronize()
    for a, b in zip(first, (dw.comp, dw.sel_blocks, dw.sel_pos, dw.sel_count, dw.out, dw.lse)):
        assert torch.equal(a, b)


# ------------------------------------------------------------------ builder folded into the indexer

# decode lengths for the folded call: tokens that complete a block whose group holds
# only that block (n_c = 16k + 1), that fill a group (n_c = 16k), the first block
# (p = 3), no visible block (p < 3), tokens left pending, n_c around 512
FUSED_SMALL = {
    "decode_fresh_edges": lambda: synth.make_workload(
        "decode_fresh_edges", "decode", 316,
        [1, 3, 4, 5, 8, 64, 68, 1028, 2048, 2052, 4096 + 4, 4096 + 7, 32768, 32772, 40001],
        hot_per_req=2),
    # no request with a complete block: the launch's scorer part has no group at all
    "decode_no_blocks": lambda: synth.make_workload("decode_no_blocks", "decode", 317, [1, 2, 3]),
    # one block at most: the only groups are the queries' own
    "decode_one_block": lambda: synth.make_workload("decode_one_block", "decode", 318, [4, 1, 5, 2]),
}


def fused_small(name):
    key = "fused:" + name
    if key not in _CACHE:
        _CACHE[key] = FUSED_SMALL[name]()
    return _CACHE[key]


def _decode_names_small():
    return ["decode_ragged", "decode_page16", "decode_batch70", "indexshare_small"]


def _decode_names_full():
    return [n for n in synth.FULL_SIZE if n.startswith("decode") or n.startswith("indexshare")]


def _valid_scores(dw, wl):
    """The FP32 score rows of the index workspace, cut to each query's visible blocks."""
    nb = (dw.max_pos + 3) // 4
    stride = (nb + 127) // 128 * 128
    sc = dw.ws_index[: wl.total_q * stride * 4].view(torch.float32).view(wl.total_q, stride).cpu().numpy()
    return [sc[t, : (int(wl.q_pos[t]) + 1) // 4].copy() for t in range(wl.total_q)]


def _check_fused_equals_separate(wl):
    sep = _device(wl)
    assert sep.can_fuse()
    sep.build_prefix()
    sep.build_step()
    sep.index()
    torch.cuda.synchronize()
    fus = _device(wl)
    fus.build_prefix()
    fus.build_index()
    torch.cuda.synchronize()
    names = ["comp", "ring", "sel_blocks", "sel_pos", "sel_count"]
    if wl.mpos is not None:
        names.append("ring_mpos")
    for name in names:
        assert torch.equal(getattr(sep, name), getattr(fus, name)), f"{wl.name}: {name} differs"
    for t, (a, b) in enumerate(zip(_valid_scores(sep, wl), _valid_scores(fus, wl))):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{wl.name}: scores of row {t}"
    P.log(f"[fused] {wl.name}: builder + indexer in one call bit-identical to the two calls")


@pytest.mark.parametrize("name", list(FUSED_SMALL))
def test_fused_build_index_edges(name):
    _check_fused_equals_separate(fused_small(name))


@pytest.mark.parametrize("name", _decode_names_small())
def test_fused_build_index_small(name):
    _check_fused_equals_separate(small(name))


@pytest.mark.parametrize("name", _decode_names_full())
def test_fused_build_index_full(name):
    _check_fused_equals_separate(full(name))


def test_fused_max_context():
    _check_fused_equals_separate(synth.make_workload("maxctx_fused", "decode", 308, [262144, 262143],
                                                     hot_per_req=16))


def _check_e2e_fused(wl):
    """The folded decode step (one call for builder and indexer, then attention)
    against the oracle."""
    dw = _device(wl)
    dw.build_prefix()
    dw.step(fused=True)
    torch.cuda.synchronize()
    states = P.oracle_index_states(wl)
    P.check_comp_cache(wl, dw.comp_numpy(), states)
    P.check_ring(dw.ring_numpy(), states)
    _check_outputs(dw, wl, tag=" fused")


@pytest.mark.parametrize("name", list(FUSED_SMALL))
def test_end_to_end_fused_edges(name):
    _check_e2e_fused(fused_small(name))


def test_end_to_end_fused_full():
    _check_e2e_fused(full("decode_b32_loguniform_4k_128k"))


# MRoPE decode through the folded call: blocks completed by the decode token whose first
# token is a vision token, with contiguous and interleaved axis maps
FUSED_MROPE = {
    "mrope_decode": lambda: mrope("mrope_decode"),
    "mrope_decode_interleaved": lambda: synth.with_mrope(
        synth.make_workload("mrope_decode_il", "decode", 320, [780, 1028, 4, 2052, 9]),
        [[(700, 1, 7, 11)], [(1020, 1, 2, 4)], [(0, 1, 2, 2)], [], [(2, 1, 2, 3)]],
        pair_axis=np.arange(64) % 3),
}


@pytest.mark.parametrize("name", list(FUSED_MROPE))
def test_fused_build_index_mrope(name):
    key = "fused_mrope:" + name
    if key not in _CACHE:
        _CACHE[key] = FUSED_MROPE[name]()
    wl = _CACHE[key]
    _check_fused_equals_separate(wl)
    _check_e2e_fused(wl)
