"""hipGraph capture: one step of each path captured once and replayed several
times, with eager work and synchronisations between the replays; every replay's
outputs must equal the eager step's bit for bit (the library enqueues no memset
and no host work, so a captured step is the eager step)."""

import numpy as np
import pytest
import torch

from block_sparse_attention_c4_amd import runner, synth

pytestmark = pytest.mark.gpu


def _outputs(dw):
    return [dw.comp, dw.ring, dw.sel_blocks, dw.sel_pos, dw.sel_count, dw.out, dw.lse]


def _replays_match(dw, step, outs, fill=None, replays=3):
    """fill: the outputs the step rewrites whole (overwritten between replays);
    default every output but the compressed cache and the ring."""
    fill = outs[2:] if fill is None else fill
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    x = torch.randn(512, 512, device=dw.dev)
    for r in range(replays):
        for o in fill:
            o.fill_(-3)
        y = x @ x                           # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, ref)):
            assert torch.equal(o, e), f"replay {r}: output {i} differs from the eager step"
        del y


def _device(wl, kv="bf16"):
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    dw = runner.DeviceWorkload(wl, "cuda:0", kv=kv)
    dw.build_prefix()
    torch.cuda.synchronize()
    return dw


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_graph_decode_step(kv):
    wl = synth.make_workload("g_decode", "decode", 330, [5, 2051, 9003, 40000, 700], hot_per_req=2)
    if kv == "fp8":
        synth.with_fp8_kv(wl)
    dw = _device(wl, kv)
    _replays_match(dw, dw.step, _outputs(dw))


def test_graph_decode_step_builder_folded():
    # the decode step as the benchmark runs it: builder and indexer in one call
    wl = synth.make_workload("g_decode_f", "decode", 333, [4, 5, 2052, 9003, 40000, 700], hot_per_req=2)
    dw = _device(wl)
    assert dw.can_fuse()
    _replays_match(dw, lambda: dw.step(fused=True), _outputs(dw))


def test_graph_decode_step_indexer_on_second_stream():
    # builder + indexer on a second stream beside unrelated work on the launch stream,
    # joined before attention, as one captured graph
    wl = synth.make_workload("g_decode_s", "decode", 334, [8, 2051, 9003, 40000, 703], hot_per_req=2)
    dw = _device(wl)
    x = torch.randn(64, 1024, device=dw.dev).to(torch.bfloat16)
    w = torch.randn(1024, 1024, device=dw.dev).to(torch.bfloat16)
    y = torch.empty(64, 1024, dtype=torch.bfloat16, device=dw.dev)
    side = torch.cuda.Stream()

    def step():
        cur = torch.cuda.current_stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            dw.build_index()
        torch.mm(x, w, out=y)
        cur.wait_stream(side)
        dw.attend()

    _replays_match(dw, step, _outputs(dw))


def test_graph_prefill_step():
    # chunks that start on block boundaries: a repeated step reads the same ring
    wl = synth.make_workload("g_prefill", "prefill", 331, [2104, 9000], chunk=40)
    assert np.all(wl.prefix_len % 4 == 0)
    dw = _device(wl)
    _replays_match(dw, dw.step, _outputs(dw))


def test_graph_verify_step_with_ring_restore():
    # 4 query tokens per request from mid-block: the step restores the pending-token
    # ring first (a device copy inside the graph), as a repeated step must
    wl = synth.make_workload("g_verify", "prefill", 332, [4101, 2050, 33003, 9002], chunk=4)
    dw = _device(wl)
    saved = dw.ring.clone()

    def step():
        dw.ring.copy_(saved)
        dw.step()
    _replays_match(dw, step, _outputs(dw))


def test_graph_indexshare_reuse_step():
    wl = synth.make_workload("g_is", "indexshare", 333, [4100, 33003, 700], reuse_steps=3)
    dw = _device(wl)
    dw.step()
    dw.set_reuse(2)
    _replays_match(dw, lambda: dw.reuse_step(2), [dw.out, dw.lse], fill=[dw.out, dw.lse])


def test_graph_decode_step_noalloc():
    # the allocation-free attention call, made for callers under capture: the folded
    # index call and qsa_sparse_gqa_decode_noalloc captured together (its scratch
    # address is taken by the eager step that precedes the capture)
    from block_sparse_attention_c4_amd import binding as B
    wl = synth.make_workload("g_decode_na", "decode", 335, [4, 2052, 9003, 40000, 700, 131072],
                             hot_per_req=2)
    dw = _device(wl)
    assert dw.can_fuse()

    def step():
        dw.build_index()
        B.qsa_sparse_gqa_decode_noalloc(dw.dims, dw.batch, dw.q, dw.k_pool, dw.v_pool, dw.page_table,
                                        dw.pt_stride, dw.sel_pos, dw.sel_count, runner.SEL_STRIDE,
                                        None, 0, dw.out, dw.lse)
    _replays_match(dw, step, _outputs(dw))
