"""The allocation-free decode call (qsa_sparse_gqa_decode_noalloc) against the
workspace call (qsa_sparse_gqa_decode), through the C ABI: two calls in a row, the
second on a smaller batch, each bit-identical to the workspace call on the same
inputs (same kernels; the split partials only move to the static scratch)."""

import numpy as np
import pytest
import torch

from block_sparse_attention_c4_amd import binding as B
from block_sparse_attention_c4_amd import runner, synth
from tests import parity as P

pytestmark = pytest.mark.gpu


def _case(name, seed, lengths, n_extra):
    wl = synth.make_workload(name, "indexshare" if n_extra else "decode", seed, lengths,
                             reuse_steps=3 if n_extra else 0, hot_per_req=2)
    dw = runner.DeviceWorkload(wl, "cuda:0")
    dw.build_prefix()
    dw.step(fused=True)
    extra = None
    if n_extra:
        dw.set_reuse(3)
        extra = dw.extra
    torch.cuda.synchronize()
    return wl, dw, extra


def _both(dw, extra, n_extra):
    """(out, lse) of the workspace call, then of the allocation-free call."""
    q = dw.reuse_q[2] if n_extra else dw.q
    dw.out.fill_(0)
    dw.lse.fill_(0)
    B.qsa_sparse_gqa_decode(dw.dims, dw.batch, q, dw.k_pool, dw.v_pool, dw.page_table, dw.pt_stride,
                            dw.sel_pos, dw.sel_count, runner.SEL_STRIDE, extra, n_extra, dw.out, dw.lse,
                            dw.ws_attn, dw.ws_attn_bytes)
    torch.cuda.synchronize()
    ref = (dw.out.clone(), dw.lse.clone())
    dw.out.fill_(0)
    dw.lse.fill_(0)
    B.qsa_sparse_gqa_decode_noalloc(dw.dims, dw.batch, q, dw.k_pool, dw.v_pool, dw.page_table,
                                    dw.pt_stride, dw.sel_pos, dw.sel_count, runner.SEL_STRIDE, extra,
                                    n_extra, dw.out, dw.lse)
    torch.cuda.synchronize()
    return ref, (dw.out.clone(), dw.lse.clone())


def test_noalloc_decode_matches_workspace_call_twice():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    # first call: 12 requests with drafted positions (11 splits per KV head); second:
    # 3 requests, no extra positions (16 splits), into the same scratch
    cases = [("noalloc_a", 401, [4100, 33003, 700, 9000, 2052, 131072, 5, 64001, 3000, 40000, 777,
                                   262140], 4),
             ("noalloc_b", 402, [9000, 2051, 70001], 0)]
    for name, seed, lengths, n_extra in cases:
        P.log(f"[noalloc] {name}: batch {len(lengths)}, n_extra {n_extra}")
        wl, dw, extra = _case(name, seed, lengths, n_extra)
        need = B.qsa_workspace_bytes(dw.dims, B.QSA_OP_GQA_DECODE, dw.batch, 0, n_extra)
        assert 0 < need <= B.QSA_ATTN_SCRATCH_BYTES   # the split partials go through the scratch
        (o_ws, l_ws), (o_st, l_st) = _both(dw, extra, n_extra)
        assert torch.equal(o_ws, o_st), f"{name}: outputs differ"
        assert torch.equal(l_ws, l_st), f"{name}: lse differs"
        assert int(torch.count_nonzero(o_st)) > 0
        P.log(f"[noalloc] {name}: bit-identical to the workspace call")
