"""qsa_profile_kernel_events on the GPU: the events of each launched kernel get the
kernel's duration, and asking for them changes no output."""

import pytest
import torch

from block_sparse_attention_c4_amd import binding as B
from block_sparse_attention_c4_amd import runner, synth

pytestmark = pytest.mark.gpu


def _events(n):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()                      # torch creates the HIP event at its first record
    torch.cuda.synchronize()
    return evs


def test_profile_events_time_each_kernel_and_change_nothing():
    wl = synth.make_workload("prof_ev", "decode", 340, [9003, 40000, 2100, 131072])
    dw = runner.DeviceWorkload(wl, "cuda:0")
    dw.build_prefix()
    torch.cuda.synchronize()
    dw.build_index()
    dw.attend()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (dw.sel_blocks, dw.sel_pos, dw.sel_count, dw.out, dw.lse)]

    n_index = 2                          # the scorer (builder folded in), the select
    n_attend = 2 if dw.ws_attn_bytes > 0 else 1   # the gather, the split combine
    ev = _events(2 * (n_index + n_attend))
    B.qsa_profile_kernel_events(ev[:2 * n_index])
    dw.build_index()
    B.qsa_profile_kernel_events(ev[2 * n_index:])
    dw.attend()
    torch.cuda.synchronize()
    for i, t in enumerate((dw.sel_blocks, dw.sel_pos, dw.sel_count, dw.out, dw.lse)):
        assert torch.equal(t, ref[i]), f"output {i} changed when its kernels were timed"
    ms = [ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(n_index + n_attend)]
    print(f"[events] kernel durations (us): {[round(1e3 * m, 2) for m in ms]}")
    assert all(0.0 < m < 50.0 for m in ms), ms
    # the kernels of one stream run in order: each starts no earlier than the one before
    for k in range(1, n_index + n_attend):
        assert ev[2 * (k - 1)].elapsed_time(ev[2 * k]) >= 0.0

    # a request lapses with the call it was made for: the next call sets no event
    ev2 = _events(2)
    t_before = ev2[0].elapsed_time(ev2[1])
    B.qsa_profile_kernel_events(ev2)
    B.qsa_profile_kernel_events([])      # cancels
    dw.build_index()
    torch.cuda.synchronize()
    assert ev2[0].elapsed_time(ev2[1]) == t_before
