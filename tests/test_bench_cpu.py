"""Host logic of bench.py (no GPU): the one-GPU refusal, the algorithmic byte
counts behind the roofline, and the rule that HBM traffic taken by the profiler is
reported only while the kernel sources are the ones it was taken on."""

import json
import os
import subprocess
import sys
import types

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_decode_bytes_hand_count():
    # two requests: p = 3 completes block 0 (4 positions attended), p = 5 leaves two
    # tokens pending (4 + 2 positions)
    wl = types.SimpleNamespace(q_pos=np.array([3, 5]))
    counts = np.array([4, 6])
    got = bench.decode_bytes(wl, counts)
    # builder: the new key in; a completing block also reads 3 ring keys and writes its
    # compressed key, a pending token writes its ring slot
    assert got["build"] == (256 + 3 * 256 + 256) + (256 + 256)
    # indexer: one 256-byte compressed key per visible block, 4 x 128 bf16 query,
    # 4 float weights, the 512-entry block list, the positions and the count
    per_query = 1024 + 16 + 2048 + 4
    assert got["index"] == (256 + per_query + 4 * 4) + (256 + per_query + 4 * 6)
    # attention: K and V rows of both KV heads (2 x 2 x 256 bf16 = 2 KB) per position,
    # the positions and count, q and out (16 x 256 bf16 each) and the 16 lse floats
    fixed = 4 + 2 * 16 * 256 * 2 + 16 * 4
    assert got["attend"] == (2048 * 4 + 4 * 4 + fixed) + (2048 * 6 + 4 * 6 + fixed)
    assert got["step"] == got["build"] + got["index"] + got["attend"]
    # FP8 pools: 1 byte per element, drafted positions add to the attended count
    got8 = bench.decode_bytes(wl, counts, n_extra=2, kv_bytes=1)
    assert got8["attend"] == (1024 * 6 + 4 * 6 + fixed) + (1024 * 8 + 4 * 8 + fixed)


def test_traffic_reported_only_for_unchanged_sources(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel v1\n")
    rec = tmp_path / "traffic.json"
    monkeypatch.setitem(bench.KERNEL_SOURCES, "attn_kernel", [str(src)])
    monkeypatch.setattr(bench, "traffic_file", lambda workload: str(rec))
    monkeypatch.setattr(bench, "ROOT", "/")
    rec.write_text(json.dumps({"attn_kernel": {"bytes_per_launch": 12345,
                                               "source_hash": bench.source_hash([str(src)])}}))
    assert bench.load_traffic("w", "attn_kernel") == 12345
    src.write_text("// kernel v2\n")
    assert bench.load_traffic("w", "attn_kernel") is None
    rec.unlink()
    assert bench.load_traffic("w", "attn_kernel") is None


def test_every_kernel_has_its_sources():
    for k in ("attn_kernel", "combine_kernel", "score_build_kernel", "score_kernel", "score_multi_kernel",
              "topk_kernel", "score_mfma_kernel", "topk_codes_kernel", "build_kernel"):
        for pth in bench.KERNEL_SOURCES[k]:
            assert os.path.exists(os.path.join(ROOT, pth)), pth


def test_attention_bytes_split_between_gather_and_combine():
    got = bench.attend_kernel_bytes(10_000_000, 32, combined=True)
    out = 32 * (16 * 256 * 2 + 16 * 4)
    assert got == {"attn_kernel": 10_000_000 - out, "combine_kernel": out}
    assert bench.attend_kernel_bytes(10_000_000, 32, combined=False) == {"attn_kernel": 10_000_000}


@pytest.mark.parametrize("kind", ["decode", "prefill", "indexshare"])
def test_oracle_baseline_over_worker_processes(kind):
    # the CPU baseline's machinery on a small workload: spawned workers map the staged
    # inputs and run the oracle's units; the report names the cores it used
    from block_sparse_attention_c4_amd import synth
    if kind == "prefill":
        wl = synth.make_workload("pool_pf", "prefill", 41, [3000], chunk=6)
    elif kind == "indexshare":
        wl = synth.make_workload("pool_is", "indexshare", 42, [2600, 1203], reuse_steps=3)
    else:
        wl = synth.make_workload("pool_dec", "decode", 43, [2600, 1203, 5000])
    b = bench.OracleBaseline(2)
    try:
        r = b.run(wl, seconds=0.5, seconds_single=0.2)
    finally:
        b.close()
    assert r["cores"] == 2 and r["kind"] == "oracle" and r["value"] > 0
    assert r["single_thread"]["cores"] == 1 and r["single_thread"]["value"] > 0
