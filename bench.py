#!/usr/bin/env python3
"""QSA c4 decode throughput on one MI355X.

Workload: batch 32 decode, context lengths log-uniform in [4096, 131072]
(seed 1003), 16 query / 2 KV heads of 256, indexer 4 x 128, top-512 blocks,
paged bf16 K/V (page 64) in one shared pool with interleaved pages.

A step is one pass of the whole hot path for the batch: ingest the query token's
indexer key (builder), score + top-512 + expansion (indexer), sparse GQA.  The
cached prefix's compressed keys are built once before timing.  Inputs are resident
in HBM; the timed loop cycles through --sets independent copies of the inputs so
that consecutive steps cannot be served from the 256 MB last-level cache.

Prints one JSON line.  --gpus above 1 is refused: nothing here spans GPUs.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QSA decode tokens/s at 128K ctx (indexer+top-k+sparse GQA); HBM GB/s vs peak"
WORKLOAD = "decode_b32_loguniform_4k_128k"
HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_b32_loguniform_4k_128k.json")


def algorithmic_bytes(wl, counts: np.ndarray) -> dict:
    """Bytes each stage must move (read + write), per step.  Counted: the new
    indexer key, ring and compressed key traffic of the builder; the compressed
    keys of every visible block, the indexer query and weights, and the written
    selection of the indexer; K and V of every selected position (both KV heads),
    the position list, the query and the output of sparse GQA.  Not counted:
    scratch scores, split partials and re-reads."""
    p = wl.q_pos.astype(np.int64)
    n_c = (p + 1) // 4
    completes = ((p + 1) % 4) == 0
    build = int(np.sum(256 + np.where(completes, 3 * 256 + 256, 256)))
    index = int(np.sum(256 * n_c + 4 * 128 * 2 + 4 * 4 + 512 * 4 + 4 * counts + 4))
    attend = int(np.sum(2 * 2 * 256 * 2 * counts + 4 * counts + 4 + 16 * 256 * 2 * 2 + 16 * 4))
    return {"build": build, "index": index, "attend": attend, "step": build + index + attend}


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for pth in paths:
        with open(pth, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


_CSRC = "block_sparse_attention_c4_amd/csrc/"
KERNEL_SOURCES = {
    "attend": [_CSRC + f for f in ("qsa_attn.hip", "qsa_device.h", "qsa_launch.h")],
    "index": [_CSRC + f for f in ("qsa_index.hip", "qsa_topk.hip", "qsa_device.h", "qsa_launch.h")],
    "build": [_CSRC + f for f in ("qsa_build.hip", "qsa_device.h", "qsa_launch.h")],
}
STAGE_KERNELS = {"build": "build_kernel", "index": "score_kernel + topk_kernel",
                 "attend": "attn_kernel + combine_kernel"}


def load_traffic(stage: str):
    """HBM bytes per launch of the stage's kernels from the committed rocprofv3
    counter runs, or None if they were taken on different kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    ent = rec.get(stage)
    if not ent:
        return None
    cur = source_hash([os.path.join(ROOT, p) for p in KERNEL_SOURCES[stage]])
    return ent["bytes_per_launch"] if ent.get("source_hash") == cur else None


def cpu_baseline(wl, seconds: float) -> dict:
    """The oracle's decode step on the same workload, single-threaded, repeated over
    the batch until `seconds` have passed (the prefix keys are built untimed)."""
    from threadpoolctl import threadpool_limits
    from oracle import qsa_oracle as O

    prefix = [O.build_index_state(wl.raw_idx_k[b], int(wl.q_pos[b]), wl.rope_theta)[0]
              for b in range(wl.batch)]
    done = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            for b in range(wl.batch):
                p = int(wl.q_pos[b])
                comp = prefix[b]
                if (p + 1) % 4 == 0:     # the query token completes a block
                    c = p // 4
                    blk = O.compress_blocks(wl.raw_idx_k[b][4 * c:4 * c + 4][None], np.array([4 * c]),
                                            wl.rope_theta)
                    comp = np.concatenate([comp, blk])
                O.query(comp, wl.idx_q[b], wl.idx_w[b], wl.q[b], p, wl.page_table[b], wl.k_pool,
                        wl.v_pool, wl.page_size, 1.0 / 16.0)
                done += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"value": done / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} decode queries ({done // wl.batch} passes over the batch of "
                      f"{wl.batch}) of the same workload, float64 numpy oracle, {el:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--sets", type=int, default=4, help="input copies cycled through (cold cache)")
    ap.add_argument("--stage-steps", type=int, default=200)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time plain stream launches")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device copy of this size (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the QSA hot path here has no multi-GPU part.", file=sys.stderr)
        return 2

    import torch
    from block_sparse_attention_c4_amd import runner, synth

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)
    wl = synth.FULL_SIZE[WORKLOAD]()
    base = runner.DeviceWorkload(wl, "cuda:0")
    base.build_prefix()
    torch.cuda.synchronize()
    sets = [base] + [base.replicate() for _ in range(args.sets - 1)]
    for d in sets:
        d.ws_attn.zero_()
    base.step()
    torch.cuda.synchronize()
    counts = base.sel_count.cpu().numpy().astype(np.int64)
    ref_out = base.out.clone()
    nbytes = algorithmic_bytes(wl, counts)

    # ---------------- headline: whole steps, hipGraph replay (or plain launches)
    launch = "stream"
    graphs = None
    if not args.no_graph:
        try:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for d in sets:
                    d.step()
            torch.cuda.current_stream().wait_stream(side)
            graphs = []
            for d in sets:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    d.step()
                graphs.append(g)
            torch.cuda.synchronize()
            # every replay must give the eager result
            for i, g in enumerate(graphs):
                sets[i].out.zero_()
                g.replay()
                torch.cuda.synchronize()
                assert torch.equal(sets[i].out, ref_out), "graph replay differs from eager step"
            launch = "hipgraph"
        except Exception as exc:  # noqa: BLE001
            print(f"graph capture unavailable ({exc}); timing stream launches", file=sys.stderr)
            graphs = None

    def run_step(i):
        if graphs is not None:
            graphs[i % len(graphs)].replay()
        else:
            sets[i % len(sets)].step()

    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    torch.cuda.synchronize()
    assert torch.equal(sets[(args.steps - 1) % len(sets)].out, ref_out)

    # ---------------- per-stage durations: HIP events on the launch stream, queued
    # behind a spin kernel so the GPU runs the stages back to back
    K = args.stage_steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(100e6))
    for i in range(K):
        d = sets[i % len(sets)]
        e = ev[i]
        e[0].record()
        d.build_step()
        e[1].record()
        d.index()
        e[2].record()
        d.attend()
        e[3].record()
    torch.cuda.synchronize()
    st = {"build": [], "index": [], "attend": [], "step": []}
    for e in ev:
        st["build"].append(e[0].elapsed_time(e[1]))
        st["index"].append(e[1].elapsed_time(e[2]))
        st["attend"].append(e[2].elapsed_time(e[3]))
        st["step"].append(e[0].elapsed_time(e[3]))
    stage_us = {k: float(np.mean(v)) * 1e3 for k, v in st.items()}
    dom = max(("build", "index", "attend"), key=lambda k: stage_us[k])
    achieved = nbytes[dom] / (stage_us[dom] * 1e-6) / 1e9

    if args.calib_copy_mib:
        # one elementwise kernel that reads and writes exactly n bytes: the scale of
        # the memory counters (FETCH_SIZE / WRITE_SIZE) against a known size
        n = args.calib_copy_mib << 20
        a = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()

    value = wl.batch / (ms_per_step * 1e-3)
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "batch": wl.batch, "seed": wl.seed,
                   "context": "log-uniform 4096..131072", "q_heads": 16, "kv_heads": 2,
                   "head_dim": 256, "indexer": "4x128", "topk_blocks": 512, "page_size": 64,
                   "input_sets": len(sets), "launch": launch},
        "step_hbm_gbps": round(nbytes["step"] / (ms_per_step * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(nbytes["step"] / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes": nbytes,
        "stage_us": {k: round(v, 2) for k, v in stage_us.items()},
        "roofline": {"bound": "hbm", "kernel": STAGE_KERNELS[dom], "entry_point": {
            "build": "qsa_build_index_keys", "index": "qsa_index_topk",
            "attend": "qsa_sparse_gqa_decode"}[dom],
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": load_traffic(dom)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
