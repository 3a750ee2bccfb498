#!/usr/bin/env python3
"""QSA c4 hot-path throughput on one MI355X.

Default workload (the headline): batch 32 decode, context lengths log-uniform in
[4096, 131072] (seed 1003), 16 query / 2 KV heads of 256, indexer 4 x 128,
top-512 blocks, paged bf16 K/V (page 64) in one shared pool with interleaved
pages.  --workload picks one of the other seeded workloads instead:

  decode_b1_l4099, decode_b8_l32k      other decode batches
  decode_b8_l131072                    batch 8 at exactly 131072 tokens (seed 1007)
  prefill_chunk4096_prefix126976       4096 new tokens on a 126976-token prefix
  indexshare_b4_l262140                batch 4 at L = 262140: IndexShare reuse steps,
                                       with full decode steps timed beside them
  verify_b32x4_loguniform_4k_128k      target verification: 4 query tokens per request
                                       (capture token + 3 drafts), batch 32, seed 1006
  decode_b32_loguniform_4k_128k_fp8kv  the headline decode with FP8 E4M3 K/V pools
  prefill_chunk4096_prefix126976_mrope the prefill chunk as image tokens (MRoPE builder)
  prefill_chunk4096_prefix126976_fp8kv the prefill chunk with FP8 E4M3 K/V pools

A step is one pass of the whole hot path for the batch: ingest the step's indexer
keys (builder), score + top-512 + expansion (indexer), sparse GQA.  A reuse step
is sparse GQA over the frozen selection plus the drafted positions.  The cached
prefix's compressed keys are built once before timing.  Inputs are resident in
HBM; the timed loop cycles through --sets independent copies of the inputs so
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

HEADLINE = "decode_b32_loguniform_4k_128k"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0

WORKLOADS = {
    "decode_b32_loguniform_4k_128k": dict(
        kind="decode", steps=2000, warmup=50, sets=4,
        metric="QSA decode tokens/s at 128K ctx (indexer+top-k+sparse GQA); HBM GB/s vs peak",
        context="log-uniform 4096..131072"),
    "decode_b8_l32k": dict(kind="decode", steps=2000, warmup=50, sets=4,
                           metric="QSA decode tokens/s, batch 8 at 32K ctx", context="32768 + U{0..3}"),
    "decode_b1_l4099": dict(kind="decode", steps=2000, warmup=50, sets=4,
                            metric="QSA decode tokens/s, batch 1 at 4099 ctx", context="4099"),
    "decode_b8_l131072": dict(kind="decode", steps=2000, warmup=50, sets=4,
                              metric="QSA decode tokens/s, batch 8 at 131072 ctx; HBM GB/s vs peak",
                              context="131072"),
    "prefill_chunk4096_prefix126976": dict(
        kind="prefill", steps=40, warmup=5, sets=2,
        metric="QSA chunked-prefill tokens/s, 4096-token chunk on a 126976-token prefix",
        context="126976 cached + 4096 new"),
    "indexshare_b4_l262140": dict(
        kind="indexshare", steps=1000, warmup=20, sets=4,
        metric="QSA IndexShare reuse-step tokens/s, batch 4 at 262140 ctx (full decode step beside it)",
        context="262140"),
    "decode_b32_loguniform_4k_128k_fp8kv": dict(
        kind="decode", kv="fp8", source="decode_b32_loguniform_4k_128k", steps=2000, warmup=50, sets=4,
        metric="QSA decode tokens/s at 128K ctx with an FP8 E4M3 K/V cache (indexer+top-k+sparse GQA); "
               "HBM GB/s vs peak",
        context="log-uniform 4096..131072"),
    "prefill_chunk4096_prefix126976_fp8kv": dict(
        kind="prefill", kv="fp8", source="prefill_chunk4096_prefix126976", steps=40, warmup=5, sets=2,
        metric="QSA chunked-prefill tokens/s with an FP8 E4M3 K/V cache, 4096-token chunk on a "
               "126976-token prefix",
        context="126976 cached + 4096 new"),
    "prefill_chunk4096_prefix126976_mrope": dict(
        kind="prefill", steps=40, warmup=5, sets=2,
        metric="QSA chunked-prefill tokens/s with MRoPE positions (the chunk is one 64 x 64 image)",
        context="126976 cached (a 4 x 32 x 32 video span inside) + 4096 new image tokens"),
    "verify_b32x4_loguniform_4k_128k": dict(
        kind="verify", steps=1000, warmup=20, sets=4,
        metric="QSA target-verify tokens/s, batch 32 x 4 query tokens, log-uniform 4K-128K ctx; "
               "HBM GB/s vs peak",
        context="log-uniform 4096..131072, 4 query tokens per request"),
}

_CSRC = "block_sparse_attention_c4_amd/csrc/"
KERNEL_SOURCES = {
    "attend": [_CSRC + f for f in ("qsa_attn.hip", "qsa_device.h", "qsa_launch.h")],
    "index": [_CSRC + f for f in ("qsa_index.hip", "qsa_topk.hip", "qsa_prefill.hip", "qsa_device.h",
                                  "qsa_keymath.h", "qsa_launch.h")],
    "build": [_CSRC + f for f in ("qsa_build.hip", "qsa_device.h", "qsa_keymath.h", "qsa_launch.h")],
    "build_index": [_CSRC + f for f in ("qsa_index.hip", "qsa_topk.hip", "qsa_device.h", "qsa_keymath.h",
                                        "qsa_launch.h")],
}
ENTRY = {"build": "qsa_build_index_keys", "index": "qsa_index_topk", "attend": "qsa_sparse_gqa_decode",
         "build_index": "qsa_decode_build_index_topk"}


def stage_kernels(kind: str, kv: str = "bf16", fused: bool = False) -> dict:
    if kind == "verify":
        return {"build": "build_kernel", "index": "score_multi_kernel + topk_kernel",
                "attend": "attn_kernel + combine_kernel"}
    if kind == "prefill":
        return {"build": "build_kernel",
                "index": "score_mfma_kernel + topk_codes_kernel (+ rescore_kernel, topk_queued_kernel)",
                "attend": "attn_kernel + combine_kernel"}
    attend = "attn_kernel<fp8> + combine_kernel" if kv == "fp8" else "attn_kernel + combine_kernel"
    if fused:
        return {"build_index": "score_build_kernel + topk_kernel", "attend": attend}
    return {"build": "build_kernel", "index": "score_kernel + topk_kernel", "attend": attend}


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


# ------------------------------------------------------------------ algorithmic work

def decode_bytes(wl, counts: np.ndarray, n_extra: int = 0, kv_bytes: int = 2) -> dict:
    """Bytes each decode stage must move (read + write), per step.  Counted: the new
    indexer key, ring and compressed key traffic of the builder; the compressed
    keys of every visible block, the indexer query and weights, and the written
    selection of the indexer; K and V of every attended position (both KV heads, at
    kv_bytes per element), the position list, the query and the output of sparse
    GQA.  Not counted: scratch scores, split partials and re-reads."""
    p = wl.q_pos.astype(np.int64)
    n_c = (p + 1) // 4
    completes = ((p + 1) % 4) == 0
    build = int(np.sum(256 + np.where(completes, 3 * 256 + 256, 256)))
    index = int(np.sum(256 * n_c + 4 * 128 * 2 + 4 * 4 + 512 * 4 + 4 * counts + 4))
    att = counts + n_extra
    attend = int(np.sum(2 * 2 * 256 * kv_bytes * att + 4 * att + 4 + 16 * 256 * 2 * 2 + 16 * 4))
    return {"build": build, "index": index, "attend": attend, "step": build + index + attend}


def verify_bytes(wl, sel_pos: np.ndarray, counts: np.ndarray) -> dict:
    """Bytes each stage must move (read + write) for a batch with a few query tokens
    per request.  Counted: the new raw keys and the compressed keys of blocks they
    complete; each request's visible compressed keys once (its queries share them),
    each query's indexer query, weights and written selection; K and V of the union
    of the positions a request's queries attend (both KV heads), each query's
    position list, query and output.  Not counted: scratch scores, split partials
    and re-reads."""
    p = wl.q_pos.astype(np.int64)
    n_new = int(np.sum(wl.lengths - wl.prefix_len))
    completed = int(np.sum(wl.lengths // 4 - wl.prefix_len // 4))
    build = n_new * 256 + completed * (256 + 3 * 256)
    index = int(256 * np.sum(wl.lengths // 4)) + int(np.sum(4 * 128 * 2 + 16 + 512 * 4 + 4 * counts + 4))
    unique = 0
    for b in range(wl.batch):
        rows = np.nonzero(wl.q_req == b)[0]
        unique += len(np.unique(np.concatenate([sel_pos[t, :counts[t]] for t in rows])))
    attend = 2 * 2 * 256 * 2 * unique + int(np.sum(4 * counts + 4 + 16 * 256 * 2 * 2 + 16 * 4))
    return {"build": build, "index": index, "attend": attend, "step": build + index + attend,
            "unique_positions": unique, "positions": int(np.sum(counts))}


def prefill_work(wl, counts: np.ndarray) -> dict:
    """FLOPs of the scorer (4 heads x 128 dims, 2 per multiply-add, for every
    visible block of every query) and of sparse GQA (QK and PV for 16 heads of 256
    over every attended position); the bytes of unique inputs and outputs."""
    p = wl.q_pos.astype(np.int64)
    n_c = (p + 1) // 4
    T = wl.total_q
    score_flops = int(np.sum(n_c) * 4 * 128 * 2)
    attn_flops = int(np.sum(counts) * 16 * 256 * 2 * 2)
    n_new = int(np.sum(wl.lengths - wl.prefix_len))
    build_bytes = n_new * 256 + (n_new // 4) * 256
    index_bytes = int(256 * np.sum(wl.lengths // 4) + T * (4 * 128 * 2 + 16 + 512 * 4 + 4 * 2051 + 4))
    attend_bytes = int(2 * 2 * 256 * 2 * np.sum(wl.lengths) + T * (16 * 256 * 2 * 2 + 4 * 2051 + 64))
    return {"score_flops": score_flops, "attn_flops": attn_flops,
            "bytes": {"build": build_bytes, "index": index_bytes, "attend": attend_bytes,
                      "step": build_bytes + index_bytes + attend_bytes}}


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for pth in paths:
        with open(pth, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, stage: str):
    """HBM bytes per launch of the stage's kernels from the committed rocprofv3
    counter runs, or None if they were taken on different kernel sources."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get(stage)
    if not ent:
        return None
    cur = source_hash([os.path.join(ROOT, p) for p in KERNEL_SOURCES[stage]])
    return ent["bytes_per_launch"] if ent.get("source_hash") == cur else None


# ------------------------------------------------------------------ CPU baseline (oracle)

def _oracle_keys_at(O, wl, b: int, prefix_keys, p: int):
    """A request's compressed keys as a query at p sees them: the prefix keys plus
    the block the query token completes, if it completes one."""
    if (p + 1) % 4:
        return prefix_keys
    c = p // 4
    blk = O.compress_blocks(wl.raw_idx_k[b][4 * c:4 * c + 4][None], np.array([4 * c]), wl.rope_theta)
    return np.concatenate([prefix_keys, blk])


def host_cpu() -> dict:
    """The host the oracle ran on: CPU model and the processors the OS reports."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count()}


def cpu_baseline(wl, seconds: float, kv: str = "bf16") -> dict:
    """The oracle on the same workload, single-threaded, for about `seconds`: decode
    queries over the batch, prefill query rows of the chunk, or IndexShare reuse
    steps.  The prefix keys are built untimed; for prefill the chunk's own
    compressed keys are built inside the timed region."""
    from threadpoolctl import threadpool_limits
    from oracle import qsa_oracle as O

    done = 0
    scale = 1.0 / 16.0
    with threadpool_limits(limits=1):
        if wl.kind == "prefill":
            pre = [O.build_index_state(wl.raw_idx_k[b], int(wl.prefix_len[b]), wl.rope_theta)[0]
                   for b in range(wl.batch)]
            t0 = time.perf_counter()
            comp = []
            for b in range(wl.batch):
                c0, c1 = int(wl.prefix_len[b]) // 4, int(wl.lengths[b]) // 4
                blk = O.compress_blocks(wl.raw_idx_k[b][4 * c0:4 * c1].reshape(-1, 4, 128),
                                        4 * np.arange(c0, c1), wl.rope_theta)
                comp.append(np.concatenate([pre[b], blk]))
            for t in range(wl.total_q):
                b = int(wl.q_req[t])
                O.query(comp[b], wl.idx_q[t], wl.idx_w[t], wl.q[t], int(wl.q_pos[t]), wl.page_table[b],
                        wl.k_pool, wl.v_pool, wl.page_size, scale)
                done += 1
                if time.perf_counter() - t0 >= seconds:
                    break
            el = time.perf_counter() - t0
            return {"value": done / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                    "sample": f"the chunk's compressed keys, then the first {done} of its "
                              f"{wl.total_q} query rows, float64 numpy oracle, {el:.1f} s"}
        prefix = [O.build_index_state(wl.raw_idx_k[b], int(wl.q_pos[b]), wl.rope_theta)[0]
                  for b in range(wl.batch)]
        if wl.kind == "indexshare":
            cap = {}
            for b in range(wl.batch):
                p = int(wl.q_pos[b])
                cap[b] = O.query(_oracle_keys_at(O, wl, b, prefix[b], p), wl.idx_q[b], wl.idx_w[b],
                                 wl.q[b], p, wl.page_table[b], wl.k_pool, wl.v_pool, wl.page_size,
                                 scale)["positions"]
            t0 = time.perf_counter()
            while True:
                for b in range(wl.batch):
                    j = 1 + done % wl.reuse_steps
                    O.indexshare_step(cap[b], int(wl.q_pos[b]), j, wl.reuse_q[j - 1, b], wl.page_table[b],
                                      wl.k_pool, wl.v_pool, wl.page_size, scale)
                    done += 1
                el = time.perf_counter() - t0
                if el >= seconds:
                    break
            return {"value": done / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                    "sample": f"{done} IndexShare reuse steps (request x step) of the same workload, "
                              f"float64 numpy oracle, {el:.1f} s"}
        k_pool, v_pool, scales = O.kv_pools(wl, kv)
        t0 = time.perf_counter()
        while True:
            for b in range(wl.batch):
                p = int(wl.q_pos[b])
                O.query(_oracle_keys_at(O, wl, b, prefix[b], p), wl.idx_q[b], wl.idx_w[b], wl.q[b], p,
                        wl.page_table[b], k_pool, v_pool, wl.page_size, scale, kv_scales=scales)
                done += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"value": done / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} decode queries ({done // wl.batch} passes over the batch of "
                      f"{wl.batch}) of the same workload, float64 numpy oracle, {el:.1f} s"}


# ------------------------------------------------------------------ GPU timing

def capture_round(torch, fns, outs, refs):
    """One hipGraph that runs every callable once, in order (one step per input copy).
    refs[i] is the eager result of fns[i] (in outs[i]); the graph is replayed twice and
    every output is checked against its eager result.  A replay covers len(fns) steps,
    so the fixed cost of launching a graph (about 4.5 us here) is paid once per round."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for fn in fns:
            fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in fns:
            fn()
    torch.cuda.synchronize()
    for _ in range(2):
        for out in outs:
            out.zero_()
        g.replay()
        torch.cuda.synchronize()
        for out, ref in zip(outs, refs):
            assert torch.equal(out, ref), "graph replay differs from the eager result"
    return g


def time_loop(torch, fns, graph, steps: int, warmup: int) -> float:
    """ms per step over exactly `steps` steps (fns cycled): whole rounds as graph
    replays when a graph is given, the remaining steps as stream launches."""
    n = len(fns)

    def run(k):
        if graph is not None:
            for _ in range(k // n):
                graph.replay()
            for i in range(k % n):
                fns[i]()
        else:
            for i in range(k):
                fns[i % n]()

    run(warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def measured_ceilings(torch) -> dict:
    """What this machine reaches on plain library work, beside the published peaks the
    roofline uses: a 1 GiB device-to-device copy (read + write bytes per second)
    and an 8192^3 bf16 matrix product (torch.mm, contiguous operands)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def best_ms(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            ev[0].record()
            fn()
            ev[1].record()
            torch.cuda.synchronize()
            best = min(best, ev[0].elapsed_time(ev[1]))
        return best

    n = 1 << 30
    a = torch.empty(n // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    copy_ms = best_ms(lambda: b.copy_(a))
    del a, b
    m = 8192
    x = torch.randn(m, m, device="cuda:0").to(torch.bfloat16)
    y = torch.randn(m, m, device="cuda:0").to(torch.bfloat16)
    z = torch.empty(m, m, dtype=torch.bfloat16, device="cuda:0")
    mm_ms = best_ms(lambda: torch.mm(x, y, out=z))
    del x, y, z
    return {"stream_copy_gbps": round(2 * n / (copy_ms * 1e-3) / 1e9, 1),
            "gemm_bf16_tflops": round(2 * m ** 3 / (mm_ms * 1e-3) / 1e12, 1),
            "how": "best of 10: a 1 GiB device copy (bytes read + written), torch.mm of two "
                   "8192x8192 bf16 matrices"}


def projection_overlap(torch, sets, hidden: int, timed, ref_out) -> dict:
    """A decode step beside a stand-in for the layer's Q/K/V projection, whose output
    the indexer does not need: x[batch, hidden] x W[hidden, 5120] in bf16 (16 + 2 + 2
    heads of 256; synthetic weights, the product is discarded).  Sequential: the
    projection, then builder + indexer, then attention, on one stream.  Overlapped:
    builder + indexer on a second stream (default priority) while the projection runs,
    joined before attention.  Both as hipGraphs of one step per input copy."""
    dev = sets[0].dev
    B = sets[0].batch
    x = torch.randn(B, hidden, device=dev).to(torch.bfloat16)
    w = (torch.randn(hidden, 5120, device=dev) * hidden ** -0.5).to(torch.bfloat16)
    y = torch.empty(B, 5120, dtype=torch.bfloat16, device=dev)
    side = torch.cuda.Stream()
    torch.mm(x, w, out=y)
    torch.cuda.synchronize()

    def seq(d):
        def run():
            torch.mm(x, w, out=y)
            d.build_index()
            d.attend()
        return run

    def par(d):
        def run():
            cur = torch.cuda.current_stream()
            side.wait_stream(cur)
            with torch.cuda.stream(side):
                d.build_index()
            torch.mm(x, w, out=y)
            cur.wait_stream(side)
            d.attend()
        return run

    outs = [d.out for d in sets]
    refs = [ref_out] * len(sets)
    ms_proj, _ = timed([lambda: torch.mm(x, w, out=y)] * len(sets), [], [])
    ms_seq, _ = timed([seq(d) for d in sets], outs, refs)
    ms_par, _ = timed([par(d) for d in sets], outs, refs)
    return {"hidden": hidden, "proj_cols": 5120, "proj_alone_us": round(ms_proj * 1e3, 2),
            "ms_per_step_sequential": round(ms_seq, 5), "ms_per_step_overlapped": round(ms_par, 5),
            "how": "stand-in projection torch.mm bf16 on the launch stream; builder + indexer "
                   "(qsa_decode_build_index_topk) on a second default-priority stream; hipGraph "
                   "replays, outputs checked against the eager step"}


def time_stages(torch, sets, stages, K: int) -> dict:
    """Mean duration (us) of each stage from HIP events recorded on the launch
    stream; the launches queue behind a spin kernel so the GPU runs them back to
    back."""
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(100e6))
    for i in range(K):
        d = sets[i % len(sets)]
        e = ev[i]
        e[0].record()
        for j, (_, fn) in enumerate(stages):
            fn(d)
            e[j + 1].record()
    torch.cuda.synchronize()
    st = {name: [] for name, _ in stages}
    st["step"] = []
    for e in ev:
        for j, (name, _) in enumerate(stages):
            st[name].append(e[j].elapsed_time(e[j + 1]))
        st["step"].append(e[0].elapsed_time(e[-1]))
    return {k: float(np.mean(v)) * 1e3 for k, v in st.items()}, \
        {k: [round(float(np.percentile(v, q)) * 1e3, 2) for q in (10, 50, 90)] for k, v in st.items()}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--sets", type=int, default=None, help="input copies cycled through (cold cache)")
    ap.add_argument("--stage-steps", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the plain-launch and warm step timings (profiled runs: every traced "
                         "step is then a cold one)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the copy and matrix-product ceilings measured beside the result")
    ap.add_argument("--no-graph", action="store_true", help="time plain stream launches")
    ap.add_argument("--projection-overlap", type=int, default=0, metavar="HIDDEN",
                    help="decode: also time the step beside a stand-in Q/K/V projection "
                         "([batch, HIDDEN] x [HIDDEN, 5120] bf16), once in sequence and once with the "
                         "builder + indexer on a second stream overlapping it")
    ap.add_argument("--unfused", action="store_true",
                    help="decode: run the builder and the indexer as two calls (by default one "
                         "qsa_decode_build_index_topk call does both)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one elementwise kernel over this size (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the QSA hot path here has no multi-GPU part.", file=sys.stderr)
        return 2

    cfg = WORKLOADS[args.workload]
    kind = cfg["kind"]
    steps = args.steps if args.steps is not None else cfg["steps"]
    warmup = args.warmup if args.warmup is not None else cfg["warmup"]
    nsets = args.sets if args.sets is not None else cfg["sets"]
    K = args.stage_steps if args.stage_steps is not None else min(200, steps)

    import torch
    from block_sparse_attention_c4_amd import runner, synth

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)
    kv = cfg.get("kv", "bf16")
    wl = synth.FULL_SIZE[cfg.get("source", args.workload)]()
    if kv == "fp8":
        synth.with_fp8_kv(wl)
    base = runner.DeviceWorkload(wl, "cuda:0", kv=kv)
    base.build_prefix()
    torch.cuda.synchronize()
    sets = [base] + [base.replicate() for _ in range(nsets - 1)]
    for d in sets:
        d.ws_attn.zero_()
    # A chunk that starts inside a block reads that block's older tokens from the
    # 4-slot ring and leaves the tokens of its own last, unfinished block in the same
    # slots, so a repeated step would read the newer tokens.  Where that happens
    # (target verification at arbitrary lengths) every step first restores the
    # ring: a device copy of 1 KB per request, counted in the step.
    restore = kind == "verify"
    if restore:
        for d in sets:
            d.ring_saved = d.ring.clone()

    # decode steps ingest each request's token inside the indexer call
    fused = kind in ("decode", "indexshare") and not args.unfused and base.can_fuse()

    def step_fn(d, fused=fused):
        if not restore:
            return lambda: d.step(fused=fused)

        def run():
            d.ring.copy_(d.ring_saved)
            d.step()
        return run

    def build_fn(d):
        if restore:
            d.ring.copy_(d.ring_saved)
        d.build_step()

    step_fn(base)()
    torch.cuda.synchronize()
    counts = base.sel_count.cpu().numpy().astype(np.int64)
    ref_out = base.out.clone()

    def timed(fns, outs, refs):
        """ms per call of fns (cycled), as replays of one hipGraph per round of
        len(fns) calls unless --no-graph."""
        graph = None
        if not args.no_graph:
            try:
                graph = capture_round(torch, fns, outs, refs)
            except AssertionError:
                raise
            except Exception as exc:  # noqa: BLE001
                print(f"graph capture unavailable ({exc}); timing stream launches", file=sys.stderr)
        launch = f"hipgraph of {len(fns)} steps per replay" if graph is not None else "stream"
        return time_loop(torch, fns, graph, steps, warmup), launch

    # ---------------- whole steps
    ms_step, launch = timed([step_fn(d) for d in sets], [d.out for d in sets], [ref_out] * len(sets))
    assert torch.equal(sets[(steps - 1) % len(sets)].out, ref_out)
    # the same steps as plain stream launches, and a warm variant: one input copy
    # every step, so the last-level cache may serve what the previous step read
    ms_stream = ms_warm = None
    if not args.headline_only:
        ms_stream = time_loop(torch, [step_fn(d) for d in sets], None, steps, warmup)
        ms_warm, _ = timed([step_fn(sets[0])], [sets[0].out], [ref_out])
    ms_unfused = None
    if fused and not args.headline_only:
        ms_unfused, _ = timed([step_fn(d, False) for d in sets], [d.out for d in sets], [ref_out] * len(sets))
    if fused:
        stages = [("build_index", lambda d: d.build_index()), ("attend", lambda d: d.attend())]
    else:
        stages = [("build", build_fn), ("index", lambda d: d.index()), ("attend", lambda d: d.attend())]
    stage_us, stage_pct = time_stages(torch, sets, stages, K)

    # ---------------- the indexer on a second stream beside a projection
    overlap = None
    if fused and args.projection_overlap > 0:
        overlap = projection_overlap(torch, sets, args.projection_overlap, timed, ref_out)

    # ---------------- IndexShare: reuse steps j = 1..3 cycled over the input copies
    reuse = None
    if kind == "indexshare":
        J = wl.reuse_steps
        extras = []
        for j in range(1, J + 1):
            ex = np.full((wl.batch, 4), -1, dtype=np.int32)
            for b in range(wl.batch):
                ex[b, :j] = np.arange(int(wl.q_pos[b]) + 1, int(wl.q_pos[b]) + j + 1)
            extras.append(torch.from_numpy(ex).to("cuda:0"))

        def mtp_iteration(d):
            # the draft steps of one MTP iteration, back to back: reuse steps 1..J
            def run():
                for j in range(1, J + 1):
                    d.attend(q=d.reuse_q[j - 1], extra=extras[j - 1], n_extra=4)
            return run

        fns = [mtp_iteration(d) for d in sets]
        refs = []
        for d, fn in zip(sets, fns):
            fn()
            torch.cuda.synchronize()
            refs.append(d.out.clone())
        ms_reuse = timed(fns, [d.out for d in sets], refs)[0] / J
        rst, _ = time_stages(torch, sets, [("reuse", lambda d: d.attend(
            q=d.reuse_q[J - 1], extra=extras[J - 1], n_extra=4))], K)
        reuse = {"ms": ms_reuse, "attend_us": rst["reuse"]}

    if args.calib_copy_mib:
        # one elementwise kernel that reads and writes exactly n bytes: the scale of
        # the memory counters (FETCH_SIZE / WRITE_SIZE) against a known size
        n = args.calib_copy_mib << 20
        a = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()

    kernels = stage_kernels(kind, kv, fused)
    config = {"workload": args.workload, "batch": wl.batch, "seed": wl.seed, "context": cfg["context"],
              "q_heads": 16, "kv_heads": 2, "head_dim": 256, "indexer": "4x128", "topk_blocks": 512,
              "page_size": wl.page_size, "input_sets": len(sets), "launch": launch}
    if kv == "fp8":
        config["kv_cache"] = "fp8 e4m3, one scale per pool"
    if kind in ("decode", "indexshare"):
        config["builder"] = ("folded into the indexer call (qsa_decode_build_index_topk)" if fused
                             else "its own call (qsa_build_index_keys)")
    if getattr(wl, "mpos", None) is not None:
        config["rope"] = "mrope, contiguous sections 16/24/24 of the 64 indexer pairs"
        config["vision_spans"] = [list(map(list, spans)) for spans in synth.PREFILL_MROPE_SPANS]
    result = {"metric": cfg["metric"], "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": steps,
              "warmup": warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": config}
    result["stage_us"] = {k: round(v, 2) for k, v in stage_us.items()}
    result["stage_us_p10_p50_p90"] = stage_pct
    if ms_stream is not None:
        result["ms_per_step_stream_launches"] = round(ms_stream, 5)
        result["ms_per_step_warm"] = round(ms_warm, 5)
    if ms_unfused is not None:
        result["ms_per_step_builder_separate"] = round(ms_unfused, 5)
    if overlap is not None:
        result["projection_overlap"] = overlap
    result["timing"] = (f"value and ms_per_step: {steps} steps after {warmup} warm-up steps, host clock "
                        f"around synchronize(), {len(sets)} input copies cycled ({launch}); "
                        "stage_us: means of HIP events on the launch stream over back-to-back steps; "
                        "ms_per_step_warm: one input copy, hipGraph replays; "
                        "ms_per_step_builder_separate: the same steps with the builder as its own call")

    if kind == "prefill":
        work = prefill_work(wl, counts)
        config["chunk"] = int(wl.total_q)
        result["value"] = round(wl.total_q / (ms_step * 1e-3), 1)
        result["ms_per_step"] = round(ms_step, 5)
        score_tf = work["score_flops"] / (stage_us["index"] * 1e-6) / 1e12
        attn_tf = work["attn_flops"] / (stage_us["attend"] * 1e-6) / 1e12
        result["stage_tflops"] = {"index_scoring": round(score_tf, 1), "attend": round(attn_tf, 1)}
        result["algorithmic"] = {"score_flops": work["score_flops"], "attn_flops": work["attn_flops"],
                                 "unique_bytes": work["bytes"]}
        # the scorer's FLOPs over the whole indexer call (scorer + code select): a
        # lower bound on the scorer kernel's own rate
        result["roofline"] = {"bound": "mfma", "kernel": kernels["index"], "entry_point": ENTRY["index"],
                              "achieved": round(score_tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(score_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                              "traffic": load_traffic(args.workload, "index")}
    elif kind == "indexshare":
        nbytes = decode_bytes(wl, counts)
        att = decode_bytes(wl, counts, n_extra=wl.reuse_steps)["attend"]
        result["value"] = round(wl.batch / (reuse["ms"] * 1e-3), 1)
        result["ms_per_step"] = round(reuse["ms"], 5)
        result["ms_per_step_without_reuse"] = round(ms_step, 5)
        result["tokens_per_s_without_reuse"] = round(wl.batch / (ms_step * 1e-3), 1)
        result["reuse_attend_us"] = round(reuse["attend_us"], 2)
        result["reuse_timing"] = (f"MTP iterations of {wl.reuse_steps} reuse steps, one per input copy, "
                                  f"in one hipGraph per round; time divided by {wl.reuse_steps}")
        result["algorithmic_bytes"] = nbytes
        result["algorithmic_bytes_reuse_step"] = att
        achieved = att / (reuse["attend_us"] * 1e-6) / 1e9
        result["roofline"] = {"bound": "hbm", "kernel": kernels["attend"], "entry_point": ENTRY["attend"],
                              "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                              "frac": round(achieved / HBM_PEAK_GBPS, 4),
                              "traffic": load_traffic(args.workload, "attend")}
    elif kind == "verify":
        nbytes = verify_bytes(wl, base.sel_pos.cpu().numpy(), counts)
        config["query_tokens_per_request"] = int(wl.total_q // wl.batch)
        config["step_includes"] = "a device copy restoring the pending-token ring (1 KB per request)"
        result["value"] = round(wl.total_q / (ms_step * 1e-3), 1)
        result["ms_per_step"] = round(ms_step, 5)
        result["step_hbm_gbps"] = round(nbytes["step"] / (ms_step * 1e-3) / 1e9, 1)
        result["step_hbm_frac"] = round(nbytes["step"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
        result["algorithmic_bytes"] = nbytes
        dom = "attend"   # it holds the step's longest kernel (attn_kernel) and most of its bytes
        achieved = nbytes[dom] / (stage_us[dom] * 1e-6) / 1e9
        entry = "qsa_sparse_gqa_prefill" if dom == "attend" else ENTRY[dom]
        result["roofline"] = {"bound": "hbm", "kernel": kernels[dom], "entry_point": entry,
                              "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                              "frac": round(achieved / HBM_PEAK_GBPS, 4),
                              "traffic": load_traffic(args.workload, dom)}
    else:
        nbytes = decode_bytes(wl, counts, kv_bytes=1 if kv == "fp8" else 2)
        result["value"] = round(wl.batch / (ms_step * 1e-3), 1)
        result["ms_per_step"] = round(ms_step, 5)
        result["step_hbm_gbps"] = round(nbytes["step"] / (ms_step * 1e-3) / 1e9, 1)
        result["step_hbm_frac"] = round(nbytes["step"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
        result["algorithmic_bytes"] = nbytes
        dom = "attend"   # it holds the step's longest kernel (attn_kernel) and most of its bytes
        achieved = nbytes[dom] / (stage_us[dom] * 1e-6) / 1e9
        entry = "qsa_sparse_gqa_decode_fp8" if (dom == "attend" and kv == "fp8") else ENTRY[dom]
        result["roofline"] = {"bound": "hbm", "kernel": kernels[dom], "entry_point": entry,
                              "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                              "frac": round(achieved / HBM_PEAK_GBPS, 4),
                              "traffic": load_traffic(args.workload, dom)}

    if not args.no_ceilings:
        result["measured_ceilings"] = measured_ceilings(torch)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, kv)
        result["cpu_baseline"]["host"] = host_cpu()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
