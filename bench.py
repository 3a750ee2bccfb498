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
_COMMON = [_CSRC + f for f in ("qsa_device.h", "qsa_launch.h")]
_SRC_OF = {
    "qsa_attn.hip": ["attn_kernel", "combine_kernel"],
    "qsa_build.hip": ["build_kernel"],
    "qsa_index.hip": ["score_kernel", "score_build_kernel", "score_multi_kernel"],
    "qsa_topk.hip": ["topk_kernel", "topk_queued_kernel"],
    "qsa_prefill.hip": ["score_mfma_kernel", "topk_codes_kernel", "rescore_kernel"],
}
# the sources each kernel is compiled from (traffic figures are kept only while they hash the same)
KERNEL_SOURCES = {k: [_CSRC + f] + _COMMON + [_CSRC + "qsa_keymath.h"] for f, ks in _SRC_OF.items() for k in ks}
ENTRY = {"build": "qsa_build_index_keys", "index": "qsa_index_topk", "attend": "qsa_sparse_gqa_decode",
         "build_index": "qsa_decode_build_index_topk"}


def stage_kernels(kind: str, dw, fused: bool = False) -> dict:
    """The kernels each stage's call launches, in order (stage -> list of names)."""
    attend = ["attn_kernel"] + (["combine_kernel"] if dw.ws_attn_bytes > 0 else [])
    if kind == "verify":
        return {"build": ["build_kernel"],
                "index": ["score_multi_kernel"] * ((dw.T + 255) // 256) + ["topk_kernel"],
                "attend": attend}
    if kind == "prefill":
        return {"build": ["build_kernel"],
                "index": ["score_mfma_kernel", "topk_codes_kernel", "rescore_kernel", "topk_queued_kernel"],
                "attend": attend}
    if fused:
        return {"build_index": ["score_build_kernel", "topk_kernel"], "attend": attend}
    return {"build": ["build_kernel"], "index": ["score_kernel"] * ((dw.T + 63) // 64) + ["topk_kernel"],
            "attend": attend}


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


def attend_kernel_bytes(attend_bytes: int, n_queries: int, combined: bool) -> dict:
    """The attention call's algorithmic bytes split between its kernels: the gather
    reads K/V, positions and q; the output (16 x 256 bf16) and lse (16 floats) of each
    query are written by the combine when the list is split, else by the gather."""
    out = n_queries * (16 * 256 * 2 + 16 * 4)
    if not combined:
        return {"attn_kernel": attend_bytes}
    return {"attn_kernel": attend_bytes - out, "combine_kernel": out}


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


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter runs, or
    None if they were taken on different kernel sources."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get(kernel)
    if not ent:
        return None
    cur = source_hash([os.path.join(ROOT, p) for p in KERNEL_SOURCES[kernel]])
    return ent["bytes_per_launch"] if ent.get("source_hash") == cur else None


# ------------------------------------------------------------------ CPU baseline (oracle)

def host_cpu() -> dict:
    """The host the oracle ran on: CPU model, the processors the OS reports and the
    ones this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity": aff}


def oracle_workers() -> int:
    """Worker processes for the oracle: the CPUs this process may use, at most 16 (a
    one-GPU share of the host)."""
    return max(1, min(16, host_cpu()["affinity"]))


# The oracle's unit of work (one decode query, one prefill query row, or one
# IndexShare reuse step) runs in this process or in spawned workers.  Its inputs are
# .npy files in a scratch directory (under /dev/shm when it exists), which every
# worker maps read-only instead of receiving copies.
_UNIT_STATE = {}


def _unit_arrays(path: str) -> dict:
    if _UNIT_STATE.get("_dir") != path:
        _UNIT_STATE.clear()
        _UNIT_STATE["_dir"] = path
        for f in os.listdir(path):
            if f.endswith(".npy"):
                _UNIT_STATE[f[:-4]] = np.load(os.path.join(path, f), mmap_mode="r")
    return _UNIT_STATE


def _worker_init() -> None:
    from threadpoolctl import threadpool_limits
    _UNIT_STATE["_limits"] = threadpool_limits(limits=1)   # one BLAS thread per worker


def oracle_unit(task) -> int:
    """One unit of oracle work: task = (scratch dir, kind, unit index, meta)."""
    from oracle import qsa_oracle as O
    path, kind, u, meta = task
    A = _unit_arrays(path)
    ps, scale = meta["page_size"], 1.0 / 16.0
    scales = meta.get("kv_scales")
    if kind == "indexshare":
        b, j = divmod(u, meta["reuse_steps"])
        j += 1
        cap = np.asarray(A["cap_pos"][b, :int(A["cap_cnt"][b])])
        O.indexshare_step(cap, int(A["q_pos"][b]), j, A["reuse_q"][j - 1, b], A["page_table"][b],
                          A["k_pool"], A["v_pool"], ps, scale, kv_scales=scales)
        return 1
    t = u
    b = int(A["q_req"][t])
    p = int(A["q_pos"][t])
    keys = A["comp"][int(A["comp_off"][b]):int(A["comp_off"][b + 1])]
    if kind == "decode" and (p + 1) % 4 == 0:
        # the query's own token completes block p // 4: its key joins the prefix keys
        c = p // 4
        keys = np.concatenate([keys, O.compress_blocks(np.asarray(A["last_block"][b])[None],
                                                       np.array([4 * c]), meta["theta"])])
    O.query(keys, A["idx_q"][t], A["idx_w"][t], A["q"][t], p, A["page_table"][b], A["k_pool"],
            A["v_pool"], ps, scale, kv_scales=scales)
    return 1


class OracleBaseline:
    """The oracle timed on the host beside the GPU result: once on one thread, once
    over `workers` spawned processes.  The pool is started before anything touches
    the GPU, so its processes never inherit a GPU context."""

    def __init__(self, workers: int):
        import multiprocessing as mp
        self.workers = workers
        self.pool = mp.get_context("spawn").Pool(workers, initializer=_worker_init) if workers > 1 else None

    def close(self) -> None:
        if self.pool is not None:
            self.pool.terminate()
            self.pool.join()

    def _stage(self, wl, kv: str):
        """Write the units' inputs to a scratch directory; returns (dir, kind, units,
        meta, timed setup seconds).  Prefix keys are built untimed; a prefill chunk's
        own compressed keys are built inside the timed region, as the GPU step does."""
        import tempfile
        from oracle import qsa_oracle as O
        root = "/dev/shm" if os.path.isdir("/dev/shm") else None
        path = tempfile.mkdtemp(prefix="qsa_oracle_", dir=root)
        k_pool, v_pool, scales = O.kv_pools(wl, kv)
        meta = {"page_size": wl.page_size, "theta": wl.rope_theta, "kv_scales": scales,
                "reuse_steps": wl.reuse_steps}
        arrays = {"k_pool": k_pool, "v_pool": v_pool, "page_table": wl.page_table, "q_req": wl.q_req,
                  "q_pos": wl.q_pos, "idx_q": wl.idx_q, "idx_w": wl.idx_w, "q": wl.q}
        timed = 0.0
        kind = wl.kind
        if kind == "prefill":
            pre = [O.build_index_state(wl.raw_idx_k[b], int(wl.prefix_len[b]), wl.rope_theta)[0]
                   for b in range(wl.batch)]
            t0 = time.perf_counter()
            comp = []
            for b in range(wl.batch):
                c0, c1 = int(wl.prefix_len[b]) // 4, int(wl.lengths[b]) // 4
                blk = O.compress_blocks(wl.raw_idx_k[b][4 * c0:4 * c1].reshape(-1, 4, 128),
                                        4 * np.arange(c0, c1), wl.rope_theta)
                comp.append(np.concatenate([pre[b], blk]))
            timed = time.perf_counter() - t0
            units = list(range(wl.total_q))
        else:
            # keys of the blocks complete before each query's own token
            comp = [O.build_index_state(wl.raw_idx_k[b], int(wl.q_pos[b]), wl.rope_theta)[0]
                    for b in range(wl.batch)]
            last = np.zeros((wl.batch, 4, 128), np.uint16)
            for b in range(wl.batch):
                p = int(wl.q_pos[b])
                c = p // 4
                last[b, :p + 1 - 4 * c] = wl.raw_idx_k[b][4 * c:p + 1]
            arrays["last_block"] = last
            units = list(range(wl.batch))
            if kind == "indexshare":
                cap_pos = np.full((wl.batch, O.MAX_SELECTED), -1, np.int64)
                cap_cnt = np.zeros(wl.batch, np.int64)
                with_block = [comp[b] if (int(wl.q_pos[b]) + 1) % 4 else np.concatenate(
                    [comp[b], O.compress_blocks(last[b][None], np.array([4 * (int(wl.q_pos[b]) // 4)]),
                                                wl.rope_theta)]) for b in range(wl.batch)]
                for b in range(wl.batch):
                    pos = O.query(with_block[b], wl.idx_q[b], wl.idx_w[b], wl.q[b], int(wl.q_pos[b]),
                                  wl.page_table[b], k_pool, v_pool, wl.page_size, 1.0 / 16.0,
                                  kv_scales=scales)["positions"]
                    cap_pos[b, :len(pos)] = pos
                    cap_cnt[b] = len(pos)
                arrays.update(cap_pos=cap_pos, cap_cnt=cap_cnt, reuse_q=wl.reuse_q)
                units = list(range(wl.batch * wl.reuse_steps))
        arrays["comp"] = np.concatenate(comp)
        arrays["comp_off"] = np.concatenate([[0], np.cumsum([len(c) for c in comp])]).astype(np.int64)
        for name, arr in arrays.items():
            np.save(os.path.join(path, name + ".npy"), np.ascontiguousarray(arr))
        return path, kind, units, meta, timed

    def run(self, wl, seconds: float, seconds_single: float, kv: str = "bf16") -> dict:
        import shutil
        from threadpoolctl import threadpool_limits
        path, kind, units, meta, t_setup = self._stage(wl, kv)
        what = {"decode": "decode queries", "prefill": "prefill query rows",
                "indexshare": "IndexShare reuse steps (request x step)"}[kind]
        try:
            tasks = [(path, kind, u, meta) for u in units]
            # one thread: whole passes over the units, for about seconds_single
            with threadpool_limits(limits=1):
                oracle_unit(tasks[0])               # maps the inputs, untimed
                done, t0 = 0, time.perf_counter()
                while time.perf_counter() - t0 < seconds_single:
                    for task in tasks:
                        done += oracle_unit(task)
                        if kind == "prefill" and time.perf_counter() - t0 >= seconds_single:
                            break
                el1 = time.perf_counter() - t0 + t_setup
            single = {"value": done / el1, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                      "sample": f"{done} {what} of the same workload on one thread, float64 numpy "
                                f"oracle, {el1:.1f} s"}
            if self.pool is None:
                return dict(single, single_thread=dict(single))
            # every worker: the same units, cycled through the pool, for about `seconds`
            warm = (tasks * (self.workers // len(tasks) + 1))[:self.workers]
            self.pool.map(oracle_unit, warm, chunksize=1)   # maps the inputs, untimed
            done, t0 = 0, time.perf_counter()
            rounds = max(1, (4 * self.workers + len(tasks) - 1) // len(tasks))
            while time.perf_counter() - t0 < seconds:
                done += sum(self.pool.imap_unordered(oracle_unit, tasks * rounds, chunksize=1))
            el = time.perf_counter() - t0 + t_setup
            return {"value": done / el, "unit": "tokens/s", "cores": self.workers, "kind": "oracle",
                    "sample": f"{done} {what} of the same workload over {self.workers} worker "
                              f"processes (one BLAS thread each), float64 numpy oracle, {el:.1f} s",
                    "single_thread": single}
        finally:
            shutil.rmtree(path, ignore_errors=True)


# ------------------------------------------------------------------ GPU timing

def capture_round(torch, fns, outs, refs):
    """One hipGraph that runs every callable once, in order (steps cycling the input copies).
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


def time_stages(torch, sets, stages, K: int):
    """Mean durations (us) of each stage and of each kernel from HIP events, over K
    back-to-back steps queued on the launch stream behind a spin kernel.

    stages: (name, fn(d), kernels) with the kernel names the stage's call launches in
    order.  Events recorded on the stream before the step and after every call time
    the stages.  Each kernel gets a (start, stop) event pair that the library passes to
    its launch (qsa_profile_kernel_events, hipExtLaunchKernelGGL), so a kernel's time
    is its own dispatch's duration.  Returns ({stage or kernel: mean us}, {stage:
    [p10, p50, p90]}); a kernel launched several times in a step is summed per step."""
    from block_sparse_attention_c4_amd import binding as Bnd
    n_k = sum(len(k) for _, _, k in stages)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(1 + len(stages) + 2 * n_k)]
          for _ in range(K)]
    for row in ev:                     # torch creates an event at its first record
        for e in row:
            e.record()
    torch.cuda.synchronize()
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(int(100e6))
    for i in range(K):
        d = sets[i % len(sets)]
        e = ev[i]
        e[0].record()
        kp = 1 + len(stages)           # this step's kernel event pairs start here
        for j, (_, fn, kernels) in enumerate(stages):
            Bnd.qsa_profile_kernel_events(e[kp:kp + 2 * len(kernels)])
            fn(d)
            e[1 + j].record()
            kp += 2 * len(kernels)
    torch.cuda.synchronize()
    st = {"step": []}
    for name, _, kernels in stages:
        st[name] = []
        for k in kernels:
            st.setdefault(k, [])
    for e in ev:
        per_kernel = {}
        kp = 1 + len(stages)
        for j, (name, _, kernels) in enumerate(stages):
            st[name].append(e[j].elapsed_time(e[1 + j]))
            for k in kernels:
                per_kernel[k] = per_kernel.get(k, 0.0) + e[kp].elapsed_time(e[kp + 1])
                kp += 2
        for k, v in per_kernel.items():
            st[k].append(v)
        st["step"].append(e[0].elapsed_time(e[len(stages)]))
    stage_names = ["step"] + [name for name, _, _ in stages]
    return {k: float(np.mean(v)) * 1e3 for k, v in st.items()}, \
        {k: [round(float(np.percentile(st[k], q)) * 1e3, 2) for q in (10, 50, 90)] for k in stage_names}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--sets", type=int, default=None, help="input copies cycled through (cold cache)")
    ap.add_argument("--stage-steps", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle time over the worker processes")
    ap.add_argument("--cpu-seconds-single", type=float, default=6.0,
                    help="oracle time on one thread, reported beside")
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
    ap.add_argument("--no-others", action="store_true",
                    help="skip the shorter runs of the other workloads reported under "
                         "other_workloads (also skipped with --headline-only)")
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

    # the oracle's worker processes start before anything touches the GPU
    baseline = None if args.no_cpu_baseline else OracleBaseline(oracle_workers())
    try:
        return run(args, cfg, kind, steps, warmup, nsets, K, baseline)
    finally:
        if baseline is not None:
            baseline.close()


def run(args, cfg, kind, steps, warmup, nsets, K, baseline) -> int:
    import torch

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    torch.cuda.set_device(0)
    result, wl, kv = measure(args, args.workload, steps, warmup, nsets, K)
    if not args.no_ceilings:
        result["measured_ceilings"] = measured_ceilings(torch)
        if "step_hbm_gbps" in result:
            result["step_frac_of_measured_copy"] = round(
                result["step_hbm_gbps"] / result["measured_ceilings"]["stream_copy_gbps"], 4)
    if baseline is not None:
        result["cpu_baseline"] = baseline.run(wl, args.cpu_seconds, args.cpu_seconds_single, kv)
        result["cpu_baseline"]["host"] = host_cpu()
    del wl
    if not (args.headline_only or args.no_others):
        result["other_workloads"] = other_workloads(args, torch)
    print(json.dumps(result), flush=True)
    return 0


OTHER_SUMMARY_KEYS = ("metric", "value", "unit", "ms_per_step", "steps", "warmup", "kernel_us",
                      "ms_per_step_without_reuse", "tokens_per_s_without_reuse", "reuse_kernel_us",
                      "step_hbm_frac", "stage_tflops")


def other_workloads(args, torch) -> dict:
    """Every other workload, timed the same way with a quarter of its steps: the whole
    step through hipGraph replays, per-kernel HIP events, and the roofline of its
    dominant kernel."""
    import copy
    import gc

    out = {}
    sub = copy.copy(args)
    sub.headline_only = True
    sub.projection_overlap = 0
    sub.calib_copy_mib = 0
    for name, cfg in WORKLOADS.items():
        if name == args.workload:
            continue
        steps = max(10, cfg["steps"] // 4)
        warmup = max(2, cfg["warmup"] // 2)
        t0 = time.time()
        r, _, _ = measure(sub, name, steps, warmup, cfg["sets"], min(100, steps))
        summary = {k: r[k] for k in OTHER_SUMMARY_KEYS if k in r}
        rf = r["roofline"]
        summary["roofline"] = {k: rf[k] for k in ("bound", "kernel", "achieved", "peak", "unit", "frac")}
        summary["wall_s"] = round(time.time() - t0, 1)
        out[name] = summary
        del r
        gc.collect()
        torch.cuda.empty_cache()
    return out


def measure(args, name, steps, warmup, nsets, K):
    """One workload: returns (result line without ceilings or CPU baseline, the
    workload, its K/V format)."""
    import torch
    from block_sparse_attention_c4_amd import runner, synth

    cfg = WORKLOADS[name]
    kind = cfg["kind"]
    kv = cfg.get("kv", "bf16")
    wl = synth.FULL_SIZE[cfg.get("source", name)]()
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
        """ms per call of fns (cycled), as replays of one hipGraph unless --no-graph.
        A replay runs the calls in order, repeated so that it holds up to 16 calls
        when the timed steps fill at least 8 replays: the fixed cost of launching a
        graph (about 4.5 us here) is then shared by up to 16 steps, as it is when a
        step is part of a larger captured forward pass."""
        rounds = max(1, min(16 // len(fns), steps // (8 * len(fns))))
        fns, outs, refs = fns * rounds, outs * rounds, refs * rounds
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
    kernels = stage_kernels(kind, base, fused)
    if fused:
        stages = [("build_index", lambda d: d.build_index(), kernels["build_index"]),
                  ("attend", lambda d: d.attend(), kernels["attend"])]
    else:
        stages = [("build", build_fn, kernels["build"]), ("index", lambda d: d.index(), kernels["index"]),
                  ("attend", lambda d: d.attend(), kernels["attend"])]
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
        n_ws = runner.B.qsa_workspace_bytes(base.dims, runner.B.QSA_OP_GQA_DECODE, wl.batch, 0, 4)
        reuse_kernels = ["attn_kernel"] + (["combine_kernel"] if n_ws > 0 else [])
        rst, _ = time_stages(torch, sets, [("reuse", lambda d: d.attend(
            q=d.reuse_q[J - 1], extra=extras[J - 1], n_extra=4), reuse_kernels)], K)
        reuse = {"ms": ms_reuse, "attend_us": rst["reuse"], "kernels": reuse_kernels,
                 "kernel_us": {k: rst[k] for k in reuse_kernels}}

    if args.calib_copy_mib:
        # one elementwise kernel that reads and writes exactly n bytes: the scale of
        # the memory counters (FETCH_SIZE / WRITE_SIZE) against a known size
        n = args.calib_copy_mib << 20
        a = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()

    config = {"workload": name, "batch": wl.batch, "seed": wl.seed, "context": cfg["context"],
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
    stage_names = [name for name, _, _ in stages]
    result["stage_us"] = {k: round(stage_us[k], 2) for k in ["step"] + stage_names}
    result["stage_us_p10_p50_p90"] = stage_pct
    result["kernel_us"] = {k: round(v, 2) for k, v in stage_us.items() if k not in result["stage_us"]}
    result["stage_kernels"] = {name: ks for name, _, ks in stages}
    if ms_stream is not None:
        result["ms_per_step_stream_launches"] = round(ms_stream, 5)
        result["ms_per_step_warm"] = round(ms_warm, 5)
    if ms_unfused is not None:
        result["ms_per_step_builder_separate"] = round(ms_unfused, 5)
    if overlap is not None:
        result["projection_overlap"] = overlap
    result["timing"] = (f"value and ms_per_step: {steps} steps after {warmup} warm-up steps, host clock "
                        f"around synchronize(), {len(sets)} input copies cycled ({launch}); "
                        "stage_us: means of HIP events on the launch stream over "
                        f"{K} back-to-back steps; kernel_us: means of each kernel's start/stop HIP "
                        "events, set from its dispatch (qsa_profile_kernel_events); "
                        "ms_per_step_warm: one input copy, hipGraph replays; "
                        "ms_per_step_builder_separate: the same steps with the builder as its own call")

    def hbm_roofline(kernel, entry, nbytes_kernel, us):
        achieved = nbytes_kernel / (us * 1e-6) / 1e9
        return {"bound": "hbm", "kernel": kernel, "entry_point": entry, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": load_traffic(name, kernel), "bytes_per_launch": int(nbytes_kernel),
                "kernel_us": round(us, 2),
                "how": "algorithmic bytes of one launch over the kernel's mean duration from HIP events "
                       "(kernel_us)"}

    combined = "combine_kernel" in kernels["attend"]
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
        us = stage_us["score_mfma_kernel"]
        tf = work["score_flops"] / (us * 1e-6) / 1e12
        result["roofline"] = {"bound": "mfma", "kernel": "score_mfma_kernel", "entry_point": ENTRY["index"],
                              "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                              "traffic": load_traffic(name, "score_mfma_kernel"),
                              "flops_per_launch": work["score_flops"], "kernel_us": round(us, 2),
                              "how": "the scorer's FLOPs (4 heads x 128 dims x 2 per visible block of "
                                     "every query) over its mean duration from HIP events; "
                                     "stage_tflops.index_scoring is the same FLOPs over the whole "
                                     "indexer call"}
    elif kind == "indexshare":
        nbytes = decode_bytes(wl, counts)
        att = decode_bytes(wl, counts, n_extra=wl.reuse_steps)["attend"]
        result["value"] = round(wl.batch / (reuse["ms"] * 1e-3), 1)
        result["ms_per_step"] = round(reuse["ms"], 5)
        result["ms_per_step_without_reuse"] = round(ms_step, 5)
        result["tokens_per_s_without_reuse"] = round(wl.batch / (ms_step * 1e-3), 1)
        result["reuse_attend_us"] = round(reuse["attend_us"], 2)
        result["reuse_kernel_us"] = {k: round(v, 2) for k, v in reuse["kernel_us"].items()}
        result["reuse_timing"] = (f"MTP iterations of {wl.reuse_steps} reuse steps, one per input copy, "
                                  f"in one hipGraph per round; time divided by {wl.reuse_steps}")
        result["algorithmic_bytes"] = nbytes
        result["algorithmic_bytes_reuse_step"] = att
        split = attend_kernel_bytes(att, wl.batch, "combine_kernel" in reuse["kernels"])
        result["roofline"] = hbm_roofline("attn_kernel", ENTRY["attend"], split["attn_kernel"],
                                          reuse["kernel_us"]["attn_kernel"])
    elif kind == "verify":
        nbytes = verify_bytes(wl, base.sel_pos.cpu().numpy(), counts)
        config["query_tokens_per_request"] = int(wl.total_q // wl.batch)
        config["step_includes"] = "a device copy restoring the pending-token ring (1 KB per request)"
        result["value"] = round(wl.total_q / (ms_step * 1e-3), 1)
        result["ms_per_step"] = round(ms_step, 5)
        result["step_hbm_gbps"] = round(nbytes["step"] / (ms_step * 1e-3) / 1e9, 1)
        result["step_hbm_frac"] = round(nbytes["step"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
        result["algorithmic_bytes"] = nbytes
        split = attend_kernel_bytes(nbytes["attend"], wl.total_q, combined)
        result["roofline"] = hbm_roofline("attn_kernel", "qsa_sparse_gqa_prefill", split["attn_kernel"],
                                          stage_us["attn_kernel"])
    else:
        nbytes = decode_bytes(wl, counts, kv_bytes=1 if kv == "fp8" else 2)
        result["value"] = round(wl.batch / (ms_step * 1e-3), 1)
        result["ms_per_step"] = round(ms_step, 5)
        result["step_hbm_gbps"] = round(nbytes["step"] / (ms_step * 1e-3) / 1e9, 1)
        result["step_hbm_frac"] = round(nbytes["step"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
        result["algorithmic_bytes"] = nbytes
        split = attend_kernel_bytes(nbytes["attend"], wl.batch, combined)
        entry = "qsa_sparse_gqa_decode_fp8" if kv == "fp8" else ENTRY["attend"]
        result["roofline"] = hbm_roofline("attn_kernel", entry, split["attn_kernel"], stage_us["attn_kernel"])
    return result, wl, kv


if __name__ == "__main__":
    sys.exit(main())
