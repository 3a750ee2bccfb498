"""Drive the QSA c4 C ABI on a synthetic workload held in device memory.

Uploads a workload from `synth`, ingests the cached prefix's indexer keys, and
runs the three stages (builder, indexer, sparse GQA) through the binding.  It
holds no arithmetic of the method: every stage runs in libqsa's kernels.
"""

from __future__ import annotations

import numpy as np
import torch

from . import binding as B
from .synth import Workload

SEL_STRIDE = 2052          # >= 2051, a multiple of 4


def _u16(a: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)


def _i32(a, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).to(dev)


class DeviceWorkload:
    """A workload resident in HBM plus its output and scratch buffers."""

    def __init__(self, wl: Workload, device: str = "cuda:0", upload_pools: bool = True,
                 kv: str = "bf16"):
        """kv = "fp8": attention reads the workload's FP8 E4M3 pools (the bf16 pools are
        not uploaded)."""
        dev = torch.device(device)
        self.dev = dev
        self.wl = wl
        self.kv = kv
        self.dims = B.default_dims(wl.page_size, wl.rope_theta)
        self.batch = wl.batch
        self.T = wl.total_q
        self.page_table = _i32(wl.page_table, dev)   # -1 past each request's pages
        self.pt_stride = int(wl.page_table.shape[1])
        nslots = wl.num_pages * wl.page_size
        if upload_pools and kv == "fp8":
            self.k_pool = torch.from_numpy(np.ascontiguousarray(wl.k_pool_fp8)).to(dev)
            self.v_pool = torch.from_numpy(np.ascontiguousarray(wl.v_pool_fp8)).to(dev)
        elif upload_pools:
            self.k_pool = _u16(wl.k_pool, dev)
            self.v_pool = _u16(wl.v_pool, dev)
        self.comp = torch.zeros((nslots // 4, 128), dtype=torch.int16, device=dev)
        self.ring = torch.zeros((self.batch, 4, 128), dtype=torch.int16, device=dev)
        self.idx_q = _u16(wl.idx_q, dev)
        self.idx_w = torch.from_numpy(np.ascontiguousarray(wl.idx_w)).to(dev)
        self.q = _u16(wl.q, dev)
        self.q_req = _i32(wl.q_req, dev)
        self.q_pos = _i32(wl.q_pos, dev)
        self.max_pos = int(wl.q_pos.max()) + 1
        self.sel_blocks = torch.full((self.T, 512), -7, dtype=torch.int32, device=dev)
        self.sel_pos = torch.full((self.T, SEL_STRIDE), -7, dtype=torch.int32, device=dev)
        self.sel_count = torch.full((self.T,), -7, dtype=torch.int32, device=dev)
        self.out = torch.zeros((self.T, 16, 256), dtype=torch.int16, device=dev)
        self.lse = torch.zeros((self.T, 16), dtype=torch.float32, device=dev)
        self.ws_index_bytes = B.qsa_workspace_bytes(self.dims, B.QSA_OP_INDEX_TOPK, self.T, self.max_pos)
        self.ws_index = torch.empty(max(self.ws_index_bytes, 256), dtype=torch.uint8, device=dev)
        op = B.QSA_OP_GQA_PREFILL if wl.kind == "prefill" else B.QSA_OP_GQA_DECODE
        n_extra = 4 if wl.kind == "indexshare" else 0
        self.ws_attn_bytes = B.qsa_workspace_bytes(self.dims, op, self.T, 0, n_extra)
        self.ws_attn = torch.empty(max(self.ws_attn_bytes, 256), dtype=torch.uint8, device=dev)

        # the step's new indexer keys: the query token (decode) or the chunk (prefill)
        lens = wl.lengths
        pre = wl.prefix_len
        self.step_new_k = _u16(np.concatenate([wl.raw_idx_k[b][pre[b]:lens[b]] for b in range(self.batch)]), dev)
        n_new = (lens - pre).astype(np.int64)
        self.step_cu = _i32(np.concatenate([[0], np.cumsum(n_new)]), dev)
        self.step_len_before = _i32(pre, dev)
        self.step_total = int(n_new.sum())
        self.step_max = int(n_new.max())
        if wl.mpos is not None:     # MRoPE positions: a position ring and the step's positions
            self.ring_mpos = torch.zeros((self.batch, 4, 3), dtype=torch.int32, device=dev)
            self.step_mpos = _i32(np.concatenate([wl.mpos[b][pre[b]:lens[b]] for b in range(self.batch)]), dev)
        if wl.kind == "indexshare":
            self.extra = torch.full((self.batch, 4), -1, dtype=torch.int32, device=dev)
            self.reuse_q = _u16(wl.reuse_q, dev)

    # ---------------------------------------------------------------- stages
    def build_prefix(self, stream=None) -> None:
        """Ingest the indexer keys of every request's cached prefix (tokens before the step)."""
        wl = self.wl
        pre = wl.prefix_len
        if int(pre.sum()) == 0:
            return
        keys = np.concatenate([wl.raw_idx_k[b][:pre[b]] for b in range(self.batch)])
        new_k = _u16(keys, self.dev)
        cu = _i32(np.concatenate([[0], np.cumsum(pre)]), self.dev)
        lb = torch.zeros(self.batch, dtype=torch.int32, device=self.dev)
        if wl.mpos is not None:
            mp = _i32(np.concatenate([wl.mpos[b][:pre[b]] for b in range(self.batch)]), self.dev)
            B.qsa_build_index_keys_mrope(self.dims, self.batch, new_k, mp, cu, lb, int(pre.sum()),
                                         int(pre.max()), self.page_table, self.pt_stride, wl.pair_axis,
                                         self.ring, self.ring_mpos, self.comp, stream)
            del mp
        else:
            B.qsa_build_index_keys(self.dims, self.batch, new_k, cu, lb, int(pre.sum()), int(pre.max()),
                                   self.page_table, self.pt_stride, self.ring, self.comp, stream)
        del new_k   # the caching allocator orders its reuse after the launch on this stream

    def build_step(self, stream=None) -> None:
        if self.wl.mpos is not None:
            B.qsa_build_index_keys_mrope(self.dims, self.batch, self.step_new_k, self.step_mpos,
                                         self.step_cu, self.step_len_before, self.step_total,
                                         self.step_max, self.page_table, self.pt_stride,
                                         self.wl.pair_axis, self.ring, self.ring_mpos, self.comp, stream)
            return
        B.qsa_build_index_keys(self.dims, self.batch, self.step_new_k, self.step_cu,
                               self.step_len_before, self.step_total, self.step_max, self.page_table,
                               self.pt_stride, self.ring, self.comp, stream)

    def can_fuse(self) -> bool:
        """A decode step whose builder can be folded into the indexer call: one new
        token per request, which is also the request's query."""
        wl = self.wl
        return (self.T == self.batch and self.step_total == self.batch
                and self.step_max == 1 and np.array_equal(wl.q_req, np.arange(self.batch))
                and np.array_equal(wl.q_pos, wl.prefix_len))

    def build_index(self, stream=None) -> None:
        """Builder and indexer of a decode step in one call (qsa_decode_build_index_topk,
        or its MRoPE form)."""
        if self.wl.mpos is not None:
            B.qsa_decode_build_index_topk_mrope(
                self.dims, self.batch, self.step_new_k, self.step_mpos, self.step_len_before,
                self.max_pos, self.page_table, self.pt_stride, self.wl.pair_axis, self.ring,
                self.ring_mpos, self.comp, self.idx_q, self.idx_w, self.sel_blocks, self.sel_pos,
                SEL_STRIDE, self.sel_count, self.ws_index, self.ws_index_bytes, stream)
            return
        B.qsa_decode_build_index_topk(self.dims, self.batch, self.step_new_k, self.step_len_before,
                                      self.max_pos, self.page_table, self.pt_stride, self.ring,
                                      self.comp, self.idx_q, self.idx_w, self.sel_blocks,
                                      self.sel_pos, SEL_STRIDE, self.sel_count, self.ws_index,
                                      self.ws_index_bytes, stream)

    def index(self, stream=None) -> None:
        B.qsa_index_topk(self.dims, self.batch, self.T, self.idx_q, self.idx_w, self.q_req, self.q_pos,
                         self.max_pos, self.page_table, self.pt_stride, self.comp, self.sel_blocks,
                         self.sel_pos, SEL_STRIDE, self.sel_count, self.ws_index, self.ws_index_bytes,
                         stream)

    def attend(self, stream=None, q=None, extra=None, n_extra: int = 0) -> None:
        q = self.q if q is None else q
        if self.kv == "fp8" and self.wl.kind == "prefill":
            B.qsa_sparse_gqa_prefill_fp8(self.dims, self.T, q, self.q_req, self.k_pool, self.v_pool,
                                         self.wl.k_scale, self.wl.v_scale, self.page_table,
                                         self.pt_stride, self.sel_pos, self.sel_count, SEL_STRIDE,
                                         self.out, self.lse, self.ws_attn, self.ws_attn_bytes, stream)
        elif self.kv == "fp8":
            B.qsa_sparse_gqa_decode_fp8(self.dims, self.batch, q, self.k_pool, self.v_pool,
                                        self.wl.k_scale, self.wl.v_scale, self.page_table,
                                        self.pt_stride, self.sel_pos, self.sel_count, SEL_STRIDE,
                                        extra, n_extra, self.out, self.lse, self.ws_attn,
                                        self.ws_attn_bytes, stream)
        elif self.wl.kind == "prefill":
            B.qsa_sparse_gqa_prefill(self.dims, self.T, q, self.q_req, self.k_pool, self.v_pool,
                                     self.page_table, self.pt_stride, self.sel_pos, self.sel_count,
                                     SEL_STRIDE, self.out, self.lse, self.ws_attn, self.ws_attn_bytes,
                                     stream)
        else:
            B.qsa_sparse_gqa_decode(self.dims, self.batch, q, self.k_pool, self.v_pool,
                                    self.page_table, self.pt_stride, self.sel_pos, self.sel_count,
                                    SEL_STRIDE, extra, n_extra, self.out, self.lse, self.ws_attn,
                                    self.ws_attn_bytes, stream)

    def step(self, stream=None, fused: bool = False) -> None:
        """One pass of the hot path: builder, indexer, sparse GQA.  fused: the builder
        and the indexer as one call (decode steps that can_fuse())."""
        if fused:
            self.build_index(stream)
        else:
            self.build_step(stream)
            self.index(stream)
        self.attend(stream)

    def set_reuse(self, j: int) -> None:
        """Extra positions of IndexShare reuse step j: p_cap+1 .. p_cap+j, then -1."""
        ex = np.full((self.batch, 4), -1, dtype=np.int32)
        for b in range(self.batch):
            p_cap = int(self.wl.q_pos[b])
            ex[b, :j] = np.arange(p_cap + 1, p_cap + j + 1)
        self.extra.copy_(torch.from_numpy(ex))

    def reuse_step(self, j: int, stream=None) -> None:
        """IndexShare reuse step j (after set_reuse(j)): sparse GQA only."""
        self.attend(stream, q=self.reuse_q[j - 1], extra=self.extra, n_extra=4)

    def replicate(self) -> "DeviceWorkload":
        """An independent device copy of every buffer (same contents, new addresses)."""
        import copy
        other = copy.copy(self)
        for k, v in vars(self).items():
            if isinstance(v, torch.Tensor) and v.device.type == "cuda":
                setattr(other, k, v.clone())
        return other

    def device_bytes(self) -> int:
        return sum(v.numel() * v.element_size() for v in vars(self).values()
                   if isinstance(v, torch.Tensor) and v.device.type == "cuda")

    # ---------------------------------------------------------------- readback
    def comp_numpy(self) -> np.ndarray:
        return self.comp.cpu().numpy().view(np.uint16)

    def ring_numpy(self) -> np.ndarray:
        return self.ring.cpu().numpy().view(np.uint16)

    def out_f64(self) -> np.ndarray:
        o = self.out.cpu().numpy().view(np.uint16).astype(np.uint32) << 16
        return o.view(np.float32).astype(np.float64)
