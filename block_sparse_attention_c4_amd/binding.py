"""Python binding of libqsa.so: the C ABI of include/qsa.h, one function per entry
point with the same name and argument order.  Argument marshalling only:
tensors become device pointers, the stream defaults to torch's current stream,
and a non-OK status raises QsaError.  Every step of the path runs in the
library's HIP kernels.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("QSA_LIB", os.path.join(_HERE, "libqsa.so"))

QSA_OK = 0
QSA_E_NULL = 1
QSA_E_SHAPE = 2
QSA_E_UNSUPPORTED = 3
QSA_E_WORKSPACE = 4
QSA_E_HIP = 5
QSA_E_SCRATCH = 6

QSA_OP_INDEX_TOPK = 1
QSA_OP_GQA_DECODE = 2
QSA_OP_GQA_PREFILL = 3

QSA_BLOCK = 4
QSA_TOPK = 512
QSA_MAX_SEL = 2051
QSA_MAX_CONTEXT = 262144
QSA_MAX_EXTRA = 8
QSA_ATTN_SCRATCH_BYTES = 8 << 20

EXPORTED = ["qsa_status_string", "qsa_workspace_bytes", "qsa_build_index_keys", "qsa_index_topk",
            "qsa_sparse_gqa_decode", "qsa_sparse_gqa_prefill", "qsa_sparse_gqa_decode_fp8",
            "qsa_sparse_gqa_prefill_fp8", "qsa_build_index_keys_mrope", "qsa_decode_build_index_topk",
            "qsa_decode_build_index_topk_mrope", "qsa_sparse_gqa_decode_noalloc",
            "qsa_profile_kernel_events"]


class QsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)}")
        self.status = status


class QsaDims(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("idx_heads", ctypes.c_int32),
                ("idx_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("sm_scale", ctypes.c_float)]


def default_dims(page_size: int = 64, rope_theta: float = 1.0e7) -> QsaDims:
    return QsaDims(16, 2, 256, 4, 128, page_size, rope_theta, 1.0 / 16.0)


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_SZ = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """Load libqsa.so; raise if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libqsa.so not found at {LIB_PATH}; build it with "
                              "`python -m block_sparse_attention_c4_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.qsa_status_string.restype = ctypes.c_char_p
        L.qsa_status_string.argtypes = [ctypes.c_int]
        L.qsa_profile_kernel_events.restype = ctypes.c_int
        L.qsa_profile_kernel_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), _I]
        L.qsa_workspace_bytes.restype = _SZ
        L.qsa_workspace_bytes.argtypes = [ctypes.POINTER(QsaDims), ctypes.c_int, _I, _I, _I]
        L.qsa_build_index_keys.restype = ctypes.c_int
        L.qsa_build_index_keys.argtypes = [ctypes.POINTER(QsaDims), _I, _P, _P, _P, _I, _I, _P, _I,
                                           _P, _P, _P]
        L.qsa_index_topk.restype = ctypes.c_int
        L.qsa_index_topk.argtypes = [ctypes.POINTER(QsaDims), _I, _I, _P, _P, _P, _P, _I, _P, _I,
                                     _P, _P, _P, _I, _P, _P, _SZ, _P]
        L.qsa_sparse_gqa_decode.restype = ctypes.c_int
        L.qsa_sparse_gqa_decode.argtypes = [ctypes.POINTER(QsaDims), _I, _P, _P, _P, _P, _I, _P, _P,
                                            _I, _P, _I, _P, _P, _P, _SZ, _P]
        L.qsa_sparse_gqa_decode_noalloc.restype = ctypes.c_int
        L.qsa_sparse_gqa_decode_noalloc.argtypes = [ctypes.POINTER(QsaDims), _I, _P, _P, _P, _P, _I,
                                                    _P, _P, _I, _P, _I, _P, _P, _P]
        L.qsa_sparse_gqa_prefill.restype = ctypes.c_int
        L.qsa_sparse_gqa_prefill.argtypes = [ctypes.POINTER(QsaDims), _I, _P, _P, _P, _P, _P, _I, _P,
                                             _P, _I, _P, _P, _P, _SZ, _P]
        _F = ctypes.c_float
        L.qsa_sparse_gqa_decode_fp8.restype = ctypes.c_int
        L.qsa_sparse_gqa_decode_fp8.argtypes = [ctypes.POINTER(QsaDims), _I, _P, _P, _P, _F, _F, _P,
                                                _I, _P, _P, _I, _P, _I, _P, _P, _P, _SZ, _P]
        L.qsa_sparse_gqa_prefill_fp8.restype = ctypes.c_int
        L.qsa_sparse_gqa_prefill_fp8.argtypes = [ctypes.POINTER(QsaDims), _I, _P, _P, _P, _P, _F, _F,
                                                 _P, _I, _P, _P, _I, _P, _P, _P, _SZ, _P]
        L.qsa_build_index_keys_mrope.restype = ctypes.c_int
        L.qsa_build_index_keys_mrope.argtypes = [ctypes.POINTER(QsaDims), _I, _P, _P, _P, _P, _I, _I,
                                                 _P, _I, _P, _P, _P, _P, _P]
        L.qsa_decode_build_index_topk.restype = ctypes.c_int
        L.qsa_decode_build_index_topk.argtypes = [ctypes.POINTER(QsaDims), _I, _P, _P, _I, _P, _I, _P,
                                                  _P, _P, _P, _P, _P, _I, _P, _P, _SZ, _P]
        L.qsa_decode_build_index_topk_mrope.restype = ctypes.c_int
        L.qsa_decode_build_index_topk_mrope.argtypes = [ctypes.POINTER(QsaDims), _I, _P, _P, _P, _I, _P,
                                                        _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P,
                                                        _P, _SZ, _P]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().qsa_status_string(int(status)).decode()


def _ptr(x) -> int | None:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, torch.Tensor):
        if not x.is_contiguous():
            raise ValueError("tensors passed to libqsa must be contiguous")
        return x.data_ptr()
    raise TypeError(f"cannot pass {type(x)} as a pointer")


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status: int, where: str) -> None:
    if status != QSA_OK:
        raise QsaError(status, where)


def qsa_profile_kernel_events(events) -> None:
    """events: torch.cuda.Event objects (or raw hipEvent_t handles), a (start, stop)
    pair for each of the first len(events) / 2 kernels of the calling thread's next
    QSA call; the events must have been created (torch creates one at its first
    record)."""
    handles = [e.cuda_event if hasattr(e, "cuda_event") else int(e) for e in events]
    arr = (ctypes.c_void_p * max(len(handles), 1))(*handles)
    _check(lib().qsa_profile_kernel_events(arr, len(handles)), "qsa_profile_kernel_events")


def qsa_workspace_bytes(dims: QsaDims, op: int, total_q: int, max_pos: int = 0, n_extra: int = 0) -> int:
    return int(lib().qsa_workspace_bytes(ctypes.byref(dims), op, total_q, max_pos, n_extra))


def qsa_build_index_keys(dims, batch, new_idx_k, cu_new, len_before, total_new, max_new, page_table,
                         pt_stride, ring, comp_cache, stream=None) -> None:
    st = lib().qsa_build_index_keys(ctypes.byref(dims), batch, _ptr(new_idx_k), _ptr(cu_new),
                                    _ptr(len_before), total_new, max_new, _ptr(page_table), pt_stride,
                                    _ptr(ring), _ptr(comp_cache), _stream(stream))
    _check(st, "qsa_build_index_keys")


def qsa_index_topk(dims, batch, total_q, idx_q, idx_w, q_req, q_pos, max_pos, page_table, pt_stride,
                   comp_cache, sel_blocks, sel_pos, sel_stride, sel_count, workspace, ws_bytes,
                   stream=None) -> None:
    st = lib().qsa_index_topk(ctypes.byref(dims), batch, total_q, _ptr(idx_q), _ptr(idx_w),
                              _ptr(q_req), _ptr(q_pos), max_pos, _ptr(page_table), pt_stride,
                              _ptr(comp_cache), _ptr(sel_blocks), _ptr(sel_pos), sel_stride,
                              _ptr(sel_count), _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "qsa_index_topk")


def qsa_decode_build_index_topk(dims, batch, new_idx_k, pos, max_pos, page_table, pt_stride, ring,
                                comp_cache, idx_q, idx_w, sel_blocks, sel_pos, sel_stride, sel_count,
                                workspace, ws_bytes, stream=None) -> None:
    st = lib().qsa_decode_build_index_topk(ctypes.byref(dims), batch, _ptr(new_idx_k), _ptr(pos), max_pos,
                                           _ptr(page_table), pt_stride, _ptr(ring), _ptr(comp_cache),
                                           _ptr(idx_q), _ptr(idx_w), _ptr(sel_blocks), _ptr(sel_pos),
                                           sel_stride, _ptr(sel_count), _ptr(workspace), ws_bytes,
                                           _stream(stream))
    _check(st, "qsa_decode_build_index_topk")


def qsa_decode_build_index_topk_mrope(dims, batch, new_idx_k, new_mpos, pos, max_pos, page_table,
                                      pt_stride, pair_axis, ring, ring_mpos, comp_cache, idx_q, idx_w,
                                      sel_blocks, sel_pos, sel_stride, sel_count, workspace, ws_bytes,
                                      stream=None) -> None:
    """pair_axis: 64 host values (0 temporal, 1 height, 2 width), e.g. a numpy array."""
    axis = (ctypes.c_uint8 * 64)(*[int(v) for v in pair_axis])
    st = lib().qsa_decode_build_index_topk_mrope(
        ctypes.byref(dims), batch, _ptr(new_idx_k), _ptr(new_mpos), _ptr(pos), max_pos, _ptr(page_table),
        pt_stride, ctypes.addressof(axis), _ptr(ring), _ptr(ring_mpos), _ptr(comp_cache), _ptr(idx_q),
        _ptr(idx_w), _ptr(sel_blocks), _ptr(sel_pos), sel_stride, _ptr(sel_count), _ptr(workspace),
        ws_bytes, _stream(stream))
    _check(st, "qsa_decode_build_index_topk_mrope")


def qsa_sparse_gqa_decode(dims, batch, q, k_pool, v_pool, page_table, pt_stride, sel_pos, sel_count,
                          sel_stride, extra_pos, n_extra, out, lse, workspace, ws_bytes,
                          stream=None) -> None:
    st = lib().qsa_sparse_gqa_decode(ctypes.byref(dims), batch, _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                     _ptr(page_table), pt_stride, _ptr(sel_pos), _ptr(sel_count),
                                     sel_stride, _ptr(extra_pos), n_extra, _ptr(out), _ptr(lse),
                                     _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "qsa_sparse_gqa_decode")


def qsa_sparse_gqa_decode_noalloc(dims, batch, q, k_pool, v_pool, page_table, pt_stride, sel_pos,
                                  sel_count, sel_stride, extra_pos, n_extra, out, lse,
                                  stream=None) -> None:
    st = lib().qsa_sparse_gqa_decode_noalloc(ctypes.byref(dims), batch, _ptr(q), _ptr(k_pool),
                                             _ptr(v_pool), _ptr(page_table), pt_stride, _ptr(sel_pos),
                                             _ptr(sel_count), sel_stride, _ptr(extra_pos), n_extra,
                                             _ptr(out), _ptr(lse), _stream(stream))
    _check(st, "qsa_sparse_gqa_decode_noalloc")


def qsa_sparse_gqa_prefill(dims, total_q, q, q_req, k_pool, v_pool, page_table, pt_stride, sel_pos,
                           sel_count, sel_stride, out, lse, workspace, ws_bytes, stream=None) -> None:
    st = lib().qsa_sparse_gqa_prefill(ctypes.byref(dims), total_q, _ptr(q), _ptr(q_req), _ptr(k_pool),
                                      _ptr(v_pool), _ptr(page_table), pt_stride, _ptr(sel_pos),
                                      _ptr(sel_count), sel_stride, _ptr(out), _ptr(lse),
                                      _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "qsa_sparse_gqa_prefill")


def qsa_sparse_gqa_decode_fp8(dims, batch, q, k_pool, v_pool, k_scale, v_scale, page_table, pt_stride,
                              sel_pos, sel_count, sel_stride, extra_pos, n_extra, out, lse, workspace,
                              ws_bytes, stream=None) -> None:
    st = lib().qsa_sparse_gqa_decode_fp8(ctypes.byref(dims), batch, _ptr(q), _ptr(k_pool),
                                         _ptr(v_pool), float(k_scale), float(v_scale),
                                         _ptr(page_table), pt_stride, _ptr(sel_pos), _ptr(sel_count),
                                         sel_stride, _ptr(extra_pos), n_extra, _ptr(out), _ptr(lse),
                                         _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "qsa_sparse_gqa_decode_fp8")


def qsa_sparse_gqa_prefill_fp8(dims, total_q, q, q_req, k_pool, v_pool, k_scale, v_scale, page_table,
                               pt_stride, sel_pos, sel_count, sel_stride, out, lse, workspace,
                               ws_bytes, stream=None) -> None:
    st = lib().qsa_sparse_gqa_prefill_fp8(ctypes.byref(dims), total_q, _ptr(q), _ptr(q_req),
                                          _ptr(k_pool), _ptr(v_pool), float(k_scale), float(v_scale),
                                          _ptr(page_table), pt_stride, _ptr(sel_pos),
                                          _ptr(sel_count), sel_stride, _ptr(out), _ptr(lse),
                                          _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "qsa_sparse_gqa_prefill_fp8")


def qsa_build_index_keys_mrope(dims, batch, new_idx_k, new_mpos, cu_new, len_before, total_new,
                               max_new, page_table, pt_stride, pair_axis, ring, ring_mpos, comp_cache,
                               stream=None) -> None:
    """pair_axis: 64 host values (0 temporal, 1 height, 2 width), e.g. a numpy array."""
    axis = (ctypes.c_uint8 * 64)(*[int(v) for v in pair_axis])
    st = lib().qsa_build_index_keys_mrope(ctypes.byref(dims), batch, _ptr(new_idx_k), _ptr(new_mpos),
                                          _ptr(cu_new), _ptr(len_before), total_new, max_new,
                                          _ptr(page_table), pt_stride, ctypes.addressof(axis),
                                          _ptr(ring), _ptr(ring_mpos), _ptr(comp_cache),
                                          _stream(stream))
    _check(st, "qsa_build_index_keys_mrope")
