"""Host-side checks of libqsa.so that need no GPU: it loads, exports every
function include/qsa.h declares, and rejects bad arguments with the documented
status before anything is launched."""

import ctypes
import os
import re

import pytest

from block_sparse_attention_c4_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qsa.h")
FAKE = 0x10000   # a non-NULL, 256-byte aligned address that is never dereferenced


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(qsa_\w+)\s*\(", text, re.M)))


def test_header_functions_are_exported():
    names = declared()
    assert set(names) == set(B.EXPORTED), names
    L = B.lib()
    for n in names:
        assert getattr(L, n) is not None


def test_header_is_plain_c_and_cxx(tmp_path):
    # the ABI header is for C callers: it must compile as strict C99 and as C++17
    import shutil
    import subprocess
    src = tmp_path / "use_qsa.c"
    src.write_text('#include "qsa.h"\n'
                   "int main(void) {\n"
                   "  qsa_dims d = {16, 2, 256, 4, 128, 64, 1.0e7f, 0.0625f};\n"
                   "  return (int)qsa_workspace_bytes(&d, QSA_OP_INDEX_TOPK, 1, 4096, 0) & 0;\n"
                   "}\n")
    inc = os.path.dirname(HEADER)
    for cc, std, lang in (("gcc", "-std=c99", "c"), ("g++", "-std=c++17", "c++")):
        if shutil.which(cc) is None:
            continue
        r = subprocess.run([cc, std, "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                            "-x", lang, "-I", inc, str(src)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_status_strings():
    for st in range(7):
        assert B.status_string(st).startswith("QSA_")
    assert "unknown" in B.status_string(99)


def test_workspace_sizes():
    d = B.default_dims()
    a = B.qsa_workspace_bytes(d, B.QSA_OP_INDEX_TOPK, 32, 131072)
    b = B.qsa_workspace_bytes(d, B.QSA_OP_INDEX_TOPK, 32, 262144)
    assert 0 < a < b and a % 256 == 0
    assert B.qsa_workspace_bytes(d, B.QSA_OP_INDEX_TOPK, 32, 262145) == 0
    assert B.qsa_workspace_bytes(d, B.QSA_OP_GQA_DECODE, 32, 0, 9) == 0
    assert B.qsa_workspace_bytes(d, B.QSA_OP_GQA_DECODE, 32, 0, 4) > 0
    assert B.qsa_workspace_bytes(d, 99, 32, 1) == 0
    bad = B.default_dims()
    bad.num_q_heads = 32
    assert B.qsa_workspace_bytes(bad, B.QSA_OP_INDEX_TOPK, 32, 4096) == 0


def _topk(dims=None, **kw):
    d = dims or B.default_dims()
    args = dict(batch=1, total_q=1, idx_q=FAKE, idx_w=FAKE, q_req=FAKE, q_pos=FAKE, max_pos=4096,
                page_table=FAKE, pt_stride=64, comp=FAKE, sel_blocks=FAKE, sel_pos=FAKE, sel_stride=2052,
                sel_count=FAKE, ws=FAKE, ws_bytes=1 << 30)
    args.update(kw)
    a = args
    return B.lib().qsa_index_topk(ctypes.byref(d), a["batch"], a["total_q"], a["idx_q"], a["idx_w"],
                                  a["q_req"], a["q_pos"], a["max_pos"], a["page_table"], a["pt_stride"],
                                  a["comp"], a["sel_blocks"], a["sel_pos"], a["sel_stride"],
                                  a["sel_count"], a["ws"], a["ws_bytes"], None)


def test_index_topk_validation():
    assert _topk(total_q=0) == B.QSA_OK                        # nothing to do, nothing launched
    assert _topk(idx_q=None) == B.QSA_E_NULL
    assert _topk(sel_count=None) == B.QSA_E_NULL
    assert _topk(sel_stride=2050) == B.QSA_E_SHAPE
    assert _topk(sel_stride=2053) == B.QSA_E_SHAPE            # rows of 4-position groups
    assert _topk(sel_pos=FAKE + 4) == B.QSA_E_SHAPE
    assert _topk(max_pos=262145) == B.QSA_E_SHAPE
    assert _topk(max_pos=0) == B.QSA_E_SHAPE
    assert _topk(idx_q=FAKE + 2) == B.QSA_E_SHAPE             # misaligned bf16 rows
    assert _topk(ws=None) == B.QSA_E_WORKSPACE
    assert _topk(ws_bytes=16) == B.QSA_E_WORKSPACE
    assert _topk(ws=FAKE + 16) == B.QSA_E_WORKSPACE           # not 256-byte aligned
    bad = B.default_dims()
    bad.idx_dim = 64
    assert _topk(dims=bad) == B.QSA_E_UNSUPPORTED
    bad = B.default_dims()
    bad.page_size = 24
    assert _topk(dims=bad) == B.QSA_E_UNSUPPORTED
    assert B.lib().qsa_index_topk(None, 1, 1, *([None] * 4), 10, None, 1, None, None, None, 2052,
                                  None, None, 0, None) == B.QSA_E_NULL


def _fused(dims=None, **kw):
    d = dims or B.default_dims()
    a = dict(batch=2, new=FAKE, pos=FAKE, max_pos=4096, page_table=FAKE, pt_stride=64, ring=FAKE,
             comp=FAKE, idx_q=FAKE, idx_w=FAKE, sel_blocks=FAKE, sel_pos=FAKE, sel_stride=2052,
             sel_count=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return B.lib().qsa_decode_build_index_topk(
        ctypes.byref(d), a["batch"], a["new"], a["pos"], a["max_pos"], a["page_table"], a["pt_stride"],
        a["ring"], a["comp"], a["idx_q"], a["idx_w"], a["sel_blocks"], a["sel_pos"], a["sel_stride"],
        a["sel_count"], a["ws"], a["ws_bytes"], None)


def test_decode_build_index_topk_validation():
    assert _fused(batch=0) == B.QSA_E_SHAPE
    assert _fused(batch=65536) == B.QSA_E_SHAPE
    assert _fused(max_pos=0) == B.QSA_E_SHAPE
    assert _fused(max_pos=262145) == B.QSA_E_SHAPE
    assert _fused(pt_stride=0) == B.QSA_E_SHAPE
    assert _fused(sel_stride=2050) == B.QSA_E_SHAPE
    assert _fused(sel_stride=2054) == B.QSA_E_SHAPE
    for k in ("new", "pos", "page_table", "ring", "comp", "idx_q", "idx_w", "sel_blocks", "sel_pos",
              "sel_count"):
        assert _fused(**{k: None}) == B.QSA_E_NULL, k
    assert _fused(new=FAKE + 4) == B.QSA_E_SHAPE               # raw keys read 8 bytes at a time
    assert _fused(ring=FAKE + 4) == B.QSA_E_SHAPE
    assert _fused(comp=FAKE + 8) == B.QSA_E_SHAPE
    assert _fused(idx_q=FAKE + 8) == B.QSA_E_SHAPE
    assert _fused(ws=None) == B.QSA_E_WORKSPACE
    assert _fused(ws_bytes=B.qsa_workspace_bytes(B.default_dims(), B.QSA_OP_INDEX_TOPK, 2, 4096) - 1) \
        == B.QSA_E_WORKSPACE
    assert _fused(ws=FAKE + 64) == B.QSA_E_WORKSPACE
    bad = B.default_dims()
    bad.idx_heads = 8
    assert _fused(dims=bad) == B.QSA_E_UNSUPPORTED


def test_decode_build_index_topk_mrope_validation():
    d = B.default_dims()
    L = B.lib()
    axis = (ctypes.c_uint8 * 64)(*([0] * 64))
    bad_axis = (ctypes.c_uint8 * 64)(*([0] * 63 + [3]))

    def call(new_mpos=FAKE, axis_ptr=ctypes.addressof(axis), ring_mpos=FAKE, new=FAKE, batch=2):
        return L.qsa_decode_build_index_topk_mrope(
            ctypes.byref(d), batch, new, new_mpos, FAKE, 4096, FAKE, 64, axis_ptr, FAKE, ring_mpos, FAKE,
            FAKE, FAKE, FAKE, FAKE, 2052, FAKE, FAKE, 1 << 30, None)
    assert call(new_mpos=None) == B.QSA_E_NULL
    assert call(axis_ptr=None) == B.QSA_E_NULL
    assert call(ring_mpos=None) == B.QSA_E_NULL
    assert call(axis_ptr=ctypes.addressof(bad_axis)) == B.QSA_E_SHAPE
    assert call(new_mpos=FAKE + 2) == B.QSA_E_SHAPE
    assert call(new=None) == B.QSA_E_NULL
    assert call(batch=0) == B.QSA_E_SHAPE


def test_build_validation():
    d = B.default_dims()
    L = B.lib()
    call = lambda **k: L.qsa_build_index_keys(
        ctypes.byref(k.get("d", d)), k.get("batch", 2), k.get("new", FAKE), FAKE, FAKE,
        k.get("total", 8), k.get("maxn", 4), FAKE, k.get("pts", 16), FAKE, k.get("comp", FAKE), None)
    assert call(total=0, maxn=0) == B.QSA_OK
    assert call(new=None) == B.QSA_E_NULL
    assert call(comp=None) == B.QSA_E_NULL
    assert call(maxn=9) == B.QSA_E_SHAPE                      # max_new > total_new
    assert call(pts=0) == B.QSA_E_SHAPE
    assert call(batch=-1) == B.QSA_E_SHAPE
    assert call(new=FAKE + 2) == B.QSA_E_SHAPE
    bad = B.default_dims()
    bad.num_kv_heads = 4
    assert call(d=bad) == B.QSA_E_UNSUPPORTED


def test_gqa_validation():
    d = B.default_dims()
    L = B.lib()
    ws = B.qsa_workspace_bytes(d, B.QSA_OP_GQA_DECODE, 8, 0, 4)

    def dec(**k):
        return L.qsa_sparse_gqa_decode(ctypes.byref(d), k.get("batch", 8), k.get("q", FAKE), FAKE, FAKE,
                                       FAKE, 64, FAKE, FAKE, 2052, k.get("extra", FAKE), k.get("n_extra", 4),
                                       k.get("out", FAKE), None, k.get("ws", FAKE), k.get("ws_bytes", ws), None)
    assert dec(batch=0) == B.QSA_OK
    assert dec(q=None) == B.QSA_E_NULL
    assert dec(out=None) == B.QSA_E_NULL
    assert dec(extra=None) == B.QSA_E_NULL                     # n_extra > 0 needs the array
    assert dec(n_extra=9) == B.QSA_E_SHAPE
    assert dec(n_extra=-1) == B.QSA_E_SHAPE
    assert dec(ws_bytes=ws - 1) == B.QSA_E_WORKSPACE
    assert dec(q=FAKE + 8) == B.QSA_E_SHAPE
    assert L.qsa_sparse_gqa_prefill(ctypes.byref(d), 4, FAKE, None, FAKE, FAKE, FAKE, 64, FAKE, FAKE,
                                    2052, FAKE, None, None, 0, None) == B.QSA_E_NULL   # q_req missing


def test_gqa_noalloc_validation():
    # the allocation-free decode call checks its arguments as the workspace call does,
    # before it looks up its static scratch (which needs a GPU)
    d = B.default_dims()
    L = B.lib()

    def dec(**k):
        return L.qsa_sparse_gqa_decode_noalloc(ctypes.byref(d), k.get("batch", 8), k.get("q", FAKE), FAKE,
                                               FAKE, FAKE, 64, FAKE, FAKE, 2052, k.get("extra", FAKE),
                                               k.get("n_extra", 4), k.get("out", FAKE), None, None)
    assert dec(batch=0) == B.QSA_OK
    assert dec(q=None) == B.QSA_E_NULL
    assert dec(out=None) == B.QSA_E_NULL
    assert dec(extra=None) == B.QSA_E_NULL
    assert dec(n_extra=9) == B.QSA_E_SHAPE
    assert dec(q=FAKE + 8) == B.QSA_E_SHAPE
    bad = B.default_dims()
    bad.head_dim = 128
    assert L.qsa_sparse_gqa_decode_noalloc(ctypes.byref(bad), 8, FAKE, FAKE, FAKE, FAKE, 64, FAKE, FAKE,
                                           2052, None, 0, FAKE, None, None) == B.QSA_E_UNSUPPORTED
    # every batch size's split partials fit the static scratch
    need = max(B.qsa_workspace_bytes(d, B.QSA_OP_GQA_DECODE, b, 0, e)
               for b in range(1, 300) for e in (0, 4, 8))
    assert 0 < need <= B.QSA_ATTN_SCRATCH_BYTES


def test_profile_kernel_events_validation():
    L = B.lib()
    ev = (ctypes.c_void_p * 18)(*([FAKE] * 18))
    assert L.qsa_profile_kernel_events(ev, 18) == B.QSA_E_SHAPE     # at most 8 kernels
    assert L.qsa_profile_kernel_events(ev, 3) == B.QSA_E_SHAPE      # (start, stop) pairs
    assert L.qsa_profile_kernel_events(ev, -2) == B.QSA_E_SHAPE
    assert L.qsa_profile_kernel_events(None, 2) == B.QSA_E_NULL
    ev[1] = None
    assert L.qsa_profile_kernel_events(ev, 2) == B.QSA_E_NULL
    assert L.qsa_profile_kernel_events(None, 0) == B.QSA_OK        # cancels
    # a request lapses with the next call, even one that fails validation and launches
    # nothing (otherwise a later call would set events the caller dropped)
    ev[1] = FAKE
    assert L.qsa_profile_kernel_events(ev, 2) == B.QSA_OK
    d = B.default_dims()
    assert L.qsa_sparse_gqa_decode(ctypes.byref(d), 8, None, FAKE, FAKE, FAKE, 64, FAKE, FAKE, 2052,
                                   None, 0, FAKE, None, FAKE, 1 << 30, None) == B.QSA_E_NULL


def test_gqa_fp8_validation():
    d = B.default_dims()
    L = B.lib()
    ws = B.qsa_workspace_bytes(d, B.QSA_OP_GQA_DECODE, 8, 0, 0)

    def dec(**k):
        return L.qsa_sparse_gqa_decode_fp8(ctypes.byref(d), k.get("batch", 8), FAKE, k.get("k", FAKE),
                                           k.get("v", FAKE), k.get("ks", 0.01), k.get("vs", 0.02), FAKE, 64,
                                           FAKE, FAKE, 2052, None, 0, FAKE, None, FAKE, ws, None)
    assert dec(batch=0) == B.QSA_OK
    assert dec(k=None) == B.QSA_E_NULL
    assert dec(v=None) == B.QSA_E_NULL
    assert dec(k=FAKE + 8) == B.QSA_E_SHAPE                     # 16-byte aligned code rows
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert dec(ks=bad) == B.QSA_E_SHAPE
        assert dec(vs=bad) == B.QSA_E_SHAPE
    assert L.qsa_sparse_gqa_prefill_fp8(ctypes.byref(d), 4, FAKE, None, FAKE, FAKE, 1.0, 1.0, FAKE, 64,
                                        FAKE, FAKE, 2052, FAKE, None, None, 0, None) == B.QSA_E_NULL


def test_build_mrope_validation():
    d = B.default_dims()
    L = B.lib()
    contiguous = (ctypes.c_uint8 * 64)(*([0] * 16 + [1] * 24 + [2] * 24))

    def build(axis=contiguous, **k):
        return L.qsa_build_index_keys_mrope(ctypes.byref(d), k.get("batch", 2), FAKE, k.get("mpos", FAKE),
                                            FAKE, FAKE, k.get("total", 8), min(4, k.get("total", 8)), FAKE, 64,
                                            None if axis is None else ctypes.addressof(axis), FAKE,
                                            k.get("ring_mpos", FAKE), FAKE, None)
    assert build(total=0) == B.QSA_OK
    assert build(axis=None) == B.QSA_E_NULL
    assert build(mpos=None) == B.QSA_E_NULL
    assert build(ring_mpos=None) == B.QSA_E_NULL
    assert build(mpos=FAKE + 2) == B.QSA_E_SHAPE                # int32 positions
    bad = (ctypes.c_uint8 * 64)(*([0] * 63 + [3]))
    assert build(axis=bad) == B.QSA_E_SHAPE                      # only t, h, w


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", "/nonexistent/libqsa.so")
    with pytest.raises(ImportError):
        B.lib()
