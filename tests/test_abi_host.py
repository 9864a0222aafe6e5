"""Host-side checks of the C ABI: the library loads, exports every declared entry
point, sizes workspaces, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

from box_decoding_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "la_pbd.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:la_status|size_t|const char\*)\s+(la_\w+)\(", src, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(b.library_path()):
        from box_decoding_amd import build
        build.build()
    return b.load()


def test_header_declares_the_named_entry_points():
    names = _declared()
    for n in ("la_pbd_step", "la_pbd_attention", "la_wgemm", "la_int4_embed_gather",
              "la_lm_head_argmax"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in _declared():
        assert hasattr(lib, n), n
    assert sorted(b.EXPORTED) == _declared()


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5):
        s = lib.la_status_str(code).decode()
        assert s and s != "unknown status"
    assert lib.la_status_str(7).decode() == "unknown status"


def _w(fmt=0, n=2560, k=2048, group=0, data=256, scales=None, layout=0):
    return b.LaWeight(fmt=fmt, n=n, k=k, group=group, layout=layout, data=ctypes.c_void_p(data),
                      scales=ctypes.c_void_p(scales) if scales else None)


def test_wgemm_rejects_bad_arguments_before_launch(lib):
    w = _w()
    ws = lib.la_wgemm_workspace(6, ctypes.byref(w), 0)
    assert ws > 0
    fake = ctypes.c_void_p(4096)
    # NULL x / y
    assert lib.la_wgemm(None, 6, ctypes.byref(w), None, 1e-6, None, None, 0, fake, fake, ws, None) == -1
    # bad epilogue
    assert lib.la_wgemm(fake, 6, ctypes.byref(w), None, 1e-6, None, None, 9, fake, fake, ws, None) == -1
    # M out of range
    assert lib.la_wgemm(fake, 0, ctypes.byref(w), None, 1e-6, None, None, 0, fake, fake, ws, None) == -2
    # K not a multiple of 256
    w2 = _w(k=2000)
    assert lib.la_wgemm(fake, 6, ctypes.byref(w2), None, 1e-6, None, None, 0, fake, fake, ws, None) == -2
    # INT4 without scales / with a wrong group
    w3 = _w(fmt=1, group=128)
    assert lib.la_wgemm(fake, 6, ctypes.byref(w3), None, 1e-6, None, None, 0, fake, fake, ws, None) == -2
    w4 = _w(fmt=1, group=64, scales=4096)
    assert lib.la_wgemm(fake, 6, ctypes.byref(w4), None, 1e-6, None, None, 0, fake, fake, ws, None) == -2
    # misaligned activations
    assert lib.la_wgemm(ctypes.c_void_p(4100), 6, ctypes.byref(w), None, 1e-6, None, None, 0, fake,
                        fake, ws, None) == -1
    # workspace too small / missing
    assert lib.la_wgemm(fake, 6, ctypes.byref(w), None, 1e-6, None, None, 0, fake, fake, ws - 1,
                        None) == -3
    assert lib.la_wgemm(fake, 6, ctypes.byref(w), None, 1e-6, None, None, 0, fake, None, ws, None) == -3


def test_attention_rejects_bad_shapes(lib):
    kv = b.LaKvCache(ctypes.c_void_p(4096), ctypes.c_void_p(8192), ctypes.c_void_p(256), 10, 4, 16, 1)
    fake = ctypes.c_void_p(4096)
    ws = lib.la_pbd_attention_workspace(1, 6, 16, 2, 128, 64)
    assert ws > 0
    call = lambda **k: lib.la_pbd_attention(
        fake, ctypes.byref(k.get("kv", kv)), k.get("layer", 0), k.get("hq", 16), k.get("hkv", 2),
        k.get("d", 128), fake, k.get("B", 1), k.get("W", 6), k.get("max_len", 64), fake, fake,
        k.get("ws", ws), None)
    assert call(d=64) == -2
    assert call(hq=15) == -2
    assert call(W=17) == -2
    assert call(hq=32, W=9) == -2   # 9 rows x 16 query heads per KV head > 128 columns
    assert call(B=65) == -2
    assert call(layer=1) == -1
    assert call(ws=ws - 1) == -3
    bad = b.LaKvCache(ctypes.c_void_p(4096), ctypes.c_void_p(8192), ctypes.c_void_p(256), 10, 4, 32, 1)
    assert call(kv=bad) == -2


def test_step_workspace_rejects_bad_model(lib):
    m = b.LaModel()
    assert lib.la_pbd_step_workspace(ctypes.byref(m), 1, 6, 64) == 0


def test_lm_head_rejects(lib):
    w = _w(n=152681)
    ws = lib.la_lm_head_argmax_workspace(6, ctypes.byref(w))
    assert ws >= 16 * 2048 * 2  # at least the packed operand of one row tile
    fake = ctypes.c_void_p(4096)
    assert lib.la_lm_head_argmax(None, 6, ctypes.byref(w), None, 1e-6, fake, None, None, fake, ws,
                                 None) == -1
    assert lib.la_lm_head_argmax(fake, 6, ctypes.byref(w), None, 1e-6, fake, None, None, fake, ws - 1,
                                 None) == -3


def test_gather_rejects(lib):
    fake = ctypes.c_void_p(4096)
    e = _w(fmt=1, n=100, k=2048, group=32)  # INT4 without scales
    assert lib.la_int4_embed_gather(fake, 6, ctypes.byref(e), fake, None, None) == -2
    e2 = _w(fmt=3, n=100, k=2048)
    assert lib.la_int4_embed_gather(fake, 6, ctypes.byref(e2), fake, None, None) == -1
    e3 = _w(n=100, k=2048)
    assert lib.la_int4_embed_gather(fake, 0, ctypes.byref(e3), fake, None, None) == 0  # empty: no-op


def test_pack_rows_and_packed_gemm_reject_bad_arguments(lib):
    fake = ctypes.c_void_p(4096)
    need = lib.la_packed_rows_bytes(6, 2048)
    assert need > 0 and lib.la_packed_rows_bytes(6, 2000) == 0 and lib.la_packed_rows_bytes(0, 2048) == 0
    # bad format, K, alignment, too small a buffer
    assert lib.la_pack_rows(fake, 6, 2048, None, 1e-6, 7, fake, need, None) == -1
    assert lib.la_pack_rows(fake, 6, 2000, None, 1e-6, 0, fake, need, None) == -2
    assert lib.la_pack_rows(ctypes.c_void_p(4100), 6, 2048, None, 1e-6, 0, fake, need, None) == -1
    assert lib.la_pack_rows(fake, 6, 2048, None, 1e-6, 0, fake, need - 1, None) == -3
    # a gain with a non-positive epsilon
    assert lib.la_pack_rows(fake, 6, 2048, fake, 0.0, 0, fake, need, None) == -1
    w = _w(layout=1)
    assert lib.la_wgemm_packed(None, 6, ctypes.byref(w), None, None, 0, fake, None) == -1
    assert lib.la_wgemm_packed(fake, 6, ctypes.byref(w), None, None, 5, fake, None) == -1
    assert lib.la_wgemm_packed(fake, 0, ctypes.byref(w), None, None, 0, fake, None) == -2
    # SiLU gating needs the gate/up layout and takes no bias or residual
    wg = _w(n=2 * 1024, layout=2)
    assert lib.la_wgemm_packed(fake, 6, ctypes.byref(wg), fake, None, 1, fake, None) == -2


def test_commit_rejects_bad_arguments_before_launch(lib):
    a, b_ = ctypes.c_void_p(4096), ctypes.c_void_p(8192)
    p = ctypes.c_void_p(12288)
    assert lib.la_pbd_commit(None, b_, p, 2, 6, 7, None) == -1
    assert lib.la_pbd_commit(a, None, p, 2, 6, 7, None) == -1
    assert lib.la_pbd_commit(a, b_, None, 2, 6, 7, None) == -1
    assert lib.la_pbd_commit(a, a, p, 2, 6, 7, None) == -1     # ids aliased
    assert lib.la_pbd_commit(a, b_, p, 0, 6, 7, None) == -2
    assert lib.la_pbd_commit(a, b_, p, 65, 6, 7, None) == -2
    assert lib.la_pbd_commit(a, b_, p, 2, 0, 7, None) == -2
    assert lib.la_pbd_commit(a, b_, p, 2, 17, 7, None) == -2


def test_repetition_penalty_entry_points_reject_bad_arguments(lib):
    a = ctypes.c_void_p(4096)
    w = b.LaWeight(fmt=0, n=1000, k=2048, group=0, layout=1, data=a)
    ws = lib.la_lm_head_argmax_workspace(6, ctypes.byref(w))
    pen = lambda bits, words=32, rows=6, theta=1.1: lib.la_lm_head_argmax_penalized(
        a, 6, ctypes.byref(w), None, 1e-6, bits, words, rows, theta, a, None, None, a, ws, None)
    assert pen(a, words=31) == -1           # 31 words hold 992 < 1000 ids
    assert pen(a, rows=0) == -1
    assert pen(a, theta=0.0) == -1
    assert pen(a, theta=float("inf")) == -1
    mark = lambda *x: lib.la_pbd_mark_tokens(*x)
    assert mark(None, 2, 6, None, None, a, 32, 1000, None) == -1
    assert mark(a, 2, 6, None, None, None, 32, 1000, None) == -1
    assert mark(a, 0, 6, None, None, a, 32, 1000, None) == -2
    assert mark(a, 2, 17, None, None, a, 32, 1000, None) == -2
    assert mark(a, 2, 6, None, None, a, 31, 1000, None) == -2
    assert mark(a, 2, 6, None, None, a, 32, 0, None) == -2


def test_prefill_workspace_rejects_bad_shapes(lib):
    m = b.LaModel()
    assert lib.la_pbd_prefill_workspace(ctypes.byref(m), 1, 16, 64) == 0   # no layers: bad model


def test_refeed_entry_points_reject_bad_arguments_before_launch(lib):
    a, w_ = ctypes.c_void_p(4096), ctypes.c_void_p(8192)
    p, c, l, n = ctypes.c_void_p(12288), ctypes.c_void_p(16384), ctypes.c_void_p(20480), ctypes.c_void_p(24576)
    ok = lambda *x: lib.la_pbd_commit_refeed(*x)
    assert ok(None, n, w_, p, c, l, 2, 11, 6, 7, None) == -1
    assert ok(a, n, w_, p, None, l, 2, 11, 6, 7, None) == -1
    assert ok(a, n, w_, p, c, None, 2, 11, 6, 7, None) == -1
    assert ok(a, n, a, p, c, l, 2, 11, 6, 7, None) == -1     # out_ids is the window
    assert ok(a, c, w_, p, c, l, 2, 11, 6, 7, None) == -1    # n_accept is causal_rows
    assert ok(a, n, w_, p, c, l, 0, 11, 6, 7, None) == -2
    assert ok(a, n, w_, p, c, l, 2, 17, 6, 7, None) == -2
    assert ok(a, n, w_, p, c, l, 2, 11, 12, 7, None) == -2   # block wider than the window
    assert ok(a, n, w_, p, c, l, 2, 11, 0, 7, None) == -2
    kv = b.LaKvCache(ctypes.c_void_p(4096), ctypes.c_void_p(8192), ctypes.c_void_p(256), 10, 4, 16, 1)
    ws = lib.la_pbd_attention_workspace(1, 11, 16, 2, 128, 64)
    att = lambda cr, wl, W=11: lib.la_pbd_attention_refeed(
        a, ctypes.byref(kv), 0, 16, 2, 128, p, cr, wl, 1, W, 64, a, a, ws, None)
    assert att(None, l) == -1
    assert att(c, None) == -1
    assert att(c, l, W=17) == -2
