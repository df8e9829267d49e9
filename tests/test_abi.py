"""C ABI checks that need no GPU: the library loads, exports every function the header
declares, and rejects invalid host-visible arguments before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oscar.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(oscar_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from int2_rotated_kv_rotate_amd import ops
    return ops.load_library()


def test_header_declares_expected_entry_points():
    from int2_rotated_kv_rotate_amd import ops
    assert _declared_functions() == sorted(ops.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(5):
        assert lib.oscar_status_string(code)
    assert lib.oscar_status_string(99) == b"unknown status"


def test_workspace_size(lib):
    from int2_rotated_kv_rotate_amd import ops
    # Q blocks, partial outputs and (m, l) per slot, then the work plan (4 header words,
    # three words per sequence, one per (sequence, head)) rounded up to 256 bytes
    plan = (4 * (4 + 3 * 64 + 64 * 32) + 255) // 256 * 256
    # per (sequence, query head): the query block, then max_splits INT2 slots and the window
    # slots of 512 + 8 bytes each
    assert ops.WINDOW_SLOTS == 8
    assert ops.decode_workspace_bytes(64, 32, 12) == \
        64 * 32 * 1024 + 64 * 32 * (12 + ops.WINDOW_SLOTS) * (512 + 8) + plan
    assert lib.oscar_decode_workspace_bytes(-1, 32, 12) == 0
    assert lib.oscar_decode_workspace_bytes(1, 32, 0) == 0


def _layout(**kw):
    from int2_rotated_kv_rotate_amd import ops
    d = dict(num_kv_heads=8, num_sink=4, window=128, num_pages=100, max_pages_per_seq=10,
             num_slots=2)
    d.update(kw)
    return ops.make_layout(**d)


FAKE = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation first


def _append(lib, lay, **kw):
    a = dict(pages=FAKE, sinkwin=FAKE, bt=FAKE, slots=None, batch=1, total=1, k=FAKE, v=FAKE,
             off=FAKE, start=FAKE, rk=FAKE, rv=FAKE, ck=0.95, cv=0.95)
    a.update(kw)
    return lib.oscar_rotate_quantize_append(
        ctypes.byref(lay) if lay is not None else None, a["pages"], a["sinkwin"], a["bt"],
        a["slots"], a["batch"], a["total"], a["k"], a["v"], a["off"], a["start"], a["rk"],
        a["rv"], a["ck"], a["cv"], None)


def test_append_validation(lib):
    assert _append(lib, None) == 1
    assert _append(lib, _layout(head_dim=64)) == 2
    assert _append(lib, _layout(page_size=32)) == 2
    assert _append(lib, _layout(group_size=64)) == 2
    assert _append(lib, _layout(num_sink=100, window=157)) == 2
    assert _append(lib, _layout(window=-1)) == 1
    assert _append(lib, _layout(), ck=0.0) == 1
    assert _append(lib, _layout(), cv=1.5) == 1
    assert _append(lib, _layout(), pages=None) == 1
    assert _append(lib, _layout(), sinkwin=None) == 1
    assert _append(lib, _layout(), k=ctypes.c_void_p(18)) == 1   # misaligned
    assert _append(lib, _layout(), batch=-1) == 1
    assert _append(lib, _layout(), batch=0) == 0                 # nothing to do, no launch
    assert _append(lib, _layout(), total=0) == 0


def test_append_ex_validation(lib):
    lay = _layout()

    def call(method, **kw):
        a = dict(pages=FAKE, batch=1)
        a.update(kw)
        return lib.oscar_rotate_quantize_append_ex(
            ctypes.byref(lay), a["pages"], FAKE, FAKE, None, a["batch"], 1, FAKE, FAKE, FAKE, FAKE,
            FAKE, FAKE, a.get("k_mean"), 0.95, 0.95, method, None)

    assert call(3) == 1
    assert call(-1) == 1
    assert call(0, k_mean=ctypes.c_void_p(18)) == 1   # a misaligned key mean
    for m in (0, 1, 2):
        assert call(m, pages=None) == 1       # every method validates before launching
        assert call(m, batch=0) == 0          # nothing to do


def test_append_hadamard_validation(lib):
    lay = _layout()

    def call(**kw):
        a = dict(pages=FAKE, batch=1, k_new=FAKE, clip_k=0.95, sinkwin=FAKE)
        a.update(kw)
        return lib.oscar_rotate_quantize_append_hadamard(
            ctypes.byref(lay), a["pages"], a["sinkwin"], FAKE, None, a["batch"], 1, a["k_new"], FAKE,
            FAKE, FAKE, None, None, a["clip_k"], 0.95, None)

    assert call(pages=None) == 1
    assert call(k_new=None) == 1
    assert call(k_new=ctypes.c_void_p(24)) == 1    # rows must be 16-byte aligned
    assert call(clip_k=0.0) == 1
    assert call(clip_k=1.5) == 1
    assert call(sinkwin=None) == 1                 # the layout has sink/window rows
    assert call(batch=0) == 0
    assert call(batch=-1) == 1


def _decode(lib, lay, **kw):
    a = dict(pages=FAKE, sinkwin=FAKE, bt=FAKE, slots=None, batch=1, hq=32, q=FAKE, lens=FAKE,
             rk=FAKE, sm=0.088, nw=0, ms=4, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.oscar_decode_attention(
        ctypes.byref(lay), a["pages"], a["sinkwin"], a["bt"], a["slots"], a["batch"], a["hq"],
        a["q"], a["lens"], a["rk"], a["sm"], a["nw"], a["ms"], a["ws"], a["wsb"], None)


def test_decode_validation(lib):
    assert _decode(lib, _layout(), hq=30) == 1          # not a multiple of Hkv
    assert _decode(lib, _layout(), hq=24) == 2          # group 3 unsupported
    assert _decode(lib, _layout(), hq=128) == 2         # group 16 unsupported
    assert _decode(lib, _layout(), nw=-1) == 1
    assert _decode(lib, _layout(), nw=(1 << 20) + 1) == 1
    assert _decode(lib, _layout(max_pages_per_seq=1 << 20), batch=1 << 10) == 2  # plan > int32
    assert _decode(lib, _layout(), ms=0) == 1
    for bad in (float("nan"), float("inf"), -float("inf"), 0.0, -0.0, -0.088):
        assert _decode(lib, _layout(), sm=bad) == 1     # the scale must be finite and > 0
    assert _decode(lib, _layout(), wsb=100) == 3
    assert _decode(lib, _layout(), q=None) == 1
    assert _decode(lib, _layout(head_dim=256)) == 2
    assert _decode(lib, _layout(), batch=0) == 0


def test_combine_and_bf16_validation(lib):
    assert lib.oscar_combine(1, 32, 8, 4, FAKE, 100, None, FAKE, None, None) == 3
    assert lib.oscar_combine(1, 32, 8, 4, None, 1 << 30, None, FAKE, None, None) == 1
    assert lib.oscar_combine(1, 33, 8, 4, FAKE, 1 << 30, None, FAKE, None, None) == 1
    assert lib.oscar_combine(0, 32, 8, 4, FAKE, 1 << 30, None, FAKE, None, None) == 0
    lay = _layout()
    assert lib.oscar_bf16_append(ctypes.byref(lay), None, FAKE, 1, 1, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert lib.oscar_bf16_decode_attention(ctypes.byref(lay), FAKE, FAKE, 1, 32, FAKE, FAKE, 0.1,
                                           128, 4, FAKE, 10, None) == 3
    for bad in (float("nan"), float("inf"), 0.0, -1.0):
        assert lib.oscar_bf16_decode_attention(ctypes.byref(lay), FAKE, FAKE, 1, 32, FAKE, FAKE,
                                               bad, 128, 4, FAKE, 1 << 30, None) == 1
        assert lib.oscar_int4_decode_attention(ctypes.byref(lay), FAKE, FAKE, FAKE, None, 1, 32,
                                               FAKE, FAKE, FAKE, bad, 16, 4, FAKE, 1 << 30,
                                               None) == 1


def test_read_records_validation(lib):
    # n < 0, an empty pool, no workers, null or misaligned pointers: rejected before any
    # launch; n = 0 is a no-op
    assert lib.oscar_read_records(FAKE, 8, FAKE, -1, 4, FAKE, None) == 1
    assert lib.oscar_read_records(FAKE, 0, FAKE, 8, 4, FAKE, None) == 1
    assert lib.oscar_read_records(FAKE, 8, FAKE, 8, 0, FAKE, None) == 1
    assert lib.oscar_read_records(FAKE, 8, FAKE, 8, (1 << 20) + 1, FAKE, None) == 1
    assert lib.oscar_read_records(None, 8, FAKE, 8, 4, FAKE, None) == 1
    assert lib.oscar_read_records(FAKE, 8, None, 8, 4, FAKE, None) == 1
    assert lib.oscar_read_records(FAKE, 8, FAKE, 8, 4, None, None) == 1
    assert lib.oscar_read_records(ctypes.c_void_p(20), 8, FAKE, 8, 4, FAKE, None) == 1
    assert lib.oscar_read_records(None, 8, None, 0, 4, None, None) == 0


def test_decode_static_validation(lib):
    lay = _layout()

    def call(**kw):
        a = dict(pages=FAKE, batch=1, hq=32, out=FAKE, sm=0.088, ms=4, rv=FAKE)
        a.update(kw)
        return lib.oscar_decode_attention_static(
            ctypes.byref(lay), a["pages"], FAKE, FAKE, None, a["batch"], a["hq"], FAKE, FAKE,
            FAKE, a["rv"], a["sm"], 0, a["ms"], a["out"], None, None)

    assert call(out=None) == 1
    assert call(pages=None) == 1
    assert call(hq=24) == 2
    assert call(sm=float("inf")) == 1
    assert call(ms=0) == 1
    assert call(rv=ctypes.c_void_p(20)) == 1     # misaligned R_V
    # 64 sequences x 32 query heads x 65 slots need ~71 MB: more than the library's buffer
    assert call(batch=64, ms=64) == 3
    assert call(batch=0) == 0


def test_prepare_and_prepared_decode_validation(lib):
    lay = _layout()

    def prep(**kw):
        a = dict(batch=1, hq=32, q=FAKE, lens=FAKE, rk=FAKE, nw=0, ms=4, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.oscar_prepare_queries(ctypes.byref(lay), a["batch"], a["hq"], a["q"], a["lens"],
                                         a["rk"], a["nw"], a["ms"], a["ws"], a["wsb"], None)

    def dec(**kw):
        a = dict(pages=FAKE, sw=FAKE, bt=FAKE, batch=1, hq=32, lens=FAKE, sm=0.088, nw=0, ms=4,
                 ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.oscar_decode_attention_prepared(
            ctypes.byref(lay), a["pages"], a["sw"], a["bt"], None, a["batch"], a["hq"], a["lens"],
            a["sm"], a["nw"], a["ms"], a["ws"], a["wsb"], None)

    for f in (prep, dec):
        assert f(hq=30) == 1               # not a multiple of Hkv
        assert f(hq=24) == 2               # group 3 unsupported
        assert f(nw=-1) == 1
        assert f(ms=0) == 1
        assert f(ws=None) == 1
        assert f(wsb=100) == 3
        assert f(ws=ctypes.c_void_p(20)) == 1   # misaligned workspace
        assert f(batch=0) == 0
    assert prep(q=None) == 1
    assert prep(rk=None) == 1
    assert prep(lens=None) == 1
    assert dec(pages=None) == 1
    assert dec(bt=None) == 1
    assert dec(sw=None) == 1               # the layout has sink/window rows
    for bad in (float("nan"), float("inf"), 0.0, -1.0):
        assert dec(sm=bad) == 1


def test_append_and_prepare_validation(lib):
    lay = _layout()

    def call(**kw):
        a = dict(pages=FAKE, sw=FAKE, bt=FAKE, batch=1, total=1, k=FAKE, v=FAKE, off=FAKE,
                 start=FAKE, rk=FAKE, rv=FAKE, km=None, ck=0.95, cv=0.95, hq=32, q=FAKE,
                 lens=FAKE, nw=0, ms=4, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.oscar_append_and_prepare(
            ctypes.byref(lay), a["pages"], a["sw"], a["bt"], None, a["batch"], a["total"], a["k"],
            a["v"], a["off"], a["start"], a["rk"], a["rv"], a["km"], a["ck"], a["cv"], a["hq"],
            a["q"], a["lens"], a["nw"], a["ms"], a["ws"], a["wsb"], None)

    # the query preparation's checks
    assert call(hq=30) == 1
    assert call(hq=24) == 2
    assert call(nw=-1) == 1
    assert call(ms=0) == 1
    assert call(q=None) == 1
    assert call(lens=None) == 1
    assert call(rk=None) == 1
    assert call(ws=None) == 1
    assert call(ws=ctypes.c_void_p(20)) == 1
    assert call(wsb=100) == 3
    assert call(batch=(1 << 22) + 1) == 2          # more than 2^27 query rows
    # the append's checks
    assert call(total=-1) == 1
    assert call(total=(1 << 30) + 1) == 2
    for bad in (0.0, -0.5, 1.5, float("nan")):
        assert call(ck=bad) == 1
        assert call(cv=bad) == 1
    assert call(pages=None) == 1
    assert call(bt=None) == 1
    assert call(k=None) == 1
    assert call(v=None) == 1
    assert call(off=None) == 1
    assert call(start=None) == 1
    assert call(rv=None) == 1
    assert call(sw=None) == 1                      # the layout has sink/window rows
    assert call(k=ctypes.c_void_p(20)) == 1        # misaligned
    assert call(km=ctypes.c_void_p(18)) == 1       # misaligned key mean
    assert call(batch=0) == 0
