"""The C ABI library (CPU-side checks, no GPU needed): it loads, exports
every entry point that include/isd.h declares, and its host-side argument
validation rejects bad calls before anything touches a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "isd.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    import invariant_speculative_decoding_amd as m
    if not os.path.exists(m.LIB_PATH):
        from invariant_speculative_decoding_amd import build
        build.build()
    return m.lib()


def test_header_declares_the_four_calls():
    assert {"qgemm_w4", "qgemm_w4_pack", "decode_attn", "spec_verify", "kv_commit"} <= set(_declared())


def test_library_exports_every_declared_symbol(L):
    for name in _declared():
        assert hasattr(L, name), name
    assert L.isd_version().decode().startswith("isd")


def test_binding_signatures_cover_the_header():
    import invariant_speculative_decoding_amd as m
    assert set(_declared()) <= set(m.SIGNATURES)


def test_validation_rejects_before_any_launch(L):
    sz = ctypes.c_size_t(0)
    # packed size, computed on the host
    assert L.qgemm_w4_packed_bytes(17, 160) == 2 * 2 * 1024
    assert L.qgemm_w4_packed_bytes(17, 100) == 0
    assert L.qgemm_w4_pack(None, None, None, None, 16, 64, None) == -1
    # qgemm_w4: null pointers, K not a multiple of 32, n outside 1..512, dtype
    assert L.qgemm_w4(None, None, None, 1, None, 16, 64, 1, None) == -1
    assert L.qgemm_w4(16, 16, 16, 1, 16, 16, 48, 1, None) == -1
    assert L.qgemm_w4(16, 16, 16, 1, 16, 16, 64, 513, None) == -1
    assert L.qgemm_w4(16, 16, 16, 7, 16, 16, 64, 1, None) == -1
    # qgemm_w4_argmax: keys per row = wave columns along N (host-side query:
    # 9504 row tiles, 5 per wave and 2 waves per work-group in the very tall
    # class, so 951 work-groups of 2 columns), null nkeys, a stride other
    # than the queried one
    nk = ctypes.c_int(0)
    assert L.qgemm_w4_argmax(None, None, None, 1, None, 152064, 5120, 1, None, ctypes.byref(nk),
                             None) == 0 and nk.value == -(-(152064 // 16) // 10) * 2
    assert L.qgemm_w4_argmax(None, None, None, 1, None, 300, 256, 1, None, ctypes.byref(nk),
                             None) == 0 and nk.value == 19
    assert L.qgemm_w4_argmax(None, None, None, 1, None, 16, 64, 1, None, None, None) == -1
    bad = ctypes.c_int(20)
    assert L.qgemm_w4_argmax(16, 16, 16, 1, None, 300, 256, 1, 16, ctypes.byref(bad), None) == -1
    # spec_verify_keys: null keys, nkeys < 1, seq_len without pos_id
    assert L.spec_verify_keys(None, 4, 16, 16, 1, 2, 16, 16, None, None, None) == -1
    assert L.spec_verify_keys(16, 0, 16, 16, 1, 2, 16, 16, None, None, None) == -1
    assert L.spec_verify_keys(16, 4, 16, 16, 1, 2, 16, 16, 16, None, None) == -1
    # qgemm_q6: packed size (2 tiles x 2 steps x (1536 + 128) + 2 tiles x 32),
    # K not a multiple of 256, n outside 1..512, dtype
    assert L.qgemm_q6_packed_bytes(17, 256) == 2 * 2 * (1536 + 128) + 2 * 32
    assert L.qgemm_q6_packed_bytes(17, 384) == 0
    assert L.qgemm_q6_pack(None, None, None, None, None, 16, 256, None) == -1
    assert L.qgemm_q6(None, None, 1, None, 16, 256, 1, None) == -1
    assert L.qgemm_q6(16, 16, 1, 16, 16, 128, 1, None) == -1
    assert L.qgemm_q6(16, 16, 1, 16, 16, 256, 513, None) == -1
    assert L.qgemm_q6(16, 16, 7, 16, 16, 256, 1, None) == -1
    # decode_attn: workspace query needs no GPU; bad shapes rejected
    assert L.decode_attn(None, None, None, None, 4, 4, None, None, None, 1, 64, 8, 128,
                         ctypes.c_float(0.1), None, ctypes.byref(sz), None) == 0
    assert sz.value > 0
    assert L.decode_attn(None, None, None, None, 4, 4, None, None, None, 1, 64, 8, 100,
                         ctypes.c_float(0.1), None, ctypes.byref(sz), None) == -1
    assert L.decode_attn(None, None, None, None, 4, 4, None, None, None, 1, 6, 4, 64,
                         ctypes.c_float(0.1), None, ctypes.byref(sz), None) == -1
    # decode_attn_append: new rows must be 16-byte aligned (keys and values)
    big = ctypes.c_size_t(1 << 40)
    assert L.decode_attn_append(16, 16, 18, 16, 16, 16, 4, 4, 16, 16, 16, 1, 64, 8, 128,
                                ctypes.c_float(0.1), 16, ctypes.byref(big), None) == -1
    assert L.decode_attn_append(16, 24, 16, 16, 16, 16, 4, 4, 16, 16, 16, 1, 64, 8, 128,
                                ctypes.c_float(0.1), 16, ctypes.byref(big), None) == -1
    # spec_verify: size queries for both modes; negative temperature rejected
    assert L.spec_verify(None, None, None, None, None, None, 2, 100, 10, ctypes.c_float(0.0),
                         ctypes.c_uint64(1), None, None, None, ctypes.byref(sz), None) == 0
    assert L.spec_verify(None, None, None, None, None, None, 2, 100, 10, ctypes.c_float(0.8),
                         ctypes.c_uint64(1), None, None, None, ctypes.byref(sz), None) == 0
    assert L.spec_verify(None, None, None, None, None, None, 2, 100, 10, ctypes.c_float(-1.0),
                         ctypes.c_uint64(1), None, None, None, ctypes.byref(sz), None) == -1
    assert L.spec_verify(None, None, None, None, None, None, 2, 100, 1, ctypes.c_float(0.0),
                         ctypes.c_uint64(1), None, None, None, ctypes.byref(sz), None) == -1
    # spec_verify_margin: size query; a NaN threshold is rejected
    assert L.spec_verify_margin(None, None, None, 2, 100, 10, ctypes.c_float(1e-3), None, None,
                                None, None, None, ctypes.byref(sz), None) == 0
    assert sz.value > 0
    assert L.spec_verify_margin(None, None, None, 2, 100, 10, ctypes.c_float(float("nan")), None,
                                None, None, None, None, ctypes.byref(sz), None) == -1
    # spec_verify_commit: size query; max_rows < B rejected
    assert L.spec_verify_commit(None, None, None, 2, 100, 10, None, None, None, None, None,
                                ctypes.byref(sz), None) == 0
    assert sz.value > 0
    assert L.spec_verify_commit(None, None, None, 2, 100, 1, None, None, None, None, None,
                                ctypes.byref(sz), None) == -1
    # kv_commit: bad head dim / missing state
    assert L.kv_commit(None, None, None, 4, 4, None, None, None, None, None, None, 1, 8, 100,
                       None) == -1
    assert L.kv_commit(None, None, None, 4, 4, None, None, None, None, None, None, 1, 8, 128,
                       None) == -1


def test_noalloc_verify_rejects_before_touching_a_device(L):
    """spec_verify_noalloc checks its arguments and its scratch limit on the
    host before it looks up the scratch's device address."""
    f = L.spec_verify_noalloc
    # greedy at V = 152064 needs 8 max_rows ceil(V/4096) bytes: 3449 rows fit
    # in the 1 MiB scratch, 3450 do not
    assert f(None, None, None, None, None, None, 1, 152064, 3450, ctypes.c_float(0.0),
             ctypes.c_uint64(1), None, None, None) == -2
    # the sampling workspace is larger per row: 2000 rows no longer fit
    assert f(None, None, None, None, None, None, 8, 152064, 2000, ctypes.c_float(0.8),
             ctypes.c_uint64(1), None, None, None) == -2
    # bad arguments: max_rows < B, negative temperature
    assert f(None, None, None, None, None, None, 2, 100, 1, ctypes.c_float(0.0),
             ctypes.c_uint64(1), None, None, None) == -1
    assert f(None, None, None, None, None, None, 2, 100, 10, ctypes.c_float(-1.0),
             ctypes.c_uint64(1), None, None, None) == -1


def test_stream_read_validates_on_the_host(L):
    """stream_read (measurement only): sizes and sink checked before any
    launch; one sink word per 32 KB work-group."""
    assert L.stream_read_sink_words(1 << 30) == (1 << 30) // 32768
    assert L.stream_read_sink_words(16) == 1
    assert L.stream_read(None, 1 << 20, None, 64, None) == -1
    assert L.stream_read(16, 100, 16, 64, None) == -1          # not a multiple of 16
    assert L.stream_read(16, 1 << 20, 16, 31, None) == -1      # sink too small (32 needed)
