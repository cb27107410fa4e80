"""Host-side argument validation of every C entry point, one documented
constraint at a time (CPU only).

For each call a baseline argument set that meets every constraint
include/isd.h states must get past validation: with no GPU present its
launch (or the device lookup before it) then fails and the call returns
ISD_EHIP.  Breaking any one constraint must return ISD_EINVAL (or
ISD_ENOSPC for a short workspace) instead, before any launch; values at
the edge of a documented range must still get through.  The baselines
pass fake, suitably aligned device addresses, so the module is skipped
wherever a GPU is visible (there the launch would be real)."""
import ctypes

import pytest

EINVAL, ENOSPC, EHIP = -1, -2, -3
A = 1 << 20  # a fake device address, 256-byte aligned; never dereferenced
BIG = 1 << 50  # a workspace size larger than any call asks for


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


pytestmark = pytest.mark.skipif(_gpu_visible(), reason="the baseline calls would launch on a GPU")


class Size:
    """A size_t in/out argument: passed by reference, read back after the call."""

    def __init__(self, v):
        self.c = ctypes.c_size_t(v)


@pytest.fixture(scope="module")
def L():
    import os

    import invariant_speculative_decoding_amd as m
    if not os.path.exists(m.LIB_PATH):
        from invariant_speculative_decoding_amd import build
        build.build()
    return m.lib()


def call(L, name, base, **changes):
    args = dict(base)
    for k, v in changes.items():
        assert k in args, k
        args[k] = v
    conv = [ctypes.byref(v.c) if isinstance(v, Size) else v for v in args.values()]
    return getattr(L, name)(*conv)


def expect(L, name, base, bad, good=()):
    """base gets past validation; each change in `bad` is rejected with its
    code; each change in `good` still gets past validation."""
    assert call(L, name, base) == EHIP, (name, "baseline")
    for change, code in bad:
        assert call(L, name, base, **change) == code, (name, change)
    for change in good:
        assert call(L, name, base, **change) == EHIP, (name, change)


def nulls(*names):
    return [({n: None}, EINVAL) for n in names]


def misaligned(**offsets):
    return [({n: A + o}, EINVAL) for n, o in offsets.items()]


def test_qgemm_w4(L):
    base = dict(codes_p=A, scales_p=A, x=A, x_dtype=1, y=A, N=64, K=256, n=4, stream=None)
    bad = (nulls("codes_p", "scales_p", "x", "y")
           + misaligned(codes_p=8, scales_p=8, x=8, y=2)
           + [({"x_dtype": 2}, EINVAL), ({"x_dtype": -1}, EINVAL),
              ({"N": 0}, EINVAL), ({"N": (1 << 30) + 1}, EINVAL),
              ({"K": 0}, EINVAL), ({"K": 48}, EINVAL), ({"K": 33}, EINVAL),
              ({"n": 0}, EINVAL), ({"n": 513}, EINVAL),
              ({"N": 1 << 30, "K": 1 << 12}, EINVAL)])  # N K / 2 = 2^41 > 2^40
    good = [{"y": A + 4}, {"x_dtype": 0}, {"N": 1}, {"K": 32}, {"n": 1}, {"n": 512},
            {"N": 1 << 30, "K": 1 << 11}]  # N K / 2 = 2^40
    expect(L, "qgemm_w4", base, bad, good)


def test_qgemm_w4_argmax(L):
    nk = ctypes.c_int(0)
    q = dict(codes_p=None, scales_p=None, x=None, x_dtype=1, y=None, N=300, K=256, n=1,
             keys=None, nkeys=ctypes.byref(nk), stream=None)
    assert call(L, "qgemm_w4_argmax", q) == 0 and nk.value == 19
    for change in ({"N": 0}, {"N": (1 << 30) + 1}, {"K": 48}, {"x_dtype": 2}, {"nkeys": None}):
        assert call(L, "qgemm_w4_argmax", q, **change) == EINVAL, change
    right, wrong = ctypes.c_int(19), ctypes.c_int(20)
    base = dict(q, codes_p=A, scales_p=A, x=A, y=A, n=4, keys=A, nkeys=ctypes.byref(right))
    bad = (nulls("codes_p", "scales_p", "x")
           + misaligned(codes_p=8, scales_p=8, x=8, y=2, keys=4)
           + [({"nkeys": ctypes.byref(wrong)}, EINVAL), ({"nkeys": None}, EINVAL),
              ({"n": 0}, EINVAL), ({"n": 513}, EINVAL)])
    good = [{"y": None}, {"n": 512}]
    expect(L, "qgemm_w4_argmax", base, bad, good)


def test_qgemm_w4_pack_and_size(L):
    assert L.qgemm_w4_packed_bytes(1 << 30, 32) == (1 << 26) * 1024
    for N, K in ((0, 32), ((1 << 30) + 1, 32), (16, 48), (16, 0)):
        assert L.qgemm_w4_packed_bytes(N, K) == 0, (N, K)
    base = dict(codes=A, scale_min=A, codes_p=A, scales_p=A, N=64, K=256, stream=None)
    bad = (nulls("codes", "scale_min", "codes_p", "scales_p")
           + misaligned(codes=2, scale_min=2, codes_p=8, scales_p=8)
           + [({"N": 0}, EINVAL), ({"N": (1 << 30) + 1}, EINVAL), ({"K": 48}, EINVAL),
              ({"N": 1 << 30, "K": 1 << 12}, EINVAL)])  # 2^26 tiles x 2^5 steps = 2^31
    good = [{"codes": A + 4}, {"N": 1 << 30, "K": 1 << 11}]
    expect(L, "qgemm_w4_pack", base, bad, good)


def test_qgemm_q6_pack_and_size(L):
    for N, K in ((0, 256), ((1 << 30) + 1, 256), (16, 384), (16, 128)):
        assert L.qgemm_q6_packed_bytes(N, K) == 0, (N, K)
    base = dict(ql=A, qh=A, sc=A, d=A, packed=A, N=64, K=512, stream=None)
    bad = (nulls("ql", "qh", "sc", "d", "packed")
           + misaligned(d=1, packed=8)
           + [({"N": 0}, EINVAL), ({"N": (1 << 30) + 1}, EINVAL), ({"K": 384}, EINVAL),
              ({"N": 1 << 30, "K": 1 << 13}, EINVAL)])  # 2^26 tiles x 2^6 steps
    good = [{"ql": A + 1}, {"qh": A + 1}, {"sc": A + 1}, {"d": A + 2}]
    expect(L, "qgemm_q6_pack", base, bad, good)


def test_qgemm_q6(L):
    base = dict(packed=A, x=A, x_dtype=1, y=A, N=64, K=512, n=4, stream=None)
    bad = (nulls("packed", "x", "y")
           + misaligned(packed=8, x=8, y=2)
           + [({"x_dtype": 2}, EINVAL), ({"K": 128}, EINVAL), ({"K": 384}, EINVAL),
              ({"N": 0}, EINVAL), ({"N": (1 << 30) + 1}, EINVAL), ({"n": 0}, EINVAL),
              ({"n": 513}, EINVAL), ({"N": 1 << 30, "K": 1 << 12}, EINVAL)])  # 2^42 > 2^41
    good = [{"x_dtype": 0}, {"n": 512}, {"K": 256}, {"N": 1 << 29, "K": 1 << 12}]
    expect(L, "qgemm_q6", base, bad, good)


def _attn_base(append):
    d = dict(q=A)
    if append:
        d.update(k_new=A, v_new=A)
    d.update(k_pages=A, v_pages=A, page_table=A, max_pages=4, num_pages=4, q_pos=A,
             row_start=A, out=A, B=2, Hq=64, Hkv=8, D=128, scale=ctypes.c_float(0.1), ws=A,
             ws_bytes=Size(BIG), stream=None)
    return d


@pytest.mark.parametrize("append", [False, True])
def test_decode_attn(L, append):
    name = "decode_attn_append" if append else "decode_attn"
    base = _attn_base(append)
    # size query: no launch, no pointers needed
    sz = Size(0)
    q = dict(base, ws=None, ws_bytes=sz)
    assert call(L, name, q) == 0
    need = sz.c.value
    assert need == 2 * 8 * 64 * 1 * (128 + 4) * 4  # B rows Hq chunks (D + 4) floats
    # a workspace one byte short: ENOSPC, and the need written back
    short = Size(need - 1)
    assert call(L, name, base, ws_bytes=short) == ENOSPC and short.c.value == need
    assert call(L, name, base, ws_bytes=Size(need)) == EHIP
    bad = (nulls("q", "k_pages", "v_pages", "page_table", "q_pos", "row_start", "out",
                 "ws_bytes")
           + misaligned(q=8, k_pages=8, v_pages=8, ws=8, out=2, page_table=2, q_pos=2,
                        row_start=2)
           + [({"B": 0}, EINVAL), ({"Hq": 0}, EINVAL), ({"Hkv": 0}, EINVAL),
              ({"Hq": 6, "Hkv": 4}, EINVAL), ({"Hq": 34, "Hkv": 2}, EINVAL),
              ({"D": 96}, EINVAL), ({"max_pages": 0}, EINVAL), ({"num_pages": 0}, EINVAL),
              ({"max_pages": (1 << 26) + 1}, EINVAL),
              # 2^18 sequences x 8 kv-heads x 256 chunks = 2^29 units, 4 query
              # tiles each: 2^31
              ({"B": 1 << 18, "max_pages": 1 << 12}, EINVAL)])
    if append:
        bad += nulls("k_new", "v_new") + misaligned(k_new=8, v_new=8)
    good = [{"Hq": 32, "Hkv": 2}, {"D": 64}, {"max_pages": 1 << 26}, {"out": A + 4},
            {"B": (1 << 18) - 1, "max_pages": 1 << 12}]
    expect(L, name, base, bad, good)
    # the unit bound holds for the size query too
    assert call(L, name, q, B=1 << 18, max_pages=1 << 12) == EINVAL


def _verify_base(sampled):
    return dict(target_logits=A, draft_logits=A if sampled else None, drafts=A, row_start=A,
                seq_id=A if sampled else None, pos0=A if sampled else None, B=2, V=1000,
                max_rows=10, temperature=ctypes.c_float(0.8 if sampled else 0.0),
                seed=ctypes.c_uint64(1), accept_len=A, out_tokens=A, ws=A, ws_bytes=Size(BIG),
                stream=None)


def _verify_common_bad():
    return (nulls("target_logits", "drafts", "row_start", "accept_len", "out_tokens")
            + misaligned(target_logits=2, drafts=2, row_start=2, accept_len=2, out_tokens=2)
            + [({"B": 0}, EINVAL), ({"V": 0}, EINVAL), ({"max_rows": 1}, EINVAL),
               ({"max_rows": (1 << 24) + 1}, EINVAL),
               ({"temperature": ctypes.c_float(-1.0)}, EINVAL),
               ({"temperature": ctypes.c_float(float("inf"))}, EINVAL),
               ({"temperature": ctypes.c_float(float("nan"))}, EINVAL)])


@pytest.mark.parametrize("sampled", [False, True])
def test_spec_verify(L, sampled):
    base = _verify_base(sampled)
    sz = Size(0)
    assert call(L, "spec_verify", base, ws=None, ws_bytes=sz) == 0 and sz.c.value > 0
    short = Size(sz.c.value - 1)
    assert call(L, "spec_verify", base, ws_bytes=short) == ENOSPC
    bad = _verify_common_bad() + misaligned(ws=8) + nulls("ws_bytes")
    good = [{"max_rows": 1 << 24}, {"max_rows": 2}]
    if sampled:
        bad += (nulls("draft_logits", "seq_id", "pos0")
                + misaligned(draft_logits=2, seq_id=2, pos0=2)
                + [({"V": (1 << 20) + 1}, EINVAL)])  # 257 chunks of 4096
        good += [{"V": 1 << 20}]
    else:
        good += [{"V": (1 << 20) + 1}]  # greedy has no chunk limit
    expect(L, "spec_verify", base, bad, good)


@pytest.mark.parametrize("sampled", [False, True])
def test_spec_verify_noalloc(L, sampled):
    """Pointers and sizes are checked before the scratch's device address is
    looked up (which fails here, giving ISD_EHIP)."""
    base = _verify_base(sampled)
    del base["ws"], base["ws_bytes"]
    bad = _verify_common_bad() + [({"max_rows": 200000}, ENOSPC)]  # > 1 MiB
    if sampled:
        bad += nulls("draft_logits", "seq_id", "pos0") + misaligned(draft_logits=2, seq_id=2,
                                                                    pos0=2)
    expect(L, "spec_verify_noalloc", base, bad)


def test_spec_verify_keys(L):
    base = dict(keys=A, nkeys=4, drafts=A, row_start=A, B=2, max_rows=10, accept_len=A,
                out_tokens=A, seq_len=None, pos_id=None, stream=None)
    bad = (nulls("keys", "drafts", "row_start", "accept_len", "out_tokens")
           + misaligned(keys=4, drafts=2, row_start=2, accept_len=2, out_tokens=2)
           + [({"nkeys": 0}, EINVAL), ({"B": 0}, EINVAL), ({"max_rows": 1}, EINVAL),
              ({"max_rows": (1 << 24) + 1}, EINVAL), ({"seq_len": A}, EINVAL),
              ({"pos_id": A}, EINVAL), ({"seq_len": A + 2, "pos_id": A}, EINVAL),
              ({"seq_len": A, "pos_id": A + 2}, EINVAL)])
    good = [{"seq_len": A, "pos_id": A}, {"nkeys": 1}, {"max_rows": 1 << 24}]
    expect(L, "spec_verify_keys", base, bad, good)


def test_spec_verify_margin(L):
    base = dict(target_logits=A, drafts=A, row_start=A, B=2, V=1000, max_rows=10,
                threshold=ctypes.c_float(1e-3), accept_len=A, out_tokens=A, margins=A,
                recheck=A, ws=A, ws_bytes=Size(BIG), stream=None)
    sz = Size(0)
    assert call(L, "spec_verify_margin", base, ws=None, ws_bytes=sz) == 0
    assert sz.c.value == 10 * 1 * 2 * 8
    assert call(L, "spec_verify_margin", base, ws_bytes=Size(sz.c.value - 1)) == ENOSPC
    bad = (nulls("target_logits", "drafts", "row_start", "accept_len", "out_tokens", "margins",
                 "recheck", "ws_bytes")
           + misaligned(target_logits=2, drafts=2, row_start=2, accept_len=2, out_tokens=2,
                        margins=2, recheck=2, ws=8)
           + [({"B": 0}, EINVAL), ({"V": 0}, EINVAL), ({"max_rows": 1}, EINVAL),
              ({"max_rows": (1 << 24) + 1}, EINVAL),
              ({"threshold": ctypes.c_float(float("nan"))}, EINVAL)])
    good = [{"threshold": ctypes.c_float(float("inf"))}, {"threshold": ctypes.c_float(-1.0)}]
    expect(L, "spec_verify_margin", base, bad, good)


def test_spec_verify_commit(L):
    base = dict(target_logits=A, drafts=A, row_start=A, B=2, V=1000, max_rows=10,
                accept_len=A, out_tokens=A, seq_len=A, pos_id=A, ws=A, ws_bytes=Size(BIG),
                stream=None)
    sz = Size(0)
    assert call(L, "spec_verify_commit", base, ws=None, ws_bytes=sz) == 0
    assert sz.c.value == 10 * 1 * 8
    assert call(L, "spec_verify_commit", base, ws_bytes=Size(sz.c.value - 1)) == ENOSPC
    bad = (nulls("target_logits", "drafts", "row_start", "accept_len", "out_tokens", "seq_len",
                 "pos_id", "ws_bytes")
           + misaligned(target_logits=2, drafts=2, row_start=2, accept_len=2, out_tokens=2,
                        seq_len=2, pos_id=2, ws=8)
           + [({"B": 0}, EINVAL), ({"V": 0}, EINVAL), ({"max_rows": 1}, EINVAL),
              ({"max_rows": (1 << 24) + 1}, EINVAL)])
    expect(L, "spec_verify_commit", base, bad)


def test_spec_verify_sampled_commit(L):
    base = dict(target_logits=A, draft_logits=A, drafts=A, row_start=A, seq_id=A, B=2, V=1000,
                max_rows=10, temperature=ctypes.c_float(0.8), seed=ctypes.c_uint64(1),
                accept_len=A, out_tokens=A, seq_len=A, pos_id=A, ws=A, ws_bytes=Size(BIG),
                stream=None)
    sz = Size(0)
    assert call(L, "spec_verify_sampled_commit", base, ws=None, ws_bytes=sz) == 0
    ref = Size(0)
    assert call(L, "spec_verify", _verify_base(True), ws=None, ws_bytes=ref) == 0
    assert sz.c.value == ref.c.value  # the workspace of the sampled spec_verify
    assert call(L, "spec_verify_sampled_commit", base, ws_bytes=Size(sz.c.value - 1)) == ENOSPC
    bad = (nulls("target_logits", "draft_logits", "drafts", "row_start", "seq_id", "accept_len",
                 "out_tokens", "seq_len", "pos_id", "ws_bytes")
           + misaligned(target_logits=2, draft_logits=2, drafts=2, row_start=2, seq_id=2,
                        accept_len=2, out_tokens=2, seq_len=2, pos_id=2, ws=8)
           + [({"B": 0}, EINVAL), ({"V": 0}, EINVAL), ({"max_rows": 1}, EINVAL),
              ({"max_rows": (1 << 24) + 1}, EINVAL), ({"V": (1 << 20) + 1}, EINVAL),
              ({"temperature": ctypes.c_float(0.0)}, EINVAL),
              ({"temperature": ctypes.c_float(-1.0)}, EINVAL),
              ({"temperature": ctypes.c_float(float("inf"))}, EINVAL),
              ({"temperature": ctypes.c_float(float("nan"))}, EINVAL)])
    good = [{"max_rows": 1 << 24}, {"V": 1 << 20}]
    expect(L, "spec_verify_sampled_commit", base, bad, good)


def test_kv_commit(L):
    commit = dict(k_pages=None, v_pages=None, page_table=None, max_pages=4, num_pages=4,
                  k_new=None, v_new=None, row_start=None, seq_len=A, pos_id=A, accept_len=A,
                  B=2, Hkv=8, D=128, stream=None)
    bad = (nulls("seq_len", "pos_id") + misaligned(seq_len=2, pos_id=2, accept_len=2)
           + [({"B": 0}, EINVAL), ({"Hkv": 0}, EINVAL), ({"D": 100}, EINVAL),
              ({"max_pages": 0}, EINVAL), ({"num_pages": 0}, EINVAL)])
    expect(L, "kv_commit", commit, bad, good=[{"D": 64}])
    append = dict(commit, k_pages=A, v_pages=A, page_table=A, k_new=A, v_new=A, row_start=A,
                  accept_len=None)
    bad = (nulls("k_pages", "v_pages", "page_table", "k_new", "v_new", "row_start", "seq_len",
                 "pos_id")
           + misaligned(k_pages=1, v_pages=1, k_new=1, v_new=1, page_table=2, row_start=2,
                        seq_len=2, pos_id=2))
    good = [{"k_pages": A + 2}, {"k_new": A + 2}]
    expect(L, "kv_commit", append, bad, good)


def test_row_wise_operations(L):
    expect(L, "embed_rows", dict(tokens=A, table=A, h=A, rows=4, V=100, H=64, stream=None),
           nulls("tokens", "table", "h") + misaligned(tokens=2, table=1, h=2)
           + [({"rows": 0}, EINVAL), ({"V": 0}, EINVAL), ({"H": 0}, EINVAL)],
           good=[{"table": A + 2}])
    expect(L, "add_rmsnorm",
           dict(h=A, d=A, w=A, y=A, rows=4, H=64, eps=ctypes.c_float(1e-6), stream=None),
           nulls("h", "w", "y") + misaligned(h=2, d=2, w=2, y=1)
           + [({"rows": 0}, EINVAL), ({"H": 0}, EINVAL), ({"H": 8193}, EINVAL),
              ({"eps": ctypes.c_float(-1.0)}, EINVAL),
              ({"eps": ctypes.c_float(float("nan"))}, EINVAL)],
           good=[{"d": None}, {"H": 8192}, {"eps": ctypes.c_float(0.0)}, {"y": A + 2}])
    expect(L, "rope_qkv",
           dict(qkv=A, row_start=A, pos_id=A, B=2, rows=4, Hq=8, Hkv=2, D=64,
                theta=ctypes.c_float(1e4), q=A, k=A, v=A, stream=None),
           nulls("qkv", "row_start", "pos_id", "q", "k", "v")
           + misaligned(qkv=2, row_start=2, pos_id=2, q=1, k=1, v=1)
           + [({"B": 0}, EINVAL), ({"rows": 0}, EINVAL), ({"Hq": 0}, EINVAL),
              ({"Hkv": 0}, EINVAL), ({"D": 0}, EINVAL), ({"D": 3}, EINVAL),
              ({"D": 130}, EINVAL), ({"theta": ctypes.c_float(1.0)}, EINVAL),
              ({"theta": ctypes.c_float(float("nan"))}, EINVAL),
              ({"Hq": 1 << 24, "Hkv": 1, "D": 128}, EINVAL)],  # row of 2^31 + 256 values
           good=[{"D": 2}, {"D": 128}, {"Hq": (1 << 24) - 3, "Hkv": 1, "D": 128}])
    expect(L, "silu_mul", dict(gu=A, y=A, rows=4, F=100, stream=None),
           nulls("gu", "y") + misaligned(gu=2, y=1)
           + [({"rows": 0}, EINVAL), ({"F": 0}, EINVAL)],
           good=[{"F": (1 << 31) - 1}])


def test_stream_read(L):
    base = dict(buf=A, bytes=1 << 20, sink=A, sink_words=32, stream=None)
    bad = (nulls("buf", "sink") + misaligned(buf=8, sink=2)
           + [({"bytes": 0}, EINVAL), ({"bytes": 8}, EINVAL), ({"bytes": 100}, EINVAL),
              ({"sink_words": 31}, EINVAL)])
    good = [{"bytes": 16, "sink_words": 1}]
    expect(L, "stream_read", base, bad, good)
