"""Batch-invariant speculative-verify kernels for AMD MI355X (gfx950).

Thin Python binding over ``libisd.so`` (C ABI declared in
``include/isd.h``): each function checks shapes and dtypes of torch device
tensors, passes their pointers and torch's current stream, and raises on a
non-zero return code.  All arithmetic runs in the library's HIP kernels;
there is no fallback -- if the library is missing, every call raises.

    qgemm_w4_pack(codes, scale_min)                       -> PackedW4 (one-time layout change)
    qgemm_w4(w: PackedW4, x, y=None)                      -> y  float32 [n][N]
    qgemm_w4_argmax(w, x, logits=True)                    -> (y or None, keys int64 [n][nkeys])
    qgemm_q6_pack(ql, qh, sc, d)                          -> PackedQ6 (6-bit super-blocks)
    qgemm_q6(w: PackedQ6, x, y=None)                      -> y  float32 [n][N]
    decode_attn(q, k_pages, v_pages, page_table, q_pos, row_start, scale)
                                                          -> out float32 [R][Hq][D]
    decode_attn_append(q, k_new, v_new, k_pages, v_pages, page_table, q_pos, row_start, scale)
                                                          -> out, with the block appended
    spec_verify(target_logits, drafts, row_start, ...)    -> (accept_len, out_tokens)
    spec_verify_noalloc(target_logits, drafts, row_start, ...)
                                                          -> the same, library-owned workspace
    spec_verify_commit(target_logits, drafts, row_start, seq_len, pos_id)
                                                          -> (accept_len, out_tokens), committed
    spec_verify_sampled_commit(target_logits, drafts, row_start, draft_logits, seq_id,
                               seq_len, pos_id, temperature, seed)
                                                          -> (accept_len, out_tokens), committed
    spec_verify_keys(keys, drafts, row_start, seq_len=None, pos_id=None)
                                                          -> (accept_len, out_tokens) from the keys
    kv_commit(k_pages, v_pages, page_table, seq_len, pos_id, row_start=..., k_new=...,
              v_new=...)            (APPEND)  or  kv_commit(..., accept_len=...)  (COMMIT)
    stream_read(buf)                                      plain HBM read (measurement only)

Half-precision tensors may be torch.float16 / torch.bfloat16 or any 16-bit
integer tensor holding the raw bits.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libisd.so")

ISD_OK, ISD_EINVAL, ISD_ENOSPC, ISD_EHIP = 0, -1, -2, -3
ISD_F32, ISD_BF16 = 0, 1
MAX_ROWS, MAX_OUT, PAGE, CHUNK = 8, 9, 16, 256

_ERR = {ISD_EINVAL: "ISD_EINVAL", ISD_ENOSPC: "ISD_ENOSPC", ISD_EHIP: "ISD_EHIP"}
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.POINTER(ctypes.c_size_t)

SIGNATURES = {
    "qgemm_w4_packed_bytes": [_I, _I],
    "qgemm_w4_pack": [_P, _P, _P, _P, _I, _I, _P],
    "qgemm_w4": [_P, _P, _P, _I, _P, _I, _I, _I, _P],
    "qgemm_w4_argmax": [_P, _P, _P, _I, _P, _I, _I, _I, _P, ctypes.POINTER(ctypes.c_int), _P],
    "qgemm_q6_packed_bytes": [_I, _I],
    "qgemm_q6_pack": [_P, _P, _P, _P, _P, _I, _I, _P],
    "qgemm_q6": [_P, _P, _I, _P, _I, _I, _I, _P],
    "decode_attn": [_P, _P, _P, _P, _I, _I, _P, _P, _P, _I, _I, _I, _I, ctypes.c_float, _P,
                    _SZ, _P],
    "decode_attn_append": [_P, _P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _I, _I, _I, _I,
                           ctypes.c_float, _P, _SZ, _P],
    "spec_verify": [_P, _P, _P, _P, _P, _P, _I, _I, _I, ctypes.c_float, ctypes.c_uint64, _P, _P,
                    _P, _SZ, _P],
    "spec_verify_noalloc": [_P, _P, _P, _P, _P, _P, _I, _I, _I, ctypes.c_float,
                            ctypes.c_uint64, _P, _P, _P],
    "kv_commit": [_P, _P, _P, _I, _I, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P],
    "spec_verify_margin": [_P, _P, _P, _I, _I, _I, ctypes.c_float, _P, _P, _P, _P, _P, _SZ, _P],
    "spec_verify_commit": [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _SZ, _P],
    "spec_verify_keys": [_P, _I, _P, _P, _I, _I, _P, _P, _P, _P, _P],
    "spec_verify_sampled_commit": [_P, _P, _P, _P, _P, _I, _I, _I, ctypes.c_float,
                                   ctypes.c_uint64, _P, _P, _P, _P, _P, _SZ, _P],
    "embed_rows": [_P, _P, _P, _I, _I, _I, _P],
    "add_rmsnorm": [_P, _P, _P, _P, _I, _I, ctypes.c_float, _P],
    "rope_qkv": [_P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_float, _P, _P, _P, _P],
    "silu_mul": [_P, _P, _I, _I, _P],
    "stream_read": [_P, ctypes.c_size_t, _P, ctypes.c_size_t, _P],
    "stream_read_sink_words": [ctypes.c_size_t],
    "isd_version": [],
}


def lib() -> ctypes.CDLL:
    """Load libisd.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m invariant_speculative_decoding_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = (ctypes.c_char_p if name == "isd_version" else
                         ctypes.c_size_t if name.endswith(("_packed_bytes", "_sink_words"))
                         else ctypes.c_int)
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != ISD_OK:
        raise RuntimeError(f"{what} failed: {_ERR.get(rc, rc)}")


def _dev(t: torch.Tensor, name: str, esize: int | None = None, dtypes=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if esize is not None and t.element_size() != esize:
        raise TypeError(f"{name}: expected {esize}-byte elements, got {t.dtype}")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    return t.data_ptr()


def _opt(t, name, **kw) -> int | None:
    return None if t is None else _dev(t, name, **kw)


def _need(ok: bool, what: str):
    """Shape checks on the host: the library indexes its arrays by the
    sizes the call states, so a short tensor is refused here."""
    if not ok:
        raise ValueError(what)


def _len_at_least(t, n: int, name: str):
    if t is not None:
        _need(t.numel() >= n, f"{name} must hold at least {n} entries")


def _nonempty(t, name: str):
    """A stand-in for an array the call will not read (no entries): the
    library takes no NULL for it."""
    if t is not None and t.numel() == 0:
        return torch.empty(1, dtype=t.dtype, device=t.device)
    return t


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


_I32 = (torch.int32,)


class PackedW4(NamedTuple):
    """4-bit weights in the library's packed layout (see qgemm_w4_pack in
    include/isd.h): codes uint8 [ceil(N/16)][ceil(K/128)][64][16] and scales
    int16 [ceil(N/16)][ceil(K/128)][16][4][2] (fp16 bits)."""
    codes: torch.Tensor
    scales: torch.Tensor
    N: int
    K: int


def qgemm_w4_pack(codes, scale_min) -> PackedW4:
    """Row-major codes uint8 [N][K/2] and scale_min [N][K/32][2] (fp16 bits)
    -> the packed layout qgemm_w4 streams."""
    N, half = codes.shape
    K = 2 * half
    if tuple(scale_min.shape) != (N, K // 32, 2):
        raise ValueError("scale_min must be [N][K/32][2]")
    nbytes = lib().qgemm_w4_packed_bytes(N, K)
    if nbytes == 0:
        raise ValueError("bad shape")
    cp = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    sp = torch.empty(nbytes // 8, dtype=torch.int16, device=codes.device)
    rc = lib().qgemm_w4_pack(_dev(codes, "codes", 1), _dev(scale_min, "scale_min", 2),
                             cp.data_ptr(), sp.data_ptr(), N, K, _stream(codes))
    _check(rc, "qgemm_w4_pack")
    return PackedW4(cp, sp, N, K)


def _packed_w4_sizes(w: PackedW4):
    nbytes = lib().qgemm_w4_packed_bytes(w.N, w.K)
    _need(nbytes > 0 and w.codes.numel() * w.codes.element_size() >= nbytes
          and w.scales.numel() * w.scales.element_size() >= nbytes // 4,
          "w does not hold a packed N x K matrix")


def qgemm_w4(w: PackedW4, x, y=None):
    """y[c][r] = sum_k W[r][k] x[c][k] for the packed 4-bit weights w."""
    N, K = w.N, w.K
    _packed_w4_sizes(w)
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError("x must be [n][K]")
    n = x.shape[0]
    if x.dtype == torch.float32:
        xd = ISD_F32
    elif x.element_size() == 2 and x.dtype != torch.float16:
        xd = ISD_BF16
    else:
        raise TypeError("x must be float32 or bf16 (bits)")
    if y is None:
        y = torch.empty((n, N), dtype=torch.float32, device=x.device)
    elif tuple(y.shape) != (n, N):
        raise ValueError("y must be [n][N]")
    rc = lib().qgemm_w4(_dev(w.codes, "codes", 1), _dev(w.scales, "scales", 2), _dev(x, "x"), xd,
                        _dev(y, "y", dtypes=(torch.float32,)), N, K, n, _stream(x))
    _check(rc, "qgemm_w4")
    return y


def qgemm_w4_argmax_nkeys(w: PackedW4, x_dtype=ISD_BF16) -> int:
    """Keys per row that qgemm_w4_argmax writes for these weights."""
    nk = ctypes.c_int(0)
    _check(lib().qgemm_w4_argmax(None, None, None, x_dtype, None, w.N, w.K, 1, None,
                                 ctypes.byref(nk), None), "qgemm_w4_argmax")
    return nk.value


def qgemm_w4_argmax(w: PackedW4, x, y=None, keys=None, logits=True):
    """qgemm_w4 that also writes each row's argmax keys (one per wave column
    along N); returns (y or None, keys [n][nkeys] int64)."""
    N, K = w.N, w.K
    _packed_w4_sizes(w)
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError("x must be [n][K]")
    n = x.shape[0]
    xd = _x_dtype(x)
    nk = qgemm_w4_argmax_nkeys(w, xd)
    if logits:
        if y is None:
            y = torch.empty((n, N), dtype=torch.float32, device=x.device)
        elif tuple(y.shape) != (n, N):
            raise ValueError("y must be [n][N]")
    else:
        y = None
    if keys is None:
        keys = torch.empty((n, nk), dtype=torch.int64, device=x.device)
    elif keys.dim() != 2 or keys.shape[0] < n or keys.shape[1] != nk:
        raise ValueError(f"keys must be [>= n][{nk}]")
    nkc = ctypes.c_int(nk)
    rc = lib().qgemm_w4_argmax(_dev(w.codes, "codes", 1), _dev(w.scales, "scales", 2),
                               _dev(x, "x"), xd, _opt(y, "y", dtypes=(torch.float32,)), N, K, n,
                               _dev(keys, "keys", dtypes=(torch.int64,)), ctypes.byref(nkc),
                               _stream(x))
    _check(rc, "qgemm_w4_argmax")
    return y, keys


def spec_verify_keys(keys, drafts, row_start, seq_len=None, pos_id=None, accept_len=None,
                     out_tokens=None, max_rows=None):
    """Greedy verify from qgemm_w4_argmax keys [rows][nkeys] (and the commit
    of kv_commit when seq_len and pos_id are given).  Returns (accept_len,
    out_tokens)."""
    R, nk = keys.shape
    B = row_start.numel() - 1
    _verify_sizes(R, B, drafts, accept_len, out_tokens)
    _len_at_least(seq_len, B, "seq_len")
    _len_at_least(pos_id, B, "pos_id")
    drafts = _nonempty(drafts, "drafts")
    if max_rows is None:
        max_rows = R
    dev = keys.device
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, MAX_OUT), dtype=torch.int32, device=dev)
    rc = lib().spec_verify_keys(_dev(keys, "keys", dtypes=(torch.int64,)), nk,
                                _dev(drafts, "drafts", dtypes=_I32),
                                _dev(row_start, "row_start", dtypes=_I32), B, max_rows,
                                _dev(accept_len, "accept_len", dtypes=_I32),
                                _dev(out_tokens, "out_tokens", dtypes=_I32),
                                _opt(seq_len, "seq_len", dtypes=_I32),
                                _opt(pos_id, "pos_id", dtypes=_I32), _stream(keys))
    _check(rc, "spec_verify_keys")
    return accept_len, out_tokens


def _x_dtype(x):
    if x.dtype == torch.float32:
        return ISD_F32
    if x.element_size() == 2 and x.dtype != torch.float16:
        return ISD_BF16
    raise TypeError("x must be float32 or bf16 (bits)")


class PackedQ6(NamedTuple):
    """6-bit super-block weights in the library's packed layout (see
    qgemm_q6_pack in include/isd.h): one uint8 buffer of
    qgemm_q6_packed_bytes(N, K) bytes."""
    packed: torch.Tensor
    N: int
    K: int


def qgemm_q6_pack(ql, qh, sc, d) -> PackedQ6:
    """Row-major ql uint8 [N][K/2], qh uint8 [N][K/4], sc int8 [N][K/16] and
    d [N][K/256] (fp16 bits) -> the packed layout qgemm_q6 streams."""
    N, half = ql.shape
    K = 2 * half
    if tuple(qh.shape) != (N, K // 4) or tuple(sc.shape) != (N, K // 16) \
            or tuple(d.shape) != (N, K // 256):
        raise ValueError("qh, sc, d must be [N][K/4], [N][K/16], [N][K/256]")
    nbytes = lib().qgemm_q6_packed_bytes(N, K)
    if nbytes == 0:
        raise ValueError("bad shape")
    buf = torch.empty(nbytes, dtype=torch.uint8, device=ql.device)
    rc = lib().qgemm_q6_pack(_dev(ql, "ql", 1), _dev(qh, "qh", 1), _dev(sc, "sc", 1),
                             _dev(d, "d", 2), buf.data_ptr(), N, K, _stream(ql))
    _check(rc, "qgemm_q6_pack")
    return PackedQ6(buf, N, K)


def qgemm_q6(w: PackedQ6, x, y=None):
    """y[c][r] = sum_k W[r][k] x[c][k] for the packed 6-bit weights w."""
    N, K = w.N, w.K
    nbytes = lib().qgemm_q6_packed_bytes(N, K)
    _need(nbytes > 0 and w.packed.numel() * w.packed.element_size() >= nbytes,
          "w does not hold a packed N x K matrix")
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError("x must be [n][K]")
    n = x.shape[0]
    xd = _x_dtype(x)
    if y is None:
        y = torch.empty((n, N), dtype=torch.float32, device=x.device)
    elif tuple(y.shape) != (n, N):
        raise ValueError("y must be [n][N]")
    rc = lib().qgemm_q6(_dev(w.packed, "packed", 1), _dev(x, "x"), xd,
                        _dev(y, "y", dtypes=(torch.float32,)), N, K, n, _stream(x))
    _check(rc, "qgemm_q6")
    return y


def _attn_sizes(B, R, Hq, D, q_pos, row_start, out):
    _need(row_start.numel() == B + 1, "row_start must hold B + 1 entries (B = table rows)")
    _len_at_least(q_pos, B, "q_pos")
    _need(out is None or tuple(out.shape) == (R, Hq, D), "out must be [R][Hq][D]")


def decode_attn(q, k_pages, v_pages, page_table, q_pos, row_start, scale, out=None, ws=None):
    R, Hq, D = q.shape
    num_pages, Hkv, page, Dk = k_pages.shape
    if page != PAGE or Dk != D or tuple(v_pages.shape) != (num_pages, Hkv, D, PAGE):
        raise ValueError("k_pages must be [P][Hkv][16][D] and v_pages [P][Hkv][D][16]")
    B, max_pages = page_table.shape
    _attn_sizes(B, R, Hq, D, q_pos, row_start, out)
    if out is None:
        out = torch.empty((R, Hq, D), dtype=torch.float32, device=q.device)
    need = ctypes.c_size_t(0)
    L = lib()
    _check(L.decode_attn(None, None, None, None, max_pages, num_pages, None, None, None, B, Hq,
                         Hkv, D, ctypes.c_float(scale), None, ctypes.byref(need), None),
           "decode_attn(size)")
    if ws is None or ws.numel() * ws.element_size() < need.value:
        ws = torch.empty(max(need.value, 16), dtype=torch.uint8, device=q.device)
    have = ctypes.c_size_t(ws.numel() * ws.element_size())
    rc = L.decode_attn(_dev(q, "q", 2), _dev(k_pages, "k_pages", 2), _dev(v_pages, "v_pages", 2),
                       _dev(page_table, "page_table", dtypes=_I32), max_pages, num_pages,
                       _dev(q_pos, "q_pos", dtypes=_I32), _dev(row_start, "row_start", dtypes=_I32),
                       _dev(out, "out", dtypes=(torch.float32,)), B, Hq, Hkv, D,
                       ctypes.c_float(scale), _dev(ws, "ws"), ctypes.byref(have), _stream(q))
    _check(rc, "decode_attn")
    return out



def decode_attn_append(q, k_new, v_new, k_pages, v_pages, page_table, q_pos, row_start, scale,
                       out=None, ws=None):
    """kv_commit APPEND of k_new / v_new at positions q_pos[s] + j, then
    decode_attn, in the launches of decode_attn alone."""
    R, Hq, D = q.shape
    num_pages, Hkv, page, Dk = k_pages.shape
    if page != PAGE or Dk != D or tuple(v_pages.shape) != (num_pages, Hkv, D, PAGE):
        raise ValueError("k_pages must be [P][Hkv][16][D] and v_pages [P][Hkv][D][16]")
    if tuple(k_new.shape) != (R, Hkv, D) or tuple(v_new.shape) != (R, Hkv, D):
        raise ValueError("k_new / v_new must be [R][Hkv][D]")
    B, max_pages = page_table.shape
    _attn_sizes(B, R, Hq, D, q_pos, row_start, out)
    if out is None:
        out = torch.empty((R, Hq, D), dtype=torch.float32, device=q.device)
    need = ctypes.c_size_t(0)
    L = lib()
    _check(L.decode_attn_append(None, None, None, None, None, None, max_pages, num_pages, None,
                                None, None, B, Hq, Hkv, D, ctypes.c_float(scale), None,
                                ctypes.byref(need), None), "decode_attn_append(size)")
    if ws is None or ws.numel() * ws.element_size() < need.value:
        ws = torch.empty(max(need.value, 16), dtype=torch.uint8, device=q.device)
    have = ctypes.c_size_t(ws.numel() * ws.element_size())
    rc = L.decode_attn_append(_dev(q, "q", 2), _dev(k_new, "k_new", 2), _dev(v_new, "v_new", 2),
                              _dev(k_pages, "k_pages", 2), _dev(v_pages, "v_pages", 2),
                              _dev(page_table, "page_table", dtypes=_I32), max_pages, num_pages,
                              _dev(q_pos, "q_pos", dtypes=_I32),
                              _dev(row_start, "row_start", dtypes=_I32),
                              _dev(out, "out", dtypes=(torch.float32,)), B, Hq, Hkv, D,
                              ctypes.c_float(scale), _dev(ws, "ws"), ctypes.byref(have),
                              _stream(q))
    _check(rc, "decode_attn_append")
    return out

def _verify_sizes(R, B, drafts, accept_len, out_tokens, V=None, draft_logits=None, seq_id=None,
                  pos0=None, sampled=False):
    """Lengths the verify calls index: R target rows and B sequences give
    R - B draft entries (and drafter rows when sampling)."""
    _need(B >= 1, "row_start must hold B + 1 >= 2 entries")
    _len_at_least(drafts, R - B, "drafts")
    _len_at_least(accept_len, B, "accept_len")
    _len_at_least(out_tokens, B * MAX_OUT, "out_tokens")
    if sampled:
        _need(draft_logits is not None and draft_logits.dim() == 2
              and draft_logits.shape[1] == V and draft_logits.shape[0] >= R - B,
              "draft_logits must be [R - B][V]")
        _len_at_least(seq_id, B, "seq_id")
        _len_at_least(pos0, B, "pos0")


def spec_verify(target_logits, drafts, row_start, draft_logits=None, seq_id=None, pos0=None,
                temperature=0.0, seed=0, accept_len=None, out_tokens=None, ws=None,
                max_rows=None):
    R, V = target_logits.shape
    B = row_start.numel() - 1
    if temperature > 0 and draft_logits is None and R <= B:  # no drafts, no drafter rows
        draft_logits = target_logits.new_empty((0, V))
    _verify_sizes(R, B, drafts, accept_len, out_tokens, V, draft_logits, seq_id, pos0,
                  sampled=temperature > 0)
    drafts, draft_logits = _nonempty(drafts, "drafts"), _nonempty(draft_logits, "draft_logits")
    if max_rows is None:
        max_rows = R
    dev = target_logits.device
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, MAX_OUT), dtype=torch.int32, device=dev)
    L = lib()
    need = ctypes.c_size_t(0)
    _check(L.spec_verify(None, None, None, None, None, None, B, V, max_rows,
                         ctypes.c_float(temperature), ctypes.c_uint64(seed), None, None, None,
                         ctypes.byref(need), None), "spec_verify(size)")
    if ws is None or ws.numel() * ws.element_size() < need.value:
        ws = torch.empty(max(need.value, 16), dtype=torch.uint8, device=dev)
    have = ctypes.c_size_t(ws.numel() * ws.element_size())
    rc = L.spec_verify(_dev(target_logits, "target_logits", dtypes=(torch.float32,)),
                       _opt(draft_logits, "draft_logits", dtypes=(torch.float32,)),
                       _dev(drafts, "drafts", dtypes=_I32), _dev(row_start, "row_start", dtypes=_I32),
                       _opt(seq_id, "seq_id", dtypes=_I32), _opt(pos0, "pos0", dtypes=_I32),
                       B, V, max_rows, ctypes.c_float(temperature), ctypes.c_uint64(seed),
                       _dev(accept_len, "accept_len", dtypes=_I32),
                       _dev(out_tokens, "out_tokens", dtypes=_I32), _dev(ws, "ws"),
                       ctypes.byref(have), _stream(target_logits))
    _check(rc, "spec_verify")
    return accept_len, out_tokens


def spec_verify_sampled_commit(target_logits, drafts, row_start, draft_logits, seq_id,
                               seq_len, pos_id, temperature, seed=0, accept_len=None,
                               out_tokens=None, ws=None, max_rows=None):
    """Rejection-sampling verify (temperature > 0) with pos0 = pos_id, then
    the commit of kv_commit (seq_len += accept_len + 1, pos_id = seq_len) in
    the same launches.  Returns (accept_len, out_tokens)."""
    R, V = target_logits.shape
    B = row_start.numel() - 1
    _need(temperature > 0, "temperature must be > 0 (the greedy commit is spec_verify_commit)")
    if draft_logits is None and R <= B:  # no drafts, no drafter rows
        draft_logits = target_logits.new_empty((0, V))
    _len_at_least(seq_len, B, "seq_len")
    _len_at_least(pos_id, B, "pos_id")
    _verify_sizes(R, B, drafts, accept_len, out_tokens, V, draft_logits, seq_id, pos_id,
                  sampled=True)
    drafts, draft_logits = _nonempty(drafts, "drafts"), _nonempty(draft_logits, "draft_logits")
    if max_rows is None:
        max_rows = R
    dev = target_logits.device
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, MAX_OUT), dtype=torch.int32, device=dev)
    L = lib()
    need = ctypes.c_size_t(0)
    _check(L.spec_verify_sampled_commit(None, None, None, None, None, B, V, max_rows,
                                        ctypes.c_float(temperature), ctypes.c_uint64(seed), None,
                                        None, None, None, None, ctypes.byref(need), None),
           "spec_verify_sampled_commit(size)")
    if ws is None or ws.numel() * ws.element_size() < need.value:
        ws = torch.empty(max(need.value, 16), dtype=torch.uint8, device=dev)
    have = ctypes.c_size_t(ws.numel() * ws.element_size())
    rc = L.spec_verify_sampled_commit(
        _dev(target_logits, "target_logits", dtypes=(torch.float32,)),
        _dev(draft_logits, "draft_logits", dtypes=(torch.float32,)),
        _dev(drafts, "drafts", dtypes=_I32), _dev(row_start, "row_start", dtypes=_I32),
        _dev(seq_id, "seq_id", dtypes=_I32), B, V, max_rows, ctypes.c_float(temperature),
        ctypes.c_uint64(seed), _dev(accept_len, "accept_len", dtypes=_I32),
        _dev(out_tokens, "out_tokens", dtypes=_I32), _dev(seq_len, "seq_len", dtypes=_I32),
        _dev(pos_id, "pos_id", dtypes=_I32), _dev(ws, "ws"), ctypes.byref(have),
        _stream(target_logits))
    _check(rc, "spec_verify_sampled_commit")
    return accept_len, out_tokens


def spec_verify_noalloc(target_logits, drafts, row_start, draft_logits=None, seq_id=None,
                        pos0=None, temperature=0.0, seed=0, accept_len=None, out_tokens=None,
                        max_rows=None):
    """spec_verify with the library's own device scratch as workspace (no
    allocation by the library; outputs are allocated here only when not
    given).  Returns (accept_len, out_tokens)."""
    R, V = target_logits.shape
    B = row_start.numel() - 1
    if temperature > 0 and draft_logits is None and R <= B:  # no drafts, no drafter rows
        draft_logits = target_logits.new_empty((0, V))
    _verify_sizes(R, B, drafts, accept_len, out_tokens, V, draft_logits, seq_id, pos0,
                  sampled=temperature > 0)
    drafts, draft_logits = _nonempty(drafts, "drafts"), _nonempty(draft_logits, "draft_logits")
    if max_rows is None:
        max_rows = R
    dev = target_logits.device
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, MAX_OUT), dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        rc = lib().spec_verify_noalloc(
            _dev(target_logits, "target_logits", dtypes=(torch.float32,)),
            _opt(draft_logits, "draft_logits", dtypes=(torch.float32,)),
            _dev(drafts, "drafts", dtypes=_I32), _dev(row_start, "row_start", dtypes=_I32),
            _opt(seq_id, "seq_id", dtypes=_I32), _opt(pos0, "pos0", dtypes=_I32),
            B, V, max_rows, ctypes.c_float(temperature), ctypes.c_uint64(seed),
            _dev(accept_len, "accept_len", dtypes=_I32),
            _dev(out_tokens, "out_tokens", dtypes=_I32), _stream(target_logits))
    _check(rc, "spec_verify_noalloc")
    return accept_len, out_tokens


def spec_verify_margin(target_logits, drafts, row_start, threshold, accept_len=None,
                       out_tokens=None, margins=None, recheck=None, ws=None, max_rows=None):
    """Greedy verify plus the top-2 margin of every target row and, per
    sequence, the first deciding row whose margin is below `threshold`
    (-1 if none).  Returns (accept_len, out_tokens, margins, recheck)."""
    R, V = target_logits.shape
    B = row_start.numel() - 1
    _verify_sizes(R, B, drafts, accept_len, out_tokens)
    _len_at_least(margins, R, "margins")
    _len_at_least(recheck, B, "recheck")
    drafts = _nonempty(drafts, "drafts")
    if max_rows is None:
        max_rows = R
    dev = target_logits.device
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, MAX_OUT), dtype=torch.int32, device=dev)
    if margins is None:
        margins = torch.empty(R, dtype=torch.float32, device=dev)
    if recheck is None:
        recheck = torch.empty(B, dtype=torch.int32, device=dev)
    L = lib()
    need = ctypes.c_size_t(0)
    _check(L.spec_verify_margin(None, None, None, B, V, max_rows, ctypes.c_float(threshold),
                                None, None, None, None, None, ctypes.byref(need), None),
           "spec_verify_margin(size)")
    if ws is None or ws.numel() * ws.element_size() < need.value:
        ws = torch.empty(max(need.value, 16), dtype=torch.uint8, device=dev)
    have = ctypes.c_size_t(ws.numel() * ws.element_size())
    rc = L.spec_verify_margin(_dev(target_logits, "target_logits", dtypes=(torch.float32,)),
                              _dev(drafts, "drafts", dtypes=_I32),
                              _dev(row_start, "row_start", dtypes=_I32), B, V, max_rows,
                              ctypes.c_float(threshold),
                              _dev(accept_len, "accept_len", dtypes=_I32),
                              _dev(out_tokens, "out_tokens", dtypes=_I32),
                              _dev(margins, "margins", dtypes=(torch.float32,)),
                              _dev(recheck, "recheck", dtypes=_I32), _dev(ws, "ws"),
                              ctypes.byref(have), _stream(target_logits))
    _check(rc, "spec_verify_margin")
    return accept_len, out_tokens, margins, recheck


def spec_verify_commit(target_logits, drafts, row_start, seq_len, pos_id, accept_len=None,
                       out_tokens=None, ws=None, max_rows=None):
    """Greedy verify, then the commit of kv_commit (seq_len += accept_len + 1,
    pos_id = seq_len) in the same launches.  Returns (accept_len, out_tokens)."""
    R, V = target_logits.shape
    B = row_start.numel() - 1
    _verify_sizes(R, B, drafts, accept_len, out_tokens)
    _len_at_least(seq_len, B, "seq_len")
    _len_at_least(pos_id, B, "pos_id")
    drafts = _nonempty(drafts, "drafts")
    if max_rows is None:
        max_rows = R
    dev = target_logits.device
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, MAX_OUT), dtype=torch.int32, device=dev)
    L = lib()
    need = ctypes.c_size_t(0)
    _check(L.spec_verify_commit(None, None, None, B, V, max_rows, None, None, None, None, None,
                                ctypes.byref(need), None), "spec_verify_commit(size)")
    if ws is None or ws.numel() * ws.element_size() < need.value:
        ws = torch.empty(max(need.value, 16), dtype=torch.uint8, device=dev)
    have = ctypes.c_size_t(ws.numel() * ws.element_size())
    rc = L.spec_verify_commit(_dev(target_logits, "target_logits", dtypes=(torch.float32,)),
                              _dev(drafts, "drafts", dtypes=_I32),
                              _dev(row_start, "row_start", dtypes=_I32), B, V, max_rows,
                              _dev(accept_len, "accept_len", dtypes=_I32),
                              _dev(out_tokens, "out_tokens", dtypes=_I32),
                              _dev(seq_len, "seq_len", dtypes=_I32),
                              _dev(pos_id, "pos_id", dtypes=_I32), _dev(ws, "ws"),
                              ctypes.byref(have), _stream(target_logits))
    _check(rc, "spec_verify_commit")
    return accept_len, out_tokens


def embed_rows(tokens, table, h=None):
    """h[r] = table[tokens[r]] (bf16 table -> fp32 rows)."""
    rows = tokens.numel()
    V, H = table.shape
    _need(h is None or tuple(h.shape) == (rows, H), "h must be [rows][H]")
    if h is None:
        h = torch.empty((rows, H), dtype=torch.float32, device=table.device)
    _check(lib().embed_rows(_dev(tokens, "tokens", dtypes=_I32), _dev(table, "table", 2),
                            _dev(h, "h", dtypes=(torch.float32,)), rows, V, H, _stream(table)),
           "embed_rows")
    return h


def add_rmsnorm(h, w, eps, d=None, y=None):
    """h += d (if given, in place); y = bf16 RMS-normalised h times w."""
    rows, H = h.shape
    _need(w.numel() == H, "w must hold H entries")
    _need(d is None or tuple(d.shape) == (rows, H), "d must be [rows][H]")
    _need(y is None or tuple(y.shape) == (rows, H), "y must be [rows][H]")
    if y is None:
        y = torch.empty((rows, H), dtype=torch.bfloat16, device=h.device)
    _check(lib().add_rmsnorm(_dev(h, "h", dtypes=(torch.float32,)),
                             _opt(d, "d", dtypes=(torch.float32,)),
                             _dev(w, "w", dtypes=(torch.float32,)), _dev(y, "y", 2), rows, H,
                             ctypes.c_float(eps), _stream(h)), "add_rmsnorm")
    return y


def rope_qkv(qkv, row_start, pos_id, Hq, Hkv, D, theta, q=None, k=None, v=None):
    """Split [q | k | v] rows and rotate q and k; returns fp16 (q, k, v)."""
    rows = qkv.shape[0]
    B = row_start.numel() - 1
    _need(qkv.dim() == 2 and qkv.shape[1] == (Hq + 2 * Hkv) * D, "qkv must be [rows][(Hq + 2 Hkv) D]")
    _need(B >= 1, "row_start must hold B + 1 >= 2 entries")
    _len_at_least(pos_id, B, "pos_id")
    for t, hn, name in ((q, Hq, "q"), (k, Hkv, "k"), (v, Hkv, "v")):
        _need(t is None or tuple(t.shape) == (rows, hn, D), f"{name} must be [rows][{hn}][D]")
    dev_ = qkv.device
    if q is None:
        q = torch.empty((rows, Hq, D), dtype=torch.float16, device=dev_)
    if k is None:
        k = torch.empty((rows, Hkv, D), dtype=torch.float16, device=dev_)
    if v is None:
        v = torch.empty((rows, Hkv, D), dtype=torch.float16, device=dev_)
    _check(lib().rope_qkv(_dev(qkv, "qkv", dtypes=(torch.float32,)),
                          _dev(row_start, "row_start", dtypes=_I32),
                          _dev(pos_id, "pos_id", dtypes=_I32), B, rows, Hq, Hkv, D,
                          ctypes.c_float(theta), _dev(q, "q", 2), _dev(k, "k", 2),
                          _dev(v, "v", 2), _stream(qkv)), "rope_qkv")
    return q, k, v


def silu_mul(gu, F, y=None):
    """y = bf16(silu(g) * u) for rows [g | u] of width 2F."""
    rows = gu.shape[0]
    _need(gu.dim() == 2 and gu.shape[1] == 2 * F, "gu must be [rows][2F]")
    _need(y is None or tuple(y.shape) == (rows, F), "y must be [rows][F]")
    if y is None:
        y = torch.empty((rows, F), dtype=torch.bfloat16, device=gu.device)
    _check(lib().silu_mul(_dev(gu, "gu", dtypes=(torch.float32,)), _dev(y, "y", 2), rows, F,
                          _stream(gu)), "silu_mul")
    return y


def kv_commit(k_pages, v_pages, page_table, seq_len, pos_id, row_start=None, k_new=None,
              v_new=None, accept_len=None):
    num_pages, Hkv, _, D = k_pages.shape
    B, max_pages = page_table.shape
    _len_at_least(seq_len, B, "seq_len")
    _len_at_least(pos_id, B, "pos_id")
    _len_at_least(accept_len, B, "accept_len")
    if accept_len is None:  # APPEND
        _need(row_start is not None and row_start.numel() == B + 1,
              "row_start must hold B + 1 entries (B = table rows)")
        _need(k_new is not None and v_new is not None and k_new.dim() == 3
              and tuple(k_new.shape[1:]) == (Hkv, D) and k_new.shape == v_new.shape,
              "k_new and v_new must be [R][Hkv][D]")
    rc = lib().kv_commit(_dev(k_pages, "k_pages", 2), _dev(v_pages, "v_pages", 2),
                         _dev(page_table, "page_table", dtypes=_I32), max_pages, num_pages,
                         _opt(k_new, "k_new", esize=2), _opt(v_new, "v_new", esize=2),
                         _opt(row_start, "row_start", dtypes=_I32),
                         _dev(seq_len, "seq_len", dtypes=_I32), _dev(pos_id, "pos_id", dtypes=_I32),
                         _opt(accept_len, "accept_len", dtypes=_I32), B, Hkv, D,
                         _stream(k_pages))
    _check(rc, "kv_commit")


def stream_read(buf, sink=None):
    """One plain read of the whole of `buf` (a contiguous GPU tensor whose
    size is a multiple of 16 bytes): the practical HBM read ceiling.
    Returns the sink buffer (pass it back in to avoid an allocation)."""
    nbytes = buf.numel() * buf.element_size()
    words = lib().stream_read_sink_words(nbytes)
    if sink is None or sink.numel() < words:
        sink = torch.empty(max(words, 1), dtype=torch.int32, device=buf.device)
    _check(lib().stream_read(_dev(buf, "buf"), nbytes, _dev(sink, "sink", 4), sink.numel(),
                             _stream(buf)), "stream_read")
    return sink


def version() -> str:
    return lib().isd_version().decode()
