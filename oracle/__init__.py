"""CPU oracle of the compress-then-sparsify attention path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package. The GPU library never calls it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, exact integers for indexer scores, OpenMP
over independent outputs); this module only marshals numpy arrays through ctypes. Every function
cites the passage it follows in ``oracle.c``.

Array conventions (all C-contiguous numpy arrays):
  q        [B, Q, H, D]    float32, or uint16 holding bf16 bits (dtype BF16)
  cache    [B, N, row]     uint8 rows (row = csah row bytes of the format)
  window   [B, w-1+Q, row] uint8 rows; row r holds position pos[b]-(w-1)+r
  idx      [B, Q, k]       int32, -1 = empty slot
  k_codes  [B, N, dI/2]    uint8 E2M1 pairs (element 2j in the low nibble)
  k_scales [B, N, dI/32]   uint8 E8M0
  q_codes  [B, Q, HI, dI/2], q_scales [B, Q, HI, dI/32]
  pos      [B]             int64, position of query 0
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DT_F32, DT_BF16 = 0, 1
FMT_ROW_F32, FMT_ROW_E4M3_BF16, FMT_FP4_E8M0 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile oracle.c with the host C compiler (no GPU toolchain involved)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wno-unused-function", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        sig = {
            "oc_version": (I, []),
            "oc_num_threads": (I, []),
            "oc_e2m1_value": (D, [I]),
            "oc_e2m1_encode": (I, [D]),
            "oc_e8m0_value": (D, [I]),
            "oc_e4m3_value": (D, [I]),
            "oc_e4m3_encode": (I, [D]),
            "oc_bf16_value": (D, [ctypes.c_uint]),
            "oc_bf16_encode": (ctypes.c_uint, [D]),
            "oc_fp4_block_encode": (None, [P, I, P, P]),
            "oc_row_bytes": (I64, [I, I]),
            "oc_encode_rows": (I, [P, I64, I, I, P, P]),
            "oc_decode_rows": (I, [P, P, I64, I, I, P]),
            "oc_kv_compress": (I, [P, I, I64, I, I64, I, I, P, P, P, I, I64, P, P, P]),
            "oc_kv_compress_span": (I, [P, I, I64, I, I64, I, I, I, I64, P, P, P, I, I64, P, P,
                                        P]),
            "oc_kv_compress_rope": (I, [P, I, I64, I, I64, I, I, I, I64, P, P, P, I, I64, P, P,
                                        I, D, P, P]),
            "oc_rope": (I, [P, I, I, I, I, I, I, P, D, I, P]),
            "oc_index_topk": (I, [P, P, I, I, P, P, I64, I64, P, I, I, I, I, P, P, P]),
            "oc_index_scores": (I, [P, P, I, I, P, P, I64, P, P]),
            "oc_csa_attend": (I, [P, I, I, I, P, I, I64, I64, P, I, P, I64, I, P, P, D, I, I, P, P]),
            "oc_hca_attend": (I, [P, I, I, I, P, I, I64, I64, I, P, I64, I, P, P, D, I, I, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (status {rc})")


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().oc_num_threads())


# ------------------------------------------------------------------------------------ codecs
def e2m1_value(code: int) -> float:
    return lib().oc_e2m1_value(int(code))


def e2m1_encode(v: float) -> int:
    return lib().oc_e2m1_encode(float(v))


def e8m0_value(b: int) -> float:
    return lib().oc_e8m0_value(int(b))


def e4m3_value(b: int) -> float:
    return lib().oc_e4m3_value(int(b))


def e4m3_encode(v: float) -> int:
    return lib().oc_e4m3_encode(float(v))


def bf16_value(bits: int) -> float:
    return lib().oc_bf16_value(int(bits))


def bf16_encode(v: float) -> int:
    return lib().oc_bf16_encode(float(v))


def fp4_block_encode(v):
    v = _c(v, np.float64)
    codes = np.zeros(len(v) // 2, np.uint8)
    scale = np.zeros(1, np.uint8)
    lib().oc_fp4_block_encode(_p(v), len(v), _p(codes), _p(scale))
    return codes, int(scale[0])


def row_bytes(fmt: int, D: int) -> int:
    return int(lib().oc_row_bytes(fmt, D))


def encode_rows(x, fmt: int, chunk_rows: int = 1 << 16):
    """x: [..., D] real values -> (rows uint8 [..., row_bytes], scales uint8 [..., D/32] | None).

    Large inputs are converted to fp64 in chunks of ``chunk_rows`` rows.
    """
    x = np.asarray(x)
    D = x.shape[-1]
    lead = x.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    flat = x.reshape(n, D)
    rows = np.zeros((n, row_bytes(fmt, D)), np.uint8)
    scales = np.zeros((n, D // 32), np.uint8) if fmt == FMT_FP4_E8M0 else None
    for r0 in range(0, n, chunk_rows):
        r1 = min(n, r0 + chunk_rows)
        xc = _c(flat[r0:r1], np.float64)
        rc = rows[r0:r1]
        sc = None if scales is None else scales[r0:r1]
        _check(lib().oc_encode_rows(_p(xc), r1 - r0, D, fmt, _p(rc), _p(sc)), "encode_rows")
    rows = rows.reshape(lead + (rows.shape[-1],))
    if scales is not None:
        scales = scales.reshape(lead + (D // 32,))
    return rows, scales


def decode_rows(rows, D: int, fmt: int, scales=None):
    rows = _c(rows, np.uint8)
    lead = rows.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    out = np.zeros(lead + (D,), np.float64)
    sc = None if scales is None else _c(scales, np.uint8)
    _check(lib().oc_decode_rows(_p(rows), _p(sc), n, D, fmt, _p(out)), "decode_rows")
    return out


# ------------------------------------------------------------------------------------ method
def kv_compress(raw, raw_dtype: int, m: int, w, beta, out_fmt: int, span: int | None = None,
                skip: int = 0, tok_pos=None, rope_dims: int = 0, rope_base: float = 10000.0):
    """raw [B, T, D] (float32, or uint16 bf16 bits) -> dict(rows, scales, pre, pi).

    span (default m) tokens per entry at stride m; the first `skip` groups are context only.
    pi is [B, T/m - skip, span] (0 for tokens before the buffer).
    rope_dims > 0: the last rope_dims dims of each pooled entry are turned by RoPE at the position
    of its group's last token, tok_pos[b] + m(g+1) - 1 (tok_pos[b]: position of raw[b, 0]); pre
    then holds the rotated values."""
    raw = _c(raw, np.float32 if raw_dtype == DT_F32 else np.uint16)
    B, T, D = raw.shape
    span = m if span is None else span
    G = T // m - skip
    w = _c(w, np.float32)
    beta = _c(beta, np.float32)
    rows = np.zeros((B, G, row_bytes(out_fmt, D)), np.uint8)
    scales = np.zeros((B, G, D // 32), np.uint8) if out_fmt == FMT_FP4_E8M0 else None
    pre = np.zeros((B, G, D), np.float64)
    pi = np.zeros((B, G, span), np.float64)
    if rope_dims:
        tp = _c(tok_pos, np.int64)
        _check(lib().oc_kv_compress_rope(_p(raw), raw_dtype, T, B, T, D, m, span, skip, _p(w),
                                         _p(beta), _p(rows), out_fmt, G, _p(scales), _p(tp),
                                         rope_dims, float(rope_base), _p(pre), _p(pi)),
               "kv_compress_rope")
    else:
        _check(lib().oc_kv_compress_span(_p(raw), raw_dtype, T, B, T, D, m, span, skip, _p(w),
                                         _p(beta), _p(rows), out_fmt, G, _p(scales), _p(pre),
                                         _p(pi)), "kv_compress")
    return dict(rows=rows, scales=scales, pre=pre, pi=pi)


def rope(x, pos, rope_dims: int, base: float = 10000.0, inverse: bool = False):
    """RoPE of rows x [B, Q, H, D] (float32, or uint16 bf16 bits) -> fp64 [B, Q, H, D].

    Row (b, i, h) sits at position pos[b] + i; its last rope_dims dims turn (inverse: turn back)
    as RoFormer's general form prescribes (see oc_rope)."""
    x = np.ascontiguousarray(x)
    dt = DT_F32 if x.dtype == np.float32 else DT_BF16
    x = _c(x, np.float32 if dt == DT_F32 else np.uint16)
    B, Q, H, D = x.shape
    pos = _c(pos, np.int64)
    out = np.zeros((B, Q, H, D), np.float64)
    _check(lib().oc_rope(_p(x), dt, B, Q, H, D, rope_dims, _p(pos), float(base), int(inverse),
                         _p(out)), "rope")
    return out


def index_topk(q_codes, q_scales, k_codes, k_scales, pos, m: int, k: int, N: int | None = None):
    """Exact top-k per query -> (idx int32 [B,Q,k], scores fp64 [B,Q,k], exact bool [B,Q])."""
    q_codes, q_scales = _c(q_codes, np.uint8), _c(q_scales, np.uint8)
    k_codes, k_scales = _c(k_codes, np.uint8), _c(k_scales, np.uint8)
    pos = _c(pos, np.int64)
    B, Q, HI, half = q_codes.shape
    dI = 2 * half
    Ncap = k_codes.shape[1]
    N = Ncap if N is None else N
    idx = np.zeros((B, Q, k), np.int32)
    sc = np.zeros((B, Q, k), np.float64)
    ex = np.zeros((B, Q), np.int32)
    _check(lib().oc_index_topk(_p(q_codes), _p(q_scales), HI, dI, _p(k_codes), _p(k_scales), Ncap,
                               N, _p(pos), m, B, Q, k, _p(idx), _p(sc), _p(ex)), "index_topk")
    return idx, sc, ex.astype(bool)


def index_scores(q_codes, q_scales, k_codes, k_scales):
    """Exact scores of one query ([HI, dI/2] codes) against n keys ([n, dI/2]) -> (fp64 [n], ok)."""
    q_codes, q_scales = _c(q_codes, np.uint8), _c(q_scales, np.uint8)
    k_codes, k_scales = _c(k_codes, np.uint8), _c(k_scales, np.uint8)
    HI, half = q_codes.shape
    n = k_codes.shape[0]
    s = np.zeros(n, np.float64)
    ok = np.zeros(n, np.int32)
    _check(lib().oc_index_scores(_p(q_codes), _p(q_scales), HI, 2 * half, _p(k_codes),
                                 _p(k_scales), n, _p(s), _p(ok)), "index_scores")
    return s, ok.astype(bool)


def _q_dtype(q):
    return DT_F32 if q.dtype == np.float32 else DT_BF16


def csa_attend(q, cache, fmt: int, idx, win, w: int, pos, sink, scale: float, N: int | None = None):
    """-> (out fp64 [B,Q,H,D], lse fp64 [B,Q,H])."""
    q = np.ascontiguousarray(q)
    B, Q, H, D = q.shape
    cache, idx = _c(cache, np.uint8), _c(idx, np.int32)
    win = _c(win, np.uint8)
    pos = _c(pos, np.int64)
    sink = None if sink is None else _c(sink, np.float32)
    Ncap = cache.shape[1]
    N = Ncap if N is None else N
    out = np.zeros((B, Q, H, D), np.float64)
    lse = np.zeros((B, Q, H), np.float64)
    _check(lib().oc_csa_attend(_p(q), _q_dtype(q), H, D, _p(cache), fmt, Ncap, N, _p(idx),
                               idx.shape[-1], _p(win), win.shape[1], w, _p(pos), _p(sink),
                               float(scale), B, Q, _p(out), _p(lse)), "csa_attend")
    return out, lse


def hca_attend(q, cache, fmt: int, m: int, win, w: int, pos, sink, scale: float,
               N: int | None = None):
    q = np.ascontiguousarray(q)
    B, Q, H, D = q.shape
    cache = _c(cache, np.uint8)
    win = _c(win, np.uint8)
    pos = _c(pos, np.int64)
    sink = None if sink is None else _c(sink, np.float32)
    Ncap = cache.shape[1]
    N = Ncap if N is None else N
    out = np.zeros((B, Q, H, D), np.float64)
    lse = np.zeros((B, Q, H), np.float64)
    _check(lib().oc_hca_attend(_p(q), _q_dtype(q), H, D, _p(cache), fmt, Ncap, N, m, _p(win),
                               win.shape[1], w, _p(pos), _p(sink), float(scale), B, Q, _p(out),
                               _p(lse)), "hca_attend")
    return out, lse
