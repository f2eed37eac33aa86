"""Python binding of libcsah (include/csah.h): compress-then-sparsify attention on MI355X.

Argument marshalling only. Every step runs in the library's HIP kernels; torch is used to hold
device memory and to name the current stream. If the library is missing, every call raises.

Tensor conventions (device tensors, C-contiguous unless a stride argument says otherwise):
  raw        [B, T, D] float32 or bfloat16 tokens
  rows       [B, S, row_bytes(fmt, D)] uint8 cache rows; scales [B, S, D/32] uint8 (FP4 only)
  q          [B, Q, H, D] bfloat16 or float32
  idx        [B, Q, k] int32;  pos [B] int64 (position of query 0)
  window     [B, w-1+Q, row_bytes] uint8
Paged caches (the *_paged calls):
  pool       [pages, page_size, row_bytes] uint8 (any shape whose rows are contiguous and whose
             last dim is the row width); scale pool [pages, page_size, D/32] uint8 (FP4 only)
  block_table [B, >= ceil(N / page_size)] int32: entry e of sequence b is row
             block_table[b, e // page_size] * page_size + e % page_size of the pool
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsah.so")

OK, INVALID_ARGUMENT, UNSUPPORTED, WORKSPACE_TOO_SMALL, LAUNCH = 0, -1, -2, -3, -4
SCRATCH_LIMIT = -5
NOALLOC_SCRATCH_BYTES = 32 << 20  # csah_csa_attend_noalloc's static scratch per GPU
DT_F32, DT_BF16 = 0, 1
FMT_ROW_F32, FMT_ROW_E4M3_BF16, FMT_FP4_E8M0 = 0, 1, 2

EXPORTS = ("csah_abi_version", "csah_status_string", "csah_row_bytes", "csah_kv_compress",
           "csah_kv_compress_span",
           "csah_index_topk_workspace", "csah_index_topk", "csah_attend_workspace",
           "csah_csa_attend", "csah_csa_attend_noalloc", "csah_hca_attend",
           "csah_kv_compress_paged",
           "csah_index_topk_paged", "csah_csa_attend_paged", "csah_hca_attend_paged",
           "csah_rope", "csah_kv_compress_rope", "csah_kv_compress_paged_rope",
           "csah_profile_next_call")

_lib = None


class CsahError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


def lib():
    """Load libcsah.so (built by build.py); raise if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python long_context_attention_03_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, F, SZ = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
        D = ctypes.c_double
        sig = {
            "csah_abi_version": (I, []),
            "csah_status_string": (ctypes.c_char_p, [I]),
            "csah_row_bytes": (I64, [I, I]),
            "csah_kv_compress": (I, [P, I, I64, I, I64, I, I, P, P, P, I, I64, P, P]),
            "csah_kv_compress_span": (I, [P, I, I64, I, I64, I, I, I, I64, P, P, P, I, I64, P,
                                          P]),
            "csah_index_topk_workspace": (SZ, [I, I, I64, I, I, I]),
            "csah_index_topk": (I, [P, P, I, I, P, P, I64, I64, P, I, I, I, I, P, P, P, SZ, P]),
            "csah_attend_workspace": (SZ, [I, I, I, I, I64]),
            "csah_csa_attend": (I, [P, I, I, I, P, I, I64, I64, P, I, P, I64, I, P, P, F, I, I,
                                    P, P, P, SZ, P]),
            "csah_hca_attend": (I, [P, I, I, I, P, I, I64, I64, I, P, I64, I, P, P, F, I, I, P,
                                    P, P, SZ, P]),
            "csah_csa_attend_noalloc": (I, [P, I, I, I, P, I, I64, I64, P, I, P, I64, I, P, P, F,
                                            I, I, P, P, P]),
            "csah_kv_compress_paged": (I, [P, I, I64, I, I64, I, I, I, I64, P, P, P, I, P, P,
                                           I64, I, I64, P]),
            "csah_index_topk_paged": (I, [P, P, I, I, P, P, P, I64, I, I64, P, I, I, I, I, P, P,
                                          P, SZ, P]),
            "csah_csa_attend_paged": (I, [P, I, I, I, P, I, P, I64, I, I64, P, I, P, I64, I, P,
                                          P, F, I, I, P, P, P, SZ, P]),
            "csah_hca_attend_paged": (I, [P, I, I, I, P, I, P, I64, I, I64, I, P, I64, I, P, P,
                                          F, I, I, P, P, P, SZ, P]),
            "csah_rope": (I, [P, I, I, I, I, I, I, P, D, I, P]),
            "csah_kv_compress_rope": (I, [P, I, I64, I, I64, I, I, I, I64, P, P, P, I, I64, P,
                                          P, I, D, P]),
            "csah_kv_compress_paged_rope": (I, [P, I, I64, I, I64, I, I, I, I64, P, P, P, I, P,
                                                P, I64, I, I64, P, I, D, P]),
            "csah_profile_next_call": (I, [P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().csah_status_string(int(status)).decode()


def profile_next_call(begin, end):
    """Record torch.cuda.Events ``begin``/``end`` around the next call's dominant kernel.

    Both events must already exist on the device (record them once beforehand).
    """
    st = lib().csah_profile_next_call(ctypes.c_void_p(begin.cuda_event),
                                      ctypes.c_void_p(end.cuda_event))
    _check("csah_profile_next_call", st)


def row_bytes(fmt: int, D: int) -> int:
    return int(lib().csah_row_bytes(fmt, D))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, st):
    if st != OK:
        raise CsahError(fn, st)


def _dt(t):
    if t.dtype == torch.float32:
        return DT_F32
    if t.dtype == torch.bfloat16:
        return DT_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _rows_dense(t) -> bool:
    """A [B, n, ...] tensor whose rows (the dims after the second) are densely packed, one after
    another along dim 1, while dim 0 (the sequence) may have any stride that is a whole number of
    rows: a sequence slice of a larger cache. The library takes that stride in rows."""
    if t.dim() < 2:
        return t.is_contiguous()
    row = 1
    for size, stride in zip(reversed(t.shape[2:]), reversed(t.stride()[2:])):
        if size > 1 and stride != row:
            return False
        row *= size
    if t.stride(1) != row:
        return False
    return t.shape[0] <= 1 or t.stride(0) % row == 0


def _validate(dev, *items):
    """Check arguments before their raw pointers are taken. items: (tensor or None, name, dtypes,
    layout), layout "dense" (contiguous) or "rows" (see _rows_dense). Dtypes are checked for every
    argument first, then the device, then the layout the kernels address."""
    items = [it for it in items if it[0] is not None]
    for t, name, dtypes, _ in items:
        if t.dtype not in dtypes:
            raise TypeError(f"{name}: dtype {t.dtype}, expected {' or '.join(map(str, dtypes))}")
    for t, name, _, _ in items:
        if t.device.type != "cuda":
            raise ValueError(f"{name}: a GPU tensor is required (got {t.device})")
        if t.device != dev:
            raise ValueError(f"{name}: on {t.device}, the call runs on {dev}")
    for t, name, _, layout in items:
        if layout == "dense" and not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous")
        if layout == "rows" and not _rows_dense(t):
            raise ValueError(f"{name}: rows must be packed (only the sequence dim may be strided)")


_U8 = (torch.uint8,)
_I32 = (torch.int32,)
_I64 = (torch.int64,)
_F32 = (torch.float32,)
_QDT = (torch.bfloat16, torch.float32)


def _check_attend_args(q, cache, cache_layout, idx, window, w, pos, sink, out, lse):
    _validate(q.device, (q, "q", _QDT, "dense"), (cache, "cache", _U8, cache_layout),
              (idx, "idx", _I32, "dense"), (window if w > 0 else None, "window", _U8, "rows"),
              (pos, "pos", _I64, "dense"), (sink, "sink", _F32, "dense"),
              (out, "out", _F32, "dense"), (lse, "lse", _F32, "dense"))


def _check_index_args(q_codes, q_scales, k_codes, k_scales, k_layout, pos, idx_out, score_out):
    _validate(q_codes.device, (q_codes, "q_codes", _U8, "dense"),
              (q_scales, "q_scales", _U8, "dense"), (k_codes, "k_codes", _U8, k_layout),
              (k_scales, "k_scales", _U8, k_layout), (pos, "pos", _I64, "dense"),
              (idx_out, "idx_out", _I32, "dense"), (score_out, "score_out", _F32, "dense"))
    if k_layout == "rows" and k_codes.dim() == 3 and k_scales.dim() == 3 and k_codes.shape[0] > 1 \
            and k_codes.stride(0) // k_codes.stride(1) != k_scales.stride(0) // k_scales.stride(1):
        raise ValueError("k_codes and k_scales must have the same sequence stride in rows")


def _workspace(nbytes: int, device, ws=None):
    if nbytes == 0:
        return None
    if ws is not None and ws.numel() >= nbytes:
        return ws
    # 256-byte alignment: torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------- kv_compress
def kv_compress(raw, m: int, w, beta, out_fmt: int, out_rows=None, out_scales=None, stream=None,
                span: int | None = None, skip: int = 0):
    """Pool every m tokens of raw [B, T, D] into one encoded entry.

    With ``span`` (> m) each entry pools the span tokens ending with its group's last token
    (beta has span values) and the first ``skip`` groups are context only.
    Returns (rows [B, T/m - skip, row_bytes], scales [B, T/m - skip, D/32] or None). When
    ``out_rows`` is given it may be a slice of a larger cache (its sequence stride is taken from
    dim 0).
    """
    B, T, D = raw.shape
    G = T // m - skip
    if out_rows is None:
        out_rows = torch.empty((B, G, row_bytes(out_fmt, D)), dtype=torch.uint8, device=raw.device)
        if out_fmt == FMT_FP4_E8M0:
            out_scales = torch.empty((B, G, D // 32), dtype=torch.uint8, device=raw.device)
    out_stride = out_rows.stride(0) // out_rows.stride(1)
    if span is None and skip == 0:
        st = lib().csah_kv_compress(_ptr(raw), _dt(raw), raw.stride(0) // raw.stride(1), B, T, D,
                                    m, _ptr(w), _ptr(beta), _ptr(out_rows), out_fmt, out_stride,
                                    _ptr(out_scales), _stream(stream))
        _check("csah_kv_compress", st)
    else:
        st = lib().csah_kv_compress_span(_ptr(raw), _dt(raw), raw.stride(0) // raw.stride(1), B,
                                         T, D, m, m if span is None else span, skip, _ptr(w),
                                         _ptr(beta), _ptr(out_rows), out_fmt, out_stride,
                                         _ptr(out_scales), _stream(stream))
        _check("csah_kv_compress_span", st)
    return out_rows, out_scales


# ----------------------------------------------------------------------------- index_topk
def index_topk_workspace(B: int, Q: int, N: int, k: int, HI: int, dI: int) -> int:
    return int(lib().csah_index_topk_workspace(B, Q, N, k, HI, dI))


def index_topk(q_codes, q_scales, k_codes, k_scales, pos, m: int, k: int, N: int | None = None,
               want_scores: bool = True, ws=None, idx_out=None, score_out=None, stream=None):
    """Top-k entries per query -> (idx int32 [B, Q, k], scores fp32 [B, Q, k] or None)."""
    _check_index_args(q_codes, q_scales, k_codes, k_scales, "rows", pos, idx_out, score_out)
    B, Q, HI, half = q_codes.shape
    dI = 2 * half
    kstride = k_codes.stride(0) // k_codes.stride(1)
    N = k_codes.shape[1] if N is None else N
    dev = q_codes.device
    if idx_out is None:
        idx_out = torch.empty((B, Q, k), dtype=torch.int32, device=dev)
    if want_scores and score_out is None:
        score_out = torch.empty((B, Q, k), dtype=torch.float32, device=dev)
    need = index_topk_workspace(B, Q, N, k, HI, dI)
    ws = _workspace(need, dev, ws)
    st = lib().csah_index_topk(_ptr(q_codes), _ptr(q_scales), HI, dI, _ptr(k_codes),
                               _ptr(k_scales), kstride, N, _ptr(pos), m, B, Q, k, _ptr(idx_out),
                               _ptr(score_out), _ptr(ws), need, _stream(stream))
    _check("csah_index_topk", st)
    return idx_out, score_out


# ----------------------------------------------------------------------------- attention
def attend_workspace(B: int, Q: int, H: int, D: int, max_rows: int) -> int:
    return int(lib().csah_attend_workspace(B, Q, H, D, max_rows))


def _fmt_of(rows, D):
    rb = rows.shape[-1]
    if rb == row_bytes(FMT_ROW_E4M3_BF16, D):
        return FMT_ROW_E4M3_BF16
    if rb == row_bytes(FMT_ROW_F32, D):
        return FMT_ROW_F32
    raise ValueError(f"row width {rb} matches no row format at D={D}")


def csa_attend(q, cache, idx, window, w: int, pos, sink, scale: float, N: int | None = None,
               ws=None, out=None, lse=None, stream=None):
    """Sparse attention over cache rows idx + window + sink -> (out fp32 [B,Q,H,D], lse [B,Q,H])."""
    _check_attend_args(q, cache, "rows", idx, window, w, pos, sink, out, lse)
    B, Q, H, D = q.shape
    fmt = _fmt_of(cache, D)
    N = cache.shape[1] if N is None else N
    k = idx.shape[-1]
    dev = q.device
    out = torch.empty((B, Q, H, D), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, Q, H), dtype=torch.float32, device=dev) if lse is None else lse
    need = attend_workspace(B, Q, H, D, k + w)
    ws = _workspace(need, dev, ws)
    wstride = window.stride(0) // window.stride(1) if w > 0 else 0
    st = lib().csah_csa_attend(_ptr(q), _dt(q), H, D, _ptr(cache), fmt,
                               cache.stride(0) // cache.stride(1), N, _ptr(idx), k,
                               _ptr(window) if w > 0 else None, wstride, w, _ptr(pos), _ptr(sink),
                               float(scale), B, Q, _ptr(out), _ptr(lse), _ptr(ws), need,
                               _stream(stream))
    _check("csah_csa_attend", st)
    return out, lse


def csa_attend_noalloc(q, cache, idx, window, w: int, pos, sink, scale: float,
                       N: int | None = None, out=None, lse=None, stream=None):
    """csa_attend whose partials use the library's static scratch (no workspace, no allocation
    inside the call); out / lse may be passed preallocated."""
    _check_attend_args(q, cache, "rows", idx, window, w, pos, sink, out, lse)
    B, Q, H, D = q.shape
    fmt = _fmt_of(cache, D)
    N = cache.shape[1] if N is None else N
    k = idx.shape[-1]
    dev = q.device
    out = torch.empty((B, Q, H, D), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, Q, H), dtype=torch.float32, device=dev) if lse is None else lse
    wstride = window.stride(0) // window.stride(1) if w > 0 else 0
    st = lib().csah_csa_attend_noalloc(_ptr(q), _dt(q), H, D, _ptr(cache), fmt,
                                       cache.stride(0) // cache.stride(1), N, _ptr(idx), k,
                                       _ptr(window) if w > 0 else None, wstride, w, _ptr(pos),
                                       _ptr(sink), float(scale), B, Q, _ptr(out), _ptr(lse),
                                       _stream(stream))
    _check("csah_csa_attend_noalloc", st)
    return out, lse


def hca_attend(q, cache, m: int, window, w: int, pos, sink, scale: float, N: int | None = None,
               ws=None, out=None, lse=None, stream=None):
    """Dense attention over every visible entry + window + sink -> (out, lse)."""
    _check_attend_args(q, cache, "rows", None, window, w, pos, sink, out, lse)
    B, Q, H, D = q.shape
    fmt = _fmt_of(cache, D)
    N = cache.shape[1] if N is None else N
    dev = q.device
    out = torch.empty((B, Q, H, D), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, Q, H), dtype=torch.float32, device=dev) if lse is None else lse
    need = attend_workspace(B, Q, H, D, N + w)
    ws = _workspace(need, dev, ws)
    wstride = window.stride(0) // window.stride(1) if w > 0 else 0
    st = lib().csah_hca_attend(_ptr(q), _dt(q), H, D, _ptr(cache), fmt,
                               cache.stride(0) // cache.stride(1), N, m,
                               _ptr(window) if w > 0 else None, wstride, w, _ptr(pos), _ptr(sink),
                               float(scale), B, Q, _ptr(out), _ptr(lse), _ptr(ws), need,
                               _stream(stream))
    _check("csah_hca_attend", st)
    return out, lse


# ----------------------------------------------------------------------------- paged caches
def _table(block_table):
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
        raise TypeError("block_table must be an int32 [B, pages] tensor with contiguous rows")
    return _ptr(block_table), block_table.stride(0)


def kv_compress_paged(raw, m: int, w, beta, out_fmt: int, pool, block_table, page_size: int,
                      first_entry: int = 0, scale_pool=None, span: int | None = None,
                      skip: int = 0, stream=None):
    """kv_compress writing entry g of sequence b to its logical entry first_entry + g of a paged
    cache (pool / scale_pool rows through block_table). Returns (pool, scale_pool)."""
    B, T, D = raw.shape
    tp, ts = _table(block_table)
    st = lib().csah_kv_compress_paged(_ptr(raw), _dt(raw), raw.stride(0) // raw.stride(1), B, T,
                                      D, m, m if span is None else span, skip, _ptr(w),
                                      _ptr(beta), _ptr(pool), out_fmt, _ptr(scale_pool), tp, ts,
                                      page_size, first_entry, _stream(stream))
    _check("csah_kv_compress_paged", st)
    return pool, scale_pool


def index_topk_paged(q_codes, q_scales, k_pool_codes, k_pool_scales, block_table,
                     page_size: int, N: int, pos, m: int, k: int, want_scores: bool = True,
                     ws=None, idx_out=None, score_out=None, stream=None):
    """index_topk over FP4 keys in a paged pool -> (logical idx [B, Q, k], scores or None)."""
    _check_index_args(q_codes, q_scales, k_pool_codes, k_pool_scales, "dense", pos, idx_out,
                      score_out)
    B, Q, HI, half = q_codes.shape
    dI = 2 * half
    dev = q_codes.device
    tp, ts = _table(block_table)
    if idx_out is None:
        idx_out = torch.empty((B, Q, k), dtype=torch.int32, device=dev)
    if want_scores and score_out is None:
        score_out = torch.empty((B, Q, k), dtype=torch.float32, device=dev)
    need = index_topk_workspace(B, Q, N, k, HI, dI)
    ws = _workspace(need, dev, ws)
    st = lib().csah_index_topk_paged(_ptr(q_codes), _ptr(q_scales), HI, dI, _ptr(k_pool_codes),
                                     _ptr(k_pool_scales), tp, ts, page_size, N, _ptr(pos), m, B,
                                     Q, k, _ptr(idx_out), _ptr(score_out), _ptr(ws), need,
                                     _stream(stream))
    _check("csah_index_topk_paged", st)
    return idx_out, score_out


def csa_attend_paged(q, cache_pool, block_table, page_size: int, N: int, idx, window, w: int,
                     pos, sink, scale: float, ws=None, out=None, lse=None, stream=None):
    """csa_attend with the compressed cache in a paged pool (idx: logical entries)."""
    _check_attend_args(q, cache_pool, "dense", idx, window, w, pos, sink, out, lse)
    B, Q, H, D = q.shape
    fmt = _fmt_of(cache_pool, D)
    k = idx.shape[-1]
    dev = q.device
    tp, ts = _table(block_table)
    out = torch.empty((B, Q, H, D), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, Q, H), dtype=torch.float32, device=dev) if lse is None else lse
    need = attend_workspace(B, Q, H, D, k + w)
    ws = _workspace(need, dev, ws)
    wstride = window.stride(0) // window.stride(1) if w > 0 else 0
    st = lib().csah_csa_attend_paged(_ptr(q), _dt(q), H, D, _ptr(cache_pool), fmt, tp, ts,
                                     page_size, N, _ptr(idx), k,
                                     _ptr(window) if w > 0 else None, wstride, w, _ptr(pos),
                                     _ptr(sink), float(scale), B, Q, _ptr(out), _ptr(lse),
                                     _ptr(ws), need, _stream(stream))
    _check("csah_csa_attend_paged", st)
    return out, lse


def hca_attend_paged(q, cache_pool, block_table, page_size: int, N: int, m: int, window, w: int,
                     pos, sink, scale: float, ws=None, out=None, lse=None, stream=None):
    """hca_attend with the compressed cache in a paged pool."""
    _check_attend_args(q, cache_pool, "dense", None, window, w, pos, sink, out, lse)
    B, Q, H, D = q.shape
    fmt = _fmt_of(cache_pool, D)
    dev = q.device
    tp, ts = _table(block_table)
    out = torch.empty((B, Q, H, D), dtype=torch.float32, device=dev) if out is None else out
    lse = torch.empty((B, Q, H), dtype=torch.float32, device=dev) if lse is None else lse
    need = attend_workspace(B, Q, H, D, N + w)
    ws = _workspace(need, dev, ws)
    wstride = window.stride(0) // window.stride(1) if w > 0 else 0
    st = lib().csah_hca_attend_paged(_ptr(q), _dt(q), H, D, _ptr(cache_pool), fmt, tp, ts,
                                     page_size, N, m, _ptr(window) if w > 0 else None, wstride,
                                     w, _ptr(pos), _ptr(sink), float(scale), B, Q, _ptr(out),
                                     _ptr(lse), _ptr(ws), need, _stream(stream))
    _check("csah_hca_attend_paged", st)
    return out, lse


# ----------------------------------------------------------------------------- RoPE
def rope(x, pos, rope_dims: int = 64, base: float = 10000.0, inverse: bool = False, stream=None):
    """Turn the last ``rope_dims`` dims of rows x [B, Q, H, D] (bfloat16 or float32, contiguous)
    in place: row group (b, i) at position pos[b] + i; ``inverse`` turns back. Returns x."""
    if not x.is_contiguous():
        raise ValueError("rope needs a contiguous [B, Q, H, D] tensor")
    B, Q, H, D = x.shape
    st = lib().csah_rope(_ptr(x), _dt(x), B, Q, H, D, rope_dims, _ptr(pos), float(base),
                         int(bool(inverse)), _stream(stream))
    _check("csah_rope", st)
    return x


def kv_compress_rope(raw, m: int, w, beta, out_fmt: int, tok_pos, rope_dims: int = 64,
                     rope_base: float = 10000.0, out_rows=None, out_scales=None,
                     span: int | None = None, skip: int = 0, stream=None):
    """kv_compress whose pooled entries are turned by RoPE before encoding: the entry of raw's
    group g sits at tok_pos[b] + m(g+1) - 1 (tok_pos [B] int64: position of raw[b, 0])."""
    B, T, D = raw.shape
    G = T // m - skip
    if out_rows is None:
        out_rows = torch.empty((B, G, row_bytes(out_fmt, D)), dtype=torch.uint8, device=raw.device)
        if out_fmt == FMT_FP4_E8M0:
            out_scales = torch.empty((B, G, D // 32), dtype=torch.uint8, device=raw.device)
    st = lib().csah_kv_compress_rope(_ptr(raw), _dt(raw), raw.stride(0) // raw.stride(1), B, T,
                                     D, m, m if span is None else span, skip, _ptr(w),
                                     _ptr(beta), _ptr(out_rows), out_fmt,
                                     out_rows.stride(0) // out_rows.stride(1), _ptr(out_scales),
                                     _ptr(tok_pos), rope_dims, float(rope_base), _stream(stream))
    _check("csah_kv_compress_rope", st)
    return out_rows, out_scales


def kv_compress_paged_rope(raw, m: int, w, beta, out_fmt: int, pool, block_table,
                           page_size: int, tok_pos, rope_dims: int = 64,
                           rope_base: float = 10000.0, first_entry: int = 0, scale_pool=None,
                           span: int | None = None, skip: int = 0, stream=None):
    """kv_compress_paged with the RoPE of kv_compress_rope. Returns (pool, scale_pool)."""
    B, T, D = raw.shape
    tp, ts = _table(block_table)
    st = lib().csah_kv_compress_paged_rope(_ptr(raw), _dt(raw), raw.stride(0) // raw.stride(1),
                                           B, T, D, m, m if span is None else span, skip,
                                           _ptr(w), _ptr(beta), _ptr(pool), out_fmt,
                                           _ptr(scale_pool), tp, ts, page_size, first_entry,
                                           _ptr(tok_pos), rope_dims, float(rope_base),
                                           _stream(stream))
    _check("csah_kv_compress_paged_rope", st)
    return pool, scale_pool
