"""CPU oracle of the blockwise Sparse GQA path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package. It wraps ``liboracle.so`` (built from ``sgqa_oracle.c`` by ``oracle/build.py``) with
ctypes and numpy; it never imports the HIP library and the HIP library never imports it.

Every function takes host numpy arrays (bf16 tensors as ``uint16`` bit patterns) and returns
numpy arrays. The definitions and their sources are documented in ``sgqa_oracle.c``
("Inside Step 5 Preview", section "Sparse GQA" and Figure 3).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _build

            _build.build()
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_to_f64.restype = D
        lib.orc_f64_to_bf16.argtypes = [D]
        lib.orc_f64_to_bf16.restype = ctypes.c_uint16
        lib.orc_compress.argtypes = [I, I, I, I, P, P]
        lib.orc_compress.restype = None
        lib.orc_block_scores.argtypes = [I, I, P, P, P, I, P]
        lib.orc_block_scores.restype = None
        lib.orc_select.argtypes = [I, P, I, P]
        lib.orc_select.restype = None
        lib.orc_index_topk.argtypes = [I, I, I, I, I, I, P, P, P, I, P, P]
        lib.orc_index_topk.restype = None
        lib.orc_scored_pairs.argtypes = [I, I]
        lib.orc_scored_pairs.restype = ctypes.c_longlong
        lib.orc_union.argtypes = [I, I, I, I, I, P, P, P]
        lib.orc_union.restype = None
        lib.orc_attend.argtypes = [I, I, I, I, I, I, D, P, P, P, P, I, P, P]
        lib.orc_attend.restype = None
        lib.orc_attend_bwd.argtypes = [I, I, I, I, I, I, D, P, P, P, P, P, P, P, P]
        lib.orc_attend_bwd.restype = None
        lib.orc_attend_bwd_part.argtypes = [I, I, I, I, I, I, D, P, P, P, P, P, I, P, P, I, I, I, P, P]
        lib.orc_attend_bwd_part.restype = None
        lib.orc_attend_sel.argtypes = [I, I, I, I, I, I, D, P, P, P, P, I, P, P]
        lib.orc_attend_sel.restype = None
        lib.orc_decode.argtypes = [I, I, I, I, I, I, I, I, I, D, P, P, P, P, P, P, I, P, P, P]
        lib.orc_decode.restype = None
        lib.orc_decode_f8.argtypes = [I, I, I, I, I, I, I, I, I, D, P, P, P, P, P, P, P, I, P, P, P]
        lib.orc_decode_f8.restype = None
        lib.orc_fp8_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        lib.orc_fp8_e4m3_to_f64.restype = ctypes.c_double
        lib.orc_coverage.argtypes = [I, I, I, I, I, P, P, I]
        lib.orc_coverage.restype = D
        _lib = lib
    return _lib


def _u16(a) -> np.ndarray:
    """Host uint16 view of a bf16 array (numpy uint16/int16, or a torch bfloat16 tensor)."""
    if hasattr(a, "detach"):  # torch tensor
        import torch

        a = a.detach()
        if a.dtype == torch.bfloat16:
            a = a.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        else:
            raise TypeError(f"expected bfloat16 tensor, got {a.dtype}")
    a = np.ascontiguousarray(a)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"expected uint16 bf16 bits, got {a.dtype}")
    return a


def _u8(a) -> np.ndarray:
    """Host uint8 codes of an FP8 array (numpy uint8, or a torch uint8 / float8 tensor)."""
    if hasattr(a, "detach"):
        import torch

        a = a.detach().cpu().contiguous()
        if a.dtype != torch.uint8:
            a = a.view(torch.uint8)
        a = a.numpy()
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint8:
        raise TypeError(f"expected uint8 FP8 codes, got {a.dtype}")
    return a


def _f32(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def bf16_to_f64(bits: int) -> float:
    return _load().orc_bf16_to_f64(int(bits))


def f64_to_bf16(x: float) -> int:
    """Nearest bf16 (ties to even) of a double, as a bit pattern."""
    return int(_load().orc_f64_to_bf16(float(x)))


def compress(ki, block: int) -> np.ndarray:
    """Block keys: ki [S][N][dI] or [N][dI] bf16 -> [S][N//B][dI] (or [N//B][dI]) bf16 bits."""
    ki = _u16(ki)
    squeeze = ki.ndim == 2
    if squeeze:
        ki = ki[None]
    S, N, dI = ki.shape
    out = np.empty((S, N // block, dI), dtype=np.uint16)
    _load().orc_compress(S, N, dI, block, _p(ki), _p(out))
    return out[0] if squeeze else out


def block_scores(qi_row, w_row, kbar, nc: int) -> np.ndarray:
    """fp64 scores of one (query, group) row: qi_row [HI][dI], w_row [HI], kbar [>=nc][dI]."""
    qi_row = _u16(qi_row)
    w_row = _f32(w_row)
    kbar = _u16(kbar)
    HI, dI = qi_row.shape
    out = np.empty(max(nc, 1), dtype=np.float64)
    _load().orc_block_scores(HI, dI, _p(qi_row), _p(w_row), _p(kbar), nc, _p(out))
    return out[:nc]


def select(scores, kb: int) -> np.ndarray:
    """First min(kb, n) candidates by (score desc, id asc), ascending ids, -1 padded to kb."""
    s = np.ascontiguousarray(scores, dtype=np.float64)
    out = np.empty(kb, dtype=np.int32)
    _load().orc_select(int(s.shape[0]), _p(s), kb, _p(out))
    return out


def index_topk(qi, w, kbar, block: int, kb: int, rows=None) -> np.ndarray:
    """Sel(i,g): qi [N][G][HI][dI], w [G][HI], kbar [N//B][dI] -> [G][len(rows)][kb] int32."""
    qi = _u16(qi)
    w = _f32(w)
    kbar = _u16(kbar)
    N, G, HI, dI = qi.shape
    if rows is None:
        nrows, rp = N, None
    else:
        rows = _i32(rows)
        nrows, rp = int(rows.shape[0]), _p(rows)
    out = np.empty((G, nrows, kb), dtype=np.int32)
    _load().orc_index_topk(N, G, HI, dI, block, kb, _p(qi), _p(w), _p(kbar), nrows, rp, _p(out))
    return out


def scored_pairs(n_tokens: int, block: int) -> int:
    """sum_i floor(i/B): (query, candidate) pairs the indexer scores per group."""
    return int(_load().orc_scored_pairs(n_tokens, block))


def union(topk, n_tokens: int, block: int, tile: int):
    """topk [G][N][kb] -> (umask [G][T][W] uint32, ucount [G][T] int32)."""
    topk = _i32(topk)
    G, N, kb = topk.shape
    assert N == n_tokens
    T = (N + tile - 1) // tile
    nbc = (N + block - 1) // block
    W = (nbc + 31) // 32
    umask = np.empty((G, T, W), dtype=np.uint32)
    ucount = np.empty((G, T), dtype=np.int32)
    _load().orc_union(N, G, block, kb, tile, _p(topk), _p(umask), _p(ucount))
    return umask, ucount


def attend(q, k, v, umask, block: int, tile: int, scale: float = 0.0, rows=None) -> np.ndarray:
    """q [N][Hq][D], k/v [G][N][D] bf16, umask [G][T][W] -> out [len(rows)][Hq][D] fp64."""
    q = _u16(q)
    k = _u16(k)
    v = _u16(v)
    umask = np.ascontiguousarray(umask, dtype=np.uint32)
    N, Hq, D = q.shape
    G = k.shape[0]
    if rows is None:
        nrows, rp = N, None
    else:
        rows = _i32(rows)
        nrows, rp = int(rows.shape[0]), _p(rows)
    out = np.empty((nrows, Hq, D), dtype=np.float64)
    _load().orc_attend(N, Hq, G, D, block, tile, float(scale), _p(q), _p(k), _p(v), _p(umask), nrows, rp, _p(out))
    return out


def attend_bwd(q, k, v, umask, dout, block: int, tile: int, scale: float = 0.0):
    """Gradient of attend(): q/dout [N][Hq][D], k/v [G][N][D] bf16, umask [G][T][W]
    -> (dq [N][Hq][D], dk [G][N][D], dv [G][N][D]) fp64."""
    q = _u16(q)
    k = _u16(k)
    v = _u16(v)
    dout = _u16(dout)
    umask = np.ascontiguousarray(umask, dtype=np.uint32)
    N, Hq, D = q.shape
    G = k.shape[0]
    dq = np.empty((N, Hq, D), dtype=np.float64)
    dk = np.empty((G, N, D), dtype=np.float64)
    dv = np.empty((G, N, D), dtype=np.float64)
    _load().orc_attend_bwd(N, Hq, G, D, block, tile, float(scale), _p(q), _p(k), _p(v), _p(umask), _p(dout),
                           _p(dq), _p(dk), _p(dv))
    return dq, dk, dv


def attend_bwd_part(q, k, v, umask, dout, block: int, tile: int, rows, g0: int, key_lo: int, key_hi: int,
                    scale: float = 0.0):
    """attend_bwd() on a subset: dq of the listed rows [len(rows)][Hq][D], and dk, dv of group g0's
    keys key_lo .. key_hi - 1 [key_hi - key_lo][D] over every row that attends them (fp64)."""
    q = _u16(q)
    k = _u16(k)
    v = _u16(v)
    dout = _u16(dout)
    umask = np.ascontiguousarray(umask, dtype=np.uint32)
    rows = _i32(rows)
    N, Hq, D = q.shape
    G = k.shape[0]
    assert 0 <= g0 < G and 0 <= key_lo <= key_hi <= N
    nr = int(rows.shape[0])
    dq = np.empty((nr, Hq, D), dtype=np.float64)
    nk = key_hi - key_lo
    dk = np.empty((max(nk, 1), D), dtype=np.float64)
    dv = np.empty((max(nk, 1), D), dtype=np.float64)
    _load().orc_attend_bwd_part(N, Hq, G, D, block, tile, float(scale), _p(q), _p(k), _p(v), _p(umask), _p(dout),
                                nr, _p(rows), _p(dq), g0, key_lo, key_hi, _p(dk), _p(dv))
    return dq, dk[:nk], dv[:nk]


def attend_sel(q, k, v, topk, block: int, scale: float = 0.0, rows=None) -> np.ndarray:
    """Each query over its own selection: q [N][Hq][D], k/v [G][N][D] bf16, topk [G][N][KB] int32
    -> out [len(rows)][Hq][D] fp64 (tokens j <= i of Sel(i,g) and of the own block)."""
    q = _u16(q)
    k = _u16(k)
    v = _u16(v)
    topk = _i32(topk)
    N, Hq, D = q.shape
    G = k.shape[0]
    KB = topk.shape[2]
    if rows is None:
        nrows, rp = N, None
    else:
        rows = _i32(rows)
        nrows, rp = int(rows.shape[0]), _p(rows)
    out = np.empty((nrows, Hq, D), dtype=np.float64)
    _load().orc_attend_sel(N, Hq, G, D, block, KB, float(scale), _p(q), _p(k), _p(v), _p(topk), nrows, rp, _p(out))
    return out


def decode(q, k_cache, v_cache, kbar, qi, w, block: int, kb: int, scale: float = 0.0, seqs=None):
    """Decode at position L-1 of every listed sequence.

    q [S][Hq][D], k/v cache [S][G][L][D], kbar [S][L//B][dI], qi [S][G][HI][dI] bf16, w [G][HI]
    -> (topk [n][G][kb] int32, out [n][Hq][D] fp64) for the n listed sequences (all if None).
    """
    q = _u16(q)
    k_cache = _u16(k_cache)
    v_cache = _u16(v_cache)
    kbar = _u16(kbar)
    qi = _u16(qi)
    w = _f32(w)
    S, Hq, D = q.shape
    _, G, L, _ = k_cache.shape
    HI, dI = qi.shape[2], qi.shape[3]
    if seqs is None:
        n, sp = S, None
    else:
        seqs = _i32(seqs)
        n, sp = int(seqs.shape[0]), _p(seqs)
    topk = np.empty((n, G, kb), dtype=np.int32)
    out = np.empty((n, Hq, D), dtype=np.float64)
    _load().orc_decode(S, L, Hq, G, D, HI, dI, block, kb, float(scale), _p(q), _p(k_cache), _p(v_cache),
                       _p(kbar), _p(qi), _p(w), n, sp, _p(topk), _p(out))
    return topk, out


def fp8_e4m3_to_f64(code: int) -> float:
    """Value of one OCP FP8 E4M3 code (0..255)."""
    return float(_load().orc_fp8_e4m3_to_f64(int(code)))


def decode_fp8(q, k8, v8, kv_scale, kbar, qi, w, block: int, kb: int, scale: float = 0.0, seqs=None):
    """decode() with FP8 E4M3 K/V caches k8, v8 [S][G][L][D] (uint8 codes) and kv_scale [S][G][2] fp32
    (key scale, value scale): the attended rows are code value * scale."""
    q = _u16(q)
    k8 = _u8(k8)
    v8 = _u8(v8)
    kv_scale = _f32(kv_scale)
    kbar = _u16(kbar)
    qi = _u16(qi)
    w = _f32(w)
    S, Hq, D = q.shape
    _, G, L, _ = k8.shape
    HI, dI = qi.shape[2], qi.shape[3]
    if seqs is None:
        n, sp = S, None
    else:
        seqs = _i32(seqs)
        n, sp = int(seqs.shape[0]), _p(seqs)
    topk = np.empty((n, G, kb), dtype=np.int32)
    out = np.empty((n, Hq, D), dtype=np.float64)
    _load().orc_decode_f8(S, L, Hq, G, D, HI, dI, block, kb, float(scale), _p(q), _p(k8), _p(v8), _p(kv_scale),
                          _p(kbar), _p(qi), _p(w), n, sp, _p(topk), _p(out))
    return topk, out


def coverage(sel1, selb, block: int, i_min: int = 0) -> float:
    """Mean token coverage of the block selection selb [G][N][kbB] against sel1 [G][N][kb1] (B=1)."""
    sel1 = _i32(sel1)
    selb = _i32(selb)
    G, N, kb1 = sel1.shape
    kbb = selb.shape[2]
    return float(_load().orc_coverage(N, G, block, kb1, kbb, _p(sel1), _p(selb), int(i_min)))
