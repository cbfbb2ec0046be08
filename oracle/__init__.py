"""CPU oracle for the block-quantized linear layer -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does, and this package never imports the product.

The arithmetic lives in ``oracle.c`` (plain scalar C, built with
``-O2 -fno-fast-math -ffp-contract=off``); this module only marshals NumPy
arrays.  Every function states the passage it follows in ``oracle.c``.

Format names: ``"q8_0"``, ``"q4k"``, ``"q6k"`` (page "Quantization types",
sections "Legacy GGML types" and "Q*K family").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_LIB names another build of oracle.c (the host-sanitizer build of
# tests/sanitize_host.py), used as is
_BUILT = os.path.join(_HERE, "liboracle.so")
_LIB = os.environ.get("ORACLE_LIB") or _BUILT

FORMATS = ("q8_0", "q4k", "q6k")
# further formats (oracle.c, "Further formats"): K-quants and the legacy
# 32-element types, with the public header's format numbers
KQ_FORMATS = {"q5k": 5, "q3k": 4, "q2k": 3}
LEG_FORMATS = {"q4_0": 7, "q4_1": 8, "q5_0": 9, "q5_1": 10}
MORE_FORMATS = tuple(KQ_FORMATS) + tuple(LEG_FORMATS)


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain C, OpenMP over
    independent rows/blocks only)."""
    if force or not os.path.exists(_BUILT):
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
               "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", _SRC,
               "-o", _BUILT + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_BUILT + ".tmp", _BUILT)
    return _BUILT


_lib = None


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.oracle_f16_from_f32.restype = ctypes.c_uint16
        lib.oracle_f16_from_f32.argtypes = [ctypes.c_float]
        lib.oracle_f32_from_f16.restype = ctypes.c_float
        lib.oracle_f32_from_f16.argtypes = [ctypes.c_uint16]
        lib.oracle_rha.restype = ctypes.c_float
        lib.oracle_rha.argtypes = [ctypes.c_float]
        sigs = {
            "oracle_f16_from_f32_array": [P, I, P],
            "oracle_f32_from_f16_array": [P, I, P],
            "oracle_rha_array": [P, I, P],
            "oracle_quantize_q8_0": [P, I, I, P, P],
            "oracle_quantize_q4k": [P, I, I, P, P, P, P, P],
            "oracle_quantize_q6k": [P, I, I, P, P, P],
            "oracle_dequant_q8_0": [P, P, I, P],
            "oracle_dequant_q4k": [P, P, P, P, P, I, P],
            "oracle_dequant_q6k": [P, P, P, I, P],
            "oracle_matmul_a16": [P, P, I, I, I, P, P],
            "oracle_matmul_a16_pairs": [P, P, I, P, P, I, P, P],
            "oracle_matmul_a8": [P, P, P, P, I, I, I, P, P, I, P, P],
            "oracle_glu": [P, P, P, P, I, I, P, P],
            "oracle_quantize_kq": [I, P, I, I, P, P, P, P, P],
            "oracle_dequant_kq": [I, P, P, P, P, P, I, P],
            "oracle_quantize_leg": [I, P, I, I, P, P, P],
            "oracle_dequant_leg": [I, P, P, P, I, P],
            "oracle_pack_kq": [I, P, P, P, P, P, I, I, P],
            "oracle_unpack_kq": [I, P, I, I, P, P, P, P, P],
            "oracle_pack_leg": [I, P, P, P, I, I, P],
            "oracle_unpack_leg": [I, P, I, I, P, P, P],
            "oracle_e4m3_from_f32_array": [P, I, P],
            "oracle_quantize_fp8": [P, I, I, P, P],
            "oracle_dequant_fp8": [P, P, I, I, P],
            "oracle_matmul_fp8": [P, P, P, P, I, P, P, I, P, P],
            "oracle_pack_q8_0": [P, P, I, I, P],
            "oracle_unpack_q8_0": [P, I, I, P, P],
            "oracle_pack_q4k": [P, P, P, P, P, I, I, P],
            "oracle_unpack_q4k": [P, I, I, P, P, P, P, P],
            "oracle_pack_q6k": [P, P, P, I, I, P],
            "oracle_unpack_q6k": [P, I, I, P, P, P],
        }
        for name, args in sigs.items():
            fn = getattr(lib, name)
            fn.restype = None
            fn.argtypes = args
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_from_f32.restype = ctypes.c_uint8
        lib.oracle_e4m3_from_f32.argtypes = [ctypes.c_float]
        lib.oracle_more_layout.restype = ctypes.c_int64
        lib.oracle_more_layout.argtypes = [I, I, I, P]
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ----------------------------------------------------------------------------
# scalar conversions (vectorised by looping in Python over small arrays only;
# bulk checks use f16_from_f32_array below)
# ----------------------------------------------------------------------------

def f16_from_f32(v: float) -> int:
    """IEEE binary32 -> binary16 bits, RNE, gradual underflow, overflow to inf."""
    return int(_L().oracle_f16_from_f32(float(v)))


def f32_from_f16(h: int) -> float:
    return float(_L().oracle_f32_from_f16(int(h)))


def rha(v: float) -> float:
    """Round half away from zero on a binary32 value."""
    return float(_L().oracle_rha(float(v)))


def f16_from_f32_array(a: np.ndarray) -> np.ndarray:
    """Element-wise binary32 -> binary16 bits (oracle_f16_from_f32)."""
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    _L().oracle_f16_from_f32_array(_p(a), a.size, _p(out))
    return out


def f32_from_f16_array(h: np.ndarray) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    _L().oracle_f32_from_f16_array(_p(h), h.size, _p(out))
    return out


def rha_array(a: np.ndarray) -> np.ndarray:
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.float32)
    _L().oracle_rha_array(_p(a), a.size, _p(out))
    return out


# ----------------------------------------------------------------------------
# quantizers -> logical fields
# ----------------------------------------------------------------------------

def quantize(fmt: str, w_bf16: np.ndarray) -> dict:
    """Quantize a [rows][cols] bf16 tensor (given as uint16 bit patterns) to
    the logical fields of ``fmt`` (oracle.c: q8_0_block / q4k_group /
    q6k_group)."""
    w = _c(w_bf16, np.uint16)
    assert w.ndim == 2
    rows, cols = w.shape
    L = _L()
    if fmt == "q8_0":
        assert cols % 32 == 0
        d16 = np.empty((rows, cols // 32), np.uint16)
        q = np.empty((rows, cols), np.int8)
        L.oracle_quantize_q8_0(_p(w), rows, cols, _p(d16), _p(q))
        return {"d16": d16, "q": q}
    if fmt in LEG_FORMATS:
        assert cols % 32 == 0
        d16 = np.empty((rows, cols // 32), np.uint16)
        m16 = np.empty((rows, cols // 32), np.uint16)
        q = np.empty((rows, cols), np.int8)
        L.oracle_quantize_leg(LEG_FORMATS[fmt], _p(w), rows, cols, _p(d16), _p(m16), _p(q))
        return {"d16": d16, "m16": m16, "q": q}
    assert cols % 256 == 0
    G = rows * cols // 256
    if fmt == "q4k":
        d16 = np.empty(G, np.uint16)
        dmin16 = np.empty(G, np.uint16)
        sc = np.empty((G, 8), np.uint8)
        mq = np.empty((G, 8), np.uint8)
        q = np.empty((rows, cols), np.uint8)
        L.oracle_quantize_q4k(_p(w), rows, cols, _p(d16), _p(dmin16), _p(sc), _p(mq), _p(q))
        return {"d16": d16, "dmin16": dmin16, "sc": sc, "mq": mq, "q": q}
    if fmt == "q6k":
        d16 = np.empty(G, np.uint16)
        sc = np.empty((G, 16), np.int8)
        q = np.empty((rows, cols), np.int8)
        L.oracle_quantize_q6k(_p(w), rows, cols, _p(d16), _p(sc), _p(q))
        return {"d16": d16, "sc": sc, "q": q}
    if fmt in KQ_FORMATS:
        d16 = np.empty(G, np.uint16)
        dmin16 = np.empty(G, np.uint16)
        sc = np.empty((G, 16), np.uint8)
        mq = np.empty((G, 16), np.uint8)
        q = np.empty((rows, cols), np.int8)
        L.oracle_quantize_kq(KQ_FORMATS[fmt], _p(w), rows, cols, _p(d16), _p(dmin16), _p(sc), _p(mq), _p(q))
        return {"d16": d16, "dmin16": dmin16, "sc": sc, "mq": mq, "q": q}
    if fmt in LEG_FORMATS:
        d16 = np.empty((rows, cols // 32), np.uint16)
        m16 = np.empty((rows, cols // 32), np.uint16)
        q = np.empty((rows, cols), np.int8)
        L.oracle_quantize_leg(LEG_FORMATS[fmt], _p(w), rows, cols, _p(d16), _p(m16), _p(q))
        return {"d16": d16, "m16": m16, "q": q}
    raise ValueError(fmt)


# ----------------------------------------------------------------------------
# FP8 E4M3 with per-row scales (oracle.c, "FP8 E4M3 ...")
# ----------------------------------------------------------------------------

def e4m3_value(b: int) -> float:
    return float(_L().oracle_e4m3_value(int(b)))


def e4m3_from_f32_array(a) -> np.ndarray:
    a = _c(np.asarray(a, np.float32), np.float32)
    out = np.empty(a.shape, np.uint8)
    _L().oracle_e4m3_from_f32_array(_p(a), a.size, _p(out))
    return out


def quantize_fp8(w_bf16: np.ndarray) -> dict:
    """Rows of a bf16 tensor -> E4M3 codes [rows][cols] and binary32 scales
    s [rows] = max|x| / 448."""
    w = _c(w_bf16, np.uint16)
    rows, cols = w.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty(rows, np.float32)
    _L().oracle_quantize_fp8(_p(w), rows, cols, _p(q), _p(s))
    return {"q": q, "s": s}


def dequant_fp8(f: dict) -> np.ndarray:
    q = _c(f["q"], np.uint8)
    rows, cols = q.shape
    out = np.empty((rows, cols), np.float64)
    _L().oracle_dequant_fp8(_p(q), _p(_c(f["s"], np.float32)), rows, cols, _p(out))
    return out


def pack_fp8(f: dict) -> np.ndarray:
    """Planar bytes: codes [rows][cols], then the fp32 scales at the first
    multiple of 16 bytes (zero padding)."""
    q = _c(f["q"], np.uint8)
    rows, cols = q.shape
    off = (rows * cols + 15) // 16 * 16
    buf = np.zeros((off + 4 * rows + 15) // 16 * 16, np.uint8)
    buf[: rows * cols] = q.ravel()
    buf[off: off + 4 * rows] = _c(f["s"], np.float32).view(np.uint8)
    return buf


def unpack_fp8(buf: np.ndarray, rows: int, cols: int) -> dict:
    b = _c(buf, np.uint8)
    off = (rows * cols + 15) // 16 * 16
    return {"q": b[: rows * cols].reshape(rows, cols).copy(),
            "s": b[off: off + 4 * rows].copy().view(np.float32)}


def matmul_fp8(fx: dict, fw: dict, mi=None, ni=None):
    """Dynamic per-token W8A8 oracle: Y = s_m s_n sum_k e4m3(qx) e4m3(qw)
    (exact), with the normaliser s_m s_n sum |e4m3(qx) e4m3(qw)|; all
    outputs or the pairs (mi, ni)."""
    qx, qw = _c(fx["q"], np.uint8), _c(fw["q"], np.uint8)
    M, K = qx.shape
    N = qw.shape[0]
    full = mi is None
    if full:
        mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        mi, ni = mm.ravel(), nn.ravel()
    mi, ni = _c(mi, np.int64), _c(ni, np.int64)
    Y = np.empty(mi.size, np.float64)
    den = np.empty(mi.size, np.float64)
    _L().oracle_matmul_fp8(_p(qx), _p(_c(fx["s"], np.float32)), _p(qw), _p(_c(fw["s"], np.float32)), K,
                           _p(mi), _p(ni), mi.size, _p(Y), _p(den))
    if full:
        return Y.reshape(M, N), den.reshape(M, N)
    return Y, den


def more_layout(fmt: str, rows: int, cols: int):
    """(plane offsets, total bytes) of a further format's planar buffer."""
    o = np.zeros(4, np.int64)
    fid = KQ_FORMATS.get(fmt, LEG_FORMATS.get(fmt))
    total = _L().oracle_more_layout(fid, rows, cols, _p(o))
    return [int(v) for v in o], int(total)


def blocks_bytes(fmt: str, rows: int, cols: int) -> int:
    """Bytes of the planar buffer: 34/32, 144/256, 210/256 bytes per element;
    the Q6K buffer is zero-padded to a multiple of 16 bytes."""
    n = rows * cols
    if fmt in MORE_FORMATS:
        return more_layout(fmt, rows, cols)[1]
    if fmt == "q6k":
        return (n * 210 // 256 + 15) // 16 * 16
    return {"q8_0": n * 34 // 32, "q4k": n * 144 // 256}[fmt]


def pack(fmt: str, f: dict, rows: int, cols: int) -> np.ndarray:
    """Logical fields -> planar bytes (layout in oracle.c, 'Planar byte layout')."""
    buf = np.zeros(blocks_bytes(fmt, rows, cols), np.uint8)
    L = _L()
    if fmt == "q8_0":
        L.oracle_pack_q8_0(_p(_c(f["d16"], np.uint16)), _p(_c(f["q"], np.int8)), rows, cols, _p(buf))
    elif fmt == "q4k":
        L.oracle_pack_q4k(_p(_c(f["d16"], np.uint16)), _p(_c(f["dmin16"], np.uint16)),
                          _p(_c(f["sc"], np.uint8)), _p(_c(f["mq"], np.uint8)),
                          _p(_c(f["q"], np.uint8)), rows, cols, _p(buf))
    elif fmt == "q6k":
        L.oracle_pack_q6k(_p(_c(f["d16"], np.uint16)), _p(_c(f["sc"], np.int8)),
                          _p(_c(f["q"], np.int8)), rows, cols, _p(buf))
    elif fmt in KQ_FORMATS:
        L.oracle_pack_kq(KQ_FORMATS[fmt], _p(_c(f["d16"], np.uint16)), _p(_c(f["dmin16"], np.uint16)),
                         _p(_c(f["sc"], np.uint8)), _p(_c(f["mq"], np.uint8)), _p(_c(f["q"], np.int8)),
                         rows, cols, _p(buf))
    elif fmt in LEG_FORMATS:
        L.oracle_pack_leg(LEG_FORMATS[fmt], _p(_c(f["d16"], np.uint16)), _p(_c(f["m16"], np.uint16)),
                          _p(_c(f["q"], np.int8)), rows, cols, _p(buf))
    else:
        raise ValueError(fmt)
    return buf


def unpack(fmt: str, buf: np.ndarray, rows: int, cols: int) -> dict:
    """Planar bytes -> logical fields (the oracle's own reader)."""
    b = _c(buf, np.uint8)
    assert b.size == blocks_bytes(fmt, rows, cols), (b.size, blocks_bytes(fmt, rows, cols))
    L = _L()
    G = rows * cols // 256
    if fmt == "q8_0":
        d16 = np.empty((rows, cols // 32), np.uint16)
        q = np.empty((rows, cols), np.int8)
        L.oracle_unpack_q8_0(_p(b), rows, cols, _p(d16), _p(q))
        return {"d16": d16, "q": q}
    if fmt == "q4k":
        d16 = np.empty(G, np.uint16)
        dmin16 = np.empty(G, np.uint16)
        sc = np.empty((G, 8), np.uint8)
        mq = np.empty((G, 8), np.uint8)
        q = np.empty((rows, cols), np.uint8)
        L.oracle_unpack_q4k(_p(b), rows, cols, _p(d16), _p(dmin16), _p(sc), _p(mq), _p(q))
        return {"d16": d16, "dmin16": dmin16, "sc": sc, "mq": mq, "q": q}
    if fmt == "q6k":
        d16 = np.empty(G, np.uint16)
        sc = np.empty((G, 16), np.int8)
        q = np.empty((rows, cols), np.int8)
        L.oracle_unpack_q6k(_p(b), rows, cols, _p(d16), _p(sc), _p(q))
        return {"d16": d16, "sc": sc, "q": q}
    if fmt in KQ_FORMATS:
        d16 = np.empty(G, np.uint16)
        dmin16 = np.empty(G, np.uint16)
        sc = np.empty((G, 16), np.uint8)
        mq = np.empty((G, 16), np.uint8)
        q = np.empty((rows, cols), np.int8)
        L.oracle_unpack_kq(KQ_FORMATS[fmt], _p(b), rows, cols, _p(d16), _p(dmin16), _p(sc), _p(mq), _p(q))
        return {"d16": d16, "dmin16": dmin16, "sc": sc, "mq": mq, "q": q}
    if fmt in LEG_FORMATS:
        d16 = np.empty((rows, cols // 32), np.uint16)
        m16 = np.empty((rows, cols // 32), np.uint16)
        q = np.empty((rows, cols), np.int8)
        L.oracle_unpack_leg(LEG_FORMATS[fmt], _p(b), rows, cols, _p(d16), _p(m16), _p(q))
        return {"d16": d16, "m16": m16, "q": q}
    raise ValueError(fmt)


def dequant(fmt: str, f: dict, rows: int, cols: int) -> np.ndarray:
    """Exact dequantized weights [rows][cols] in fp64."""
    out = np.empty((rows, cols), np.float64)
    n = rows * cols
    L = _L()
    if fmt == "q8_0":
        L.oracle_dequant_q8_0(_p(_c(f["d16"], np.uint16)), _p(_c(f["q"], np.int8)), n, _p(out))
    elif fmt == "q4k":
        L.oracle_dequant_q4k(_p(_c(f["d16"], np.uint16)), _p(_c(f["dmin16"], np.uint16)),
                             _p(_c(f["sc"], np.uint8)), _p(_c(f["mq"], np.uint8)),
                             _p(_c(f["q"], np.uint8)), n, _p(out))
    elif fmt == "q6k":
        L.oracle_dequant_q6k(_p(_c(f["d16"], np.uint16)), _p(_c(f["sc"], np.int8)),
                             _p(_c(f["q"], np.int8)), n, _p(out))
    elif fmt in KQ_FORMATS:
        L.oracle_dequant_kq(KQ_FORMATS[fmt], _p(_c(f["d16"], np.uint16)), _p(_c(f["dmin16"], np.uint16)),
                            _p(_c(f["sc"], np.uint8)), _p(_c(f["mq"], np.uint8)), _p(_c(f["q"], np.int8)),
                            n, _p(out))
    elif fmt in LEG_FORMATS:
        L.oracle_dequant_leg(LEG_FORMATS[fmt], _p(_c(f["d16"], np.uint16)), _p(_c(f["m16"], np.uint16)),
                             _p(_c(f["q"], np.int8)), n, _p(out))
    else:
        raise ValueError(fmt)
    return out


def embed(W: np.ndarray, ids) -> np.ndarray:
    """Quantized embedding lookup (page "Quantization types", section
    "Sensitive tensor precision": token embeddings are stored quantized and a
    tied output head reuses them): row i is row ids[i] of the exact
    dequantized table W [N][K] (from ``dequant``), and an id outside [0, N)
    gives a row of zeros.  Indexing only, no arithmetic."""
    ids = np.asarray(ids, np.int64)
    N, K = W.shape
    out = np.zeros((ids.size, K), np.float64)
    ok = (ids >= 0) & (ids < N)
    out[ok] = W[ids[ok]]
    return out


def select_rows(fmt: str, f: dict, rows, cols: int) -> dict:
    """Fields of the selected weight rows only (for sampled parity checks)."""
    rows = np.asarray(rows, np.int64)
    if fmt == "q8_0":
        return {"d16": f["d16"][rows], "q": f["q"][rows]}
    gpr = cols // 256
    gsel = (rows[:, None] * gpr + np.arange(gpr)[None, :]).ravel()
    out = {k: v[gsel] for k, v in f.items() if k != "q"}
    out["q"] = f["q"][rows]
    return out


def rows_of_buffer(fmt: str, buf: np.ndarray, rows: int, cols: int, sel) -> np.ndarray:
    """The planar buffer of the sub-tensor made of rows ``sel`` of a
    [rows][cols] buffer (each plane sliced per row; layout in oracle.c)."""
    sel = np.asarray(sel, np.int64)
    b = np.asarray(buf, np.uint8)
    E = rows * cols
    if fmt == "q8_0":
        planes = [(0, cols), (E, cols // 16)]
    elif fmt == "q4k":
        G = E // 256
        planes = [(0, cols // 2), (128 * G, cols // 16)]
    elif fmt == "q6k":
        G = E // 256
        planes = [(0, cols * 192 // 256), (192 * G, cols // 16), (208 * G, cols // 128)]
    else:
        raise ValueError(fmt)
    parts = []
    for off, per_row in planes:
        idx = off + sel[:, None] * per_row + np.arange(per_row)[None, :]
        parts.append(b[idx.ravel()])
    return np.concatenate(parts)


# ----------------------------------------------------------------------------
# fp64 matmuls and the error metric
# ----------------------------------------------------------------------------

def matmul_a16(W: np.ndarray, x_bf16: np.ndarray):
    """Y = x . W^T in fp64 with W the exact dequantized weight [N][K] and x
    bf16 [M][K]; also returns the normaliser sum_k |w||x| per output."""
    W = _c(W, np.float64)
    x = _c(x_bf16, np.uint16)
    N, K = W.shape
    M = x.shape[0]
    assert x.shape[1] == K
    Y = np.empty((M, N), np.float64)
    den = np.empty((M, N), np.float64)
    _L().oracle_matmul_a16(_p(W), _p(x), M, N, K, _p(Y), _p(den))
    return Y, den


def matmul_a16_pairs(W_rows: np.ndarray, x_bf16: np.ndarray, mi, wrow):
    """The same sums for selected outputs only: output i is row ``mi[i]`` of x
    against row ``wrow[i]`` of ``W_rows``."""
    W = _c(W_rows, np.float64)
    x = _c(x_bf16, np.uint16)
    mi = _c(mi, np.int64)
    wrow = _c(wrow, np.int64)
    K = W.shape[1]
    Y = np.empty(mi.size, np.float64)
    den = np.empty(mi.size, np.float64)
    _L().oracle_matmul_a16_pairs(_p(W), _p(x), K, _p(mi), _p(wrow), mi.size, _p(Y), _p(den))
    return Y, den


def matmul_a8(fw: dict, fx: dict, M: int, N: int, K: int, mi=None, ni=None):
    """A8 oracle: both operands Q8_0 (weights fw, activations fx, the logical
    fields of ``quantize('q8_0', ...)``); integer block sums exact, the rest
    fp64.  Returns (Y, den) for all outputs or for the pairs (mi, ni)."""
    full = mi is None
    if full:
        mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        mi, ni = mm.ravel(), nn.ravel()
    mi = _c(mi, np.int64)
    ni = _c(ni, np.int64)
    Y = np.empty(mi.size, np.float64)
    den = np.empty(mi.size, np.float64)
    _L().oracle_matmul_a8(_p(_c(fw["d16"], np.uint16)), _p(_c(fw["q"], np.int8)),
                          _p(_c(fx["d16"], np.uint16)), _p(_c(fx["q"], np.int8)),
                          M, N, K, _p(mi), _p(ni), mi.size, _p(Y), _p(den))
    if full:
        return Y.reshape(M, N), den.reshape(M, N)
    return Y, den


ACTS = {"silu": 0, "relu": 1, "sigmoid": 2}


def glu_act(act: str, g, u, eg=None, eu=None):
    """h = act(g) * u in fp64 (oracle.c: oracle_glu) and the bound on
    |h' - h| for any g', u' within eg, eu of g, u (zeros when omitted)."""
    g = _c(np.asarray(g, np.float64), np.float64)
    u = _c(np.asarray(u, np.float64), np.float64)
    eg = _c(np.zeros_like(g) if eg is None else np.asarray(eg, np.float64), np.float64)
    eu = _c(np.zeros_like(u) if eu is None else np.asarray(eu, np.float64), np.float64)
    h = np.empty_like(g)
    bound = np.empty_like(g)
    _L().oracle_glu(_p(g), _p(u), _p(eg), _p(eu), g.size, ACTS[act], _p(h), _p(bound))
    return h, bound


def glu(Wg: np.ndarray, Wu: np.ndarray, x_bf16: np.ndarray, act: str):
    """Gated projection of bf16 x [M][K] with exact dequantized gate and up
    weights [F][K]: returns h* = act(g*) u* and its normaliser, the bound
    on |h - h*| when g and u each carry the matmul error bar (1 per unit of
    sum_k |w||x|); a GPU result passes when |h - h*| <= 1e-3 * normaliser
    (zero normaliser: h must be exactly 0)."""
    g, dg = matmul_a16(Wg, x_bf16)
    u, du = matmul_a16(Wu, x_bf16)
    return glu_act(act, g, u, dg, du)


def normalized_error(y_gpu, y_ref, den) -> np.ndarray:
    """e = |y_gpu - y_ref| / sum_k |w||x| per output; where the normaliser is
    0 the output must be exactly 0, so e is 0 there if y_gpu == 0 else inf."""
    y_gpu = np.asarray(y_gpu, np.float64)
    diff = np.abs(y_gpu - np.asarray(y_ref, np.float64))
    den = np.asarray(den, np.float64)
    e = np.where(den > 0, diff / np.where(den > 0, den, 1.0), np.where(y_gpu == 0, 0.0, np.inf))
    return e
