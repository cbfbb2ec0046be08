"""Block-quantized linear layers on AMD MI355X (gfx950).

A thin Python binding over the C ABI of ``libqlinear.so`` (declared in
``include/qlinear.h``): in-situ quantization of bf16 weights into Q8_0, Q4K
or Q6K blocks (and Q5K, Q3K, Q2K, Q4_0, Q4_1, Q5_0, Q5_1), the fused
dequantize-matmul that consumes them, the gated feed-forward projection and
the quantized embedding lookup.  Every
step of the computation runs in the library's HIP kernels; this module only
checks tensors and passes pointers, sizes and the current HIP stream.
PyTorch provides device memory and streams.

Formats and policy follow page "Quantization types" (mistral.rs reference):
sections "Numeric shorthands", "Sensitive tensor precision", "Q*K family"
and "Legacy GGML types".
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# QLINEAR_LIB names another build of the same library (the host-sanitizer
# build of tests/sanitize_host.py); there is no other implementation
LIB_PATH = os.environ.get("QLINEAR_LIB") or os.path.join(_HERE, "libqlinear.so")

FMT = {"q8_0": 0, "q4k": 1, "q6k": 2, "q2k": 3, "q3k": 4, "q5k": 5, "q8k": 6,
       "q4_0": 7, "q4_1": 8, "q5_0": 9, "q5_1": 10, "q8_1": 11, "fp8": 12}
FMT_NAME = {v: k for k, v in FMT.items()}
PATH = {"auto": 0, "gemv": 1, "mfma_bf16": 2, "mfma_i8": 3, "mfma_fp8": 4}
ACT = {"silu": 0, "relu": 1, "sigmoid": 2}

Q_OK, Q_EINVAL, Q_ESHAPE, Q_EALIGN, Q_ENOTSUP, Q_EHIP, Q_ESCRATCH = 0, -1, -2, -3, -4, -5, -6
STATIC_SCRATCH_BYTES = 32 << 20  # QLINEAR_STATIC_SCRATCH_BYTES

# every symbol include/qlinear.h declares, with its ctypes signature
_P, _I64, _INT, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
_IP = ctypes.POINTER(ctypes.c_int)
SIGNATURES = {
    "q_blocks_bytes": (_SZ, [_INT, _I64, _I64]),
    "isq_quantize": (_INT, [_INT, _P, _I64, _I64, _P, _P]),
    "q_act_quantize": (_INT, [_P, _I64, _I64, _P, _P]),
    "qmatmul": (_INT, [_INT, _P, _P, _P, _I64, _I64, _I64, _P]),
    "qmatmul_workspace_bytes": (_SZ, [_INT, _INT, _I64, _I64]),
    "qmatmul_ex": (_INT, [_INT, _P, _P, _P, _I64, _I64, _I64, _INT, _P, _SZ, _P]),
    "qmatmul_static": (_INT, [_INT, _P, _P, _P, _I64, _I64, _I64, _INT, _P]),
    "q_embed": (_INT, [_INT, _P, _I64, _I64, _P, _I64, _P, _P]),
    "qmatmul_glu_workspace_bytes": (_SZ, [_INT, _I64, _I64, _I64]),
    "qmatmul_glu": (_INT, [_INT, _P, _P, _P, _P, _I64, _I64, _I64, _INT, _P, _SZ, _P]),
    "q_dequantize": (_INT, [_INT, _P, _I64, _I64, _P, _P]),
    "isq_resolve_level": (_INT, [_INT, _IP]),
    "isq_sensitive_fmt": (_INT, [_INT, _IP]),
    "isq_tensor_fmt": (_INT, [_INT, _INT, _INT, _IP]),
    "q_fmt_supported": (_INT, [_INT]),
    "q_fmt_name": (ctypes.c_char_p, [_INT]),
    "q_strerror": (ctypes.c_char_p, [_INT]),
    "q_probe_read": (_INT, [_P, _I64, _P, _P]),
    "q_probe_mfma": (_INT, [_P, _I64, _P]),
    "q_probe_mfma_flops": (_I64, [_I64]),
    "q_probe_mix": (_INT, [_P, _I64, _INT, _INT, _P]),
    "q_probe_mix_valu": (_I64, [_I64, _INT]),
}


class QLinearError(RuntimeError):
    """A call into libqlinear returned an error status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status} ({strerror(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library.  Raises ImportError if it has not been built:
    there is no fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m ggml_block_quant_amd.build` "
                              "or __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().q_strerror(status).decode()


def _fmt(fmt) -> int:
    return FMT[fmt] if isinstance(fmt, str) else int(fmt)


def _check(fn: str, status: int):
    if status != Q_OK:
        raise QLinearError(fn, status)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


# ----------------------------------------------------------------------------
# host-side helpers (no GPU needed)
# ----------------------------------------------------------------------------

def blocks_bytes(fmt, N: int, K: int) -> int:
    return int(lib().q_blocks_bytes(_fmt(fmt), N, K))


def workspace_bytes(fmt, path, M: int, K: int) -> int:
    p = PATH[path] if isinstance(path, str) else int(path)
    return int(lib().qmatmul_workspace_bytes(_fmt(fmt), p, M, K))


def resolve_level(level: int) -> str:
    out = ctypes.c_int()
    _check("isq_resolve_level", lib().isq_resolve_level(level, ctypes.byref(out)))
    return FMT_NAME[out.value]


def sensitive_fmt(model_default) -> str:
    out = ctypes.c_int()
    _check("isq_sensitive_fmt", lib().isq_sensitive_fmt(_fmt(model_default), ctypes.byref(out)))
    return FMT_NAME[out.value]


def tensor_fmt(level: int, is_embedding_or_head: bool, explicit=None) -> str:
    out = ctypes.c_int()
    e = -1 if explicit is None else _fmt(explicit)
    _check("isq_tensor_fmt", lib().isq_tensor_fmt(level, int(bool(is_embedding_or_head)), e, ctypes.byref(out)))
    return FMT_NAME[out.value]


def fmt_supported(fmt) -> bool:
    return bool(lib().q_fmt_supported(_fmt(fmt)))


# ----------------------------------------------------------------------------
# device calls
# ----------------------------------------------------------------------------

def isq(fmt, W: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Quantize bf16 weights W [N][K] (device) into a uint8 block buffer."""
    if W.dim() != 2:
        raise ValueError("W must be 2-D [N][K]")
    N, K = W.shape
    nbytes = blocks_bytes(fmt, N, K)
    if nbytes == 0:
        raise QLinearError("q_blocks_bytes", Q_ESHAPE)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
    elif out.numel() < nbytes or out.dtype != torch.uint8:
        raise ValueError("out is too small or not uint8")
    _check("isq_quantize", lib().isq_quantize(_fmt(fmt), _dev(W, "W", torch.bfloat16), N, K,
                                              _dev(out, "out"), _stream()))
    return out


def act_quantize(X: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Quantize bf16 activations X [M][K] to Q8_0 blocks (codes then scales)."""
    M, K = X.shape
    nbytes = blocks_bytes("q8_0", M, K)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=X.device)
    _check("q_act_quantize", lib().q_act_quantize(_dev(X, "X", torch.bfloat16), M, K,
                                                  _dev(out, "out"), _stream()))
    return out


def qmatmul(fmt, blocks: torch.Tensor, X: torch.Tensor, N: int, path="auto",
            out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X . deq(W)^T as fp32 [M][N] for X bf16 [M][K] and the blocks of a
    [N][K] weight.  ``path``: auto | gemv | mfma_bf16 | mfma_i8 | mfma_fp8."""
    if X.dim() != 2:
        raise ValueError("X must be 2-D [M][K]")
    M, K = X.shape
    p = PATH[path] if isinstance(path, str) else int(path)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=X.device)
    ws_ptr, ws_bytes = None, 0
    need = workspace_bytes(fmt, p, M, K)
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel()
    _check("qmatmul_ex", lib().qmatmul_ex(_fmt(fmt), _dev(blocks, "blocks", torch.uint8),
                                          _dev(X, "X", torch.bfloat16), _dev(out, "Y", torch.float32),
                                          M, N, K, p, ws_ptr, ws_bytes, _stream()))
    return out


def qmatmul_static(fmt, blocks: torch.Tensor, X: torch.Tensor, N: int, path="auto",
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """As ``qmatmul``, with no workspace: the int8 and FP8 paths keep X's
    activation blocks in the library's fixed per-GPU buffer (calls that
    overlap in time on one GPU race on it).  With ``out`` given, the call
    itself allocates nothing."""
    if X.dim() != 2:
        raise ValueError("X must be 2-D [M][K]")
    M, K = X.shape
    p = PATH[path] if isinstance(path, str) else int(path)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=X.device)
    _check("qmatmul_static", lib().qmatmul_static(_fmt(fmt), _dev(blocks, "blocks", torch.uint8),
                                                  _dev(X, "X", torch.bfloat16), _dev(out, "Y", torch.float32),
                                                  M, N, K, p, _stream()))
    return out


def glu_workspace_bytes(fmt, M: int, F: int, K: int) -> int:
    return lib().qmatmul_glu_workspace_bytes(_fmt(fmt), M, F, K)


def qmatmul_glu(fmt, gate_blocks: torch.Tensor, up_blocks: torch.Tensor, X: torch.Tensor, F: int,
                act="silu", out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """H = act(X . deq(Wg)^T) * (X . deq(Wu)^T) as fp32 [M][F] for the blocks
    of the [F][K] gate and up weights; ``act``: silu | relu | sigmoid."""
    if X.dim() != 2:
        raise ValueError("X must be 2-D [M][K]")
    M, K = X.shape
    if out is None:
        out = torch.empty((M, F), dtype=torch.float32, device=X.device)
    ws_ptr, ws_bytes = None, 0
    need = glu_workspace_bytes(fmt, M, F, K)
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    a = ACT[act] if isinstance(act, str) else int(act)
    _check("qmatmul_glu", lib().qmatmul_glu(_fmt(fmt), _dev(gate_blocks, "gate_blocks", torch.uint8),
                                            _dev(up_blocks, "up_blocks", torch.uint8),
                                            _dev(X, "X", torch.bfloat16), _dev(out, "H", torch.float32),
                                            M, F, K, a, ws_ptr, ws_bytes, _stream()))
    return out


def embed(fmt, blocks: torch.Tensor, N: int, K: int, ids: torch.Tensor,
          out: torch.Tensor | None = None) -> torch.Tensor:
    """Rows ``ids`` (int32, device) of the quantized [N][K] table, dequantized
    exactly to fp32 [len(ids)][K]; ids outside [0, N) give zero rows.  The
    same blocks serve ``qmatmul`` as a tied output head."""
    if ids.dim() != 1:
        raise ValueError("ids must be 1-D")
    n = ids.numel()
    if out is None:
        out = torch.empty((n, K), dtype=torch.float32, device=blocks.device)
    if n == 0:
        return out
    _check("q_embed", lib().q_embed(_fmt(fmt), _dev(blocks, "blocks", torch.uint8), N, K,
                                    _dev(ids, "ids", torch.int32), n, _dev(out, "out", torch.float32),
                                    _stream()))
    return out


def dequantize(fmt, blocks: torch.Tensor, N: int, K: int) -> torch.Tensor:
    """Test aid: exact fp32 [N][K] values of a block buffer."""
    out = torch.empty((N, K), dtype=torch.float32, device=blocks.device)
    _check("q_dequantize", lib().q_dequantize(_fmt(fmt), _dev(blocks, "blocks", torch.uint8), N, K,
                                              _dev(out, "W"), _stream()))
    return out


# ----------------------------------------------------------------------------
# measurement aids (the benchmark's ceilings; not part of the computation)
# ----------------------------------------------------------------------------

def probe_read(buf: torch.Tensor, sink: torch.Tensor):
    """Read every byte of device tensor ``buf`` once (streaming-read ceiling)."""
    n = buf.numel() * buf.element_size()
    _check("q_probe_read", lib().q_probe_read(_dev(buf, "buf"), n, _dev(sink, "sink", torch.float32), _stream()))


def probe_mfma(iters: int, sink: torch.Tensor) -> int:
    """A loop of bf16 MFMAs with no memory traffic; returns its FLOP count."""
    _check("q_probe_mfma", lib().q_probe_mfma(_dev(sink, "sink", torch.float32), iters, _stream()))
    return int(lib().q_probe_mfma_flops(iters))


def probe_mix(iters: int, mode: int, waves_per_simd: int, sink: torch.Tensor):
    """The MFMA loop with 16 fp32 fmas per MFMA, waves_per_simd waves on
    each SIMD: mode 0 MFMAs only, 1 fmas only, 2 both interleaved; returns
    (MFMA FLOP, wave-level fma instructions) of the call."""
    _check("q_probe_mix", lib().q_probe_mix(_dev(sink, "sink", torch.float32), iters, mode, waves_per_simd,
                                            _stream()))
    fmas = int(lib().q_probe_mix_valu(iters, waves_per_simd))
    flops = fmas // 16 * 32 * 32 * 16 * 2 if mode != 1 else 0
    return flops, (fmas if mode != 0 else 0)
