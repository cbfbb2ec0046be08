"""Host-side tests of the C ABI (no GPU needed): the library loads and
exports every symbol the header declares, sizes and workspace sizes, the ISQ
policy tables of page "Quantization types", and every argument error, which
must be reported before anything is launched (the fake pointers below are
never dereferenced)."""
import ctypes
import json
import os
import re

import pytest

import ggml_block_quant_amd as ql
from conftest import GOLDEN, ROOT

HEADER = os.path.join(ROOT, "include", "qlinear.h")


def test_library_exports_every_declared_symbol():
    text = open(HEADER).read()
    body = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", body)) - {"sizeof", "defined"}
    assert names == set(ql.SIGNATURES), (names ^ set(ql.SIGNATURES))
    L = ql.lib()
    for n in names:
        assert hasattr(L, n), n


def test_blocks_bytes():
    assert ql.blocks_bytes("q8_0", 1024, 1024) == 1024 * 1024 * 34 // 32
    assert ql.blocks_bytes("q4k", 14336, 4096) == 33_030_144
    assert ql.blocks_bytes("q8_0", 14336, 4096) == 62_390_272
    assert ql.blocks_bytes("q6k", 131072, 5120) == 550_502_400
    assert ql.blocks_bytes("q8_0", 3, 32) == 3 * 34
    assert ql.blocks_bytes("q4k", 3, 32) == 0          # K % 256
    assert ql.blocks_bytes("q4k", 0, 256) == 0
    assert ql.blocks_bytes("q8k", 4, 256) == 0         # named but not implemented
    # further formats: GGML byte counts per 256 / 32 elements, planes padded to 16 bytes
    assert ql.blocks_bytes("q5k", 4, 256) == 4 * 176
    assert ql.blocks_bytes("q3k", 4, 256) == 448       # d plane at 108*4 = 432, + 8 bytes, rounded up to 16
    assert ql.blocks_bytes("q2k", 4, 256) == 336
    assert ql.blocks_bytes("q4_0", 4, 256) == 4 * 8 * 18
    assert ql.blocks_bytes("q4_1", 4, 256) == 4 * 8 * 20
    assert ql.blocks_bytes("q5_0", 4, 256) == 4 * 8 * 22
    assert ql.blocks_bytes("q5_1", 4, 256) == 4 * 8 * 24
    assert ql.blocks_bytes("q4_0", 4, 32) == 0         # the further formats need K % 256
    assert ql.blocks_bytes("fp8", 3, 256) == 3 * 256 + 16   # codes, then 3 fp32 scales rounded up to 16
    assert ql.blocks_bytes(99, 4, 256) == 0
    # bits per weight: 8.5, 4.5, 6.5625 (nominal 8, 4, 6 on the page's tables)
    assert ql.blocks_bytes("q8_0", 1, 256) * 8 / 256 == 8.5
    assert ql.blocks_bytes("q4k", 1, 256) * 8 / 256 == 4.5
    assert ql.blocks_bytes("q6k", 8, 256) * 8 / 2048 == 6.5625
    assert ql.blocks_bytes("q6k", 1, 256) == 224          # 210, zero-padded to 16


def test_workspace_bytes():
    assert ql.workspace_bytes("q8_0", "mfma_i8", 2048, 4096) == ql.blocks_bytes("q8_0", 2048, 4096)
    assert ql.workspace_bytes("q8_0", "mfma_bf16", 2048, 4096) == 0
    assert ql.workspace_bytes("q4k", "mfma_i8", 16, 4096) == 0
    assert ql.workspace_bytes("fp8", "mfma_fp8", 2048, 4096) == 2048 * 4096 + 2048 * 4
    assert ql.workspace_bytes("q8_0", "mfma_fp8", 16, 4096) == 0


def test_policy_tables_match_the_page():
    g = json.load(open(os.path.join(GOLDEN, "isq_policy_tables.json")))
    for level, fmt in g["shorthand_cuda_cpu"].items():
        assert ql.resolve_level(int(level)) == fmt.lower(), level
    for default, eff in g["sensitive_promotion"].items():
        assert ql.sensitive_fmt(default.lower()) == eff.lower(), default
    for bad in (0, 1, 7, 9, 16, -4):
        with pytest.raises(ql.QLinearError) as e:
            ql.resolve_level(bad)
        assert e.value.status == ql.Q_EINVAL


def test_tensor_fmt_precedence():
    # level 4 -> Q4K; an embedding or output head is promoted to Q6K; an
    # explicit per-tensor type wins over both
    assert ql.tensor_fmt(4, False) == "q4k"
    assert ql.tensor_fmt(4, True) == "q6k"
    assert ql.tensor_fmt(8, True) == "q8_0"
    assert ql.tensor_fmt(6, True) == "q8_0"
    assert ql.tensor_fmt(4, True, explicit="q4k") == "q4k"
    assert ql.tensor_fmt(99, True, explicit="q8_0") == "q8_0"
    # the workload's 32-layer decoder at level 4: layers Q4K, lm_head Q6K
    assert [ql.tensor_fmt(4, k == "lm_head") for k in ("q", "down", "lm_head")] == ["q4k", "q4k", "q6k"]


def test_supported_formats():
    assert [ql.fmt_supported(f) for f in ("q8_0", "q4k", "q6k")] == [True] * 3
    assert all(ql.fmt_supported(f) for f in ("q2k", "q3k", "q5k", "q4_0", "q4_1", "q5_0", "q5_1"))
    assert not any(ql.fmt_supported(f) for f in ("q8k", "q8_1"))
    L = ql.lib()
    assert L.q_fmt_name(1) == b"q4k" and L.q_fmt_name(12) == b"fp8" and L.q_fmt_name(42) is None
    assert ql.fmt_supported("fp8")
    for s in range(-6, 1):
        assert L.q_strerror(s)
    assert b"scratch" in L.q_strerror(ql.Q_ESCRATCH)


A = ctypes.c_void_p(0x10000)     # 16-byte aligned, never dereferenced
A2 = ctypes.c_void_p(0x20000)
A3 = ctypes.c_void_p(0x30000)
MIS = ctypes.c_void_p(0x10004)   # misaligned
NULL = ctypes.c_void_p(0)


def test_isq_argument_errors():
    L = ql.lib()
    assert L.isq_quantize(0, NULL, 4, 256, A, NULL) == ql.Q_EINVAL
    assert L.isq_quantize(0, A, 4, 256, NULL, NULL) == ql.Q_EINVAL
    assert L.isq_quantize(17, A, 4, 256, A2, NULL) == ql.Q_EINVAL
    assert L.isq_quantize(6, A, 4, 256, A2, NULL) == ql.Q_ENOTSUP   # Q8K
    assert L.isq_quantize(11, A, 4, 256, A2, NULL) == ql.Q_ENOTSUP  # Q8_1
    assert L.isq_quantize(7, A, 4, 32, A2, NULL) == ql.Q_ESHAPE     # Q4_0 here needs K % 256
    assert L.isq_quantize(1, MIS, 4, 256, A2, NULL) == ql.Q_EALIGN
    assert L.isq_quantize(1, A, 4, 256, MIS, NULL) == ql.Q_EALIGN
    assert L.isq_quantize(1, A, 4, 250, A2, NULL) == ql.Q_ESHAPE
    assert L.isq_quantize(1, A, 4, 32, A2, NULL) == ql.Q_ESHAPE     # Q4K needs K % 256
    assert L.isq_quantize(1, A, 0, 256, A2, NULL) == ql.Q_ESHAPE
    assert L.isq_quantize(1, A, -1, 256, A2, NULL) == ql.Q_ESHAPE
    assert L.isq_quantize(1, A, 1 << 25, 256, A2, NULL) == ql.Q_ESHAPE
    assert L.isq_quantize(0, A, 4, 48, A2, NULL) == ql.Q_ESHAPE     # Q8_0 needs K % 32
    assert L.q_act_quantize(NULL, 4, 256, A2, NULL) == ql.Q_EINVAL
    assert L.q_act_quantize(A, 4, 100, A2, NULL) == ql.Q_ESHAPE
    assert L.q_dequantize(1, A, 4, 100, A2, NULL) == ql.Q_ESHAPE
    assert L.q_dequantize(1, MIS, 4, 256, A2, NULL) == ql.Q_EALIGN


def test_qmatmul_argument_errors():
    L = ql.lib()
    ok = dict(M=4, N=64, K=256)

    def call(fmt=1, b=A, x=A2, y=A3, M=4, N=64, K=256, path=0, ws=NULL, wsb=0):
        return L.qmatmul_ex(fmt, b, x, y, M, N, K, path, ws, wsb, NULL)

    assert call(b=NULL) == ql.Q_EINVAL
    assert call(x=NULL) == ql.Q_EINVAL
    assert call(y=NULL) == ql.Q_EINVAL
    assert call(fmt=13) == ql.Q_EINVAL
    assert call(fmt=6) == ql.Q_ENOTSUP                 # Q8K
    assert call(y=MIS) == ql.Q_EALIGN
    assert call(K=128) == ql.Q_ESHAPE
    assert call(K=384) == ql.Q_ESHAPE
    assert call(M=0) == ql.Q_ESHAPE
    assert call(M=70000) == ql.Q_ESHAPE
    assert call(N=0) == ql.Q_ESHAPE
    assert call(path=9) == ql.Q_EINVAL
    assert call(path=1, M=9) == ql.Q_ESHAPE            # GEMV is for M <= 8
    assert call(path=3) == ql.Q_ENOTSUP                # int8 path needs Q8_0 weights
    assert call(fmt=0, path=3) == ql.Q_EINVAL          # ... and a workspace
    assert call(fmt=0, path=3, ws=A, wsb=10) == ql.Q_EINVAL
    assert call(fmt=0, path=3, ws=MIS, wsb=1 << 20) == ql.Q_EALIGN
    assert call(path=4) == ql.Q_ENOTSUP                # the FP8 path needs FP8 weights
    assert call(fmt=12, path=4) == ql.Q_EINVAL         # ... and a workspace
    assert call(fmt=12, path=4, ws=A, wsb=100) == ql.Q_EINVAL
    assert call(fmt=13) == ql.Q_EINVAL
    # Q8_0 rows may end in a tail of whole blocks (K % 32); other formats and
    # the int8 path need K % 256 (no launch happens for these errors)
    assert call(fmt=0, K=100) == ql.Q_ESHAPE
    assert call(fmt=0, K=16) == ql.Q_ESHAPE
    assert call(fmt=7, K=96) == ql.Q_ESHAPE
    assert call(fmt=12, K=96) == ql.Q_ESHAPE
    assert call(fmt=0, K=96, path=3, ws=A, wsb=1 << 20) == ql.Q_ESHAPE
    assert L.qmatmul_workspace_bytes(0, 3, 4, 96) == 0
    assert L.qmatmul_workspace_bytes(0, 3, 4, 256) > 0
    assert L.qmatmul(1, A, A2, NULL, 4, 64, 256, NULL) == ql.Q_EINVAL
    assert ok


def test_qmatmul_static_argument_errors():
    """The no-allocation entry point checks its arguments like qmatmul_ex and
    refuses activation blocks larger than its fixed buffer, all before any
    HIP call (the pointers are never dereferenced)."""
    L = ql.lib()

    def call(fmt=0, b=A, x=A2, y=A3, M=4, N=64, K=256, path=3):
        return L.qmatmul_static(fmt, b, x, y, M, N, K, path, NULL)

    assert call(b=NULL) == ql.Q_EINVAL
    assert call(x=NULL) == ql.Q_EINVAL
    assert call(y=MIS) == ql.Q_EALIGN
    assert call(fmt=13) == ql.Q_EINVAL
    assert call(K=100) == ql.Q_ESHAPE
    assert call(M=0) == ql.Q_ESHAPE
    assert call(fmt=1, path=3) == ql.Q_ENOTSUP          # int8 path: Q8_0 weights only
    assert call(K=96) == ql.Q_ESHAPE                     # int8 path: K % 256
    assert call(path=9) == ql.Q_EINVAL
    assert call(fmt=0, path=1, M=9) == ql.Q_ESHAPE      # GEMV: M <= 8
    # the activation blocks of 8192 x 4096 (35.7 MB) exceed the 32 MiB buffer
    assert ql.workspace_bytes("q8_0", "mfma_i8", 8192, 4096) > ql.STATIC_SCRATCH_BYTES
    assert call(M=8192, K=4096) == ql.Q_ESCRATCH
    assert call(fmt=12, path=4, M=8192, K=4096) == ql.Q_ESCRATCH
    assert ql.workspace_bytes("q8_0", "mfma_i8", 7680, 4096) <= ql.STATIC_SCRATCH_BYTES


def test_probe_argument_errors():
    """The measurement aids check their arguments before any HIP call."""
    L = ql.lib()
    assert L.q_probe_read(NULL, 1024, A2, NULL) == ql.Q_EINVAL
    assert L.q_probe_read(A, 1024, NULL, NULL) == ql.Q_EINVAL
    assert L.q_probe_read(MIS, 1024, A2, NULL) == ql.Q_EALIGN
    assert L.q_probe_read(A, 1000, A2, NULL) == ql.Q_ESHAPE
    assert L.q_probe_read(A, 0, A2, NULL) == ql.Q_ESHAPE
    assert L.q_probe_mfma(NULL, 10, NULL) == ql.Q_EINVAL
    assert L.q_probe_mfma(A, -1, NULL) == ql.Q_ESHAPE
    assert L.q_probe_mfma(A, 0, NULL) == ql.Q_OK          # nothing to launch
    assert L.q_probe_mix(NULL, 10, 2, 1, NULL) == ql.Q_EINVAL
    assert L.q_probe_mix(A, -1, 2, 1, NULL) == ql.Q_ESHAPE
    assert L.q_probe_mix(A, 10, 3, 1, NULL) == ql.Q_ESHAPE
    assert L.q_probe_mix(A, 10, -1, 1, NULL) == ql.Q_ESHAPE
    assert L.q_probe_mix(A, 10, 2, 0, NULL) == ql.Q_ESHAPE
    assert L.q_probe_mix(A, 10, 2, 9, NULL) == ql.Q_ESHAPE
    assert L.q_probe_mix(A, 0, 2, 1, NULL) == ql.Q_OK     # nothing to launch
    assert L.q_probe_mix_valu(1, 2) == 256 * 2 * 4 * 4 * 16
    assert L.q_probe_mix_valu(-1, 2) == 0
    assert L.q_probe_mix_valu(1, 0) == 0
    # 1024 workgroups x 8 waves x 4 chains x 32*32*16 multiply-adds x 2
    assert L.q_probe_mfma_flops(1) == 1024 * 8 * 4 * 32 * 32 * 16 * 2
    assert L.q_probe_mfma_flops(-3) == 0


def test_embed_argument_errors():
    L = ql.lib()
    IDS = ctypes.c_void_p(0x40004)   # int32 ids need only 4-byte alignment

    def call(fmt=2, b=A, N=1000, K=512, ids=IDS, n=8, out=A3):
        return L.q_embed(fmt, b, N, K, ids, n, out, NULL)

    assert call(b=NULL) == ql.Q_EINVAL
    assert call(ids=NULL) == ql.Q_EINVAL
    assert call(out=NULL) == ql.Q_EINVAL
    assert call(fmt=13) == ql.Q_EINVAL
    assert call(fmt=11) == ql.Q_ENOTSUP                      # Q8_1: named, not implemented
    assert call(b=MIS) == ql.Q_EALIGN
    assert call(out=MIS) == ql.Q_EALIGN
    assert call(ids=ctypes.c_void_p(0x40002)) == ql.Q_EALIGN
    assert call(K=100) == ql.Q_ESHAPE
    assert call(N=0) == ql.Q_ESHAPE
    assert call(n=-1) == ql.Q_ESHAPE
    assert call(n=(1 << 24) + 1) == ql.Q_ESHAPE
    assert call(n=0) == ql.Q_OK                              # nothing to launch


def test_glu_argument_errors_and_workspace_sizes():
    L = ql.lib()

    def call(fmt=1, g=A, u=A2, x=A3, h=A, M=1, F=64, K=256, act=0, ws=NULL, wsb=0):
        return L.qmatmul_glu(fmt, g, u, x, h, M, F, K, act, ws, wsb, NULL)

    assert call(g=NULL) == ql.Q_EINVAL
    assert call(u=NULL) == ql.Q_EINVAL
    assert call(x=NULL) == ql.Q_EINVAL
    assert call(h=NULL) == ql.Q_EINVAL
    assert call(u=MIS) == ql.Q_EALIGN
    assert call(fmt=6) == ql.Q_ENOTSUP
    assert call(act=3) == ql.Q_EINVAL
    assert call(act=-1) == ql.Q_EINVAL
    assert call(K=100) == ql.Q_ESHAPE
    assert call(M=0) == ql.Q_ESHAPE
    assert call(M=5) == ql.Q_EINVAL                          # two-matmul path without a workspace
    assert call(M=5, ws=A2, wsb=4 * 5 * 64 - 1) == ql.Q_EINVAL
    assert call(M=5, ws=MIS, wsb=1 << 20) == ql.Q_EALIGN
    assert ql.glu_workspace_bytes("q4k", 2, 64, 8192) == 0   # fused kernel
    assert ql.glu_workspace_bytes("q4k", 3, 64, 256) == 0   # fused up to four tokens where X fits
    assert ql.glu_workspace_bytes("q8_0", 4, 64, 256) == 4 * 4 * 64   # four Q8_0 tokens: two-matmul path
    assert ql.glu_workspace_bytes("q4k", 5, 64, 256) == 4 * 5 * 64
    assert ql.glu_workspace_bytes("q4k", 1, 64, 8448) == 4 * 64
    assert ql.glu_workspace_bytes("q8k", 1, 64, 256) == 0
    assert ql.glu_workspace_bytes("q2k", 1, 64, 256) == 4 * 64   # generic formats: two-matmul path
    # Q8_0 rows ending in a block tail (K % 32) take both paths as well: the
    # two-matmul path needs its workspace, and an undersized one is refused
    assert ql.glu_workspace_bytes("q8_0", 5, 64, 4128) == 4 * 5 * 64
    assert ql.glu_workspace_bytes("q8_0", 2, 64, 4128) == 0      # fused kernel
    assert call(fmt=0, M=5, K=4128) == ql.Q_EINVAL
    assert call(fmt=0, M=5, K=4128, ws=A2, wsb=4 * 5 * 64 - 16) == ql.Q_EINVAL
