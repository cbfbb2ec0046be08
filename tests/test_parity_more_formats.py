"""GPU parity of the further formats (Q5K, Q3K, Q2K, Q4_0, Q4_1, Q5_0,
Q5_1): ISQ bytes bit-exact with the oracle's packing, exact dequantization
and embedding rows, and the generic GEMV / MFMA matmuls within the 1e-3 bar
(one-hot rows exact)."""
import numpy as np
import pytest
import torch

import ggml_block_quant_amd as ql
import oracle
import synth
from gpu_util import assert_blocks_equal, assert_split_exact, check_outputs, to_dev_bf16
from test_parity_isq import _edge_tensor

pytestmark = pytest.mark.gpu

MORE = oracle.MORE_FORMATS


def isq_host(fmt, w):
    return ql.isq(fmt, to_dev_bf16(w)).cpu().numpy()


@pytest.mark.parametrize("fmt", MORE)
def test_isq_bit_exact(fmt):
    for N, K in ((1, 256), (7, 512), (64, 1024), (300, 4096), (3, 14336)):
        w = synth.weights_bf16(9600 + K + N, N, K, outliers=True)
        assert_blocks_equal(fmt, isq_host(fmt, w), w, f"isq {N}x{K}")


@pytest.mark.parametrize("fmt", MORE)
def test_isq_edge_tensors(fmt):
    """Zeros (with -0.0), constants of both signs, one-signed rows, ties,
    1e30 / 1e-6 / 1e-30 magnitudes, isolated outliers and zero sub-blocks."""
    w = _edge_tensor()
    assert_blocks_equal(fmt, isq_host(fmt, w), w, "edge")


@pytest.mark.parametrize("fmt", MORE)
def test_isq_worked_blocks_on_gpu(fmt):
    """The hand-derived worked block of each format, quantized by the GPU."""
    import json
    import os
    from conftest import GOLDEN
    for blk in json.load(open(os.path.join(GOLDEN, "more_formats_worked.json")))["blocks"]:
        if blk["name"] != fmt:
            continue
        if "x" in blk:
            x = np.array(blk["x"] * 8, np.float32)   # the block repeated over 256 columns
        elif blk["rule"].startswith("x[32j+i]"):
            x = np.array([(i - 8) * (j + 1) * 2.0 ** -10 for j in range(8) for i in range(32)], np.float32)
        else:
            x = np.array([(i - 8) * (j + 1) * 2.0 ** -6 for j in range(16) for i in range(16)], np.float32)
        w = synth.bf16_bits_from_f32(x)[None, :]
        assert_blocks_equal(fmt, isq_host(fmt, w), w, "worked block")
        f = oracle.unpack(fmt, isq_host(fmt, w), 1, 256)
        assert f["q"][0][: len(blk["q"])].tolist() == blk["q"]


@pytest.mark.parametrize("fmt", MORE)
def test_dequantize_and_embed_exact(fmt):
    N, K = 48, 1024
    w = synth.weights_bf16(9700, N, K, outliers=True)
    blocks = ql.isq(fmt, to_dev_bf16(w))
    ref = oracle.dequant(fmt, oracle.quantize(fmt, w), N, K).astype(np.float32)
    assert np.array_equal(ql.dequantize(fmt, blocks, N, K).cpu().numpy(), ref)
    ids = np.array([3, 0, 47, -1, 47, 48, 20], np.int32)
    got = ql.embed(fmt, blocks, N, K, torch.from_numpy(ids).cuda()).cpu().numpy()
    assert np.array_equal(got, oracle.embed(ref.astype(np.float64), ids).astype(np.float32))


@pytest.mark.parametrize("fmt", MORE)
def test_matmul_paths(fmt):
    """Generic GEMV (explicit path, M = 1..8; AUTO for M <= 2) and generic
    MFMA GEMM (M up to 130, K splits) on ragged shapes."""
    for N, K in ((7, 256), (300, 1024), (129, 4096)):
        w = synth.weights_bf16(9800 + N, N, K, outliers=True)
        blocks = ql.isq(fmt, to_dev_bf16(w))
        Wd = oracle.dequant(fmt, oracle.quantize(fmt, w), N, K)
        for M, path in ((1, "gemv"), (2, "auto"), (3, "gemv"), (8, "gemv"), (1, "mfma_bf16"), (3, "auto"),
                        (16, "mfma_bf16"), (40, "auto"), (130, "mfma_bf16")):
            x = synth.activations_bf16(9801 + M, M, K)
            Yr, den = oracle.matmul_a16(Wd, x)
            Y = ql.qmatmul(fmt, blocks, to_dev_bf16(x), N, path=path).cpu().numpy()
            check_outputs(Y, Yr, den, f"{fmt} {path} M={M} N={N} K={K}")


@pytest.mark.parametrize("fmt", MORE)
def test_one_hot_exact(fmt):
    """One-hot rows: the GEMV returns the fp32 weight exactly (one product,
    sums of zeros), the MFMA path its hi + lo bf16 pair (within 2^-17)."""
    N, K = 70, 512
    w = synth.weights_bf16(9900, N, K, outliers=True)
    blocks = ql.isq(fmt, to_dev_bf16(w))
    Wf = oracle.dequant(fmt, oracle.quantize(fmt, w), N, K).astype(np.float32)
    for ks in ((0, 1, 2, 3, 255, 256, 300, 511), (4, 5, 6, 7, 12, 13, 14, 15)):  # every element of a task
        x = np.zeros((len(ks), K), np.uint16)
        x[np.arange(len(ks)), list(ks)] = 0x3F80
        Yg = ql.qmatmul(fmt, blocks, to_dev_bf16(x), N, path="gemv").cpu().numpy()
        assert np.array_equal(Yg, Wf[:, list(ks)].T)
        Ym = ql.qmatmul(fmt, blocks, to_dev_bf16(x), N, path="mfma_bf16").cpu().numpy()
        assert_split_exact(Ym, Wf[:, list(ks)].T, f"{fmt} mfma one-hot")


@pytest.mark.parametrize("fmt", MORE)
def test_glu_on_further_formats(fmt):
    """The gated projection takes its two-matmul path for these formats."""
    F, K, M = 200, 1024, 1
    wg = synth.weights_bf16(9950, F, K)
    wu = synth.weights_bf16(9951, F, K)
    x = synth.activations_bf16(9952, M, K)
    bg, bu = ql.isq(fmt, to_dev_bf16(wg)), ql.isq(fmt, to_dev_bf16(wu))
    h = ql.qmatmul_glu(fmt, bg, bu, to_dev_bf16(x), F, act="silu").cpu().numpy()
    Wg = oracle.dequant(fmt, oracle.quantize(fmt, wg), F, K)
    Wu = oracle.dequant(fmt, oracle.quantize(fmt, wu), F, K)
    h_ref, bound = oracle.glu(Wg, Wu, x, "silu")
    assert np.all(np.abs(h - h_ref) <= 1e-3 * bound + 1e-6 * np.abs(h_ref))
