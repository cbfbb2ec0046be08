"""GPU parity of FP8 E4M3 with per-row scales (page "Quantization types",
section "FP8"): ISQ codes and scales bit-exact, exact dequantization, W8A16
on the generic kernels, and dynamic per-token W8A8 on the FP8 MFMA path (the
activation codes and scales in the workspace bit-exact, outputs within 1e-3
of the oracle's exact product, normalised by s_x s_w sum |e4m3 e4m3|)."""
import numpy as np
import pytest
import torch

import ggml_block_quant_amd as ql
import oracle
import synth
from gpu_util import check_outputs, to_dev_bf16
from test_parity_isq import _edge_tensor

pytestmark = pytest.mark.gpu


def _isq(w):
    return ql.isq("fp8", to_dev_bf16(w))


@pytest.mark.parametrize("N,K", [(1, 256), (7, 512), (300, 4096), (5, 14336), (3, 5120), (2, 16384), (3, 16640),
                                 (2, 24576)])
def test_isq_fp8_bit_exact(N, K):
    """Row lengths on every register-tile size of the workgroup-per-row
    kernel (K <= 16384) and on the long-row kernel beyond."""
    w = synth.weights_bf16(10000 + K + N, N, K, outliers=True)
    got = _isq(w).cpu().numpy()
    want = oracle.pack_fp8(oracle.quantize_fp8(w))
    assert np.array_equal(got, want)


def _e4m3_midpoints():
    vals = np.array(sorted({oracle.e4m3_value(c) for c in range(0x7F)}), np.float64)
    return (vals[:-1] + vals[1:]) / 2


@pytest.mark.parametrize("s", [1.0, 3.0, 7.0, 0.75])
def test_isq_fp8_ties_and_near_ties(s):
    """Rows whose quotients x / s fall exactly on E4M3 rounding midpoints
    (ties to even) or one bf16 step beside them, with s = max|x| / 448 exact:
    the kernel rounds x * (1/s) and must take the quotient wherever the two
    could round differently (for s = 3, x * (1/s) lands just above many
    midpoints that x / s hits exactly)."""
    mids = _e4m3_midpoints() * s
    x = mids.astype(np.float32)
    x = x[synth.bf16_bits_to_f32(synth.bf16_bits_from_f32(x)) == x]   # exactly representable in bf16
    b = synth.bf16_bits_from_f32(x)
    near = np.concatenate([b, b + 1, b - 1]).astype(np.uint16)        # the bf16 neighbours too
    vals = np.concatenate([near, near ^ 0x8000])                      # both signs
    K = (vals.size + 1 + 255) // 256 * 256
    row = np.zeros(K, np.uint16)
    row[: vals.size] = vals
    row[vals.size] = synth.bf16_bits_from_f32(np.array([448.0 * s], np.float32))[0]  # the row maximum: s exact
    assert synth.bf16_bits_to_f32(row[vals.size]) == np.float32(448.0 * s)
    w = np.stack([row, np.roll(row, 7)])
    got = _isq(w).cpu().numpy()
    want = oracle.pack_fp8(oracle.quantize_fp8(w))
    assert np.array_equal(got, want)


def test_isq_fp8_edge_tensor():
    """Zero rows (with -0.0), constants, one-signed rows, ties, 1e30 / 1e-6 /
    1e-30 magnitudes, isolated outliers."""
    w = _edge_tensor()
    assert np.array_equal(_isq(w).cpu().numpy(), oracle.pack_fp8(oracle.quantize_fp8(w)))


def test_fp8_dequant_and_embed_exact():
    N, K = 64, 1024
    w = synth.weights_bf16(10100, N, K, outliers=True)
    b = _isq(w)
    ref = oracle.dequant_fp8(oracle.quantize_fp8(w)).astype(np.float32)   # s * value, rounded once
    assert np.array_equal(ql.dequantize("fp8", b, N, K).cpu().numpy(), ref)
    ids = np.array([0, 63, 5, -3, 64], np.int32)
    got = ql.embed("fp8", b, N, K, torch.from_numpy(ids).cuda()).cpu().numpy()
    assert np.array_equal(got, oracle.embed(ref.astype(np.float64), ids).astype(np.float32))


def test_fp8_w8a16_paths_and_one_hot():
    for N, K in ((7, 256), (300, 1024), (129, 4096)):
        w = synth.weights_bf16(10200 + N, N, K, outliers=True)
        b = _isq(w)
        Wd = oracle.dequant_fp8(oracle.quantize_fp8(w))
        for M, path in ((1, "auto"), (2, "gemv"), (8, "gemv"), (3, "auto"), (16, "mfma_bf16"), (130, "auto")):
            x = synth.activations_bf16(10201 + M, M, K)
            Yr, den = oracle.matmul_a16(Wd, x)
            Y = ql.qmatmul("fp8", b, to_dev_bf16(x), N, path=path).cpu().numpy()
            check_outputs(Y, Yr, den, f"fp8 w8a16 {path} M={M} N={N} K={K}")
        x = np.zeros((3, K), np.uint16)
        x[[0, 1, 2], [0, 77, K - 1]] = 0x3F80
        Y = ql.qmatmul("fp8", b, to_dev_bf16(x), N, path="gemv").cpu().numpy()
        assert np.array_equal(Y, Wd[:, [0, 77, K - 1]].T.astype(np.float32))


def test_fp8_gemv_long_rows():
    """The one-shot FP8 GEMV at 5 .. 16 pieces of 1024 codes per lane and
    row (K = 5120 .. 16384, ragged N), two tokens up to K = 8192 and the
    generic kernel beyond; a one-hot X returns s * e4m3 of every column."""
    for N, K, Ms in ((129, 5120, (1, 2)), (70, 8192, (1, 2)), (33, 14336, (1, 2)), (17, 16384, (1,))):
        w = synth.weights_bf16(10250 + K, N, K, outliers=True)
        b = _isq(w)
        Wd = oracle.dequant_fp8(oracle.quantize_fp8(w))
        for M in Ms:
            x = synth.activations_bf16(10251 + M, M, K)
            Yr, den = oracle.matmul_a16(Wd, x)
            Y = ql.qmatmul("fp8", b, to_dev_bf16(x), N, path="gemv").cpu().numpy()
            check_outputs(Y, Yr, den, f"fp8 gemv M={M} N={N} K={K}")
        x = np.zeros((1, K), np.uint16)
        x[0, K - 17] = 0x3F80
        Y = ql.qmatmul("fp8", b, to_dev_bf16(x), N, path="gemv").cpu().numpy()
        assert np.array_equal(Y[0], Wd[:, K - 17].astype(np.float32))


def test_fp8_w8a8_path():
    """Dynamic per-token W8A8: the workspace holds X's E4M3 codes and
    scales bit for bit; outputs within the bar of the exact product."""
    for N, K in ((7, 256), (300, 1024), (129, 4096)):
        w = synth.weights_bf16(10300 + N, N, K, outliers=True)
        b = _isq(w)
        fw = oracle.quantize_fp8(w)
        for M in (1, 9, 16, 40, 130):
            x = synth.activations_bf16(10301 + M, M, K)
            ws = torch.empty(ql.workspace_bytes("fp8", "mfma_fp8", M, K), dtype=torch.uint8, device="cuda")
            Y = ql.qmatmul("fp8", b, to_dev_bf16(x), N, path="mfma_fp8", workspace=ws).cpu().numpy()
            fx = oracle.quantize_fp8(x)
            assert np.array_equal(ws.cpu().numpy(), oracle.pack_fp8(fx)), f"activation codes M={M} K={K}"
            Yr, den = oracle.matmul_fp8(fx, fw)
            check_outputs(Y, Yr, den, f"fp8 w8a8 M={M} N={N} K={K}")


def test_fp8_w8a8_prefill_shape_sampled():
    """The prefill shape (2048 tokens, 14336 x 4096 weights) on the W8A8
    path, checked on 2048 sampled outputs."""
    M, N, K = 2048, 14336, 4096
    w = synth.weights_bf16(10400, N, K)
    x = synth.activations_bf16(10401, M, K)
    b = _isq(w)
    ws = torch.empty(ql.workspace_bytes("fp8", "mfma_fp8", M, K), dtype=torch.uint8, device="cuda")
    Y = ql.qmatmul("fp8", b, to_dev_bf16(x), N, path="mfma_fp8", workspace=ws).cpu().numpy()
    rng = np.random.default_rng(10402)
    mi = rng.integers(0, M, 2048)
    ni = rng.integers(0, N, 2048)
    mi[:2], ni[:2] = [0, M - 1], [0, N - 1]
    rows_w, inv_w = np.unique(ni, return_inverse=True)
    rows_x, inv_x = np.unique(mi, return_inverse=True)
    fw = oracle.quantize_fp8(w[rows_w])
    fx = oracle.quantize_fp8(x[rows_x])
    Yr, den = oracle.matmul_fp8(fx, fw, inv_x, inv_w)
    check_outputs(Y[mi, ni], Yr, den, "fp8 w8a8 prefill sampled")


@pytest.mark.parametrize("M,N,K", [(2125, 7300, 512), (2304, 7169, 256)])
def test_fp8_w8a8_large_tiles_ragged(M, N, K):
    """Shapes with at least 256 tiles of 256 x 256 take the eight-wave
    kernel: ragged M and N (partial last tiles), K of 8 and 4 steps (the
    latter exactly the ring depth); sampled outputs cover every edge."""
    w = synth.weights_bf16(10500 + K, N, K, outliers=True)
    x = synth.activations_bf16(10501 + K, M, K)
    b = _isq(w)
    ws = torch.empty(ql.workspace_bytes("fp8", "mfma_fp8", M, K), dtype=torch.uint8, device="cuda")
    Y = ql.qmatmul("fp8", b, to_dev_bf16(x), N, path="mfma_fp8", workspace=ws).cpu().numpy()
    rng = np.random.default_rng(10502 + K)
    edge_m = [0, 255, 256, M - 1, M - 2, min((M // 256) * 256, M - 1)]
    edge_n = [0, 255, 256, N - 1, N - 2, min((N // 256) * 256, N - 1)]
    mi = np.concatenate([rng.integers(0, M, 3000), np.repeat(edge_m, len(edge_n))])
    ni = np.concatenate([rng.integers(0, N, 3000), np.tile(edge_n, len(edge_m))])
    rows_w, inv_w = np.unique(ni, return_inverse=True)
    rows_x, inv_x = np.unique(mi, return_inverse=True)
    fw = oracle.quantize_fp8(w[rows_w])
    fx = oracle.quantize_fp8(x[rows_x])
    Yr, den = oracle.matmul_fp8(fx, fw, inv_x, inv_w)
    check_outputs(Y[mi, ni], Yr, den, f"fp8 w8a8 large tiles M={M} N={N} K={K}")
    assert np.isfinite(Y).all()
