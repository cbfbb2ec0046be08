"""The entry point that allocates nothing, qmatmul_static, through the C ABI:
its int8 (Q8_0 x Q8_0) and FP8 W8A8 paths keep X's activation blocks in the
library's fixed per-GPU buffer instead of a caller workspace.  Compared with
qmatmul_ex on the same inputs (the same kernels, which take the workspace
from the caller) and with the oracle, on two calls in a row, the second with
a smaller input, so that a stale buffer would show; the paths without a
workspace must give qmatmul_ex's results bit for bit."""
import numpy as np
import pytest
import torch

import ggml_block_quant_amd as ql
import oracle
import synth
from gpu_util import check_outputs, to_dev_bf16

pytestmark = pytest.mark.gpu

# (M, N, K): a K-split shape first, then a smaller one
SHAPES = ((300, 520, 4096), (7, 130, 1024))


def _oracle(fmt, w, x):
    M, K = x.shape
    N = w.shape[0]
    if fmt == "q8_0":
        return oracle.matmul_a8(oracle.quantize("q8_0", w), oracle.quantize("q8_0", x), M, N, K)
    return oracle.matmul_fp8(oracle.quantize_fp8(x), oracle.quantize_fp8(w))


@pytest.mark.parametrize("fmt,path", [("q8_0", "mfma_i8"), ("fp8", "mfma_fp8")])
def test_static_scratch_matches_caller_workspace(fmt, path):
    for i, (M, N, K) in enumerate(SHAPES):
        print(f"qmatmul_static {fmt} {path} M={M} N={N} K={K}", flush=True)
        w = synth.weights_bf16(8100 + i, N, K, outliers=True)
        x = synth.activations_bf16(8200 + i, M, K)
        blocks = ql.isq(fmt, to_dev_bf16(w))
        X = to_dev_bf16(x)
        out = torch.empty((M, N), dtype=torch.float32, device="cuda")
        a = ql.qmatmul_static(fmt, blocks, X, N, path=path, out=out).cpu().numpy()
        b = ql.qmatmul(fmt, blocks, X, N, path=path).cpu().numpy()
        Yr, den = _oracle(fmt, w, x)
        # same kernels; only the order of fp32 atomic adds of K splits may differ
        e = oracle.normalized_error(a, b, den)
        assert e.max() <= 1e-6, (fmt, M, N, K, e.max())
        check_outputs(a, Yr, den, f"qmatmul_static {fmt} M={M} N={N} K={K}")


@pytest.mark.parametrize("fmt,path", [("q4k", "gemv"), ("q6k", "mfma_bf16"), ("q8_0", "auto")])
def test_static_other_paths_equal_qmatmul_ex(fmt, path):
    """Paths without a workspace run exactly as in qmatmul_ex: the GEMV bit
    for bit; the MFMA kernels up to the order of their K splits' fp32
    atomic adds."""
    M = 4 if path == "gemv" else 40
    N, K = 96, 1024
    w = synth.weights_bf16(8300, N, K)
    x = synth.activations_bf16(8301, M, K)
    blocks = ql.isq(fmt, to_dev_bf16(w))
    X = to_dev_bf16(x)
    a = ql.qmatmul_static(fmt, blocks, X, N, path=path)
    b = ql.qmatmul(fmt, blocks, X, N, path=path)
    if path == "gemv":
        assert torch.equal(a, b), (fmt, path)
    else:
        _, den = oracle.matmul_a16(oracle.dequant(fmt, oracle.quantize(fmt, w), N, K), x)
        e = oracle.normalized_error(a.cpu().numpy(), b.cpu().numpy(), den)
        assert e.max() <= 1e-6, (fmt, path, e.max())


def test_static_rejects_oversized_activations():
    M, N, K = 8192, 64, 4096
    X = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    blocks = ql.isq("q8_0", torch.zeros((N, K), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ql.QLinearError) as err:
        ql.qmatmul_static("q8_0", blocks, X, N, path="mfma_i8")
    assert err.value.status == ql.Q_ESCRATCH
