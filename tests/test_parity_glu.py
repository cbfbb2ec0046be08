"""GPU parity of the gated feed-forward projection (qmatmul_glu): the fused
one-shot kernel (M <= 4 where X fits its LDS budget, K <= 8192) and the two-matmul path with a
workspace, against the oracle's h* = act(g*) u*.

Bar: g and u each carry the matmul bar (1e-3 of sum_k |w||x|), so
|h - h*| <= 1e-3 * B with B the oracle's propagated bound
(oracle.glu), plus 1e-6 |h*| for the fp32 activation and product roundings
(a few ulps).  Where B = 0 (x = 0) h must be exactly 0."""
import numpy as np
import pytest
import torch

import ggml_block_quant_amd as ql
import oracle
import synth
from gpu_util import TOL, to_dev_bf16

pytestmark = pytest.mark.gpu

FMTS = ("q8_0", "q4k", "q6k")
ACTS = ("silu", "relu", "sigmoid")


def check_glu(h, h_ref, bound, label):
    h = np.asarray(h, np.float64)
    diff = np.abs(h - h_ref)
    allowed = TOL * bound + 1e-6 * np.abs(h_ref)
    zero = bound == 0
    assert np.all(h[zero] == 0), f"{label}: nonzero output where g = u = 0"
    ok = diff <= allowed
    if not ok.all():
        i = np.unravel_index(np.argmax(diff - allowed), diff.shape)
        raise AssertionError(f"{label}: |h - h*| = {diff[i]:.3e} > {allowed[i]:.3e} at {i}")


def _case(fmt, F, K, M, seed, act):
    wg = synth.weights_bf16(seed, F, K, outliers=True)
    wu = synth.weights_bf16(seed + 1, F, K)
    x = synth.activations_bf16(seed + 2, M, K)
    bg, bu = ql.isq(fmt, to_dev_bf16(wg)), ql.isq(fmt, to_dev_bf16(wu))
    h = ql.qmatmul_glu(fmt, bg, bu, to_dev_bf16(x), F, act=act).cpu().numpy()
    Wg = oracle.dequant(fmt, oracle.quantize(fmt, wg), F, K)
    Wu = oracle.dequant(fmt, oracle.quantize(fmt, wu), F, K)
    h_ref, bound = oracle.glu(Wg, Wu, x, act)
    check_glu(h, h_ref, bound, f"glu {fmt} {act} M={M} F={F} K={K}")
    return bg, bu, Wg, Wu


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("act", ACTS)
def test_glu_fused_kernel(fmt, act):
    """One to four tokens where X fits the one-shot kernel (three tokens up
    to K = 8192, four up to 6144; four Q8_0 tokens take the two-matmul
    path): no workspace."""
    assert ql.glu_workspace_bytes(fmt, 2, 300, 8192) == 0   # fused: no workspace
    assert ql.glu_workspace_bytes(fmt, 3, 300, 8192) == 0
    for F, K in ((300, 256), (1000, 1024), (129, 4096), (64, 8192)):
        for M in (1, 2, 3, 4):
            if M == 4 and K > 6144:
                continue
            _case(fmt, F, K, M, 9000 + K + M, act)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("act", ACTS)
def test_glu_two_matmul_path(fmt, act):
    """M > 4, K > 8192 or beyond the one-shot kernel's X budget: G through
    the workspace, U through H, then the elementwise pass."""
    assert ql.glu_workspace_bytes(fmt, 5, 1000, 1024) == 4 * 5 * 1000
    assert ql.glu_workspace_bytes(fmt, 4, 1000, 8192) == 4 * 4 * 1000
    assert ql.glu_workspace_bytes(fmt, 1, 64, 14336) == 4 * 64
    for F, K, M in ((1000, 1024, 5), (300, 4096, 9), (130, 512, 40), (64, 14336, 1), (200, 8192, 4)):
        _case(fmt, F, K, M, 9100 + K + M, act)


@pytest.mark.parametrize("fmt", FMTS)
def test_glu_one_hot_rounding(fmt):
    """One-hot rows make g and u the exact fp32 weights (the GEMV sums one
    product); ReLU's h = max(g, 0) * u is then one fp32 product -- equal to
    the host's, bit for bit -- and SiLU / sigmoid lie within 4 ulps of the
    host's fp32 formula.  Zero rows give exact zeros."""
    F, K = 200, 1024
    wg = synth.weights_bf16(9200, F, K)
    wu = synth.weights_bf16(9201, F, K)
    bg, bu = ql.isq(fmt, to_dev_bf16(wg)), ql.isq(fmt, to_dev_bf16(wu))
    Wg = oracle.dequant(fmt, oracle.quantize(fmt, wg), F, K).astype(np.float32)
    Wu = oracle.dequant(fmt, oracle.quantize(fmt, wu), F, K).astype(np.float32)
    for k in (0, 37, K - 1):
        x = np.zeros((2, K), np.uint16)
        x[0, k] = 0x3F80
        g, u = Wg[:, k], Wu[:, k]
        for act in ACTS:
            h = ql.qmatmul_glu(fmt, bg, bu, to_dev_bf16(x), F, act=act).cpu().numpy()
            assert not h[1].any(), "zero row"
            with np.errstate(over="ignore"):
                e = np.float32(1.0) + np.exp(-g)
                a = {"relu": np.maximum(g, np.float32(0.0)), "silu": g / e, "sigmoid": np.float32(1.0) / e}[act]
            want = (a * u).astype(np.float32)
            if act == "relu":
                assert np.array_equal(h[0], want), (fmt, act, k)
            else:
                ulp = np.spacing(np.abs(want)).astype(np.float64)
                assert np.all(np.abs(h[0].astype(np.float64) - want) <= 4 * ulp), (fmt, act, k)


def test_glu_workload_shape_sampled():
    """The FFN gate/up shape of the workload's decoder (14336 x 4096, Q4K,
    one token) on the fused kernel, checked on 256 sampled outputs."""
    F, K = 14336, 4096
    wg = synth.weights_bf16(9300, F, K)
    wu = synth.weights_bf16(9301, F, K)
    x = synth.activations_bf16(9302, 1, K)
    bg, bu = ql.isq("q4k", to_dev_bf16(wg)), ql.isq("q4k", to_dev_bf16(wu))
    h = ql.qmatmul_glu("q4k", bg, bu, to_dev_bf16(x), F, act="silu").cpu().numpy()
    rows = np.random.default_rng(9303).choice(F, 256, replace=False)
    rows[:2] = [0, F - 1]
    Wg = oracle.dequant("q4k", oracle.quantize("q4k", wg[rows]), rows.size, K)
    Wu = oracle.dequant("q4k", oracle.quantize("q4k", wu[rows]), rows.size, K)
    h_ref, bound = oracle.glu(Wg, Wu, x, "silu")
    check_glu(h[:, rows], h_ref, bound, "glu workload shape")


def test_glu_zero_input_and_argument_errors():
    F, K = 64, 256
    w = synth.weights_bf16(9400, F, K)
    b = ql.isq("q4k", to_dev_bf16(w))
    x = torch.zeros((2, K), dtype=torch.bfloat16, device="cuda")
    for act in ACTS:
        assert not ql.qmatmul_glu("q4k", b, b, x, F, act=act).any()
    with pytest.raises(ql.QLinearError):
        ql.qmatmul_glu("q4k", b, b, x, F, act=7)
    # no workspace where the two-matmul path needs one (five tokens)
    L = ql.lib()
    x5 = torch.zeros((5, K), dtype=torch.bfloat16, device="cuda")
    H = torch.empty((5, F), dtype=torch.float32, device="cuda")
    st = L.qmatmul_glu(1, b.data_ptr(), b.data_ptr(), x5.data_ptr(), H.data_ptr(), 5, F, K, 0, None, 0, None)
    assert st == ql.Q_EINVAL
