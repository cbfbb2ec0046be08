"""GPU parity of the quantized matmuls against the fp64 oracle:
  * GEMV (M <= 8) and the bf16 MFMA path against the A16 oracle
    (exact dequantized weights times bf16 activations);
  * the int8 MFMA path against the A8 oracle (activations quantized to
    Q8_0 as well), and its activation blocks bit-exact;
every output within 1e-3 of the oracle, normalised by sum |w||x|."""
import numpy as np
import pytest
import torch

import ggml_block_quant_amd as ql
import oracle
import synth
from gpu_util import TOL, assert_blocks_equal, assert_split_exact, check_outputs, to_dev_bf16

pytestmark = pytest.mark.gpu

FMTS = ("q8_0", "q4k", "q6k")


def run(fmt, path, w, x):
    N, K = w.shape
    blocks = ql.isq(fmt, to_dev_bf16(w))
    Y = ql.qmatmul(fmt, blocks, to_dev_bf16(x), N, path=path)
    return Y.cpu().numpy()


def a16_ref(fmt, w, x):
    N, K = w.shape
    return oracle.matmul_a16(oracle.dequant(fmt, oracle.quantize(fmt, w), N, K), x)


def a8_ref(w, x):
    N, K = w.shape
    M = x.shape[0]
    return oracle.matmul_a8(oracle.quantize("q8_0", w), oracle.quantize("q8_0", x), M, N, K)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("K", [256, 1024, 4096, 5120, 14336])
def test_gemv_shapes(fmt, K):
    for M in (1, 2, 3, 4, 5, 8):
        for N in (1, 7, 300):
            w = synth.weights_bf16(1000 + K + N, N, K)
            x = synth.activations_bf16(2000 + M, M, K)
            y = run(fmt, "gemv", w, x)
            Yr, den = a16_ref(fmt, w, x)
            check_outputs(y, Yr, den, f"gemv {fmt} M={M} N={N} K={K}")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_long_rows(fmt):
    """K = 20480 (two chunks per lane over 8 waves) and K = 32768 (M = 1,
    four chunks per lane)."""
    for M, K in ((1, 20480), (4, 20480), (1, 32768)):
        if fmt == "q8_0" and M > 1:
            continue  # Q8_0 keeps one chunk of X per lane for M > 1
        w = synth.weights_bf16(3000 + K, 64, K)
        x = synth.activations_bf16(3001, M, K)
        Yr, den = a16_ref(fmt, w, x)
        check_outputs(run(fmt, "gemv", w, x), Yr, den, f"gemv {fmt} M={M} K={K}")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_row_runs_one_hot(fmt):
    """K = 5120 (160 chunks a row), M = 1: the four rows of a wave form one
    run of 640 chunks, ten per lane, and the items at lanes 0..31 / 32..63
    of the third and eighth step fall in different rows.  One-hot X at
    chunk boundaries and inside those items returns every weight column
    bit for bit, for rows at each position of the run (N = 8201: row runs
    from 8192 rows, and a last run shifted back to end at the last row)."""
    N, K = 8201, 5120
    w = synth.weights_bf16(4100, N, K, outliers=True)
    blocks = ql.isq(fmt, to_dev_bf16(w))
    Wref = oracle.dequant(fmt, oracle.quantize(fmt, w), N, K).astype(np.float32)
    for k in (0, 31, 32, 1023, 1024, 2047, 4095, 4096, 4127, 4128, 5119):
        x = np.zeros((1, K), np.uint16)
        x[0, k] = 0x3F80
        y = ql.qmatmul(fmt, blocks, to_dev_bf16(x), N, path="gemv").cpu().numpy()
        assert np.array_equal(y[0], Wref[:, k]), f"{fmt} k={k}"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("K", [1024, 4096, 5120, 14336])
def test_gemv_wide_weights(fmt, K):
    """From 8192 rows a wave takes two or four rows (as one run of chunks at
    the widths where that measured faster), for one to four tokens where the
    one-shot kernel takes them: N = 8195 leaves a partial last workgroup
    (K = 14336 keeps one row per wave at any N: 2051 rows); random X within
    the bar, and one-hot X at the first, a middle and the last element exact
    in every token row."""
    N = 8195 if K <= 5120 else 2051
    w = synth.weights_bf16(4300 + K, N, K, outliers=True)
    blocks = ql.isq(fmt, to_dev_bf16(w))
    Wd = oracle.dequant(fmt, oracle.quantize(fmt, w), N, K)
    Wf = Wd.astype(np.float32)
    for M in ((1, 2, 3, 4) if K <= 5120 else (1, 2)):
        x = synth.activations_bf16(4301 + M, M, K)
        Yr, den = oracle.matmul_a16(Wd, x)
        y = ql.qmatmul(fmt, blocks, to_dev_bf16(x), N, path="gemv").cpu().numpy()
        check_outputs(y, Yr, den, f"gemv wide {fmt} M={M} K={K}")
        for k in (0, K // 2 + 5, K - 1):
            x = np.zeros((M, K), np.uint16)
            for m in range(M):
                x[m, (k + 33 * m) % K] = 0x3F80
            y = ql.qmatmul(fmt, blocks, to_dev_bf16(x), N, path="gemv").cpu().numpy()
            for m in range(M):
                assert np.array_equal(y[m], Wf[:, (k + 33 * m) % K]), f"{fmt} M={M} m={m} K={K} k={k}"


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_one_hot_is_exact(fmt):
    """X = e_k: the GEMV must return the fp32 value of the dequantized weight
    bit for bit (products with 1 and sums of zeros are exact), for every
    position k of a 256-element group -- this pins the decoding of every
    nibble, high-bit field and 6-bit scale of the layout."""
    N, K = 40, 512
    w = synth.weights_bf16(4000, N, K, outliers=True)
    blocks = ql.isq(fmt, to_dev_bf16(w))
    Wref = oracle.dequant(fmt, oracle.quantize(fmt, w), N, K).astype(np.float32)
    for k0 in range(0, 512, 8):
        x = np.zeros((8, K), np.uint16)
        for m in range(8):
            x[m, k0 + m] = 0x3F80  # 1.0
        Y = ql.qmatmul(fmt, blocks, to_dev_bf16(x), N, path="gemv").cpu().numpy()
        assert np.array_equal(Y, Wref[:, k0:k0 + 8].T), f"{fmt} k0={k0}"


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_one_and_two_tokens_all_widths(fmt):
    """One- and two-token GEMVs stage X in LDS with one to eight chunks of 32
    per lane (K = 32*64*CPT at most); K = 8192 ... 16384 complete the widths
    the shape test does not reach, with ragged N and rows past the last
    full workgroup."""
    for K in (8192, 10240, 12288, 16384):
        for M in (1, 2):
            for N in (1, 9, 300):
                w = synth.weights_bf16(5000 + K + N, N, K, outliers=True)
                x = synth.activations_bf16(5001 + M, M, K)
                Yr, den = a16_ref(fmt, w, x)
                check_outputs(run(fmt, "gemv", w, x), Yr, den, f"gemv {fmt} M={M} N={N} K={K}")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_three_four_tokens_wide(fmt):
    """Three and four tokens around the one-shot kernel's LDS budget (M times
    chunks per lane at most 14): K = 6144 (three chunks per lane, both M
    one-shot), K = 6400 (200 chunks in four slots per lane, ragged: three
    tokens one-shot, four on the persistent kernel) and K = 8192 (likewise),
    ragged N, on the GEMV path and on AUTO."""
    for K, Ms in ((6144, (3, 4)), (6400, (3, 4)), (8192, (3, 4))):
        for M in Ms:
            for N in (5, 300):
                w = synth.weights_bf16(5100 + K + N, N, K, outliers=True)
                x = synth.activations_bf16(5101 + M, M, K)
                Yr, den = a16_ref(fmt, w, x)
                for path in ("gemv", "auto"):
                    check_outputs(run(fmt, path, w, x), Yr, den, f"{path} {fmt} M={M} N={N} K={K}")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_five_to_eight_tokens(fmt):
    """Five to eight tokens at up to two chunks per lane (K = 2048, 4096):
    Q4K and Q6K on the one-shot kernel (X staged in LDS, one row per wave
    below 8192 rows, two from 8192), Q8_0 on the persistent kernel; ragged
    N, on the GEMV path and on AUTO."""
    for K in (2048, 4096):
        for M in (5, 6, 7, 8):
            for N in (300, 8196):
                w = synth.weights_bf16(5300 + K + N, N, K, outliers=True)
                x = synth.activations_bf16(5301 + M, M, K)
                Yr, den = a16_ref(fmt, w, x)
                for path in ("gemv", "auto"):
                    check_outputs(run(fmt, path, w, x), Yr, den, f"{path} {fmt} M={M} N={N} K={K}")


@pytest.mark.parametrize("fmt", ["q4k", "q6k"])
@pytest.mark.parametrize("M", [5, 8])
def test_gemv_one_hot_is_exact_five_eight_tokens(fmt, M):
    """The one-hot pin for the one-shot kernel at five and eight tokens."""
    N, K = 40, 4096
    w = synth.weights_bf16(4300 + M, N, K, outliers=True)
    blocks = ql.isq(fmt, to_dev_bf16(w))
    Wref = oracle.dequant(fmt, oracle.quantize(fmt, w), N, K).astype(np.float32)
    for k in list(range(0, 256, 5)) + list(range(2048, 2304, 7)) + [3000, 4095]:
        x = np.zeros((M, K), np.uint16)
        for m in range(M):
            x[m, (k + 37 * m) % K] = 0x3F80  # 1.0
        Y = ql.qmatmul(fmt, blocks, to_dev_bf16(x), N, path="gemv").cpu().numpy()
        for m in range(M):
            km = (k + 37 * m) % K
            assert np.array_equal(Y[m], Wref[:, km]), f"{fmt} M={M} m={m} k={km}"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_gemv_one_hot_is_exact_one_two_tokens(fmt, M):
    """The one-hot pin for the one-shot kernel (one to four tokens; four
    Q8_0 tokens take the persistent kernel): every position of the first
    256-element group, and positions of the second chunk slot of each lane
    (K = 4096: chunks 64..127) and the row's last element, must return the
    dequantized weight bit for bit, in every token row."""
    N, K = 40, 4096
    w = synth.weights_bf16(4200 + M, N, K, outliers=True)
    blocks = ql.isq(fmt, to_dev_bf16(w))
    Wref = oracle.dequant(fmt, oracle.quantize(fmt, w), N, K).astype(np.float32)
    ks = list(range(0, 256)) + list(range(2048, 2304, 3)) + [3000, 4095]
    for k in ks:
        x = np.zeros((M, K), np.uint16)
        for m in range(M):
            x[m, (k + 37 * m) % K] = 0x3F80  # 1.0
        Y = ql.qmatmul(fmt, blocks, to_dev_bf16(x), N, path="gemv").cpu().numpy()
        for m in range(M):
            km = (k + 37 * m) % K
            assert np.array_equal(Y[m], Wref[:, km]), f"{fmt} M={M} m={m} k={km}"


@pytest.mark.parametrize("fmt", FMTS)
def test_mfma_bf16_one_hot(fmt):
    """Same pin for the bf16 MFMA path: one-hot rows give every weight to
    within 2^-17 of its value (the hi + lo bf16 pair of the kernels)."""
    N, K = 130, 512
    w = synth.weights_bf16(4100, N, K, outliers=True)
    blocks = ql.isq(fmt, to_dev_bf16(w))
    Wref = oracle.dequant(fmt, oracle.quantize(fmt, w), N, K).astype(np.float32)
    x = np.zeros((K, K), np.uint16)
    x[np.arange(K), np.arange(K)] = 0x3F80
    Y = ql.qmatmul(fmt, blocks, to_dev_bf16(x), N, path="mfma_bf16").cpu().numpy()
    assert_split_exact(Y, Wref.T, f"mfma one-hot {fmt}")


@pytest.mark.parametrize("fmt", FMTS)
def test_mfma_bf16_shapes(fmt):
    for M in (9, 16, 17, 64, 100, 128, 200):
        for N, K in ((7, 256), (64, 1024), (300, 4096), (129, 512)):
            w = synth.weights_bf16(5000 + N, N, K)
            x = synth.activations_bf16(5001 + M, M, K)
            Yr, den = a16_ref(fmt, w, x)
            check_outputs(run(fmt, "mfma_bf16", w, x), Yr, den, f"mfma_bf16 {fmt} M={M} N={N} K={K}")


@pytest.mark.parametrize("fmt", FMTS)
def test_mfma_bf16_prefill_tiles(fmt):
    """Large-M paths: 65..512 tokens on 128 x 256 tiles and from 513 tokens
    on 256 x 256 tiles, each split over K when the tiles are few; ragged M
    and N around the tile edges, K with one, two and eight splits."""
    for M, N, K in ((128, 255, 256), (257, 513, 1024), (600, 300, 4096), (300, 1, 768), (129, 1000, 4096),
                    (65, 257, 512), (512, 300, 1024), (513, 255, 256), (777, 513, 1024), (1100, 1, 768),
                    (2049, 130, 512)):
        w = synth.weights_bf16(5100 + N + K, N, K, outliers=True)
        x = synth.activations_bf16(5101 + M, M, K)
        Yr, den = a16_ref(fmt, w, x)
        check_outputs(run(fmt, "mfma_bf16", w, x), Yr, den, f"prefill tiles {fmt} M={M} N={N} K={K}")


@pytest.mark.parametrize("fmt", FMTS)
def test_mfma_bf16_batched_stream(fmt):
    """Batched-decode path (3..32 tokens, more than 2^24 weights): ragged N
    past the 64-row tiles, K split over workgroups, one and two m-tiles."""
    N, K = 4100, 4352
    w = synth.weights_bf16(5200, N, K, outliers=True)
    for M in (3, 17, 32):
        x = synth.activations_bf16(5201 + M, M, K)
        Yr, den = a16_ref(fmt, w, x)
        check_outputs(run(fmt, "mfma_bf16", w, x), Yr, den, f"batched stream {fmt} M={M}")


def test_mfma_bf16_q4k_quad_stream():
    """Q4K batched decode through the exact-code kernel (up to 32 tokens,
    more than 2^24 weights): K = 14336, 16384, 5120 and 4096 split over
    workgroups, rows ragged past the 16- and 64-row tiles.  One-hot rows pin
    the layout: every weight to within 2^-17 of its value (the kernel gives
    the fp32 weight itself: exact products, one rounding of S u - Mn)."""
    for N, K, Ms in ((1300, 14336, (1, 3, 4, 7, 16)), (1100, 16384, (2, 4)), (3300, 5120, (4, 13)),
                     (4150, 4096, (2, 9))):
        w = synth.weights_bf16(5300 + K, N, K, outliers=True)
        blocks = ql.isq("q4k", to_dev_bf16(w))
        Wd = oracle.dequant("q4k", oracle.quantize("q4k", w), N, K)
        for M in Ms:
            x = synth.activations_bf16(5301 + M, M, K)
            Yr, den = oracle.matmul_a16(Wd, x)
            Y = ql.qmatmul("q4k", blocks, to_dev_bf16(x), N, path="mfma_bf16").cpu().numpy()
            check_outputs(Y, Yr, den, f"quad stream q4k M={M} N={N} K={K}")
        ks = np.array([0, 33, K // 2 + 7, K - 1])
        x = np.zeros((4, K), np.uint16)
        x[np.arange(4), ks] = 0x3F80
        Y = ql.qmatmul("q4k", blocks, to_dev_bf16(x), N, path="mfma_bf16").cpu().numpy()
        assert_split_exact(Y, Wd[:, ks].astype(np.float32).T, f"quad stream one-hot N={N} K={K}")


def test_q8_0_block_tails():
    """Q8_0 rows of K % 32 == 0 that are not whole 256-element groups: ISQ
    and dequantization exact, GEMV (M = 1, 2 on the one-shot kernel, 3 and 8
    on the persistent one) and the MFMA path (the generic kernel) within the
    bar, one-hot columns exact on the GEMV."""
    for N, K in ((7, 32), (300, 96), (129, 992), (65, 4128)):
        w = synth.weights_bf16(5200 + K, N, K, outliers=True)
        blocks = ql.isq("q8_0", to_dev_bf16(w))
        assert_blocks_equal("q8_0", blocks.cpu().numpy(), w, f"isq K={K}")
        Wd = oracle.dequant("q8_0", oracle.quantize("q8_0", w), N, K)
        assert np.array_equal(ql.dequantize("q8_0", blocks, N, K).cpu().numpy(), Wd.astype(np.float32))
        for M, path in ((1, "gemv"), (2, "auto"), (3, "gemv"), (8, "gemv"), (3, "auto"), (16, "mfma_bf16"),
                        (130, "auto")):
            x = synth.activations_bf16(5201 + M, M, K)
            Yr, den = oracle.matmul_a16(Wd, x)
            Y = ql.qmatmul("q8_0", blocks, to_dev_bf16(x), N, path=path).cpu().numpy()
            check_outputs(Y, Yr, den, f"q8_0 tail {path} M={M} N={N} K={K}")
        x = np.zeros((2, K), np.uint16)
        x[0, 0], x[1, K - 1] = 0x3F80, 0x3F80
        Y = ql.qmatmul("q8_0", blocks, to_dev_bf16(x), N, path="gemv").cpu().numpy()
        assert np.array_equal(Y, Wd[:, [0, K - 1]].T.astype(np.float32))


def test_mfma_i8_shapes_and_activation_blocks():
    """Ragged tiles and K splits; K = 1280 with one tile splits 40 steps of
    one block into 16 runs of 3, the last two of them empty."""
    for M in (1, 9, 16, 64, 130, 256):
        for N, K in ((7, 256), (64, 1024), (300, 4096), (129, 512), (7, 1280), (200, 768)):
            w = synth.weights_bf16(6000 + N, N, K)
            x = synth.activations_bf16(6001 + M, M, K)
            ws = torch.empty(ql.workspace_bytes("q8_0", "mfma_i8", M, K), dtype=torch.uint8, device="cuda")
            blocks = ql.isq("q8_0", to_dev_bf16(w))
            Y = ql.qmatmul("q8_0", blocks, to_dev_bf16(x), N, path="mfma_i8", workspace=ws).cpu().numpy()
            # the activation blocks left in the workspace are X's Q8_0 blocks, bit for bit
            assert_blocks_equal("q8_0", ws.cpu().numpy(), x, "activation quantization")
            Yr, den = a8_ref(w, x)
            check_outputs(Y, Yr, den, f"mfma_i8 M={M} N={N} K={K}")


def test_act_quantize_entry_point():
    x = synth.activations_bf16(6100, 37, 1024)
    assert_blocks_equal("q8_0", ql.act_quantize(to_dev_bf16(x)).cpu().numpy(), x, "q_act_quantize")


@pytest.mark.parametrize("fmt", FMTS)
def test_auto_path_dispatch(fmt):
    """AUTO = GEMV for M <= 2, and for 3 or 4 tokens where the one-shot GEMV
    takes the shape (K = 1024 here; four Q8_0 tokens excepted) -- bit for
    bit, the GEMV is deterministic -- and the bf16 MFMA GEMM above (equal up
    to the order of fp32 sums, so compared to 1e-6 of sum |w||x|)."""
    N, K = 200, 1024
    w = synth.weights_bf16(7000, N, K)
    blocks = ql.isq(fmt, to_dev_bf16(w))
    for M, path in ((1, "gemv"), (2, "gemv"), (3, "gemv"), (4, "mfma_bf16" if fmt == "q8_0" else "gemv"),
                    (5, "mfma_bf16"), (8, "mfma_bf16"), (9, "mfma_bf16"), (100, "mfma_bf16")):
        x = synth.activations_bf16(7001, M, K)
        X = to_dev_bf16(x)
        a = ql.qmatmul(fmt, blocks, X, N, path="auto")
        b = ql.qmatmul(fmt, blocks, X, N, path=path)
        if path == "gemv":
            assert torch.equal(a, b), (fmt, M)
        else:
            _, den = a16_ref(fmt, w, x)
            e = oracle.normalized_error(a.cpu().numpy(), b.cpu().numpy(), den)
            assert e.max() <= 1e-6, (fmt, M, e.max())


@pytest.mark.parametrize("path", ["gemv", "mfma_bf16", "mfma_i8"])
def test_zero_inputs_give_zero(path):
    fmt = "q8_0" if path == "mfma_i8" else "q4k"
    M = 4 if path == "gemv" else 32
    N, K = 70, 512
    w = synth.weights_bf16(7100, N, K)
    w[5] = 0  # an all-zero weight row
    x = synth.activations_bf16(7101, M, K)
    x[1] = 0  # an all-zero activation row
    y = run(fmt, path, w, x)
    assert (y[1] == 0).all() and (y[:, 5] == 0).all()


def test_gemv_is_deterministic():
    w = synth.weights_bf16(7200, 512, 4096)
    x = synth.activations_bf16(7201, 3, 4096)
    blocks = ql.isq("q4k", to_dev_bf16(w))
    X = to_dev_bf16(x)
    a = ql.qmatmul("q4k", blocks, X, 512, path="gemv")
    b = ql.qmatmul("q4k", blocks, X, 512, path="gemv")
    assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# full-size workloads
# ---------------------------------------------------------------------------

def test_workload_gemv_1024_q8_0():
    w = synth.weights_bf16(synth.seed_for(1, 0), 1024, 1024)
    x = synth.activations_bf16(synth.seed_for(1, 1), 1, 1024)
    Yr, den = a16_ref("q8_0", w, x)
    check_outputs(run("q8_0", "auto", w, x), Yr, den, "1024x1024 q8_0")


def test_workload_gemv_ffn_up_q4k_and_q8_0():
    w = synth.weights_bf16(synth.seed_for(2, 0), 14336, 4096)
    x = synth.activations_bf16(synth.seed_for(2, 1), 1, 4096)
    for fmt in ("q4k", "q8_0"):
        Yr, den = a16_ref(fmt, w, x)
        check_outputs(run(fmt, "auto", w, x), Yr, den, f"14336x4096 {fmt} M=1")


def test_workload_batched_decode_down_proj():
    """M in {4, 16, 64} x K = 14336 x N = 4096, Q4K weights with 1 % outliers
    at 10 sigma, on the AUTO path (bf16 MFMA for all three) and, for M = 4,
    also on the GEMV."""
    w = synth.weights_bf16(synth.seed_for(3, 0), 4096, 14336, outliers=True)
    x = synth.activations_bf16(synth.seed_for(3, 1), 64, 14336)
    W = oracle.dequant("q4k", oracle.quantize("q4k", w), 4096, 14336)
    blocks = ql.isq("q4k", to_dev_bf16(w))
    for M in (4, 16, 64):
        Yr, den = oracle.matmul_a16(W, x[:M])
        y = ql.qmatmul("q4k", blocks, to_dev_bf16(x[:M]), 4096).cpu().numpy()
        check_outputs(y, Yr, den, f"down-proj M={M}")
        if M == 4:
            y = ql.qmatmul("q4k", blocks, to_dev_bf16(x[:M]), 4096, path="gemv").cpu().numpy()
            check_outputs(y, Yr, den, "down-proj M=4 gemv")


def test_qkv_concatenated_launch():
    """The q, k and v projections of a layer quantized as one [6144][4096]
    Q4K tensor: its blocks are the three tensors' blocks row after row (ISQ
    works per row), and one launch gives every output within the bar, for
    one to four tokens on AUTO and on the GEMV path."""
    parts = [synth.weights_bf16(synth.seed_for(2, 10 + t), n, 4096) for t, n in enumerate((4096, 1024, 1024))]
    w = np.concatenate(parts)
    blocks = ql.isq("q4k", to_dev_bf16(w)).cpu().numpy()
    r0 = 0
    for t, wt in enumerate(parts):
        rows = np.arange(r0, r0 + wt.shape[0])
        sep = ql.isq("q4k", to_dev_bf16(wt)).cpu().numpy()
        assert np.array_equal(oracle.rows_of_buffer("q4k", blocks, 6144, 4096, rows), sep), f"part {t}"
        r0 += wt.shape[0]
    W = oracle.dequant("q4k", oracle.quantize("q4k", w), 6144, 4096)
    x = synth.activations_bf16(synth.seed_for(2, 13), 4, 4096)
    dev = torch.from_numpy(blocks).cuda()
    for M in (1, 2, 3, 4):
        Yr, den = oracle.matmul_a16(W, x[:M])
        for path in ("auto", "gemv"):
            y = ql.qmatmul("q4k", dev, to_dev_bf16(x[:M]), 6144, path=path).cpu().numpy()
            check_outputs(y, Yr, den, f"qkv 6144x4096 M={M} {path}")


def _sampled(N, M, count, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, M, count), rng.integers(0, N, count)


@pytest.mark.parametrize("fmt,M,N,K", [("q4k", 100, 8300, 4096), ("q6k", 300, 8200, 4352), ("q8_0", 257, 9000, 4096)])
def test_mid_token_counts_wide_weights(fmt, M, N, K):
    """65..512 tokens on weights above 2^25 elements (128 x 256 tiles, K split
    as far as one workgroup per CU): ragged M and N, 3000 sampled outputs
    plus every edge row and column pair."""
    w = synth.weights_bf16(5600 + M, N, K, outliers=True)
    x = synth.activations_bf16(5601 + M, M, K)
    blocks = ql.isq(fmt, to_dev_bf16(w))
    y = ql.qmatmul(fmt, blocks, to_dev_bf16(x), N).cpu().numpy()
    mi, ni = _sampled(N, M, 3000, 5602 + M)
    em, en = [0, min(127, M - 1), min(128, M - 1), M - 1], [0, 255, 256, N - 1]
    mi = np.concatenate([mi, np.repeat(em, len(en))])
    ni = np.concatenate([ni, np.tile(en, len(em))])
    rows, inv = np.unique(ni, return_inverse=True)
    Wr = oracle.dequant(fmt, oracle.quantize(fmt, w[rows]), len(rows), K)
    Yr, den = oracle.matmul_a16_pairs(Wr, x, mi, inv)
    check_outputs(y[mi, ni], Yr, den, f"mid tokens {fmt} M={M} N={N} K={K}")


def test_workload_prefill_2048_both_paths():
    """M = 2048 x K = 4096 x N = 14336, Q8_0 weights; the bf16 MFMA path and
    the int8 path, checked on 4096 sampled outputs (rows of W quantized by
    the oracle one by one)."""
    M, N, K = 2048, 14336, 4096
    w = synth.weights_bf16(synth.seed_for(4, 0), N, K)
    x = synth.activations_bf16(synth.seed_for(4, 1), M, K)
    blocks = ql.isq("q8_0", to_dev_bf16(w))
    X = to_dev_bf16(x)
    mi, ni = _sampled(N, M, 4096, 11)
    rows, inv = np.unique(ni, return_inverse=True)
    fw = oracle.quantize("q8_0", w[rows])
    Wr = oracle.dequant("q8_0", fw, len(rows), K)
    Yr, den = oracle.matmul_a16_pairs(Wr, x, mi, inv)
    y = ql.qmatmul("q8_0", blocks, X, N, path="mfma_bf16").cpu().numpy()
    check_outputs(y[mi, ni], Yr, den, "prefill bf16")
    ws = torch.empty(ql.workspace_bytes("q8_0", "mfma_i8", M, K), dtype=torch.uint8, device="cuda")
    y8 = ql.qmatmul("q8_0", blocks, X, N, path="mfma_i8", workspace=ws).cpu().numpy()
    fx = oracle.quantize("q8_0", x)
    assert_blocks_equal("q8_0", ws.cpu().numpy(), x, "prefill activations")
    Y8, den8 = oracle.matmul_a8(fw, fx, M, len(rows), K, mi=mi, ni=inv)
    check_outputs(y8[mi, ni], Y8, den8, "prefill int8")


def test_workload_lm_head_q6k_m1_m8():
    """131072 x 5120 output head in Q6K, M = 1 and M = 8, on 512 sampled rows."""
    N, K = 131072, 5120
    W = synth.device_normal_bf16(synth.LM_HEAD_W_SEED, (N, K), synth.W_SIGMA)
    blocks = ql.isq("q6k", W)
    x = synth.activations_bf16(synth.LM_HEAD_X_SEED, 8, K)
    rng = np.random.Generator(np.random.PCG64(12))
    rows = np.sort(rng.choice(N, 512, replace=False))
    from gpu_util import from_dev_bf16
    w_rows = from_dev_bf16(W[torch.from_numpy(rows).cuda()])
    Wr = oracle.dequant("q6k", oracle.quantize("q6k", w_rows), len(rows), K)
    for M, path in ((1, "auto"), (8, "auto"), (8, "gemv")):
        y = ql.qmatmul("q6k", blocks, to_dev_bf16(x[:M]), N, path=path).cpu().numpy()
        Yr, den = oracle.matmul_a16(Wr, x[:M])
        check_outputs(y[:, rows], Yr, den, f"lm_head M={M} {path}")


def test_graph_replays_match_eager():
    """Every path captured once in a HIP graph (the split-K paths include the
    fill kernel that zeroes Y) and replayed several times, with eager work
    that overwrites the outputs between replays: every replay must give the
    eager result (bit for bit where no atomics are involved, within 1e-6
    where K splits add partial tiles in a run-dependent order)."""
    cases = [("q4k", "gemv", 1, 4096, 4096, True),
             ("q6k", "gemv", 2, 300, 1024, True),
             ("q4k", "mfma_bf16", 16, 4100, 4352, False),   # batched stream, split K
             ("q4k", "mfma_bf16", 4, 4100, 4352, True),     # one-pass batched kernel (LDS reduction)
             ("q5k", "mfma_bf16", 16, 300, 1024, False),    # generic LDS-staged MFMA
             ("fp8", "mfma_bf16", 16, 300, 1024, False),    # FP8 W8A16 on exact codes
             ("q3k", "gemv", 3, 300, 1024, True),           # generic GEMV, X in LDS
             ("q8_0", "mfma_bf16", 128, 255, 4096, False),  # 128 x 256 tiles, split K
             ("q8_0", "mfma_bf16", 640, 255, 4096, False),  # prefill tiles, split K
             ("q8_0", "mfma_bf16", 1024, 1024, 512, True),  # prefill tiles, no split
             ("q8_0", "mfma_i8", 64, 300, 1024, False)]
    bufs = []
    for i, (fmt, path, M, N, K, exact) in enumerate(cases):
        w = synth.weights_bf16(5300 + i, N, K)
        x = to_dev_bf16(synth.activations_bf16(5310 + i, M, K))
        blocks = ql.isq(fmt, to_dev_bf16(w))
        ws = None
        if path == "mfma_i8":
            ws = torch.empty(ql.workspace_bytes(fmt, path, M, K), dtype=torch.uint8, device=x.device)
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
        ref = ql.qmatmul(fmt, blocks, x, N, path=path, workspace=ws).clone()
        bufs.append((fmt, path, blocks, x, N, y, ws, ref, exact))
    torch.cuda.synchronize()

    def launch_all():
        for fmt, path, blocks, x, N, y, ws, _, _ in bufs:
            ql.qmatmul(fmt, blocks, x, N, path=path, out=y, workspace=ws)

    launch_all()  # warm before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            launch_all()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        for _, _, _, _, _, y, _, _, _ in bufs:
            y.fill_(float("nan"))  # eager work between replays
        other = bufs[rep % len(bufs)]
        ql.qmatmul(other[0], other[2], other[3], other[4], path=other[1], workspace=other[6])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for fmt, path, _, _, N, y, _, ref, exact in bufs:
            label = f"replay {rep} {fmt} {path} M={y.shape[0]} N={N}"
            if exact:
                assert torch.equal(y, ref), label
            else:
                err = ((y - ref).abs().max() / ref.abs().max()).item()
                assert err < 1e-6, f"{label}: {err}"
