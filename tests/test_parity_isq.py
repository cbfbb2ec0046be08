"""GPU parity of in-situ quantization (ISQ) and of the exact dequantizer:
block bytes must equal the oracle's, bit for bit, on ragged shapes, edge
tensors, the hand-derived worked blocks and the full-size workloads."""
import json
import os

import numpy as np
import pytest
import torch

import ggml_block_quant_amd as ql
import oracle
import synth
from conftest import GOLDEN
from gpu_util import assert_blocks_equal, from_dev_bf16, to_dev_bf16

pytestmark = pytest.mark.gpu

FMTS = ("q8_0", "q4k", "q6k")


def isq_host(fmt, w):
    return ql.isq(fmt, to_dev_bf16(w)).cpu().numpy()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", [(1, 256), (7, 512), (33, 1024), (64, 4096), (3, 1280), (129, 2304)])
def test_isq_random_shapes(fmt, shape):
    w = synth.weights_bf16(100 + shape[0], *shape)
    assert_blocks_equal(fmt, isq_host(fmt, w), w)


def test_isq_q8_0_k_multiple_of_32():
    for shape in [(5, 96), (1, 32), (17, 224)]:
        w = synth.weights_bf16(7, *shape)
        assert_blocks_equal("q8_0", isq_host("q8_0", w), w)


def _bf16(v):
    return synth.bf16_bits_from_f32(np.asarray(v, np.float32))


def test_isq_golden_blocks_on_gpu():
    g8 = json.load(open(os.path.join(GOLDEN, "q8_0_blocks.json")))["blocks"]
    rows = np.zeros((len(g8), 256), np.uint16)
    for r, blk in enumerate(g8):
        if "x_bits_all" in blk:
            rows[r, :32] = int(blk["x_bits_all"], 16)
        rows[r, : len(blk["x"])] = _bf16(blk["x"]) if blk["x"] else rows[r, :0]
    got = isq_host("q8_0", rows)
    f = oracle.unpack("q8_0", got, len(g8), 256)
    for r, blk in enumerate(g8):
        assert int(f["d16"][r, 0]) == int(blk["d16"], 16), blk["name"]
        want = np.zeros(32, np.int8)
        want[: len(blk["q"])] = blk["q"]
        assert np.array_equal(f["q"][r, :32], want), blk["name"]
    assert_blocks_equal("q8_0", got, rows)

    g4 = json.load(open(os.path.join(GOLDEN, "q4k_worked_block.json")))
    x = np.array([(i - 8) * (j + 1) * 2.0 ** -10 for j in range(8) for i in range(32)], np.float32)
    f = oracle.unpack("q4k", isq_host("q4k", _bf16(x)[None, :]), 1, 256)
    assert int(f["d16"][0]) == int(g4["d16"], 16) and int(f["dmin16"][0]) == int(g4["dmin16"], 16)
    assert f["sc"][0].tolist() == g4["sc"] and f["mq"][0].tolist() == g4["m"]
    assert f["q"][0, :32].tolist() == g4["q_sub0"] and f["q"][0, 224:].tolist() == g4["q_sub7"]

    g6 = json.load(open(os.path.join(GOLDEN, "q6k_worked_block.json")))
    x = np.array([(i - 8) * (j + 1) * 2.0 ** -6 for j in range(16) for i in range(16)], np.float32)
    f = oracle.unpack("q6k", isq_host("q6k", _bf16(x)[None, :]), 1, 256)
    assert int(f["d16"][0]) == int(g6["d16"], 16) and f["sc"][0].tolist() == g6["sc"]
    assert f["q"][0, :16].tolist() == g6["q_sub0"] and f["q"][0, 240:].tolist() == g6["q_sub15"]


def _edge_tensor():
    """Rows exercising the degenerate cases: zeros, -0.0, constants, an
    all-negative row, ties, huge and tiny magnitudes, isolated outliers."""
    K = 512
    rng = np.random.Generator(np.random.PCG64(5))
    rows = []
    rows.append(np.zeros(K, np.float32))
    rows.append(np.full(K, 0.3, np.float32))
    rows.append(np.full(K, -0.3, np.float32))
    rows.append(-np.abs(rng.standard_normal(K)).astype(np.float32) * 0.02)
    rows.append(np.abs(rng.standard_normal(K)).astype(np.float32) * 0.02)
    rows.append((rng.integers(-254, 255, K) / 2.0 * 2.0 ** -8).astype(np.float32))   # ties
    rows.append((rng.standard_normal(K) * 1e30).astype(np.float32))                    # d clamps to 65504
    rows.append((rng.standard_normal(K) * 1e-6).astype(np.float32))                    # subnormal fp16 scales
    rows.append((rng.standard_normal(K) * 1e-30).astype(np.float32))                   # scales flush to 0
    r = (rng.standard_normal(K) * 0.02).astype(np.float32)
    r[::37] = 5.0
    rows.append(r)
    r = np.zeros(K, np.float32)
    r[100] = 1.0
    rows.append(r)
    r = (rng.standard_normal(K) * 0.02).astype(np.float32)
    r[:16] = 0.0
    r[256:288] = 0.0
    rows.append(r)
    w = _bf16(np.stack(rows))
    w[0, ::3] = 0x8000      # -0.0 mixed into the zero row
    return w


@pytest.mark.parametrize("fmt", FMTS)
def test_isq_edge_tensors(fmt):
    w = _edge_tensor()
    assert_blocks_equal(fmt, isq_host(fmt, w), w, "edge")


@pytest.mark.parametrize("fmt", FMTS)
def test_dequantize_matches_oracle(fmt):
    N, K = 48, 1024
    w = synth.weights_bf16(200, N, K, outliers=True)
    blocks = ql.isq(fmt, to_dev_bf16(w))
    got = ql.dequantize(fmt, blocks, N, K).cpu().numpy().astype(np.float64)
    ref = oracle.dequant(fmt, oracle.quantize(fmt, w), N, K)
    # Q8_0 and Q6K values are exact in fp32; Q4K is rounded once
    assert np.array_equal(got, ref.astype(np.float32).astype(np.float64))


# ---------------------------------------------------------------------------
# full-size workloads
# ---------------------------------------------------------------------------

def test_isq_gemv_workload_shapes_full():
    """1024x1024 to Q8_0; 14336x4096 to Q4K and Q8_0; 4096x14336 with 1 %
    outliers to Q4K: every byte."""
    cases = [("q8_0", synth.weights_bf16(synth.seed_for(1, 0), 1024, 1024)),
             ("q4k", synth.weights_bf16(synth.seed_for(2, 0), 14336, 4096)),
             ("q8_0", synth.weights_bf16(synth.seed_for(2, 0), 14336, 4096)),
             ("q4k", synth.weights_bf16(synth.seed_for(3, 0), 4096, 14336, outliers=True))]
    for fmt, w in cases:
        print(f"isq full {fmt} {w.shape}", flush=True)
        assert_blocks_equal(fmt, isq_host(fmt, w), w, "full")


DECODER = [("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
           ("gate", 14336, 4096), ("up", 14336, 4096), ("down", 4096, 14336)]


def _row_range_planes(fmt, buf, N, K, r0, r1):
    """The planar buffer of rows [r0, r1) of a [N][K] buffer, made of the
    contiguous slice of each plane (layout in oracle.c), zero-padded to the
    16-byte multiple that a buffer of that many rows has."""
    E = N * K
    if fmt == "q6k":
        G = E // 256
        planes = [(0, K * 192 // 256), (192 * G, K // 16), (208 * G, K // 128)]
    elif fmt == "q4k":
        G = E // 256
        planes = [(0, K // 2), (128 * G, K // 16)]
    else:
        raise ValueError(fmt)
    out = np.concatenate([buf[off + r0 * per:off + r1 * per] for off, per in planes])
    return np.concatenate([out, np.zeros(-out.size % 16, np.uint8)])  # buffer ends 16-aligned


def _every_byte(fmt, W, label, chunk):
    """Every byte of the GPU blocks of device tensor W against the oracle's
    packing of its own quantization, row ranges of `chunk` rows at a time."""
    N, K = W.shape
    blocks = ql.isq(fmt, W).cpu().numpy()
    nb = ql.blocks_bytes(fmt, N, K)
    assert blocks.size == nb
    if fmt == "q6k":
        tail = blocks[210 * N * K // 256:]
        assert not tail.any(), f"{label}: padding bytes not zero"
    for r0 in range(0, N, chunk):
        r1 = min(N, r0 + chunk)
        w = from_dev_bf16(W[r0:r1])
        got = _row_range_planes(fmt, blocks, N, K, r0, r1)
        assert_blocks_equal(fmt, got, w, f"{label} rows {r0}..{r1}")
        print(f"  {label}: rows {r0}..{r1} bit-exact", flush=True)


def test_isq_head_q6k_every_byte():
    """The 131072 x 5120 output head, promoted to Q6K: every byte of its 550 MB
    of blocks equals the oracle's (page "Quantization types", section
    "Sensitive tensor precision", promotes the head from Q4K to Q6K)."""
    fmt = ql.tensor_fmt(4, True)
    assert fmt == "q6k"
    W = synth.device_normal_bf16(synth.LM_HEAD_W_SEED, (131072, 5120), synth.W_SIGMA)
    _every_byte(fmt, W, "head", 16384)


@pytest.mark.parametrize("layer", range(32))
def test_isq_decoder_layer_every_byte(layer):
    """Every byte of the Q4K blocks (level 4) of each of the 32 decoder
    layers: q, k, v, o, gate, up and down, drawn on the GPU."""
    fmt = ql.tensor_fmt(4, False)
    for kind, (name, N, K) in enumerate(DECODER):
        W = synth.device_normal_bf16(synth.decoder_seed(layer, kind), (N, K), synth.W_SIGMA)
        _every_byte(fmt, W, f"layer {layer} {name}", 4096)
        del W
