"""GPU parity of the quantized embedding lookup (q_embed) against the oracle,
and the tied output head: one block buffer serves the lookup and qmatmul
(page "Quantization types", section "Sensitive tensor precision")."""
import numpy as np
import pytest
import torch

import ggml_block_quant_amd as ql
import oracle
import synth
from gpu_util import check_outputs, to_dev_bf16

pytestmark = pytest.mark.gpu

FMTS = ("q8_0", "q4k", "q6k")


def _ids(seed, n, N):
    """In-range ids with repeats, plus every out-of-range kind: -1, N,
    INT32_MIN and INT32_MAX (those rows must come back as zeros)."""
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, N, n).astype(np.int32)
    ids[:4] = [0, N - 1, N - 1, 0]
    ids[4:8] = [-1, N, np.iinfo(np.int32).min, np.iinfo(np.int32).max]
    return ids


@pytest.mark.parametrize("fmt", FMTS)
def test_embed_rows_bit_exact(fmt):
    for N, K, n in ((1000, 512, 300), (300, 5120, 64), (7, 256, 9)):
        w = synth.weights_bf16(8000 + K, N, K, outliers=True)
        blocks = ql.isq(fmt, to_dev_bf16(w))
        ids = _ids(8001 + N, n, N)
        got = ql.embed(fmt, blocks, N, K, torch.from_numpy(ids).cuda()).cpu().numpy()
        W = oracle.dequant(fmt, oracle.quantize(fmt, w), N, K)
        want = oracle.embed(W, ids).astype(np.float32)
        assert np.array_equal(got, want), f"embed {fmt} N={N} K={K}"


@pytest.mark.parametrize("fmt", FMTS)
def test_embed_large_table_and_empty(fmt):
    """A 131072-row table (the workload's vocabulary size) with ids near
    the end; an empty id list returns an empty result."""
    N, K = 131072, 512
    w = synth.weights_bf16(8100, N, K)
    blocks = ql.isq(fmt, to_dev_bf16(w))
    ids = _ids(8101, 2048, N)
    ids[8:16] = np.arange(N - 8, N)
    got = ql.embed(fmt, blocks, N, K, torch.from_numpy(ids).cuda()).cpu().numpy()
    rows = np.unique(ids[(ids >= 0) & (ids < N)])
    sub = oracle.dequant(fmt, oracle.quantize(fmt, w[rows]), rows.size, K)
    pos = {int(r): i for i, r in enumerate(rows)}
    want = np.zeros((ids.size, K), np.float32)
    for i, r in enumerate(ids):
        if 0 <= r < N:
            want[i] = sub[pos[int(r)]]
    assert np.array_equal(got, want)
    empty = ql.embed(fmt, blocks, N, K, torch.zeros(0, dtype=torch.int32, device="cuda"))
    assert empty.shape == (0, K)


@pytest.mark.parametrize("fmt", FMTS)
def test_tied_head_reuses_the_embedding(fmt):
    """The output head of a tied model is the embedding table itself: the
    same blocks give the looked-up rows and the logits X . E^T, with the
    logits within the matmul bar of the oracle's product with the rows the
    lookup returns."""
    N, K, M = 2000, 1024, 3
    w = synth.weights_bf16(8200, N, K)
    blocks = ql.isq(fmt, to_dev_bf16(w))
    table = ql.embed(fmt, blocks, N, K, torch.arange(N, dtype=torch.int32, device="cuda")).cpu().numpy()
    W = oracle.dequant(fmt, oracle.quantize(fmt, w), N, K)
    assert np.array_equal(table, W.astype(np.float32))
    x = synth.activations_bf16(8201, M, K)
    for path in ("auto", "mfma_bf16"):
        logits = ql.qmatmul(fmt, blocks, to_dev_bf16(x), N, path=path).cpu().numpy()
        Yr, den = oracle.matmul_a16(table.astype(np.float64), x)
        check_outputs(logits, Yr, den, f"tied head {fmt} {path}")
