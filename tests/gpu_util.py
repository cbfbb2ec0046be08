"""Helpers shared by the GPU parity tests (device transfer, comparisons)."""
import numpy as np
import torch

import oracle

TOL = 1e-3  # normalised error bar: |y - y*| / sum_k |w||x| per output


def to_dev_bf16(a: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns (host) -> bf16 device tensor (same bytes)."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def from_dev_bf16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_blocks_equal(fmt, got: np.ndarray, w: np.ndarray, label=""):
    """GPU block bytes must equal the oracle's packing of its own
    quantization of the same bf16 input; on a mismatch, report which logical
    field differs (via the oracle's own unpacker)."""
    N, K = w.shape
    f = oracle.quantize(fmt, w)
    ref = oracle.pack(fmt, f, N, K)
    if np.array_equal(got, ref):
        return
    g = oracle.unpack(fmt, got, N, K)
    msgs = []
    for k in f:
        bad = np.argwhere(f[k] != g[k])
        if bad.size:
            i = tuple(bad[0])
            msgs.append(f"{k}: {len(bad)} mismatches, first at {i}: oracle {f[k][i]} gpu {g[k][i]}")
    raise AssertionError(f"{label} {fmt} {N}x{K}: " + "; ".join(msgs or ["layout bytes differ"]))


def check_outputs(y_gpu: np.ndarray, y_ref: np.ndarray, den: np.ndarray, label=""):
    e = oracle.normalized_error(y_gpu, y_ref, den)
    worst = float(e.max()) if e.size else 0.0
    assert worst <= TOL, f"{label}: max normalised error {worst:.3e} > {TOL}"
    return worst


# The bf16 MFMA kernels give each weight w to the matrix cores as two bf16
# values, hi = bf16(w) and lo = bf16(w - hi); with one-hot activations an
# output is hi + lo, within 2^-17 |w| of the fp32 weight.
SPLIT_REL = 2.0 ** -17


def assert_split_exact(y: np.ndarray, w32: np.ndarray, label=""):
    """One-hot outputs of a bf16 MFMA kernel against the fp32 weights they
    select: |y - w| <= 2^-17 |w| element by element (w = 0 gives y = 0)."""
    y = np.asarray(y, np.float64)
    w = np.asarray(w32, np.float32).astype(np.float64)
    bad = np.abs(y - w) > SPLIT_REL * np.abs(w)
    assert not bad.any(), f"{label}: {int(bad.sum())} one-hot outputs off, first at {np.argwhere(bad)[0]}"
