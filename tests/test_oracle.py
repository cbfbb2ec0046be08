"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test names what it pins and why a plausible mistake in the oracle would
fail it: hand-derived worked blocks (tests/golden), exhaustive comparison
with an independent library routine (NumPy's IEEE float16 cast), exact
rational arithmetic (decimal / fractions), brute force over the code grid,
lossless special cases, and fp64 matmuls against BLAS and math.fsum.
"""
import decimal
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from conftest import GOLDEN


def _bf16(values):
    return synth.bf16_bits_from_f32(np.asarray(values, np.float32))


def _h(s):
    return int(s, 16)


# ---------------------------------------------------------------------------
# scalar conversions
# ---------------------------------------------------------------------------

def _f16_chunk(start, size):
    bits = np.arange(start, start + size, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    got = oracle.f16_from_f32_array(f)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = f.astype(np.float16).view(np.uint16)
    nan_in = np.isnan(f)
    ok = (got == ref) | (nan_in & ((got & 0x7C00) == 0x7C00) & ((got & 0x3FF) != 0))
    return None if ok.all() else hex(int(bits[~ok][0]))


def test_f16_from_f32_exhaustive():
    """All 2^32 binary32 patterns: oracle RNE conversion == NumPy's IEEE cast
    (NaNs: both NaN).  A wrong tie rule, a lost subnormal or a bad carry into
    the exponent fails here."""
    from concurrent.futures import ThreadPoolExecutor

    chunk = 1 << 24
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        bad = [r for r in ex.map(lambda s: _f16_chunk(s, chunk), range(0, 1 << 32, chunk)) if r]
    assert not bad, f"mismatch at {bad[:4]}"


def test_f32_from_f16_all_patterns():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.f32_from_f16_array(h)
    ref = h.view(np.float16).astype(np.float32)
    same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def _rha_decimal(v: float) -> float:
    with decimal.localcontext() as ctx:
        ctx.prec = 200
        d = decimal.Decimal(v)  # exact value of the binary32 (via double)
        r = d.quantize(decimal.Decimal(1), rounding=decimal.ROUND_HALF_UP)  # half away from zero
        return float(r)


def test_rha_against_decimal_half_up():
    rng = np.random.Generator(np.random.PCG64(7))
    ties = np.array([k + 0.5 for k in range(-300, 300)], np.float32)
    near = np.concatenate([np.nextafter(ties, np.float32(np.inf)), np.nextafter(ties, np.float32(-np.inf))])
    rnd = (rng.standard_normal(20000) * 200).astype(np.float32)
    vals = np.concatenate([ties, near, rnd, np.float32([0.0, -0.0, 0.49999997, -0.49999997, 1e30, -1e30])])
    got = oracle.rha_array(vals)
    for v, g in zip(vals.tolist(), got.tolist()):
        assert g == _rha_decimal(v) or (g == 0 and _rha_decimal(v) == 0), (v, g)
    # the ties the Q8_0 worked example relies on: half away, never half even
    assert oracle.rha(2.5) == 3 and oracle.rha(-2.5) == -3 and oracle.rha(0.5) == 1 and oracle.rha(126.5) == 127


# ---------------------------------------------------------------------------
# Q8_0
# ---------------------------------------------------------------------------

def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_q8_0_worked_blocks():
    """Hand-derived blocks (tests/golden/q8_0_blocks.json)."""
    for blk in _golden("q8_0_blocks.json")["blocks"]:
        row = np.zeros(32, np.uint16)
        if "x_bits_all" in blk:
            row[:] = _h(blk["x_bits_all"])
        xs = _bf16(blk["x"]) if blk["x"] else np.zeros(0, np.uint16)
        row[: len(xs)] = xs
        # the listed decimals must be exact in bf16
        assert np.array_equal(synth.bf16_bits_to_f32(xs), np.float32(blk["x"])), blk["name"]
        f = oracle.quantize("q8_0", row[None, :])
        assert int(f["d16"][0, 0]) == _h(blk["d16"]), blk["name"]
        want = np.zeros(32, np.int8)
        want[: len(blk["q"])] = blk["q"]
        assert np.array_equal(f["q"][0], want), (blk["name"], f["q"][0])


def test_embed_rows_are_the_worked_blocks():
    """Embedding lookup on a 3-row Q8_0 table built from the hand-derived
    blocks: each looked-up row is d16 * q of its block, listed in
    tests/golden/q8_0_blocks.json; ids outside the table give zero rows."""
    blks = {b["name"]: b for b in _golden("q8_0_blocks.json")["blocks"]}
    table = np.zeros((3, 32), np.uint16)
    for r, name in enumerate(("A_basic", "C_zero_block", "B_ties")):
        xs = _bf16(blks[name]["x"]) if blks[name]["x"] else np.zeros(0, np.uint16)
        table[r, : len(xs)] = xs
    W = oracle.dequant("q8_0", oracle.quantize("q8_0", table), 3, 32)
    E = oracle.embed(W, [2, 0, -1, 3, 0, 1])
    for i, name in ((0, "B_ties"), (1, "A_basic"), (4, "A_basic")):
        d = float(np.frombuffer(np.uint16(_h(blks[name]["d16"])).tobytes(), np.float16)[0])
        want = np.zeros(32)
        want[: len(blks[name]["q"])] = np.array(blks[name]["q"], np.float64) * d
        assert np.array_equal(E[i], want), name
    assert not E[2].any() and not E[3].any() and not E[5].any()


def _q8_blocks(seed, n_blocks, scale):
    w = synth.normal_bf16(seed, (n_blocks, 32), scale)
    return w, oracle.quantize("q8_0", w)


@pytest.mark.parametrize("scale", [0.02, 1.0, 3e-3, 50.0])
def test_q8_0_invariants(scale):
    """|q| <= 127; the largest |x| gets |q| = 127; |x - q d| <= d (1/2 + 2^-17)
    whenever d16 is a normal binary16; sign symmetry Q(-x) = (d, -q)."""
    w, f = _q8_blocks(11, 100_000, scale)
    x = synth.bf16_bits_to_f32(w).astype(np.float64)
    d16 = f["d16"][:, 0]
    df = oracle.f32_from_f16_array(d16).astype(np.float64)
    q = f["q"].astype(np.int64)
    assert np.abs(q).max() <= 127
    normal = (d16 & 0x7C00) != 0
    imax = np.argmax(np.abs(x), axis=1)
    assert (np.abs(q[np.arange(len(q)), imax])[normal] == 127).all()
    err = np.abs(x - q * df[:, None])
    bound = df[:, None] * (0.5 + 2.0 ** -17)
    assert (err[normal] <= bound[normal]).all()
    neg = oracle.quantize("q8_0", w ^ np.uint16(0x8000))
    nz = (w & 0x7FFF) != 0
    assert np.array_equal(neg["d16"], f["d16"])
    assert np.array_equal(neg["q"][nz], -f["q"][nz])


def test_q8_0_lossless_case():
    """x = qx * 2^-7 with a +-127 in every block is reproduced exactly:
    d = 2^-7, codes = qx, dequant = x."""
    rng = np.random.Generator(np.random.PCG64(3))
    qx = rng.integers(-127, 128, size=(64, 256))
    qx[:, ::32] = 127 * rng.choice([-1, 1], size=(64, 8))
    x = qx.astype(np.float32) * np.float32(2.0 ** -7)
    w = _bf16(x)
    f = oracle.quantize("q8_0", w)
    assert (f["d16"] == oracle.f16_from_f32(2.0 ** -7)).all()
    assert np.array_equal(f["q"].astype(np.int64), qx)
    assert np.array_equal(oracle.dequant("q8_0", f, 64, 256), x.astype(np.float64))


# ---------------------------------------------------------------------------
# Q4K
# ---------------------------------------------------------------------------

def _worked_q4k_input():
    x = np.array([(i - 8) * (j + 1) * 2.0 ** -10 for j in range(8) for i in range(32)], np.float32)
    w = _bf16(x)
    assert np.array_equal(synth.bf16_bits_to_f32(w), x)
    return w[None, :]


def test_q4k_worked_block():
    g = _golden("q4k_worked_block.json")
    f = oracle.quantize("q4k", _worked_q4k_input())
    assert int(f["d16"][0]) == _h(g["d16"])
    assert int(f["dmin16"][0]) == _h(g["dmin16"])
    assert f["sc"][0].tolist() == g["sc"]
    assert f["mq"][0].tolist() == g["m"]
    assert f["q"][0, :32].tolist() == g["q_sub0"]
    assert f["q"][0, 224:].tolist() == g["q_sub7"]
    # dequantized value of element (sub-block 0, i = 24): S q - M by hand
    S0 = oracle.f32_from_f16(0x0C33) * 8
    M0 = oracle.f32_from_f16(0x1410) * 8
    W = oracle.dequant("q4k", f, 1, 256)
    assert W[0, 24] == S0 * 11 - M0
    assert W[0, 0] == -M0


def _grid_check(x, S, M, q, qmin, qmax):
    """Brute force: q is a nearest point of the grid {S k - M : qmin <= k <=
    qmax} to x, up to the fp32 rounding slack of the quantizer (2^-18 S)."""
    ks = np.arange(qmin, qmax + 1, dtype=np.float64)
    grid = S[:, None] * ks[None, :] - M[:, None]
    dist = np.abs(grid - x[:, None])
    best = dist.min(axis=1)
    mine = np.abs(S * q - M - x)
    return mine <= best + S * 2.0 ** -18


@pytest.mark.parametrize("outliers", [False, True])
def test_q4k_invariants_and_nearest_grid(outliers):
    w = synth.weights_bf16(21, 64, 4096, outliers=outliers)
    f = oracle.quantize("q4k", w)
    assert f["q"].max() <= 15 and f["sc"].max() <= 63 and f["mq"].max() <= 63
    G = w.size // 256
    x = synth.bf16_bits_to_f32(w).astype(np.float64).reshape(G, 8, 32)
    d = oracle.f32_from_f16_array(f["d16"]).astype(np.float64)
    dm = oracle.f32_from_f16_array(f["dmin16"]).astype(np.float64)
    S = (d[:, None] * f["sc"]).reshape(G, 8, 1) * np.ones((1, 1, 32))
    M = (dm[:, None] * f["mq"]).reshape(G, 8, 1) * np.ones((1, 1, 32))
    q = f["q"].reshape(G, 8, 32).astype(np.float64)
    live = S > 0
    ok = _grid_check(x[live], S[live], M[live], q[live], 0, 15)
    assert ok.all()
    # scale quantization error: |d sc_j - s_j| <= d/2 (+slack), s_j from min/max
    lo = np.minimum(0, x.min(axis=2))
    hi = x.max(axis=2)
    s = (hi - lo) / 15
    m = -lo
    assert (np.abs(d[:, None] * f["sc"] - s) <= d[:, None] * (0.5 + 2.0 ** -16)).all()
    assert (np.abs(dm[:, None] * f["mq"] - m) <= dm[:, None] * (0.5 + 2.0 ** -16)).all()
    # the sub-block with the largest range gets the full 6-bit scale
    assert (f["sc"].max(axis=1)[(f["d16"] & 0x7C00) != 0] == 63).all()


def test_q4k_zero_and_constant_groups():
    w = np.zeros((2, 256), np.uint16)
    w[1, :] = _bf16([0.5])[0]  # constant positive group: lo = 0, hi = 0.5
    f = oracle.quantize("q4k", w)
    assert f["d16"][0] == 0 and f["dmin16"][0] == 0 and not f["q"][0].any()
    # constant 0.5: s = 0.5/15, m = 0 -> dmin = 0, codes RHA(0.5/S) = 15
    assert f["dmin16"][1] == 0 and (f["q"][1] == 15).all()


# ---------------------------------------------------------------------------
# Q6K
# ---------------------------------------------------------------------------

def test_q6k_worked_block():
    g = _golden("q6k_worked_block.json")
    x = np.array([(i - 8) * (j + 1) * 2.0 ** -6 for j in range(16) for i in range(16)], np.float32)
    w = _bf16(x)
    assert np.array_equal(synth.bf16_bits_to_f32(w), x)
    f = oracle.quantize("q6k", w[None, :])
    assert int(f["d16"][0]) == _h(g["d16"])
    assert f["sc"][0].tolist() == g["sc"]
    assert f["q"][0, :16].tolist() == g["q_sub0"]
    assert f["q"][0, 240:].tolist() == g["q_sub15"]
    W = oracle.dequant("q6k", f, 1, 256)
    d = oracle.f32_from_f16(0x1029)
    assert W[0, 4] == d * 8 * -15
    assert W[0, 240] == d * 127 * -31 and W[0, 244] == d * 127 * -16


@pytest.mark.parametrize("outliers", [False, True])
def test_q6k_invariants_and_nearest_grid(outliers):
    w = synth.weights_bf16(31, 64, 4096, outliers=outliers)
    f = oracle.quantize("q6k", w)
    assert f["q"].min() >= -32 and f["q"].max() <= 31
    assert f["sc"].min() >= 0 and f["sc"].max() <= 127
    G = w.size // 256
    x = synth.bf16_bits_to_f32(w).astype(np.float64).reshape(G, 16, 16)
    d = oracle.f32_from_f16_array(f["d16"]).astype(np.float64)
    S = (d[:, None] * f["sc"]).reshape(G, 16, 1) * np.ones((1, 1, 16))
    q = f["q"].reshape(G, 16, 16).astype(np.float64)
    live = S > 0
    assert _grid_check(x[live], S[live], np.zeros(live.sum()), q[live], -32, 31).all()
    s = np.abs(x).max(axis=2) / 31
    assert (np.abs(d[:, None] * f["sc"] - s) <= d[:, None] * (0.5 + 2.0 ** -16)).all()


@pytest.mark.parametrize("fmt,sub", [("q8_0", 32), ("q4k", 32), ("q6k", 16)])
def test_dequant_round_trip_bound(fmt, sub):
    """|x - deq(x)| <= (step of x's own sub-block)/2 (+ fp32 slack) for every
    element that lies within half a step of its sub-block's code range.  The step comes from
    the fields by the format's definition; a dequantizer that reads the wrong
    sub-block scale, drops the min or flips a sign fails by orders of
    magnitude."""
    rows, cols = 32, 2048
    w = synth.weights_bf16(91, rows, cols)
    f = oracle.quantize(fmt, w)
    W = oracle.dequant(fmt, f, rows, cols)
    x = synth.bf16_bits_to_f32(w).astype(np.float64)
    nsub = rows * cols // sub
    if fmt == "q8_0":
        step = oracle.f32_from_f16_array(f["d16"]).astype(np.float64).reshape(nsub)
        top = 127 * step
        bot = -top
    elif fmt == "q4k":
        d = oracle.f32_from_f16_array(f["d16"]).astype(np.float64)
        dm = oracle.f32_from_f16_array(f["dmin16"]).astype(np.float64)
        step = (d[:, None] * f["sc"]).reshape(nsub)
        bot = -(dm[:, None] * f["mq"]).reshape(nsub)
        top = bot + 15 * step
    else:
        d = oracle.f32_from_f16_array(f["d16"]).astype(np.float64)
        step = (d[:, None] * f["sc"]).reshape(nsub)
        bot, top = -32 * step, 31 * step
    xs = x.reshape(nsub, sub)
    half = step[:, None] / 2
    inside = (xs >= bot[:, None] - half) & (xs <= top[:, None] + half)
    err = np.abs(xs - W.reshape(nsub, sub))
    lim = step[:, None] * (0.5 + 2.0 ** -16) * np.ones_like(xs)
    assert inside.mean() > 0.99
    assert (err[inside] <= lim[inside]).all()


# ---------------------------------------------------------------------------
# planar layout
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", oracle.FORMATS)
def test_pack_unpack_roundtrip(fmt):
    rows, cols = 7, 1024
    w = synth.weights_bf16(41, rows, cols)
    f = oracle.quantize(fmt, w)
    buf = oracle.pack(fmt, f, rows, cols)
    assert buf.size == oracle.blocks_bytes(fmt, rows, cols)
    g = oracle.unpack(fmt, buf, rows, cols)
    for k in f:
        assert np.array_equal(f[k], g[k]), k
    # random field values (not only those the quantizer makes)
    rng = np.random.Generator(np.random.PCG64(5))
    r = {k: rng.integers(np.iinfo(v.dtype).min, np.iinfo(v.dtype).max + 1, size=v.shape, dtype=v.dtype)
         for k, v in f.items()}
    if fmt == "q4k":
        r["q"] &= 15
        r["sc"] &= 63
        r["mq"] &= 63
    if fmt == "q6k":
        r["q"] = rng.integers(-32, 32, size=f["q"].shape).astype(np.int8)
    g = oracle.unpack(fmt, oracle.pack(fmt, r, rows, cols), rows, cols)
    for k in r:
        assert np.array_equal(r[k], g[k]), k


def test_layout_bytes_by_hand():
    """A few bytes of each layout written out by hand from its description."""
    # Q4K: codes q[e] = e % 16 in sub-block 0.  Dword 0 holds elements 0..7:
    # nibbles p=0..3 = elements 0,2,4,6 and p=4..7 = elements 1,3,5,7.
    f = {"d16": np.array([0x3C00], np.uint16), "dmin16": np.array([0x3800], np.uint16),
         "sc": np.array([[1, 2, 3, 4, 5, 6, 7, 63]], np.uint8),
         "mq": np.array([[17, 0, 0, 0, 0, 0, 0, 48]], np.uint8),
         "q": (np.arange(256) % 16).astype(np.uint8)[None, :]}
    b = oracle.pack("q4k", f, 1, 256)
    dw0 = int.from_bytes(bytes(b[0:4]), "little")
    assert dw0 == (0 | 2 << 4 | 4 << 8 | 6 << 12 | 1 << 16 | 3 << 20 | 5 << 24 | 7 << 28)
    hdr = b[128:144]
    assert bytes(hdr[0:4]) == bytes([0x00, 0x3C, 0x00, 0x38])
    assert int.from_bytes(bytes(hdr[4:8]), "little") == 0xF7654321
    assert int.from_bytes(bytes(hdr[8:12]), "little") == 0x00000001
    # high bits: sc_7 = 63 -> 3 at bits 14..15; mq_0 = 17 -> 1 at bits 16..17;
    # mq_7 = 48 -> 3 at bits 30..31
    assert int.from_bytes(bytes(hdr[12:16]), "little") == (3 << 14) | (1 << 16) | (3 << 30)
    # Q6K: element 0 has u = 63 (q = 31), element 1 has u = 0 (q = -32),
    # element 17 (chunk 0, h=1, o=0, s=0, odd) has u = 0x30 (q = 16).
    q = np.zeros(256, np.int8)
    q[0], q[1], q[17] = 31, -32, 16
    fq = {"d16": np.array([0x3C00], np.uint16), "sc": np.arange(16, dtype=np.int8)[None, :], "q": q[None, :]}
    b = oracle.pack("q6k", fq, 1, 256)
    lo0 = int.from_bytes(bytes(b[0:4]), "little")
    assert lo0 & 0xF == 0xF and (lo0 >> 16) & 0xF == 0x0  # u0 low = 15, u1 low = 0
    hi_h0 = int.from_bytes(bytes(b[128:132]), "little")
    hi_h1 = int.from_bytes(bytes(b[132:136]), "little")
    assert hi_h0 & 3 == 3 and (hi_h0 >> 16) & 3 == 0
    assert (hi_h1 >> 16) & 3 == 3
    assert bytes(b[192:208]) == bytes(range(16)) and bytes(b[208:210]) == bytes([0x00, 0x3C])
    # one group: 210 bytes of planes, zero-padded to 224
    assert b.size == 224 and not b[210:].any()
    # Q8_0: codes then scales
    fq8 = {"d16": np.array([[0x1234]], np.uint16), "q": np.arange(-16, 16, dtype=np.int8)[None, :]}
    b = oracle.pack("q8_0", fq8, 1, 32)
    assert b[0] == 0xF0 and b[31] == 15 and bytes(b[32:34]) == bytes([0x34, 0x12])


# ---------------------------------------------------------------------------
# fp64 matmuls
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", oracle.FORMATS)
def test_matmul_a16_against_blas(fmt):
    M, N, K = 5, 96, 1024
    w = synth.weights_bf16(51, N, K)
    x = synth.activations_bf16(52, M, K)
    W = oracle.dequant(fmt, oracle.quantize(fmt, w), N, K)
    Y, den = oracle.matmul_a16(W, x)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    ref = xf @ W.T
    assert np.allclose(den, np.abs(xf) @ np.abs(W).T, rtol=1e-12)
    # a transposed operand or a dropped term would be far off
    assert np.max(np.abs(Y - ref) / den) < 1e-13


def test_matmul_a16_bruteforce_fsum():
    N, K = 4, 256
    w = synth.weights_bf16(61, N, K)
    x = synth.activations_bf16(62, 1, K)
    W = oracle.dequant("q4k", oracle.quantize("q4k", w), N, K)
    Y, den = oracle.matmul_a16(W, x)
    xf = synth.bf16_bits_to_f32(x)[0].astype(np.float64)
    for n in range(N):
        exact = math.fsum(W[n, k] * xf[k] for k in range(K))  # products exact in fp64
        assert abs(Y[0, n] - exact) <= K * 2.0 ** -53 * den[0, n]
    Yp, denp = oracle.matmul_a16_pairs(W, x, [0, 0], [3, 1])
    assert Yp[0] == Y[0, 3] and Yp[1] == Y[0, 1] and denp[0] == den[0, 3]


def test_matmul_a8_reduces_to_a16_when_activations_are_exact():
    """When every activation is q * 2^-7 with a +-127 in each block, the Q8_0
    activation quantization is lossless, so the A8 result equals the A16
    result on the same weights (up to fp64 summation order)."""
    M, N, K = 3, 40, 512
    rng = np.random.Generator(np.random.PCG64(8))
    qx = rng.integers(-127, 128, size=(M, K))
    qx[:, ::32] = 127
    x = _bf16(qx.astype(np.float32) * np.float32(2.0 ** -7))
    w = synth.weights_bf16(71, N, K)
    fw = oracle.quantize("q8_0", w)
    fx = oracle.quantize("q8_0", x)
    Y8, den8 = oracle.matmul_a8(fw, fx, M, N, K)
    W = oracle.dequant("q8_0", fw, N, K)
    Y16, den16 = oracle.matmul_a16(W, x)
    assert np.max(np.abs(Y8 - Y16) / den16) < 1e-14
    assert np.allclose(den8, den16, rtol=1e-14)
    # pairs form agrees with the full form
    Yp, _ = oracle.matmul_a8(fw, fx, M, N, K, mi=[2, 0], ni=[39, 5])
    assert Yp[0] == Y8[2, 39] and Yp[1] == Y8[0, 5]


def test_matmul_a8_close_to_a16_on_random_activations():
    """Activation quantization moves outputs by at most about 2^-8 of the
    normaliser (each x moves by <= d/2 <= max|x|/254)."""
    M, N, K = 4, 64, 1024
    w = synth.weights_bf16(81, N, K)
    x = synth.activations_bf16(82, M, K)
    fw = oracle.quantize("q8_0", w)
    Y8, _ = oracle.matmul_a8(fw, oracle.quantize("q8_0", x), M, N, K)
    Y16, den = oracle.matmul_a16(oracle.dequant("q8_0", fw, N, K), x)
    e = np.abs(Y8 - Y16) / den
    assert e.max() < 2.0 ** -8 and e.max() > 0


def test_normalized_error_zero_denominator():
    e = oracle.normalized_error([0.0, 1e-30, 2.0], [0.0, 0.0, 1.0], [0.0, 0.0, 4.0])
    assert e[0] == 0 and np.isinf(e[1]) and e[2] == 0.25


@pytest.mark.parametrize("act", ["silu", "relu", "sigmoid"])
def test_glu_activations_closed_forms(act):
    """The gated projection's activations against forms written with tanh
    (an independent library routine): sigmoid(x) = (1 + tanh(x/2)) / 2,
    SiLU(x) = x sigmoid(x); ReLU by cases; h = act(g) * u."""
    import math
    g = np.array([0.0, 1e-8, -1e-8, 0.5, -0.5, 1.0, -1.0, 3.0, -3.0, 20.0, -20.0, 40.0, -40.0, 700.0, -700.0])
    u = np.linspace(-2.0, 3.0, g.size)
    h, bound = oracle.glu_act(act, g, u)
    assert not bound.any()
    for gi, ui, hi in zip(g, u, h):
        sig = (1.0 + math.tanh(gi / 2.0)) / 2.0
        a = {"silu": gi * sig, "relu": max(gi, 0.0), "sigmoid": sig}[act]
        assert abs(hi - a * ui) <= 1e-15 * max(1.0, abs(a * ui)), (act, gi, ui, hi, a * ui)
    if act == "silu":
        hp, _ = oracle.glu_act(act, g, np.ones_like(g))
        hm, _ = oracle.glu_act(act, -g, np.ones_like(g))
        assert np.allclose(hp - hm, g, rtol=1e-15, atol=1e-300)   # SiLU(x) - SiLU(-x) = x
    if act == "sigmoid":
        assert oracle.glu_act(act, [0.0], [1.0])[0][0] == 0.5


@pytest.mark.parametrize("act", ["silu", "relu", "sigmoid"])
def test_glu_error_bound_holds(act):
    """The stated bound holds for perturbations of g and u up to eg and eu
    (random points, including kinks of ReLU at 0), and matches a hand value."""
    rng = np.random.default_rng(11)
    g = np.concatenate([rng.normal(0, 3, 2000), [0.0, 0.0, -1e-3]])
    u = rng.normal(0, 2, g.size)
    eg = np.abs(rng.normal(0, 0.05, g.size))
    eu = np.abs(rng.normal(0, 0.05, g.size))
    h, bound = oracle.glu_act(act, g, u, eg, eu)
    for sg in (-1, 1):
        for su in (-1, 1):
            h2, _ = oracle.glu_act(act, g + sg * eg * rng.random(g.size), u + su * eu * rng.random(g.size))
            assert np.all(np.abs(h2 - h) <= bound * (1 + 1e-12) + 1e-300), act
    if act == "relu":
        # g = 2, u = 3, eg = 0.1, eu = 0.2: 1 * 0.1 * (3 + 0.2) + 2 * 0.2 = 0.72
        assert abs(oracle.glu_act(act, [2.0], [3.0], [0.1], [0.2])[1][0] - 0.72) < 1e-15


# ----------------------------------------------------------------------------
# further formats (oracle.c, "Further formats")
# ----------------------------------------------------------------------------

KQ_PARAMS = {"q5k": (8, 32, 5, True, 6), "q3k": (16, 16, 3, False, 6), "q2k": (16, 16, 2, True, 4)}
LEG_PARAMS = {"q4_0": (4, False), "q5_0": (5, False), "q4_1": (4, True), "q5_1": (5, True)}


def _ramp(rule, n):
    if rule.startswith("x[32j+i]"):
        return [float((i - 8) * (j + 1) * 2.0 ** -10) for j in range(8) for i in range(32)]
    return [float((i - 8) * (j + 1) * 2.0 ** -6) for j in range(16) for i in range(16)]


def test_more_formats_worked_blocks():
    """Worked blocks of the seven further formats (tests/golden/more_formats_worked.json,
    derived with IEEE binary32/binary16 steps and exact half-away rounding,
    independently of oracle.c)."""
    for blk in _golden("more_formats_worked.json")["blocks"]:
        fmt = blk["name"]
        x = blk["x"] if "x" in blk else _ramp(blk["rule"], 256)
        w = _bf16(x)[None, :]
        assert np.array_equal(synth.bf16_bits_to_f32(w[0]), np.float32(x)), fmt
        f = oracle.quantize(fmt, w)
        assert int(f["d16"].ravel()[0]) == _h(blk["d16"]), (fmt, hex(int(f["d16"].ravel()[0])))
        assert np.array_equal(f["q"][0], np.array(blk["q"], np.int8)), (fmt, f["q"][0][:16])
        if fmt in KQ_PARAMS:
            ns = KQ_PARAMS[fmt][0]
            assert int(f["dmin16"][0]) == _h(blk["dmin16"]), fmt
            assert list(f["sc"][0][:ns]) == blk["sc"] and list(f["mq"][0][:ns]) == blk["mq"], fmt
        else:
            assert int(f["m16"].ravel()[0]) == _h(blk["m16"]), fmt


def _f16v(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


@pytest.mark.parametrize("fmt", list(KQ_PARAMS) + list(LEG_PARAMS))
@pytest.mark.parametrize("outliers", [False, True])
def test_more_formats_ranges_and_nearest_grid(fmt, outliers):
    """Codes lie in range; every unclamped code is the nearest grid point
    (|w - x| <= step/2, by brute force over all codes of the element's
    sub-block or block); the largest sub-scale is the top scale code."""
    rows, cols = 64, 512
    w = synth.weights_bf16(7700 + outliers, rows, cols, outliers=outliers)
    x = synth.bf16_bits_to_f32(w).astype(np.float64)
    f = oracle.quantize(fmt, w)
    W = oracle.dequant(fmt, f, rows, cols)
    q = f["q"].astype(np.int64)
    if fmt in KQ_PARAMS:
        ns, ln, bits, affine, sbits = KQ_PARAMS[fmt]
        lo, hi = (0, 2 ** bits - 1) if affine else (-(2 ** (bits - 1)), 2 ** (bits - 1) - 1)
        G = rows * cols // 256
        d = _f16v(f["d16"])[:, None]
        dm = _f16v(f["dmin16"])[:, None]
        S = (d * f["sc"][:, :ns]).repeat(ln, axis=1).reshape(rows, cols)
        M = (dm * f["mq"][:, :ns]).repeat(ln, axis=1).reshape(rows, cols) if affine else 0 * S
        assert f["sc"][:, :ns].max() <= 2 ** sbits - 1 and f["sc"].max(axis=1).min() == 2 ** sbits - 1
        assert not f["sc"][:, ns:].any() and (affine or not f["mq"].any())
    else:
        bits, affine = LEG_PARAMS[fmt]
        lo, hi = (0, 2 ** bits - 1) if affine else (-(2 ** (bits - 1)), 2 ** (bits - 1) - 1)
        S = _f16v(f["d16"]).repeat(32, axis=1)
        M = -_f16v(f["m16"]).repeat(32, axis=1) if affine else 0 * S
    assert q.min() >= lo and q.max() <= hi
    assert np.array_equal(W, S * q - M)
    grid = S[..., None] * np.arange(lo, hi + 1)[None, None, :] - M[..., None]
    best = np.abs(grid - x[..., None]).min(axis=-1)
    err = np.abs(W - x)
    # unclamped elements: the chosen code is a nearest grid point (ties aside, within fp32 slack)
    inside = (x + M > S * (lo - 0.5)) & (x + M < S * (hi + 0.5)) & (S > 0)
    assert np.all(err[inside] <= best[inside] + 1e-6 * S[inside])
    assert np.all(err[inside] <= S[inside] * (0.5 + 2 ** -17))


@pytest.mark.parametrize("fmt", list(KQ_PARAMS) + list(LEG_PARAMS))
def test_more_formats_pack_roundtrip_and_bytes(fmt):
    """Pack -> unpack is the identity on random fields over their full
    ranges; single codes and scales land on the bytes and bits the layout
    states (written out here by hand)."""
    rows, cols = 3, 512
    rng = np.random.default_rng(3)
    if fmt in KQ_PARAMS:
        ns, ln, bits, affine, sbits = KQ_PARAMS[fmt]
        G = rows * cols // 256
        lo, hi = (0, 2 ** bits - 1) if affine else (-(2 ** (bits - 1)), 2 ** (bits - 1) - 1)
        f = {"d16": rng.integers(0, 0x7c00, G).astype(np.uint16),
             "dmin16": rng.integers(0, 0x7c00, G).astype(np.uint16) if affine else np.zeros(G, np.uint16),
             "sc": np.zeros((G, 16), np.uint8), "mq": np.zeros((G, 16), np.uint8),
             "q": rng.integers(lo, hi + 1, (rows, cols)).astype(np.int8)}
        f["sc"][:, :ns] = rng.integers(0, 2 ** sbits, (G, ns))
        if affine:
            f["mq"][:, :ns] = rng.integers(0, 2 ** sbits, (G, ns))
    else:
        bits, affine = LEG_PARAMS[fmt]
        lo, hi = (0, 2 ** bits - 1) if affine else (-(2 ** (bits - 1)), 2 ** (bits - 1) - 1)
        f = {"d16": rng.integers(0, 0x7c00, (rows, cols // 32)).astype(np.uint16),
             "m16": rng.integers(0, 0xfc00, (rows, cols // 32)).astype(np.uint16) if affine
             else np.zeros((rows, cols // 32), np.uint16),
             "q": rng.integers(lo, hi + 1, (rows, cols)).astype(np.int8)}
    buf = oracle.pack(fmt, f, rows, cols)
    g = oracle.unpack(fmt, buf, rows, cols)
    for k in f:
        assert np.array_equal(f[k], g[k]), (fmt, k)

    # one element at the top code, everything else at the code whose stored value is 0
    n, G, B = rows * cols, rows * cols // 256, rows * cols // 32
    zero_code = {"q5k": 0, "q3k": -4, "q2k": 0, "q4_0": -8, "q5_0": -16, "q4_1": 0, "q5_1": 0}[fmt]
    e = 256 + 37   # group 1, element 37 (block 9, element 5)
    q = np.full((rows, cols), zero_code, np.int8)
    q.ravel()[e] = hi
    h = dict(f, q=q)
    for k in h:
        if k != "q":
            h[k] = np.zeros_like(h[k])
    b = oracle.pack(fmt, h, rows, cols)
    nz = {int(i): int(b[i]) for i in np.flatnonzero(b)}
    if fmt == "q5k":      # low nibble plane: byte 128*1 + 37/2, high nibble; high-bit plane at 128G: byte 32 + 4, bit 5
        assert nz == {128 + 18: 0xF0, 128 * G + 32 + 4: 1 << 5}
    elif fmt == "q3k":    # u = 7: low 2 bits at byte 64 + 9, bits 2..3; bit 2 at plane 64G, byte 32 + 4, bit 5
        assert nz == {64 + 9: 3 << 2, 64 * G + 32 + 4: 1 << 5}
    elif fmt == "q2k":    # code 3 at byte 64 + 9, bits 2..3
        assert nz == {64 + 9: 3 << 2}
    elif fmt in ("q4_0", "q4_1"):   # u = 15 at byte 16*9 + 2, high nibble
        assert nz == {16 * 9 + 2: 0xF0}
    else:                 # u = 31: low nibble 15 at byte 16*9 + 2 (high half), high bit at plane 16B, dword 9, bit 5
        assert nz == {16 * 9 + 2: 0xF0, 16 * B + 4 * 9 + 0: 1 << 5}
    # scales: a value in the second group / tenth block
    if fmt in KQ_PARAMS:
        s = dict(h, q=np.full((rows, cols), zero_code, np.int8))
        s["d16"] = np.zeros(G, np.uint16)
        s["d16"][1] = 0x1234
        s["sc"] = np.zeros((G, 16), np.uint8)
        s["sc"][1, 3] = 2 ** sbits - 1
        b = oracle.pack(fmt, s, rows, cols)
        nz = {int(i): int(b[i]) for i in np.flatnonzero(b)}
        if fmt == "q5k":   # header of group 1 at 160G + 16: d, sc low nibble 3 of dword 1, high pair 3 of dword 3
            h0 = 160 * G + 16
            assert nz == {h0: 0x34, h0 + 1: 0x12, h0 + 4 + 1: 0xF0, h0 + 12 + 0: 3 << 6}
        elif fmt == "q3k":  # scales of group 1 at 96G + 12: nibble 3 of dword 0, pair 3 of dword 2; d at up16(108G) + 2
            s0 = 96 * G + 12
            d0 = (108 * G + 15) // 16 * 16 + 2
            assert nz == {s0 + 1: 0xF0, s0 + 8: 3 << 6, d0: 0x34, d0 + 1: 0x12}
        else:              # Q2K: byte 64G + 16 + 3 = sc | mq << 4; d at 80G + 4
            assert nz == {64 * G + 16 + 3: 15, 80 * G + 4: 0x34, 80 * G + 5: 0x12}
    else:
        s = dict(h, q=np.full((rows, cols), zero_code, np.int8))
        s["d16"] = np.zeros((rows, cols // 32), np.uint16)
        s["d16"].ravel()[9] = 0x1234
        b = oracle.pack(fmt, s, rows, cols)
        nz = {int(i): int(b[i]) for i in np.flatnonzero(b)}
        dplane = 16 * B if fmt in ("q4_0", "q4_1") else 20 * B
        assert nz == {dplane + 18: 0x34, dplane + 19: 0x12}


# ----------------------------------------------------------------------------
# FP8 E4M3 with per-row scales (oracle.c, "FP8 E4M3 ...")
# ----------------------------------------------------------------------------

def _e4m3_closed_form(b):
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    if e == 15 and m == 7:
        return float("nan")
    v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


def test_e4m3_decode_every_code():
    """All 256 codes against the closed form (bias 7, 3 mantissa bits,
    subnormals m/8 * 2^-6, no infinities, NaN at 0x7F / 0xFF) and against
    torch's float8_e4m3fn (a library routine)."""
    import torch
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for b in range(256):
        v = oracle.e4m3_value(b)
        want = _e4m3_closed_form(b)
        assert (np.isnan(v) and np.isnan(want) and np.isnan(t[b])) or (v == want == t[b]), b
    assert oracle.e4m3_value(0x7E) == 448.0 and oracle.e4m3_value(0x01) == 2.0 ** -9


def test_e4m3_encode_ties_and_saturation():
    """Round to nearest even on every exact midpoint between neighbouring
    positive codes and on random values, against torch's cast (within
    +-448); saturation to +-448 by hand above it."""
    import torch
    pos = np.array([oracle.e4m3_value(b) for b in range(0x7F)])
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)   # the midpoints are exact in fp32
    rng = np.random.default_rng(5)
    rnd = (rng.standard_normal(400_000) * np.exp(rng.uniform(-14, 7, 400_000))).astype(np.float32)
    x = np.concatenate([mids, -mids, rnd[np.abs(rnd) <= 448], np.float32([0.0, 448.0, -448.0, 2 ** -10, 2 ** -11])])
    got = oracle.e4m3_from_f32_array(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)
    # ties go to the even code: 1 + 1/16 lies between 1 (0x38) and 1.125 (0x39) -> 0x38
    assert oracle.e4m3_from_f32_array([1.0625, 1.1875])[0] == 0x38
    assert oracle.e4m3_from_f32_array([1.1875])[0] == 0x3A          # between 1.125 and 1.25 -> 1.25 (even)
    sat = oracle.e4m3_from_f32_array([448.5, 464.0, 1e6, -500.0, 3e38])
    assert sat.tolist() == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E]


def test_fp8_quantizer_worked_rows():
    """Row with max 448: s = 1 and the codes are the values' own E4M3
    patterns; row of zeros: s = 0, codes 0; row with max 2: s = 2/448 and
    the max element maps to the top code 0x7E."""
    x = np.zeros((3, 256), np.float32)
    x[0, :6] = [448.0, -224.0, 1.0, 0.5, 2.0 ** -9, -0.09375]
    x[2, :3] = [2.0, -1.0, 0.25]
    f = oracle.quantize_fp8(synth.bf16_bits_from_f32(x))
    assert f["s"].tolist() == [1.0, 0.0, np.float32(2.0) / np.float32(448.0)]
    # 448 = 1.75 2^8: 0x7E; -224 = -1.75 2^7: 0xF6; 1: 0x38; 0.5: 0x30; 2^-9: subnormal 0x01;
    # -0.09375 = -1.5 2^-4: exponent field 3, mantissa 4: 0x9C
    assert f["q"][0, :6].tolist() == [0x7E, 0xF6, 0x38, 0x30, 0x01, 0x9C]
    assert not f["q"][1].any()
    assert f["q"][2, 0] == 0x7E
    W = oracle.dequant_fp8(f)
    assert W[0, 1] == -224.0 and W[2, 0] == 448.0 * float(f["s"][2])


def test_fp8_round_trip_bound_and_matmul_bruteforce():
    """|s e4m3(q) - x| <= s * half a code step (2^-4 relative for normals,
    s 2^-10 absolute below); the W8A8 product equals a brute-force fp64 sum
    over the decoded values."""
    w = synth.weights_bf16(8800, 40, 512, outliers=True)
    x = synth.bf16_bits_to_f32(w).astype(np.float64)
    f = oracle.quantize_fp8(w)
    W = oracle.dequant_fp8(f)
    s = f["s"].astype(np.float64)[:, None]
    a = np.abs(x / s)
    bound = np.where(a >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 4), 2.0 ** -10) * s
    assert np.all(np.abs(W - x) <= bound * (1 + 1e-6))
    xa = synth.activations_bf16(8801, 3, 512)
    fx = oracle.quantize_fp8(xa)
    Y, den = oracle.matmul_fp8(fx, f)
    vals = np.array([oracle.e4m3_value(b) for b in range(256)])
    dx, dw = vals[fx["q"]], vals[f["q"]]
    want = (fx["s"].astype(np.float64)[:, None] * f["s"].astype(np.float64)[None, :]) * (dx @ dw.T)
    assert np.allclose(Y, want, rtol=1e-12, atol=0)
    assert np.all(den >= np.abs(Y))
