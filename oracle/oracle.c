/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the
 * block-quantized linear layer (Q8_0, Q4K, Q6K).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library; the two meet only in the byte layout, which each side
 * implements on its own.
 *
 * Source of the method:
 *   - page "Quantization types" (mistral.rs reference), sections
 *     "Q*K family" (q4k = 4 bits, q6k = 6 bits, GGML K-quant formats) and
 *     "Legacy GGML types" (q8_0 = 8 bits).  The page names the formats and
 *     their bit widths; it prints no block layout and no quantizer.
 *   - the block definitions this library implements: Q8_0 = blocks of 32
 *     elements, fp16 scale d = max|x|/127, int8 codes q = round(x/d) with
 *     round-half-away-from-zero; Q4K = 256-element super-blocks of 8
 *     sub-blocks of 32 with 6-bit scales and mins and fp16 d/dmin, 4-bit
 *     codes; Q6K = 256-element super-blocks with 6-bit codes.
 *   Every point those leave open is settled by a stated reading, listed in
 *   the design notes and repeated at the function that applies it.
 *
 * Arithmetic rules (identical on both sides of the parity check):
 *   - quantizer arithmetic is IEEE binary32, round-to-nearest-even, one
 *     operation at a time: no contraction, no reciprocal-multiply, no
 *     denormal flushing (build with -O2 -fno-fast-math -ffp-contract=off);
 *   - fp32 -> fp16 conversion is written out from IEEE 754 below;
 *   - RHA(v) = round half away from zero = C roundf;
 *   - a -0.0 input element is read as +0.0, so no sign of zero can reach a
 *     scale's bit pattern (it never changes a code);
 *   - dequantized values and matmuls are exact / fp64.
 *
 * Parity status of each function is stated in its comment.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Scalar conversions                                                  */
/* ------------------------------------------------------------------ */

/* bf16 bit pattern -> binary32 (exact: bf16 is the top half of binary32).
 * -0.0 is returned as +0.0 (the reading above). */
static float bf16_in(uint16_t h)
{
    uint32_t u = (h == 0x8000u) ? 0u : ((uint32_t)h << 16);
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 -> binary16 bits, round to nearest, ties to even, gradual
 * underflow, overflow to infinity (IEEE 754-2008, section 4.3.1 / 7.4).
 * Pinned exhaustively against NumPy's float16 cast. */
uint16_t oracle_f16_from_f32(float v)
{
    uint32_t x;
    memcpy(&x, &v, sizeof x);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t bexp = (x >> 23) & 0xffu;
    uint32_t frac = x & 0x7fffffu;

    if (bexp == 0xffu) /* inf or NaN */
        return (uint16_t)(sign | 0x7c00u | (frac ? (0x200u | (frac >> 13)) : 0u));
    if (bexp == 0u) /* zero or binary32 subnormal: |v| < 2^-126, rounds to 0 */
        return (uint16_t)sign;

    int e = (int)bexp - 127; /* v = 1.frac * 2^e */
    if (e > 15)
        return (uint16_t)(sign | 0x7c00u);
    if (e >= -14) {
        /* normal binary16: keep 10 of the 23 fraction bits */
        uint32_t keep = frac >> 13;
        uint32_t rest = frac & 0x1fffu;
        uint32_t h = ((uint32_t)(e + 15) << 10) | keep;
        if (rest > 0x1000u || (rest == 0x1000u && (keep & 1u)))
            h += 1u; /* a carry may step the exponent, up to 0x7c00 = inf */
        return (uint16_t)(sign | h);
    }
    /* subnormal binary16: units of 2^-24.  The 24-bit significand sig
     * (with its leading 1) is worth sig * 2^(e-23) = sig * 2^(e+1) units,
     * so drop -(e+1) >= 14 low bits. */
    int drop = -(e + 1);
    if (drop > 24)
        return (uint16_t)sign; /* below half the smallest subnormal */
    uint32_t sig = frac | 0x800000u;
    uint32_t keep = sig >> drop;
    uint32_t rest = sig & ((1u << drop) - 1u);
    uint32_t half = 1u << (drop - 1);
    if (rest > half || (rest == half && (keep & 1u)))
        keep += 1u; /* may become 0x400 = smallest normal, which is right */
    return (uint16_t)(sign | keep);
}

/* binary16 bits -> binary32 (exact). */
float oracle_f32_from_f16(uint16_t h)
{
    uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    uint32_t bexp = ((uint32_t)h >> 10) & 0x1fu;
    uint32_t frac = (uint32_t)h & 0x3ffu;
    uint32_t u;
    float f;
    if (bexp == 0u) {
        f = (float)frac * 0x1p-24f; /* exact: frac < 2^10 */
        return sign ? -f : f;
    }
    if (bexp == 0x1fu)
        u = sign | 0x7f800000u | (frac << 13);
    else
        u = sign | ((bexp - 15u + 127u) << 23) | (frac << 13);
    memcpy(&f, &u, sizeof f);
    return f;
}

/* The scale conversion F16(v) for v >= 0: clamp to the largest finite
 * binary16 (65504) first, then round to nearest even.  The clamp replaces
 * overflow to infinity [reading: the pages give no overflow rule]. */
static uint16_t scale_f16(float v)
{
    if (v > 65504.0f)
        v = 65504.0f;
    return oracle_f16_from_f32(v);
}

/* Round half away from zero.  Pinned against decimal ROUND_HALF_UP. */
float oracle_rha(float v) { return roundf(v); }

/* Array forms of the two scalar helpers, for the bulk pins. */
void oracle_f16_from_f32_array(const float *in, int64_t n, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_f16_from_f32(in[i]);
}

void oracle_f32_from_f16_array(const uint16_t *in, int64_t n, float *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_f32_from_f16(in[i]);
}

void oracle_rha_array(const float *in, int64_t n, float *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = roundf(in[i]);
}

static int clamp_code(float r, int lo, int hi)
{
    if (r < (float)lo)
        return lo;
    if (r > (float)hi)
        return hi;
    return (int)r;
}

/* ------------------------------------------------------------------ */
/* Q8_0: blocks of 32, fp16 d = max|x|/127, q = RHA(x / d)             */
/* ------------------------------------------------------------------ */

/* One block.  Steps:
 *   a   = max |x_i|                     (exact)
 *   d16 = F16(a / 127)                  (fp32 division, then F16)
 *   q_i = clamp(RHA(x_i / F32(d16)), -127, 127), or 0 when d16 == 0.
 * Readings: the code divides by the stored fp16 scale (so that the
 * round-trip bound |x - q d| <= d/2 holds), codes are symmetric in
 * [-127, 127], and an all-zero block stores d = 0 and zero codes. */
static void q8_0_block(const uint16_t *x16, uint16_t *d16_out, int8_t *q)
{
    float x[32];
    float a = 0.0f;
    for (int i = 0; i < 32; i++) {
        x[i] = bf16_in(x16[i]);
        float ax = fabsf(x[i]);
        if (ax > a)
            a = ax;
    }
    float d32 = a / 127.0f;
    uint16_t d16 = scale_f16(d32);
    float df = oracle_f32_from_f16(d16);
    for (int i = 0; i < 32; i++)
        q[i] = (int8_t)(df == 0.0f ? 0 : clamp_code(roundf(x[i] / df), -127, 127));
    *d16_out = d16;
}

/* Quantize rows*cols bf16 values (row-major, cols % 32 == 0) to Q8_0
 * logical fields: d16[rows][cols/32], q[rows][cols]. */
void oracle_quantize_q8_0(const uint16_t *w, int64_t rows, int64_t cols,
                          uint16_t *d16, int8_t *q)
{
    int64_t nb = rows * (cols / 32);
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; b++)
        q8_0_block(w + 32 * b, d16 + b, q + 32 * b);
}

/* ------------------------------------------------------------------ */
/* Q4K: groups of 256 = 8 sub-blocks of 32; 6-bit sc/m; fp16 d, dmin   */
/* ------------------------------------------------------------------ */

/* One group, plain min/max affine rule [reading: the pages name the fields
 * only].  Steps:
 *   per sub-block j: lo_j = min(0, min x), hi_j = max x,
 *                    s_j = (hi_j - lo_j) / 15,  m_j = 0 - lo_j
 *   d16 = F16(max_j s_j / 63),  dmin16 = F16(max_j m_j / 63)
 *   sc_j = clamp(RHA(s_j / d), 0, 63)   (0 when d == 0)
 *   mq_j = clamp(RHA(m_j / dmin), 0, 63) (0 when dmin == 0)
 *   S_j = d * sc_j,  M_j = dmin * mq_j   (both exact in binary32)
 *   q_i = clamp(RHA((x_i + M_j) / S_j), 0, 15)  (0 when S_j == 0)
 * so that the decoded value is S_j * q_i - M_j. */
static void q4k_group(const uint16_t *x16, uint16_t *d16_out, uint16_t *dmin16_out,
                      uint8_t *sc, uint8_t *mq, uint8_t *q)
{
    float x[256], s[8], m[8];
    for (int i = 0; i < 256; i++)
        x[i] = bf16_in(x16[i]);
    for (int j = 0; j < 8; j++) {
        float lo = 0.0f, hi = x[32 * j];
        for (int i = 0; i < 32; i++) {
            float v = x[32 * j + i];
            if (v < lo)
                lo = v;
            if (v > hi)
                hi = v;
        }
        s[j] = (hi - lo) / 15.0f;
        m[j] = 0.0f - lo;
    }
    float smax = 0.0f, mmax = 0.0f;
    for (int j = 0; j < 8; j++) {
        if (s[j] > smax)
            smax = s[j];
        if (m[j] > mmax)
            mmax = m[j];
    }
    uint16_t d16 = scale_f16(smax / 63.0f);
    uint16_t dm16 = scale_f16(mmax / 63.0f);
    float df = oracle_f32_from_f16(d16);
    float dmf = oracle_f32_from_f16(dm16);
    for (int j = 0; j < 8; j++) {
        sc[j] = (uint8_t)(df > 0.0f ? clamp_code(roundf(s[j] / df), 0, 63) : 0);
        mq[j] = (uint8_t)(dmf > 0.0f ? clamp_code(roundf(m[j] / dmf), 0, 63) : 0);
        float S = df * (float)sc[j];
        float M = dmf * (float)mq[j];
        for (int i = 0; i < 32; i++) {
            float t = x[32 * j + i] + M;
            q[32 * j + i] = (uint8_t)(S > 0.0f ? clamp_code(roundf(t / S), 0, 15) : 0);
        }
    }
    *d16_out = d16;
    *dmin16_out = dm16;
}

/* rows*cols bf16 (cols % 256 == 0) -> Q4K logical fields per group g:
 * d16[g], dmin16[g], sc[g][8], mq[g][8], q[g][256] (q is [rows][cols]). */
void oracle_quantize_q4k(const uint16_t *w, int64_t rows, int64_t cols,
                         uint16_t *d16, uint16_t *dmin16, uint8_t *sc,
                         uint8_t *mq, uint8_t *q)
{
    int64_t ng = rows * (cols / 256);
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < ng; g++)
        q4k_group(w + 256 * g, d16 + g, dmin16 + g, sc + 8 * g, mq + 8 * g, q + 256 * g);
}

/* ------------------------------------------------------------------ */
/* Q6K: groups of 256 = 16 sub-blocks of 16; int8 sc; one fp16 d       */
/* ------------------------------------------------------------------ */

/* One group, symmetric rule [reading: 6-bit symmetric codes, 16 sub-blocks
 * of 16 with 8-bit sub-scales and one fp16 d, no mins -- the field set
 * that gives 210 bytes per 256 elements].  Steps:
 *   s_j = max_i |x_i| / 31 over sub-block j
 *   d16 = F16(max_j s_j / 127)
 *   sc_j = clamp(RHA(s_j / d), 0, 127)  (0 when d == 0)
 *   S_j = d * sc_j                       (exact in binary32)
 *   q_i = clamp(RHA(x_i / S_j), -32, 31) (0 when S_j == 0)
 * decoded value S_j * q_i. */
static void q6k_group(const uint16_t *x16, uint16_t *d16_out, int8_t *sc, int8_t *q)
{
    float x[256], s[16];
    for (int i = 0; i < 256; i++)
        x[i] = bf16_in(x16[i]);
    float smax = 0.0f;
    for (int j = 0; j < 16; j++) {
        float a = 0.0f;
        for (int i = 0; i < 16; i++) {
            float ax = fabsf(x[16 * j + i]);
            if (ax > a)
                a = ax;
        }
        s[j] = a / 31.0f;
        if (s[j] > smax)
            smax = s[j];
    }
    uint16_t d16 = scale_f16(smax / 127.0f);
    float df = oracle_f32_from_f16(d16);
    for (int j = 0; j < 16; j++) {
        sc[j] = (int8_t)(df > 0.0f ? clamp_code(roundf(s[j] / df), 0, 127) : 0);
        float S = df * (float)sc[j];
        for (int i = 0; i < 16; i++)
            q[16 * j + i] = (int8_t)(S > 0.0f ? clamp_code(roundf(x[16 * j + i] / S), -32, 31) : 0);
    }
    *d16_out = d16;
}

/* rows*cols bf16 (cols % 256 == 0) -> Q6K fields per group g:
 * d16[g], sc[g][16] (int8, never negative), q[g][256] signed in [-32, 31]. */
void oracle_quantize_q6k(const uint16_t *w, int64_t rows, int64_t cols,
                         uint16_t *d16, int8_t *sc, int8_t *q)
{
    int64_t ng = rows * (cols / 256);
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < ng; g++)
        q6k_group(w + 256 * g, d16 + g, sc + 16 * g, q + 256 * g);
}

/* ------------------------------------------------------------------ */
/* Exact dequantization to fp64                                        */
/* ------------------------------------------------------------------ */

/* Q8_0: w = d * q (exact). */
void oracle_dequant_q8_0(const uint16_t *d16, const int8_t *q, int64_t n_elems, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < n_elems; e++)
        out[e] = (double)oracle_f32_from_f16(d16[e / 32]) * (double)q[e];
}

/* Q4K: w = (d * sc_j) * q - (dmin * mq_j), evaluated exactly in fp64. */
void oracle_dequant_q4k(const uint16_t *d16, const uint16_t *dmin16, const uint8_t *sc,
                        const uint8_t *mq, const uint8_t *q, int64_t n_elems, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < n_elems; e++) {
        int64_t g = e / 256;
        int j = (int)((e % 256) / 32);
        double S = (double)oracle_f32_from_f16(d16[g]) * (double)sc[8 * g + j];
        double M = (double)oracle_f32_from_f16(dmin16[g]) * (double)mq[8 * g + j];
        out[e] = S * (double)q[e] - M;
    }
}

/* Q6K: w = (d * sc_j) * q (exact). */
void oracle_dequant_q6k(const uint16_t *d16, const int8_t *sc, const int8_t *q,
                        int64_t n_elems, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < n_elems; e++) {
        int64_t g = e / 256;
        int j = (int)((e % 256) / 16);
        out[e] = (double)oracle_f32_from_f16(d16[g]) * (double)sc[16 * g + j] * (double)q[e];
    }
}

/* ------------------------------------------------------------------ */
/* fp64 matmuls and the error normaliser                               */
/* ------------------------------------------------------------------ */

/* A16 oracle: Y[m][n] = sum_k W[n][k] * x[m][k] in fp64, sequential k,
 * and den[m][n] = sum_k |W[n][k]| * |x[m][k]|.  x is bf16 bits [M][K];
 * W is the exact dequantized weight [N][K] in fp64. */
void oracle_matmul_a16(const double *W, const uint16_t *x16, int64_t M, int64_t N,
                       int64_t K, double *Y, double *den)
{
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            double acc = 0.0, a = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double x = (double)bf16_in(x16[m * K + k]);
                double w = W[n * K + k];
                acc += w * x;
                a += fabs(w) * fabs(x);
            }
            Y[m * N + n] = acc;
            den[m * N + n] = a;
        }
}

/* The same sum for a list of (m, n) pairs only, for shapes too large to
 * evaluate in full.  Wrow(n) is taken from W given as dequantized rows:
 * W is [n_rows][K] and rowsel[i] is the row of W that output i uses. */
void oracle_matmul_a16_pairs(const double *W, const uint16_t *x16, int64_t K,
                             const int64_t *mi, const int64_t *wrow, int64_t npairs,
                             double *Y, double *den)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < npairs; i++) {
        double acc = 0.0, a = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double x = (double)bf16_in(x16[mi[i] * K + k]);
            double w = W[wrow[i] * K + k];
            acc += w * x;
            a += fabs(w) * fabs(x);
        }
        Y[i] = acc;
        den[i] = a;
    }
}

/* Gated feed-forward projection (page "Quantization types", section
 * "NVFP4": gated feed-forward projections with SiLU, ReLU or sigmoid):
 * h = act(g) * u in fp64 on the fp64 projections g and u, with
 * act 0: SiLU g / (1 + exp(-g)); 1: ReLU max(g, 0); 2: sigmoid 1 / (1 + exp(-g)).
 * Also a bound on |h' - h| when g' and u' are within eg and eu of g and u:
 * |act(g') u' - act(g) u| <= |act(g') - act(g)| |u'| + |act(g)| |u' - u|
 *                         <= L eg (|u| + eu) + |act(g)| eu,
 * with L = 1.1, 1 and 1/4 bounding |act'| (SiLU's derivative lies in
 * (-0.1, 1.1)). */
static double act64(int act, double g)
{
    if (act == 1)
        return g > 0.0 ? g : 0.0;
    double e = 1.0 + exp(-g);
    return act == 0 ? g / e : 1.0 / e;
}

void oracle_glu(const double *g, const double *u, const double *eg, const double *eu, int64_t n, int64_t act,
                double *h, double *bound)
{
    const double L = act == 0 ? 1.1 : (act == 1 ? 1.0 : 0.25);
    for (int64_t i = 0; i < n; i++) {
        double a = act64((int)act, g[i]);
        h[i] = a * u[i];
        bound[i] = L * eg[i] * (fabs(u[i]) + eu[i]) + fabs(a) * eu[i];
    }
}

/* A8 oracle (activations quantized to Q8_0 as well):
 *   Y[m][n] = sum_b dw[n][b] * dx[m][b] * (sum_{i in b} qw * qx)
 * with the integer block sums exact in int64 and the rest in fp64.
 * den[m][n] = sum_k |dw qw| * |dx qx| (the normaliser on the same values). */
void oracle_matmul_a8(const uint16_t *dw16, const int8_t *qw, const uint16_t *dx16,
                      const int8_t *qx, int64_t M, int64_t N, int64_t K,
                      const int64_t *mi, const int64_t *ni, int64_t npairs,
                      double *Y, double *den)
{
    int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < npairs; i++) {
        int64_t m = mi[i], n = ni[i];
        double acc = 0.0, a = 0.0;
        for (int64_t b = 0; b < nb; b++) {
            int64_t isum = 0, iabs = 0;
            for (int64_t t = 0; t < 32; t++) {
                int64_t pw = qw[n * K + 32 * b + t], px = qx[m * K + 32 * b + t];
                isum += pw * px;
                iabs += (pw < 0 ? -pw : pw) * (px < 0 ? -px : px);
            }
            double dw = (double)oracle_f32_from_f16(dw16[n * nb + b]);
            double dx = (double)oracle_f32_from_f16(dx16[m * nb + b]);
            acc += dw * dx * (double)isum;
            a += fabs(dw) * fabs(dx) * (double)iabs;
        }
        Y[i] = acc;
        den[i] = a;
    }
    (void)M;
    (void)N;
}

/* ------------------------------------------------------------------ */
/* Planar byte layout: logical fields <-> bytes                        */
/* ------------------------------------------------------------------ */
/*
 * One buffer per tensor [rows][cols], cols % 256 == 0 (Q8_0: cols % 32),
 * made of planes that each start 16-byte aligned.  G = rows*cols/256.
 *
 * Q8_0  [C: rows*cols int8, row-major]            code of element (n,k)
 *       [S: rows*cols/32 fp16, row-major]          d of block (n, k/32)
 * Q4K   [C: G*128 bytes] [S: G*16 bytes]
 *       C: group g owns bytes 128g..128g+127; sub-block j owns the 16
 *          bytes 16j..16j+15 of its group, read as 4 little-endian dwords;
 *          dword w holds elements e = 8w..8w+7 of the sub-block: nibble p
 *          (bits 4p..4p+3) holds e = 8w + 2p for p < 4 and
 *          e = 8w + 2(p-4) + 1 for p >= 4 (even elements in the low half,
 *          odd elements in the high half).
 *       S: bytes 0-1 d (fp16), 2-3 dmin (fp16), bytes 4-7 a dword whose
 *          nibble j is sc_j & 15, bytes 8-11 a dword whose nibble j is
 *          mq_j & 15, bytes 12-15 a dword with bits 2j..2j+1 = sc_j >> 4
 *          and bits 16+2j..17+2j = mq_j >> 4.
 * Q6K   [C: G*192 bytes] [S: G*16 bytes] [D: G*2 bytes]
 *       stored code u = q + 32 in [0, 63].
 *       C: group g owns bytes 192g..192g+191 (layout at q6k_pack_group).
 *       S: 16 int8 sub-scales sc_j per group.  D: fp16 d per group (the
 *          plane starts at byte 208*G, a multiple of 16).  The buffer is
 *          zero-padded to a multiple of 16 bytes (the caller allocates it;
 *          these routines touch only the 210*G bytes of the planes).
 */

/* Q8_0 pack/unpack: the planes are the fields themselves. */
void oracle_pack_q8_0(const uint16_t *d16, const int8_t *q, int64_t rows, int64_t cols,
                      uint8_t *buf)
{
    int64_t n = rows * cols;
    memcpy(buf, q, (size_t)n);
    memcpy(buf + n, d16, (size_t)(n / 32) * 2);
}

void oracle_unpack_q8_0(const uint8_t *buf, int64_t rows, int64_t cols, uint16_t *d16,
                        int8_t *q)
{
    int64_t n = rows * cols;
    memcpy(q, buf, (size_t)n);
    memcpy(d16, buf + n, (size_t)(n / 32) * 2);
}

/* nibble position p (0..7) within a dword -> element offset 0..7 */
static int nib_elem(int p) { return p < 4 ? 2 * p : 2 * (p - 4) + 1; }

static void put_u32(uint8_t *p, uint32_t v)
{
    p[0] = (uint8_t)v;
    p[1] = (uint8_t)(v >> 8);
    p[2] = (uint8_t)(v >> 16);
    p[3] = (uint8_t)(v >> 24);
}

static uint32_t get_u32(const uint8_t *p)
{
    return (uint32_t)p[0] | (uint32_t)p[1] << 8 | (uint32_t)p[2] << 16 | (uint32_t)p[3] << 24;
}

/* 32 four-bit values v[0..31] -> 16 bytes in the nibble order above. */
static void pack_nibbles32(const uint8_t *v, uint8_t *out16)
{
    for (int w = 0; w < 4; w++) {
        uint32_t d = 0;
        for (int p = 0; p < 8; p++)
            d |= (uint32_t)(v[8 * w + nib_elem(p)] & 15u) << (4 * p);
        put_u32(out16 + 4 * w, d);
    }
}

static void unpack_nibbles32(const uint8_t *in16, uint8_t *v)
{
    for (int w = 0; w < 4; w++) {
        uint32_t d = get_u32(in16 + 4 * w);
        for (int p = 0; p < 8; p++)
            v[8 * w + nib_elem(p)] = (uint8_t)((d >> (4 * p)) & 15u);
    }
}

void oracle_pack_q4k(const uint16_t *d16, const uint16_t *dmin16, const uint8_t *sc,
                     const uint8_t *mq, const uint8_t *q, int64_t rows, int64_t cols,
                     uint8_t *buf)
{
    int64_t G = rows * cols / 256;
    uint8_t *C = buf, *S = buf + 128 * G;
    for (int64_t g = 0; g < G; g++) {
        for (int j = 0; j < 8; j++)
            pack_nibbles32(q + 256 * g + 32 * j, C + 128 * g + 16 * j);
        uint8_t *h = S + 16 * g;
        h[0] = (uint8_t)d16[g];
        h[1] = (uint8_t)(d16[g] >> 8);
        h[2] = (uint8_t)dmin16[g];
        h[3] = (uint8_t)(dmin16[g] >> 8);
        uint32_t lo_s = 0, lo_m = 0, hi = 0;
        for (int j = 0; j < 8; j++) {
            lo_s |= (uint32_t)(sc[8 * g + j] & 15u) << (4 * j);
            lo_m |= (uint32_t)(mq[8 * g + j] & 15u) << (4 * j);
            hi |= (uint32_t)((sc[8 * g + j] >> 4) & 3u) << (2 * j);
            hi |= (uint32_t)((mq[8 * g + j] >> 4) & 3u) << (16 + 2 * j);
        }
        put_u32(h + 4, lo_s);
        put_u32(h + 8, lo_m);
        put_u32(h + 12, hi);
    }
}

void oracle_unpack_q4k(const uint8_t *buf, int64_t rows, int64_t cols, uint16_t *d16,
                       uint16_t *dmin16, uint8_t *sc, uint8_t *mq, uint8_t *q)
{
    int64_t G = rows * cols / 256;
    const uint8_t *C = buf, *S = buf + 128 * G;
    for (int64_t g = 0; g < G; g++) {
        for (int j = 0; j < 8; j++)
            unpack_nibbles32(C + 128 * g + 16 * j, q + 256 * g + 32 * j);
        const uint8_t *h = S + 16 * g;
        d16[g] = (uint16_t)(h[0] | h[1] << 8);
        dmin16[g] = (uint16_t)(h[2] | h[3] << 8);
        uint32_t lo_s = get_u32(h + 4), lo_m = get_u32(h + 8), hi = get_u32(h + 12);
        for (int j = 0; j < 8; j++) {
            sc[8 * g + j] = (uint8_t)(((lo_s >> (4 * j)) & 15u) | ((hi >> (2 * j)) & 3u) << 4);
            mq[8 * g + j] = (uint8_t)(((lo_m >> (4 * j)) & 15u) | ((hi >> (16 + 2 * j)) & 3u) << 4);
        }
    }
}

/* Q6K code plane of one group (192 bytes).  The group is 8 chunks of 32
 * elements (chunk c = elements 32c..32c+31 = sub-blocks 2c and 2c+1).
 *   bytes 0..127:   low 4 bits of u; chunk c in bytes 16c..16c+15, in the
 *                   Q4K nibble order (dword w = elements 8w..8w+7).
 *   bytes 128..191: high 2 bits of u; chunk c owns the two dwords at
 *                   128+8c+4h (h = 0, 1).  Dword h covers the octets
 *                   o = 0, 1 (elements 16h+8o .. 16h+8o+7); for the pair
 *                   s = 0..3 of an octet, bits 8o+2s..8o+2s+1 hold the high
 *                   bits of element 16h+8o+2s and bits 16+8o+2s..17+8o+2s
 *                   those of element 16h+8o+2s+1.
 */
static void q6k_pack_group(const int8_t *qg, uint8_t *C)
{
    for (int c = 0; c < 8; c++) {
        uint8_t lo[32];
        for (int i = 0; i < 32; i++)
            lo[i] = (uint8_t)((qg[32 * c + i] + 32) & 15);
        pack_nibbles32(lo, C + 16 * c);
        for (int h = 0; h < 2; h++) {
            uint32_t d = 0;
            for (int o = 0; o < 2; o++)
                for (int s = 0; s < 4; s++) {
                    int e = 32 * c + 16 * h + 8 * o + 2 * s;
                    uint32_t u0 = (uint32_t)(qg[e] + 32) >> 4;
                    uint32_t u1 = (uint32_t)(qg[e + 1] + 32) >> 4;
                    d |= u0 << (2 * s + 8 * o);
                    d |= u1 << (16 + 2 * s + 8 * o);
                }
            put_u32(C + 128 + 8 * c + 4 * h, d);
        }
    }
}

static void q6k_unpack_group(const uint8_t *C, int8_t *qg)
{
    for (int c = 0; c < 8; c++) {
        uint8_t lo[32];
        unpack_nibbles32(C + 16 * c, lo);
        for (int h = 0; h < 2; h++) {
            uint32_t d = get_u32(C + 128 + 8 * c + 4 * h);
            for (int o = 0; o < 2; o++)
                for (int s = 0; s < 4; s++) {
                    int i0 = 16 * h + 8 * o + 2 * s;
                    uint32_t u0 = lo[i0] | ((d >> (2 * s + 8 * o)) & 3u) << 4;
                    uint32_t u1 = lo[i0 + 1] | ((d >> (16 + 2 * s + 8 * o)) & 3u) << 4;
                    qg[32 * c + i0] = (int8_t)((int)u0 - 32);
                    qg[32 * c + i0 + 1] = (int8_t)((int)u1 - 32);
                }
        }
    }
}

void oracle_pack_q6k(const uint16_t *d16, const int8_t *sc, const int8_t *q, int64_t rows,
                     int64_t cols, uint8_t *buf)
{
    int64_t G = rows * cols / 256;
    uint8_t *C = buf, *S = buf + 192 * G, *D = buf + 208 * G;
    for (int64_t g = 0; g < G; g++) {
        q6k_pack_group(q + 256 * g, C + 192 * g);
        memcpy(S + 16 * g, sc + 16 * g, 16);
        D[2 * g] = (uint8_t)d16[g];
        D[2 * g + 1] = (uint8_t)(d16[g] >> 8);
    }
}

void oracle_unpack_q6k(const uint8_t *buf, int64_t rows, int64_t cols, uint16_t *d16,
                       int8_t *sc, int8_t *q)
{
    int64_t G = rows * cols / 256;
    const uint8_t *C = buf, *S = buf + 192 * G, *D = buf + 208 * G;
    for (int64_t g = 0; g < G; g++) {
        q6k_unpack_group(C + 192 * g, q + 256 * g);
        memcpy(sc + 16 * g, S + 16 * g, 16);
        d16[g] = (uint16_t)(D[2 * g] | D[2 * g + 1] << 8);
    }
}

/* ------------------------------------------------------------------ */
/* Further formats: Q5K, Q3K, Q2K and Q4_0, Q4_1, Q5_0, Q5_1           */
/* ------------------------------------------------------------------ */
/*
 * Page "Quantization types": section "Numeric shorthands" resolves ISQ
 * levels 5, 3 and 2 to Q5K, Q3K and Q2K on CUDA / CPU; sections "Q*K
 * family" (q2k 2, q3k 3, q5k 5 bits) and "Legacy GGML types" (q4_0/q4_1
 * 4 bits, q5_0/q5_1 5 bits) name the formats.  The page gives bit widths
 * only.  Readings, chosen to match the Q4K / Q6K / Q8_0 readings above and
 * to keep the GGML byte counts (Q5K 176, Q3K 110, Q2K 84 bytes per 256
 * elements; Q4_0 18, Q4_1 20, Q5_0 22, Q5_1 24 bytes per 32):
 *   K-quants, groups of 256:
 *     Q5K: 8 sub-blocks of 32, affine (the Q4K rule with 5-bit codes and
 *          s_j = (hi - lo) / 31), 6-bit sc/m, fp16 d and dmin.
 *     Q3K: 16 sub-blocks of 16, symmetric (the Q6K rule with 3-bit codes:
 *          s_j = max|x| / 3, codes in [-4, 3]), 6-bit sc (d = max s / 63).
 *     Q2K: 16 sub-blocks of 16, affine (s_j = (hi - lo) / 3, codes in
 *          [0, 3]), 4-bit sc/m (d = max s / 15, dmin = max m / 15).
 *   Legacy, blocks of 32:
 *     Q4_0 / Q5_0: symmetric, d = F16(max|x| / 7 or / 15) (as Q8_0's
 *          max|x| / 127), codes RHA(x / d) in [-8, 7] / [-16, 15].
 *     Q4_1 / Q5_1: affine on the true min and max, d = F16((max - min) /
 *          15 or 31), m = F16(min) (signed, clamped to +-65504), codes
 *          RHA((x - m) / d) in [0, 15] / [0, 31]; decoded as d q + m.
 * Every step is binary32, one operation at a time, as for the formats
 * above; d = 0 (or S_j = 0) gives codes 0.
 */

#define FMT_Q2K 3
#define FMT_Q3K 4
#define FMT_Q5K 5
#define FMT_Q4_0 7
#define FMT_Q4_1 8
#define FMT_Q5_0 9
#define FMT_Q5_1 10

/* K-quant parameters: sub-blocks, their length, code bits, affine?, scale bits */
static void kq_params(int64_t fmt, int *ns, int *len, int *bits, int *affine, int *sbits)
{
    if (fmt == FMT_Q5K) {
        *ns = 8; *len = 32; *bits = 5; *affine = 1; *sbits = 6;
    } else if (fmt == FMT_Q3K) {
        *ns = 16; *len = 16; *bits = 3; *affine = 0; *sbits = 6;
    } else {
        *ns = 16; *len = 16; *bits = 2; *affine = 1; *sbits = 4;
    }
}

/* One K-quant group.  Affine: per sub-block lo = min(0, min x), hi = max x,
 * s = (hi - lo) / (2^b - 1), m = 0 - lo; symmetric: s = max|x| /
 * (2^(b-1) - 1).  Then d16 = F16(max s / (2^sb - 1)), dmin16 likewise from
 * m, sc/mq = clamp(RHA(s / d), 0, 2^sb - 1), S = d sc, M = dmin mq (exact),
 * codes clamp(RHA((x + M) / S), 0, 2^b - 1) or clamp(RHA(x / S),
 * -2^(b-1), 2^(b-1) - 1). */
static void kq_group(int64_t fmt, const uint16_t *x16, uint16_t *d16o, uint16_t *dm16o, uint8_t *sc,
                     uint8_t *mq, int8_t *q)
{
    int ns, len, bits, affine, sbits;
    kq_params(fmt, &ns, &len, &bits, &affine, &sbits);
    const float qden = affine ? (float)((1 << bits) - 1) : (float)((1 << (bits - 1)) - 1);
    const float sden = (float)((1 << sbits) - 1);
    float x[256], s[16], m[16];
    for (int i = 0; i < 256; i++)
        x[i] = bf16_in(x16[i]);
    float smax = 0.0f, mmax = 0.0f;
    for (int j = 0; j < ns; j++) {
        if (affine) {
            float lo = 0.0f, hi = x[len * j];
            for (int i = 0; i < len; i++) {
                float v = x[len * j + i];
                if (v < lo)
                    lo = v;
                if (v > hi)
                    hi = v;
            }
            s[j] = (hi - lo) / qden;
            m[j] = 0.0f - lo;
        } else {
            float a = 0.0f;
            for (int i = 0; i < len; i++) {
                float ax = fabsf(x[len * j + i]);
                if (ax > a)
                    a = ax;
            }
            s[j] = a / qden;
            m[j] = 0.0f;
        }
        if (s[j] > smax)
            smax = s[j];
        if (m[j] > mmax)
            mmax = m[j];
    }
    uint16_t d16 = scale_f16(smax / sden);
    uint16_t dm16 = affine ? scale_f16(mmax / sden) : 0;
    float df = oracle_f32_from_f16(d16), dmf = oracle_f32_from_f16(dm16);
    const int smaxc = (1 << sbits) - 1;
    for (int j = 0; j < ns; j++) {
        sc[j] = (uint8_t)(df > 0.0f ? clamp_code(roundf(s[j] / df), 0, smaxc) : 0);
        mq[j] = (uint8_t)(affine && dmf > 0.0f ? clamp_code(roundf(m[j] / dmf), 0, smaxc) : 0);
        float S = df * (float)sc[j];
        float M = dmf * (float)mq[j];
        for (int i = 0; i < len; i++) {
            float v = x[len * j + i];
            int c;
            if (!(S > 0.0f))
                c = 0;
            else if (affine)
                c = clamp_code(roundf((v + M) / S), 0, (1 << bits) - 1);
            else
                c = clamp_code(roundf(v / S), -(1 << (bits - 1)), (1 << (bits - 1)) - 1);
            q[len * j + i] = (int8_t)c;
        }
    }
    *d16o = d16;
    *dm16o = dm16;
}

/* rows*cols bf16 (cols % 256 == 0) -> K-quant fields per group g: d16[g],
 * dmin16[g] (0 for Q3K), sc[g][16], mq[g][16] (the first 8 used by Q5K;
 * mq 0 for Q3K), q[rows][cols]. */
void oracle_quantize_kq(int64_t fmt, const uint16_t *w, int64_t rows, int64_t cols, uint16_t *d16,
                        uint16_t *dmin16, uint8_t *sc, uint8_t *mq, int8_t *q)
{
    int64_t ng = rows * (cols / 256);
#pragma omp parallel for schedule(static)
    for (int64_t g = 0; g < ng; g++) {
        memset(sc + 16 * g, 0, 16);
        memset(mq + 16 * g, 0, 16);
        kq_group(fmt, w + 256 * g, d16 + g, dmin16 + g, sc + 16 * g, mq + 16 * g, q + 256 * g);
    }
}

/* Exact values: affine (d sc_j) q - (dmin mq_j); symmetric (d sc_j) q. */
void oracle_dequant_kq(int64_t fmt, const uint16_t *d16, const uint16_t *dmin16, const uint8_t *sc,
                       const uint8_t *mq, const int8_t *q, int64_t n_elems, double *out)
{
    int ns, len, bits, affine, sbits;
    kq_params(fmt, &ns, &len, &bits, &affine, &sbits);
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < n_elems; e++) {
        int64_t g = e / 256;
        int j = (int)((e % 256) / len);
        double S = (double)oracle_f32_from_f16(d16[g]) * (double)sc[16 * g + j];
        double M = affine ? (double)oracle_f32_from_f16(dmin16[g]) * (double)mq[16 * g + j] : 0.0;
        out[e] = S * (double)q[e] - M;
    }
}

/* One legacy block of 32 (rule in the section comment). */
static void leg_block(int64_t fmt, const uint16_t *x16, uint16_t *d16o, uint16_t *m16o, int8_t *q)
{
    const int bits = (fmt == FMT_Q4_0 || fmt == FMT_Q4_1) ? 4 : 5;
    const int affine = fmt == FMT_Q4_1 || fmt == FMT_Q5_1;
    float x[32];
    for (int i = 0; i < 32; i++)
        x[i] = bf16_in(x16[i]);
    if (!affine) {
        float a = 0.0f;
        for (int i = 0; i < 32; i++)
            if (fabsf(x[i]) > a)
                a = fabsf(x[i]);
        uint16_t d16 = scale_f16(a / (float)((1 << (bits - 1)) - 1));
        float df = oracle_f32_from_f16(d16);
        for (int i = 0; i < 32; i++)
            q[i] = (int8_t)(df == 0.0f ? 0 : clamp_code(roundf(x[i] / df), -(1 << (bits - 1)), (1 << (bits - 1)) - 1));
        *d16o = d16;
        *m16o = 0;
        return;
    }
    float lo = x[0], hi = x[0];
    for (int i = 1; i < 32; i++) {
        if (x[i] < lo)
            lo = x[i];
        if (x[i] > hi)
            hi = x[i];
    }
    uint16_t d16 = scale_f16((hi - lo) / (float)((1 << bits) - 1));
    float mc = lo < -65504.0f ? -65504.0f : (lo > 65504.0f ? 65504.0f : lo);
    uint16_t m16 = oracle_f16_from_f32(mc);
    float df = oracle_f32_from_f16(d16), mf = oracle_f32_from_f16(m16);
    for (int i = 0; i < 32; i++)
        q[i] = (int8_t)(df == 0.0f ? 0 : clamp_code(roundf((x[i] - mf) / df), 0, (1 << bits) - 1));
    *d16o = d16;
    *m16o = m16;
}

/* rows*cols bf16 (cols % 32 == 0) -> legacy fields per block b: d16[b],
 * m16[b] (0 for the symmetric types), q[rows][cols]. */
void oracle_quantize_leg(int64_t fmt, const uint16_t *w, int64_t rows, int64_t cols, uint16_t *d16,
                         uint16_t *m16, int8_t *q)
{
    int64_t nb = rows * (cols / 32);
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nb; b++)
        leg_block(fmt, w + 32 * b, d16 + b, m16 + b, q + 32 * b);
}

/* Exact values: d q (+ m for the affine types). */
void oracle_dequant_leg(int64_t fmt, const uint16_t *d16, const uint16_t *m16, const int8_t *q,
                        int64_t n_elems, double *out)
{
    const int affine = fmt == FMT_Q4_1 || fmt == FMT_Q5_1;
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < n_elems; e++) {
        double d = (double)oracle_f32_from_f16(d16[e / 32]);
        double m = affine ? (double)oracle_f32_from_f16(m16[e / 32]) : 0.0;
        out[e] = d * (double)q[e] + m;
    }
}

/*
 * Planar layouts of the further formats (G = rows*cols/256 groups, B =
 * rows*cols/32 blocks; every plane starts at a multiple of 16 bytes, the
 * buffer is zero-padded to one; codes are stored in natural element order):
 *   Q5K  [L: G*128, element e of a group at byte e/2, low nibble for even e]
 *        [H: G*32, high bit of element e at bit e%8 of byte e/8]
 *        [S: G*16, the Q4K header: d, dmin, sc/mq low-nibble dwords, high-pair dword]
 *   Q3K  [L: G*64, low 2 bits of u = q+4 of element e at bits 2(e%4) of byte e/4]
 *        [H: G*32, bit 2 of u at bit e%8 of byte e/8]
 *        [S: G*12, dwords: nibble j of dword 0 / 1 = sc_j & 15 for j < 8 / j >= 8,
 *                  bits 2j..2j+1 of dword 2 = sc_j >> 4]
 *        [D: at round16(108 G), G*2 fp16 d]
 *   Q2K  [C: G*64, code of element e at bits 2(e%4) of byte e/4]
 *        [S: G*16, byte j = sc_j | mq_j << 4]  [D: G*4, d then dmin]
 *   Q4_0 / Q4_1  [C: B*16, u (= q+8 for Q4_0) of element i of a block at byte i/2,
 *                 low nibble for even i] [D: B*2 fp16 d] [M: B*2 fp16 m (Q4_1)]
 *   Q5_0 / Q5_1  [C: B*16 low nibbles of u (= q+16 for Q5_0)] [H: B*4, bit 4 of u
 *                 at bit i of the block's dword] [D: B*2] [M: B*2 (Q5_1)]
 */
static int64_t up16(int64_t v) { return (v + 15) / 16 * 16; }

/* plane offsets o[0..3] and total bytes */
int64_t oracle_more_layout(int64_t fmt, int64_t rows, int64_t cols, int64_t *o)
{
    int64_t n = rows * cols, G = n / 256, B = n / 32;
    o[0] = o[1] = o[2] = o[3] = 0;
    switch (fmt) {
    case FMT_Q5K: o[1] = 128 * G; o[2] = 160 * G; return 176 * G;
    case FMT_Q3K: o[1] = 64 * G; o[2] = 96 * G; o[3] = up16(108 * G); return up16(o[3] + 2 * G);
    case FMT_Q2K: o[1] = 64 * G; o[2] = 80 * G; return up16(84 * G);
    case FMT_Q4_0: o[1] = 16 * B; return up16(18 * B);
    case FMT_Q4_1: o[1] = 16 * B; o[2] = up16(18 * B); return up16(o[2] + 2 * B);
    case FMT_Q5_0: o[1] = 16 * B; o[2] = up16(20 * B); return up16(o[2] + 2 * B);
    default: /* Q5_1 */ o[1] = 16 * B; o[2] = up16(20 * B); o[3] = up16(o[2] + 2 * B); return up16(o[3] + 2 * B);
    }
}

static void put_u16(uint8_t *p, uint16_t v)
{
    p[0] = (uint8_t)v;
    p[1] = (uint8_t)(v >> 8);
}
static uint16_t get_u16(const uint8_t *p) { return (uint16_t)(p[0] | p[1] << 8); }

/* K-quant fields -> bytes (buf zeroed by the caller) */
void oracle_pack_kq(int64_t fmt, const uint16_t *d16, const uint16_t *dmin16, const uint8_t *sc,
                    const uint8_t *mq, const int8_t *q, int64_t rows, int64_t cols, uint8_t *buf)
{
    int64_t o[4];
    oracle_more_layout(fmt, rows, cols, o);
    int64_t G = rows * cols / 256;
    for (int64_t g = 0; g < G; g++) {
        const int8_t *qg = q + 256 * g;
        const uint8_t *s = sc + 16 * g, *m = mq + 16 * g;
        if (fmt == FMT_Q5K) {
            for (int e = 0; e < 256; e++) {
                uint32_t u = (uint32_t)qg[e];
                buf[o[0] + 128 * g + e / 2] |= (uint8_t)((u & 15u) << (4 * (e % 2)));
                buf[o[1] + 32 * g + e / 8] |= (uint8_t)((u >> 4) << (e % 8));
            }
            uint8_t *h = buf + o[2] + 16 * g;
            put_u16(h, d16[g]);
            put_u16(h + 2, dmin16[g]);
            uint32_t a = 0, b = 0, c = 0;
            for (int j = 0; j < 8; j++) {
                a |= (uint32_t)(s[j] & 15u) << (4 * j);
                b |= (uint32_t)(m[j] & 15u) << (4 * j);
                c |= (uint32_t)(s[j] >> 4) << (2 * j) | (uint32_t)(m[j] >> 4) << (16 + 2 * j);
            }
            put_u32(h + 4, a);
            put_u32(h + 8, b);
            put_u32(h + 12, c);
        } else if (fmt == FMT_Q3K) {
            for (int e = 0; e < 256; e++) {
                uint32_t u = (uint32_t)(qg[e] + 4);
                buf[o[0] + 64 * g + e / 4] |= (uint8_t)((u & 3u) << (2 * (e % 4)));
                buf[o[1] + 32 * g + e / 8] |= (uint8_t)((u >> 2) << (e % 8));
            }
            uint32_t a = 0, b = 0, c = 0;
            for (int j = 0; j < 16; j++) {
                if (j < 8)
                    a |= (uint32_t)(s[j] & 15u) << (4 * j);
                else
                    b |= (uint32_t)(s[j] & 15u) << (4 * (j - 8));
                c |= (uint32_t)(s[j] >> 4) << (2 * j);
            }
            put_u32(buf + o[2] + 12 * g, a);
            put_u32(buf + o[2] + 12 * g + 4, b);
            put_u32(buf + o[2] + 12 * g + 8, c);
            put_u16(buf + o[3] + 2 * g, d16[g]);
        } else {
            for (int e = 0; e < 256; e++)
                buf[o[0] + 64 * g + e / 4] |= (uint8_t)(((uint32_t)qg[e] & 3u) << (2 * (e % 4)));
            for (int j = 0; j < 16; j++)
                buf[o[1] + 16 * g + j] = (uint8_t)(s[j] | m[j] << 4);
            put_u16(buf + o[2] + 4 * g, d16[g]);
            put_u16(buf + o[2] + 4 * g + 2, dmin16[g]);
        }
    }
}

void oracle_unpack_kq(int64_t fmt, const uint8_t *buf, int64_t rows, int64_t cols, uint16_t *d16,
                      uint16_t *dmin16, uint8_t *sc, uint8_t *mq, int8_t *q)
{
    int64_t o[4];
    oracle_more_layout(fmt, rows, cols, o);
    int64_t G = rows * cols / 256;
    for (int64_t g = 0; g < G; g++) {
        int8_t *qg = q + 256 * g;
        uint8_t *s = sc + 16 * g, *m = mq + 16 * g;
        memset(s, 0, 16);
        memset(m, 0, 16);
        if (fmt == FMT_Q5K) {
            for (int e = 0; e < 256; e++) {
                uint32_t lo = (buf[o[0] + 128 * g + e / 2] >> (4 * (e % 2))) & 15u;
                uint32_t hi = (buf[o[1] + 32 * g + e / 8] >> (e % 8)) & 1u;
                qg[e] = (int8_t)(lo | hi << 4);
            }
            const uint8_t *h = buf + o[2] + 16 * g;
            d16[g] = get_u16(h);
            dmin16[g] = get_u16(h + 2);
            uint32_t a = get_u32(h + 4), b = get_u32(h + 8), c = get_u32(h + 12);
            for (int j = 0; j < 8; j++) {
                s[j] = (uint8_t)(((a >> (4 * j)) & 15u) | ((c >> (2 * j)) & 3u) << 4);
                m[j] = (uint8_t)(((b >> (4 * j)) & 15u) | ((c >> (16 + 2 * j)) & 3u) << 4);
            }
        } else if (fmt == FMT_Q3K) {
            for (int e = 0; e < 256; e++) {
                uint32_t lo = (buf[o[0] + 64 * g + e / 4] >> (2 * (e % 4))) & 3u;
                uint32_t hi = (buf[o[1] + 32 * g + e / 8] >> (e % 8)) & 1u;
                qg[e] = (int8_t)((int)(lo | hi << 2) - 4);
            }
            uint32_t a = get_u32(buf + o[2] + 12 * g), b = get_u32(buf + o[2] + 12 * g + 4),
                     c = get_u32(buf + o[2] + 12 * g + 8);
            for (int j = 0; j < 16; j++)
                s[j] = (uint8_t)((((j < 8 ? a : b) >> (4 * (j % 8))) & 15u) | ((c >> (2 * j)) & 3u) << 4);
            d16[g] = get_u16(buf + o[3] + 2 * g);
            dmin16[g] = 0;
        } else {
            for (int e = 0; e < 256; e++)
                qg[e] = (int8_t)((buf[o[0] + 64 * g + e / 4] >> (2 * (e % 4))) & 3u);
            for (int j = 0; j < 16; j++) {
                s[j] = buf[o[1] + 16 * g + j] & 15u;
                m[j] = buf[o[1] + 16 * g + j] >> 4;
            }
            d16[g] = get_u16(buf + o[2] + 4 * g);
            dmin16[g] = get_u16(buf + o[2] + 4 * g + 2);
        }
    }
}

void oracle_pack_leg(int64_t fmt, const uint16_t *d16, const uint16_t *m16, const int8_t *q, int64_t rows,
                     int64_t cols, uint8_t *buf)
{
    int64_t o[4];
    oracle_more_layout(fmt, rows, cols, o);
    int64_t B = rows * cols / 32;
    const int five = fmt == FMT_Q5_0 || fmt == FMT_Q5_1;
    const int bias = fmt == FMT_Q4_0 ? 8 : (fmt == FMT_Q5_0 ? 16 : 0);
    const int affine = fmt == FMT_Q4_1 || fmt == FMT_Q5_1;
    for (int64_t b = 0; b < B; b++) {
        uint32_t hib = 0;
        for (int i = 0; i < 32; i++) {
            uint32_t u = (uint32_t)(q[32 * b + i] + bias);
            buf[o[0] + 16 * b + i / 2] |= (uint8_t)((u & 15u) << (4 * (i % 2)));
            hib |= (u >> 4) << i;
        }
        if (five) {
            put_u32(buf + o[1] + 4 * b, hib);
            put_u16(buf + o[2] + 2 * b, d16[b]);
            if (affine)
                put_u16(buf + o[3] + 2 * b, m16[b]);
        } else {
            put_u16(buf + o[1] + 2 * b, d16[b]);
            if (affine)
                put_u16(buf + o[2] + 2 * b, m16[b]);
        }
    }
}

void oracle_unpack_leg(int64_t fmt, const uint8_t *buf, int64_t rows, int64_t cols, uint16_t *d16,
                       uint16_t *m16, int8_t *q)
{
    int64_t o[4];
    oracle_more_layout(fmt, rows, cols, o);
    int64_t B = rows * cols / 32;
    const int five = fmt == FMT_Q5_0 || fmt == FMT_Q5_1;
    const int bias = fmt == FMT_Q4_0 ? 8 : (fmt == FMT_Q5_0 ? 16 : 0);
    const int affine = fmt == FMT_Q4_1 || fmt == FMT_Q5_1;
    for (int64_t b = 0; b < B; b++) {
        uint32_t hib = five ? get_u32(buf + o[1] + 4 * b) : 0u;
        for (int i = 0; i < 32; i++) {
            uint32_t u = ((buf[o[0] + 16 * b + i / 2] >> (4 * (i % 2))) & 15u) | ((hib >> i) & 1u) << 4;
            q[32 * b + i] = (int8_t)((int)u - bias);
        }
        d16[b] = get_u16(buf + (five ? o[2] : o[1]) + 2 * b);
        m16[b] = affine ? get_u16(buf + (five ? o[3] : o[2]) + 2 * b) : 0;
    }
}

/* ------------------------------------------------------------------ */
/* FP8 E4M3 with per-row (channel) scales; W8A16 and dynamic W8A8      */
/* ------------------------------------------------------------------ */
/*
 * Page "Quantization types", section "FP8": E4M3 FP8 (4-bit exponent, 3-bit
 * mantissa) produced by ISQ; symmetric E4M3 weights with tensor, channel or
 * block scales; W8A16 converts each weight tile to BF16 inside the GEMM;
 * dynamic per-token W8A8 quantizes the activations per token before an FP8
 * GEMM.  Readings: channel (per output row) scales; the E4M3 variant
 * without infinities (largest finite 448, exponent bias 7, subnormals of
 * 2^-9); a scale is s = max|x| / 448 in binary32 and a code is E4M3(x / s),
 * rounded to nearest even after the binary32 division and saturated to
 * +-448; s = 0 gives codes 0.  Values: s * e4m3(q); the W8A8 product is
 * s_m s_n sum_k e4m3(qx) e4m3(qw), exact in fp64.
 */

/* E4M3 bits -> value (exact).  0x7F / 0xFF are NaN (never produced here). */
double oracle_e4m3_value(uint8_t b)
{
    int sgn = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9); /* m/8 * 2^-6 */
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sgn ? -v : v;
}

/* binary32 -> E4M3 bits: round to nearest, ties to even, saturate to 448. */
uint8_t oracle_e4m3_from_f32(float v)
{
    uint8_t sgn = signbit(v) ? 0x80 : 0;
    double a = fabs((double)v);
    if (a >= 448.0)
        return (uint8_t)(sgn | 0x7E); /* 448 = 1.75 * 2^8 */
    /* the grid near a: spacing 2^(e-10) for normals (e = floor(log2 a) >= -6), 2^-9 below */
    int e;
    frexp(a, &e);          /* a = f * 2^e, f in [0.5, 1) */
    e -= 1;                /* a in [2^e, 2^(e+1)) */
    double ulp = e < -6 ? ldexp(1.0, -9) : ldexp(1.0, e - 3);
    double k = a / ulp;    /* exact: a is binary32, ulp a power of two */
    double r = floor(k);
    double rest = k - r;
    if (rest > 0.5 || (rest == 0.5 && fmod(r, 2.0) == 1.0))
        r += 1.0;
    double q = r * ulp;    /* the rounded magnitude, exact */
    if (q >= 448.0)
        return (uint8_t)(sgn | 0x7E);
    if (q == 0.0)
        return sgn;
    int qe;
    frexp(q, &qe);
    qe -= 1;
    uint8_t bits;
    if (qe < -6)
        bits = (uint8_t)(q / ldexp(1.0, -9)); /* subnormal: m = q / 2^-9 */
    else
        bits = (uint8_t)(((qe + 7) << 3) | (int)((q / ldexp(1.0, qe) - 1.0) * 8.0));
    return (uint8_t)(sgn | bits);
}

void oracle_e4m3_from_f32_array(const float *in, int64_t n, uint8_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_e4m3_from_f32(in[i]);
}

/* rows*cols bf16 -> codes [rows][cols] and s [rows] (binary32 bits).
 * Steps: a = max|x| (exact), s = a / 448, code = E4M3(x / s) (0 if s == 0). */
void oracle_quantize_fp8(const uint16_t *w, int64_t rows, int64_t cols, uint8_t *q, float *s)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        const uint16_t *x = w + r * cols;
        float a = 0.0f;
        for (int64_t i = 0; i < cols; i++) {
            float ax = fabsf(bf16_in(x[i]));
            if (ax > a)
                a = ax;
        }
        float sc = a / 448.0f;
        s[r] = sc;
        for (int64_t i = 0; i < cols; i++)
            q[r * cols + i] = sc == 0.0f ? 0 : oracle_e4m3_from_f32(bf16_in(x[i]) / sc);
    }
}

/* W = s_row * e4m3(q), exact in fp64 */
void oracle_dequant_fp8(const uint8_t *q, const float *s, int64_t rows, int64_t cols, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < rows * cols; e++)
        out[e] = (double)s[e / cols] * oracle_e4m3_value(q[e]);
}

/* W8A8: Y[m][n] = sx[m] sw[n] sum_k e4m3(qx[m][k]) e4m3(qw[n][k]) (exact
 * sum in fp64), den = sx sw sum |..|, for a list of (m, n) pairs. */
void oracle_matmul_fp8(const uint8_t *qx, const float *sx, const uint8_t *qw, const float *sw, int64_t K,
                       const int64_t *mi, const int64_t *ni, int64_t npairs, double *Y, double *den)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < npairs; i++) {
        double acc = 0.0, a = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double p = oracle_e4m3_value(qx[mi[i] * K + k]) * oracle_e4m3_value(qw[ni[i] * K + k]);
            acc += p;
            a += fabs(p);
        }
        double sc = (double)sx[mi[i]] * (double)sw[ni[i]];
        Y[i] = sc * acc;
        den[i] = sc * a;
    }
}
