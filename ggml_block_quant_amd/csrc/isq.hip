// isq.hip -- block-parallel in-situ quantization (ISQ) of bf16 weights into
// Q8_0, Q4K and Q6K blocks, and the exact dequantizer used as a test aid.
//
// Page "Quantization types" (mistral.rs reference): ISQ quantizes weights at
// load time (introduction: "--isq N forces runtime ISQ"); the formats are
// q8_0 ("Legacy GGML types"), q4k and q6k ("Q*K family").
//
// Work split: one lane owns 8 consecutive elements of the flattened [N][K]
// tensor (one 16-byte load).  A Q8_0 block (32 elements) is 4 lanes; a Q4K
// or Q6K group (256 elements) is 32 lanes, so every reduction runs inside a
// wavefront with cross-lane shuffles and no LDS.  Codes leave as one dword
// per lane, so stores are coalesced too.
//
// Arithmetic is binary32 IEEE, one rounding per operation, in exactly the
// order of the reference definition, so that codes and scales are
// bit-exact:  this file is compiled with -ffp-contract=off; x / y is the
// correctly rounded division; max/min are exact; roundf rounds half away
// from zero; fp16 scales are clamped to 65504 and converted with
// v_cvt_f16_f32 (round to nearest even, subnormals kept).  A -0.0 input is
// read as +0.0 (x + 0.0f), so the sign of a zero never reaches a scale.
#include "qlinear_internal.h"
#include "decode.h"

namespace ql {
namespace {

__device__ __forceinline__ void load8(const uint4 v, float x[8])
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        x[2 * i] = __uint_as_float(w[i] << 16) + 0.0f;
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u) + 0.0f;
    }
}

// F16 of a non-negative scale: clamp to the largest finite binary16, round
// to nearest even.  Returns the bits; *back receives the fp16 value as fp32.
__device__ __forceinline__ uint32_t scale_f16(float v, float *back)
{
    v = fminf(v, 65504.0f);
    const _Float16 h = (_Float16)v;
    *back = (float)h;
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// Round half away from zero, then clamp to [lo, hi] (integer-valued bounds).
__device__ __forceinline__ int code_of(float v, float lo, float hi)
{
    float r = roundf(v);
    r = fminf(fmaxf(r, lo), hi);
    return (int)r;
}

// RHA of the correctly rounded quotient fl(u / S), for S > 0, given
// r = fl(1 / S).  t = u*r rounds twice (r, the product), so it lies within
// 3 * 2^-24 * |t| of fl(u / S); both round (half away from zero) to the same
// integer unless a half-integer lies that close to t.  Only then is the
// quotient computed by the correctly rounded division, so the code is the
// one the definition gives, with one multiply in the common case.  Away
// from those cases RHA(t) = sign(t) floor(|t| + 1/2) exactly: the sum's
// rounding error (at most 2^-24 (|t| + 1/2) <= 2^-23 |t| for |t| >= 1/2,
// 2^-25 below) is smaller than the distance of |t| + 1/2 from an integer.
__device__ __forceinline__ float rha_quot(float u, float S, float r)
{
    const float t = u * r;
    const float a = fabsf(t);
    float q = copysignf(floorf(a + 0.5f), t);
    if (fabsf(__builtin_amdgcn_fractf(a) - 0.5f) <= 2.5e-7f * a)
        q = roundf(u / S);
    return q;
}

// rha_quot where the code is clamped at 0 from below (Q4K): for t < 0 both
// RHA(t) and floor(t + 0.5) are at most 0, so the sign restore is dropped;
// for t >= 0 they are the same value
__device__ __forceinline__ float rha_quot_nonneg(float u, float S, float r)
{
    const float t = u * r;
    float q = floorf(t + 0.5f);
    if (fabsf(__builtin_amdgcn_fractf(t) - 0.5f) <= 2.5e-7f * fabsf(t))
        q = roundf(u / S);
    return q;
}

// Even elements of an octet in the low half of a dword, odd ones in the high
// half: nibble p holds element 2p (p < 4) or 2(p-4)+1 (p >= 4).
__device__ __forceinline__ uint32_t pack_nibbles(const int q[8])
{
    return (uint32_t)q[0] | (uint32_t)q[2] << 4 | (uint32_t)q[4] << 8 | (uint32_t)q[6] << 12 |
           (uint32_t)q[1] << 16 | (uint32_t)q[3] << 20 | (uint32_t)q[5] << 24 |
           (uint32_t)q[7] << 28;
}

// One lane per 32 consecutive elements (a Q8_0 block, a Q4K sub-block, a
// Q6K chunk of two sub-blocks): 64 bytes of bf16 in flight per lane, and
// the per-block scale arithmetic (IEEE divisions included) done once per
// 32 elements.  Scales that span a 256-element group combine over the
// group's 8 lanes with xor shuffles (groups never straddle a row, since
// K % 256 == 0, so the 8 lanes are active together).
__device__ __forceinline__ void load32(const uint4 *__restrict__ W, int64_t t, float x[32])
{
    const uint4 *p = W + 4 * t;
    uint4 v[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
        v[i] = p[i];
#pragma unroll
    for (int i = 0; i < 4; i++)
        load8(v[i], x + 8 * i);
}

// ---------------------------------------------------------------------------
// Q8_0: d = F16(max|x| / 127), q = clamp(RHA(x / d), -127, 127)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void isq_q8_0_kernel(const uint4 *__restrict__ W, int64_t tasks,
                                                       uint4 *__restrict__ codes,
                                                       uint16_t *__restrict__ scales)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < tasks; t += stride) {
        float x[32];
        load32(W, t, x);
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; i++)
            a = fmaxf(a, fabsf(x[i]));
        float df;
        const uint32_t d16 = scale_f16(a / 127.0f, &df);
        const float rd = df > 0.0f ? 1.0f / df : 0.0f;  // d = 0: every code is 0
        uint32_t w[8];
#pragma unroll
        for (int k = 0; k < 8; k++) {
            w[k] = 0;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int q = (int)__builtin_amdgcn_fmed3f(rha_quot(x[4 * k + i], df, rd), -127.0f, 127.0f);
                w[k] |= ((uint32_t)q & 0xffu) << (8 * i);
            }
        }
        codes[2 * t] = make_uint4(w[0], w[1], w[2], w[3]);
        codes[2 * t + 1] = make_uint4(w[4], w[5], w[6], w[7]);
        scales[t] = (uint16_t)d16;
    }
}

// ---------------------------------------------------------------------------
// Q4K: plain min/max affine rule per sub-block of 32; 8 lanes per group
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void isq_q4k_kernel(const uint4 *__restrict__ W, int64_t tasks,
                                                      uint4 *__restrict__ codes,
                                                      uint4 *__restrict__ headers)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < tasks; t += stride) {
        float x[32];
        load32(W, t, x);
        float lo = 0.0f, hi = x[0];
#pragma unroll
        for (int i = 0; i < 32; i++) {
            lo = fminf(lo, x[i]);
            hi = fmaxf(hi, x[i]);
        }
        const float s = (hi - lo) / 15.0f;
        const float m = 0.0f - lo;
        float smax = s, mmax = m;
#pragma unroll
        for (int k = 1; k <= 4; k <<= 1) {
            smax = fmaxf(smax, __shfl_xor(smax, k));
            mmax = fmaxf(mmax, __shfl_xor(mmax, k));
        }
        float df, dmf;
        const uint32_t d16 = scale_f16(smax / 63.0f, &df);
        const uint32_t dm16 = scale_f16(mmax / 63.0f, &dmf);
        const int sc = df > 0.0f ? code_of(s / df, 0.0f, 63.0f) : 0;
        const int mq = dmf > 0.0f ? code_of(m / dmf, 0.0f, 63.0f) : 0;
        const float S = df * (float)sc;
        const float M = dmf * (float)mq;
        const float rS = S > 0.0f ? 1.0f / S : 0.0f;  // S = 0: every code is 0
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            int q[8];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const float u = x[8 * k + i] + M;
                q[i] = (int)__builtin_amdgcn_fmed3f(rha_quot_nonneg(u, S, rS), 0.0f, 15.0f);
            }
            w[k] = pack_nibbles(q);
        }
        codes[t] = make_uint4(w[0], w[1], w[2], w[3]);

        const int j = (int)(t & 7);  // sub-block of the group
        uint32_t h0 = ((uint32_t)sc & 15u) << (4 * j);
        uint32_t h1 = ((uint32_t)mq & 15u) << (4 * j);
        uint32_t h2 = (((uint32_t)sc >> 4) << (2 * j)) | (((uint32_t)mq >> 4) << (16 + 2 * j));
#pragma unroll
        for (int k = 1; k <= 4; k <<= 1) {
            h0 |= __shfl_xor(h0, k);
            h1 |= __shfl_xor(h1, k);
            h2 |= __shfl_xor(h2, k);
        }
        if (j == 0)
            headers[t >> 3] = make_uint4(d16 | (dm16 << 16), h0, h1, h2);
    }
}

// ---------------------------------------------------------------------------
// Q6K: symmetric 6-bit codes, 16 sub-blocks of 16, int8 sub-scales, fp16 d;
// lane c of a group's 8 takes chunk c (elements 32c..32c+31: two sub-blocks)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void isq_q6k_kernel(const uint4 *__restrict__ W, int64_t tasks,
                                                      uint8_t *__restrict__ C,
                                                      int8_t *__restrict__ SC,
                                                      uint16_t *__restrict__ D, uint8_t *__restrict__ pad,
                                                      int npad)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    // the tail padding of the buffer (to a multiple of 16 bytes) is zero
    if (blockIdx.x == 0 && (int)threadIdx.x < npad)
        pad[threadIdx.x] = 0;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < tasks; t += stride) {
        float x[32];
        load32(W, t, x);
        float a[2] = {0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 32; i++)
            a[i >> 4] = fmaxf(a[i >> 4], fabsf(x[i]));
        const float s[2] = {a[0] / 31.0f, a[1] / 31.0f};
        float smax = fmaxf(s[0], s[1]);
#pragma unroll
        for (int k = 1; k <= 4; k <<= 1)
            smax = fmaxf(smax, __shfl_xor(smax, k));
        float df;
        const uint32_t d16 = scale_f16(smax / 127.0f, &df);
        int sc[2];
        float S[2], rS[2];
#pragma unroll
        for (int h = 0; h < 2; h++) {
            sc[h] = df > 0.0f ? code_of(s[h] / df, 0.0f, 127.0f) : 0;
            S[h] = df * (float)sc[h];
            rS[h] = S[h] > 0.0f ? 1.0f / S[h] : 0.0f;  // S = 0: every code is 0
        }
        uint32_t lw[4], hw[2] = {0u, 0u};
#pragma unroll
        for (int w = 0; w < 4; w++) {  // octet w of the chunk
            int u[8], lo4[8];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                u[i] = (int)__builtin_amdgcn_fmed3f(rha_quot(x[8 * w + i], S[w >> 1], rS[w >> 1]), -32.0f, 31.0f) + 32;
                lo4[i] = u[i] & 15;
            }
            lw[w] = pack_nibbles(lo4);
            const int o = w & 1;
#pragma unroll
            for (int p = 0; p < 4; p++) {
                hw[w >> 1] |= (uint32_t)(u[2 * p] >> 4) << (8 * o + 2 * p);
                hw[w >> 1] |= (uint32_t)(u[2 * p + 1] >> 4) << (16 + 8 * o + 2 * p);
            }
        }
        const int64_t g = t >> 3;
        const int c = (int)(t & 7);
        uint8_t *Cg = C + 192 * g;
        *reinterpret_cast<uint4 *>(Cg + 16 * c) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
        *reinterpret_cast<uint2 *>(Cg + 128 + 8 * c) = make_uint2(hw[0], hw[1]);
        *reinterpret_cast<uint16_t *>(SC + 16 * g + 2 * c) = (uint16_t)(((uint32_t)sc[0] & 0xffu) | ((uint32_t)sc[1] & 0xffu) << 8);
        if (c == 0)
            D[g] = (uint16_t)d16;
    }
}

// ---------------------------------------------------------------------------
// Exact dequantization to fp32 (test aid): one lane per 8 elements
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dequant_kernel(int fmt, const uint8_t *__restrict__ B, int64_t tasks, Planes p,
                                                      float4 *__restrict__ out)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < tasks; t += stride) {
        float v[8];
        dequant8_any(fmt, B, p, t, v);
        out[2 * t] = make_float4(v[0], v[1], v[2], v[3]);
        out[2 * t + 1] = make_float4(v[4], v[5], v[6], v[7]);
    }
}

// ---------------------------------------------------------------------------
// Quantized embedding lookup: row ids[i] of the [N][K] table, dequantized
// exactly, becomes row i of the output.  Workgroup (x, y) writes 2048
// elements of output row x; ids outside [0, N) give a row of zeros.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void embed_kernel(int fmt, const uint8_t *__restrict__ B, Planes p,
                                                    const int32_t *__restrict__ ids, int64_t N, int64_t K,
                                                    float4 *__restrict__ out)
{
    const int64_t row = blockIdx.x;
    const int64_t k8 = (int64_t)blockIdx.y * 256 + threadIdx.x;  // task in the row
    if (k8 >= K / 8)
        return;
    const int32_t id = ids[row];
    float v[8];
    if (id >= 0 && id < N) {
        dequant8_any(fmt, B, p, (int64_t)id * (K / 8) + k8, v);
    } else {
#pragma unroll
        for (int i = 0; i < 8; i++)
            v[i] = 0.0f;
    }
    float4 *o = out + 2 * (row * (K / 8) + k8);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// ---------------------------------------------------------------------------
// Further formats (Q5K, Q3K, Q2K; Q4_0, Q4_1, Q5_0, Q5_1): same lane split,
// one lane per 8 elements; a K-quant group is 32 lanes (a sub-block 4 lanes
// for Q5K, 2 for Q3K and Q2K), a legacy block 4 lanes.  Steps follow the
// reference definitions one binary32 operation at a time:
//   affine K-quants: lo = min(0, min x), hi = max x per sub-block,
//     s = (hi - lo) / (2^b - 1), m = 0 - lo; d = F16(max s / (2^sb - 1)),
//     dmin = F16(max m / (2^sb - 1)); sc, mq = clamp(RHA(s / d)), ...;
//     codes clamp(RHA((x + dmin mq) / (d sc)), 0, 2^b - 1)
//   Q3K: s = max|x| / 3, d = F16(max s / 63), codes clamp(RHA(x / (d sc)), -4, 3)
//   Q4_0 / Q5_0: d = F16(max|x| / 7 or 15), codes clamp(RHA(x / d))
//   Q4_1 / Q5_1: d = F16((max - min) / 15 or 31), m = F16(min) (signed,
//     clamped to 65504), codes clamp(RHA((x - m) / d), 0, 2^b - 1)
// Block 0 also zeroes the padding between planes and at the end (< 16 bytes each).
// ---------------------------------------------------------------------------
struct Gaps {
    int64_t off[3];
    int len[3];
};

template <int FMT>
__global__ __launch_bounds__(256) void isq_more_kernel(const uint4 *__restrict__ W, int64_t tasks,
                                                       uint8_t *__restrict__ out, Planes p, Gaps gaps)
{
    if (blockIdx.x == 0 && threadIdx.x < 48) {
        const int r = threadIdx.x / 16, i = threadIdx.x % 16;
        if (i < gaps.len[r])
            out[gaps.off[r] + i] = 0;
    }
    constexpr bool KQ = FMT == FMT_Q5K || FMT == FMT_Q3K || FMT == FMT_Q2K;
    constexpr bool AFF = FMT == FMT_Q5K || FMT == FMT_Q2K || FMT == FMT_Q4_1 || FMT == FMT_Q5_1;
    constexpr int BITS = FMT == FMT_Q5K || FMT == FMT_Q5_0 || FMT == FMT_Q5_1 ? 5
                         : FMT == FMT_Q3K                                     ? 3
                         : FMT == FMT_Q2K                                     ? 2
                                                                              : 4;
    constexpr int SBITS = FMT == FMT_Q2K ? 4 : 6;
    constexpr int QLO = AFF ? 0 : -(1 << (BITS - 1));
    constexpr int QHI = AFF ? (1 << BITS) - 1 : (1 << (BITS - 1)) - 1;
    const float qden = AFF ? (float)((1 << BITS) - 1) : (float)((1 << (BITS - 1)) - 1);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < tasks; t += stride) {
        float x[8];
        load8(W[t], x);
        // statistics of the lane's 8 elements, then of its sub-block / block
        float lo = AFF && KQ ? 0.0f : x[0], hi = x[0], a = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            lo = fminf(lo, x[i]);
            hi = fmaxf(hi, x[i]);
            a = fmaxf(a, fabsf(x[i]));
        }
        constexpr int SUBL = FMT == FMT_Q5K || !KQ ? 4 : 2;  // lanes per sub-block / block
#pragma unroll
        for (int k = 1; k < SUBL; k <<= 1) {
            lo = fminf(lo, __shfl_xor(lo, k));
            hi = fmaxf(hi, __shfl_xor(hi, k));
            a = fmaxf(a, __shfl_xor(a, k));
        }
        float S, M, rS;   // code step, subtracted min, 1 / step
        uint32_t d16 = 0, m16 = 0, sc = 0, mq = 0;
        if constexpr (KQ) {
            const float sden = (float)((1 << SBITS) - 1);
            const float s = AFF ? (hi - lo) / qden : a / qden;
            const float m = AFF ? 0.0f - lo : 0.0f;
            float smax = s, mmax = m;
#pragma unroll
            for (int k = SUBL; k < 32; k <<= 1) {
                smax = fmaxf(smax, __shfl_xor(smax, k));
                mmax = fmaxf(mmax, __shfl_xor(mmax, k));
            }
            float df, dmf = 0.0f;
            d16 = scale_f16(smax / sden, &df);
            if (AFF)
                m16 = scale_f16(mmax / sden, &dmf);
            sc = df > 0.0f ? (uint32_t)code_of(s / df, 0.0f, sden) : 0u;
            mq = AFF && dmf > 0.0f ? (uint32_t)code_of(m / dmf, 0.0f, sden) : 0u;
            S = df * (float)sc;
            M = dmf * (float)mq;
        } else if constexpr (AFF) {
            float df;
            d16 = scale_f16((hi - lo) / qden, &df);
            const _Float16 mh = (_Float16)fmaxf(-65504.0f, fminf(lo, 65504.0f));
            m16 = (uint32_t)__builtin_bit_cast(uint16_t, mh);
            S = df;
            M = -(float)mh;  // codes of (x - m) / d
        } else {
            float df;
            d16 = scale_f16(a / qden, &df);
            S = df;
            M = 0.0f;
        }
        rS = S > 0.0f ? 1.0f / S : 0.0f;
        int q[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const float u = AFF ? (KQ ? x[i] + M : x[i] - (-M)) : x[i];
            q[i] = S > 0.0f ? (int)__builtin_amdgcn_fmed3f(rha_quot(u, S, rS), (float)QLO, (float)QHI) : 0;
        }
        // stores
        const int tl = (int)(t & 31);
        const int64_t g = t >> 5;
        if constexpr (FMT == FMT_Q5K) {
            uint32_t lw = 0, hb = 0;
#pragma unroll
            for (int k = 0; k < 8; k++) {
                lw |= (uint32_t)(q[k] & 15) << (4 * k);
                hb |= (uint32_t)(q[k] >> 4) << k;
            }
            reinterpret_cast<uint32_t *>(out)[t] = lw;
            out[p.hi + 32 * g + tl] = (uint8_t)hb;
            const int j = tl >> 2;
            const bool own = (tl & 3) == 0;
            uint32_t w1 = own ? (sc & 15u) << (4 * j) : 0u, w2 = own ? (mq & 15u) << (4 * j) : 0u;
            uint32_t w3 = own ? (sc >> 4) << (2 * j) | (mq >> 4) << (16 + 2 * j) : 0u;
#pragma unroll
            for (int k = 1; k < 32; k <<= 1) {
                w1 |= (uint32_t)__shfl_xor((int)w1, k);
                w2 |= (uint32_t)__shfl_xor((int)w2, k);
                w3 |= (uint32_t)__shfl_xor((int)w3, k);
            }
            if (tl == 0)
                reinterpret_cast<uint4 *>(out + p.scales)[g] = make_uint4(d16 | m16 << 16, w1, w2, w3);
        } else if constexpr (FMT == FMT_Q3K) {
            uint32_t lw = 0, hb = 0;
#pragma unroll
            for (int k = 0; k < 8; k++) {
                const uint32_t u = (uint32_t)(q[k] + 4);
                lw |= (u & 3u) << (2 * k);
                hb |= (u >> 2) << k;
            }
            reinterpret_cast<uint16_t *>(out)[t] = (uint16_t)lw;
            out[p.hi + 32 * g + tl] = (uint8_t)hb;
            const int j = tl >> 1;
            const bool own = (tl & 1) == 0;
            uint32_t s0 = own && j < 8 ? (sc & 15u) << (4 * j) : 0u;
            uint32_t s1 = own && j >= 8 ? (sc & 15u) << (4 * (j - 8)) : 0u;
            uint32_t s2 = own ? (sc >> 4) << (2 * j) : 0u;
#pragma unroll
            for (int k = 1; k < 32; k <<= 1) {
                s0 |= (uint32_t)__shfl_xor((int)s0, k);
                s1 |= (uint32_t)__shfl_xor((int)s1, k);
                s2 |= (uint32_t)__shfl_xor((int)s2, k);
            }
            if (tl == 0) {
                uint32_t *o3 = reinterpret_cast<uint32_t *>(out + p.scales + 12 * g);
                o3[0] = s0;
                o3[1] = s1;
                o3[2] = s2;
                reinterpret_cast<uint16_t *>(out + p.d)[g] = (uint16_t)d16;
            }
        } else if constexpr (FMT == FMT_Q2K) {
            uint32_t lw = 0;
#pragma unroll
            for (int k = 0; k < 8; k++)
                lw |= (uint32_t)q[k] << (2 * k);
            reinterpret_cast<uint16_t *>(out)[t] = (uint16_t)lw;
            if ((tl & 1) == 0)
                out[p.scales + 16 * g + (tl >> 1)] = (uint8_t)(sc | mq << 4);
            if (tl == 0)
                reinterpret_cast<uint32_t *>(out + p.d)[g] = d16 | m16 << 16;
        } else {
            constexpr int bias = FMT == FMT_Q4_0 ? 8 : (FMT == FMT_Q5_0 ? 16 : 0);
            uint32_t lw = 0, hb = 0;
#pragma unroll
            for (int k = 0; k < 8; k++) {
                const uint32_t u = (uint32_t)(q[k] + bias);
                lw |= (u & 15u) << (4 * k);
                hb |= (u >> 4) << k;
            }
            reinterpret_cast<uint32_t *>(out)[t] = lw;
            if constexpr (FMT == FMT_Q5_0 || FMT == FMT_Q5_1)
                out[p.hi + t] = (uint8_t)hb;
            if ((t & 3) == 0) {
                reinterpret_cast<uint16_t *>(out + p.d)[t >> 2] = (uint16_t)d16;
                if constexpr (AFF)
                    reinterpret_cast<uint16_t *>(out + p.m)[t >> 2] = (uint16_t)m16;
            }
        }
    }
}

// padding bytes of a further format's buffer: after each plane up to the next
// plane start, and up to the end
Gaps gaps_of(int fmt, int64_t N, int64_t K, const Planes &p)
{
    const int64_t E = N * K, G = E / 256, B = E / 32;
    Gaps z{{0, 0, 0}, {0, 0, 0}};
    int n = 0;
    auto gap = [&](int64_t from, int64_t to) {
        if (to > from && n < 3) {
            z.off[n] = from;
            z.len[n] = (int)(to - from);
            n++;
        }
    };
    switch (fmt) {
    case FMT_Q3K: gap(108 * G, p.d); gap(p.d + 2 * G, p.total); break;
    case FMT_Q2K: gap(84 * G, p.total); break;
    case FMT_Q4_0: gap(18 * B, p.total); break;
    case FMT_Q4_1: gap(18 * B, p.m); gap(p.m + 2 * B, p.total); break;
    case FMT_Q5_0: gap(20 * B, p.d); gap(p.d + 2 * B, p.total); break;
    case FMT_Q5_1: gap(20 * B, p.d); gap(p.d + 2 * B, p.m); gap(p.m + 2 * B, p.total); break;
    default: break;
    }
    return z;
}

// ---------------------------------------------------------------------------
// FP8 E4M3 with a scale per row (page "Quantization types", section "FP8"):
// one wave per row; s = max|x| / 448, codes E4M3(x / s) -- the binary32
// quotient rounded to the nearest even E4M3 value, saturated to +-448 (the
// variant without infinities).  Also the dynamic per-token quantizer of the
// activations on the W8A8 path.
// ---------------------------------------------------------------------------
// E4M3 code of v, rounded to nearest even, saturated to +-448: with e the
// binade of |v| (at least -6, the subnormal grid) and u = |v| 2^(3 - e) in
// [0, 16), r = rint(u) and the code is 8 (e + 7) + r - 8 -- one formula for
// subnormals (e = -6, u < 8), normals and the carry r = 16 into the next
// binade; codes above 0x7E saturate (the variant without infinities).  near
// is set where u lies within 2^-19 u of a rounding midpoint, which flags
// every value within three ulps of a change of code.
__device__ __forceinline__ uint32_t e4m3_rne(float v, bool &near)
{
    const uint32_t sgn = (__float_as_uint(v) >> 24) & 0x80u;
    const float a = fabsf(v);
    const int e = max((int)(__float_as_uint(a) >> 23) - 127, -6);
    const float u = __builtin_ldexpf(a, 3 - e);
    const float r = rintf(u);
    near |= fabsf(u - r) >= fmaf(-0x1p-19f, u, 0.5f);
    return sgn | (uint32_t)min(8 * (e + 7) + (int)r - 8, 0x7E);
}

// Codes of 16-byte pieces (8 elements) of a row: the E4M3 code of each
// product t = x * rs; bit j of *redo is set where one of them is near a tie
// (or where fast is false).
__device__ __forceinline__ uint2 fp8_piece(uint4 v, float rs, bool fast, uint32_t &redo, int j)
{
    float x[8];
    load8(v, x);
    uint32_t lo = 0, hi = 0;
    bool near = !fast;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        lo |= e4m3_rne(x[k] * rs, near) << (8 * k);
        hi |= e4m3_rne(x[k + 4] * rs, near) << (8 * k);
    }
    redo |= (near ? 1u : 0u) << j;
    return make_uint2(lo, hi);
}

// the same piece from the binary32 quotients x / sc
__device__ __forceinline__ uint2 fp8_piece_exact(uint4 v, float sc)
{
    float x[8];
    load8(v, x);
    uint32_t lo = 0, hi = 0;
    bool unused = false;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        lo |= e4m3_rne(x[k] / sc, unused) << (8 * k);
        hi |= e4m3_rne(x[k + 4] / sc, unused) << (8 * k);
    }
    return make_uint2(lo, hi);
}

// max of the bf16 magnitudes of a piece into two 15-bit lanes of mx
__device__ __forceinline__ void absmax_piece(uint4 v, uint32_t &mx)
{
    const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint32_t m = q[k] & 0x7fff7fffu;
        mx = max(mx & 0xffffu, m & 0xffffu) | (max(mx >> 16, m >> 16) << 16);
    }
}

// One workgroup per row of up to 2048 CPT elements: thread t holds pieces
// t + 256 j (j < CPT) in registers; max|x| over the row (exact, on the bf16
// magnitude bits) by shuffles and LDS, then the codes.  A code is the
// E4M3 rounding of the binary32 quotient q = x / sc; the kernel rounds
// t = x * (1 / sc) instead, which differs from q by at most 1.5 * 2^-23 |q|
// and so rounds the same way unless t is near a rounding midpoint: the
// 16-byte pieces holding such a t (rare) are recomputed from q afterwards.
template <int CPT>
__global__ __launch_bounds__(256) void isq_fp8_row_kernel(const uint4 *__restrict__ W, int K, uint8_t *__restrict__ out,
                                                          int64_t scales_off, int64_t pad, int npad)
{
    __shared__ uint32_t red[4];
    const int tid = threadIdx.x, lane = tid & 63;
    if (blockIdx.x == 0 && tid < npad)
        out[pad + tid] = 0;
    const int64_t row = blockIdx.x;
    const int T = K / 8;
    const uint4 *w = W + row * T;
    uint4 v[CPT];
    uint32_t mx = 0;
#pragma unroll
    for (int j = 0; j < CPT; j++) {
        const int i = tid + 256 * j;
        v[j] = i < T ? w[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < CPT; j++)
        absmax_piece(v[j], mx);
    uint32_t m16 = max(mx & 0xffffu, mx >> 16);
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1)
        m16 = max(m16, (uint32_t)__shfl_xor((int)m16, k));
    if (lane == 0)
        red[tid >> 6] = m16;
    __syncthreads();
    m16 = max(max(red[0], red[1]), max(red[2], red[3]));
    const float sc = __uint_as_float(m16 << 16) / 448.0f;
    if (tid == 0)
        reinterpret_cast<float *>(out + scales_off)[row] = sc;
    uint2 *o = reinterpret_cast<uint2 *>(out + row * K);
    if (!(sc > 0.0f)) {  // a zero row: zero codes
#pragma unroll
        for (int j = 0; j < CPT; j++)
            if (tid + 256 * j < T)
                o[tid + 256 * j] = make_uint2(0, 0);
        return;
    }
    // 1 / sc is finite and the bound above holds where sc is normal;
    // otherwise every piece takes the quotient
    const bool fast = sc >= 0x1p-120f;
    const float rs = 1.0f / sc;
    uint32_t redo = 0;
#pragma unroll
    for (int j = 0; j < CPT; j++) {
        const uint2 c = fp8_piece(v[j], rs, fast, redo, j);
        if (tid + 256 * j < T)
            o[tid + 256 * j] = c;
    }
    // the rare pieces, from the quotients (same thread, same address: the
    // later store wins)
    while (redo) {
        const int j = __builtin_ctz(redo);
        redo &= redo - 1;
        const int i = tid + 256 * j;
        if (i < T)
            o[i] = fp8_piece_exact(w[i], sc);
    }
}

// Rows longer than 16384 elements: one wave per row, max|x| over segments
// of 4096 elements (eight 16-byte loads per lane in flight), then the codes
// segment by segment, re-read.
__global__ __launch_bounds__(256) void isq_fp8_kernel(const uint4 *__restrict__ W, int64_t N, int K,
                                                      uint8_t *__restrict__ out, int64_t scales_off, int64_t pad,
                                                      int npad)
{
    if (blockIdx.x == 0 && (int)threadIdx.x < npad)
        out[pad + threadIdx.x] = 0;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= N)
        return;  // the whole wave
    constexpr int S = 8;  // 16-byte loads per lane and segment
    const int T = K / 8;
    const uint4 *w = W + row * T;
    uint4 v[S];
    uint32_t mx = 0;  // two 15-bit magnitudes
    for (int s0 = 0; s0 < T; s0 += 64 * S) {
#pragma unroll
        for (int j = 0; j < S; j++) {
            const int i = s0 + lane + 64 * j;
            v[j] = i < T ? w[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < S; j++)
            absmax_piece(v[j], mx);
    }
    uint32_t m16 = max(mx & 0xffffu, mx >> 16);
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1)
        m16 = max(m16, (uint32_t)__shfl_xor((int)m16, k));
    const float sc = __uint_as_float(m16 << 16) / 448.0f;
    if (lane == 0)
        reinterpret_cast<float *>(out + scales_off)[row] = sc;
    if (!(sc > 0.0f)) {  // a zero row: zero codes
        for (int i = lane; i < T; i += 64)
            reinterpret_cast<uint2 *>(out + row * K)[i] = make_uint2(0, 0);
        return;
    }
    // 1 / sc is finite and the bound above holds where sc is normal;
    // otherwise every piece takes the quotient
    const bool fast = sc >= 0x1p-120f;
    const float rs = 1.0f / sc;
    uint2 *o = reinterpret_cast<uint2 *>(out + row * K);
    for (int s0 = 0; s0 < T; s0 += 64 * S) {
#pragma unroll
        for (int j = 0; j < S; j++) {
            const int i = s0 + lane + 64 * j;
            v[j] = i < T ? w[i] : make_uint4(0, 0, 0, 0);
        }
        uint32_t redo = 0;
#pragma unroll
        for (int j = 0; j < S; j++) {
            const int i = s0 + lane + 64 * j;
            const uint2 c = fp8_piece(v[j], rs, fast, redo, j);
            if (i < T)
                o[i] = c;
        }
        // the rare pieces, from the quotients (same lane, same address: the
        // later store wins)
        while (redo) {
            const int j = __builtin_ctz(redo);
            redo &= redo - 1;
            const int i = s0 + lane + 64 * j;
            if (i < T)
                o[i] = fp8_piece_exact(w[i], sc);
        }
    }
}

inline unsigned grid_for(int64_t tasks)
{
    int64_t b = (tasks + 255) / 256;
    const int64_t cap = int64_t(1) << 22;
    return (unsigned)(b < 1 ? 1 : (b > cap ? cap : b));
}

}  // namespace

hipError_t launch_isq(int fmt, const uint16_t *W, int64_t N, int64_t K, uint8_t *out, hipStream_t s)
{
    const int64_t tasks = N * K / 8;
    const Planes p = planes_of(fmt, N, K);
    const uint4 *w = reinterpret_cast<const uint4 *>(W);
    const int64_t blocks32 = N * K / 32;  // lanes of the Q8_0 / Q4K / Q6K quantizers
    if (fmt == FMT_Q8_0)
        hipLaunchKernelGGL(isq_q8_0_kernel, dim3(grid_for(blocks32)), dim3(256), 0, s, w, blocks32,
                           reinterpret_cast<uint4 *>(out),
                           reinterpret_cast<uint16_t *>(out + p.scales));
    else if (fmt == FMT_Q4K)
        hipLaunchKernelGGL(isq_q4k_kernel, dim3(grid_for(blocks32)), dim3(256), 0, s, w, blocks32,
                           reinterpret_cast<uint4 *>(out),
                           reinterpret_cast<uint4 *>(out + p.scales));
    else if (fmt == FMT_Q6K)
        hipLaunchKernelGGL(isq_q6k_kernel, dim3(grid_for(blocks32)), dim3(256), 0, s, w, blocks32, out,
                           reinterpret_cast<int8_t *>(out + p.scales),
                           reinterpret_cast<uint16_t *>(out + p.d), out + 210 * (N * K / 256),
                           (int)(p.total - 210 * (N * K / 256)));
    else if (fmt == FMT_FP8) {
        const int64_t pad = p.scales + 4 * N;
        const int npad = (int)(p.total - pad);
        switch ((K + 2047) / 2048) {
#define C(CPT)                                                                                                      \
    case CPT:                                                                                                       \
        hipLaunchKernelGGL(isq_fp8_row_kernel<CPT>, dim3((unsigned)N), dim3(256), 0, s, w, (int)K, out, p.scales, pad, \
                           npad);                                                                                   \
        break;
            C(1) C(2) C(3) C(4) C(5) C(6) C(7) C(8)
#undef C
        default:
            hipLaunchKernelGGL(isq_fp8_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s, w, N, (int)K, out,
                               p.scales, pad, npad);
        }
    } else {
        const Gaps z = gaps_of(fmt, N, K, p);
        const dim3 grid(grid_for(tasks)), block(256);
        switch (fmt) {
        case FMT_Q5K: hipLaunchKernelGGL(isq_more_kernel<FMT_Q5K>, grid, block, 0, s, w, tasks, out, p, z); break;
        case FMT_Q3K: hipLaunchKernelGGL(isq_more_kernel<FMT_Q3K>, grid, block, 0, s, w, tasks, out, p, z); break;
        case FMT_Q2K: hipLaunchKernelGGL(isq_more_kernel<FMT_Q2K>, grid, block, 0, s, w, tasks, out, p, z); break;
        case FMT_Q4_0: hipLaunchKernelGGL(isq_more_kernel<FMT_Q4_0>, grid, block, 0, s, w, tasks, out, p, z); break;
        case FMT_Q4_1: hipLaunchKernelGGL(isq_more_kernel<FMT_Q4_1>, grid, block, 0, s, w, tasks, out, p, z); break;
        case FMT_Q5_0: hipLaunchKernelGGL(isq_more_kernel<FMT_Q5_0>, grid, block, 0, s, w, tasks, out, p, z); break;
        case FMT_Q5_1: hipLaunchKernelGGL(isq_more_kernel<FMT_Q5_1>, grid, block, 0, s, w, tasks, out, p, z); break;
        default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

hipError_t launch_embed(int fmt, const uint8_t *blocks, int64_t N, int64_t K, const int32_t *ids, int64_t n_ids,
                        float *out, hipStream_t s)
{
    const Planes p = planes_of(fmt, N, K);
    const dim3 grid((unsigned)n_ids, (unsigned)((K / 8 + 255) / 256));
    hipLaunchKernelGGL(embed_kernel, grid, dim3(256), 0, s, fmt, blocks, p, ids, N, K,
                       reinterpret_cast<float4 *>(out));
    return hipGetLastError();
}

hipError_t launch_dequant(int fmt, const uint8_t *blocks, int64_t N, int64_t K, float *W, hipStream_t s)
{
    const int64_t tasks = N * K / 8;
    const Planes p = planes_of(fmt, N, K);
    hipLaunchKernelGGL(dequant_kernel, dim3(grid_for(tasks)), dim3(256), 0, s, fmt, blocks, tasks, p,
                       reinterpret_cast<float4 *>(W));
    return hipGetLastError();
}

}  // namespace ql
