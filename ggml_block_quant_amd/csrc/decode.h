// decode.h -- exact decode of 8 consecutive elements of a block buffer, for
// every implemented format; shared by the dequantizer, the embedding lookup
// and the generic GEMV / GEMM of the formats without a tuned kernel.
//
// Element t*8 .. t*8+7 of the flattened [N][K] tensor (t is a "task"; K is a
// multiple of 256, so a task never crosses a row, a block or a sub-block).
// Values are exact in fp32 except where one rounding is unavoidable: Q4K,
// Q5K, Q2K (d sc q - dmin m) and Q4_1, Q5_1 (d q + m) are computed with one
// fused multiply-add, i.e. rounded once from the exact value.
#pragma once

#include "qlinear_internal.h"

namespace ql {

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xffffu));
}

// Q4K / Q6K nibble order: within a dword, element 2p at nibble p (p < 4) and
// element 2p+1 at nibble p + 4
__device__ __forceinline__ void unpack_nibbles_eo(uint32_t d, int q[8])
{
#pragma unroll
    for (int p = 0; p < 4; p++) {
        q[2 * p] = (d >> (4 * p)) & 15;
        q[2 * p + 1] = (d >> (16 + 4 * p)) & 15;
    }
}

// E4M3 (no infinities, bias 7) code -> value, exact in fp32
__device__ __forceinline__ float e4m3_value(uint32_t b)
{
    const int e = (int)((b >> 3) & 15u), m = (int)(b & 7u);
    const float v = e ? __builtin_ldexpf(1.0f + (float)m * 0.125f, e - 7) : (float)m * 0x1p-9f;
    return (b & 0x80u) ? -v : v;
}

template <int FMT>
__device__ __forceinline__ void dequant8(const uint8_t *__restrict__ B, const Planes &p, int64_t t, float v[8])
{
    if constexpr (FMT == FMT_Q8_0) {
        const uint2 c = reinterpret_cast<const uint2 *>(B)[t];
        const float d = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(B + p.scales)[t >> 2]);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            v[i] = d * (float)(int8_t)(c.x >> (8 * i));
            v[i + 4] = d * (float)(int8_t)(c.y >> (8 * i));
        }
    } else if constexpr (FMT == FMT_Q4K) {
        const uint32_t c = reinterpret_cast<const uint32_t *>(B)[t];
        const uint4 h = reinterpret_cast<const uint4 *>(B + p.scales)[t >> 5];
        const int j = (int)((t & 31) >> 2);
        const uint32_t sc = ((h.y >> (4 * j)) & 15u) | ((h.w >> (2 * j)) & 3u) << 4;
        const uint32_t mq = ((h.z >> (4 * j)) & 15u) | ((h.w >> (16 + 2 * j)) & 3u) << 4;
        const float S = f16_bits_to_f32(h.x) * (float)sc;
        const float M = f16_bits_to_f32(h.x >> 16) * (float)mq;
        int q[8];
        unpack_nibbles_eo(c, q);
#pragma unroll
        for (int i = 0; i < 8; i++)
            v[i] = fmaf(S, (float)q[i], -M);
    } else if constexpr (FMT == FMT_Q6K) {
        const int64_t g = t >> 5;
        const int l = (int)(t & 31), c = l >> 2, w = l & 3, o = w & 1;
        const uint8_t *Cg = B + 192 * g;
        const uint32_t lo = *reinterpret_cast<const uint32_t *>(Cg + 4 * l);
        const uint32_t hd = *reinterpret_cast<const uint32_t *>(Cg + 128 + 8 * c + 4 * (w >> 1));
        const int sc = reinterpret_cast<const int8_t *>(B + p.scales)[16 * g + (l >> 1)];
        const float S = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(B + p.d)[g]) * (float)sc;
        int q[8];
        unpack_nibbles_eo(lo, q);
#pragma unroll
        for (int k = 0; k < 4; k++) {
            q[2 * k] |= (int)((hd >> (8 * o + 2 * k)) & 3u) << 4;
            q[2 * k + 1] |= (int)((hd >> (16 + 8 * o + 2 * k)) & 3u) << 4;
        }
#pragma unroll
        for (int i = 0; i < 8; i++)
            v[i] = S * (float)(q[i] - 32);
    } else if constexpr (FMT == FMT_Q5K) {
        // natural order: element 8t' + k at nibble k of the dword, its top
        // bit at bit k of byte t' of the high-bit plane
        const int64_t g = t >> 5;
        const int tl = (int)(t & 31), j = tl >> 2;
        const uint32_t lo = reinterpret_cast<const uint32_t *>(B)[t];
        const uint32_t hb = B[p.hi + 32 * g + tl];
        const uint4 h = reinterpret_cast<const uint4 *>(B + p.scales)[g];
        const uint32_t sc = ((h.y >> (4 * j)) & 15u) | ((h.w >> (2 * j)) & 3u) << 4;
        const uint32_t mq = ((h.z >> (4 * j)) & 15u) | ((h.w >> (16 + 2 * j)) & 3u) << 4;
        const float S = f16_bits_to_f32(h.x) * (float)sc;
        const float M = f16_bits_to_f32(h.x >> 16) * (float)mq;
#pragma unroll
        for (int k = 0; k < 8; k++)
            v[k] = fmaf(S, (float)(((lo >> (4 * k)) & 15u) | ((hb >> k) & 1u) << 4), -M);
    } else if constexpr (FMT == FMT_Q3K) {
        const int64_t g = t >> 5;
        const int tl = (int)(t & 31), j = tl >> 1;
        const uint32_t lo = reinterpret_cast<const uint16_t *>(B)[t];
        const uint32_t hb = B[p.hi + 32 * g + tl];
        const uint32_t *s3 = reinterpret_cast<const uint32_t *>(B + p.scales + 12 * g);
        const uint32_t sc = (((j < 8 ? s3[0] : s3[1]) >> (4 * (j & 7))) & 15u) | ((s3[2] >> (2 * j)) & 3u) << 4;
        const float S = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(B + p.d)[g]) * (float)sc;
#pragma unroll
        for (int k = 0; k < 8; k++)
            v[k] = S * (float)((int)(((lo >> (2 * k)) & 3u) | ((hb >> k) & 1u) << 2) - 4);
    } else if constexpr (FMT == FMT_Q2K) {
        const int64_t g = t >> 5;
        const int j = (int)(t & 31) >> 1;
        const uint32_t c = reinterpret_cast<const uint16_t *>(B)[t];
        const uint32_t sm = B[p.scales + 16 * g + j];
        const uint32_t dd = reinterpret_cast<const uint32_t *>(B + p.d)[g];
        const float S = f16_bits_to_f32(dd) * (float)(sm & 15u);
        const float M = f16_bits_to_f32(dd >> 16) * (float)(sm >> 4);
#pragma unroll
        for (int k = 0; k < 8; k++)
            v[k] = fmaf(S, (float)((c >> (2 * k)) & 3u), -M);
    } else if constexpr (FMT == FMT_FP8) {
        // codes of row t*8/K, each times the row's scale (rounded once)
        const uint2 c = reinterpret_cast<const uint2 *>(B)[t];
        const int64_t tpr = p.K / 8;  // tasks per row
        const int64_t row = t < 0x80000000ll ? (int64_t)((uint32_t)t / (uint32_t)tpr) : t / tpr;
        const float sc = reinterpret_cast<const float *>(B + p.scales)[row];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            v[k] = sc * e4m3_value(c.x >> (8 * k));
            v[k + 4] = sc * e4m3_value(c.y >> (8 * k));
        }
    } else {
        // legacy blocks of 32: element 8 (t & 3) + k at nibble k of dword t,
        // the fifth bit (Q5_0, Q5_1) at bit k of byte t of the high-bit plane
        const int64_t b = t >> 2;
        const uint32_t c = reinterpret_cast<const uint32_t *>(B)[t];
        const float d = f16_bits_to_f32(reinterpret_cast<const uint16_t *>(B + p.d)[b]);
        constexpr bool five = FMT == FMT_Q5_0 || FMT == FMT_Q5_1;
        constexpr bool affine = FMT == FMT_Q4_1 || FMT == FMT_Q5_1;
        const uint32_t hb = five ? B[p.hi + t] : 0u;
        const float m = affine ? f16_bits_to_f32(reinterpret_cast<const uint16_t *>(B + p.m)[b]) : 0.0f;
        constexpr int bias = FMT == FMT_Q4_0 ? 8 : (FMT == FMT_Q5_0 ? 16 : 0);
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const int u = (int)(((c >> (4 * k)) & 15u) | ((hb >> k) & 1u) << 4);
            v[k] = affine ? fmaf(d, (float)u, m) : d * (float)(u - bias);
        }
    }
}

// The formats whose weights are a scale times a signed code, w = S * q, with
// one S per 8-element task: Q4_0 (d (u - 8)), Q5_0 (d (u - 16)) and Q3K
// (d sc (u - 4)).  S * q is exact in fp32 (at most 11 + 6 + 5 bits), so a
// dot product can form sum q * x with exact products and scale the task's
// sum once.
template <int FMT>
constexpr bool signed_code_fmt = FMT == FMT_Q4_0 || FMT == FMT_Q5_0 || FMT == FMT_Q3K;

// The codes q of task t as fp32 integers; returns their scale S.  The same
// fields as dequant8, with the bias subtracted in the integer domain: a
// field u of width n and bias 2^(n-1) gives q = u - 2^(n-1), which is u with
// its top bit flipped read as a signed n-bit field.  For the split codes
// (Q5_0, Q3K) the flipped top bit comes from the high-bit plane as 0 or -1
// (a signed 1-bit field of the complemented byte) and is shifted above the
// low bits.
template <int FMT>
__device__ __forceinline__ float codes8(const uint8_t *__restrict__ B, const Planes &p, int64_t t, float q[8])
{
    static_assert(signed_code_fmt<FMT>, "scale-times-signed-code formats only");
    if constexpr (FMT == FMT_Q4_0) {
        const uint32_t c = reinterpret_cast<const uint32_t *>(B)[t] ^ 0x88888888u;
#pragma unroll
        for (int k = 0; k < 8; k++)
            q[k] = (float)(int)__builtin_amdgcn_sbfe((int)c, 4 * k, 4);  // the builtin returns unsigned
        return f16_bits_to_f32(reinterpret_cast<const uint16_t *>(B + p.d)[t >> 2]);
    } else if constexpr (FMT == FMT_Q5_0) {
        const uint32_t c = reinterpret_cast<const uint32_t *>(B)[t];
        const int nh = ~(int)B[p.hi + t];
#pragma unroll
        for (int k = 0; k < 8; k++)
            q[k] = (float)(int)(((uint32_t)__builtin_amdgcn_sbfe(nh, k, 1) << 4) | __builtin_amdgcn_ubfe(c, 4 * k, 4));
        return f16_bits_to_f32(reinterpret_cast<const uint16_t *>(B + p.d)[t >> 2]);
    } else {
        const int64_t g = t >> 5;
        const int tl = (int)(t & 31), j = tl >> 1;
        const uint32_t lo = reinterpret_cast<const uint16_t *>(B)[t];
        const int nh = ~(int)B[p.hi + 32 * g + tl];
        const uint32_t *s3 = reinterpret_cast<const uint32_t *>(B + p.scales + 12 * g);
        const uint32_t sc = (((j < 8 ? s3[0] : s3[1]) >> (4 * (j & 7))) & 15u) | ((s3[2] >> (2 * j)) & 3u) << 4;
#pragma unroll
        for (int k = 0; k < 8; k++)
            q[k] = (float)(int)(((uint32_t)__builtin_amdgcn_sbfe(nh, k, 1) << 2) | __builtin_amdgcn_ubfe(lo, 2 * k, 2));
        return f16_bits_to_f32(reinterpret_cast<const uint16_t *>(B + p.d)[g]) * (float)sc;
    }
}

// runtime dispatch of dequant8 (the dequantizer and the embedding lookup)
__device__ __forceinline__ void dequant8_any(int fmt, const uint8_t *__restrict__ B, const Planes &p, int64_t t,
                                             float v[8])
{
    switch (fmt) {
    case FMT_Q8_0: dequant8<FMT_Q8_0>(B, p, t, v); break;
    case FMT_Q4K: dequant8<FMT_Q4K>(B, p, t, v); break;
    case FMT_Q6K: dequant8<FMT_Q6K>(B, p, t, v); break;
    case FMT_Q5K: dequant8<FMT_Q5K>(B, p, t, v); break;
    case FMT_Q3K: dequant8<FMT_Q3K>(B, p, t, v); break;
    case FMT_Q2K: dequant8<FMT_Q2K>(B, p, t, v); break;
    case FMT_Q4_0: dequant8<FMT_Q4_0>(B, p, t, v); break;
    case FMT_Q4_1: dequant8<FMT_Q4_1>(B, p, t, v); break;
    case FMT_Q5_0: dequant8<FMT_Q5_0>(B, p, t, v); break;
    case FMT_FP8: dequant8<FMT_FP8>(B, p, t, v); break;
    default: dequant8<FMT_Q5_1>(B, p, t, v); break;
    }
}

}  // namespace ql
