// gemv.hip -- fused dequantize-GEMV for small decode batches (M <= 8):
// Y[m][n] = sum_k X[m][k] * deq(W)[n][k] with W in Q8_0, Q4K or Q6K blocks.
//
// Page "Quantization types", section "NVFP4": small decode batches use a
// dedicated matrix-vector kernel, and when the packed weights fill the GPU
// cache the decode tile is weight-first.  Here every weight byte is read
// from HBM exactly once, with coalesced 128-bit loads, and everything else
// (X, partial sums) stays in registers.
//
// Work split.  A row of K elements is cut into K/32 chunks of 32 elements
// (a Q8_0 block, a Q4K sub-block, two Q6K sub-blocks).  A workgroup of KS
// wavefronts covers a whole row: lane `lane` of wave `wv` owns chunks
// c = wv*64 + lane + i*KS*64 (i < CPT), so each load instruction of a wave
// reads 64 consecutive chunks.  The lane keeps X for its chunks in VGPRs for
// the whole kernel and walks down the rows R at a time (all R rows' loads
// are issued before any is consumed).  Partial sums are reduced across the
// wave with a halving butterfly (each step halves the values a lane keeps),
// then across the KS waves through LDS.
//
// Workgroups are persistent: each walks batches b, b+G, b+2G, ... and the
// loads of the next batch are issued before the current one is computed.
// Rows and chunks past the end are clamped (they re-read valid bytes and
// their contribution is dropped or multiplied by a zero X), so the load
// path has no branches.
//
// Arithmetic: every product of a code and an activation is exact and only
// the fp32 sums round, so an output's error is relative to sum |w||x|.
//   * Q4K: the 4-bit codes u are taken as E4M3 bytes -- a byte 0..15 is the
//     E4M3 value u * 2^-9 (subnormal up to 7, the first binade from 8) --
//     and v_cvt_scalef32_pk_bf16_fp8 with scale 2^9 turns two of them into
//     the bf16 pair (u, u') exactly.  The layout's nibble order gives the
//     pairs (0,4), (1,5), (2,6), (3,7) of each group of eight elements, so X
//     is staged in that pairing.  v_dot2_f32_bf16 forms sum u*x; the chunk
//     adds S * sum u*x - Mn * sum x.
//   * Q6K: the codes q = u - 32 (-32 .. 31) are exact in fp16: the bits
//     0x6400 | u are 1024 + u, and one v_pk_add_f16 of -1056 leaves q for
//     two elements.  X is staged in fp16 after scaling each chunk of 32 by a
//     power of two that puts its largest magnitude in [2^14, 2^15), where
//     every bf16 value down to 2^-32 of that maximum is exact; the scale is
//     undone on the chunk's sum.  v_dot2_f32_f16 forms sum q*x.
//   * Q8_0: signed codes converted with v_cvt_f32_i32 on a sign-extended
//     byte (SDWA), fused multiply-adds with X.
// (Adding a bias to the codes instead, sum x*(128+u) - 128 sum x, rounds at
// the scale of the bias and fails the bar on blocks whose codes are mostly
// zero where X is large.)
#include "qlinear_internal.h"
#include "decode.h"

namespace ql {
namespace {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float h2f(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xffffu));
}

__device__ __forceinline__ float lo_bf16(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// ----------------------------------------------------------------------------
// Per-format chunk data (one row, one 32-element chunk) and its dot product
// ----------------------------------------------------------------------------
template <int FMT> struct Chunk;
template <> struct Chunk<FMT_Q4K> { uint4 c; uint4 h; };
template <> struct Chunk<FMT_Q6K> { uint4 lo; uint2 hi; uint32_t sc2; uint32_t d; };
template <> struct Chunk<FMT_Q8_0> { uint4 c0, c1; uint32_t d; };

struct Geo {
    const uint8_t *B;
    int64_t scales_off, d_off;
    int K;
};

template <int FMT>
__device__ __forceinline__ void load_chunk(const Geo &g, int64_t n, int c, Chunk<FMT> &ck);

template <>
__device__ __forceinline__ void load_chunk<FMT_Q4K>(const Geo &g, int64_t n, int c, Chunk<FMT_Q4K> &ck)
{
    const int64_t sub = n * (g.K / 32) + c;  // global sub-block index
    ck.c = *reinterpret_cast<const uint4 *>(g.B + 16 * sub);
    ck.h = *reinterpret_cast<const uint4 *>(g.B + g.scales_off + 16 * (sub >> 3));
}

template <>
__device__ __forceinline__ void load_chunk<FMT_Q6K>(const Geo &g, int64_t n, int c, Chunk<FMT_Q6K> &ck)
{
    const int64_t grp = n * (g.K / 256) + (c >> 3);
    const int cc = c & 7;
    const uint8_t *Cg = g.B + 192 * grp;
    ck.lo = *reinterpret_cast<const uint4 *>(Cg + 16 * cc);
    ck.hi = *reinterpret_cast<const uint2 *>(Cg + 128 + 8 * cc);
    ck.sc2 = *reinterpret_cast<const uint16_t *>(g.B + g.scales_off + 16 * grp + 2 * cc);
    ck.d = *reinterpret_cast<const uint16_t *>(g.B + g.d_off + 2 * grp);
}

template <>
__device__ __forceinline__ void load_chunk<FMT_Q8_0>(const Geo &g, int64_t n, int c, Chunk<FMT_Q8_0> &ck)
{
    const int64_t blk = n * (g.K / 32) + c;
    const uint4 *p = reinterpret_cast<const uint4 *>(g.B + 32 * blk);
    ck.c0 = p[0];
    ck.c1 = p[1];
    ck.d = *reinterpret_cast<const uint16_t *>(g.B + g.scales_off + 2 * blk);
}

// X of one chunk for M rows: 16 pairs per row (Q4K: bf16 in the pairing of
// the codes; Q6K: scaled fp16; Q8_0: bf16), plus Q4K's sum over the chunk
// (sum) or Q6K's scale exponent (e: X was multiplied by 2^e).
template <int M> struct XChunk {
    uint32_t p[M][16];
    float sum[M];
    int e[M];
};

typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2_t;
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2h(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}

// bytes 2H, 2H+1 of w, each 0..15, as the bf16 pair of those integers
template <bool H>
__device__ __forceinline__ uint32_t nib_pair(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 512.0f, H));
}

// the bf16 dwords of eight consecutive activations (elements 0-1, 2-3, 4-5,
// 6-7) -> the pairs (0,4), (1,5), (2,6), (3,7) the Q4K codes come in
__device__ __forceinline__ uint4 octet_pairs(uint4 v)
{
    return make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u), __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                      __builtin_amdgcn_perm(v.w, v.y, 0x05040100u), __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
}

// the exponent e that puts max|x| (> 0) of a chunk in [2^14, 2^15)
__device__ __forceinline__ int chunk_exp(float amax)
{
    return amax > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(amax) : 0;
}

// a bf16 pair scaled by 2^e -> fp16 pair (exact for every value down to
// 2^-32 of the chunk maximum; below, rounded toward zero)
__device__ __forceinline__ uint32_t bf16_pair_to_f16(uint32_t p, int e)
{
    const float a = __builtin_amdgcn_ldexpf(__uint_as_float(p << 16), e);
    const float b = __builtin_amdgcn_ldexpf(__uint_as_float(p & 0xffff0000u), e);
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

__device__ __forceinline__ float bf16_pair_absmax(uint32_t p, float m)
{
    return fmaxf(m, fmaxf(fabsf(__uint_as_float(p << 16)), fabsf(__uint_as_float(p & 0xffff0000u))));
}

// Smallest nonzero magnitude of two bf16 values, as (magnitude bits - 1) in
// 16 bits: a zero wraps to 0xFFFF and never wins; min with m (same form).
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2_t bf16_pair_minnz(uint32_t p, u16x2_t m)
{
    const u16x2_t a = __builtin_bit_cast(u16x2_t, p & 0x7FFF7FFFu) - u16x2_t{1, 1};
    return __builtin_elementwise_min(a, m);
}

// A Q6K chunk's activations are staged in fp16 after scaling the largest
// magnitude into [2^14, 2^15); every nonzero bf16 value of at least 2^-28 of
// that maximum is then exact in fp16 (at least 2^-14, a normal).  A chunk
// holding a smaller nonzero value is flagged: the dot product takes the exact
// fp32 path for it.  Flagged exponents carry +1024.
constexpr int Q6K_EXACT_FLAG = 1024;
__device__ __forceinline__ int chunk_exp_flagged(float amax, uint32_t minnz1)
{
    const int e = chunk_exp(amax);
    const bool tiny = minnz1 != 0xFFFFu && __uint_as_float((minnz1 + 1u) << 16) < __builtin_amdgcn_ldexpf(amax, -28);
    return tiny ? e + Q6K_EXACT_FLAG : e;
}

// Loop-invariant constants held in VGPRs: a VOP3 and-or on gfx950 takes at
// most one SGPR/constant operand, so the masks live in registers and the
// bias in an SGPR, which gives one v_and_or_b32 per bf16 pair.
struct Masks {
    uint32_t nib;     // 0x000F000F
    uint32_t hi2;     // 0x00300030
    uint32_t nibx16;  // 0x00F000F0
    uint32_t hi2x16;  // 0x03000300
};

__device__ __forceinline__ Masks make_masks()
{
    Masks k;
    asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(k.nib));
    asm volatile("v_mov_b32 %0, 0x00300030" : "=v"(k.hi2));
    asm volatile("v_mov_b32 %0, 0x00f000f0" : "=v"(k.nibx16));
    asm volatile("v_mov_b32 %0, 0x03000300" : "=v"(k.hi2x16));
    return k;
}

// (a & m) | b in one instruction; the compiler would otherwise fold
// (x & m1) | (y & m2) | b into two ands and an or3
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t b)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(b));
    return r;
}

template <int M>
__device__ __forceinline__ void q4k_dot(const Chunk<FMT_Q4K> &ck, const XChunk<M> &x, int j, float acc[M])
{
    const uint32_t sc = __builtin_amdgcn_ubfe(ck.h.y, 4 * j, 4) | (__builtin_amdgcn_ubfe(ck.h.w, 2 * j, 2) << 4);
    const uint32_t mq = __builtin_amdgcn_ubfe(ck.h.z, 4 * j, 4) | (__builtin_amdgcn_ubfe(ck.h.w, 16 + 2 * j, 2) << 4);
    const float S = h2f(ck.h.x) * (float)sc;
    const float Mn = h2f(ck.h.x >> 16) * (float)mq;
    const uint32_t w[4] = {ck.c.x, ck.c.y, ck.c.z, ck.c.w};
    uint32_t pr[16];
#pragma unroll
    for (int q = 0; q < 4; q++) {
        // nibble p of dword q is element 2p (p < 4) or 2(p-4)+1 of its octet:
        // the bytes of lo are elements 0, 4, 1, 5, those of hi 2, 6, 3, 7
        const uint32_t lo = w[q] & 0x0F0F0F0Fu, hi = (w[q] >> 4) & 0x0F0F0F0Fu;
        pr[4 * q + 0] = nib_pair<false>(lo);
        pr[4 * q + 1] = nib_pair<true>(lo);
        pr[4 * q + 2] = nib_pair<false>(hi);
        pr[4 * q + 3] = nib_pair<true>(hi);
    }
#pragma unroll
    for (int m = 0; m < M; m++) {
        float d = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; e++)
            d = dot2(pr[e], x.p[m][e], d);
        acc[m] = fmaf(S, d, acc[m]);
        acc[m] = fmaf(-Mn, x.sum[m], acc[m]);
    }
}

// Q6K codes of one chunk: dword q of the low nibbles holds octet q (nibble
// s: element 2s, nibble s + 4: element 2s + 1); the two high bits of the
// pair s of octet q sit at bit 8(q & 1) + 2s (and 16 + that) of high-bit
// dword q / 2.  Pairs s = 0, 2 take the nibble at bits 0-3 of lw (s = 2:
// lw >> 8) and the high bits at 4-5 -- fp16 1024 + u; pairs s = 1, 3 take it
// at bits 4-7 and the high bits at 8-9 -- fp16 1024 + 16 u -- which saves
// a shift of lw per pair.  v_pk_add_f16 then leaves q or 16 q exactly.
template <int M>
__device__ __forceinline__ void q6k_dot(const Chunk<FMT_Q6K> &ck, const XChunk<M> &x, float acc[M],
                                        const Masks &k, const uint16_t *__restrict__ xg, int64_t K)
{
    const float d = h2f(ck.d);
    const float Sa = d * (float)(int8_t)(ck.sc2 & 0xffu);
    const float Sb = d * (float)(int8_t)(ck.sc2 >> 8);
    const uint32_t lw[4] = {ck.lo.x, ck.lo.y, ck.lo.z, ck.lo.w};
    const uint32_t hw[2] = {ck.hi.x, ck.hi.y};
    const f16x2_t off1 = {(_Float16)-1056.0f, (_Float16)-1056.0f};   // 1024 + u   -> q
    const f16x2_t off16 = {(_Float16)-1536.0f, (_Float16)-1536.0f};  // 1024 + 16u -> 16 q
    auto shl = [](uint32_t v, int n) { return n >= 0 ? v << n : v >> -n; };
    uint32_t pr[16];
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const int o = 8 * (q & 1);
        const uint32_t l01 = lw[q], l23 = lw[q] >> 8, H = hw[q >> 1];
        const uint32_t u0 = and_or(shl(H, 4 - o), k.hi2, and_or(l01, k.nib, 0x64006400u));
        const uint32_t u1 = and_or(shl(H, 6 - o), k.hi2x16, and_or(l01, k.nibx16, 0x64006400u));
        const uint32_t u2 = and_or(shl(H, 0 - o), k.hi2, and_or(l23, k.nib, 0x64006400u));
        const uint32_t u3 = and_or(shl(H, 2 - o), k.hi2x16, and_or(l23, k.nibx16, 0x64006400u));
        pr[4 * q + 0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, u0) + off1);
        pr[4 * q + 1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, u1) + off16);
        pr[4 * q + 2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, u2) + off1);
        pr[4 * q + 3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, u3) + off16);
    }
#pragma unroll
    for (int m = 0; m < M; m++) {
        if (x.e[m] >= Q6K_EXACT_FLAG / 2) {
            // exact path: the chunk's bf16 activations from memory (xg: chunk
            // of token 0, rows K apart) times the codes, fp32 products (exact)
            // and sums; pair j of the codes holds elements 2j, 2j+1 (q, or 16 q
            // for odd j % 4), as does dword j of X
            const uint4 *xq = reinterpret_cast<const uint4 *>(xg + (int64_t)m * K);
            float a1 = 0.0f, a16 = 0.0f, b1 = 0.0f, b16 = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const uint4 v = xq[q];
                const uint32_t xd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    const uint32_t pv = pr[4 * q + t];
                    float r = (float)__builtin_bit_cast(_Float16, (uint16_t)(pv & 0xffffu)) * __uint_as_float(xd[t] << 16);
                    r = fmaf((float)__builtin_bit_cast(_Float16, (uint16_t)(pv >> 16)), __uint_as_float(xd[t] & 0xffff0000u), r);
                    if (q < 2)
                        (t & 1 ? a16 : a1) += r;
                    else
                        (t & 1 ? b16 : b1) += r;
                }
            }
            const float da = fmaf(a16, 0.0625f, a1), db = fmaf(b16, 0.0625f, b1);
            acc[m] += fmaf(Sa, da, Sb * db);
            continue;
        }
        // sub-block a (octets 0, 1) and b (octets 2, 3); the pairs holding
        // 16 q in their own sums
        float a1 = 0.0f, a16 = 0.0f, b1 = 0.0f, b16 = 0.0f;
#pragma unroll
        for (int q = 0; q < 2; q++) {
#pragma unroll
            for (int s = 0; s < 4; s += 2) {
                a1 = dot2h(pr[4 * q + s], x.p[m][4 * q + s], a1);
                a16 = dot2h(pr[4 * q + s + 1], x.p[m][4 * q + s + 1], a16);
                b1 = dot2h(pr[8 + 4 * q + s], x.p[m][8 + 4 * q + s], b1);
                b16 = dot2h(pr[8 + 4 * q + s + 1], x.p[m][8 + 4 * q + s + 1], b16);
            }
        }
        const float da = fmaf(a16, 0.0625f, a1), db = fmaf(b16, 0.0625f, b1);
        // X of this chunk was scaled by 2^e
        acc[m] += __builtin_amdgcn_ldexpf(fmaf(Sa, da, Sb * db), -x.e[m]);
    }
}

// Q8_0: signed codes converted with v_cvt_f32_i32 on a sign-extended byte
// (SDWA), X either kept in fp32 (small M) or widened from bf16 on the fly.
template <int M>
__device__ __forceinline__ void q8_0_dot(const Chunk<FMT_Q8_0> &ck, const XChunk<M> &x, float acc[M])
{
    const float dw = h2f(ck.d);
    const uint32_t w[8] = {ck.c0.x, ck.c0.y, ck.c0.z, ck.c0.w, ck.c1.x, ck.c1.y, ck.c1.z, ck.c1.w};
    float d[M];
#pragma unroll
    for (int m = 0; m < M; m++)
        d[m] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float f0 = (float)(int8_t)(w[i]), f1 = (float)(int8_t)(w[i] >> 8);
        const float f2 = (float)(int8_t)(w[i] >> 16), f3 = (float)(int8_t)(w[i] >> 24);
#pragma unroll
        for (int m = 0; m < M; m++) {
            d[m] = fmaf(f0, lo_bf16(x.p[m][2 * i]), d[m]);
            d[m] = fmaf(f1, hi_bf16(x.p[m][2 * i]), d[m]);
            d[m] = fmaf(f2, lo_bf16(x.p[m][2 * i + 1]), d[m]);
            d[m] = fmaf(f3, hi_bf16(x.p[m][2 * i + 1]), d[m]);
        }
    }
#pragma unroll
    for (int m = 0; m < M; m++)
        acc[m] = fmaf(dw, d[m], acc[m]);
}

// ----------------------------------------------------------------------------
// Halving butterfly over the 64 lanes.  V values per lane (V a power of two
// <= 64).  Lane bits are taken in the order 0, 1, ..., 5.  While more than
// one value is left, a step keeps half of them (the lane whose bit is set
// keeps the upper half) and adds the partner's copy, so the partner must be
// lane ^ (1 << bit) exactly: quad_perm DPP for bits 0 and 1, shuffles above.
// Once one value is left, plain sums only need a partner with the same low
// (already halved) bits: row_ror:4 and row_ror:8 DPP within a 16-lane row.
// Afterwards lanes 0..V-1 hold the totals of distinct indices idx(lane).
// ----------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

template <int STEP, bool HALVING>
__device__ __forceinline__ float partner(float v)
{
    if constexpr (STEP == 0)
        return dpp_f<0xB1>(v);  // quad_perm [1,0,3,2]: lane ^ 1
    else if constexpr (STEP == 1)
        return dpp_f<0x4E>(v);  // quad_perm [2,3,0,1]: lane ^ 2
    else if constexpr (STEP == 2)
        return HALVING ? __shfl_xor(v, 4) : dpp_f<0x124>(v);  // row_ror:4
    else if constexpr (STEP == 3)
        return HALVING ? __shfl_xor(v, 8) : dpp_f<0x128>(v);  // row_ror:8
    else if constexpr (STEP == 4)
        return __shfl_xor(v, 16);
    else
        return __shfl_xor(v, 32);
}

template <int V, int STEP>
__device__ __forceinline__ void bfly_step(float (&v)[V], int lane)
{
    constexpr int CNT = (V >> STEP) > 1 ? (V >> STEP) : 1;  // values left before this step
    if constexpr (CNT > 1) {
        constexpr int HALF = CNT / 2;
        const bool up = (lane >> STEP) & 1;
#pragma unroll
        for (int i = 0; i < HALF; i++) {
            const float keep = up ? v[i + HALF] : v[i];
            const float send = up ? v[i] : v[i + HALF];
            v[i] = keep + partner<STEP, true>(send);
        }
    } else {
        v[0] += partner<STEP, false>(v[0]);
    }
}

template <int V>
__device__ __forceinline__ float butterfly_sum(float (&v)[V], int lane)
{
    bfly_step<V, 0>(v, lane);
    bfly_step<V, 1>(v, lane);
    bfly_step<V, 2>(v, lane);
    bfly_step<V, 3>(v, lane);
    bfly_step<V, 4>(v, lane);
    bfly_step<V, 5>(v, lane);
    return v[0];
}

template <int V>
__device__ __forceinline__ int butterfly_index(int lane)
{
    int idx = 0, part = V;
#pragma unroll
    for (int b = 0; b < 6 && part > 1; b++) {
        part >>= 1;
        if ((lane >> b) & 1)
            idx += part;
    }
    return idx;
}

// the lane that holds index idx after butterfly_sum (the inverse of
// butterfly_index: a bit reversal over log2(V) bits)
template <int V>
__device__ __forceinline__ int butterfly_lane(int idx)
{
    int lane = 0, part = V;
#pragma unroll
    for (int b = 0; b < 6 && part > 1; b++) {
        part >>= 1;
        if (idx & part)
            lane |= 1 << b;
    }
    return lane;
}

constexpr int pow2_at_least(int v)
{
    int p = 1;
    while (p < v)
        p <<= 1;
    return p;
}

// ----------------------------------------------------------------------------
// The kernel
// ----------------------------------------------------------------------------
template <int FMT, int M, int CPT, int R> struct Batch {
    Chunk<FMT> ck[R][CPT];
};

template <int FMT, int M, int CPT, int R>
__device__ __forceinline__ void load_batch(const Geo &g, int64_t b, int64_t N, const int (&cl)[CPT],
                                           Batch<FMT, M, CPT, R> &bt)
{
#pragma unroll
    for (int r = 0; r < R; r++) {
        // rows past the end re-read the last row; their results are dropped
        const int64_t n = b * R + r < N ? b * R + r : N - 1;
#pragma unroll
        for (int i = 0; i < CPT; i++)
            load_chunk<FMT>(g, n, cl[i], bt.ck[r][i]);
    }
}

template <int FMT, int M, int CPT, int R>
__device__ __forceinline__ void process_batch(const Batch<FMT, M, CPT, R> &bt, const XChunk<M> (&xr)[CPT],
                                              const int (&cj)[CPT], const int (&cl)[CPT],
                                              const uint16_t *__restrict__ X, int K, const Masks &k, int64_t b, int64_t N,
                                              float *__restrict__ Y, int lane, int wv, int KS,
                                              float (*part)[pow2_at_least(R * M)])
{
    constexpr int V = pow2_at_least(R * M);
    float v[V];
#pragma unroll
    for (int t = 0; t < V; t++)
        v[t] = 0.0f;
#pragma unroll
    for (int r = 0; r < R; r++) {
        float acc[M];
#pragma unroll
        for (int m = 0; m < M; m++)
            acc[m] = 0.0f;
#pragma unroll
        for (int i = 0; i < CPT; i++) {
            if constexpr (FMT == FMT_Q4K)
                q4k_dot<M>(bt.ck[r][i], xr[i], cj[i], acc);
            else if constexpr (FMT == FMT_Q6K)
                q6k_dot<M>(bt.ck[r][i], xr[i], acc, k, X + 32 * (int64_t)cl[i], K);
            else
                q8_0_dot<M>(bt.ck[r][i], xr[i], acc);
        }
#pragma unroll
        for (int m = 0; m < M; m++)
            v[r * M + m] = acc[m];
    }
    const float tot = butterfly_sum<V>(v, lane);
    const int idx = butterfly_index<V>(lane);
    const bool writer = lane < V && idx < R * M;
    const int64_t n0 = b * R;
    if (KS == 1) {
        if (writer) {
            const int r = idx / M, m = idx % M;
            if (n0 + r < N)
                Y[(int64_t)m * N + n0 + r] = tot;
        }
    } else {
        if (writer)
            part[wv][idx] = tot;
        __syncthreads();
        if (threadIdx.x < R * M) {
            float s = 0.0f;
            for (int w = 0; w < KS; w++)
                s += part[w][threadIdx.x];
            const int r = threadIdx.x / M, m = threadIdx.x % M;
            if (n0 + r < N)
                Y[(int64_t)m * N + n0 + r] = s;
        }
        __syncthreads();
    }
}

template <int FMT, int M, int CPT, int R>
__global__ __launch_bounds__(512) void gemv_kernel(Geo g, const uint16_t *__restrict__ X,
                                                   float *__restrict__ Y, int64_t N)
{
    constexpr int V = pow2_at_least(R * M);
    __shared__ float part[8][V];

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int KS = blockDim.x >> 6;
    const int S = g.K / 32;
    const Masks k = make_masks();

    // chunks of this lane; lanes past the row end read the last chunk with a
    // zero X, so they add exactly nothing and need no branch
    int cl[CPT], cj[CPT];
    XChunk<M> xr[CPT];
#pragma unroll
    for (int i = 0; i < CPT; i++) {
        const int c = wv * 64 + lane + i * KS * 64;
        const bool live = c < S;
        cl[i] = live ? c : S - 1;
        cj[i] = cl[i] & 7;
#pragma unroll
        for (int m = 0; m < M; m++) {
            uint4 q[4];
            const uint4 *xp = reinterpret_cast<const uint4 *>(X + (int64_t)m * g.K + 32 * cl[i]);
#pragma unroll
            for (int t = 0; t < 4; t++) {
                q[t] = xp[t];
                if (!live)
                    q[t] = make_uint4(0u, 0u, 0u, 0u);
            }
            // Q4K: pairs (i, i+4) of each octet and the chunk sum; Q6K: the
            // chunk scaled by 2^e in fp16; Q8_0: as loaded
            float amax = 0.0f, sum = 0.0f;
            u16x2_t mnz = {0xFFFF, 0xFFFF};
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const uint32_t v[4] = {q[t].x, q[t].y, q[t].z, q[t].w};
#pragma unroll
                for (int c = 0; c < 4; c++) {
                    if constexpr (FMT == FMT_Q4K)
                        sum = dot2(v[c], 0x3F803F80u, sum);
                    if constexpr (FMT == FMT_Q6K) {
                        amax = bf16_pair_absmax(v[c], amax);
                        mnz = bf16_pair_minnz(v[c], mnz);
                    }
                }
                const uint4 o = FMT == FMT_Q4K ? octet_pairs(q[t]) : q[t];
                xr[i].p[m][4 * t + 0] = o.x;
                xr[i].p[m][4 * t + 1] = o.y;
                xr[i].p[m][4 * t + 2] = o.z;
                xr[i].p[m][4 * t + 3] = o.w;
            }
            xr[i].sum[m] = sum;
            xr[i].e[m] = 0;
            if constexpr (FMT == FMT_Q6K) {
                xr[i].e[m] = chunk_exp_flagged(amax, min((uint32_t)mnz.x, (uint32_t)mnz.y));
                const int es = xr[i].e[m] >= Q6K_EXACT_FLAG / 2 ? xr[i].e[m] - Q6K_EXACT_FLAG : xr[i].e[m];
#pragma unroll
                for (int e = 0; e < 16; e++)
                    xr[i].p[m][e] = bf16_pair_to_f16(xr[i].p[m][e], es);
            }
        }
    }

    // persistent workgroups; the next batch's loads are in flight while the
    // current one is computed
    const int64_t nbatch = (N + R - 1) / R;
    const int64_t G = gridDim.x;
    Batch<FMT, M, CPT, R> A, B;
    int64_t b = blockIdx.x;
    if (b < nbatch)
        load_batch<FMT, M, CPT, R>(g, b, N, cl, A);
    for (; b < nbatch; b += 2 * G) {
        const bool hasB = b + G < nbatch;
        if (hasB)
            load_batch<FMT, M, CPT, R>(g, b + G, N, cl, B);
        process_batch<FMT, M, CPT, R>(A, xr, cj, cl, X, g.K, k, b, N, Y, lane, wv, KS, part);
        if (b + 2 * G < nbatch)
            load_batch<FMT, M, CPT, R>(g, b + 2 * G, N, cl, A);
        if (hasB)
            process_batch<FMT, M, CPT, R>(B, xr, cj, cl, X, g.K, k, b + G, N, Y, lane, wv, KS, part);
    }
}

// ----------------------------------------------------------------------------
// One-shot GEMV for one to four tokens (while M times the chunks per lane
// stays within 14, so that X fits the workgroup's LDS), and for five to
// eight Q4K / Q6K tokens at up to two chunks per lane.  Each wave owns R
// whole rows and issues every weight load for them at once; the four waves
// of a workgroup share one copy of X, staged in LDS (zero-padded to CPT*64
// chunks) by the workgroup before any weight is consumed.  The threads that
// stage X also produce the per-chunk terms (Q4K: the sum of X over the
// chunk; Q6K: its power-of-two scale), so no wave recomputes them.  There is no loop over rows: the grid covers N, and the weight bytes
// of a wave are in flight from its first instructions.
// ----------------------------------------------------------------------------
constexpr int LW = 4;  // waves per workgroup of the one-shot kernel

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

// weight bytes are read once: non-temporal loads keep them from displacing X
// and the scale planes in the caches
__device__ __forceinline__ uint4 ld_stream16(const uint8_t *p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_stream8(const uint8_t *p)
{
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
    return make_uint2(v.x, v.y);
}

// what a lane loads for one chunk of one row; Q4K takes one dword of the
// 16-byte group header (dword lane%4) and the quad shares the four by DPP
template <int FMT> struct WLoad;
template <> struct WLoad<FMT_Q4K> { uint4 c; uint32_t h; };
template <> struct WLoad<FMT_Q6K> { Chunk<FMT_Q6K> ck; };
template <> struct WLoad<FMT_Q8_0> { Chunk<FMT_Q8_0> ck; };

template <int FMT>
__device__ __forceinline__ void load_w(const Geo &g, int64_t n, int c, int lane, WLoad<FMT> &w)
{
    if constexpr (FMT == FMT_Q4K) {
        const int64_t sub = n * (g.K / 32) + c;
        w.c = ld_stream16(g.B + 16 * sub);
        w.h = *reinterpret_cast<const uint32_t *>(g.B + g.scales_off + 16 * (sub >> 3) + 4 * (lane & 3));
    } else if constexpr (FMT == FMT_Q6K) {
        const int64_t grp = n * (g.K / 256) + (c >> 3);
        const int cc = c & 7;
        const uint8_t *Cg = g.B + 192 * grp;
        w.ck.lo = ld_stream16(Cg + 16 * cc);
        w.ck.hi = ld_stream8(Cg + 128 + 8 * cc);
        w.ck.sc2 = *reinterpret_cast<const uint16_t *>(g.B + g.scales_off + 16 * grp + 2 * cc);
        w.ck.d = *reinterpret_cast<const uint16_t *>(g.B + g.d_off + 2 * grp);
    } else {
        const int64_t blk = n * (g.K / 32) + c;
        w.ck.c0 = ld_stream16(g.B + 32 * blk);
        w.ck.c1 = ld_stream16(g.B + 32 * blk + 16);
        w.ck.d = *reinterpret_cast<const uint16_t *>(g.B + g.scales_off + 2 * blk);
    }
}

// Loads of a row run (rows of 8G chunks, G = K / 256 groups, starting at
// row n0 whose rows all exist): item i of lane l is chunk f = l + 64 i of
// the run, i.e. chunk l % 8 of group n0 G + 8 i + l / 8 (Q8_0: block
// 8 (n0 G + 8 i) + l) -- every address is a wave-uniform base plus a lane
// constant.
template <int FMT>
__device__ __forceinline__ void load_run(const Geo &g, int64_t n0, int i, int lane, WLoad<FMT> &w)
{
    const int64_t grp0 = n0 * (g.K / 256) + 8 * i;  // uniform
    const uint32_t lg = lane >> 3, lc = lane & 7;
    if constexpr (FMT == FMT_Q4K) {
        w.c = ld_stream16(g.B + 128 * grp0 + 16 * (uint32_t)lane);
        w.h = *reinterpret_cast<const uint32_t *>(g.B + g.scales_off + 16 * grp0 + (16 * lg + 4 * (lane & 3)));
    } else if constexpr (FMT == FMT_Q6K) {
        const uint8_t *Cg = g.B + 192 * grp0;
        w.ck.lo = ld_stream16(Cg + (192 * lg + 16 * lc));
        w.ck.hi = ld_stream8(Cg + (192 * lg + 128 + 8 * lc));
        w.ck.sc2 = *reinterpret_cast<const uint16_t *>(g.B + g.scales_off + 16 * grp0 + (16 * lg + 2 * lc));
        w.ck.d = *reinterpret_cast<const uint16_t *>(g.B + g.d_off + 2 * grp0 + 2 * lg);
    } else {
        // Q8_0: block n0 S + f, 32 code bytes and one fp16 d each
        const int64_t blk0 = 8 * grp0;
        w.ck.c0 = ld_stream16(g.B + 32 * blk0 + 32 * (uint32_t)lane);
        w.ck.c1 = ld_stream16(g.B + 32 * blk0 + (32 * (uint32_t)lane + 16));
        w.ck.d = *reinterpret_cast<const uint16_t *>(g.B + g.scales_off + 2 * blk0 + 2 * (uint32_t)lane);
    }
}

template <int FMT>
__device__ __forceinline__ Chunk<FMT> chunk_of(const WLoad<FMT> &w)
{
    if constexpr (FMT == FMT_Q4K) {
        const int h = (int)w.h;
        Chunk<FMT_Q4K> ck;
        ck.c = w.c;
        ck.h.x = __builtin_amdgcn_update_dpp(0, h, 0x00, 0xF, 0xF, false);  // quad_perm [0,0,0,0]
        ck.h.y = __builtin_amdgcn_update_dpp(0, h, 0x55, 0xF, 0xF, false);  // quad_perm [1,1,1,1]
        ck.h.z = __builtin_amdgcn_update_dpp(0, h, 0xAA, 0xF, 0xF, false);  // quad_perm [2,2,2,2]
        ck.h.w = __builtin_amdgcn_update_dpp(0, h, 0xFF, 0xF, 0xF, false);  // quad_perm [3,3,3,3]
        return ck;
    } else {
        return w.ck;
    }
}

// GLU: the fused gated projection -- wave w computes output f = row w of
// the gate weights (g) and of the up weights (g2) as its two rows, and
// writes act(gate) * up (same fp32 activation and product as the unfused
// path); N is then the number of outputs F.
//
// FS (rows of exactly FS chunks, FS not a multiple of 64): the R rows of a
// wave are one run of R * FS chunks and lane l takes chunks l, l + 64, ...
// of the run, so no lane decodes a padding chunk (K = 5120: 160 chunks a
// row, ten per lane for four rows instead of twelve slots).  A lane item
// may then fall in either of two rows, picked per lane.
template <int FMT, int M, int CPT, int R, bool GLU = false, int FS = 0>
__global__ __launch_bounds__(64 * LW) void gemv_lds_kernel(Geo g, Geo g2, const uint16_t *__restrict__ X,
                                                           float *__restrict__ Y, int64_t N, int act)
{
    static_assert(!GLU || R == 2, "gate and up rows");
    static_assert(FS == 0 || (!GLU && FS % 8 == 0 && FS >= 32 && FS <= 64 * CPT && (FS < 64 * CPT || R * FS % 64 == 0)),
                  "whole groups, items within two rows, a zero X slot where the run ends inside an item");
    // the wave's items: (row, chunk) pairs, NI per lane
    constexpr int NI = FS ? (R * FS + 63) / 64 : R * CPT;
    constexpr int SLOTS = 64 * CPT;           // chunk slots per row
    constexpr bool SUMS = FMT != FMT_Q8_0;    // per-chunk terms: Q4K sum of X, Q6K scale exponent
    constexpr int XU = M * CPT;               // uint4 of X staged per thread
    static_assert(64 * LW * XU == M * 4 * SLOTS, "the workgroup stages every quarter of X exactly once");
    __shared__ uint4 sx[M][4][SLOTS];         // quarter t of chunk c at sx[m][t][c]
    // per-chunk terms; the last slot takes the stores of the lanes that own
    // none (stores without branches, so the compiler keeps every X load
    // ahead of the weight loads instead of sinking them into the branches)
    __shared__ float ss[SUMS ? M : 1][SUMS ? SLOTS + 1 : 1];

    // (the row runs want a wave index the compiler knows to be uniform; the
    // other instances measured faster with the plain one)
    const int tid = threadIdx.x, lane = tid & 63, wv = FS != 0 ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
    const int S = g.K / 32;
    const int64_t n0 = ((int64_t)blockIdx.x * LW + wv) * (GLU ? 1 : R);
    // FS: the run starts at row n0c <= n0 so that all its R rows exist
    // (N >= R); the rows below n0 belong to the previous wave and are not
    // written
    const int64_t n0c = FS != 0 && n0 > N - R ? N - R : n0;

    // X first, so that waiting for it never waits for the weights
    uint4 xs[XU];
#pragma unroll
    for (int j = 0; j < XU; j++) {
        const int u = tid + 64 * LW * j;
        const int m = u / (4 * SLOTS), c = (u >> 2) % SLOTS, t = u & 3;
        const int cc = c < S ? c : S - 1;
        xs[j] = *reinterpret_cast<const uint4 *>(X + (int64_t)m * g.K + 32 * cc + 8 * t);
    }
    // every weight load of the wave; rows past N re-read row N-1 and slots
    // past the row end re-read its last chunk (their X is zero)
    auto item = [&](int i, int &r, int &c) {
        if constexpr (FS != 0) {
            const int f = min(lane + 64 * i, R * FS - 1);
            r = f / FS;
            c = f - r * FS;
        } else {
            r = i / CPT;
            c = lane + 64 * (i % CPT);
        }
    };
    WLoad<FMT> w[NI];
#pragma unroll
    for (int i = 0; i < NI; i++) {
        if constexpr (FS != 0) {
            load_run<FMT>(g, n0c, i, lane, w[i]);
        } else {
            int r, c;
            item(i, r, c);
            const int64_t n = GLU ? (n0 < N ? n0 : N - 1) : (n0 + r < N ? n0 + r : N - 1);
            load_w<FMT>(GLU && r == 1 ? g2 : g, n, c < S ? c : S - 1, lane, w[i]);
        }
    }
    // keep the staging below (and its wait for X) after every weight load
    __builtin_amdgcn_sched_barrier(0);
    // stage X and the per-chunk terms (four consecutive lanes hold the four
    // octets of one chunk)
#pragma unroll
    for (int j = 0; j < XU; j++) {
        const int u = tid + 64 * LW * j;
        const int m = u / (4 * SLOTS), c = (u >> 2) % SLOTS, t = u & 3;
        const uint32_t keep = c < S ? ~0u : 0u;
        const uint4 v = make_uint4(xs[j].x & keep, xs[j].y & keep, xs[j].z & keep, xs[j].w & keep);
        if constexpr (FMT == FMT_Q4K) {
            sx[m][t][c] = octet_pairs(v);
            float p = dot2(v.x, 0x3F803F80u, 0.0f);
            p = dot2(v.y, 0x3F803F80u, p);
            p = dot2(v.z, 0x3F803F80u, p);
            p = dot2(v.w, 0x3F803F80u, p);
            p += dpp_f<0xB1>(p);  // quarters t, t^1
            p += dpp_f<0x4E>(p);  // all four: the chunk
            ss[m][t == 0 ? c : SLOTS] = p;
        } else if constexpr (FMT == FMT_Q6K) {
            float a = bf16_pair_absmax(v.x, bf16_pair_absmax(v.y, bf16_pair_absmax(v.z, bf16_pair_absmax(v.w, 0.0f))));
            a = fmaxf(a, dpp_f<0xB1>(a));
            a = fmaxf(a, dpp_f<0x4E>(a));
            const u16x2_t mz = bf16_pair_minnz(v.x, bf16_pair_minnz(v.y, bf16_pair_minnz(v.z, bf16_pair_minnz(v.w, u16x2_t{0xFFFF, 0xFFFF}))));
            uint32_t mn = min((uint32_t)mz.x, (uint32_t)mz.y);
            mn = min(mn, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mn, 0xB1, 0xF, 0xF, false));  // quarters t, t^1
            mn = min(mn, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mn, 0x4E, 0xF, 0xF, false));  // the chunk
            const int ef = chunk_exp_flagged(a, mn);
            const int e = ef >= Q6K_EXACT_FLAG / 2 ? ef - Q6K_EXACT_FLAG : ef;
            sx[m][t][c] = make_uint4(bf16_pair_to_f16(v.x, e), bf16_pair_to_f16(v.y, e), bf16_pair_to_f16(v.z, e),
                                     bf16_pair_to_f16(v.w, e));
            ss[m][t == 0 ? c : SLOTS] = __int_as_float(ef);
        } else {
            sx[m][t][c] = v;
        }
    }
    lds_barrier();

    const Masks k = make_masks();
    constexpr int V = pow2_at_least(R * M);
    float v[V];
#pragma unroll
    for (int t = 0; t < V; t++)
        v[t] = 0.0f;
    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int m = 0; m < M; m++)
            acc[r][m] = 0.0f;
#pragma unroll
    for (int i = 0; i < NI; i++) {
        int r, c;
        item(i, r, c);
        // X slot: items past the run (FS) read the zero slot FS
        const int cx = FS != 0 && lane + 64 * i >= R * FS ? FS : c;
        XChunk<M> xc;
#pragma unroll
        for (int m = 0; m < M; m++) {
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const uint4 q = sx[m][t][cx];
                xc.p[m][4 * t + 0] = q.x;
                xc.p[m][4 * t + 1] = q.y;
                xc.p[m][4 * t + 2] = q.z;
                xc.p[m][4 * t + 3] = q.w;
            }
            if constexpr (FMT == FMT_Q4K)
                xc.sum[m] = ss[m][cx];
            else if constexpr (FMT == FMT_Q6K)
                xc.e[m] = __float_as_int(ss[m][cx]);
        }
        auto dot = [&](float (&a)[M]) {
            const Chunk<FMT> ck = chunk_of<FMT>(w[i]);
            if constexpr (FMT == FMT_Q4K)
                q4k_dot<M>(ck, xc, c & 7, a);
            else if constexpr (FMT == FMT_Q6K)
                q6k_dot<M>(ck, xc, a, k, X + 32 * (int64_t)c, g.K);
            else
                q8_0_dot<M>(ck, xc, a);
        };
        // the rows this item can fall in (constants once the loop is
        // unrolled; with FS >= 32 at most two)
        constexpr int FD = FS ? FS : 1;
        const int RLO = FS ? 64 * i / FD : i / CPT;
        const int RHI = FS ? min((64 * i + 63) / FD, R - 1) : RLO;
        if (RLO == RHI) {
            dot(acc[RLO]);
        } else {
            float t[M];
#pragma unroll
            for (int m = 0; m < M; m++)
                t[m] = 0.0f;
            dot(t);
            const bool hi = r > RLO;
#pragma unroll
            for (int m = 0; m < M; m++) {
                acc[RLO][m] += hi ? 0.0f : t[m];
                acc[RLO + 1][m] += hi ? t[m] : 0.0f;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int m = 0; m < M; m++)
            v[r * M + m] = acc[r][m];
    const float tot = butterfly_sum<V>(v, lane);
    const int idx = butterfly_index<V>(lane);
    if constexpr (GLU) {
        // gate of token m sits at index m, up at index M + m
        const float up = __shfl(tot, butterfly_lane<V>(idx + M < V ? idx + M : idx));
        if (lane < V && idx < M && n0 < N)
            Y[(int64_t)idx * N + n0] = act_f32(act, tot) * up;
    } else if (lane < V && idx < R * M) {
        const int r = idx / M, m = idx % M;
        if (n0c + r >= n0 && n0c + r < N)
            Y[(int64_t)m * N + n0c + r] = tot;
    }
}

constexpr int64_t GEMV_WIDE_N = 8192;

template <int FMT, int M, int CPT>
hipError_t go_lds(const Geo &g, const uint16_t *X, float *Y, int64_t N, hipStream_t s)
{
    // rows per wave from sweeps on MI355X: two for K <= 4096, four for
    // K = 5120 (the 131072 x 5120 head: 10 % faster than one), one above;
    // one for weights below GEMV_WIDE_N rows, whose grid would otherwise
    // leave CUs idle or run few workgroups per CU (one token, same process:
    // Q4K 4096 x 4096 4.22 -> 4.15 us, 6144 x 4096 5.01 -> 4.97 us, Q6K
    // 4096 x 4096 6.04 -> 5.62 us against two rows per wave)
    constexpr int R = CPT <= 2 ? 2 : CPT == 3 ? 4 : 1;
    if (R > 1 && N < GEMV_WIDE_N) {
        hipLaunchKernelGGL((gemv_lds_kernel<FMT, M, CPT, 1>), dim3((unsigned)((N + LW - 1) / LW)), dim3(64 * LW), 0, s,
                           g, g, X, Y, N, 0);
        return hipGetLastError();
    }
    const int64_t grid = (N + LW * R - 1) / (LW * R);
    // the wave's rows as one run (uniform-base loads; no padding slots where
    // 64 does not divide K/32) where measured faster with weight copies
    // rotated past the caches: K = 1024 and 5120, and Q6K also at K = 4096
    // and 14336 (Q4K and Q8_0 there: 1-4 % slower); for two tokens too (the
    // head at two tokens: 149 -> 110 us with four rows per wave as a run)
    constexpr int FSV = CPT == 1 ? 32 : FMT == FMT_Q8_0 ? 0 : CPT == 3 ? 160 : FMT == FMT_Q4K ? 0 : CPT == 2 ? 128
                        : CPT == 7 ? 448 : 0;
    if (FSV != 0 && g.K == 32 * FSV && N >= R)
        hipLaunchKernelGGL((gemv_lds_kernel<FMT, M, CPT, R, false, FSV>),
                           dim3((unsigned)grid), dim3(64 * LW), 0, s, g, g, X, Y, N, 0);
    else
        hipLaunchKernelGGL((gemv_lds_kernel<FMT, M, CPT, R>), dim3((unsigned)grid), dim3(64 * LW), 0, s, g, g, X, Y,
                           N, 0);
    return hipGetLastError();
}

// fused gated projection: one output per wave, gate and up rows together
template <int FMT, int M, int CPT>
hipError_t go_glu(const Geo &gg, const Geo &gu, const uint16_t *X, float *H, int64_t F, int act, hipStream_t s)
{
    const int64_t grid = (F + LW - 1) / LW;
    hipLaunchKernelGGL((gemv_lds_kernel<FMT, M, CPT, 2, true>), dim3((unsigned)grid), dim3(64 * LW), 0, s, gg, gu, X,
                       H, F, act);
    return hipGetLastError();
}

// one-shot kernel for M <= 4 while X fits the workgroup's LDS budget
// (M * CPT <= 14: at most 63 KiB), except four Q8_0 tokens (measured slower
// than the persistent kernel: 27.9 vs 21.9 us at 14336 x 4096); for five to
// eight Q4K and Q6K tokens up to two chunks per lane (K <= 4096: at most
// 64 KiB of X), where it measured 1.3-1.9x faster than the persistent
// kernel (Q4K 4096 x 4096, five tokens: 11.7 -> 6.5 us; 14336 x 4096:
// 25.3 -> 16.7 us; eight tokens 35.4 -> 32.8 us; Q6K 41.9 -> 27.7 us at five
// tokens), while five and six Q8_0 tokens ran 1-7 % slower; false when the
// shape needs the persistent kernel
bool one_shot_fits(int fmt, int M, int64_t K)
{
    const int64_t cpt = (K / 32 + 63) / 64;
    if (M >= 5 && M <= 8)
        return (fmt == FMT_Q4K || fmt == FMT_Q6K) && cpt <= 2;
    return !generic_fmt(fmt) && M >= 1 && M <= 4 && !(fmt == FMT_Q8_0 && M == 4) && cpt <= 8 && M * cpt <= 14;
}

template <int FMT, int M>
bool pick_lds(const Geo &g, const uint16_t *X, float *Y, int64_t N, hipStream_t s, hipError_t &e)
{
    const int S = g.K / 32;
    const int cpt = (S + 63) / 64;
    if (!one_shot_fits(FMT, M, g.K))
        return false;
    if constexpr (M > 4) {
        switch (cpt) {
        case 1: e = go_lds<FMT, M, 1>(g, X, Y, N, s); return true;
        case 2: e = go_lds<FMT, M, 2>(g, X, Y, N, s); return true;
        default: return false;
        }
    } else {
        switch (cpt) {
        case 1: e = go_lds<FMT, M, 1>(g, X, Y, N, s); return true;
        case 2: e = go_lds<FMT, M, 2>(g, X, Y, N, s); return true;
        case 3: e = go_lds<FMT, M, 3>(g, X, Y, N, s); return true;
        case 4: e = go_lds<FMT, M, 4>(g, X, Y, N, s); return true;
        case 5: e = go_lds<FMT, M, 5>(g, X, Y, N, s); return true;
        case 6: e = go_lds<FMT, M, 6>(g, X, Y, N, s); return true;
        case 7: e = go_lds<FMT, M, 7>(g, X, Y, N, s); return true;
        default:
            if constexpr (M == 1) {
                e = go_lds<FMT, M, 8>(g, X, Y, N, s);
                return true;
            }
            return false;
        }
    }
}

template <int FMT, int M, int CPT, int R>
hipError_t go(const Geo &g, const uint16_t *X, float *Y, int64_t N, int KS, int wgs_per_cu, hipStream_t s)
{
    const int64_t nbatch = (N + R - 1) / R;
    const int64_t target = (int64_t)256 * wgs_per_cu;
    const int64_t grid = nbatch < target ? nbatch : target;
    hipLaunchKernelGGL((gemv_kernel<FMT, M, CPT, R>), dim3((unsigned)grid), dim3(64 * KS), 0, s, g, X, Y, N);
    return hipGetLastError();
}

// Launch shape per (format, M, K), chosen from measured sweeps on MI355X at
// the decode shapes (14336 x 4096, 4096 x 14336, 131072 x 5120).
template <int FMT, int M>
hipError_t pick(const Geo &g, const uint16_t *X, float *Y, int64_t N, hipStream_t s)
{
    const int S = g.K / 32;  // chunks per row
    {
        hipError_t e;
        if (pick_lds<FMT, M>(g, X, Y, N, s, e))
            return e;
    }
    constexpr int R = M <= 4 ? 2 : 1;
    // Two chunks of X per lane fit in registers only for small M; Q8_0
    // streams twice the bytes per chunk and prefers one chunk per lane.
    constexpr bool wide = FMT == FMT_Q8_0 ? false : M <= 4;
    if (S <= 64)
        return go<FMT, M, 1, R>(g, X, Y, N, 1, 16, s);
    if constexpr (wide)
        if (S <= 128)
            return go<FMT, M, 2, R>(g, X, Y, N, 1, 8, s);
    if (S <= 512) {
        const int KS = (S + 63) / 64;
        return go<FMT, M, 1, R>(g, X, Y, N, KS, 16 / KS > 1 ? 16 / KS : 1, s);
    }
    if constexpr (wide)
        if (S <= 1024)
            return go<FMT, M, 2, 1>(g, X, Y, N, 8, 1, s);
    if constexpr (M == 1)
        if (S <= 2048)
            return go<FMT, M, 4, 1>(g, X, Y, N, 8, 1, s);
    return hipErrorNotSupported;  // the caller falls back to the MFMA path
}

template <int FMT>
hipError_t by_m(const Geo &g, const uint16_t *X, float *Y, int M, int64_t N, hipStream_t s)
{
    switch (M) {
    case 1: return pick<FMT, 1>(g, X, Y, N, s);
    case 2: return pick<FMT, 2>(g, X, Y, N, s);
    case 3: return pick<FMT, 3>(g, X, Y, N, s);
    case 4: return pick<FMT, 4>(g, X, Y, N, s);
    case 5: return pick<FMT, 5>(g, X, Y, N, s);
    case 6: return pick<FMT, 6>(g, X, Y, N, s);
    case 7: return pick<FMT, 7>(g, X, Y, N, s);
    case 8: return pick<FMT, 8>(g, X, Y, N, s);
    default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------
// Generic GEMV for the formats without a tuned kernel (Q5K, Q3K, Q2K, the
// legacy 32-element types, FP8): one wave per output row; lane l takes the
// 8-element tasks l, l + 64, ... of the row, decodes them exactly
// (dequant8) and accumulates w * x in fp32, and a butterfly over the wave
// sums the lanes.
// ---------------------------------------------------------------------------
template <int FMT, int M>
__global__ __launch_bounds__(256) void gemv_gen_kernel(const uint8_t *__restrict__ B, Planes p,
                                                       const uint16_t *__restrict__ X, float *__restrict__ Y,
                                                       int64_t N, int K)
{
    const int lane = threadIdx.x & 63;
    const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= N)
        return;  // the whole wave
    const int T = K / 8;
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; m++)
        acc[m] = 0.0f;
    // U tasks per lane per step with a trip count the whole wave shares
    // (tail lanes re-read the last task and add nothing), so the loads of
    // all U tasks are in flight together
    constexpr int U = 4;
    for (int i0 = 0; i0 < T; i0 += 64 * U) {
        float w[U][8];
        int ic[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            ic[u] = min(i0 + 64 * u + lane, T - 1);
            dequant8<FMT>(B, p, n * T + ic[u], w[u]);
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            const bool live = i0 + 64 * u + lane < T;
#pragma unroll
            for (int m = 0; m < M; m++) {
                const uint4 xv = *reinterpret_cast<const uint4 *>(X + (int64_t)m * K + 8 * ic[u]);
                const uint32_t xw[4] = {live ? xv.x : 0u, live ? xv.y : 0u, live ? xv.z : 0u, live ? xv.w : 0u};
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    acc[m] = fmaf(w[u][2 * k], __uint_as_float(xw[k] << 16), acc[m]);
                    acc[m] = fmaf(w[u][2 * k + 1], __uint_as_float(xw[k] & 0xffff0000u), acc[m]);
                }
            }
        }
    }
#pragma unroll
    for (int m = 0; m < M; m++)
#pragma unroll
        for (int k = 32; k >= 1; k >>= 1)
            acc[m] += __shfl_xor(acc[m], k);
    if (lane == 0)
#pragma unroll
        for (int m = 0; m < M; m++)
            Y[(int64_t)m * N + n] = acc[m];
}

// The same arithmetic with X staged once per workgroup in LDS and R rows per
// wave (while M * K * 2 bytes of X fit 64 KiB): the kernel above reads X
// from the caches once per row, so for one token its X traffic (K * 2 bytes
// per row) is larger than the weights it streams; here each 16-byte slice of
// X is read from LDS once per wave and applied to R rows.  Q4_0, Q5_0 and
// Q3K take their signed codes and the task's scale (codes8): sum q * x over
// the task with exact products, then one fused multiply-add of the scale
// into the row's sum.
//
// A scheduling barrier between a step's weight loads (with their decode)
// and its products, for the formats and token counts where it measured
// faster.  Without it the compiler interleaves, for some formats, each
// task's loads, a wait for them and its products, so that a step's loads
// are not in flight together (MI355X, 14336 x 4096, microseconds without ->
// with the barrier: Q4_1 26.4 -> 16.7 at two tokens, 33.6 -> 22.5 at four;
// Q3K 53.2 -> 27.7 at four; Q2K 33.2 -> 22.8 at four).  The signed-code
// formats go without: the barrier takes away the overlap of their decode
// with the products (Q4_0 10.9 -> 12.5 at one token, 21.0 -> 21.7 at four).
template <int FMT>
constexpr int gen_fence_from_m = FMT == FMT_Q5K ? 1
                                 : (FMT == FMT_Q3K || FMT == FMT_Q4_1 || FMT == FMT_Q5_1) ? 2
                                 : FMT == FMT_Q2K ? 4
                                                  : 1 << 20;

template <int FMT, int M, int R>
__global__ __launch_bounds__(256) void gemv_genx_kernel(const uint8_t *__restrict__ B, Planes p,
                                                        const uint16_t *__restrict__ X, float *__restrict__ Y,
                                                        int64_t N, int K)
{
    extern __shared__ uint4 sxs[];  // X as [M][K / 8] 16-byte slices
    constexpr bool SC = signed_code_fmt<FMT>;
    const int T = K / 8;
    for (int i = threadIdx.x; i < M * T; i += 256)
        sxs[i] = *reinterpret_cast<const uint4 *>(X + 8 * (int64_t)i);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int64_t n0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int m = 0; m < M; m++)
            acc[r][m] = 0.0f;
    constexpr int U = 4;  // tasks per lane per step, all loads of a step in flight together
    for (int i0 = 0; i0 < T; i0 += 64 * U) {
        float w[R][U][8], S[R][U];
        int ic[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            ic[u] = min(i0 + 64 * u + lane, T - 1);
#pragma unroll
            for (int r = 0; r < R; r++) {
                const int64_t t = min(n0 + r, N - 1) * T + ic[u];  // rows past N: not stored
                if constexpr (SC)
                    S[r][u] = codes8<FMT>(B, p, t, w[r][u]);
                else
                    dequant8<FMT>(B, p, t, w[r][u]);
            }
        }
        if constexpr (M >= gen_fence_from_m<FMT>)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; u++) {
            const bool live = i0 + 64 * u + lane < T;
#pragma unroll
            for (int m = 0; m < M; m++) {
                const uint4 xv = sxs[m * T + ic[u]];
                const uint32_t xw[4] = {live ? xv.x : 0u, live ? xv.y : 0u, live ? xv.z : 0u, live ? xv.w : 0u};
                float xf[8];
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    xf[2 * k] = __uint_as_float(xw[k] << 16);
                    xf[2 * k + 1] = __uint_as_float(xw[k] & 0xffff0000u);
                }
#pragma unroll
                for (int r = 0; r < R; r++) {
                    if constexpr (SC) {
                        float d = 0.0f;
#pragma unroll
                        for (int k = 0; k < 8; k++)
                            d = fmaf(w[r][u][k], xf[k], d);
                        acc[r][m] = fmaf(S[r][u], d, acc[r][m]);
                    } else {
#pragma unroll
                        for (int k = 0; k < 8; k++)
                            acc[r][m] = fmaf(w[r][u][k], xf[k], acc[r][m]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int m = 0; m < M; m++)
#pragma unroll
            for (int k = 32; k >= 1; k >>= 1)
                acc[r][m] += __shfl_xor(acc[r][m], k);
    if (lane == 0)
#pragma unroll
        for (int r = 0; r < R; r++)
            if (n0 + r < N)
#pragma unroll
                for (int m = 0; m < M; m++)
                    Y[(int64_t)m * N + n0 + r] = acc[r][m];
}

template <int FMT>
hipError_t gen_by_m(const uint8_t *blocks, const Planes &p, const uint16_t *X, float *Y, int M, int64_t N,
                    int64_t K, hipStream_t s)
{
    const dim3 block(256);
    // X in LDS, two rows per wave (14336 x 4096, microseconds before -> after:
    // one token Q5K 22.8 -> 21.2, Q2K 13.7 -> 11.9, Q4_0 13.6 -> 11.8, Q5_1
    // 16.3 -> 14.2; three tokens Q3K 41.5 -> 25.1, Q4_0 29.8 -> 17.6, Q5_0
    // 32.5 -> 20.6); four FP8 tokens measured slower (37.2 -> 41.0)
    if (M * K * 2 <= 65536 && !(FMT == FMT_FP8 && M >= 4)) {
        const dim3 grid2((unsigned)((N + 7) / 8));
        const size_t lds = (size_t)M * K * 2;
        switch (M) {
#define C(MM)                                                                                                   \
    case MM:                                                                                                    \
        hipLaunchKernelGGL((gemv_genx_kernel<FMT, MM, 2>), grid2, block, lds, s, blocks, p, X, Y, N, (int)K); \
        break;
            C(1) C(2) C(3) C(4) C(5) C(6) C(7) C(8)
#undef C
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((N + 3) / 4));
    switch (M) {
#define C(MM) \
    case MM: hipLaunchKernelGGL((gemv_gen_kernel<FMT, MM>), grid, block, 0, s, blocks, p, X, Y, N, (int)K); break;
    C(1) C(2) C(3) C(4) C(5) C(6) C(7) C(8)
#undef C
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemv_gen(int fmt, const uint8_t *blocks, const uint16_t *X, float *Y, int M, int64_t N,
                           int64_t K, hipStream_t s)
{
    const Planes p = planes_of(fmt, N, K);
    switch (fmt) {
    case FMT_Q5K: return gen_by_m<FMT_Q5K>(blocks, p, X, Y, M, N, K, s);
    case FMT_Q3K: return gen_by_m<FMT_Q3K>(blocks, p, X, Y, M, N, K, s);
    case FMT_Q2K: return gen_by_m<FMT_Q2K>(blocks, p, X, Y, M, N, K, s);
    case FMT_Q4_0: return gen_by_m<FMT_Q4_0>(blocks, p, X, Y, M, N, K, s);
    case FMT_Q4_1: return gen_by_m<FMT_Q4_1>(blocks, p, X, Y, M, N, K, s);
    case FMT_Q5_0: return gen_by_m<FMT_Q5_0>(blocks, p, X, Y, M, N, K, s);
    case FMT_Q5_1: return gen_by_m<FMT_Q5_1>(blocks, p, X, Y, M, N, K, s);
    case FMT_FP8: return gen_by_m<FMT_FP8>(blocks, p, X, Y, M, N, K, s);
    default: return hipErrorInvalidValue;
    }
}

template <int FMT, int M>
hipError_t glu_by_cpt(const Geo &gg, const Geo &gu, const uint16_t *X, float *H, int64_t F, int act, hipStream_t s)
{
    switch ((gg.K / 32 + 63) / 64) {
    case 1: return go_glu<FMT, M, 1>(gg, gu, X, H, F, act, s);
    case 2: return go_glu<FMT, M, 2>(gg, gu, X, H, F, act, s);
    case 3: return go_glu<FMT, M, 3>(gg, gu, X, H, F, act, s);
    case 4: return go_glu<FMT, M, 4>(gg, gu, X, H, F, act, s);
    default: return hipErrorNotSupported;
    }
}

template <int FMT>
hipError_t glu_by_m(const Geo &gg, const Geo &gu, const uint16_t *X, float *H, int M, int64_t F, int act,
                    hipStream_t s)
{
    switch (M) {
    case 1: return glu_by_cpt<FMT, 1>(gg, gu, X, H, F, act, s);
    case 2: return glu_by_cpt<FMT, 2>(gg, gu, X, H, F, act, s);
    case 3: return glu_by_cpt<FMT, 3>(gg, gu, X, H, F, act, s);
    default: return glu_by_cpt<FMT, 4>(gg, gu, X, H, F, act, s);
    }
}

}  // namespace

bool gemv_one_shot_fits(int fmt, int M, int64_t K) { return one_shot_fits(fmt, M, K); }

// the fused gated projection takes the one-shot kernel's shapes (one to
// four tokens; at 14336 x 4096, three tokens: 25.2 us fused against 28.7 us
// for two GEMVs and the elementwise pass) up to four chunks of X per lane
bool glu_fused_fits(int fmt, int M, int64_t K)
{
    return M <= 4 && one_shot_fits(fmt, M, K) && (K / 32 + 63) / 64 <= 4;
}

hipError_t launch_glu_fused(int fmt, const uint8_t *gate, const uint8_t *up, const uint16_t *X, float *H, int M,
                            int64_t F, int64_t K, int act, hipStream_t s)
{
    if (!glu_fused_fits(fmt, M, K))
        return hipErrorNotSupported;
    const Planes p = planes_of(fmt, F, K);
    const Geo gg{gate, p.scales, p.d, (int)K}, gu{up, p.scales, p.d, (int)K};
    if (fmt == FMT_Q4K)
        return glu_by_m<FMT_Q4K>(gg, gu, X, H, M, F, act, s);
    if (fmt == FMT_Q6K)
        return glu_by_m<FMT_Q6K>(gg, gu, X, H, M, F, act, s);
    return glu_by_m<FMT_Q8_0>(gg, gu, X, H, M, F, act, s);
}

hipError_t launch_gemv(int fmt, const uint8_t *blocks, const uint16_t *X, float *Y, int M,
                       int64_t N, int64_t K, hipStream_t s)
{
    if (generic_fmt(fmt))
        return launch_gemv_gen(fmt, blocks, X, Y, M, N, K, s);
    const Planes p = planes_of(fmt, N, K);
    Geo g{blocks, p.scales, p.d, (int)K};
    if (fmt == FMT_Q4K)
        return by_m<FMT_Q4K>(g, X, Y, M, N, s);
    if (fmt == FMT_Q6K)
        return by_m<FMT_Q6K>(g, X, Y, M, N, s);
    return by_m<FMT_Q8_0>(g, X, Y, M, N, s);
}

}  // namespace ql
