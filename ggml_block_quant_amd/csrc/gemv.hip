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
// Arithmetic.  Q4K / Q6K codes u (4 or 6 bits) become bf16 pairs with one
// and/or: bits 0x4300 | u are exactly the bf16 value 128 + u, and the
// nibble order of the layout puts two consecutive elements in the two
// halves of a dword.  v_dot2_f32_bf16 multiplies them by the bf16 pair of
// X directly (products exact in fp32), and the bias is removed once per
// sub-block:  sum x*(128+u) - 128*sum x.  Q8_0 codes are turned to fp32
// with v_cvt_f32_ubyte after an xor (offset-binary bytes) and FMA'd.  All
// accumulation is fp32.
#include "qlinear_internal.h"

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

// X of one chunk for M rows: 16 bf16 pairs per row, plus the sums the bias
// correction needs (s0: whole chunk or first half, s1: second half).
template <int M> struct XChunk {
    uint32_t p[M][16];
    float s0[M], s1[M];
};

template <int M>
__device__ __forceinline__ void q4k_dot(const Chunk<FMT_Q4K> &ck, const XChunk<M> &x, int c, float acc[M])
{
    const int j = c & 7;
    const uint32_t sc = __builtin_amdgcn_ubfe(ck.h.y, 4 * j, 4) | (__builtin_amdgcn_ubfe(ck.h.w, 2 * j, 2) << 4);
    const uint32_t mq = __builtin_amdgcn_ubfe(ck.h.z, 4 * j, 4) | (__builtin_amdgcn_ubfe(ck.h.w, 16 + 2 * j, 2) << 4);
    const float S = h2f(ck.h.x) * (float)sc;
    const float Mn = h2f(ck.h.x >> 16) * (float)mq;
    const uint32_t w[4] = {ck.c.x, ck.c.y, ck.c.z, ck.c.w};
    uint32_t pr[16];
#pragma unroll
    for (int q = 0; q < 4; q++)
#pragma unroll
        for (int s = 0; s < 4; s++)
            pr[4 * q + s] = ((w[q] >> (4 * s)) & 0x000F000Fu) | 0x43004300u;
#pragma unroll
    for (int m = 0; m < M; m++) {
        float d = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; e++)
            d = dot2(pr[e], x.p[m][e], d);
        // S*(d - 128*sum x) - Mn*sum x
        acc[m] = fmaf(S, d - 128.0f * x.s0[m], acc[m]);
        acc[m] = fmaf(-Mn, x.s0[m], acc[m]);
    }
}

template <int M>
__device__ __forceinline__ void q6k_dot(const Chunk<FMT_Q6K> &ck, const XChunk<M> &x, float acc[M])
{
    const float d = h2f(ck.d);
    const float Sa = d * (float)(int8_t)(ck.sc2 & 0xffu);
    const float Sb = d * (float)(int8_t)(ck.sc2 >> 8);
    const uint32_t lw[4] = {ck.lo.x, ck.lo.y, ck.lo.z, ck.lo.w};
    const uint32_t hw[2] = {ck.hi.x, ck.hi.y};
    uint32_t pr[16];
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const int o = q & 1;
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const uint32_t lo = (lw[q] >> (4 * s)) & 0x000F000Fu;
            const int sh = 8 * o + 2 * s;  // high bits of this pair start at bit sh (and 16+sh)
            const uint32_t hi = (sh >= 4 ? (hw[q >> 1] >> (sh - 4)) : (hw[q >> 1] << (4 - sh))) & 0x00300030u;
            pr[4 * q + s] = lo | hi | 0x43004300u;
        }
    }
#pragma unroll
    for (int m = 0; m < M; m++) {
        float da = 0.0f, db = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            da = dot2(pr[e], x.p[m][e], da);
            db = dot2(pr[8 + e], x.p[m][8 + e], db);
        }
        // stored u = q + 32, so 128 + u = 160 + q
        acc[m] = fmaf(Sa, da - 160.0f * x.s0[m], acc[m]);
        acc[m] = fmaf(Sb, db - 160.0f * x.s1[m], acc[m]);
    }
}

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
        const uint32_t u = w[i] ^ 0x80808080u;  // offset-binary bytes: u = q + 128
        const float f0 = (float)(u & 0xffu), f1 = (float)((u >> 8) & 0xffu);
        const float f2 = (float)((u >> 16) & 0xffu), f3 = (float)(u >> 24);
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
        acc[m] = fmaf(dw, d[m] - 128.0f * x.s0[m], acc[m]);
}

template <int FMT, int M>
__device__ __forceinline__ void dot_any(const Chunk<FMT> &ck, const XChunk<M> &x, int c, float acc[M])
{
    if constexpr (FMT == FMT_Q4K)
        q4k_dot<M>(ck, x, c, acc);
    else if constexpr (FMT == FMT_Q6K)
        q6k_dot<M>(ck, x, acc);
    else
        q8_0_dot<M>(ck, x, acc);
}

// ----------------------------------------------------------------------------
// Halving butterfly: V values per lane (V a power of two <= 64) are summed
// over the 64 lanes.  Afterwards lane l holds the total of value index
// idx(l) = sum_t bit(5-t of l) * V/2^(t+1) over the log2(V) halving steps,
// and every lane whose low 6-log2(V) bits are zero holds a distinct index.
// ----------------------------------------------------------------------------
template <int V>
__device__ __forceinline__ float butterfly_sum(float (&v)[V], int lane)
{
    int cnt = V;
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) {
        if (cnt > 1) {
            const int half = cnt / 2;
            const bool up = (lane & k) != 0;
#pragma unroll
            for (int i = 0; i < V / 2; i++) {
                if (i < half) {
                    const float keep = up ? v[i + half] : v[i];
                    const float send = up ? v[i] : v[i + half];
                    v[i] = keep + __shfl_xor(send, k);
                }
            }
            cnt = half;
        } else {
            v[0] += __shfl_xor(v[0], k);
        }
    }
    return v[0];
}

template <int V>
__device__ __forceinline__ int butterfly_index(int lane)
{
    int idx = 0, part = V;
#pragma unroll
    for (int k = 32; k >= 1 && part > 1; k >>= 1) {
        part >>= 1;
        if (lane & k)
            idx += part;
    }
    return idx;
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

    int cidx[CPT];
    bool live[CPT];
    XChunk<M> xr[CPT];
#pragma unroll
    for (int i = 0; i < CPT; i++) {
        cidx[i] = wv * 64 + lane + i * KS * 64;
        live[i] = cidx[i] < S;
#pragma unroll
        for (int m = 0; m < M; m++) {
            uint4 q[4] = {};
            if (live[i]) {
                const uint4 *xp = reinterpret_cast<const uint4 *>(X + (int64_t)m * g.K + 32 * cidx[i]);
#pragma unroll
                for (int t = 0; t < 4; t++)
                    q[t] = xp[t];
            }
#pragma unroll
            for (int t = 0; t < 4; t++) {
                xr[i].p[m][4 * t + 0] = q[t].x;
                xr[i].p[m][4 * t + 1] = q[t].y;
                xr[i].p[m][4 * t + 2] = q[t].z;
                xr[i].p[m][4 * t + 3] = q[t].w;
            }
            float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                s0 = dot2(xr[i].p[m][e], 0x3F803F80u, s0);
                s1 = dot2(xr[i].p[m][8 + e], 0x3F803F80u, s1);
            }
            if constexpr (FMT == FMT_Q6K) {
                xr[i].s0[m] = s0;
                xr[i].s1[m] = s1;
            } else {
                xr[i].s0[m] = s0 + s1;
                xr[i].s1[m] = 0.0f;
            }
        }
    }

    const int64_t nbatch = (N + R - 1) / R;
    for (int64_t b = blockIdx.x; b < nbatch; b += gridDim.x) {
        const int64_t n0 = b * R;
        Chunk<FMT> ck[R][CPT];
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int i = 0; i < CPT; i++)
                if (live[i] && n0 + r < N)
                    load_chunk<FMT>(g, n0 + r, cidx[i], ck[r][i]);
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
            for (int i = 0; i < CPT; i++)
                if (live[i] && n0 + r < N)
                    dot_any<FMT, M>(ck[r][i], xr[i], cidx[i], acc);
#pragma unroll
            for (int m = 0; m < M; m++)
                v[r * M + m] = acc[m];
        }
        const float tot = butterfly_sum<V>(v, lane);
        const int idx = butterfly_index<V>(lane);
        constexpr int low_mask = (64 / V) - 1;  // lanes sharing one index
        const bool writer = (lane & low_mask) == 0 && idx < R * M;
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
}

template <int FMT, int M, int CPT, int R>
hipError_t go(const Geo &g, const uint16_t *X, float *Y, int64_t N, int KS, hipStream_t s)
{
    const int64_t nbatch = (N + R - 1) / R;
    // enough workgroups to keep every CU busy while each walks many rows
    const int64_t target = (int64_t)256 * 16 / KS;
    const int64_t grid = nbatch < target ? nbatch : target;
    hipLaunchKernelGGL((gemv_kernel<FMT, M, CPT, R>), dim3((unsigned)grid), dim3(64 * KS), 0, s, g, X, Y, N);
    return hipGetLastError();
}

template <int FMT, int M>
hipError_t pick(const Geo &g, const uint16_t *X, float *Y, int64_t N, hipStream_t s)
{
    const int S = g.K / 32;  // chunks per row
    constexpr int R = M <= 2 ? 4 : (M <= 4 ? 2 : 1);
    // Two chunks of X per lane fit in registers only for small M.
    constexpr bool wide = FMT == FMT_Q8_0 ? M <= 1 : M <= 4;
    // One wave per row while a lane can hold the row's share of X, else
    // split K over up to 8 waves, then give lanes more chunks.
    if (S <= 64)
        return go<FMT, M, 1, R>(g, X, Y, N, 1, s);
    if constexpr (wide)
        if (S <= 128)
            return go<FMT, M, 2, R>(g, X, Y, N, 1, s);
    if (S <= 512)
        return go<FMT, M, 1, R>(g, X, Y, N, (S + 63) / 64, s);
    if constexpr (wide)
        if (S <= 1024)
            return go<FMT, M, 2, 1>(g, X, Y, N, 8, s);
    if constexpr (M == 1)
        if (S <= 2048)
            return go<FMT, M, 4, 1>(g, X, Y, N, 8, s);
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

}  // namespace

hipError_t launch_gemv(int fmt, const uint8_t *blocks, const uint16_t *X, float *Y, int M,
                       int64_t N, int64_t K, hipStream_t s)
{
    const Planes p = planes_of(fmt, N, K);
    Geo g{blocks, p.scales, p.d, (int)K};
    if (fmt == FMT_Q4K)
        return by_m<FMT_Q4K>(g, X, Y, M, N, s);
    if (fmt == FMT_Q6K)
        return by_m<FMT_Q6K>(g, X, Y, M, N, s);
    return by_m<FMT_Q8_0>(g, X, Y, M, N, s);
}

}  // namespace ql
