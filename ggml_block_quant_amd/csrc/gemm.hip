// gemm.hip -- tiled quantized matmuls on the MFMA matrix cores for batched
// decode and prefill (M > 8):
//   * dequant-to-bf16 path: each 128 x 64 tile of W is decoded from its
//     blocks in registers, rounded to bf16 and staged in LDS next to the
//     bf16 X tile; v_mfma_f32_16x16x32_bf16 accumulates in fp32.
//   * Q8_0 x Q8_0 int8 path: X is first quantized to Q8_0 blocks (the same
//     rule as the weights); per 32-element block, v_mfma_i32_32x32x32_i8
//     forms the exact integer dot products, which are scaled by
//     d_w * d_x and accumulated in fp32.
//
// Page "Quantization types": section "NVFP4" (larger dense batches use
// tiled matrix multiplication; activations are quantized once and reused
// across output tiles) and section "FP8" (a weight tile is converted to
// BF16 inside the GEMM; dynamic per-token activation quantizers feed the
// quantized GEMM).
//
// Both kernels use 256 threads (4 wavefronts) per output tile and optionally
// split K over gridDim.z with fp32 atomics into a zeroed Y when the (n, m)
// tiles alone cannot fill the 256 CUs.
#include "qlinear_internal.h"
#include "decode.h"

#include <type_traits>

namespace ql {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float h2f(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xffffu));
}

// two fp32 -> one dword of two bf16 (round to nearest even, v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    const f32x2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// weight bytes are read once: a non-temporal load keeps them from displacing
// X and the scale planes in the caches
__device__ __forceinline__ uint4 ld_nt16(const uint8_t *p)
{
    typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------
// Dequant-to-bf16 path.  Output tile BN (n) x BM (m) per workgroup of 4
// wavefronts; wave w owns rows n0 + w*16*NT .. +16*NT of W and all BM rows
// of X.  K advances in slabs of 128 = 4 blocks of 32.
//
// W never goes through LDS: in a slab, lane l of a wave decodes the whole
// 32-element block (4*s + l/16) of row l%16 of its n-tile -- one 16/32-byte
// load, one scale decode -- straight into the four bf16 B-operand
// fragments of the slab's four MFMAs.  MFMA t then pairs, for lane group
// g = l/16, elements 8t..8t+7 of block 4s+g with the same elements of X:
// the k order inside the slab is permuted, identically on both operands,
// which leaves every dot product unchanged.  Only X is staged in LDS
// (double-buffered, one barrier per slab), and the next slab's W bytes and
// X are loaded while the current slab is computed.
//
// v_mfma_f32_16x16x32_bf16: A = X (16 m x 32 k), B = W^T (32 k x 16 n);
// lane l holds D[m = 4*(l/16) + r][n = l%16], r = 0..3.
// ---------------------------------------------------------------------------
constexpr int SLAB = 128;            // k per slab
constexpr int XPITCH = SLAB * 2 + 16; // bytes per LDS row of X (272: conflict-free 16-byte reads)

template <int FMT> struct WBlk;  // raw bytes of one 32-element block + its scales
template <> struct WBlk<FMT_Q8_0> { uint4 c0, c1; uint32_t d; };
template <> struct WBlk<FMT_Q4K> { uint4 c; uint4 h; };
template <> struct WBlk<FMT_Q6K> { uint4 lo; uint2 hi; uint32_t sc2, d; };

template <int FMT>
__device__ __forceinline__ void load_wblk(const uint8_t *__restrict__ B, int64_t sc_off, int64_t d_off, int K,
                                          int64_t n, int c, WBlk<FMT> &w)
{
    if constexpr (FMT == FMT_Q8_0) {
        const int64_t blk = n * (K / 32) + c;
        const uint4 *p = reinterpret_cast<const uint4 *>(B + 32 * blk);
        w.c0 = p[0];
        w.c1 = p[1];
        w.d = *reinterpret_cast<const uint16_t *>(B + sc_off + 2 * blk);
    } else if constexpr (FMT == FMT_Q4K) {
        const int64_t sub = n * (K / 32) + c;
        w.c = *reinterpret_cast<const uint4 *>(B + 16 * sub);
        w.h = *reinterpret_cast<const uint4 *>(B + sc_off + 16 * (sub >> 3));
    } else {
        const int64_t grp = n * (K / 256) + (c >> 3);
        const int cc = c & 7;
        const uint8_t *Cg = B + 192 * grp;
        w.lo = *reinterpret_cast<const uint4 *>(Cg + 16 * cc);
        w.hi = *reinterpret_cast<const uint2 *>(Cg + 128 + 8 * cc);
        w.sc2 = *reinterpret_cast<const uint16_t *>(B + sc_off + 16 * grp + 2 * cc);
        w.d = *reinterpret_cast<const uint16_t *>(B + d_off + 2 * grp);
    }
}

// Each weight w (fp32) reaches the MFMA as two bf16 operands, hi = bf16(w)
// (round to nearest even) and lo = bf16(w - hi): w - hi is exact in fp32
// and at most 2^-8 |w|, so |hi + lo - w| <= 2^-17 |w|.  A single bf16 per
// weight would leave up to 2^-8 |w| per product, and those errors add up
// when they share a sign (a constant row against positive activations).
__device__ __forceinline__ void split_bf16(float a, float b, uint32_t &hi, uint32_t &lo)
{
    hi = pack_bf16(a, b);
    lo = pack_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// 32 dequantized weights of one block -> 16 dwords of hi bf16 pairs and 16
// of lo pairs (element 2e, 2e+1 in dword e)
template <int FMT>
__device__ __forceinline__ void decode_wblk(const WBlk<FMT> &w, int c, uint32_t hi[16], uint32_t lo[16])
{
    if constexpr (FMT == FMT_Q8_0) {
        const float d = h2f(w.d);
        const uint32_t v[8] = {w.c0.x, w.c0.y, w.c0.z, w.c0.w, w.c1.x, w.c1.y, w.c1.z, w.c1.w};
#pragma unroll
        for (int i = 0; i < 8; i++) {
            split_bf16(d * (float)(int8_t)(v[i]), d * (float)(int8_t)(v[i] >> 8), hi[2 * i], lo[2 * i]);
            split_bf16(d * (float)(int8_t)(v[i] >> 16), d * (float)(int8_t)(v[i] >> 24), hi[2 * i + 1], lo[2 * i + 1]);
        }
    } else if constexpr (FMT == FMT_Q4K) {
        const int j = c & 7;
        const uint32_t sc = __builtin_amdgcn_ubfe(w.h.y, 4 * j, 4) | (__builtin_amdgcn_ubfe(w.h.w, 2 * j, 2) << 4);
        const uint32_t mq = __builtin_amdgcn_ubfe(w.h.z, 4 * j, 4) | (__builtin_amdgcn_ubfe(w.h.w, 16 + 2 * j, 2) << 4);
        const float S = h2f(w.h.x) * (float)sc;
        const float Mn = h2f(w.h.x >> 16) * (float)mq;
        const uint32_t v[4] = {w.c.x, w.c.y, w.c.z, w.c.w};
#pragma unroll
        for (int q = 0; q < 4; q++) {
            // nibble p holds element 2p (p < 4) or 2(p-4)+1, so the bytes of
            // lo = v & 0x0F0F0F0F are elements 0,4,1,5 and those of
            // hi = (v >> 4) & 0x0F0F0F0F are elements 2,6,3,7
            uint32_t nl = v[q] & 0x0F0F0F0Fu, nh = (v[q] >> 4) & 0x0F0F0F0Fu;
            // opaque to the optimizer, so that each element converts with one
            // byte-selecting v_cvt_f32_ubyteN instead of a bfe and a convert
            asm("" : "+v"(nl));
            asm("" : "+v"(nh));
            const float e0 = (float)(nl & 0xffu), e4 = (float)((nl >> 8) & 0xffu);
            const float e1 = (float)((nl >> 16) & 0xffu), e5 = (float)(nl >> 24);
            const float e2 = (float)(nh & 0xffu), e6 = (float)((nh >> 8) & 0xffu);
            const float e3 = (float)((nh >> 16) & 0xffu), e7 = (float)(nh >> 24);
            split_bf16(fmaf(S, e0, -Mn), fmaf(S, e1, -Mn), hi[4 * q + 0], lo[4 * q + 0]);
            split_bf16(fmaf(S, e2, -Mn), fmaf(S, e3, -Mn), hi[4 * q + 1], lo[4 * q + 1]);
            split_bf16(fmaf(S, e4, -Mn), fmaf(S, e5, -Mn), hi[4 * q + 2], lo[4 * q + 2]);
            split_bf16(fmaf(S, e6, -Mn), fmaf(S, e7, -Mn), hi[4 * q + 3], lo[4 * q + 3]);
        }
    } else {
        const float d = h2f(w.d);
        const float Sab[2] = {d * (float)(int8_t)(w.sc2 & 0xffu), d * (float)(int8_t)(w.sc2 >> 8)};
        const uint32_t l4[4] = {w.lo.x, w.lo.y, w.lo.z, w.lo.w};
        const uint32_t h2[2] = {w.hi.x, w.hi.y};
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int o = q & 1;
            const float S = Sab[q >> 1], B = -32.0f * S;  // S (u - 32) = fma(S, u, -32 S), exact
            // the four codes u = q + 32 of bytes (e0, e4, e1, e5) and (e2, e6, e3, e7) of the octet:
            // low nibbles masked out of the dword, the two high bits of each moved to bits 4-5 of
            // its byte (element 2p's pair at bit 8o + 2p of the high-bit dword, 2p + 1's at 16 + 8o + 2p)
            const uint32_t x = h2[q >> 1] >> (8 * o);
            uint32_t ua = (l4[q] & 0x0F0F0F0Fu) | ((x << 4) & 0x00300030u) | ((x << 8) & 0x30003000u);
            uint32_t ub = ((l4[q] >> 4) & 0x0F0F0F0Fu) | ((x << 2) & 0x00300030u) | ((x << 6) & 0x30003000u);
            // opaque, so that each element converts with one byte-selecting v_cvt_f32_ubyteN
            asm("" : "+v"(ua));
            asm("" : "+v"(ub));
            const float e0 = (float)(ua & 0xffu), e4 = (float)((ua >> 8) & 0xffu);
            const float e1 = (float)((ua >> 16) & 0xffu), e5 = (float)(ua >> 24);
            const float e2 = (float)(ub & 0xffu), e6 = (float)((ub >> 8) & 0xffu);
            const float e3 = (float)((ub >> 16) & 0xffu), e7 = (float)(ub >> 24);
            split_bf16(fmaf(S, e0, B), fmaf(S, e1, B), hi[4 * q + 0], lo[4 * q + 0]);
            split_bf16(fmaf(S, e2, B), fmaf(S, e3, B), hi[4 * q + 1], lo[4 * q + 1]);
            split_bf16(fmaf(S, e4, B), fmaf(S, e5, B), hi[4 * q + 2], lo[4 * q + 2]);
            split_bf16(fmaf(S, e6, B), fmaf(S, e7, B), hi[4 * q + 3], lo[4 * q + 3]);
        }
    }
}

template <int FMT, int TM, int NT>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const uint8_t *__restrict__ B, int64_t sc_off,
                                                        int64_t d_off, const uint16_t *__restrict__ X,
                                                        float *__restrict__ Y, int M, int N, int K,
                                                        int slabs_per_split)
{
    constexpr int BM = 16 * TM;
    constexpr int XU4 = BM * SLAB * 2 / 16 / 256;  // uint4 of X per thread per slab
    static_assert(XU4 >= 1 || BM * SLAB * 2 / 16 < 256, "X staging");
    constexpr int XPER = BM * SLAB * 2 / 16;        // uint4 of X per slab
    __shared__ __attribute__((aligned(16))) uint8_t sX[2][BM * XPITCH];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const int64_t n_wave = (int64_t)blockIdx.x * (64 * NT) + wave * 16 * NT;
    const int m0 = blockIdx.y * BM;
    const int nslab = K / SLAB;
    const int s0 = blockIdx.z * slabs_per_split;
    const int s1 = min(nslab, s0 + slabs_per_split);
    if (s0 >= s1)
        return;

    // rows of W this lane decodes (clamped: rows past N are decoded but not stored)
    int64_t wrow[NT];
#pragma unroll
    for (int i = 0; i < NT; i++) {
        const int64_t n = n_wave + 16 * i + r16;
        wrow[i] = n < N ? n : N - 1;
    }

    auto load_x = [&](int s, uint4 (&xr)[XU4 > 0 ? XU4 : 1]) {
#pragma unroll
        for (int t = 0; t < (XU4 > 0 ? XU4 : 1); t++) {
            const int i = tid + 256 * t;
            const int row = i / (SLAB / 8), q = i % (SLAB / 8);
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (i < XPER && m0 + row < M)
                v = *reinterpret_cast<const uint4 *>(X + (int64_t)(m0 + row) * K + s * SLAB + 8 * q);
            xr[t] = v;
        }
    };
    auto store_x = [&](int buf, const uint4 (&xr)[XU4 > 0 ? XU4 : 1]) {
#pragma unroll
        for (int t = 0; t < (XU4 > 0 ? XU4 : 1); t++) {
            const int i = tid + 256 * t;
            const int row = i / (SLAB / 8), q = i % (SLAB / 8);
            if (i < XPER)
                *reinterpret_cast<uint4 *>(&sX[buf][row * XPITCH + 16 * q]) = xr[t];
        }
    };

    f32x4_t acc[NT][TM];
#pragma unroll
    for (int i = 0; i < NT; i++)
#pragma unroll
        for (int j = 0; j < TM; j++)
            acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // Prefetch distance 2: while slab s is computed, X of slab s+1 waits in
    // registers for its LDS stage and the bytes of slab s+2 are in flight.
    uint4 x1[XU4 > 0 ? XU4 : 1], x2[XU4 > 0 ? XU4 : 1];
    WBlk<FMT> wa[NT], wb[NT], wc[NT];
    load_x(s0, x1);
#pragma unroll
    for (int i = 0; i < NT; i++)
        load_wblk<FMT>(B, sc_off, d_off, K, wrow[i], 4 * s0 + g, wa[i]);
    store_x(0, x1);
    if (s0 + 1 < s1) {
        load_x(s0 + 1, x1);
#pragma unroll
        for (int i = 0; i < NT; i++)
            load_wblk<FMT>(B, sc_off, d_off, K, wrow[i], 4 * (s0 + 1) + g, wb[i]);
    }
    lds_barrier();

    for (int s = s0; s < s1; s++) {
        const int buf = (s - s0) & 1;
        if (s + 2 < s1) {
            load_x(s + 2, x2);
#pragma unroll
            for (int i = 0; i < NT; i++)
                load_wblk<FMT>(B, sc_off, d_off, K, wrow[i], 4 * (s + 2) + g, wc[i]);
        }
#pragma unroll
        for (int i = 0; i < NT; i++) {
            uint32_t wh[16], wl[16];
            decode_wblk<FMT>(wa[i], 4 * s + g, wh, wl);
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, make_uint4(wh[4 * t], wh[4 * t + 1], wh[4 * t + 2], wh[4 * t + 3]));
                const bf16x8_t bl = __builtin_bit_cast(bf16x8_t, make_uint4(wl[4 * t], wl[4 * t + 1], wl[4 * t + 2], wl[4 * t + 3]));
#pragma unroll
                for (int j = 0; j < TM; j++) {
                    const bf16x8_t xa = *reinterpret_cast<const bf16x8_t *>(
                        &sX[buf][(16 * j + r16) * XPITCH + 64 * g + 16 * t]);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bh, acc[i][j], 0, 0, 0);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bl, acc[i][j], 0, 0, 0);
                }
            }
        }
        if (s + 1 < s1)
            store_x(buf ^ 1, x1);
        lds_barrier();
#pragma unroll
        for (int i = 0; i < NT; i++) {
            wa[i] = wb[i];
            wb[i] = wc[i];
        }
#pragma unroll
        for (int t = 0; t < (XU4 > 0 ? XU4 : 1); t++)
            x1[t] = x2[t];
    }

    // lane holds D[m = 4*g + r][n = r16] of each 16 x 16 tile
    const bool atomic = gridDim.z > 1;
#pragma unroll
    for (int i = 0; i < NT; i++) {
        const int64_t n = n_wave + 16 * i + r16;
        if (n >= N)
            continue;
#pragma unroll
        for (int j = 0; j < TM; j++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int m = m0 + 16 * j + 4 * g + r;
                if (m < M) {
                    float *y = Y + (int64_t)m * N + n;
                    if (atomic)
                        atomicAdd(y, acc[i][j][r]);
                    else
                        *y = acc[i][j][r];
                }
            }
    }
}

// ---------------------------------------------------------------------------
// Prefill dequant-to-bf16 path (M > 64): v_mfma_f32_32x32x16_bf16, which
// keeps the matrix cores full with four independent accumulators per wave
// (16x16x32 needs sixteen).  Workgroup tile 256 (n) x 128 (m), four waves
// along n, each 64 n x 128 m = 2 x 4 tiles of 32 x 32.  Per slab of 128 k a
// lane decodes the blocks 2h and 2h+1 of the slab (h = lane/32) for its two
// rows n = n_wave + 32 i + lane%32, i.e. 64 weights per row; MFMA step t
// (0..7) takes elements 8t..8t+7 of those 64 from every lane, which is
// X[m][128 s + 64 h + 8 t ..] on the A side -- contiguous 16-byte LDS reads.
// A = X (32 m x 16 k), B = W^T (16 k x 32 n); lane l holds
// D[m = 8*(r/4) + 4*(l/32) + r%4][n = l%32], r = 0..15.
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Skinny dequant-to-bf16 path for small M (M <= 16 * TM): a weight stream.
// A workgroup of KS wavefronts owns 16*NT rows of W; wave w takes slabs
// [w*per, (w+1)*per) of K.  Each wave is independent until the end: it
// keeps a ring of PF slabs of W bytes in flight (PF * NT * 32 bytes per lane)
// and reads its X fragments straight from L2 (X is small and shared by all
// workgroups), decodes W into the MFMA B operand as in gemm_bf16_kernel,
// and accumulates 16 x 16 tiles.  The KS partial tiles are summed once
// through LDS, so Y is written with plain stores.
// ---------------------------------------------------------------------------
template <int FMT, int TM, int NT, int PF>
__global__ __launch_bounds__(512) void gemm_skinny_kernel(const uint8_t *__restrict__ B, int64_t sc_off,
                                                          int64_t d_off, const uint16_t *__restrict__ X,
                                                          float *__restrict__ Y, int M, int N, int K, int per)
{
    extern __shared__ float red[];  // [KS][NT*TM*4][64]
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, KS = blockDim.x >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * NT;
    const int nslab = K / SLAB;
    const int sb = wv * per;
    const int se = min(nslab, sb + per);

    int64_t wrow[NT];
#pragma unroll
    for (int i = 0; i < NT; i++) {
        const int64_t n = n0 + 16 * i + r16;
        wrow[i] = n < N ? n : N - 1;
    }
    const uint16_t *xrow[TM];
    bool xlive[TM];
#pragma unroll
    for (int j = 0; j < TM; j++) {
        const int m = 16 * j + r16;
        xlive[j] = m < M;
        xrow[j] = X + (int64_t)(xlive[j] ? m : 0) * K + 32 * g;
    }

    f32x4_t acc[NT][TM];
#pragma unroll
    for (int i = 0; i < NT; i++)
#pragma unroll
        for (int j = 0; j < TM; j++)
            acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // ring of PF slabs in flight: W bytes and X fragments
    WBlk<FMT> ring[PF][NT];
    uint4 xq[PF][TM][4];
    auto load_slab = [&](int u, int su) {
#pragma unroll
        for (int i = 0; i < NT; i++)
            load_wblk<FMT>(B, sc_off, d_off, K, wrow[i], 4 * su + g, ring[u][i]);
#pragma unroll
        for (int j = 0; j < TM; j++) {
            const uint4 *xp = reinterpret_cast<const uint4 *>(xrow[j] + su * SLAB);
            // rows of the 16-row tile past M are not read (they are zeroed at use)
            if (xlive[j])
#pragma unroll
                for (int t = 0; t < 4; t++)
                    xq[u][j][t] = xp[t];
        }
    };
#pragma unroll
    for (int u = 0; u < PF; u++)
        if (sb + u < se)
            load_slab(u, sb + u);

    for (int s = sb; s < se; s += PF) {
#pragma unroll
        for (int u = 0; u < PF; u++) {
            const int su = s + u;
            if (su < se) {
#pragma unroll
                for (int i = 0; i < NT; i++) {
                    uint32_t wh[16], wl[16];
                    decode_wblk<FMT>(ring[u][i], 4 * su + g, wh, wl);
#pragma unroll
                    for (int t = 0; t < 4; t++) {
                        const bf16x8_t bh = __builtin_bit_cast(
                            bf16x8_t, make_uint4(wh[4 * t], wh[4 * t + 1], wh[4 * t + 2], wh[4 * t + 3]));
                        const bf16x8_t bl = __builtin_bit_cast(
                            bf16x8_t, make_uint4(wl[4 * t], wl[4 * t + 1], wl[4 * t + 2], wl[4 * t + 3]));
#pragma unroll
                        for (int j = 0; j < TM; j++) {
                            // rows of X past M read row 0 and are zeroed here
                            const bf16x8_t xa = __builtin_bit_cast(
                                bf16x8_t, xlive[j] ? xq[u][j][t] : make_uint4(0u, 0u, 0u, 0u));
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bh, acc[i][j], 0, 0, 0);
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bl, acc[i][j], 0, 0, 0);
                        }
                    }
                }
                if (su + PF < se)
                    load_slab(u, su + PF);
            }
        }
    }

    // sum the KS partial tiles: red[w][e][lane], e = (i*TM + j)*4 + r
    constexpr int E = NT * TM * 4;
#pragma unroll
    for (int i = 0; i < NT; i++)
#pragma unroll
        for (int j = 0; j < TM; j++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                red[(wv * E + (i * TM + j) * 4 + r) * 64 + lane] = acc[i][j][r];
    __syncthreads();
    for (int q = threadIdx.x; q < E * 64; q += blockDim.x) {
        const int e = q >> 6, l = q & 63;
        float sum = 0.0f;
        for (int w = 0; w < KS; w++)
            sum += red[(w * E + e) * 64 + l];
        const int i = e / (TM * 4), j = (e / 4) % TM, r = e & 3;
        const int64_t n = n0 + 16 * i + (l & 15);
        const int m = 16 * j + 4 * (l >> 4) + r;
        if (n < N && m < M)
            Y[(int64_t)m * N + n] = sum;
    }
}

// ---------------------------------------------------------------------------
// Prefill dequant-to-bf16 path (large M): output tile 256 (m) x 256 (n) per
// workgroup of eight waves (two per SIMD), each wave 128 x 64 = 4 x 2 tiles
// of v_mfma_f32_32x32x16_bf16 (128 accumulator registers).  K advances in
// slabs of 32 (one Q8_0 block / one K-quant sub-block per row).
//
//   * Every global read is a direct global->LDS load (no registers, no LDS
//     store instruction): the X slab (bf16) into a ring of four stages (two
//     loads per wave) and the raw block bytes of the 256 W rows into a ring
//     of three (waves 0..3).  The only waits on them are the explicit vmcnt
//     waits below, each wave counting its own loads.
//   * Thread t < 256 (waves 0..3) decodes row t of the W slab from its raw
//     bytes to bf16 and stores it into a double-buffered W stage, one slab
//     ahead, while its wave's first eight MFMAs of the current slab run;
//     waves 4..7 decode nothing, so each SIMD pairs a decoding wave with one
//     whose MFMAs fill the decode's issue slots.
//   * Both bf16 operand stages use one layout: 16-byte chunk c (k = 8c..8c+7)
//     of row r sits at slot 4r + (c ^ ((r >> 2) & 3)), so the sixteen rows a
//     ds_read_b128 phase touches land on distinct banks.
//   * One barrier per slab, between its two k-steps; after it the fragments
//     of the next slab are read and the loads of slab s+4 are issued.
//   * When the tiles alone cannot fill the chip, gridDim.y splits K: each
//     workgroup takes a run of slabs and adds its partial tile into Y
//     (zeroed beforehand) with fp32 atomics.
// ---------------------------------------------------------------------------
constexpr int PBM = 256, PBN = 256, PBK = 32;
constexpr int PF_MIN_M = 513;                   // smallest M routed here (measured crossover)
constexpr int PNX = 4, PNR = 3, PNW = 2;        // X, raw W and bf16 W stages
constexpr int PSTAGE = 256 * PBK * 2;           // bytes per bf16 operand stage
constexpr int PAHEAD = 4;                       // slabs between issue and use
static_assert(PAHEAD == PNR + 1 && PAHEAD <= PNX, "stage counts");

__device__ __forceinline__ int pslot(int row, int c) { return row * 4 + (c ^ ((row >> 2) & 3)); }

// Raw bytes of one W slab (256 rows, 32 elements each) in LDS, and the
// direct loads per wave that fill them (WD):
//   Q8_0: codes 32 B/row at 32r; the scale dword holding d at 8192 + 4r
//   Q4K:  codes 16 B/row at 16r; the 16-byte group header at 4096 + 16r
//   Q6K:  low nibbles 16 B at 16r; the 16 high-bit bytes holding this chunk
//         at 4096 + 16r; the sub-scale dword at 8192 + 4r; the d dword at
//         9216 + 4r
template <int FMT> struct PRaw;
// (vpm: decode VALU instructions scheduled per MFMA)
template <> struct PRaw<FMT_Q8_0> { static constexpr int bytes = 9216, wd = 3, vpm = 8; };
template <> struct PRaw<FMT_Q4K> { static constexpr int bytes = 8192, wd = 2, vpm = 12; };
template <> struct PRaw<FMT_Q6K> { static constexpr int bytes = 10240, wd = 4, vpm = 13; };

typedef __attribute__((address_space(3))) void *lds_ptr_t;
typedef __attribute__((address_space(1))) void *gbl_ptr_t;
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Direct global->LDS loads in the scalar-base form: lane i reads base + off_i
// (base the same for the whole wave, off_i a 32-bit byte offset) and its
// bytes land at LDS address lds + 16*i (dma16) or lds + 4*i (dma4); lds is
// the same for the whole wave.  Per-slab address updates are then scalar
// adds.  Issued from inline assembly so that the compiler adds no waits of
// its own for them: they write no register, and every read of the bytes
// they bring is preceded by an explicit vmcnt wait and a barrier.
__device__ __forceinline__ void dma16(const uint8_t *base, uint32_t off, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(const uint8_t *base, uint32_t off, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p) { return (uint32_t)(uintptr_t)(lds_ptr_t)p; }

template <int FMT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_pf_kernel(
    const uint8_t *__restrict__ B, int64_t sc_off, int64_t d_off, const uint16_t *__restrict__ X,
    float *__restrict__ Y, int M, int N, int K, int slabs_per_split)
{
    // Q8_0: the W stage holds the codes (exact in bf16) and the block scale
    // enters through a running rescale of the accumulators; the K-quants:
    // each weight as a bf16 hi + lo pair (two W stages)
    constexpr bool CODE = FMT == FMT_Q8_0;
    constexpr int NWS = CODE ? 1 : 2;                      // bf16 W planes per stage
    constexpr int RAWB = PRaw<FMT>::bytes;
    constexpr int RHO = CODE ? (PNW + 1) * 256 * 4 : 0;   // rescale factors per stage, final scales
    __shared__ __attribute__((aligned(1024))) uint8_t smem[PNX * PSTAGE + NWS * PNW * PSTAGE + PNR * RAWB + RHO];
    uint8_t *const sx = smem;
    uint8_t *const sw = smem + PNX * PSTAGE;               // hi parts of the decoded W (Q8_0: codes)
    uint8_t *const swl = smem + (PNX + PNW) * PSTAGE;      // lo parts (K-quants)
    uint8_t *const sr = smem + (PNX + NWS * PNW) * PSTAGE;
    float *const srho = reinterpret_cast<float *>(sr + PNR * RAWB);  // [PNW + 1][256]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;  // 2 x 4 waves of 128 x 64

    // Consecutive workgroup ids land on different XCDs (round robin over 8);
    // give each XCD a contiguous run of tiles, which walks the m tiles of
    // one n tile, so the W rows and X slabs it shares stay in its L2.
    const int mt = (M + PBM - 1) / PBM, nt = (N + PBN - 1) / PBN, ntiles = mt * nt;
    const int xcd = blockIdx.x % 8, q = ntiles / 8, rem = ntiles % 8;
    const int t = xcd * q + min(xcd, rem) + (int)blockIdx.x / 8;
    const int n_tile = t / mt, m_tile = t % mt;
    const int m0 = m_tile * PBM, n0 = n_tile * PBN;
    // this workgroup's slabs [sb, se)
    const int sb = blockIdx.y * slabs_per_split;
    const int se = min(K / PBK, sb + slabs_per_split);

    // X: load j of this wave fills slots (4*wave + j)*64 + lane of a stage;
    // byte offsets from row m0 (rows past M re-read row M-1, results dropped)
    const int wv = __builtin_amdgcn_readfirstlane(wave);  // known uniform
    uint32_t ox[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int p = (2 * wv + j) * 64 + lane, row = p >> 2;
        const int c = (p & 3) ^ ((row >> 2) & 3);
        ox[j] = (uint32_t)(((int64_t)(min(m0 + row, M - 1) - m0) * K + 8 * c) * 2);
    }
    const uint8_t *const xbase = reinterpret_cast<const uint8_t *>(X + (int64_t)m0 * K);
    // W: the row this lane loads for (row 64*wave + lane; Q8_0 codes: two
    // lanes per row), clamped to N-1 (results dropped), relative to row n0
    const int rl = (int)(min((int64_t)n0 + 64 * wv + lane, (int64_t)N - 1) - n0);
    const int rq = (int)(min((int64_t)n0 + 64 * wv + (lane >> 1), (int64_t)N - 1) - n0);
    const int rq1 = (int)(min((int64_t)n0 + 64 * wv + 32 + (lane >> 1), (int64_t)N - 1) - n0);
    const int64_t g0 = (int64_t)n0 * (K / 256);  // first group of row n0 (K-quants)

    auto issue = [&](int s) {
        const uint32_t xs = lds_addr(sx + (s % PNX) * PSTAGE) + 2048 * wv;
#pragma unroll
        for (int j = 0; j < 2; j++)
            dma16(xbase + 2 * PBK * s, ox[j], xs + 1024 * j);
        if (wv >= 4)
            return;  // the raw W bytes: waves 0..3
        const uint32_t rs = lds_addr(sr + (s % PNR) * RAWB);
        if constexpr (FMT == FMT_Q8_0) {
            const uint32_t half = lane & 1;
            const uint8_t *cb = B + (int64_t)n0 * K + 32 * s;
            dma16(cb, (uint32_t)rq * K + 16 * half, rs + 2048 * wv);
            dma16(cb, (uint32_t)rq1 * K + 16 * half, rs + 2048 * wv + 1024);
            dma4(B + sc_off + 2 * (int64_t)n0 * (K / 32) + 4 * (s >> 1), (uint32_t)rl * (K / 16), rs + 8192 + 256 * wv);
        } else if constexpr (FMT == FMT_Q4K) {
            dma16(B + 16 * ((int64_t)n0 * (K / 32) + s), (uint32_t)rl * (K / 2), rs + 1024 * wv);
            dma16(B + sc_off + 16 * (g0 + (s >> 3)), (uint32_t)rl * (K / 16), rs + 4096 + 1024 * wv);
        } else {
            const int cc = s & 7;
            const uint8_t *gb = B + 192 * (g0 + (s >> 3));
            const uint32_t og = (uint32_t)rl * (K / 256) * 192;
            dma16(gb + 16 * cc, og, rs + 1024 * wv);
            dma16(gb + 128 + 16 * (cc >> 1), og, rs + 4096 + 1024 * wv);
            dma4(B + sc_off + 16 * (g0 + (s >> 3)) + 4 * (cc >> 1), (uint32_t)rl * (K / 16), rs + 8192 + 256 * wv);
            // the d dword holding group grp: 4*(grp >> 1) from the d plane,
            // counted from the dword holding group g0
            const int64_t grp = g0 + (int64_t)rl * (K / 256) + (s >> 3);
            dma4(B + d_off + 4 * (g0 >> 1), (uint32_t)(4 * ((grp >> 1) - (g0 >> 1))), rs + 9216 + 256 * wv);
        }
    };
    // row tid of slab s: raw bytes -> bf16 W stage, in two parts (the LDS
    // reads, then the arithmetic and the stores) so the reads can be issued
    // early
    const int64_t nd = min((int64_t)n0 + tid, (int64_t)N - 1);
    auto raw_of = [&](int s) {
        const uint8_t *rs = sr + (s % PNR) * RAWB;
        WBlk<FMT> w;
        if constexpr (FMT == FMT_Q8_0) {
            w.c0 = *reinterpret_cast<const uint4 *>(rs + 32 * tid);
            w.c1 = *reinterpret_cast<const uint4 *>(rs + 32 * tid + 16);
            w.d = *reinterpret_cast<const uint32_t *>(rs + 8192 + 4 * tid);
        } else if constexpr (FMT == FMT_Q4K) {
            w.c = *reinterpret_cast<const uint4 *>(rs + 16 * tid);
            w.h = *reinterpret_cast<const uint4 *>(rs + 4096 + 16 * tid);
        } else {
            w.lo = *reinterpret_cast<const uint4 *>(rs + 16 * tid);
            const uint4 h = *reinterpret_cast<const uint4 *>(rs + 4096 + 16 * tid);
            w.hi = ((s & 7) & 1) ? make_uint2(h.z, h.w) : make_uint2(h.x, h.y);
            w.sc2 = *reinterpret_cast<const uint32_t *>(rs + 8192 + 4 * tid);
            w.d = *reinterpret_cast<const uint32_t *>(rs + 9216 + 4 * tid);
        }
        return w;
    };
    // Q8_0 running scale of row tid: the block scale of the latest slab that
    // has one (a block of zeros, d = 0, keeps the previous scale)
    float e_run = 1.0f;
    auto decode = [&](int s, WBlk<FMT> w) {
        // pick the 16-bit halves out of the dwords the loads brought
        if constexpr (FMT == FMT_Q8_0) {
            w.d = (s & 1) ? w.d >> 16 : w.d & 0xffffu;
        } else if constexpr (FMT == FMT_Q6K) {
            w.sc2 = ((s & 7) & 1) ? w.sc2 >> 16 : w.sc2 & 0xffffu;
            const int64_t grp = nd * (K / 256) + (s >> 3);
            w.d = (grp & 1) ? w.d >> 16 : w.d & 0xffffu;
        }
        uint8_t *wh = sw + (s % PNW) * PSTAGE, *wl = swl + (s % PNW) * PSTAGE;
        if constexpr (CODE) {
            // the 32 codes as bf16 (exact), and the factor that takes the
            // accumulators from the previous slab's scale to this one's
            const uint32_t v[8] = {w.c0.x, w.c0.y, w.c0.z, w.c0.w, w.c1.x, w.c1.y, w.c1.z, w.c1.w};
            uint32_t vh[16];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                vh[2 * i] = pack_bf16((float)(int8_t)(v[i]), (float)(int8_t)(v[i] >> 8));
                vh[2 * i + 1] = pack_bf16((float)(int8_t)(v[i] >> 16), (float)(int8_t)(v[i] >> 24));
            }
#pragma unroll
            for (int c = 0; c < 4; c++)
                *reinterpret_cast<uint4 *>(wh + 16 * pslot(tid, c)) = make_uint4(vh[4 * c], vh[4 * c + 1], vh[4 * c + 2], vh[4 * c + 3]);
            const float dn = h2f(w.d);
            const float en = dn != 0.0f ? dn : e_run;
            srho[(s % PNW) * 256 + tid] = e_run / en;  // IEEE division
            e_run = en;
        } else {
            uint32_t vh[16], vl[16];
            decode_wblk<FMT>(w, s, vh, vl);
#pragma unroll
            for (int c = 0; c < 4; c++) {
                *reinterpret_cast<uint4 *>(wh + 16 * pslot(tid, c)) = make_uint4(vh[4 * c], vh[4 * c + 1], vh[4 * c + 2], vh[4 * c + 3]);
                *reinterpret_cast<uint4 *>(wl + 16 * pslot(tid, c)) = make_uint4(vl[4 * c], vl[4 * c + 1], vl[4 * c + 2], vl[4 * c + 3]);
            }
        }
    };

    const int r32 = lane & 31, kh = lane >> 5;
    int offa[4][2], offb[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; kk++) {
#pragma unroll
        for (int i = 0; i < 4; i++)
            offa[i][kk] = 16 * pslot(128 * wm + 32 * i + r32, 2 * kk + kh);
#pragma unroll
        for (int j = 0; j < 2; j++)
            offb[j][kk] = 16 * pslot(64 * wn + 32 * j + r32, 2 * kk + kh);
    }
    // Q8_0: rescale factors of the lane's two columns for the next slab
    float rho[2] = {1.0f, 1.0f};
    auto frags = [&](int s, int kk, bf16x8_t (&af)[4], bf16x8_t (&bw)[4]) {
        const uint8_t *xs = sx + (s % PNX) * PSTAGE, *ws = sw + (s % PNW) * PSTAGE, *wl = swl + (s % PNW) * PSTAGE;
#pragma unroll
        for (int i = 0; i < 4; i++)
            af[i] = *reinterpret_cast<const bf16x8_t *>(xs + offa[i][kk]);
#pragma unroll
        for (int j = 0; j < 2; j++) {
            bw[j] = *reinterpret_cast<const bf16x8_t *>(ws + offb[j][kk]);
            if constexpr (!CODE)
                bw[2 + j] = *reinterpret_cast<const bf16x8_t *>(wl + offb[j][kk]);
        }
        if constexpr (CODE) {
            if (kk == 0) {
#pragma unroll
                for (int j = 0; j < 2; j++)
                    rho[j] = srho[(s % PNW) * 256 + 64 * wn + 32 * j + r32];
            }
        }
    };
    // one output tile's k-step: Q8_0 one MFMA on the codes, the K-quants two
    // (hi and lo parts of the weights)
    auto mfma = [&](f32x16_t &c, const bf16x8_t &a, const bf16x8_t (&bw)[4], int j) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bw[j], c, 0, 0, 0);
        if constexpr (!CODE)
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bw[2 + j], c, 0, 0, 0);
    };
    // Q8_0: the accumulators of a tile, from the previous slab's scale to this slab's
    auto rescale = [&](f32x16_t &c, int j) {
        if constexpr (CODE) {
#pragma unroll
            for (int r = 0; r < 16; r++)
                c[r] *= rho[j];
        }
    };

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
            acc[i][j] = f32x16_t{};

    // prologue: slabs sb..sb+2 landed and the W of slab sb decoded; slab
    // sb+3 goes out only then, since its raw W takes the stage of slab sb
    for (int s = sb; s < sb + PNR && s < se; s++)
        issue(s);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt 0, lgkmcnt 0
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (wv < 4)
        decode(sb, raw_of(sb));
    lds_barrier();
    if (sb + PNR < se)
        issue(sb + PNR);
    bf16x8_t a0[4], b0[4], a1[4], b1[4];  // b: hi parts of the two n tiles, then lo parts
    frags(sb, 0, a0, b0);

    // Slab s.  Steady state (s + 4 < se): the loads of slab s+4 go out
    // after the barrier.  The barrier needs X of slab s+1 and the raw W of
    // slab s+2: both came with the loads issued two slabs ago, so one slab's
    // loads may remain (waves 0..3: 2 of X + WD of raw W; waves 4..7: 2).
    constexpr int VMD = 2 + PRaw<FMT>::wd, VMX = 2;
    static_assert(VMD < 16, "vmcnt immediate");
    auto body = [&](int s, auto steady, auto decoder) {
        constexpr bool ST = decltype(steady)::value, DEC = decltype(decoder)::value;
        const bool dec = ST || s + 1 < se;
        rescale(acc[0][0], 0);
        mfma(acc[0][0], a0[0], b0, 0);
        __builtin_amdgcn_sched_barrier(0);
        WBlk<FMT> w{};
        if (DEC && dec)
            w = raw_of(s + 1);
        frags(s, 1, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        if (DEC && dec)
            decode(s + 1, w);
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
                if (i + j > 0) {
                    rescale(acc[i][j], j);
                    mfma(acc[i][j], a0[i], b0, j);
                }
        if constexpr (CODE) {
            // Q8_0: each MFMA of this k-step follows the 16 multiplies that
            // rescale its tile, so that one tile's MFMA runs while the next
            // tile is rescaled; the decoding waves add a share of the next
            // slab's decode to each group
#pragma unroll
            for (int q = 0; q < 7; q++) {
                __builtin_amdgcn_sched_group_barrier(0x002, 16 + (DEC ? PRaw<FMT>::vpm : 0), 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            if constexpr (DEC)
                __builtin_amdgcn_sched_group_barrier(0x200, 4, 0);
        } else if constexpr (DEC) {
            // MFMAs of this k-step after the first, each followed by a share
            // of the next slab's decode
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
#pragma unroll
            for (int q = 0; q < 14; q++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, PRaw<FMT>::vpm, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x200, 8, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if constexpr (ST)
            __builtin_amdgcn_s_waitcnt(0x0070 | (DEC ? VMD : VMX));
        else
            __builtin_amdgcn_s_waitcnt(0x0070);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if constexpr (ST)
            issue(s + PAHEAD);
        frags(s + 1, 0, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
                mfma(acc[i][j], a1[i], b1, j);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto run = [&](auto decoder) {
        int s = sb;
        for (; s + PAHEAD < se; s++)
            body(s, std::true_type{}, decoder);
        for (; s < se; s++)
            body(s, std::false_type{}, decoder);
    };
    if (wv < 4)
        run(std::true_type{});
    else
        run(std::false_type{});

    // Q8_0: the accumulators hold the sums in units of the last slab's
    // scale of each row; multiply it back
    float eout[2] = {1.0f, 1.0f};
    if constexpr (CODE) {
        if (wv < 4)
            srho[PNW * 256 + tid] = e_run;
        lds_barrier();
#pragma unroll
        for (int j = 0; j < 2; j++)
            eout[j] = srho[PNW * 256 + 64 * wn + 32 * j + r32];
    }

    // lane holds D[m = 8*(r/4) + 4*(lane/32) + r%4][n = lane%32] of each tile
    const bool split = gridDim.y > 1;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int n = n0 + 64 * wn + 32 * j + r32;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = m0 + 128 * wm + 32 * i + 8 * (r / 4) + 4 * kh + (r % 4);
                const float v = CODE ? acc[i][j][r] * eout[j] : acc[i][j][r];
                if (m < M && n < N) {
                    if (split)
                        atomicAdd(Y + (int64_t)m * N + n, v);
                    else
                        Y[(int64_t)m * N + n] = v;
                }
            }
        }
}

// ---------------------------------------------------------------------------
// Batched-decode path (a few to 32 tokens): a weight stream.  A workgroup of
// four waves owns 64 rows of W and one split of K; wave w owns rows
// 16w..16w+15 and all 16*TM rows of X, so no weight is decoded twice.  K
// advances in slabs of 128 (four blocks of 32 per row).
//
//   * X and the raw block bytes of the 64 rows reach LDS by direct
//     global->LDS loads into a ring of four stages, three slabs ahead; the
//     only waits on them are the explicit vmcnt waits.
//   * Lane (g = lane/16, r = lane%16) decodes block g of the slab in row
//     16w + r straight into the four B fragments of the slab's four
//     v_mfma_f32_16x16x32_bf16 steps; step t pairs elements 8t..8t+7 of that
//     block with X[m][32g + 8t + e] -- the k order inside the slab is
//     permuted identically on both operands.
//   * X stage: row m holds the slab's 16 chunks of 8 elements, chunk c at
//     position c ^ (m & 15), so the 16 rows a ds_read_b128 phase touches
//     land on distinct banks.
//   * K splits add their partial tiles into Y (zeroed first) with fp32
//     atomics.
// ---------------------------------------------------------------------------
constexpr int TBN = 64, TBK = 128, TNS = 4;

// raw bytes of one slab of 64 rows in LDS, and the direct loads per wave (WD):
//   Q8_0: codes [64][128] at 0; scales [64][8] at 8192
//   Q4K:  codes [64][64] at 0; group headers [64][16] at 4096
//   Q6K:  low nibbles [64][64] at 0; high bits [64][32] at 4096; sub-scales
//         [64][8] at 6144; the dword holding d, [64][4] at 6656
template <int FMT> struct TRaw;
template <> struct TRaw<FMT_Q8_0> { static constexpr int bytes = 8704, wd = 3; };
template <> struct TRaw<FMT_Q4K> { static constexpr int bytes = 5120, wd = 2; };
template <> struct TRaw<FMT_Q6K> { static constexpr int bytes = 6912, wd = 4; };

template <int FMT, int TM>
__global__ __launch_bounds__(256) void gemm_bt_kernel(const uint8_t *__restrict__ B, int64_t sc_off, int64_t d_off,
                                                      const uint16_t *__restrict__ X, float *__restrict__ Y, int M,
                                                      int N, int K, int slabs_per_split)
{
    constexpr int XSTG = 16 * TM * TBK * 2;  // bytes of one X stage
    constexpr int RAWB = TRaw<FMT>::bytes;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[TNS * (XSTG + RAWB)];
    uint8_t *const sx = smem;
    uint8_t *const sr = smem + TNS * XSTG;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int g = lane >> 4, r16 = lane & 15;
    const int n0 = blockIdx.x * TBN, m0 = blockIdx.y * 16 * TM;
    const int sb = blockIdx.z * slabs_per_split;
    const int se = min(K / TBK, sb + slabs_per_split);

    // X: load j of wave w fills slots (4j + w)*64 + lane: row p/16, position
    // p%16 holding chunk (p%16) ^ (row & 15); offsets from row m0
    uint32_t ox[TM];
#pragma unroll
    for (int j = 0; j < TM; j++) {
        const int p = (4 * j + wv) * 64 + lane, row = p >> 4;
        const int c = (p & 15) ^ (row & 15);
        ox[j] = (uint32_t)(((int64_t)(min(m0 + row, M - 1) - m0) * K + 8 * c) * 2);
    }
    const uint8_t *const xbase = reinterpret_cast<const uint8_t *>(X + (int64_t)m0 * K);
    const int64_t g0 = (int64_t)n0 * (K / 256);
    auto rn = [&](int row) { return (uint32_t)(min(n0 + row, N - 1) - n0); };  // rows past N: results dropped

    auto issue = [&](int s) {
        const uint32_t xs = lds_addr(sx + (s % TNS) * XSTG);
#pragma unroll
        for (int j = 0; j < TM; j++)
            dma16(xbase + 2 * TBK * s, ox[j], xs + (4 * j + wv) * 1024);
        const uint32_t rs = lds_addr(sr + (s % TNS) * RAWB);
        if constexpr (FMT == FMT_Q8_0) {
            const uint8_t *cb = B + (int64_t)n0 * K + TBK * s;
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int p = (2 * wv + j) * 64 + lane;
                dma16(cb, rn(p >> 3) * K + 16 * (p & 7), rs + (2 * wv + j) * 1024);
            }
            const int q = 32 * wv + lane;
            if (lane < 32)
                dma4(B + sc_off + (int64_t)n0 * (K / 16) + 8 * s, rn(q >> 1) * (K / 16) + 4 * (q & 1),
                     rs + 8192 + 128 * wv);
        } else if constexpr (FMT == FMT_Q4K) {
            const int p = 64 * wv + lane;
            dma16(B + (int64_t)n0 * (K / 2) + 64 * s, rn(p >> 2) * (K / 2) + 16 * (p & 3), rs + 1024 * wv);
            if (lane < 16)
                dma16(B + sc_off + 16 * (g0 + (s >> 1)), rn(16 * wv + lane) * (K / 16), rs + 4096 + 256 * wv);
        } else {
            const int cc0 = 4 * (s & 1);
            const uint8_t *gb = B + 192 * (g0 + (s >> 1));
            const int p = 64 * wv + lane;
            dma16(gb + 16 * cc0, rn(p >> 2) * (K / 256) * 192 + 16 * (p & 3), rs + 1024 * wv);
            const int q = 32 * wv + lane;
            if (lane < 32) {
                dma16(gb + 128 + 8 * cc0, rn(q >> 1) * (K / 256) * 192 + 16 * (q & 1), rs + 4096 + 512 * wv);
                dma4(B + sc_off + 16 * (g0 + (s >> 1)) + 2 * cc0, rn(q >> 1) * (K / 16) + 4 * (q & 1),
                     rs + 6144 + 128 * wv);
            }
            if (lane < 16) {
                // the d dword of group grp, counted from the dword holding g
                const int64_t gs = g0 + (s >> 1);
                const int64_t grp = gs + (int64_t)rn(16 * wv + lane) * (K / 256);
                dma4(B + d_off + 4 * (gs >> 1), (uint32_t)(4 * ((grp >> 1) - (gs >> 1))), rs + 6656 + 64 * wv);
            }
        }
    };

    const int row = 16 * wv + r16;  // the W row this lane decodes
    const int64_t nd = min(n0 + row, N - 1);
    auto decode = [&](int s, uint32_t (&vh)[16], uint32_t (&vl)[16]) {
        const uint8_t *rs = sr + (s % TNS) * RAWB;
        WBlk<FMT> w;
        if constexpr (FMT == FMT_Q8_0) {
            w.c0 = *reinterpret_cast<const uint4 *>(rs + 128 * row + 32 * g);
            w.c1 = *reinterpret_cast<const uint4 *>(rs + 128 * row + 32 * g + 16);
            w.d = *reinterpret_cast<const uint16_t *>(rs + 8192 + 8 * row + 2 * g);
        } else if constexpr (FMT == FMT_Q4K) {
            w.c = *reinterpret_cast<const uint4 *>(rs + 64 * row + 16 * g);
            w.h = *reinterpret_cast<const uint4 *>(rs + 4096 + 16 * row);
        } else {
            w.lo = *reinterpret_cast<const uint4 *>(rs + 64 * row + 16 * g);
            w.hi = *reinterpret_cast<const uint2 *>(rs + 4096 + 32 * row + 8 * g);
            w.sc2 = *reinterpret_cast<const uint16_t *>(rs + 6144 + 8 * row + 2 * g);
            const uint32_t dd = *reinterpret_cast<const uint32_t *>(rs + 6656 + 4 * row);
            const int64_t grp = nd * (K / 256) + (s >> 1);
            w.d = (grp & 1) ? dd >> 16 : dd & 0xffffu;
        }
        decode_wblk<FMT>(w, 4 * s + g, vh, vl);
    };

    f32x4_t acc[TM];
#pragma unroll
    for (int j = 0; j < TM; j++)
        acc[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    for (int s = sb; s < sb + TNS - 1 && s < se; s++)
        issue(s);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt 0, lgkmcnt 0
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);

    // at the end of slab s the next slab must have landed: the loads of
    // slab s+2 (TM + WD per wave) may remain in flight
    constexpr int VM = TM + TRaw<FMT>::wd;
    static_assert(VM < 16, "vmcnt immediate");
    auto body = [&](int s, auto steady) {
        constexpr bool ST = decltype(steady)::value;
        uint32_t vh[16], vl[16];
        decode(s, vh, vl);
        const uint8_t *xs = sx + (s % TNS) * XSTG;
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, make_uint4(vh[4 * t], vh[4 * t + 1], vh[4 * t + 2], vh[4 * t + 3]));
            const bf16x8_t bl = __builtin_bit_cast(bf16x8_t, make_uint4(vl[4 * t], vl[4 * t + 1], vl[4 * t + 2], vl[4 * t + 3]));
#pragma unroll
            for (int j = 0; j < TM; j++) {
                const int xr = 16 * j + r16;
                const bf16x8_t xa = *reinterpret_cast<const bf16x8_t *>(xs + 256 * xr + 16 * ((4 * g + t) ^ r16));
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bh, acc[j], 0, 0, 0);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bl, acc[j], 0, 0, 0);
            }
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if constexpr (ST)
            __builtin_amdgcn_s_waitcnt(0x0070 | VM);  // vmcnt VM, lgkmcnt 0
        else
            __builtin_amdgcn_s_waitcnt(0x0070);       // vmcnt 0, lgkmcnt 0
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if constexpr (ST)
            issue(s + TNS - 1);
    };
    int s = sb;
    for (; s + TNS - 1 < se; s++)
        body(s, std::true_type{});
    for (; s < se; s++)
        body(s, std::false_type{});

    // lane holds D[m = 4g + i][n = r16] of each 16 x 16 tile
    const bool split = gridDim.z > 1;
    const int n = n0 + row;
    if (n < N) {
#pragma unroll
        for (int j = 0; j < TM; j++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int m = m0 + 16 * j + 4 * g + i;
                if (m < M) {
                    if (split)
                        atomicAdd(Y + (int64_t)m * N + n, acc[j][i]);
                    else
                        Y[(int64_t)m * N + n] = acc[j][i];
                }
            }
    }
}

// ---------------------------------------------------------------------------
// Q4K batched decode with exact codes (a few to 32 tokens).  The structure of
// gemm_bt_kernel -- four waves of 16 rows of W, X and the raw blocks staged
// by direct loads in a ring of four slabs of 128 -- but the matrix cores see
// the 4-bit codes u themselves, which bf16 holds exactly, and each 32-element
// sub-block's scale and min are applied to its partial sums:
//   y += S sum_k x u - Mn sum_k x,   S = d sc, Mn = dmin m (exact in fp32),
// one v_mfma_f32_16x16x32_bf16 on the codes and one on ones (the sums of X)
// per sub-block and 16-token tile.  Products are exact and only fp32 sums
// round.  MFMA t of a slab covers sub-block t: lane (g, r) gives elements
// 8g..8g+7 of it for row r.
//   * Codes: a nibble 0..15 read as an E4M3 byte is the value u 2^-9, so
//     v_cvt_scalef32_pk_bf16_fp8 with scale 2^9 turns two of them into a
//     bf16 pair exactly; a byte permute first puts the nibbles of elements
//     (0, 1, 4, 5) and (2, 3, 6, 7) in the bytes of two dwords.
//   * Raw codes in LDS: sub-block c of row r at slot 4r + (c ^ ((r >> 2) & 3))
//     (16-byte slots), so the dword reads of one sub-block by 64 lanes fall
//     in distinct banks.
// ---------------------------------------------------------------------------
template <int TM>
__global__ __launch_bounds__(256) void gemm_bx_kernel(const uint8_t *__restrict__ B, int64_t sc_off,
                                                      const uint16_t *__restrict__ X, float *__restrict__ Y, int M,
                                                      int N, int K, int slabs_per_split)
{
    constexpr int XSTG = 16 * TM * TBK * 2;  // bytes of one X stage
    constexpr int RAWB = TRaw<FMT_Q4K>::bytes;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[TNS * (XSTG + RAWB)];
    uint8_t *const sx = smem;
    uint8_t *const sr = smem + TNS * XSTG;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int g = lane >> 4, r16 = lane & 15;
    const int n0 = blockIdx.x * TBN, m0 = blockIdx.y * 16 * TM;
    const int sb = blockIdx.z * slabs_per_split;
    const int se = min(K / TBK, sb + slabs_per_split);

    // X: as in gemm_bt_kernel (row m of a stage: chunk c of 8 elements at c ^ (m & 15))
    uint32_t ox[TM];
#pragma unroll
    for (int j = 0; j < TM; j++) {
        const int p = (4 * j + wv) * 64 + lane, row = p >> 4;
        const int c = (p & 15) ^ (row & 15);
        ox[j] = (uint32_t)(((int64_t)(min(m0 + row, M - 1) - m0) * K + 8 * c) * 2);
    }
    const uint8_t *const xbase = reinterpret_cast<const uint8_t *>(X + (int64_t)m0 * K);
    const int64_t g0 = (int64_t)n0 * (K / 256);
    auto rn = [&](int row) { return (uint32_t)(min(n0 + row, N - 1) - n0); };  // rows past N: results dropped
    // W codes: lane p of wave wv fills slot 64 wv + p of the codes region with
    // sub-block c of row r, where slot = 4r + (c ^ ((r >> 2) & 3))
    const int wslot = 64 * wv + lane, wrow = wslot >> 2, wsub = (wslot & 3) ^ ((wrow >> 2) & 3);
    const uint32_t ocode = rn(wrow) * (uint32_t)(K / 2) + 16 * wsub;

    auto issue = [&](int s) {
        const uint32_t xs = lds_addr(sx + (s % TNS) * XSTG);
#pragma unroll
        for (int j = 0; j < TM; j++)
            dma16(xbase + 2 * TBK * s, ox[j], xs + (4 * j + wv) * 1024);
        const uint32_t rs = lds_addr(sr + (s % TNS) * RAWB);
        dma16(B + (int64_t)n0 * (K / 2) + 64 * s, ocode, rs + 1024 * wv);
        if (lane < 16)
            dma16(B + sc_off + 16 * (g0 + (s >> 1)), rn(16 * wv + lane) * (K / 16), rs + 4096 + 256 * wv);
    };

    const int row = 16 * wv + r16;  // the W row this lane decodes
    typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
    auto pair = [](uint32_t w, bool h) {
        return h ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 512.0f, true))
                 : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 512.0f, false));
    };
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));

    f32x4_t acc[TM];
#pragma unroll
    for (int j = 0; j < TM; j++)
        acc[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    for (int s = sb; s < sb + TNS - 1 && s < se; s++)
        issue(s);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt 0, lgkmcnt 0
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);

    constexpr int VM = TM + TRaw<FMT_Q4K>::wd;
    static_assert(VM < 16, "vmcnt immediate");
    auto body = [&](int s, auto steady) {
        constexpr bool ST = decltype(steady)::value;
        const uint8_t *rs = sr + (s % TNS) * RAWB;
        const uint8_t *xs = sx + (s % TNS) * XSTG;
        const uint4 h = *reinterpret_cast<const uint4 *>(rs + 4096 + 16 * row);
        const float d = h2f(h.x), dmin = h2f(h.x >> 16);
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 4; t++)
            w[t] = *reinterpret_cast<const uint32_t *>(rs + 16 * (4 * row + (t ^ ((row >> 2) & 3))) + 4 * g);
#pragma unroll
        for (int t = 0; t < 4; t++) {
            // sub-block j of the group: its 6-bit scale and min
            const int j = 4 * (s & 1) + t;
            const uint32_t sc = __builtin_amdgcn_ubfe(h.y, 4 * j, 4) | (__builtin_amdgcn_ubfe(h.w, 2 * j, 2) << 4);
            const uint32_t mq = __builtin_amdgcn_ubfe(h.z, 4 * j, 4) | (__builtin_amdgcn_ubfe(h.w, 16 + 2 * j, 2) << 4);
            const float S = d * (float)sc, Mn = dmin * (float)mq;
            // nibbles of elements (0,1,4,5) and (2,3,6,7): bytes 0, 2, 1, 3 of the dword
            const uint32_t P = __builtin_amdgcn_perm(w[t], w[t], 0x03010200u);
            const uint32_t lo = P & 0x0F0F0F0Fu, hi = (P >> 4) & 0x0F0F0F0Fu;
            const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, make_uint4(pair(lo, false), pair(hi, false),
                                                                        pair(lo, true), pair(hi, true)));
#pragma unroll
            for (int m = 0; m < TM; m++) {
                const int xr = 16 * m + r16;
                const bf16x8_t xa = *reinterpret_cast<const bf16x8_t *>(xs + 256 * xr + 16 * ((4 * t + g) ^ r16));
                const f32x4_t D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bw, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                const f32x4_t T = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, ones, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; i++)
                    acc[m][i] = fmaf(-Mn, T[i], fmaf(S, D[i], acc[m][i]));
            }
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if constexpr (ST)
            __builtin_amdgcn_s_waitcnt(0x0070 | VM);  // vmcnt VM, lgkmcnt 0
        else
            __builtin_amdgcn_s_waitcnt(0x0070);       // vmcnt 0, lgkmcnt 0
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if constexpr (ST)
            issue(s + TNS - 1);
    };
    int s = sb;
    for (; s + TNS - 1 < se; s++)
        body(s, std::true_type{});
    for (; s < se; s++)
        body(s, std::false_type{});

    // lane holds D[m = 4g + i][n = r16] of each 16 x 16 tile
    const bool split = gridDim.z > 1;
    const int n = n0 + row;
    if (n < N) {
#pragma unroll
        for (int j = 0; j < TM; j++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int m = m0 + 16 * j + 4 * g + i;
                if (m < M) {
                    if (split)
                        atomicAdd(Y + (int64_t)m * N + n, acc[j][i]);
                    else
                        Y[(int64_t)m * N + n] = acc[j][i];
                }
            }
    }
}

// ---------------------------------------------------------------------------
// Q4K batched decode in one pass (up to 16 tokens).  A workgroup owns 16 rows
// of W and all of K; its KW waves split K by 256-element groups (wave w:
// groups [w G / KW, (w + 1) G / KW)) and add their partial results through
// LDS at the end -- no K split across workgroups, hence no atomics and no
// zero-fill launch.  Nothing is staged in LDS and the loop has no barrier:
// each wave loads its weight blocks and its X straight into registers, DG
// groups ahead, already in the layout of the v_mfma_f32_16x16x32_bf16
// operands (all loads of a wave are register loads, so the compiler's
// in-order vmcnt waits are exact).  DG = 1 measured fastest: 1 / 4 / 16
// tokens at 4096 x 14336 ran 13.2 / 14.5 / 20.9 us with one group in
// flight per wave, 13.5 / 15.2 / 20.9 with two, 15.4 / 17.6 / 22.3 with
// four -- the kernel is bound by its VALU work and by the L2 reads of X
// (every workgroup reads all of X), not by load latency.
//   * B (W): lane (g, r) loads sub-block 4h + g of row r (its four octets)
//     for each half h of a group; a 4 x 4 transpose across the four 16-lane
//     rows (v_permlane32_swap, then v_permlane16_swap) leaves in dword t
//     octet g of sub-block 4h + t: the lane's 8 elements of MFMA t.
//   * A (X): lane (g, r) loads elements 8g..8g+7 of each sub-block for
//     token r (tokens past M re-read token M - 1; their outputs are not
//     stored).
// The codes enter the MFMA exactly (as in gemm_bx_kernel); per sub-block j,
// D = MFMA(x, u) is added as acc += S_j D, while MFMA(x, m_j), whose B holds
// the 6-bit min code m_j at every k, accumulates sum_j m_j sum_k x over the
// group, subtracted once per group as acc -= dmin * that.  Products are
// exact and only fp32 sums round.
// ---------------------------------------------------------------------------
template <int KW, int DG>
__global__ __launch_bounds__(64 * KW) void gemm_bs_kernel(const uint8_t *__restrict__ B, int64_t sc_off,
                                                           const uint16_t *__restrict__ X, float *__restrict__ Y,
                                                           int M, int N, int K)
{
    __shared__ f32x4_t red[KW - 1][64];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int g = lane >> 4, r = lane & 15;
    const int n0 = blockIdx.x * 16;
    const int G = K / 256, S = K / 32;
    const int gb = wv * G / KW, ng = (wv + 1) * G / KW - gb;
    const int64_t row = min(n0 + r, N - 1);  // rows past N: results dropped
    const int tok = min(r, M - 1);
    const uint8_t *const wp = B + 16 * (row * S + 8 * gb + g);
    const uint8_t *const hp = B + sc_off + 16 * (row * G + gb);
    const uint16_t *const xp = X + (int64_t)tok * K + 256 * gb + 8 * g;

    struct Stage {
        uint4 w[2];  // sub-blocks g and 4 + g of the group
        uint4 h;     // the group header of row r
        uint4 x[8];  // elements 8g..8g+7 of each sub-block, token r
    };
    Stage st[DG];
    auto issue = [&](Stage &q, int i) {
        q.w[0] = ld_nt16(wp + 128 * i);
        q.w[1] = ld_nt16(wp + 128 * i + 64);
        q.h = *reinterpret_cast<const uint4 *>(hp + 16 * i);
#pragma unroll
        for (int j = 0; j < 8; j++)
            q.x[j] = *reinterpret_cast<const uint4 *>(xp + 256 * i + 32 * j);
    };
    auto pair = [](uint32_t w, bool h) {
        return h ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 512.0f, true))
                 : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 512.0f, false));
    };
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    auto compute = [&](const Stage &q) {
        const float d = h2f(q.h.x), dmin = h2f(q.h.x >> 16);
        f32x4_t dm = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int h = 0; h < 2; h++) {
            uint32_t a0 = q.w[h].x, a1 = q.w[h].y, a2 = q.w[h].z, a3 = q.w[h].w;
            const auto p02 = __builtin_amdgcn_permlane32_swap(a0, a2, false, false);
            const auto p13 = __builtin_amdgcn_permlane32_swap(a1, a3, false, false);
            const auto q01 = __builtin_amdgcn_permlane16_swap(p02[0], p13[0], false, false);
            const auto q23 = __builtin_amdgcn_permlane16_swap(p02[1], p13[1], false, false);
            const uint32_t wt[4] = {q01[0], q01[1], q23[0], q23[1]};
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const int j = 4 * h + t;
                const uint32_t sc = __builtin_amdgcn_ubfe(q.h.y, 4 * j, 4) | (__builtin_amdgcn_ubfe(q.h.w, 2 * j, 2) << 4);
                const uint32_t mq = __builtin_amdgcn_ubfe(q.h.z, 4 * j, 4) | (__builtin_amdgcn_ubfe(q.h.w, 16 + 2 * j, 2) << 4);
                const float Sj = d * (float)sc;
                const uint32_t mb = __float_as_uint((float)mq) >> 16;  // bf16 of the integer m_j (exact)
                const uint32_t mm = mb | (mb << 16);
                const bf16x8_t bm = __builtin_bit_cast(bf16x8_t, make_uint4(mm, mm, mm, mm));
                // nibbles of elements (0,1,4,5) and (2,3,6,7): bytes 0, 2, 1, 3 of the dword
                const uint32_t P = __builtin_amdgcn_perm(wt[t], wt[t], 0x03010200u);
                const uint32_t lo = P & 0x0F0F0F0Fu, hi = (P >> 4) & 0x0F0F0F0Fu;
                const bf16x8_t bw = __builtin_bit_cast(bf16x8_t, make_uint4(pair(lo, false), pair(hi, false),
                                                                            pair(lo, true), pair(hi, true)));
                const bf16x8_t xa = __builtin_bit_cast(bf16x8_t, q.x[j]);
                const f32x4_t D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bw, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                dm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bm, dm, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; i++)
                    acc[i] = fmaf(Sj, D[i], acc[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; i++)
            acc[i] = fmaf(-dmin, dm[i], acc[i]);
    };

#pragma unroll
    for (int j = 0; j < DG; j++)
        if (j < ng)
            issue(st[j], j);
    for (int i0 = 0; i0 < ng; i0 += DG) {
#pragma unroll
        for (int j = 0; j < DG; j++) {
            const int i = i0 + j;
            if (i < ng) {
                compute(st[j]);
                if (i + DG < ng)
                    issue(st[j], i + DG);
            }
        }
    }

    // lane (g, r) holds tokens 4g..4g+3 of row r; wave 0 adds the others'
    if (wv > 0)
        red[wv - 1][lane] = acc;
    __syncthreads();
    if (wv == 0) {
#pragma unroll
        for (int w = 0; w < KW - 1; w++) {
            const f32x4_t o = red[w][lane];
#pragma unroll
            for (int i = 0; i < 4; i++)
                acc[i] += o[i];
        }
        const int n = n0 + r;
        if (n < N)
#pragma unroll
            for (int i = 0; i < 4; i++)
                if (4 * g + i < M)
                    Y[(int64_t)(4 * g + i) * N + n] = acc[i];
    }
}

// ---------------------------------------------------------------------------
// Generic MFMA GEMM (the formats without a tuned kernel): the structure of
// gemm_bf16_kernel -- X slabs of 128 staged in LDS once per
// workgroup and shared by its four waves, 16 TM tokens and 64 NT rows of W
// per workgroup -- with the weights decoded by the shared exact decoder
// (dequant8) straight from the blocks: lane (g, r) decodes block 4s + g of
// its rows in slab s into bf16 hi + lo pairs and feeds four pairs of
// v_mfma_f32_16x16x32_bf16 steps.  FP8 (W8A16) takes its E4M3 codes, exact
// in bf16, as one operand and multiplies the sums by the row scale at the
// end.  Each weight is decoded once per 16 TM tokens, and X is read once
// per workgroup rather than once per wave.
// ---------------------------------------------------------------------------
template <int FMT, int TM, int NT>
__global__ __launch_bounds__(256) void gemm_gen_lds_kernel(const uint8_t *__restrict__ B, Planes p,
                                                           const uint16_t *__restrict__ X, float *__restrict__ Y,
                                                           int M, int N, int K, int slabs_per_split)
{
    constexpr int BM = 16 * TM;
    constexpr int XPER = BM * SLAB * 2 / 16;  // uint4 of X per slab
    constexpr int XU4 = XPER / 256;           // per thread
    static_assert(XU4 * 256 == XPER, "X staging");
    __shared__ __attribute__((aligned(16))) uint8_t sX[2][BM * XPITCH];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const int64_t n_wave = (int64_t)blockIdx.x * (64 * NT) + wave * 16 * NT;
    const int m0 = blockIdx.y * BM;
    const int nslab = K / SLAB;
    const int s0 = blockIdx.z * slabs_per_split;
    const int s1 = min(nslab, s0 + slabs_per_split);
    if (s0 >= s1)
        return;
    int64_t wpiece[NT];  // first 8-element piece of this lane's rows (clamped: rows past N are not stored)
#pragma unroll
    for (int i = 0; i < NT; i++)
        wpiece[i] = min(n_wave + 16 * i + r16, (int64_t)N - 1) * (K / 8);

    auto load_x = [&](int s, uint4 (&xr)[XU4]) {
#pragma unroll
        for (int t = 0; t < XU4; t++) {
            const int i = tid + 256 * t;
            const int row = i / (SLAB / 8), q = i % (SLAB / 8);
            xr[t] = m0 + row < M ? *reinterpret_cast<const uint4 *>(X + (int64_t)(m0 + row) * K + s * SLAB + 8 * q)
                                 : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_x = [&](int buf, const uint4 (&xr)[XU4]) {
#pragma unroll
        for (int t = 0; t < XU4; t++) {
            const int i = tid + 256 * t;
            const int row = i / (SLAB / 8), q = i % (SLAB / 8);
            *reinterpret_cast<uint4 *>(&sX[buf][row * XPITCH + 16 * q]) = xr[t];
        }
    };

    f32x4_t acc[NT][TM];
#pragma unroll
    for (int i = 0; i < NT; i++)
#pragma unroll
        for (int j = 0; j < TM; j++)
            acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    uint4 x1[XU4];
    load_x(s0, x1);
    store_x(0, x1);
    if (s0 + 1 < s1)
        load_x(s0 + 1, x1);
    lds_barrier();
    for (int s = s0; s < s1; s++) {
        const int buf = (s - s0) & 1;
#pragma unroll
        for (int i = 0; i < NT; i++) {
#pragma unroll
            for (int t = 0; t < 4; t++) {
                if constexpr (FMT == FMT_FP8) {
                    // E4M3 codes are exact in bf16: one MFMA on the codes, the
                    // row scale applied to the sums at the end
                    const uint2 c = reinterpret_cast<const uint2 *>(B)[wpiece[i] + 16 * s + 4 * g + t];
                    const bf16x8_t bc = __builtin_bit_cast(
                        bf16x8_t, make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, false)),
                                             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, 1.0f, true)),
                                             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, false)),
                                             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, 1.0f, true))));
#pragma unroll
                    for (int j = 0; j < TM; j++) {
                        const bf16x8_t xa = *reinterpret_cast<const bf16x8_t *>(
                            &sX[buf][(16 * j + r16) * XPITCH + 64 * g + 16 * t]);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bc, acc[i][j], 0, 0, 0);
                    }
                } else {
                    float w[8];
                    dequant8<FMT>(B, p, wpiece[i] + 16 * s + 4 * g + t, w);
                    uint32_t h[4], l[4];
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        split_bf16(w[2 * e], w[2 * e + 1], h[e], l[e]);
                    const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
                    const bf16x8_t bl = __builtin_bit_cast(bf16x8_t, make_uint4(l[0], l[1], l[2], l[3]));
#pragma unroll
                    for (int j = 0; j < TM; j++) {
                        const bf16x8_t xa = *reinterpret_cast<const bf16x8_t *>(
                            &sX[buf][(16 * j + r16) * XPITCH + 64 * g + 16 * t]);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bh, acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, bl, acc[i][j], 0, 0, 0);
                    }
                }
            }
        }
        if (s + 1 < s1) {
            store_x(buf ^ 1, x1);
            if (s + 2 < s1)
                load_x(s + 2, x1);
        }
        lds_barrier();
    }

    // lane holds D[m = 4*g + r][n = r16] of each 16 x 16 tile
    const bool atomic = gridDim.z > 1;
#pragma unroll
    for (int i = 0; i < NT; i++) {
        const int64_t n = n_wave + 16 * i + r16;
        if constexpr (FMT == FMT_FP8) {
            const float sc = reinterpret_cast<const float *>(B + p.scales)[min(n, (int64_t)N - 1)];
#pragma unroll
            for (int j = 0; j < TM; j++)
#pragma unroll
                for (int r = 0; r < 4; r++)
                    acc[i][j][r] *= sc;
        }
        if (n >= N)
            continue;
#pragma unroll
        for (int j = 0; j < TM; j++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int m = m0 + 16 * j + 4 * g + r;
                if (m < M) {
                    float *y = Y + (int64_t)m * N + n;
                    if (atomic)
                        atomicAdd(y, acc[i][j][r]);
                    else
                        *y = acc[i][j][r];
                }
            }
    }
}

// ---------------------------------------------------------------------------
// Per-step generic MFMA GEMM (Q8_0 rows that end in a tail of blocks, and
// any row length that is not a whole number of 128-element slabs): a
// workgroup of four waves owns 64 rows of W (16 per wave) and 16*TM tokens;
// K advances in steps of 32.  Lane (g = l/16, r = l%16) decodes elements 8g..8g+7 of the
// step in row r of its wave exactly (dequant8), rounds them to bf16 and uses
// them as its B operand of v_mfma_f32_16x16x32_bf16; the A operand is the
// same 8 elements of X read straight from memory.  K splits over gridDim.z
// add into a zeroed Y with fp32 atomics.
// ---------------------------------------------------------------------------
template <int FMT, int TM>
__global__ __launch_bounds__(256) void gemm_gen_kernel(const uint8_t *__restrict__ B, Planes p,
                                                       const uint16_t *__restrict__ X, float *__restrict__ Y, int M,
                                                       int N, int K, int steps_per_split)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const int n = blockIdx.x * 64 + 16 * wv + r16;
    const int64_t nr = min(n, N - 1);  // rows past N are decoded but not stored
    const int m0 = blockIdx.y * 16 * TM;
    const int s0 = blockIdx.z * steps_per_split, s1 = min(K / 32, s0 + steps_per_split);
    f32x4_t acc[TM];
#pragma unroll
    for (int j = 0; j < TM; j++)
        acc[j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const uint16_t *xr[TM];
#pragma unroll
    for (int j = 0; j < TM; j++)
        xr[j] = X + (int64_t)min(m0 + 16 * j + r16, M - 1) * K;
    // U steps at a time (the last group re-reads step s1 - 1 and skips it),
    // so that their loads are in flight together
    constexpr int U = 4;
    for (int s = s0; s < s1; s += U) {
        float w[U][8];
        bf16x8_t xa[U][TM];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int su = min(s + u, s1 - 1);
            dequant8<FMT>(B, p, nr * (K / 8) + 4 * su + g, w[u]);
#pragma unroll
            for (int j = 0; j < TM; j++)
                xa[u][j] = *reinterpret_cast<const bf16x8_t *>(xr[j] + 32 * su + 8 * g);
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            if (s + u < s1) {
                uint32_t h[4], l[4];
#pragma unroll
                for (int e = 0; e < 4; e++)
                    split_bf16(w[u][2 * e], w[u][2 * e + 1], h[e], l[e]);
                const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
                const bf16x8_t bl = __builtin_bit_cast(bf16x8_t, make_uint4(l[0], l[1], l[2], l[3]));
#pragma unroll
                for (int j = 0; j < TM; j++) {
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[u][j], bh, acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[u][j], bl, acc[j], 0, 0, 0);
                }
            }
        }
    }
    if (n >= N)
        return;
    const bool split = gridDim.z > 1;
#pragma unroll
    for (int j = 0; j < TM; j++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int m = m0 + 16 * j + 4 * g + i;
            if (m < M) {
                if (split)
                    atomicAdd(Y + (int64_t)m * N + n, acc[j][i]);
                else
                    Y[(int64_t)m * N + n] = acc[j][i];
            }
        }
}

// FP8 W8A8 (dynamic per-token activation scales, per-channel weight scales;
// X quantized per row into the workspace by the same quantizer as the
// weights): a workgroup of WMW x WNW waves owns an output
// tile of TM = 32 TI WMW tokens by TN = 32 TJ WNW rows of W; wave (wm, wn)
// owns TI x TJ tiles of 32 x 32.  K advances in steps of 64 codes, one
// v_mfma_f32_32x32x64_f8f6f4 per tile and step (E4M3 operands, unit block
// scales).  Lane (h, r) of a fragment holds the 32 codes k = 32h .. 32h + 31
// of row r for both operands: the instruction pairs A and B elements by the
// same lane and byte, so any such common placement of k gives the same dot
// products.
//
// X and W codes reach LDS by direct global->LDS loads into a ring of four
// stages (TM X rows then TN W rows of 64 bytes each), issued four steps
// ahead; the only waits on them are explicit vmcnt waits, one barrier per
// step.  16-byte chunk c of row r sits at slot 4r + (c ^ ((r>>1 ^ r>>2) &
// 3)), so the 16 (or 8) rows one ds_read_b128 phase touches land on distinct
// banks.  Step kt + 1's operands are read while step kt's products run.
constexpr int F8K = 64;  // k per step
constexpr int F8S = 4;   // ring stages
constexpr int F8MINSPLIT = 16;  // fewest K steps (of 64 codes) per split

// s_waitcnt immediate: vmcnt n (bits 3:0 and 15:14), lgkmcnt 0, expcnt any
constexpr int vm_wait(int n) { return 0x0070 | (n & 15) | ((n >> 4) << 14); }

__device__ __forceinline__ int f8slot(int r, int c) { return 4 * r + (c ^ (((r >> 1) ^ (r >> 2)) & 3)); }

template <int WMW, int WNW, int TI, int TJ>
struct F8Tile {
    static constexpr int W = WMW * WNW;              // waves
    static constexpr int TM = 32 * TI * WMW, TN = 32 * TJ * WNW;
    static constexpr int STG = (TM + TN) * F8K;      // bytes per stage
    static constexpr int LX = TM / 16 / W, LW = TN / 16 / W;  // loads per wave and stage
    static_assert(LX * 16 * W == TM && LW * 16 * W == TN, "whole load instructions per wave");
    static_assert(4 * (LX + LW) * (F8S - 1) < 64, "vmcnt range");
};

template <int WMW, int WNW, int TI, int TJ>
__global__ __launch_bounds__(64 * WMW * WNW) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_fp8_tile_kernel(
    const uint8_t *__restrict__ Wq, const float *__restrict__ ws, const uint8_t *__restrict__ Xq,
    const float *__restrict__ xs, float *__restrict__ Y, int M, int N, int K, int steps_per_split)
{
    using T = F8Tile<WMW, WNW, TI, TJ>;
    constexpr int LX = T::LX, LW = T::LW, NL = LX + LW;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[F8S * T::STG];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv / WNW, wn = wv % WNW;
    const int m0 = blockIdx.y * T::TM, n0 = blockIdx.x * T::TN;
    // this workgroup's K steps: [kb, kb + nk) of K / F8K (gridDim.z splits)
    const int kb = blockIdx.z * steps_per_split;
    const int nk = min(K / F8K - kb, steps_per_split);
    if (nk <= 0)
        return;  // an empty split (the whole workgroup): adds nothing

    // direct loads: instruction j of wave w fills slots 64 (L w + j) + lane
    // of the X (L = LX) or the W (L = LW) region; rows past M / N re-read the
    // last row (results dropped); byte offsets from row m0 / n0 of the step
    uint32_t ox[LX], ow[LW];
#pragma unroll
    for (int j = 0; j < LX; j++) {
        const int sl = 64 * (LX * wv + j) + lane, r = sl >> 2;
        const int c = (sl & 3) ^ (((r >> 1) ^ (r >> 2)) & 3);
        ox[j] = (uint32_t)((min(m0 + r, M - 1) - m0) * K + 16 * c);
    }
#pragma unroll
    for (int j = 0; j < LW; j++) {
        const int sl = 64 * (LW * wv + j) + lane, r = sl >> 2;
        const int c = (sl & 3) ^ (((r >> 1) ^ (r >> 2)) & 3);
        ow[j] = (uint32_t)((min(n0 + r, N - 1) - n0) * K + 16 * c);
    }
    const uint8_t *const xbase = Xq + (int64_t)m0 * K + F8K * kb;
    const uint8_t *const wbase = Wq + (int64_t)n0 * K + F8K * kb;
    auto issue = [&](int kt) {
        const uint32_t st = lds_addr(smem + (kt % F8S) * T::STG);
#pragma unroll
        for (int j = 0; j < LX; j++)
            dma16(xbase + F8K * kt, ox[j], st + 1024 * (LX * wv + j));
#pragma unroll
        for (int j = 0; j < LW; j++)
            dma16(wbase + F8K * kt, ow[j], st + T::TM * F8K + 1024 * (LW * wv + j));
    };

    // fragment offsets in a stage: A = X rows 32 (TI wm + i) + r, B = W rows
    // 32 (TJ wn + j) + r; chunks 2h and 2h + 1
    const int r32 = lane & 31, h = lane >> 5;
    int oa[TI][2], ob[TJ][2];
#pragma unroll
    for (int q = 0; q < 2; q++) {
#pragma unroll
        for (int i = 0; i < TI; i++)
            oa[i][q] = 16 * f8slot(32 * (TI * wm + i) + r32, 2 * h + q);
#pragma unroll
        for (int j = 0; j < TJ; j++)
            ob[j][q] = T::TM * F8K + 16 * f8slot(32 * (TJ * wn + j) + r32, 2 * h + q);
    }
    auto frag = [&](const uint8_t *p0, const uint8_t *p1) {
        const i32x4_t u = *reinterpret_cast<const i32x4_t *>(p0), v = *reinterpret_cast<const i32x4_t *>(p1);
        return i32x8_t{u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
    };
    i32x8_t a[TI], b[TJ], an[TI], bn[TJ];
    auto reads = [&](int kt) {
        const uint8_t *st = smem + (kt % F8S) * T::STG;
#pragma unroll
        for (int i = 0; i < TI; i++)
            an[i] = frag(st + oa[i][0], st + oa[i][1]);
#pragma unroll
        for (int j = 0; j < TJ; j++)
            bn[j] = frag(st + ob[j][0], st + ob[j][1]);
    };
    auto take = [&]() {
#pragma unroll
        for (int i = 0; i < TI; i++)
            a[i] = an[i];
#pragma unroll
        for (int j = 0; j < TJ; j++)
            b[j] = bn[j];
    };
    f32x16_t acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; i++)
#pragma unroll
        for (int j = 0; j < TJ; j++)
            acc[i][j] = f32x16_t{};
    auto products = [&]() {
#pragma unroll
        for (int i = 0; i < TI; i++)
#pragma unroll
            for (int j = 0; j < TJ; j++)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 0, 0, 0, 127, 0,
                                                                           127);
    };

    for (int kt = 0; kt < F8S && kt < nk; kt++)
        issue(kt);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (nk >= F8S)
        __builtin_amdgcn_s_waitcnt(vm_wait(NL * (F8S - 1)));  // step 0 landed
    else
        __builtin_amdgcn_s_waitcnt(vm_wait(0));
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    reads(0);
    // Step kt: wait until step kt + 1 has landed (the loads of steps kt + 2
    // and kt + 3 may remain) and every wave's reads of step kt are done, so
    // that the loads of step kt + 4 can take its stage; read step kt + 1's
    // operands, then multiply step kt's.
    for (int kt = 0; kt + 1 < nk; kt++) {
        take();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (kt + F8S - 1 < nk)
            __builtin_amdgcn_s_waitcnt(vm_wait(NL * (F8S - 2)));
        else
            __builtin_amdgcn_s_waitcnt(vm_wait(0));
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (kt + F8S < nk)
            issue(kt + F8S);
        reads(kt + 1);
        products();
    }
    take();
    products();

    // lane holds D[m = 8 (r / 4) + 4 h + r % 4][n = r32] of tile (i, j).  The
    // scales load unconditionally (clamped rows), and whole tiles store
    // without guards: a scale used inside a guarded store makes the compiler
    // wait for every earlier memory operation before each store.
    float sx[TI][16], swn[TJ];
#pragma unroll
    for (int i = 0; i < TI; i++)
#pragma unroll
        for (int r = 0; r < 16; r++)
            sx[i][r] = xs[min(m0 + 32 * (TI * wm + i) + 8 * (r >> 2) + 4 * h + (r & 3), M - 1)];
#pragma unroll
    for (int j = 0; j < TJ; j++)
        swn[j] = ws[min(n0 + 32 * (TJ * wn + j) + r32, N - 1)];
    auto store = [&](auto guard_t, auto atomic_t) {
        constexpr bool GUARD = decltype(guard_t)::value, ATOMIC = decltype(atomic_t)::value;
#pragma unroll
        for (int j = 0; j < TJ; j++) {
            const int n = n0 + 32 * (TJ * wn + j) + r32;
#pragma unroll
            for (int i = 0; i < TI; i++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int m = m0 + 32 * (TI * wm + i) + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (!GUARD || (m < M && n < N)) {
                        const float v = acc[i][j][r] * (sx[i][r] * swn[j]);
                        if constexpr (ATOMIC)
                            atomicAdd(Y + (int64_t)m * N + n, v);
                        else
                            Y[(int64_t)m * N + n] = v;
                    }
                }
        }
    };
    // K splits add their partial tiles into a zeroed Y: each product of the
    // scales is formed the same way in every split, so the result differs
    // from the unsplit one only in the order of the fp32 additions
    const bool whole = m0 + T::TM <= M && n0 + T::TN <= N;
    if (gridDim.z > 1) {
        if (whole)
            store(std::false_type{}, std::true_type{});
        else
            store(std::true_type{}, std::true_type{});
    } else if (whole) {
        store(std::false_type{}, std::false_type{});
    } else {
        store(std::true_type{}, std::false_type{});
    }
}

hipError_t zero_y(float *Y, int64_t count, hipStream_t s);

// `slots`: workgroups that run at once (CUs x workgroups per CU); K splits
// (fp32 atomics into a zeroed Y) while the split tiles still fit them
template <int WMW, int WNW, int TI, int TJ>
hipError_t go_fp8_tile(const uint8_t *wblocks, const float *ws, const uint8_t *xblocks, const float *xs, float *Y,
                       int64_t M, int64_t N, int64_t K, hipStream_t s, int64_t slots)
{
    using T = F8Tile<WMW, WNW, TI, TJ>;
    const int64_t gx = (N + T::TN - 1) / T::TN, gy = (M + T::TM - 1) / T::TM;
    const int steps = (int)(K / F8K);
    int splits = 1;
    while (gx * gy * splits * 2 <= slots && splits < 16 && steps / (2 * splits) >= F8MINSPLIT)
        splits *= 2;
    const int per = (steps + splits - 1) / splits;
    if (splits > 1) {
        const hipError_t e = zero_y(Y, M * N, s);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((gemm_fp8_tile_kernel<WMW, WNW, TI, TJ>), dim3((unsigned)gx, (unsigned)gy, (unsigned)splits),
                       dim3(64 * T::W), 0, s, wblocks, ws, xblocks, xs, Y, (int)M, (int)N, (int)K, per);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Q8_0 x Q8_0 int8 path.  Output tile 128 (n) x 128 (m) per workgroup of
// four waves (2 x 2, 64 x 64 each = 2 x 2 tiles of 32 x 32), two workgroups
// per CU; K in steps of one Q8_0 block (32).
//
//   * Codes of W and X and the fp16 scales of both reach LDS by direct
//     global->LDS loads into a ring of six stages, five steps ahead; the
//     only waits on them are explicit vmcnt waits, one barrier per step.
//     Codes: 16-byte chunk c of row r at slot 2r + (c ^ ((r >> 3) & 1)), so
//     the 16 rows a ds_read_b128 phase touches land on distinct banks.
//   * Per 32 x 32 tile: v_mfma_i32_32x32x32_i8 forms the exact integer dot
//     products P[m][n] of the block (X codes the A operand, W codes the B
//     operand); v_mfma_f32_32x32x8_f16 with d_x in k-slot 0 of A and d_w in
//     k-slot 0 of B forms the outer product d_x[m] d_w[n] in the same output
//     layout -- exact, since a product of two fp16 values fits binary32 --
//     and each output then costs one conversion and one fused multiply-add:
//     acc += float(P) * (d_x d_w).  The 32 lanes of an output row hold 32
//     consecutive n, so stores and atomics are 128-byte rows.
//   * K splits add into a zeroed Y with fp32 atomics.
// ---------------------------------------------------------------------------
constexpr int BN = 128;     // n tile
constexpr int BK = 32;      // k per step (one Q8_0 block)
constexpr int IBM = 128;    // m tile
constexpr int INS = 6;      // stages
constexpr int ISC = 8192;   // offset of the scales in a stage: d_w [128] dwords, then d_x [128]
constexpr int ISTG = ISC + 1024;

typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int islot(int row, int c) { return 2 * row + (c ^ ((row >> 3) & 1)); }

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_i8_kernel(
    const int8_t *__restrict__ Wq, const uint16_t *__restrict__ Wd, const int8_t *__restrict__ Xq,
    const uint16_t *__restrict__ Xd, float *__restrict__ Y, int M, int N, int K, int kt_per_split)
{
    __shared__ __attribute__((aligned(1024))) uint8_t smem[INS * ISTG];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wv & 1, wm = wv >> 1;  // 2 x 2 waves, 64 x 64 each
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * IBM;
    const int kt0 = blockIdx.z * kt_per_split;
    const int kt1 = min(K / BK, kt0 + kt_per_split);
    const int KB = K / 32;
    if (kt0 >= kt1)
        return;  // an empty K split (the whole workgroup): adds nothing

    // direct loads: the load of wave w fills code slots 64w + lane of the
    // W and the X region; rows past N / M re-read the last row (results
    // dropped); byte offsets from row n0 / m0 of the step
    const int p = 64 * wv + lane, pr = p >> 1, pc = (p & 1) ^ ((pr >> 3) & 1);
    const uint32_t ow = (uint32_t)((min(n0 + pr, N - 1) - n0) * K + 16 * pc);
    const uint32_t ox = (uint32_t)((min(m0 + pr, M - 1) - m0) * K + 16 * pc);
    // scales: waves 0, 1 load the d_w dword holding the step's block of rows
    // 64w + lane, waves 2, 3 the d_x dword of rows 64(w - 2) + lane
    const bool sw = wv < 2;
    const int srow = 64 * (wv & 1) + lane;
    const uint32_t osc = (uint32_t)((sw ? min(n0 + srow, N - 1) - n0 : min(m0 + srow, M - 1) - m0) * KB * 2);
    const uint8_t *const wbase = reinterpret_cast<const uint8_t *>(Wq) + (int64_t)n0 * K;
    const uint8_t *const xbase = reinterpret_cast<const uint8_t *>(Xq) + (int64_t)m0 * K;
    const uint8_t *const sbase = sw ? reinterpret_cast<const uint8_t *>(Wd + (int64_t)n0 * KB)
                                    : reinterpret_cast<const uint8_t *>(Xd + (int64_t)m0 * KB);
    auto issue = [&](int kt) {
        const uint32_t st = lds_addr(smem + (kt % INS) * ISTG);
        dma16(wbase + BK * kt, ow, st + 1024 * wv);
        dma16(xbase + BK * kt, ox, st + 4096 + 1024 * wv);
        dma4(sbase + 4 * (kt >> 1), osc, st + ISC + (sw ? 0 : 512) + 256 * (wv & 1));
    };

    const int r32 = lane & 31, kh = lane >> 5;
    int oa[2], ob[2], sa[2], sb[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        oa[i] = 16 * islot(64 * wn + 32 * i + r32, kh);
        ob[i] = 4096 + 16 * islot(64 * wm + 32 * i + r32, kh);
        sa[i] = ISC + 4 * (64 * wn + 32 * i + r32);
        sb[i] = ISC + 512 + 4 * (64 * wm + 32 * i + r32);
    }

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
            acc[i][j] = f32x16_t{};
    const i32x16_t izero = {};
    const f32x16_t fzero = {};

    // the step's operands: codes, and d in k-slot 0 of lanes 0..31 (zeros
    // elsewhere; read by every lane and masked, so that no branch serializes
    // the reads); the scale operands of two steps are held
    const uint32_t dmask = kh ? 0u : 0xffffu;
    i32x4_t a[2], x[2];
    f16x4_t as[2], xs[2], asn[2], xsn[2];  // this step's and the next step's
    auto reads = [&](int kt) {
        const uint8_t *st = smem + (kt % INS) * ISTG;
        const int hs = 16 * (kt & 1);  // the step's fp16 half of the scale dwords
#pragma unroll
        for (int i = 0; i < 2; i++) {
            a[i] = *reinterpret_cast<const i32x4_t *>(st + oa[i]);
            x[i] = *reinterpret_cast<const i32x4_t *>(st + ob[i]);
            const uint32_t hw = (*reinterpret_cast<const uint32_t *>(st + sa[i]) >> hs) & dmask;
            const uint32_t hx = (*reinterpret_cast<const uint32_t *>(st + sb[i]) >> hs) & dmask;
            asn[i] = __builtin_bit_cast(f16x4_t, make_uint2(hw, 0u));
            xsn[i] = __builtin_bit_cast(f16x4_t, make_uint2(hx, 0u));
        }
    };
    i32x16_t P[4];  // tile t = 2i + j
    auto products = [&]() {
#pragma unroll
        for (int t = 0; t < 4; t++)
            P[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(x[t & 1], a[t >> 1], izero, 0, 0, 0);
    };

    for (int kt = kt0; kt < kt0 + INS - 1 && kt < kt1; kt++)
        issue(kt);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt 0, lgkmcnt 0
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    reads(kt0);
    products();
#pragma unroll
    for (int i = 0; i < 2; i++) {
        as[i] = asn[i];
        xs[i] = xsn[i];
    }

    // Step kt: its integer products are in flight.  Wait until step kt + 1
    // has landed (the loads of steps kt + 2 .. kt + 4, three per wave each,
    // may remain) and every wave is past its reads of step kt - 1, whose
    // stage the loads of step kt + 5 then take; read step kt + 1's operands
    // (their latency hides behind the rescale); rescale step kt, each
    // tile's d_w d_x product issued one tile ahead; then issue step kt + 1's
    // integer products (their latency hides behind the next barrier).
    auto step = [&](int kt, auto more_t) {
        constexpr bool MORE = decltype(more_t)::value;  // a step kt + 1 follows
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (kt + INS - 2 < kt1)
            __builtin_amdgcn_s_waitcnt(0x0070 | 3 * (INS - 3));  // vmcnt 9, lgkmcnt 0
        else
            __builtin_amdgcn_s_waitcnt(0x0070);                  // vmcnt 0, lgkmcnt 0
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (kt + INS - 1 < kt1)
            issue(kt + INS - 1);
        if constexpr (MORE)
            reads(kt + 1);
        f32x16_t S[2];
        S[0] = __builtin_amdgcn_mfma_f32_32x32x8f16(xs[0], as[0], fzero, 0, 0, 0);
#pragma unroll
        for (int t = 0; t < 4; t++) {
            if (t + 1 < 4)
                S[(t + 1) & 1] = __builtin_amdgcn_mfma_f32_32x32x8f16(xs[(t + 1) & 1], as[(t + 1) >> 1], fzero, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < 16; r++)
                acc[t >> 1][t & 1][r] = fmaf((float)P[t][r], S[t & 1][r], acc[t >> 1][t & 1][r]);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (MORE) {
            products();
#pragma unroll
            for (int i = 0; i < 2; i++) {
                as[i] = asn[i];
                xs[i] = xsn[i];
            }
        }
    };
    for (int kt = kt0; kt < kt1 - 1; kt++)
        step(kt, std::true_type{});
    step(kt1 - 1, std::false_type{});

    // X is the A operand and W the B operand of both products, so
    // acc[i][j][r] = D[m = 8 (r / 4) + 4 (lane / 32) + r % 4][n = lane % 32]
    // of tile (W part i, X part j): the 32 lanes of a row write 128
    // consecutive bytes (plain stores, or fp32 atomics for K splits)
    const bool atomic = gridDim.z > 1;
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int n = n0 + wn * 64 + 32 * i + r32;
        if (n >= N)
            continue;
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = m0 + wm * 64 + 32 * j + 8 * (r >> 2) + 4 * kh + (r & 3);
                if (m < M) {
                    if (atomic)
                        atomicAdd(Y + (int64_t)m * N + n, acc[i][j][r]);
                    else
                        Y[(int64_t)m * N + n] = acc[i][j][r];
                }
            }
    }
}

// Zero-fill of Y before a split-K accumulation (a kernel, not a memset, so
// that the call can be captured in a HIP graph).
__global__ void zero_kernel(float *__restrict__ p, int64_t n)
{
    const int64_t n4 = n / 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        reinterpret_cast<float4 *>(p)[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (blockIdx.x == 0 && threadIdx.x == 0)
        for (int64_t i = 4 * n4; i < n; i++)
            p[i] = 0.0f;
}

// Split K so that at least ~2 workgroups per CU exist.
inline int splits_for(int64_t tiles, int nkt)
{
    int s = 1;
    while (tiles * s < 512 && s < 16 && nkt / (2 * s) >= 2)
        s *= 2;
    return s;
}

hipError_t zero_y(float *Y, int64_t count, hipStream_t s)
{
    int64_t g = (count / 4 + 255) / 256;
    g = g < 1 ? 1 : (g > 65536 ? 65536 : g);
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)g), dim3(256), 0, s, Y, count);
    return hipGetLastError();
}

// `fill`: workgroups (tiles x K splits) to aim for; more splits also mean
// more fp32 atomics into Y, which measured slower past ~256 workgroups for
// small M
template <int FMT, int TM, int NT>
hipError_t go_bf16(const uint8_t *blocks, const Planes &p, const uint16_t *X, float *Y, int64_t M,
                   int64_t N, int64_t K, hipStream_t s, int fill = 512, bool within = false)
{
    const int64_t gx = (N + 64 * NT - 1) / (64 * NT), gy = (M + 16 * TM - 1) / (16 * TM);
    const int nslab = (int)(K / SLAB);
    // K splits until the workgroups reach `fill` (within: without passing it)
    int splits = 1;
    while ((within ? gx * gy * splits * 2 <= fill : gx * gy * splits < fill) && splits < 32 &&
           nslab / (2 * splits) >= 2)
        splits *= 2;
    const int per = (nslab + splits - 1) / splits;
    if (splits > 1) {
        const hipError_t e = zero_y(Y, M * N, s);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((gemm_bf16_kernel<FMT, TM, NT>), dim3((unsigned)gx, (unsigned)gy, (unsigned)splits), dim3(256), 0,
                       s, blocks, p.scales, p.d, X, Y, (int)M, (int)N, (int)K, per);
    return hipGetLastError();
}

template <int FMT, int TM, int NT, int PF>
hipError_t go_skinny(const uint8_t *blocks, const Planes &p, const uint16_t *X, float *Y, int64_t M,
                     int64_t N, int64_t K, hipStream_t s)
{
    const int64_t gx = (N + 16 * NT - 1) / (16 * NT);
    const int nslab = (int)(K / SLAB);
    // enough waves to keep ~8 per CU streaming: split K over up to 8 waves
    int KS = 1;
    while (gx * KS < 2048 && KS < 8 && nslab / (2 * KS) >= PF)
        KS *= 2;
    const int per = (nslab + KS - 1) / KS;
    const size_t lds = (size_t)KS * NT * TM * 4 * 64 * sizeof(float);
    hipLaunchKernelGGL((gemm_skinny_kernel<FMT, TM, NT, PF>), dim3((unsigned)gx), dim3(64 * KS), lds, s, blocks,
                       p.scales, p.d, X, Y, (int)M, (int)N, (int)K, per);
    return hipGetLastError();
}

// split K while the tiles fill less than one round of the 256 CUs, keeping
// at least 16 slabs per split
int pf_splits(int64_t tiles, int nslab)
{
    int sp = 1;
    while (sp < 8 && tiles * sp * 2 <= 256 && nslab / (sp * 2) >= 16)
        sp *= 2;
    return sp;
}

template <int FMT>
hipError_t go_pf(const uint8_t *blocks, const Planes &p, const uint16_t *X, float *Y, int64_t M, int64_t N,
                 int64_t K, hipStream_t s)
{
    const int64_t tiles = ((M + PBM - 1) / PBM) * ((N + PBN - 1) / PBN);
    if (tiles > (int64_t)1 << 30)
        return hipErrorInvalidValue;
    const int nslab = (int)(K / PBK);
    const int sp = pf_splits(tiles, nslab);
    const int per = (nslab + sp - 1) / sp;
    if (sp > 1) {
        const hipError_t e = zero_y(Y, M * N, s);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((gemm_pf_kernel<FMT>), dim3((unsigned)tiles, (unsigned)sp), dim3(512), 0, s, blocks, p.scales,
                       p.d, X, Y, (int)M, (int)N, (int)K, per);
    return hipGetLastError();
}

// Split K towards ~1024 workgroups (four per CU), at least four slabs each.
template <int FMT, int TM>
hipError_t go_bt(const uint8_t *blocks, const Planes &p, const uint16_t *X, float *Y, int64_t M, int64_t N,
                 int64_t K, hipStream_t s)
{
    const int64_t gx = (N + TBN - 1) / TBN, gy = (M + 16 * TM - 1) / (16 * TM);
    const int nslab = (int)(K / TBK);
    int sp = 1;
    while (sp < 32 && gx * gy * sp * 2 <= 1024 && nslab / (sp * 2) >= 4)
        sp *= 2;
    const int per = (nslab + sp - 1) / sp;
    if (sp > 1) {
        const hipError_t e = zero_y(Y, M * N, s);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((gemm_bt_kernel<FMT, TM>), dim3((unsigned)gx, (unsigned)gy, (unsigned)sp), dim3(256), 0, s,
                       blocks, p.scales, p.d, X, Y, (int)M, (int)N, (int)K, per);
    return hipGetLastError();
}

// one workgroup per 16 rows, K split over its KW waves
template <int KW, int DG>
hipError_t go_bs(const uint8_t *blocks, const Planes &p, const uint16_t *X, float *Y, int64_t M, int64_t N, int64_t K,
                 hipStream_t s)
{
    hipLaunchKernelGGL((gemm_bs_kernel<KW, DG>), dim3((unsigned)((N + 15) / 16)), dim3(64 * KW), 0, s, blocks,
                       p.scales, X, Y, (int)M, (int)N, (int)K);
    return hipGetLastError();
}

// Split K towards ~1024 workgroups (four per CU), at least four slabs each.
template <int TM>
hipError_t go_bx(const uint8_t *blocks, const Planes &p, const uint16_t *X, float *Y, int64_t M, int64_t N, int64_t K,
                 hipStream_t s)
{
    const int64_t gx = (N + TBN - 1) / TBN, gy = (M + 16 * TM - 1) / (16 * TM);
    const int nslab = (int)(K / TBK);
    int sp = 1;
    while (sp < 32 && gx * gy * sp * 2 <= 1024 && nslab / (sp * 2) >= 4)
        sp *= 2;
    const int per = (nslab + sp - 1) / sp;
    if (sp > 1) {
        const hipError_t e = zero_y(Y, M * N, s);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((gemm_bx_kernel<TM>), dim3((unsigned)gx, (unsigned)gy, (unsigned)sp), dim3(256), 0, s, blocks,
                       p.scales, X, Y, (int)M, (int)N, (int)K, per);
    return hipGetLastError();
}

template <int FMT>
hipError_t bf16_by_m(const uint8_t *blocks, const Planes &p, const uint16_t *X, float *Y, int64_t M,
                     int64_t N, int64_t K, hipStream_t s)
{
    // tall matrices (many row tiles) stream two 16-row tiles per wave
    // launch shapes from measured sweeps on MI355X (4096 x 14336,
    // 14336 x 4096, 4096 x 4096 and 131072 x 5120 weights): the direct-load
    // weight stream wins for up to 32 tokens once W has more than 2^24
    // elements; for Q4K the one-pass kernel up to five tokens (4096 x 14336,
    // eager launches: 1 / 4 / 8 / 16 tokens 13.4 / 14.8 / 17.1 / 21.0 us
    // against 16.9 / 17.3 / 17.3 / 17.2 us for the ring kernel and its
    // zero-fill launch; 14336 x 4096: 14.3 / 16.5 / 18.1 / 22.8 against
    // 17.5 / 18.1 / 17.6 / 17.9 us)
    if (M <= 32 && N * K > ((int64_t)1 << 24)) {
        if constexpr (FMT == FMT_Q4K)
            return M <= 5 ? go_bs<8, 1>(blocks, p, X, Y, M, N, K, s)
                   : M <= 16 ? go_bx<1>(blocks, p, X, Y, M, N, K, s) : go_bx<2>(blocks, p, X, Y, M, N, K, s);
        return M <= 16 ? go_bt<FMT, 1>(blocks, p, X, Y, M, N, K, s) : go_bt<FMT, 2>(blocks, p, X, Y, M, N, K, s);
    }
    const bool tall = N >= 32768;
    if (M <= 8)
        return tall ? go_skinny<FMT, 1, 2, 4>(blocks, p, X, Y, M, N, K, s)
                    : go_skinny<FMT, 1, 1, 2>(blocks, p, X, Y, M, N, K, s);
    if (M <= 16)
        return tall ? go_skinny<FMT, 1, 2, 4>(blocks, p, X, Y, M, N, K, s)
                    : go_bf16<FMT, 1, 2>(blocks, p, X, Y, M, N, K, s, 256);
    if (M <= 32)
        return go_skinny<FMT, 2, 1, 4>(blocks, p, X, Y, M, N, K, s);
    // 64-token tiles up to 64 tokens, and up to 512 for weights of at most
    // 2^25 elements (4096 x 4096 at 128 tokens: 20.3 us against 36.2 on the
    // 128-token tiles; 1024 x 4096 at 512 tokens: 21.4 against 37.0)
    if (M <= 64 || (M <= 512 && N * K <= ((int64_t)1 << 25)))
        return go_bf16<FMT, 4, 2>(blocks, p, X, Y, M, N, K, s, 256);
    // the prefill kernel from 513 tokens, and from 256 where its 256 x 256
    // tiles number at least 200 (wide weights: the 131072 x 5120 head at 256
    // tokens ran 510 us there against 692 us on the tiles below)
    if (M >= PF_MIN_M || (M >= 256 && ((M + 255) / 256) * ((N + 255) / 256) >= 200))
        return go_pf<FMT>(blocks, p, X, Y, M, N, K, s);
    // otherwise 65..512 tokens: 128 x 256 tiles, K split only as far as the
    // workgroups stay within one per CU (measured: at 96 tokens 14336 x 4096
    // ran 94 us with 16 splits, 44 us with 4; up to 512 tokens this beats the
    // prefill kernel there, e.g. 97.7 vs 115.4 us at 512 x 14336 x 4096)
    return go_bf16<FMT, 8, 4>(blocks, p, X, Y, M, N, K, s, 256, true);
}


template <int FMT, int TM>
hipError_t go_gen(const uint8_t *blocks, const uint16_t *X, float *Y, int64_t M, int64_t N, int64_t K, hipStream_t s)
{
    const Planes p = planes_of(FMT, N, K);
    const int64_t gx = (N + 63) / 64, gy = (M + 16 * TM - 1) / (16 * TM);
    const int steps = (int)(K / 32);
    int sp = 1;
    while (gx * gy * sp < 512 && sp < 32 && steps / (2 * sp) >= 8)
        sp *= 2;
    const int per = (steps + sp - 1) / sp;
    if (sp > 1) {
        const hipError_t e = zero_y(Y, M * N, s);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((gemm_gen_kernel<FMT, TM>), dim3((unsigned)gx, (unsigned)gy, (unsigned)sp), dim3(256), 0, s,
                       blocks, p, X, Y, (int)M, (int)N, (int)K, per);
    return hipGetLastError();
}

template <int FMT, int GTM, int GNT>
hipError_t go_gen_lds(const uint8_t *blocks, const uint16_t *X, float *Y, int64_t M, int64_t N, int64_t K,
                      hipStream_t s)
{
    const Planes p = planes_of(FMT, N, K);
    const int64_t gx = (N + 64 * GNT - 1) / (64 * GNT), gy = (M + 16 * GTM - 1) / (16 * GTM);
    const int nslab = (int)(K / SLAB);
    int splits = 1;
    while (gx * gy * splits * 2 <= 256 && splits < 32 && nslab / (2 * splits) >= 2)
        splits *= 2;
    const int per = (nslab + splits - 1) / splits;
    if (splits > 1) {
        const hipError_t e = zero_y(Y, M * N, s);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((gemm_gen_lds_kernel<FMT, GTM, GNT>), dim3((unsigned)gx, (unsigned)gy, (unsigned)splits),
                       dim3(256), 0, s, blocks, p, X, Y, (int)M, (int)N, (int)K, per);
    return hipGetLastError();
}

template <int FMT>
hipError_t gen_tm(const uint8_t *blocks, const uint16_t *X, float *Y, int64_t M, int64_t N, int64_t K, hipStream_t s)
{
    // the LDS-staged kernel, tiles of 16..128 tokens by 128..256 rows (Q8_0
    // here serves block tails, whose remainder operand only the per-step
    // kernel carries)
    if (FMT != FMT_Q8_0 && K % SLAB == 0) {
        if (M <= 16)
            return go_gen_lds<FMT, 1, 4>(blocks, X, Y, M, N, K, s);
        if (M <= 32)
            return go_gen_lds<FMT, 2, 4>(blocks, X, Y, M, N, K, s);
        if (M <= 64)
            return go_gen_lds<FMT, 4, 2>(blocks, X, Y, M, N, K, s);
        return go_gen_lds<FMT, 8, 2>(blocks, X, Y, M, N, K, s);
    }
    if (M <= 16)
        return go_gen<FMT, 1>(blocks, X, Y, M, N, K, s);
    if (M <= 32)
        return go_gen<FMT, 2>(blocks, X, Y, M, N, K, s);
    return go_gen<FMT, 4>(blocks, X, Y, M, N, K, s);
}

hipError_t launch_gemm_gen(int fmt, const uint8_t *blocks, const uint16_t *X, float *Y, int64_t M, int64_t N,
                           int64_t K, hipStream_t s)
{
    switch (fmt) {
    case FMT_Q5K: return gen_tm<FMT_Q5K>(blocks, X, Y, M, N, K, s);
    case FMT_Q3K: return gen_tm<FMT_Q3K>(blocks, X, Y, M, N, K, s);
    case FMT_Q2K: return gen_tm<FMT_Q2K>(blocks, X, Y, M, N, K, s);
    case FMT_Q4_0: return gen_tm<FMT_Q4_0>(blocks, X, Y, M, N, K, s);
    case FMT_Q4_1: return gen_tm<FMT_Q4_1>(blocks, X, Y, M, N, K, s);
    case FMT_Q5_0: return gen_tm<FMT_Q5_0>(blocks, X, Y, M, N, K, s);
    case FMT_Q5_1: return gen_tm<FMT_Q5_1>(blocks, X, Y, M, N, K, s);
    case FMT_FP8: return gen_tm<FMT_FP8>(blocks, X, Y, M, N, K, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gemm_bf16(int fmt, const uint8_t *blocks, const uint16_t *X, float *Y, int64_t M,
                            int64_t N, int64_t K, hipStream_t s)
{
    if (generic_fmt(fmt))
        return launch_gemm_gen(fmt, blocks, X, Y, M, N, K, s);
    // Q8_0 rows that end in a tail of blocks (K % 256 != 0): the generic
    // kernel, which steps K by one block (the tuned ones take 128-element
    // slabs and two blocks' scales per dword)
    if (fmt == FMT_Q8_0 && K % 256 != 0)
        return gen_tm<FMT_Q8_0>(blocks, X, Y, M, N, K, s);
    const Planes p = planes_of(fmt, N, K);
    if (fmt == FMT_Q4K)
        return bf16_by_m<FMT_Q4K>(blocks, p, X, Y, M, N, K, s);
    if (fmt == FMT_Q6K)
        return bf16_by_m<FMT_Q6K>(blocks, p, X, Y, M, N, K, s);
    return bf16_by_m<FMT_Q8_0>(blocks, p, X, Y, M, N, K, s);
}

// Unfused gated projection, second step: H = act(G) * H, where H holds the
// up projection (the fused kernel evaluates the same fp32 expression).
__global__ __launch_bounds__(256) void glu_apply_kernel(const float *__restrict__ G, float *__restrict__ H, int64_t n,
                                                        int act)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        H[i] = act_f32(act, G[i]) * H[i];
}

hipError_t launch_glu_apply(const float *G, float *H, int64_t n, int act, hipStream_t s)
{
    int64_t g = (n + 255) / 256;
    g = g < 1 ? 1 : (g > 65536 ? 65536 : g);
    hipLaunchKernelGGL(glu_apply_kernel, dim3((unsigned)g), dim3(256), 0, s, G, H, n, act);
    return hipGetLastError();
}

hipError_t launch_gemm_fp8(const uint8_t *wblocks, const uint8_t *xblocks, float *Y, int64_t M, int64_t N,
                           int64_t K, hipStream_t s)
{
    const Planes pw = planes_of(FMT_FP8, N, K), px = planes_of(FMT_FP8, M, K);
    const float *ws = reinterpret_cast<const float *>(wblocks + pw.scales);
    const float *xs = reinterpret_cast<const float *>(xblocks + px.scales);
    // 256 x 256 tiles (eight waves) move half the bytes per product of the
    // 128 x 128 ones, where there are enough of them for every CU; fewer
    // tiles split K up to one workgroup per CU with at least 16 steps each
    // (measured over 1..512 tokens at 14336 x 4096, 4096 x 14336 and
    // 4096 x 4096: 448 split workgroups of 256 tokens ran 50 us against 35
    // whole, while one token over 32 tiles ran 21 us split eight ways and 43
    // split two ways)
    if (((M + 255) / 256) * ((N + 255) / 256) >= 256)
        return go_fp8_tile<4, 2, 2, 4>(wblocks, ws, xblocks, xs, Y, M, N, K, s, 256);
    return go_fp8_tile<2, 2, 2, 2>(wblocks, ws, xblocks, xs, Y, M, N, K, s, 256);
}

hipError_t launch_gemm_i8(const uint8_t *wblocks, const uint8_t *xblocks, float *Y, int64_t M, int64_t N,
                          int64_t K, hipStream_t s)
{
    const Planes pw = planes_of(FMT_Q8_0, N, K), px = planes_of(FMT_Q8_0, M, K);
    const int64_t gx = (N + BN - 1) / BN, gy = (M + IBM - 1) / IBM;
    const int nkt = (int)(K / BK);
    // K splits only while the workgroups still fit one round (two per CU):
    // 448 tiles at 512 x 14336 ran 158 us split in two, 138 us whole
    int splits = 1;
    while (gx * gy * 2 * splits <= 512 && splits < 16 && nkt / (2 * splits) >= 2)
        splits *= 2;
    const int per = (nkt + splits - 1) / splits;
    if (splits > 1) {
        const hipError_t e = zero_y(Y, M * N, s);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL(gemm_i8_kernel, dim3((unsigned)gx, (unsigned)gy, (unsigned)splits), dim3(256), 0, s,
                       reinterpret_cast<const int8_t *>(wblocks),
                       reinterpret_cast<const uint16_t *>(wblocks + pw.scales),
                       reinterpret_cast<const int8_t *>(xblocks),
                       reinterpret_cast<const uint16_t *>(xblocks + px.scales), Y, (int)M, (int)N, (int)K, per);
    return hipGetLastError();
}

}  // namespace ql
