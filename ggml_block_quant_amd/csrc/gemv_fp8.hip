// gemv_fp8.hip -- one-shot GEMV for FP8 E4M3 weights with per-row fp32
// scales, one or two bf16 tokens (page "Quantization types", section "FP8":
// weight-only FP8 keeps 16-bit activations).
//
// E4M3 values are exact in bf16 (3 mantissa bits, exponents 2^-9 .. 2^8),
// so v_cvt_scalef32_pk_bf16_fp8 with scale 1.0 turns two codes into a bf16
// pair with no rounding, v_dot2_f32_bf16 multiplies them with X exactly and
// accumulates in fp32, and the row scale multiplies the reduced sum once.
//
// Layout: codes [N][K] (one byte each), then the fp32 scales [N] at the
// 16-byte-rounded offset.  A row of K codes is K/16 pieces of 16 bytes;
// lane l of a wave takes pieces l, l + 64, ... (CP of them) of each of its
// R rows and issues every one of those loads at its start.  The workgroup
// stages X once in LDS: piece i's elements 16i..16i+7 in one plane and
// 16i+8..16i+15 in another, so lane-consecutive ds_read_b128 are
// conflict-free.
#include "qlinear_internal.h"
#include "gemv_fp8.h"

namespace ql {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int FW = 4;  // waves per workgroup

// codes are read once: non-temporal loads keep them from displacing X
__device__ __forceinline__ uint4 ld_codes(const uint8_t *p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, a), __builtin_bit_cast(v2bf, b), c, false);
}

// two E4M3 codes (bytes 2H, 2H+1 of w) -> their bf16 pair, exactly
template <bool H>
__device__ __forceinline__ uint32_t pair_of(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, H));
}

template <int M, int CP, int R>
__global__ __launch_bounds__(64 * FW) void gemv_fp8_kernel(const uint8_t *__restrict__ C, const float *__restrict__ S,
                                                           const uint16_t *__restrict__ X, float *__restrict__ Y,
                                                           int64_t N, int K)
{
    constexpr int SL = 64 * CP;                          // piece slots per row
    constexpr int XU = (M * 2 * SL + 64 * FW - 1) / (64 * FW);  // uint4 of X staged per thread
    constexpr int XT = M * 2 * SL;                       // uint4 of staged X
    __shared__ uint4 sx[XT + 1];  // [m][half][slot]; the last entry takes the stores of idle threads
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int P = K / 16;
    const int64_t n0 = ((int64_t)blockIdx.x * FW + wv) * R;

    // X first, so that waiting for it never waits for the codes; slots past
    // the row read its last piece and stage zeros
    uint4 xs[XU];
#pragma unroll
    for (int j = 0; j < XU; j++) {
        const int u = min(tid + 64 * FW * j, XT - 1);
        const int m = u / (2 * SL), h = (u / SL) & 1, i = u % SL;
        xs[j] = *reinterpret_cast<const uint4 *>(X + (int64_t)m * K + 16 * min(i, P - 1) + 8 * h);
    }
    // every code load of the wave; rows past N re-read row N - 1 (not written)
    uint4 w[R][CP];
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int64_t n = min(n0 + r, N - 1);
#pragma unroll
        for (int j = 0; j < CP; j++)
            w[r][j] = ld_codes(C + n * K + 16 * min(lane + 64 * j, P - 1));
    }
    // keep the staging (and its wait for X) after every code load
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < XU; j++) {
        // stores without branches (a branch here lets the compiler sink the
        // X loads below the code loads)
        const int u = min(tid + 64 * FW * j, XT);
        const uint32_t keep = u % SL < P ? ~0u : 0u;
        sx[u] = make_uint4(xs[j].x & keep, xs[j].y & keep, xs[j].z & keep, xs[j].w & keep);
    }
    __syncthreads();

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int m = 0; m < M; m++)
            acc[r][m] = 0.0f;
#pragma unroll
    for (int j = 0; j < CP; j++) {
        const int i = lane + 64 * j;
        uint32_t xp[M][8];
#pragma unroll
        for (int m = 0; m < M; m++) {
            const uint4 a = sx[(2 * m) * SL + i], b = sx[(2 * m + 1) * SL + i];
            xp[m][0] = a.x, xp[m][1] = a.y, xp[m][2] = a.z, xp[m][3] = a.w;
            xp[m][4] = b.x, xp[m][5] = b.y, xp[m][6] = b.z, xp[m][7] = b.w;
        }
#pragma unroll
        for (int r = 0; r < R; r++) {
            const uint32_t c[4] = {w[r][j].x, w[r][j].y, w[r][j].z, w[r][j].w};
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const uint32_t p0 = pair_of<false>(c[q]), p1 = pair_of<true>(c[q]);
#pragma unroll
                for (int m = 0; m < M; m++) {
                    acc[r][m] = dot2(p0, xp[m][2 * q], acc[r][m]);
                    acc[r][m] = dot2(p1, xp[m][2 * q + 1], acc[r][m]);
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
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < R; r++)
            if (n0 + r < N) {
                const float s = S[n0 + r];
#pragma unroll
                for (int m = 0; m < M; m++)
                    Y[(int64_t)m * N + n0 + r] = acc[r][m] * s;
            }
    }
}

template <int M, int CP>
hipError_t go_fp8(const uint8_t *blocks, const float *S, const uint16_t *X, float *Y, int64_t N, int64_t K,
                  hipStream_t s)
{
    constexpr int R = CP >= 8 ? 1 : 8 / CP;  // ~8 code loads per lane in flight
    const int64_t grid = (N + FW * R - 1) / (FW * R);
    hipLaunchKernelGGL((gemv_fp8_kernel<M, CP, R>), dim3((unsigned)grid), dim3(64 * FW), 0, s, blocks, S, X, Y, N,
                       (int)K);
    return hipGetLastError();
}

template <int M>
bool fp8_by_cp(const uint8_t *blocks, const float *S, const uint16_t *X, float *Y, int64_t N, int64_t K,
               hipStream_t s, hipError_t &e)
{
    const int64_t cp = (K / 16 + 63) / 64;
    switch (cp) {
#define C(CC)                                                  \
    case CC:                                                   \
        if constexpr (M * CC <= 16) { /* X within 32 KiB */    \
            e = go_fp8<M, CC>(blocks, S, X, Y, N, K, s);       \
            return true;                                       \
        } else {                                               \
            return false;                                      \
        }
        C(1) C(2) C(3) C(4) C(5) C(6) C(7) C(8) C(9) C(10) C(11) C(12) C(13) C(14) C(15) C(16)
#undef C
    default: return false;
    }
}

}  // namespace

bool launch_gemv_fp8(const uint8_t *blocks, const uint16_t *X, float *Y, int M, int64_t N, int64_t K,
                     hipStream_t s, hipError_t &e)
{
    const Planes p = planes_of(FMT_FP8, N, K);
    const float *S = reinterpret_cast<const float *>(blocks + p.scales);
    if (M == 1)
        return fp8_by_cp<1>(blocks, S, X, Y, N, K, s, e);
    if (M == 2)
        return fp8_by_cp<2>(blocks, S, X, Y, N, K, s, e);
    return false;
}

}  // namespace ql
