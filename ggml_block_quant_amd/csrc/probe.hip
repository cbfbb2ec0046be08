// probe.hip -- measurement aids: the two ceilings the benchmark reports next
// to the published peaks (page "Quantization types", section "NVFP4": the
// benchmark reports measured latencies; repeated projections benefit from
// the cache, so a ceiling is taken on a buffer read once per launch).
//
//   * read_probe_kernel: every byte of a buffer read once with 16-byte
//     non-temporal loads (the weight stream of the GEMV kernels), each
//     workgroup a contiguous span, eight loads in flight per thread (the
//     grid shrinks for small buffers so that each thread has eight);
//     nothing is written unless the XOR of all
//     loaded words equals a value that the caller's buffer contents make
//     impossible in practice, so the loads stay live.
//   * mfma_probe_kernel: dependent chains of v_mfma_f32_32x32x16_bf16 on
//     four accumulators per wave, eight waves per workgroup (two per SIMD),
//     no memory traffic inside the loop.
//   * mix_probe_kernel: the same loop with sixteen independent fp32 fmas
//     (eight chains) after each MFMA -- the MFMAs only, the fmas only, or
//     both interleaved in one instruction stream -- with one to eight waves
//     per SIMD (workgroups of four waves, 256 per wave-per-SIMD), which
//     measures how far the VALU work of a kernel can hide behind its MFMAs
//     at a given occupancy.
#include <algorithm>

#include "qlinear_internal.h"

namespace ql {
namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kReadBlocks = 2048, kReadThreads = 256;
constexpr int kMfmaBlocks = 1024, kMfmaThreads = 512, kMfmaChains = 4;
constexpr int kMixFmas = 16;  // fp32 fmas per MFMA in the mixed probe

__global__ __launch_bounds__(kReadThreads) void read_probe_kernel(const u32x4_t *__restrict__ p, int64_t n16,
                                                                  float *__restrict__ out)
{
    // workgroup b reads a contiguous span; each thread keeps kInFlight
    // 16-byte loads outstanding (consecutive threads, consecutive addresses)
    constexpr int kInFlight = 8;
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t lo = (int64_t)blockIdx.x * per, hi = min(lo + per, n16);
    uint32_t acc = 0;
    int64_t i = lo + threadIdx.x;
    for (; i + (kInFlight - 1) * kReadThreads < hi; i += kInFlight * kReadThreads) {
        u32x4_t v[kInFlight];
#pragma unroll
        for (int k = 0; k < kInFlight; k++)
            v[k] = __builtin_nontemporal_load(p + i + k * kReadThreads);
#pragma unroll
        for (int k = 0; k < kInFlight; k++)
            acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    for (; i < hi; i += kReadThreads) {
        const u32x4_t a = __builtin_nontemporal_load(p + i);
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9E3779B9u)
        out[0] = (float)acc;
}

__global__ __launch_bounds__(kMfmaThreads) void mfma_probe_kernel(float *__restrict__ out, int64_t iters)
{
    f32x16_t acc[kMfmaChains] = {};
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        a[i] = (__bf16)(float)((threadIdx.x + i) & 7);
        b[i] = (__bf16)(0.0009765625f * (float)i);
    }
    for (int64_t it = 0; it < iters; it++) {
#pragma unroll
        for (int t = 0; t < kMfmaChains; t++)
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[t], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int t = 0; t < kMfmaChains; t++)
#pragma unroll
        for (int r = 0; r < 16; r++)
            s += acc[t][r];
    if (s == -1.0f)  // the sums are non-negative: never taken, keeps the chains live
        out[0] = s;
}

// MODE 0: the MFMAs only; 1: the fmas only; 2: both, interleaved
constexpr int kMixThreads = 256;  // one wave per SIMD per workgroup
template <int MODE>
__global__ __launch_bounds__(kMixThreads) void mix_probe_kernel(float *__restrict__ out, int64_t iters, float s)
{
    f32x16_t acc[kMfmaChains] = {};
    bf16x8_t a, b;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        a[i] = (__bf16)(float)((threadIdx.x + i) & 7);
        b[i] = (__bf16)(0.0009765625f * (float)i);
    }
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; i++)
        v[i] = (float)(threadIdx.x & 7) + (float)i;
    for (int64_t it = 0; it < iters; it++) {
#pragma unroll
        for (int t = 0; t < kMfmaChains; t++) {
            if constexpr (MODE != 1)
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[t], 0, 0, 0);
            if constexpr (MODE != 0) {
#pragma unroll
                for (int u = 0; u < kMixFmas / 8; u++)
#pragma unroll
                    for (int i = 0; i < 8; i++)
                        v[i] = fmaf(v[i], s, 1.0f);
            }
        }
    }
    // every term is non-negative (s = 0.5: the chains stay in [0, 8]), so
    // the store is never taken; it keeps both kinds of work live
    float r = 0.0f;
#pragma unroll
    for (int t = 0; t < kMfmaChains; t++)
#pragma unroll
        for (int q = 0; q < 16; q++)
            r += acc[t][q];
#pragma unroll
    for (int i = 0; i < 8; i++)
        r += v[i];
    if (r == -1.0f)
        out[0] = r;
}

}  // namespace

hipError_t launch_read_probe(const void *buf, int64_t bytes, float *out, hipStream_t s)
{
    // at most kReadBlocks workgroups, fewer for small buffers so that every
    // thread still has a full batch of kInFlight loads (a 33 MB buffer: 1008
    // workgroups, one batch each)
    const int64_t n16 = bytes / 16;
    const int64_t per_wg = (int64_t)kReadThreads * 8;
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(kReadBlocks, n16 / per_wg));
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(kReadThreads), 0, s,
                       static_cast<const u32x4_t *>(buf), n16, out);
    return hipGetLastError();
}

hipError_t launch_mfma_probe(float *out, int64_t iters, hipStream_t s)
{
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(kMfmaBlocks), dim3(kMfmaThreads), 0, s, out, iters);
    return hipGetLastError();
}

int64_t mfma_probe_flops(int64_t iters)
{
    // waves x iterations x chains x (32 x 32 x 16 multiply-adds x 2)
    return (int64_t)kMfmaBlocks * (kMfmaThreads / 64) * iters * kMfmaChains * 32 * 32 * 16 * 2;
}

hipError_t launch_mix_probe(float *out, int64_t iters, int mode, int waves_per_simd, hipStream_t s)
{
    const dim3 grid(256u * (unsigned)waves_per_simd), block(kMixThreads);
    if (mode == 0)
        hipLaunchKernelGGL(mix_probe_kernel<0>, grid, block, 0, s, out, iters, 0.5f);
    else if (mode == 1)
        hipLaunchKernelGGL(mix_probe_kernel<1>, grid, block, 0, s, out, iters, 0.5f);
    else
        hipLaunchKernelGGL(mix_probe_kernel<2>, grid, block, 0, s, out, iters, 0.5f);
    return hipGetLastError();
}

int64_t mix_probe_valu_insts(int64_t iters, int waves_per_simd)
{
    // wave-level fp32 fma instructions of one mode-1 or mode-2 launch
    return (int64_t)256 * waves_per_simd * (kMixThreads / 64) * iters * kMfmaChains * kMixFmas;
}

}  // namespace ql
