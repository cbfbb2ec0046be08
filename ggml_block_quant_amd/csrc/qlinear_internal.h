// qlinear_internal.h -- shared declarations of the HIP implementation of the
// block-quantized linear layer (gfx950).  Host launchers live next to their
// kernels; api.hip validates arguments and dispatches to them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ql {

enum Fmt {
    FMT_Q8_0 = 0,
    FMT_Q4K = 1,
    FMT_Q6K = 2,
    FMT_Q2K = 3,
    FMT_Q3K = 4,
    FMT_Q5K = 5,
    FMT_Q4_0 = 7,
    FMT_Q4_1 = 8,
    FMT_Q5_0 = 9,
    FMT_Q5_1 = 10,
    FMT_FP8 = 12
};

// the formats served by the generic kernels (exact decode of 8 elements at
// a time, then an fp32 GEMV or a bf16 MFMA GEMM)
inline bool generic_fmt(int fmt) { return (fmt >= FMT_Q2K && fmt != 6 && fmt <= FMT_Q5_1) || fmt == FMT_FP8; }

// Byte offsets of the planes of a [N][K] block buffer (see q_blocks_bytes in
// the public header).  G = N*K/256 groups, B = N*K/32 blocks of 32.
struct Planes {
    int64_t codes;   // always 0 (Q5K, Q3K, Q5_0, Q5_1: the low bits of each code)
    int64_t scales;  // Q8_0: fp16 d per 32; Q4K, Q5K: 16-byte headers; Q6K: int8 sub-scales;
                     // Q3K: 12 bytes of 6-bit scales; Q2K: sc | m << 4 bytes
    int64_t d;       // Q6K, Q3K: fp16 d per group; Q2K: fp16 d, dmin; legacy: fp16 d per block
    int64_t total;
    int64_t hi = 0;  // Q5K, Q3K, Q5_0, Q5_1: the top bit of each code
    int64_t m = 0;   // Q4_1, Q5_1: fp16 min per block
    int64_t K = 0;   // FP8: row length (its scales are per row)
};

inline int64_t up16(int64_t v) { return (v + 15) / 16 * 16; }

inline Planes planes_of(int fmt, int64_t N, int64_t K)
{
    const int64_t E = N * K, G = E / 256, B = E / 32;
    Planes p{0, 0, 0, 0};
    switch (fmt) {
    case FMT_FP8:  // E4M3 codes [N][K], then fp32 scales [N]
        p.scales = up16(E);
        p.total = up16(p.scales + 4 * N);
        p.K = K;
        return p;
    case FMT_Q5K:
        p.hi = 128 * G;
        p.scales = 160 * G;
        p.total = 176 * G;
        return p;
    case FMT_Q3K:
        p.hi = 64 * G;
        p.scales = 96 * G;
        p.d = up16(108 * G);
        p.total = up16(p.d + 2 * G);
        return p;
    case FMT_Q2K:
        p.scales = 64 * G;
        p.d = 80 * G;
        p.total = up16(84 * G);
        return p;
    case FMT_Q4_0:
        p.d = 16 * B;
        p.total = up16(18 * B);
        return p;
    case FMT_Q4_1:
        p.d = 16 * B;
        p.m = up16(18 * B);
        p.total = up16(p.m + 2 * B);
        return p;
    case FMT_Q5_0:
        p.hi = 16 * B;
        p.d = up16(20 * B);
        p.total = up16(p.d + 2 * B);
        return p;
    case FMT_Q5_1:
        p.hi = 16 * B;
        p.d = up16(20 * B);
        p.m = up16(p.d + 2 * B);
        p.total = up16(p.m + 2 * B);
        return p;
    default:
        break;
    }
    if (fmt == FMT_Q8_0) {
        p.scales = E;
        p.total = E + E / 16;  // E/32 scales of 2 bytes
    } else if (fmt == FMT_Q4K) {
        p.scales = 128 * G;
        p.total = 144 * G;
    } else {
        // the buffer is padded to a multiple of 16 bytes, so that every
        // aligned dword holding a d value lies inside it
        p.scales = 192 * G;
        p.d = 208 * G;
        p.total = (210 * G + 15) & ~(int64_t)15;
    }
    return p;
}

// Workgroup barrier for LDS hand-offs only.  __syncthreads() also fences
// global memory, which makes the compiler drain every outstanding global
// load (s_waitcnt vmcnt(0)) -- including loads meant to stay in flight
// across the barrier.  Here only this wave's LDS accesses must be complete
// (lgkmcnt(0)); the signal fences keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Activations of the gated projection, evaluated in fp32 by the fused
// kernel and by the unfused elementwise pass alike: 0 SiLU g / (1 + e^-g),
// 1 ReLU max(g, 0), 2 sigmoid 1 / (1 + e^-g).
__device__ __forceinline__ float act_f32(int act, float g)
{
    if (act == 1)
        return g > 0.0f ? g : 0.0f;
    const float e = 1.0f + expf(-g);
    return act == 0 ? g / e : 1.0f / e;
}

hipError_t launch_isq(int fmt, const uint16_t *W, int64_t N, int64_t K, uint8_t *out,
                      hipStream_t s);
hipError_t launch_dequant(int fmt, const uint8_t *blocks, int64_t N, int64_t K, float *W,
                          hipStream_t s);
hipError_t launch_embed(int fmt, const uint8_t *blocks, int64_t N, int64_t K, const int32_t *ids,
                        int64_t n_ids, float *out, hipStream_t s);
hipError_t launch_gemv(int fmt, const uint8_t *blocks, const uint16_t *X, float *Y, int M,
                       int64_t N, int64_t K, hipStream_t s);
// whether the one-shot GEMV (X staged in LDS) takes M tokens of row length K
bool gemv_one_shot_fits(int fmt, int M, int64_t K);
bool glu_fused_fits(int fmt, int M, int64_t K);
hipError_t launch_glu_fused(int fmt, const uint8_t *gate, const uint8_t *up, const uint16_t *X, float *H, int M,
                            int64_t F, int64_t K, int act, hipStream_t s);
hipError_t launch_glu_apply(const float *G, float *H, int64_t n, int act, hipStream_t s);
hipError_t launch_gemm_bf16(int fmt, const uint8_t *blocks, const uint16_t *X, float *Y,
                            int64_t M, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_gemm_fp8(const uint8_t *wblocks, const uint8_t *xblocks, float *Y, int64_t M, int64_t N,
                           int64_t K, hipStream_t s);
hipError_t launch_gemm_i8(const uint8_t *wblocks, const uint8_t *xblocks, float *Y, int64_t M,
                          int64_t N, int64_t K, hipStream_t s);
hipError_t launch_read_probe(const void *buf, int64_t bytes, float *out, hipStream_t s);
hipError_t launch_mfma_probe(float *out, int64_t iters, hipStream_t s);
int64_t mfma_probe_flops(int64_t iters);
hipError_t launch_mix_probe(float *out, int64_t iters, int mode, int waves_per_simd, hipStream_t s);
int64_t mix_probe_valu_insts(int64_t iters, int waves_per_simd);

}  // namespace ql
