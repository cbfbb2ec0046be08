// qlinear_internal.h -- shared declarations of the HIP implementation of the
// block-quantized linear layer (gfx950).  Host launchers live next to their
// kernels; api.hip validates arguments and dispatches to them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ql {

enum Fmt { FMT_Q8_0 = 0, FMT_Q4K = 1, FMT_Q6K = 2 };

// Byte offsets of the planes of a [N][K] block buffer (see q_blocks_bytes in
// the public header).  G = N*K/256 groups.
struct Planes {
    int64_t codes;   // always 0
    int64_t scales;  // Q8_0: fp16 d per 32; Q4K: 16-byte headers; Q6K: int8 sub-scales
    int64_t d;       // Q6K only: fp16 d per group
    int64_t total;
};

inline Planes planes_of(int fmt, int64_t N, int64_t K)
{
    const int64_t E = N * K;
    Planes p{0, 0, 0, 0};
    if (fmt == FMT_Q8_0) {
        p.scales = E;
        p.total = E + E / 16;  // E/32 scales of 2 bytes
    } else if (fmt == FMT_Q4K) {
        const int64_t G = E / 256;
        p.scales = 128 * G;
        p.total = 144 * G;
    } else {
        // the buffer is padded to a multiple of 16 bytes, so that every
        // aligned dword holding a d value lies inside it
        const int64_t G = E / 256;
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
bool glu_fused_fits(int M, int64_t K);
hipError_t launch_glu_fused(int fmt, const uint8_t *gate, const uint8_t *up, const uint16_t *X, float *H, int M,
                            int64_t F, int64_t K, int act, hipStream_t s);
hipError_t launch_glu_apply(const float *G, float *H, int64_t n, int act, hipStream_t s);
hipError_t launch_gemm_bf16(int fmt, const uint8_t *blocks, const uint16_t *X, float *Y,
                            int64_t M, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_gemm_i8(const uint8_t *wblocks, const uint8_t *xblocks, float *Y, int64_t M,
                          int64_t N, int64_t K, hipStream_t s);

}  // namespace ql
