/*
 * qlinear.h -- C ABI of the block-quantized linear layer for AMD MI355X
 * (gfx950): in-situ quantization (ISQ) of bf16 weights into Q8_0, Q4K or
 * Q6K blocks, and the fused dequantize-matmul that consumes them.
 *
 * The operations come from page "Quantization types" (mistral.rs
 * reference): ISQ levels and their formats (section "Numeric shorthands",
 * column "CUDA / CPU resolves to"), the higher-precision default for
 * embeddings and output heads (section "Sensitive tensor precision"), and
 * the formats themselves (sections "Q*K family": q4k 4 bits, q6k 6 bits;
 * "Legacy GGML types": q8_0 8 bits).  The same page describes the kernel
 * split this library follows: a matrix-vector kernel for small decode
 * batches, a tiled matrix multiplication for larger batches, and
 * activations quantized once and reused across output tiles (section
 * "NVFP4").
 *
 * Conventions for every call:
 *   - Tensors are row-major.  W is [N][K] (N = output features, K = input
 *     features), X is [M][K] (M = tokens), Y is [M][N].
 *     Y[m][n] = sum_k X[m][k] * deq(W)[n][k]   (Y = X . deq(W)^T).
 *   - bf16 and fp16 values are passed as their 16-bit patterns.
 *   - Device pointers must come from the same HIP device as the stream,
 *     be non-NULL and 16-byte aligned.  Buffers are owned by the caller;
 *     the library allocates nothing and keeps no state, so every call is
 *     thread-safe and re-entrant.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls return
 *     once the work is enqueued; a fault inside a kernel surfaces at the
 *     caller's next synchronization.
 *   - Status codes are below.  An argument error returns before anything
 *     is launched.  Q_EHIP means the HIP runtime refused a launch.
 *   - Inputs with Inf or NaN break a precondition: the results are then
 *     unspecified (but the call still returns).
 *
 * Block formats (quantized along K, each row independently, in groups of
 * 256 consecutive elements of a row; the byte layout is given at
 * q_blocks_bytes below):
 *   Q8_0: blocks of 32, fp16 scale d = max|x|/127, int8 codes
 *         q = round-half-away-from-zero(x / d), 34 bytes per 32 elements.
 *   Q4K:  super-blocks of 256 = 8 sub-blocks of 32, 6-bit scale and 6-bit
 *         min per sub-block, fp16 d and dmin, 4-bit codes, w = d*sc*q -
 *         dmin*m, 144 bytes per 256 elements.
 *   Q6K:  super-blocks of 256 = 16 sub-blocks of 16, 8-bit sub-scales, one
 *         fp16 d, 6-bit symmetric codes, w = d*sc*q, 210 bytes per 256.
 * Further formats (levels 5, 3, 2 of the shorthand table and the legacy
 * 32-element types; same rules with other widths, GGML byte counts):
 *   Q5K:  as Q4K with 5-bit codes, 176 bytes per 256.
 *   Q3K:  16 sub-blocks of 16, 6-bit scales, one fp16 d, symmetric codes
 *         in [-4, 3], w = d*sc*q, 110 bytes per 256.
 *   Q2K:  16 sub-blocks of 16, 4-bit scales and mins, fp16 d and dmin,
 *         2-bit codes, w = d*sc*q - dmin*m, 84 bytes per 256.
 *   Q4_0 / Q5_0: blocks of 32, fp16 d = max|x| / 7 (/ 15), codes in
 *         [-8, 7] ([-16, 15]), 18 (22) bytes per 32.
 *   Q4_1 / Q5_1: blocks of 32, fp16 d = (max - min) / 15 (/ 31) and fp16
 *         m = min, codes in [0, 15] ([0, 31]), w = d*q + m, 20 (24) bytes.
 * These run on generic kernels (exact decode of 8 elements, then an fp32
 * GEMV or a bf16 MFMA GEMM) and need K % 256 == 0 as well.
 *   FP8:  E4M3 codes (no infinities: largest finite 448) with one fp32 scale
 *         per row s = max|x| / 448, codes E4M3(x / s) rounded to nearest
 *         even and saturated (page "Quantization types", section "FP8":
 *         symmetric E4M3 with channel scales).  W8A16 on the generic
 *         kernels; W8A8 with per-token activation scales on QPATH_MFMA_FP8.
 */
#ifndef QLINEAR_H
#define QLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Quantization types.  All are implemented except Q8K and Q8_1, which the
 * pages' tables name (so that the level and promotion helpers can answer
 * for every row) and the compute calls reject with Q_ENOTSUP. */
typedef enum {
    QFMT_Q8_0 = 0,
    QFMT_Q4K = 1,
    QFMT_Q6K = 2,
    QFMT_Q2K = 3,
    QFMT_Q3K = 4,
    QFMT_Q5K = 5,
    QFMT_Q8K = 6,
    QFMT_Q4_0 = 7,
    QFMT_Q4_1 = 8,
    QFMT_Q5_0 = 9,
    QFMT_Q5_1 = 10,
    QFMT_Q8_1 = 11,
    QFMT_FP8 = 12 /* E4M3 codes with one fp32 scale per row (page section "FP8") */
} qfmt;

/* Matmul path.  AUTO: GEMV for M <= 2, and for M <= 4 where the one-shot
 * GEMV takes the row length (and for Q5K, Q3K, Q2K and the legacy
 * 32-element formats), and for five or six Q4K tokens on weights of at most
 * 2^25 elements with K <= 4096; bf16 MFMA GEMM above (crossovers measured
 * on MI355X at decode shapes). */
typedef enum {
    QPATH_AUTO = 0,
    QPATH_GEMV = 1,      /* fused dequant-GEMV, M <= 8 only */
    QPATH_MFMA_BF16 = 2, /* weights dequantized to bf16 in LDS, MFMA bf16 */
    QPATH_MFMA_I8 = 3,   /* Q8_0 weights only: X quantized to Q8_0, int8 MFMA */
    QPATH_MFMA_FP8 = 4   /* FP8 weights only: X quantized per token to E4M3, FP8 MFMA (W8A8) */
} qpath;

enum {
    Q_OK = 0,
    Q_EINVAL = -1,  /* NULL pointer, unknown format/path, bad workspace */
    Q_ESHAPE = -2,  /* M, N, K out of range or K not a multiple of 256 (Q8_0: 32) */
    Q_EALIGN = -3,  /* a pointer is not 16-byte aligned */
    Q_ENOTSUP = -4, /* format or path not implemented for these arguments */
    Q_EHIP = -5,    /* the HIP runtime refused a launch or a query */
    Q_ESCRATCH = -6 /* qmatmul_static: the activation blocks exceed the fixed buffer */
};

/* Largest accepted dimension values (element counts N*K and M*K must also
 * stay below 2^40). */
#define QLINEAR_MAX_M 65536
#define QLINEAR_MAX_N (1 << 24)
#define QLINEAR_MAX_K (1 << 20)

/* Bytes of the block buffer of a [N][K] tensor in `fmt` (page "Quantization
 * types", sections "Q*K family" and "Legacy GGML types": the formats and
 * their bit widths; the byte counts per block are the formats' own):
 * 34*N*K/32 (Q8_0),
 * 144*N*K/256 (Q4K), 210*N*K/256 rounded up to a multiple of 16 (Q6K; the
 * padding bytes are zero after isq_quantize).  Returns 0 for an unsupported
 * format or an invalid shape.  The buffer is made of planes, each 16-byte aligned
 * (G = N*K/256 groups, group g = row n, columns 256*kb .. 256*kb+255 with
 * g = n*K/256 + kb):
 *   Q8_0: [codes int8 N*K, row-major][d fp16 N*K/32, row-major]
 *   Q4K:  [codes G*128][headers G*16: d, dmin, 12 bytes of 6-bit sc/m]
 *   Q6K:  [codes G*192: 128 bytes low 4 bits + 64 bytes high 2 bits of
 *          q+32][sub-scales G*16 int8][d G*2 fp16]
 * Further formats (natural element order; u = stored code; B = N*K/32;
 * every plane start rounded up to 16 bytes, padding zero):
 *   Q5K:  [low nibbles G*128][top bits G*32][Q4K-style headers G*16]
 *   Q3K:  [low 2 bits of u = q+4, G*64][top bits G*32][6-bit scales G*12][d G*2]
 *   Q2K:  [codes 2-bit G*64][sc | m << 4, G*16][d, dmin G*4]
 *   Q4_0: [nibbles of q+8, B*16][d B*2]      Q4_1: [nibbles B*16][d B*2][m B*2]
 *   Q5_0: [low nibbles of q+16, B*16][fifth bits B*4][d B*2]
 *   Q5_1: [low nibbles B*16][fifth bits B*4][d B*2][m B*2]
 *   FP8:  [E4M3 codes N*K, row-major][fp32 scale per row N*4]           */
size_t q_blocks_bytes(int fmt, int64_t N, int64_t K);

/* In-situ quantization (page "Quantization types": ISQ, --isq N).
 * W_bf16: device [N][K] bf16.  out_blocks: device, q_blocks_bytes(fmt,N,K)
 * bytes, fully overwritten.  Codes and scales are bit-exact with the
 * library's reference definition (fp32 IEEE arithmetic, fp16 scales rounded
 * to nearest even after clamping to 65504, round-half-away-from-zero codes).
 * Requires K % 256 == 0 (Q8_0: K % 32 == 0), 1 <= N <= QLINEAR_MAX_N; the
 * gaps between planes and the end padding are written as zeros. */
int isq_quantize(int fmt, const void *W_bf16, int64_t N, int64_t K, void *out_blocks,
                 void *stream);

/* Activation quantization to Q8_0 for the int8 path (page "Quantization
 * types", section "NVFP4": activations quantized once and reused across
 * output tiles; section "FP8": dynamic per-token activation quantizers).
 * X_bf16 device [M][K]; out_blocks device, q_blocks_bytes(QFMT_Q8_0, M, K)
 * bytes: codes [M][K] int8 then scales [M][K/32] fp16 -- the same rule and
 * layout as isq_quantize(QFMT_Q8_0, ...). */
int q_act_quantize(const void *X_bf16, int64_t M, int64_t K, void *out_blocks, void *stream);

/* Quantized matmul Y = X . deq(W)^T on the AUTO path (no workspace): the
 * matrix-vector kernel for small decode batches and tiled MFMA kernels for
 * larger ones (page "Quantization types", section "NVFP4", which splits a
 * quantized linear layer's kernels that way; section "FP8": the weight tile
 * is dequantized inside the GEMM).
 * blocks: device, from isq_quantize(fmt, W, N, K).  X_bf16: device [M][K].
 * Y_fp32: device [M][N], overwritten (not accumulated).
 * 1 <= M <= QLINEAR_MAX_M, K % 256 == 0; Q8_0 weights also take rows that end
 * in a tail of whole blocks (K % 32 == 0, K >= 32: the GEMV kernels, and for
 * the MFMA path the generic exact-decode kernel).
 * Accuracy: each output is within 1e-3 of sum_k |w||x| of the exact product,
 * with one known exception: the Q4K kernels that take the codes exactly
 * (decode GEMV, batched decode up to 32 tokens) form a sub-block's sum as
 * S * sum(u x) - M * sum(x), whose error is bounded by ~2^-23 (S * 15 + M)
 * sum |x| instead; on sub-blocks whose other weights dequantize to exactly 0
 * while X is (near) 0 at the nonzero ones, that exceeds the bar. */
int qmatmul(int fmt, const void *blocks, const void *X_bf16, float *Y_fp32, int64_t M,
            int64_t N, int64_t K, void *stream);

/* Workspace bytes `qmatmul_ex` needs for (fmt, path, M, K) -- room for the
 * activations quantized once per call and reused by every output tile (page
 * "Quantization types", section "NVFP4"; section "FP8": dynamic per-token
 * activation quantizers): the Q8_0 blocks
 * of X for QPATH_MFMA_I8 (q_blocks_bytes(QFMT_Q8_0, M, K)), its FP8 codes
 * and scales for QPATH_MFMA_FP8 (q_blocks_bytes(QFMT_FP8, M, K)), 0 otherwise. */
size_t qmatmul_workspace_bytes(int fmt, int path, int64_t M, int64_t K);

/* Quantized matmul on an explicit path.  QPATH_GEMV needs M <= 8.
 * QPATH_MFMA_I8 needs fmt == QFMT_Q8_0, K % 256 == 0 and a device workspace of at least
 * qmatmul_workspace_bytes() bytes (16-byte aligned); on return it holds
 * the Q8_0 blocks of X (codes then scales).  QPATH_MFMA_FP8 (page section
 * "FP8": dynamic per-token W8A8) needs fmt == QFMT_FP8 and a workspace of
 * qmatmul_workspace_bytes() bytes, which on return holds X quantized per
 * token (E4M3 codes, then one fp32 scale per row); Y = s_x s_w * the exact
 * E4M3 products summed in fp32.  Other paths ignore the workspace. */
int qmatmul_ex(int fmt, const void *blocks, const void *X_bf16, float *Y_fp32, int64_t M,
               int64_t N, int64_t K, int path, void *workspace, size_t workspace_bytes,
               void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): qmatmul_ex
 * without a caller workspace.  QPATH_MFMA_I8 and QPATH_MFMA_FP8 keep X's
 * activation blocks in a buffer of QLINEAR_STATIC_SCRATCH_BYTES that the
 * library holds in device memory, one per GPU, from the first such call on
 * that GPU (with that GPU current, hipGetDevice) until the process ends;
 * a call whose qmatmul_workspace_bytes exceeds it returns Q_ESCRATCH before
 * anything is launched.  The buffer is fully rewritten by each call that
 * uses it (nothing in it needs to start at zero), and every call on one
 * GPU shares it: calls whose work overlaps in time on one GPU (different
 * streams, or no ordering between host threads) race; calls on one stream
 * are ordered.  The other paths need no workspace and run as in qmatmul_ex.
 * Nothing is allocated by the call itself; the stream must belong to the
 * current device. */
#define QLINEAR_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
int qmatmul_static(int fmt, const void *blocks, const void *X_bf16, float *Y_fp32, int64_t M,
                   int64_t N, int64_t K, int path, void *stream);

/* Gated feed-forward projection (page "Quantization types", section
 * "NVFP4": compatible gated feed-forward projections fuse the activation
 * and the multiplication, keeping the activation and product rounding of
 * the unfused path, for SiLU, ReLU and sigmoid):
 *   H[m][f] = act(G[m][f]) * U[m][f],  G = X . deq(Wg)^T,  U = X . deq(Wu)^T,
 * with G and U accumulated in fp32 and act(g) = g / (1 + e^-g) (SiLU),
 * max(g, 0) (ReLU) or 1 / (1 + e^-g) (sigmoid) evaluated in fp32.
 * gate_blocks / up_blocks: device, isq_quantize(fmt, W, F, K) of the [F][K]
 * gate and up weights (a packed [2F][K] checkpoint tensor is quantized as
 * its two halves).  X_bf16: device [M][K].  H_fp32: device [M][F],
 * overwritten.  For Q8_0, Q4K and Q6K with M <= 2 and K <= 8192, M = 3 and
 * K <= 8192, or M = 4 and K <= 6144 (not Q8_0), one fused kernel computes the
 * gate and up rows of each output together and needs no workspace;
 * otherwise G goes through `workspace` (qmatmul_glu_workspace_bytes bytes,
 * 16-byte aligned; Q_EINVAL without it) and U through H, followed by an
 * elementwise pass with the same fp32 expression. */
enum { QACT_SILU = 0, QACT_RELU = 1, QACT_SIGMOID = 2 };
size_t qmatmul_glu_workspace_bytes(int fmt, int64_t M, int64_t F, int64_t K);
int qmatmul_glu(int fmt, const void *gate_blocks, const void *up_blocks, const void *X_bf16, float *H_fp32,
                int64_t M, int64_t F, int64_t K, int act, void *workspace, size_t workspace_bytes,
                void *stream);

/* Quantized embedding lookup (page "Quantization types", section
 * "Sensitive tensor precision": token embeddings are stored quantized, and
 * a tied output head reuses the embedding instead of a second copy -- the
 * same block buffer serves this call and qmatmul).
 * blocks: device, from isq_quantize(fmt, E, N, K) of the [N][K] table.
 * ids: device int32 [n_ids], 4-byte aligned.  out_fp32: device [n_ids][K],
 * row i = the exact dequantized row ids[i] (bit-exact: fp32 holds Q8_0 and
 * Q6K weights exactly and Q4K's d*sc*q - dmin*m rounded once).  An id
 * outside [0, N) gives a row of zeros.  n_ids == 0 launches nothing;
 * 0 <= n_ids <= QLINEAR_MAX_EMBED_IDS. */
#define QLINEAR_MAX_EMBED_IDS (1 << 24)
int q_embed(int fmt, const void *blocks, int64_t N, int64_t K, const int32_t *ids, int64_t n_ids,
            float *out_fp32, void *stream);

/* Test aid: exact dequantization of a block buffer to fp32 [N][K] (device). */
int q_dequantize(int fmt, const void *blocks, int64_t N, int64_t K, float *W_fp32,
                 void *stream);

/* Measurement aids, not part of the computation: the two ceilings the
 * benchmark reports beside the published peaks (page "Quantization types",
 * section "NVFP4": measured latencies, with the caveat that repeated
 * projections benefit from the cache -- so the read ceiling is taken on a
 * buffer read once per launch).
 * q_probe_read: every byte of device buffer `buf` read once with 16-byte
 * non-temporal loads; `bytes` a positive multiple of 16, `buf` 16-byte
 * aligned; `out` a device float that is written only if the XOR of all
 * words read equals 0x9E3779B9 (it keeps the loads from being removed).
 * q_probe_mfma: `iters` rounds of four dependent v_mfma_f32_32x32x16_bf16
 * chains in each of 8192 waves (two per SIMD), no memory traffic; `out`
 * as above (never written for iters >= 0).  q_probe_mfma_flops: the FLOP
 * count of one q_probe_mfma call (0 for iters < 0).
 * q_probe_mix: the q_probe_mfma loop with sixteen independent fp32 fmas
 * after each MFMA, in 1024 * waves_per_simd waves (waves_per_simd per SIMD
 * of the 256 CUs); `mode` 0 runs the MFMAs only, 1 the fmas only, 2 both
 * interleaved in one instruction stream (how far a kernel's VALU work can
 * hide behind its MFMAs at that occupancy); `out` as above; Q_ESHAPE for
 * iters < 0, a mode outside 0..2 or waves_per_simd outside 1..8.
 * q_probe_mix_valu: the wave-level fma instructions of one call in mode 1
 * or 2 (each MFMA of mode 0 or 2 stands for 16 of them; 0 for invalid
 * arguments). */
int q_probe_read(const void *buf, int64_t bytes, float *out, void *stream);
int q_probe_mfma(float *out, int64_t iters, void *stream);
int64_t q_probe_mfma_flops(int64_t iters);
int q_probe_mix(float *out, int64_t iters, int mode, int waves_per_simd, void *stream);
int64_t q_probe_mix_valu(int64_t iters, int waves_per_simd);

/* ISQ level -> format, page "Quantization types", section "Numeric
 * shorthands", column "CUDA / CPU resolves to": 2 Q2K, 3 Q3K, 4 Q4K, 5 Q5K,
 * 6 Q6K, 8 Q8_0.  Other levels: Q_EINVAL.  *out_fmt may name a format this
 * library does not implement (q_fmt_supported tells). */
int isq_resolve_level(int level, int *out_fmt);

/* Effective type of token embeddings and output heads for a model whose
 * default type is `model_default`, page "Quantization types", section
 * "Sensitive tensor precision": Q2K, Q3K, Q4K, Q4_0, Q4_1 -> Q6K; Q5K, Q6K,
 * Q8K, Q5_0, Q5_1, Q8_0, Q8_1 -> Q8_0. */
int isq_sensitive_fmt(int model_default, int *out_fmt);

/* The type one tensor gets: an explicit per-tensor type (explicit_fmt >= 0)
 * takes precedence; otherwise the level's format, promoted by
 * isq_sensitive_fmt when is_embedding_or_head is nonzero (same section). */
int isq_tensor_fmt(int level, int is_embedding_or_head, int explicit_fmt, int *out_fmt);

/* 1 if the compute calls implement `fmt`, else 0. */
int q_fmt_supported(int fmt);

/* Name of a format ("q8_0", "q4k", ...) or NULL. */
const char *q_fmt_name(int fmt);

/* Static description of a status code. */
const char *q_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* QLINEAR_H */
