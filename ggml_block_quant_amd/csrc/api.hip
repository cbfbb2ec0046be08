// api.hip -- the C ABI declared in include/qlinear.h: argument checks, path
// selection and launches.  Every check happens before any HIP call, so an
// argument error never launches anything.
#include "../../include/qlinear.h"
#include "gemv_fp8.h"
#include "qlinear_internal.h"

#include <stdint.h>

#include <atomic>
#include <mutex>

namespace {

bool implemented(int fmt)
{
    return fmt == QFMT_Q8_0 || fmt == QFMT_Q4K || fmt == QFMT_Q6K || ql::generic_fmt(fmt);
}
bool known(int fmt) { return fmt >= QFMT_Q8_0 && fmt <= QFMT_FP8; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxElems = int64_t(1) << 40;

// shape of a [rows][K] tensor in `fmt`: K % 256 (Q8_0: K % 32)
int check_tensor(int fmt, int64_t rows, int64_t K, int64_t max_rows)
{
    if (rows < 1 || rows > max_rows || K < 1 || K > QLINEAR_MAX_K)
        return Q_ESHAPE;
    if (K % (fmt == QFMT_Q8_0 ? 32 : 256) != 0)
        return Q_ESHAPE;
    if (rows * K > kMaxElems)
        return Q_ESHAPE;
    return Q_OK;
}

int status_of(hipError_t e)
{
    if (e == hipSuccess)
        return Q_OK;
    if (e == hipErrorNotSupported)
        return Q_ENOTSUP;
    return Q_EHIP;
}

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

int matmul_args(int fmt, const void *blocks, const void *X, const float *Y, int64_t M, int64_t N,
                int64_t K)
{
    if (!known(fmt))
        return Q_EINVAL;
    if (!implemented(fmt))
        return Q_ENOTSUP;
    if (!blocks || !X || !Y)
        return Q_EINVAL;
    if (!aligned16(blocks) || !aligned16(X) || !aligned16(Y))
        return Q_EALIGN;
    // K % 256 (Q8_0: K % 32, the tail of whole blocks)
    const int kq = fmt == QFMT_Q8_0 ? 32 : 256;
    if (M < 1 || M > QLINEAR_MAX_M || N < 1 || N > QLINEAR_MAX_N || K < kq || K > QLINEAR_MAX_K || K % kq != 0 ||
        N * K > kMaxElems || M * K > kMaxElems || M * N > kMaxElems)
        return Q_ESHAPE;
    return Q_OK;
}

// the GEMV of a format: FP8 one- and two-token shapes on their own one-shot
// kernel, everything else on the GEMV kernels of the format
int gemv(int fmt, const uint8_t *B, const uint16_t *X, float *Y, int64_t M, int64_t N, int64_t K, hipStream_t s)
{
    if (fmt == QFMT_FP8) {
        hipError_t e = hipSuccess;
        if (ql::launch_gemv_fp8(B, X, Y, (int)M, N, K, s, e))
            return status_of(e);
    }
    return status_of(ql::launch_gemv(fmt, B, X, Y, (int)M, N, K, s));
}

// The fixed device buffer of qmatmul_static: one copy per GPU, held until the
// process ends.  Host code never uses the array's name as an address: the
// device address of each GPU's copy comes from hipGetSymbolAddress, taken
// once per device with that device current.
__device__ __align__(256) uint8_t scratch[QLINEAR_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> scratch_addr[kMaxDevices];
std::mutex scratch_mu;

int scratch_of_current_device(void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return Q_EHIP;
    if (dev < 0 || dev >= kMaxDevices)
        return Q_ENOTSUP;
    void *p = scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(scratch_mu);
        p = scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
                return Q_EHIP;
            scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return Q_OK;
}

}  // namespace

extern "C" {

size_t q_blocks_bytes(int fmt, int64_t N, int64_t K)
{
    if (!implemented(fmt) || check_tensor(fmt, N, K, QLINEAR_MAX_N) != Q_OK)
        return 0;
    return (size_t)ql::planes_of(fmt, N, K).total;
}

int isq_quantize(int fmt, const void *W_bf16, int64_t N, int64_t K, void *out_blocks, void *stream)
{
    if (!known(fmt))
        return Q_EINVAL;
    if (!implemented(fmt))
        return Q_ENOTSUP;
    if (!W_bf16 || !out_blocks)
        return Q_EINVAL;
    if (!aligned16(W_bf16) || !aligned16(out_blocks))
        return Q_EALIGN;
    const int st = check_tensor(fmt, N, K, QLINEAR_MAX_N);
    if (st != Q_OK)
        return st;
    return status_of(ql::launch_isq(fmt, static_cast<const uint16_t *>(W_bf16), N, K,
                                    static_cast<uint8_t *>(out_blocks), as_stream(stream)));
}

int q_act_quantize(const void *X_bf16, int64_t M, int64_t K, void *out_blocks, void *stream)
{
    if (!X_bf16 || !out_blocks)
        return Q_EINVAL;
    if (!aligned16(X_bf16) || !aligned16(out_blocks))
        return Q_EALIGN;
    const int st = check_tensor(QFMT_Q8_0, M, K, QLINEAR_MAX_M);
    if (st != Q_OK)
        return st;
    return status_of(ql::launch_isq(ql::FMT_Q8_0, static_cast<const uint16_t *>(X_bf16), M, K,
                                    static_cast<uint8_t *>(out_blocks), as_stream(stream)));
}

size_t qmatmul_workspace_bytes(int fmt, int path, int64_t M, int64_t K)
{
    if (path == QPATH_MFMA_I8 && fmt == QFMT_Q8_0 && K % 256 == 0 && check_tensor(QFMT_Q8_0, M, K, QLINEAR_MAX_M) == Q_OK)
        return (size_t)ql::planes_of(ql::FMT_Q8_0, M, K).total;
    if (path == QPATH_MFMA_FP8 && fmt == QFMT_FP8 && check_tensor(QFMT_FP8, M, K, QLINEAR_MAX_M) == Q_OK)
        return (size_t)ql::planes_of(ql::FMT_FP8, M, K).total;
    return 0;
}

int qmatmul_ex(int fmt, const void *blocks, const void *X_bf16, float *Y_fp32, int64_t M, int64_t N,
               int64_t K, int path, void *workspace, size_t workspace_bytes, void *stream)
{
    int st = matmul_args(fmt, blocks, X_bf16, Y_fp32, M, N, K);
    if (st != Q_OK)
        return st;
    const auto *B = static_cast<const uint8_t *>(blocks);
    const auto *X = static_cast<const uint16_t *>(X_bf16);
    const hipStream_t s = as_stream(stream);
    switch (path) {
    case QPATH_AUTO:
        // measured crossovers on MI355X: the fused GEMV wins for one or two
        // tokens, and for three or four where its one-shot kernel takes the
        // shape (Q6K 14336 x 4096, 3 tokens: 13.2 vs 21.7 us on the MFMA
        // stream); for the generic formats, whose MFMA kernel streams the
        // weights less well, up to four (Q5K 14336 x 4096, 3 tokens: 33.6 vs
        // 54.3 us); beyond, the MFMA weight stream
        // (and for five or six Q4K tokens on weights of at most 2^25
        // elements where the one-shot kernel takes them: 4096 x 4096 at
        // five tokens 6.5 vs 7.2 us, 6144 x 4096 8.6 vs 9.3 us; from
        // 14336 x 4096 or eight tokens the MFMA stream is faster)
        if (M <= 2 || (M <= 4 && ((ql::generic_fmt(fmt) && fmt != QFMT_FP8) || ql::gemv_one_shot_fits(fmt, (int)M, K))) ||
            (fmt == QFMT_Q4K && M <= 6 && N * K <= ((int64_t)1 << 25) && ql::gemv_one_shot_fits(fmt, (int)M, K))) {
            st = gemv(fmt, B, X, Y_fp32, M, N, K, s);
            if (st != Q_ENOTSUP)
                return st;
        }
        return status_of(ql::launch_gemm_bf16(fmt, B, X, Y_fp32, M, N, K, s));
    case QPATH_GEMV:
        if (M > 8)
            return Q_ESHAPE;
        return gemv(fmt, B, X, Y_fp32, M, N, K, s);
    case QPATH_MFMA_BF16:
        return status_of(ql::launch_gemm_bf16(fmt, B, X, Y_fp32, M, N, K, s));
    case QPATH_MFMA_I8: {
        if (fmt != QFMT_Q8_0)
            return Q_ENOTSUP;
        if (K % 256 != 0)
            return Q_ESHAPE;  // the int8 kernels take the scales of two blocks per dword
        if (!workspace)
            return Q_EINVAL;
        if (!aligned16(workspace))
            return Q_EALIGN;
        if (workspace_bytes < qmatmul_workspace_bytes(fmt, path, M, K))
            return Q_EINVAL;
        auto *ws = static_cast<uint8_t *>(workspace);
        st = status_of(ql::launch_isq(ql::FMT_Q8_0, X, M, K, ws, s));
        if (st != Q_OK)
            return st;
        return status_of(ql::launch_gemm_i8(B, ws, Y_fp32, M, N, K, s));
    }
    case QPATH_MFMA_FP8: {
        if (fmt != QFMT_FP8)
            return Q_ENOTSUP;
        if (!workspace)
            return Q_EINVAL;
        if (!aligned16(workspace))
            return Q_EALIGN;
        if (workspace_bytes < qmatmul_workspace_bytes(fmt, path, M, K))
            return Q_EINVAL;
        auto *ws = static_cast<uint8_t *>(workspace);
        st = status_of(ql::launch_isq(ql::FMT_FP8, X, M, K, ws, s));
        if (st != Q_OK)
            return st;
        return status_of(ql::launch_gemm_fp8(B, ws, Y_fp32, M, N, K, s));
    }
    default:
        return Q_EINVAL;
    }
}

int qmatmul(int fmt, const void *blocks, const void *X_bf16, float *Y_fp32, int64_t M, int64_t N, int64_t K,
            void *stream)
{
    return qmatmul_ex(fmt, blocks, X_bf16, Y_fp32, M, N, K, QPATH_AUTO, nullptr, 0, stream);
}

int qmatmul_static(int fmt, const void *blocks, const void *X_bf16, float *Y_fp32, int64_t M, int64_t N, int64_t K,
                   int path, void *stream)
{
    const int st = matmul_args(fmt, blocks, X_bf16, Y_fp32, M, N, K);
    if (st != Q_OK)
        return st;
    const size_t need = qmatmul_workspace_bytes(fmt, path, M, K);
    if (need == 0)  // no workspace on this path (or invalid arguments, which qmatmul_ex reports)
        return qmatmul_ex(fmt, blocks, X_bf16, Y_fp32, M, N, K, path, nullptr, 0, stream);
    if (need > QLINEAR_STATIC_SCRATCH_BYTES)
        return Q_ESCRATCH;
    void *ws = nullptr;
    const int sst = scratch_of_current_device(&ws);
    if (sst != Q_OK)
        return sst;
    return qmatmul_ex(fmt, blocks, X_bf16, Y_fp32, M, N, K, path, ws, need, stream);
}

size_t qmatmul_glu_workspace_bytes(int fmt, int64_t M, int64_t F, int64_t K)
{
    // every valid shape (check_tensor: K % 256, Q8_0 K % 32) that the fused
    // kernel does not take needs G in the workspace
    if (!implemented(fmt) || M < 1 || M > QLINEAR_MAX_M || check_tensor(fmt, F, K, QLINEAR_MAX_N) != Q_OK ||
        M * F > kMaxElems)
        return 0;
    return ql::glu_fused_fits(fmt, (int)M, K) ? 0 : (size_t)(4 * M * F);
}

int qmatmul_glu(int fmt, const void *gate_blocks, const void *up_blocks, const void *X_bf16, float *H_fp32,
                int64_t M, int64_t F, int64_t K, int act, void *workspace, size_t workspace_bytes, void *stream)
{
    int st = matmul_args(fmt, gate_blocks, X_bf16, H_fp32, M, F, K);
    if (st != Q_OK)
        return st;
    if (!up_blocks)
        return Q_EINVAL;
    if (!aligned16(up_blocks))
        return Q_EALIGN;
    if (act < QACT_SILU || act > QACT_SIGMOID)
        return Q_EINVAL;
    const auto *Bg = static_cast<const uint8_t *>(gate_blocks);
    const auto *Bu = static_cast<const uint8_t *>(up_blocks);
    const auto *X = static_cast<const uint16_t *>(X_bf16);
    const hipStream_t s = as_stream(stream);
    if (ql::glu_fused_fits(fmt, (int)M, K))
        return status_of(ql::launch_glu_fused(fmt, Bg, Bu, X, H_fp32, (int)M, F, K, act, s));
    // two matmuls and the elementwise product: G in the workspace, U in H
    if (!workspace)
        return Q_EINVAL;
    if (!aligned16(workspace))
        return Q_EALIGN;
    if (workspace_bytes < qmatmul_glu_workspace_bytes(fmt, M, F, K))
        return Q_EINVAL;
    float *G = static_cast<float *>(workspace);
    st = qmatmul(fmt, gate_blocks, X_bf16, G, M, F, K, stream);
    if (st != Q_OK)
        return st;
    st = qmatmul(fmt, up_blocks, X_bf16, H_fp32, M, F, K, stream);
    if (st != Q_OK)
        return st;
    return status_of(ql::launch_glu_apply(G, H_fp32, M * F, act, s));
}

int q_dequantize(int fmt, const void *blocks, int64_t N, int64_t K, float *W_fp32, void *stream)
{
    if (!known(fmt))
        return Q_EINVAL;
    if (!implemented(fmt))
        return Q_ENOTSUP;
    if (!blocks || !W_fp32)
        return Q_EINVAL;
    if (!aligned16(blocks) || !aligned16(W_fp32))
        return Q_EALIGN;
    const int st = check_tensor(fmt, N, K, QLINEAR_MAX_N);
    if (st != Q_OK)
        return st;
    return status_of(ql::launch_dequant(fmt, static_cast<const uint8_t *>(blocks), N, K, W_fp32,
                                        as_stream(stream)));
}

int q_embed(int fmt, const void *blocks, int64_t N, int64_t K, const int32_t *ids, int64_t n_ids, float *out_fp32,
            void *stream)
{
    if (!known(fmt))
        return Q_EINVAL;
    if (!implemented(fmt))
        return Q_ENOTSUP;
    if (!blocks || !ids || !out_fp32)
        return Q_EINVAL;
    if (!aligned16(blocks) || !aligned16(out_fp32) || (reinterpret_cast<uintptr_t>(ids) & 3u) != 0)
        return Q_EALIGN;
    const int st = check_tensor(fmt, N, K, QLINEAR_MAX_N);
    if (st != Q_OK)
        return st;
    if (n_ids < 0 || n_ids > QLINEAR_MAX_EMBED_IDS || n_ids * K > kMaxElems)
        return Q_ESHAPE;
    if (n_ids == 0)
        return Q_OK;
    return status_of(ql::launch_embed(fmt, static_cast<const uint8_t *>(blocks), N, K, ids, n_ids, out_fp32,
                                      as_stream(stream)));
}

int q_probe_read(const void *buf, int64_t bytes, float *out, void *stream)
{
    if (!buf || !out)
        return Q_EINVAL;
    if (!aligned16(buf))
        return Q_EALIGN;
    if (bytes < 16 || bytes % 16 != 0 || bytes > kMaxElems)
        return Q_ESHAPE;
    return status_of(ql::launch_read_probe(buf, bytes, out, as_stream(stream)));
}

int q_probe_mfma(float *out, int64_t iters, void *stream)
{
    if (!out)
        return Q_EINVAL;
    if (iters < 0 || iters > (int64_t(1) << 24))
        return Q_ESHAPE;
    if (iters == 0)
        return Q_OK;
    return status_of(ql::launch_mfma_probe(out, iters, as_stream(stream)));
}

int64_t q_probe_mfma_flops(int64_t iters) { return iters < 0 ? 0 : ql::mfma_probe_flops(iters); }

int q_probe_mix(float *out, int64_t iters, int mode, int waves_per_simd, void *stream)
{
    if (!out)
        return Q_EINVAL;
    if (iters < 0 || iters > (int64_t(1) << 24) || mode < 0 || mode > 2 || waves_per_simd < 1 || waves_per_simd > 8)
        return Q_ESHAPE;
    if (iters == 0)
        return Q_OK;
    return status_of(ql::launch_mix_probe(out, iters, mode, waves_per_simd, as_stream(stream)));
}

int64_t q_probe_mix_valu(int64_t iters, int waves_per_simd)
{
    return iters < 0 || waves_per_simd < 1 || waves_per_simd > 8 ? 0 : ql::mix_probe_valu_insts(iters, waves_per_simd);
}

int isq_resolve_level(int level, int *out_fmt)
{
    if (!out_fmt)
        return Q_EINVAL;
    int f;
    switch (level) {
    case 2: f = QFMT_Q2K; break;
    case 3: f = QFMT_Q3K; break;
    case 4: f = QFMT_Q4K; break;
    case 5: f = QFMT_Q5K; break;
    case 6: f = QFMT_Q6K; break;
    case 8: f = QFMT_Q8_0; break;
    default: return Q_EINVAL;
    }
    *out_fmt = f;
    return Q_OK;
}

int isq_sensitive_fmt(int model_default, int *out_fmt)
{
    if (!out_fmt)
        return Q_EINVAL;
    switch (model_default) {
    case QFMT_Q2K:
    case QFMT_Q3K:
    case QFMT_Q4K:
    case QFMT_Q4_0:
    case QFMT_Q4_1:
        *out_fmt = QFMT_Q6K;
        return Q_OK;
    case QFMT_Q5K:
    case QFMT_Q6K:
    case QFMT_Q8K:
    case QFMT_Q5_0:
    case QFMT_Q5_1:
    case QFMT_Q8_0:
    case QFMT_Q8_1:
        *out_fmt = QFMT_Q8_0;
        return Q_OK;
    default:
        return Q_EINVAL;
    }
}

int isq_tensor_fmt(int level, int is_embedding_or_head, int explicit_fmt, int *out_fmt)
{
    if (!out_fmt)
        return Q_EINVAL;
    if (explicit_fmt >= 0) {
        if (!known(explicit_fmt))
            return Q_EINVAL;
        *out_fmt = explicit_fmt;
        return Q_OK;
    }
    int f;
    int st = isq_resolve_level(level, &f);
    if (st != Q_OK)
        return st;
    if (is_embedding_or_head) {
        st = isq_sensitive_fmt(f, &f);
        if (st != Q_OK)
            return st;
    }
    *out_fmt = f;
    return Q_OK;
}

int q_fmt_supported(int fmt) { return implemented(fmt) ? 1 : 0; }

const char *q_fmt_name(int fmt)
{
    static const char *names[] = {"q8_0", "q4k", "q6k", "q2k", "q3k", "q5k", "q8k",
                                  "q4_0", "q4_1", "q5_0", "q5_1", "q8_1", "fp8"};
    return known(fmt) ? names[fmt] : nullptr;
}

const char *q_strerror(int status)
{
    switch (status) {
    case Q_OK: return "ok";
    case Q_EINVAL: return "invalid argument (null pointer, unknown format or path, bad workspace)";
    case Q_ESHAPE: return "shape out of range (M, N, K limits; K a multiple of 256, or of 32 for Q8_0)";
    case Q_EALIGN: return "pointer not 16-byte aligned";
    case Q_ENOTSUP: return "format or path not implemented for these arguments";
    case Q_EHIP: return "HIP runtime error at launch";
    case Q_ESCRATCH: return "activation blocks larger than the library's fixed scratch buffer (QLINEAR_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}

}  // extern "C"
