// C ABI of the CSA / HCA library: argument validation, then dispatch to the launchers.
// Every check below runs before anything is enqueued; a failed check launches nothing.
#include <atomic>
#include <cmath>
#include <string>

#include "common.hpp"
#include "internal.hpp"

namespace csa {

static thread_local std::string g_err;

void set_error(const std::string &msg) { g_err = msg; }
void clear_error() { g_err.clear(); }
int fail(int status, const std::string &msg) {
    g_err = msg;
    return status;
}
int check_launch(const char *what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(CSA_EHIP, std::string(what) + ": " + hipGetErrorString(e));
    return CSA_OK;
}

// compute units of the current device, queried once per device (the library's only
// global state)
int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
    if (dev < 64) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return -1;
    if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace csa

using namespace csa;

#define REQUIRE(cond, code, msg) \
    do {                         \
        if (!(cond)) return fail((code), (msg)); \
    } while (0)

extern "C" {

const char *csa_status_str(int status) {
    switch (status) {
        case CSA_OK: return "CSA_OK";
        case CSA_EINVAL: return "CSA_EINVAL";
        case CSA_EUNSUPPORTED: return "CSA_EUNSUPPORTED";
        case CSA_EWORKSPACE: return "CSA_EWORKSPACE";
        case CSA_EHIP: return "CSA_EHIP";
        default: return "CSA_UNKNOWN";
    }
}

const char *csa_last_error(void) { return g_err.c_str(); }

int csa_compress(const void *C_a, const void *C_b, const void *Z_a, const void *Z_b,
                 const void *carry_C_b, const void *carry_Z_b, const float *logit_bias, int B, int64_t n,
                 int c, int ratio, int overlap, csa_dtype dt, void *out, int64_t out_bstride, void *stream) {
    clear_error();
    REQUIRE(B >= 0 && n >= 0 && c > 0, CSA_EINVAL, "csa_compress: need B >= 0, n >= 0, c > 0");
    REQUIRE(ratio > 0 && (overlap == 0 || overlap == 1), CSA_EINVAL, "csa_compress: ratio > 0, overlap in {0,1}");
    REQUIRE(dt == CSA_F32 || dt == CSA_BF16, CSA_EINVAL, "csa_compress: dt must be CSA_F32 or CSA_BF16");
    REQUIRE((ratio == 4 && overlap == 1) || (ratio == 128 && overlap == 0), CSA_EUNSUPPORTED,
            "csa_compress: supported (ratio, overlap) pairs are (4, 1) and (128, 0)");
    const int64_t E = n / ratio;
    REQUIRE((carry_C_b == nullptr) == (carry_Z_b == nullptr), CSA_EINVAL,
            "csa_compress: carry_C_b and carry_Z_b must both be given or both be NULL");
    REQUIRE(overlap || carry_C_b == nullptr, CSA_EINVAL, "csa_compress: a carry needs overlap == 1");
    REQUIRE(out_bstride == 0 || out_bstride >= E * c, CSA_EINVAL, "csa_compress: out_bstride < (n/ratio)*c");
    if (B == 0 || E == 0) return CSA_OK;
    REQUIRE(C_a && Z_a && out, CSA_EINVAL, "csa_compress: C_a, Z_a and out are required");
    REQUIRE(!overlap || (C_b && Z_b), CSA_EINVAL, "csa_compress: C_b and Z_b are required when overlap == 1");
    return launch_compress(C_a, overlap ? C_b : nullptr, Z_a, overlap ? Z_b : nullptr, carry_C_b, carry_Z_b,
                           logit_bias, B, n, c, ratio, overlap, dt, out, out_bstride, (hipStream_t)stream);
}

int csa_compress_batch(const csa_compress_job *jobs, int njobs, csa_dtype dt, void *stream) {
    clear_error();
    REQUIRE(njobs >= 0 && (njobs == 0 || jobs != nullptr), CSA_EINVAL, "csa_compress_batch: need jobs for njobs > 0");
    REQUIRE(njobs <= 8, CSA_EUNSUPPORTED, "csa_compress_batch: at most 8 jobs per call");
    REQUIRE(dt == CSA_F32 || dt == CSA_BF16, CSA_EINVAL, "csa_compress_batch: dt must be CSA_F32 or CSA_BF16");
    CompressJobArgs args[8];
    for (int i = 0; i < njobs; ++i) {
        const csa_compress_job &j = jobs[i];
        REQUIRE(j.B >= 0 && j.n >= 0 && j.c > 0, CSA_EINVAL, "csa_compress_batch: a job needs B >= 0, n >= 0, c > 0");
        REQUIRE(j.ratio > 0 && (j.overlap == 0 || j.overlap == 1), CSA_EINVAL,
                "csa_compress_batch: a job needs ratio > 0, overlap in {0,1}");
        REQUIRE((j.ratio == 4 && j.overlap == 1) || (j.ratio == 128 && j.overlap == 0), CSA_EUNSUPPORTED,
                "csa_compress_batch: supported (ratio, overlap) pairs are (4, 1) and (128, 0)");
        const int64_t E = j.n / j.ratio;
        REQUIRE((j.carry_C_b == nullptr) == (j.carry_Z_b == nullptr), CSA_EINVAL,
                "csa_compress_batch: carry_C_b and carry_Z_b must both be given or both be NULL");
        REQUIRE(j.overlap || j.carry_C_b == nullptr, CSA_EINVAL, "csa_compress_batch: a carry needs overlap == 1");
        REQUIRE(j.out_bstride == 0 || j.out_bstride >= E * j.c, CSA_EINVAL, "csa_compress_batch: out_bstride < (n/ratio)*c");
        if (j.B > 0 && E > 0) {
            REQUIRE(j.C_a && j.Z_a && j.out, CSA_EINVAL, "csa_compress_batch: C_a, Z_a and out are required");
            REQUIRE(!j.overlap || (j.C_b && j.Z_b), CSA_EINVAL,
                    "csa_compress_batch: C_b and Z_b are required when overlap == 1");
        }
        args[i] = CompressJobArgs{j.C_a, j.overlap ? j.C_b : nullptr, j.Z_a, j.overlap ? j.Z_b : nullptr,
                                  j.carry_C_b, j.carry_Z_b, j.logit_bias, j.B, j.n, j.c, j.ratio, j.overlap,
                                  j.out, j.out_bstride};
    }
    return launch_compress_batch(args, njobs, dt, (hipStream_t)stream);
}

int csa_compress_hidden(const void *hidden, const void *carry_hidden, const void *W, const float *logit_bias, int B,
                        int64_t n, int64_t d, int c, int ratio, int overlap, csa_dtype out_dt, void *out,
                        int64_t out_bstride, void *stream) {
    clear_error();
    REQUIRE(B >= 0 && n >= 0 && d > 0 && c > 0, CSA_EINVAL, "csa_compress_hidden: need B >= 0, n >= 0, d > 0, c > 0");
    REQUIRE(ratio > 0 && (overlap == 0 || overlap == 1), CSA_EINVAL,
            "csa_compress_hidden: ratio > 0, overlap in {0,1}");
    REQUIRE(out_dt == CSA_F32 || out_dt == CSA_BF16, CSA_EINVAL, "csa_compress_hidden: out_dt must be CSA_F32 or CSA_BF16");
    REQUIRE((ratio == 4 && overlap == 1) || (ratio == 128 && overlap == 0), CSA_EUNSUPPORTED,
            "csa_compress_hidden: supported (ratio, overlap) pairs are (4, 1) and (128, 0)");
    REQUIRE(d % 32 == 0, CSA_EUNSUPPORTED, "csa_compress_hidden: d must be a multiple of 32");
    REQUIRE(n * d * 2 < ((int64_t)1 << 32) - 64 && (int64_t)(2 + 2 * overlap) * c * d * 2 < ((int64_t)1 << 32) - 64,
            CSA_EUNSUPPORTED, "csa_compress_hidden: one sequence's hidden rows and the weights must each stay under 4 GiB");
    REQUIRE(overlap || carry_hidden == nullptr, CSA_EINVAL, "csa_compress_hidden: a carry needs overlap == 1");
    const int64_t E = n / ratio;
    REQUIRE(out_bstride == 0 || out_bstride >= E * c, CSA_EINVAL, "csa_compress_hidden: out_bstride < (n/ratio)*c");
    if (B == 0 || E == 0) return CSA_OK;
    REQUIRE(hidden && W && out, CSA_EINVAL, "csa_compress_hidden: hidden, W and out are required");
    return launch_compress_hidden((const bf16_t *)hidden, (const bf16_t *)carry_hidden, (const bf16_t *)W, logit_bias,
                                  B, n, d, c, ratio, out, out_dt == CSA_F32, out_bstride, (hipStream_t)stream);
}

size_t csa_out_proj_workspace_bytes(int T, int G, int d_g) {
    if (T <= 0 || G <= 0 || d_g <= 0) return 0;
    return (size_t)T * (size_t)G * (size_t)d_g * sizeof(uint16_t);
}

int csa_out_proj(const void *o, int T, int H, int D, int G, const void *W_a, int d_g, const void *W_b, int d_model,
                 csa_dtype out_dt, void *out, void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    REQUIRE(T >= 0 && H > 0 && D > 0 && G > 0 && d_g > 0, CSA_EINVAL, "csa_out_proj: need T >= 0 and H, D, G, d_g > 0");
    REQUIRE(H % G == 0, CSA_EINVAL, "csa_out_proj: H must be a multiple of G");
    REQUIRE(W_b == nullptr || d_model > 0, CSA_EINVAL, "csa_out_proj: d_model must be positive with W_b");
    REQUIRE(out_dt == CSA_F32 || out_dt == CSA_BF16, CSA_EINVAL, "csa_out_proj: out_dt must be CSA_F32 or CSA_BF16");
    const int64_t K1 = (int64_t)(H / G) * D, K2 = (int64_t)G * d_g;
    REQUIRE(K1 % 32 == 0 && (W_b == nullptr || K2 % 32 == 0), CSA_EUNSUPPORTED,
            "csa_out_proj: (H/G)*D and G*d_g must be multiples of 32");
    REQUIRE(128 * (int64_t)H * D * 2 < ((int64_t)1 << 32) && (int64_t)d_g * K1 * 2 < ((int64_t)1 << 32) &&
                (W_b == nullptr || (int64_t)d_model * K2 * 2 < ((int64_t)1 << 32)),
            CSA_EUNSUPPORTED, "csa_out_proj: operand tiles must stay under 4 GiB");
    if (T == 0) return CSA_OK;
    REQUIRE(o && W_a && out, CSA_EINVAL, "csa_out_proj: o, W_a and out are required");
    hipStream_t st = (hipStream_t)stream;
    if (W_b == nullptr)  // the grouped stage alone: out [T][G * d_g]
        return launch_gemm_bf16((const bf16_t *)o, (int64_t)H * D, K1, (const bf16_t *)W_a, K1, (int64_t)d_g * K1, out,
                                K2, d_g, out_dt == CSA_F32, T, d_g, K1, G, st);
    const size_t need = csa_out_proj_workspace_bytes(T, G, d_g);
    REQUIRE(workspace && workspace_bytes >= need, CSA_EWORKSPACE,
            "csa_out_proj: workspace smaller than csa_out_proj_workspace_bytes()");
    int rc = launch_gemm_bf16((const bf16_t *)o, (int64_t)H * D, K1, (const bf16_t *)W_a, K1, (int64_t)d_g * K1,
                              workspace, K2, d_g, false, T, d_g, K1, G, st);
    if (rc != CSA_OK) return rc;
    return launch_gemm_bf16((const bf16_t *)workspace, K2, 0, (const bf16_t *)W_b, K2, 0, out, d_model, 0,
                            out_dt == CSA_F32, T, d_model, K2, 1, st);
}

int csa_index_scores(const void *q_I, const uint8_t *q_I_scale, const float *w, const void *k_I,
                     const uint8_t *k_I_scale, const int32_t *q_seq, const int64_t *q_pos, int T, int B,
                     int64_t N, int H_I, int D_I, int k_heads, int ratio, csa_dtype dt, float *scores,
                     void *stream) {
    clear_error();
    REQUIRE(T >= 0 && B > 0 && N >= 0 && ratio > 0, CSA_EINVAL, "csa_index_scores: need T >= 0, B > 0, N >= 0, ratio > 0");
    REQUIRE(H_I > 0 && D_I > 0, CSA_EINVAL, "csa_index_scores: H_I and D_I must be positive");
    REQUIRE(dt == CSA_F32 || dt == CSA_BF16 || dt == CSA_MXFP4, CSA_EINVAL, "csa_index_scores: bad dtype");
    REQUIRE(dt != CSA_MXFP4 || D_I % 32 == 0, CSA_EINVAL, "csa_index_scores: MXFP4 needs D_I % 32 == 0");
    REQUIRE(k_heads == H_I || k_heads == 1, CSA_EINVAL, "csa_index_scores: k_heads must be H_I or 1");
    REQUIRE(H_I == 64 && D_I == 128, CSA_EUNSUPPORTED, "csa_index_scores: only H_I = 64, D_I = 128 is built");
    REQUIRE(k_heads == H_I || dt == CSA_BF16, CSA_EUNSUPPORTED,
            "csa_index_scores: shared keys (k_heads = 1) are built for CSA_BF16 only");
    if (T == 0 || N == 0) return CSA_OK;
    REQUIRE(q_I && w && k_I && q_seq && q_pos && scores, CSA_EINVAL, "csa_index_scores: NULL tensor");
    REQUIRE(dt != CSA_MXFP4 || (q_I_scale && k_I_scale), CSA_EINVAL, "csa_index_scores: MXFP4 needs both scale tensors");
    return launch_index_scores(q_I, q_I_scale, w, k_I, k_I_scale, q_seq, q_pos, T, B, N, k_heads, ratio, dt,
                               scores, (hipStream_t)stream);
}

size_t csa_index_topk_workspace_bytes(int T, int64_t N, int k) {
    if (T <= 0 || N < 0) return 0;
    return index_topk_workspace_bytes(T, N, k);
}

int csa_index_topk(const uint8_t *q_I, const uint8_t *q_I_scale, const float *w, const uint8_t *k_I,
                   const uint8_t *k_I_scale, const int32_t *q_seq, const int64_t *q_pos, int T, int B, int64_t N,
                   int H_I, int D_I, int ratio, int k, int32_t *topk_idxs, float *topk_vals, void *workspace,
                   size_t workspace_bytes, void *stream) {
    clear_error();
    REQUIRE(T >= 0 && B > 0 && N >= 0 && ratio > 0, CSA_EINVAL, "csa_index_topk: need T >= 0, B > 0, N >= 0, ratio > 0");
    REQUIRE(k >= 1, CSA_EINVAL, "csa_index_topk: need k >= 1");
    REQUIRE(H_I == 64 && D_I == 128, CSA_EUNSUPPORTED, "csa_index_topk: only H_I = 64, D_I = 128 is built");
    REQUIRE(k <= 4096, CSA_EUNSUPPORTED, "csa_index_topk: k must be <= 4096");
    REQUIRE(T <= 65535, CSA_EUNSUPPORTED, "csa_index_topk: at most 65,535 queries per call");
    REQUIRE(N < (int64_t{1} << 31), CSA_EUNSUPPORTED, "csa_index_topk: N must be below 2^31 (32-bit entry indices)");
    if (T == 0) return CSA_OK;
    REQUIRE(q_I && q_I_scale && w && q_seq && q_pos && topk_idxs && (N == 0 || (k_I && k_I_scale)), CSA_EINVAL,
            "csa_index_topk: NULL tensor");
    return launch_index_topk_mxfp4(q_I, q_I_scale, w, k_I, k_I_scale, q_seq, q_pos, T, B, N, ratio, k, topk_idxs,
                                   topk_vals, workspace, workspace_bytes, (hipStream_t)stream);
}

int csa_index_rescore(const void *q_I, const float *w, const void *k_I, const int32_t *cand, int M,
                      const int32_t *q_seq, const int64_t *q_pos, int T, int B, int64_t N, int H_I, int D_I,
                      int ratio, csa_dtype dt, float *scores, void *stream) {
    clear_error();
    REQUIRE(T >= 0 && M >= 0 && B > 0 && N >= 0 && ratio > 0, CSA_EINVAL,
            "csa_index_rescore: need T >= 0, M >= 0, B > 0, N >= 0, ratio > 0");
    REQUIRE(dt == CSA_F32 || dt == CSA_BF16, CSA_EINVAL, "csa_index_rescore: dt must be CSA_F32 or CSA_BF16");
    REQUIRE(H_I == 64 && D_I == 128, CSA_EUNSUPPORTED, "csa_index_rescore: only H_I = 64, D_I = 128 is built");
    if (T == 0 || M == 0) return CSA_OK;
    REQUIRE(q_I && w && k_I && cand && q_seq && q_pos && scores, CSA_EINVAL, "csa_index_rescore: NULL tensor");
    return launch_index_rescore(q_I, w, k_I, cand, M, q_seq, q_pos, T, B, N, ratio, dt, scores, (hipStream_t)stream);
}

int csa_quantize_mxfp4(const void *x, int64_t rows, int D, csa_dtype dt, int hadamard, uint8_t *codes,
                       uint8_t *scales, int64_t out_group_rows, int64_t out_group_stride, void *stream) {
    clear_error();
    REQUIRE(rows >= 0 && D > 0, CSA_EINVAL, "csa_quantize_mxfp4: need rows >= 0 and D > 0");
    REQUIRE(D % 32 == 0, CSA_EINVAL, "csa_quantize_mxfp4: D must be a multiple of 32");
    REQUIRE(dt == CSA_F32 || dt == CSA_BF16, CSA_EINVAL, "csa_quantize_mxfp4: dt must be CSA_F32 or CSA_BF16");
    REQUIRE(D == 128 || D == 256 || D == 512, CSA_EUNSUPPORTED, "csa_quantize_mxfp4: D must be 128, 256 or 512");
    REQUIRE(out_group_rows >= 0 && (out_group_rows == 0 || out_group_stride >= out_group_rows), CSA_EINVAL,
            "csa_quantize_mxfp4: need out_group_rows >= 0 and out_group_stride >= out_group_rows");
    if (rows == 0) return CSA_OK;
    REQUIRE(x && codes && scales, CSA_EINVAL, "csa_quantize_mxfp4: NULL tensor");
    return launch_quantize_mxfp4(x, rows, D, dt, hadamard != 0, codes, scales, out_group_rows, out_group_stride,
                                 (hipStream_t)stream);
}

int csa_quantize_kv8(const void *x, int64_t rows, csa_dtype dt, uint8_t *out, int64_t out_group_rows,
                     int64_t out_group_stride, void *stream) {
    clear_error();
    REQUIRE(rows >= 0, CSA_EINVAL, "csa_quantize_kv8: need rows >= 0");
    REQUIRE(dt == CSA_F32 || dt == CSA_BF16, CSA_EINVAL, "csa_quantize_kv8: dt must be CSA_F32 or CSA_BF16");
    REQUIRE(out_group_rows >= 0 && (out_group_rows == 0 || out_group_stride >= out_group_rows), CSA_EINVAL,
            "csa_quantize_kv8: need out_group_rows >= 0 and out_group_stride >= out_group_rows");
    if (rows == 0) return CSA_OK;
    REQUIRE(x && out, CSA_EINVAL, "csa_quantize_kv8: NULL tensor");
    REQUIRE((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(out)) % 16 == 0, CSA_EINVAL,
            "csa_quantize_kv8: x and out must be 16-byte aligned");
    return launch_quantize_kv8(x, rows, dt, out, out_group_rows, out_group_stride, (hipStream_t)stream);
}

int csa_rmsnorm_rope(const void *x, csa_dtype dt_in, int64_t rows, int D, const float *g, float eps,
                     const float *rope_cs, int R, int64_t rope_group, void *out, csa_dtype dt_out, void *stream) {
    clear_error();
    REQUIRE(rows >= 0 && D > 0, CSA_EINVAL, "csa_rmsnorm_rope: need rows >= 0 and D > 0");
    REQUIRE((dt_in == CSA_F32 || dt_in == CSA_BF16) && (dt_out == CSA_F32 || dt_out == CSA_BF16), CSA_EINVAL,
            "csa_rmsnorm_rope: dt_in and dt_out must be CSA_F32 or CSA_BF16");
    REQUIRE(std::isfinite(eps) && eps >= 0.f, CSA_EINVAL, "csa_rmsnorm_rope: eps must be finite and >= 0");
    REQUIRE(R >= 0 && R % 2 == 0 && R <= D, CSA_EINVAL, "csa_rmsnorm_rope: R must be even and in [0, D]");
    REQUIRE(rope_group >= 1, CSA_EINVAL, "csa_rmsnorm_rope: rope_group must be >= 1");
    REQUIRE(D == 128 || D == 256 || D == 512, CSA_EUNSUPPORTED, "csa_rmsnorm_rope: D must be 128, 256 or 512");
    REQUIRE(R % (D / 64) == 0, CSA_EUNSUPPORTED, "csa_rmsnorm_rope: R must be a multiple of D / 64");
    if (rows == 0) return CSA_OK;
    REQUIRE(x && g && out && (R == 0 || rope_cs), CSA_EINVAL, "csa_rmsnorm_rope: NULL tensor");
    REQUIRE(x != out || dt_in == dt_out, CSA_EINVAL, "csa_rmsnorm_rope: in place needs dt_out == dt_in");
    REQUIRE((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(g) |
             reinterpret_cast<uintptr_t>(R > 0 ? rope_cs : g)) % 16 == 0,
            CSA_EINVAL, "csa_rmsnorm_rope: x, out, g and rope_cs must be 16-byte aligned");
    return launch_rmsnorm_rope(x, dt_in, rows, D, g, eps, rope_cs, R, rope_group, out, dt_out, (hipStream_t)stream);
}

size_t csa_topk_workspace_bytes(int T, int64_t N, int k) {
    if (T <= 0 || N <= 0 || k <= 0) return 0;
    return topk_workspace_bytes(T, N, k);
}

int csa_topk(const float *scores, int T, int64_t N, int k, int32_t *topk_idxs, float *topk_vals, void *workspace,
             size_t workspace_bytes, void *stream) {
    clear_error();
    REQUIRE(T >= 0 && N >= 0, CSA_EINVAL, "csa_topk: need T >= 0 and N >= 0");
    REQUIRE(k > 0, CSA_EINVAL, "csa_topk: k must be positive");
    REQUIRE(k <= 4096, CSA_EUNSUPPORTED, "csa_topk: k > 4096 is not built");
    REQUIRE(N < ((int64_t)1 << 31), CSA_EUNSUPPORTED, "csa_topk: N must fit int32 indices");
    if (T == 0) return CSA_OK;
    REQUIRE(topk_idxs && (scores || N == 0), CSA_EINVAL, "csa_topk: NULL tensor");
    return launch_topk(scores, nullptr, T, N, k, topk_idxs, topk_vals, workspace, workspace_bytes, (hipStream_t)stream);
}

int csa_topk_noalloc(const float *scores, int T, int64_t N, int k, int32_t *topk_idxs, float *topk_vals,
                     void *stream) {
    clear_error();
    REQUIRE(T >= 0 && N >= 0, CSA_EINVAL, "csa_topk_noalloc: need T >= 0 and N >= 0");
    REQUIRE(k > 0, CSA_EINVAL, "csa_topk_noalloc: k must be positive");
    REQUIRE(k <= 4096, CSA_EUNSUPPORTED, "csa_topk_noalloc: k > 4096 is not built");
    REQUIRE(N < ((int64_t)1 << 31), CSA_EUNSUPPORTED, "csa_topk_noalloc: N must fit int32 indices");
    if (T == 0) return CSA_OK;
    REQUIRE(topk_idxs && (scores || N == 0), CSA_EINVAL, "csa_topk_noalloc: NULL tensor");
    const size_t need = topk_workspace_bytes(T, N, k);
    REQUIRE(need <= topk_scratch_bytes(), CSA_EWORKSPACE,
            "csa_topk_noalloc: T, N, k need " + std::to_string(need) + " bytes of scratch, more than the " +
                std::to_string(topk_scratch_bytes()) + " the library holds; use csa_topk with a workspace");
    void *ws = nullptr;
    if (need > 0) {
        const int rc = topk_scratch_ptr(&ws);
        if (rc != CSA_OK) return rc;
    }
    return launch_topk(scores, nullptr, T, N, k, topk_idxs, topk_vals, ws, need, (hipStream_t)stream);
}

int csa_topk_ids(const float *scores, const int32_t *ids, int T, int64_t M, int k, int32_t *topk_idxs,
                 float *topk_vals, void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    REQUIRE(T >= 0 && M >= 0, CSA_EINVAL, "csa_topk_ids: need T >= 0 and M >= 0");
    REQUIRE(k > 0, CSA_EINVAL, "csa_topk_ids: k must be positive");
    REQUIRE(k <= 4096, CSA_EUNSUPPORTED, "csa_topk_ids: k > 4096 is not built");
    REQUIRE(M < ((int64_t)1 << 31), CSA_EUNSUPPORTED, "csa_topk_ids: M must fit int32 positions");
    if (T == 0) return CSA_OK;
    REQUIRE(topk_idxs && (M == 0 || (scores && ids)), CSA_EINVAL, "csa_topk_ids: NULL tensor");
    return launch_topk(scores, ids, T, M, k, topk_idxs, topk_vals, workspace, workspace_bytes, (hipStream_t)stream);
}

size_t csa_attn_workspace_bytes(int T, int H, int D, int64_t max_rows) {
    if (T <= 0 || H <= 0 || D <= 0 || max_rows <= 0) return 0;
    return attn_workspace_bytes(T, H, D, max_rows);
}

static int check_attn_common(const void *q, const void *kv, const float *sink, const void *swa,
                             const int64_t *swa_pos0, int swa_rows, int window, const int32_t *q_seq,
                             const int64_t *q_pos, const float *rope_cs, int rope_dim, int T, int B, int64_t N,
                             int H, int D, csa_dtype dt, void *out, const char *who) {
    const std::string w(who);
    REQUIRE(T >= 0 && B > 0 && N >= 0 && H > 0 && D > 0, CSA_EINVAL, w + ": need T >= 0, B > 0, N >= 0, H > 0, D > 0");
    REQUIRE(window >= 0 && swa_rows >= 0, CSA_EINVAL, w + ": window and swa_rows must be >= 0");
    REQUIRE(dt == CSA_F32 || dt == CSA_BF16 || dt == CSA_KV8, CSA_EINVAL,
            w + ": dt must be CSA_F32, CSA_BF16 or CSA_KV8");
    REQUIRE(dt != CSA_KV8 || (D == 512 && H % 64 == 0), CSA_EUNSUPPORTED,
            w + ": FP8 KV rows (CSA_KV8) need D = 512 and H a multiple of 64");
    REQUIRE(!rope_cs || (rope_dim > 0 && rope_dim % 2 == 0 && rope_dim <= D), CSA_EINVAL,
            w + ": rope_dim must be even, positive and <= D");
    REQUIRE(D % 64 == 0 && D <= 1024, CSA_EUNSUPPORTED, w + ": D must be a multiple of 64 and <= 1024");
    if (T == 0) return CSA_OK;
    REQUIRE(q && sink && q_seq && q_pos && out, CSA_EINVAL, w + ": NULL tensor");
    REQUIRE(kv || N == 0, CSA_EINVAL, w + ": NULL key/value rows");
    REQUIRE(!swa || swa_pos0, CSA_EINVAL, w + ": swa_kv needs swa_pos0");
    return CSA_OK;
}

int csa_sparse_attn(const void *q, const void *kv, const float *attn_sink, const int32_t *topk_idxs, int k,
                    float softmax_scale, const void *swa_kv, const int64_t *swa_pos0, int swa_rows, int window,
                    const int32_t *q_seq, const int64_t *q_pos, const float *rope_cs, int rope_dim, int T, int B,
                    int64_t N, int H, int D, csa_dtype dt, void *out, float *lse, void *workspace,
                    size_t workspace_bytes, void *stream) {
    clear_error();
    int rc = check_attn_common(q, kv, attn_sink, swa_kv, swa_pos0, swa_rows, window, q_seq, q_pos, rope_cs,
                               rope_dim, T, B, N, H, D, dt, out, "csa_sparse_attn");
    if (rc != CSA_OK) return rc;
    REQUIRE(k >= 0, CSA_EINVAL, "csa_sparse_attn: k must be >= 0");
    REQUIRE(k <= 4096, CSA_EUNSUPPORTED, "csa_sparse_attn: k > 4096 is not built");
    REQUIRE(std::isfinite(softmax_scale), CSA_EINVAL, "csa_sparse_attn: softmax_scale must be finite");
    // the matrix-core kernels take the largest raw score as the largest logit
    REQUIRE(softmax_scale > 0.f, CSA_EUNSUPPORTED, "csa_sparse_attn: softmax_scale must be positive");
    if (T == 0) return CSA_OK;
    REQUIRE(k == 0 || topk_idxs, CSA_EINVAL, "csa_sparse_attn: NULL topk_idxs");
    AttnArgs a{q, kv, attn_sink, topk_idxs, k, 0, softmax_scale, swa_kv, swa_pos0, swa_rows, window, q_seq, q_pos,
               rope_cs, rope_cs ? rope_dim : 0, T, B, N, H, D, dt, out, lse, workspace, workspace_bytes};
    return launch_attn(a, (hipStream_t)stream);
}

int hca_attn(const void *q, const void *summ, const float *attn_sink, int ratio, float softmax_scale,
             const void *swa_kv, const int64_t *swa_pos0, int swa_rows, int window, const int32_t *q_seq,
             const int64_t *q_pos, const float *rope_cs, int rope_dim, int T, int B, int64_t N, int H, int D,
             csa_dtype dt, void *out, float *lse, void *workspace, size_t workspace_bytes, void *stream) {
    clear_error();
    int rc = check_attn_common(q, summ, attn_sink, swa_kv, swa_pos0, swa_rows, window, q_seq, q_pos, rope_cs,
                               rope_dim, T, B, N, H, D, dt, out, "hca_attn");
    if (rc != CSA_OK) return rc;
    REQUIRE(ratio > 0, CSA_EINVAL, "hca_attn: ratio must be positive");
    REQUIRE(std::isfinite(softmax_scale), CSA_EINVAL, "hca_attn: softmax_scale must be finite");
    REQUIRE(softmax_scale > 0.f, CSA_EUNSUPPORTED, "hca_attn: softmax_scale must be positive");
    if (T == 0) return CSA_OK;
    AttnArgs a{q, summ, attn_sink, nullptr, 0, ratio, softmax_scale, swa_kv, swa_pos0, swa_rows, window, q_seq,
               q_pos, rope_cs, rope_cs ? rope_dim : 0, T, B, N, H, D, dt, out, lse, workspace, workspace_bytes};
    return launch_attn(a, (hipStream_t)stream);
}

}  // extern "C"
