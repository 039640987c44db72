// Launchers behind the C ABI (arguments already validated by api.cpp).
#pragma once

#include "common.hpp"

namespace csa {

// one pooling of a batch (the arguments of csa_compress)
struct CompressJobArgs {
    const void *Ca, *Cb, *Za, *Zb, *cCb, *cZb;
    const float *bias;
    int B;
    int64_t n;
    int c, ratio, overlap;
    void *out;
    int64_t out_bstride;
};
int launch_compress_batch(const CompressJobArgs *jobs, int njobs, csa_dtype dt, hipStream_t st);
int launch_compress(const void *Ca, const void *Cb, const void *Za, const void *Zb,
                    const void *cCb, const void *cZb, const float *bias, int B, int64_t n, int c,
                    int ratio, int overlap, csa_dtype dt, void *out, int64_t out_bstride,
                    hipStream_t st);

int launch_index_scores(const void *qI, const uint8_t *qs, const float *w, const void *kI,
                        const uint8_t *ks, const int32_t *q_seq, const int64_t *q_pos, int T,
                        int B, int64_t N, int k_heads, int ratio, csa_dtype dt, float *scores,
                        hipStream_t st);

int launch_index_mxfp4(const uint8_t *qI, const uint8_t *qs, const float *w, const uint8_t *kI,
                       const uint8_t *ks, const int32_t *q_seq, const int64_t *q_pos, int T, int B, int64_t N,
                       int ratio, float *scores, hipStream_t st);
size_t index_topk_workspace_bytes(int T, int64_t N, int k);
int launch_index_topk_mxfp4(const uint8_t *qI, const uint8_t *qs, const float *w, const uint8_t *kI,
                            const uint8_t *ks, const int32_t *q_seq, const int64_t *q_pos, int T, int B, int64_t N,
                            int ratio, int k, int32_t *idx, float *vals, void *ws, size_t ws_bytes, hipStream_t st);

int launch_quantize_mxfp4(const void *x, int64_t rows, int D, csa_dtype dt, bool hadamard, uint8_t *codes,
                          uint8_t *scales, int64_t group_rows, int64_t group_stride, hipStream_t st);

int launch_quantize_kv8(const void *x, int64_t rows, csa_dtype dt, uint8_t *out, int64_t group_rows,
                        int64_t group_stride, hipStream_t st);

int launch_rmsnorm_rope(const void *x, csa_dtype dt_in, int64_t rows, int D, const float *g, float eps,
                        const float *rope_cs, int R, int64_t group, void *out, csa_dtype dt_out, hipStream_t st);

size_t topk_workspace_bytes(int T, int64_t N, int k);
int launch_index_rescore(const void *qI, const float *w, const void *kI, const int32_t *cand, int M,
                         const int32_t *q_seq, const int64_t *q_pos, int T, int B, int64_t N, int ratio,
                         csa_dtype dt, float *scores, hipStream_t st);

// ids: NULL (position p of a row is entry p) or [T][N] entry ids of the row's positions
int launch_topk(const float *scores, const int32_t *ids, int T, int64_t N, int k, int32_t *idx, float *vals,
                void *ws, size_t ws_bytes, hipStream_t st);
// the allocation-free top-k's file-scope device scratch: its size, and its device address
// on the current device (looked up once per device)
size_t topk_scratch_bytes();
int topk_scratch_ptr(void **ptr);

// Rows of one query: the first `k` slots come from topk_idxs (sparse mode) or from
// the visible summaries 0..nvis-1 (dense mode, k < 0 selects it with ratio = -k),
// then the SWA window rows.
struct AttnArgs {
    const void *q;
    const void *kv;
    const float *sink;
    const int32_t *idx;
    int k;          // sparse: slots per query from idx
    int ratio;      // dense: visibility ratio (0 = sparse mode)
    float scale;
    const void *swa;
    const int64_t *swa_pos0;
    int swa_rows;
    int window;
    const int32_t *q_seq;
    const int64_t *q_pos;
    const float *rope_cs;
    int rope_dim;
    int T, B;
    int64_t N;
    int H, D;
    csa_dtype dt;
    void *out;
    float *lse;
    void *ws;
    size_t ws_bytes;
};

// bf16 matrix-core GEMMs (gemm.hip): C[z][m][n] = sum_k A[z][m][k] B[z][n][k], K % 32 == 0
int launch_gemm_bf16(const bf16_t *A, int64_t lda, int64_t sA, const bf16_t *B, int64_t ldb, int64_t sB, void *C,
                     int64_t ldc, int64_t sC, bool c_f32, int64_t M, int64_t N, int64_t K, int batch,
                     hipStream_t st);
// projection of hidden rows + compressor pooling in one kernel (ratio 4 overlapped, 128)
int launch_compress_hidden(const bf16_t *Hs, const bf16_t *carry, const bf16_t *W, const float *bias, int B,
                           int64_t n, int64_t d, int c, int ratio, void *out, bool out_f32, int64_t out_bstride,
                           hipStream_t st);

size_t attn_workspace_bytes(int T, int H, int D, int64_t max_rows);
int launch_attn(const AttnArgs &a, hipStream_t st);
bool wide_attn_ok(csa_dtype dt, int H, int D);
int launch_attn_wide(const AttnArgs &a, float sl2, int nsplit, int64_t split_slots, hipStream_t st);
int device_cu_count();
bool w32_attn_ok(csa_dtype dt, int H, int D, int64_t N, int swa_rows, int ratio, int k);
int launch_attn_w32(const AttnArgs &a, float sl2, int nsplit, int64_t split_slots, hipStream_t st);

}  // namespace csa
