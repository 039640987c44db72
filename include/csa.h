/*
 * csa.h - C ABI of the MI355X (gfx950) DeepSeek-V4 CSA / HCA attention hot path.
 *
 * The operations follow "DeepSeek-V4 混合注意力：从压缩记忆到百万上下文" (brenchcc
 * technical note, built on the DeepSeek-V4 technical report and inference code):
 *   csa_compress      §4.1 (ratio 4, overlapped two-branch pooling) and §5 (ratio 128)
 *   csa_index_scores  §4.2 (Lightning Indexer score), FP4 operands per §2 and §4.2
 *   csa_topk          §2 table and §4.2 (top-k 512 / 1,024 compressed entries per query)
 *   csa_sparse_attn   §4.2 (shared-KV MQA over the selected entries), §6 (SWA 128,
 *                     partial RoPE and inverse RoPE, attention sink), §7 call chain;
 *                     argument order of the sparse_attn(q, kv, attn_sink, topk_idxs,
 *                     softmax_scale) call on the DeepSeek-V4-Flash page
 *   hca_attn          §5 (dense MQA over every visible 128:1 summary) plus §6
 *
 * Conventions for every call:
 *  - Every tensor pointer is a DEVICE pointer (hipMalloc'd or a torch tensor's
 *    data_ptr()). Tensors are row-major with the innermost dimension contiguous.
 *  - The caller owns every buffer, including outputs and workspaces. The library
 *    allocates no device memory and keeps no pointer after a call returns (the one
 *    exception is the fixed device array behind csa_topk_noalloc, below).
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null
 *    stream). Results are ready when that stream is synchronised.
 *  - Positions are 0-based absolute token positions. Compressed entry i of a
 *    ratio-m compressor pools the block of tokens [i*m, (i+1)*m); a query at
 *    position t sees entry i iff (i+1)*m <= t.
 *  - Return value: CSA_OK, or an error code. Scalar/pointer arguments are validated
 *    before anything is launched: on CSA_EINVAL / CSA_EUNSUPPORTED /
 *    CSA_EWORKSPACE no work is enqueued. CSA_EHIP reports a HIP launch error.
 *    csa_last_error() gives a detail string (thread-local). Nothing is printed and
 *    nothing throws across the ABI.
 *  - Device-resident index data (q_seq, q_pos, topk_idxs, swa_pos0) cannot be
 *    validated without a synchronisation: out-of-range row indices are skipped,
 *    never dereferenced; an out-of-range q_seq yields a query that sees no rows.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* CSA_KV8: compressed KV rows in the FP8 storage format of csa_quantize_kv8 (the other
 * tensors of the call are bf16); accepted by csa_sparse_attn and hca_attn for kv / summ. */
typedef enum { CSA_F32 = 0, CSA_BF16 = 1, CSA_MXFP4 = 2, CSA_KV8 = 3 } csa_dtype;

typedef enum {
    CSA_OK = 0,
    CSA_EINVAL = 1,       /* bad shape, NULL required pointer, bad combination */
    CSA_EUNSUPPORTED = 2, /* valid request that this library does not implement */
    CSA_EWORKSPACE = 3,   /* workspace missing or smaller than the *_workspace_bytes query */
    CSA_EHIP = 4          /* the HIP runtime reported an error */
} csa_status;

/*
 * csa_compress - token-level KV compressor (§4.1, §5).
 *
 * ratio 4, overlap 1 (CSA): for entry i and channel j, a softmax over the 8 logits
 *   [Z_b rows 4(i-1)..4i-1 ; Z_a rows 4i..4i+3] (+ logit_bias), and
 *   out[i][j] = sum of the weights times the matching C_b / C_a rows.
 *   For i = 0 the b-branch rows come from carry_C_b / carry_Z_b (the b-branch of the
 *   block just before row 0, e.g. from the previous chunk); when the carry is NULL
 *   those slots are absent (weight 0) and entry 0 pools block 0's a-branch alone.
 * ratio 128, overlap 0 (HCA): out[i][j] = sum_r softmax_r(Z_a[128i + r][j]) C_a[128i + r][j].
 *
 * C_a, Z_a:   [B][n][c]           dtype dt (F32 or BF16)
 * C_b, Z_b:   [B][n][c]           dtype dt; required iff overlap == 1, else ignored
 * carry_C_b, carry_Z_b: [B][ratio][c] dtype dt, or both NULL (overlap == 1 only)
 * logit_bias: [(1+overlap)*ratio][c] fp32 added to the slot logits (b-slots first), or NULL
 * out:        [B][n/ratio][c] dtype dt, sequence b starting at out + b*out_bstride
 *             elements (out_bstride == 0 means (n/ratio)*c). A trailing partial block
 *             (n % ratio rows) is not compressed.
 * Supported: (ratio, overlap) = (4, 1) or (128, 0); any other pair is CSA_EUNSUPPORTED.
 * Softmax and sums are fp32; the output is rounded once to dt.
 */
int csa_compress(const void *C_a, const void *C_b, const void *Z_a, const void *Z_b,
                 const void *carry_C_b, const void *carry_Z_b, const float *logit_bias,
                 int B, int64_t n, int c, int ratio, int overlap, csa_dtype dt,
                 void *out, int64_t out_bstride, void *stream);

/*
 * csa_compress_batch - several csa_compress poolings in one launch (a decode step's new KV
 * entry, index key and HCA summary: §4.1 and §5 applied to the block that completes with
 * the step). Each job has exactly the arguments and meaning of csa_compress; all jobs share
 * dt. Jobs whose rows allow 16-byte accesses (c a multiple of 8 for bf16 / 4 for fp32,
 * 16-byte aligned tensors and batch stride) run in one kernel; otherwise the jobs run one
 * launch each, in order. Jobs must not write what another job of the call reads.
 * Supported: 0 <= njobs <= 8; each job as csa_compress. Errors: as csa_compress, checked
 * for every job before anything is launched.
 */
typedef struct csa_compress_job {
    const void *C_a, *C_b, *Z_a, *Z_b;     /* [B][n][c] (C_b, Z_b for overlap == 1) */
    const void *carry_C_b, *carry_Z_b;     /* [B][ratio][c] or both NULL */
    const float *logit_bias;               /* [(1+overlap)*ratio][c] or NULL */
    int B;
    int64_t n;
    int c, ratio, overlap;
    void *out;                             /* [B][n/ratio][c], batch stride out_bstride */
    int64_t out_bstride;
} csa_compress_job;
int csa_compress_batch(const csa_compress_job *jobs, int njobs, csa_dtype dt, void *stream);

/*
 * csa_compress_hidden - the compressor fed from hidden states (§4.1: the compressor forms
 * C^a, C^b, Z^a, Z^b from H; §7: Compressor.forward opens with project_a / project_b of
 * the hidden rows): the projections and the pooling of csa_compress in one kernel.
 *
 *   C^a = H Wa_C^T, Z^a = H Wa_Z^T (and C^b = H Wb_C^T, Z^b = H Wb_Z^T for ratio 4),
 *   then out = csa_compress(C^a, C^b, Z^a, Z^b, ...) on those values, computed in fp32:
 *   the projected values are not rounded before the pooling, the output is rounded once.
 *
 * hidden:       [B][n][d] bf16 hidden rows of the chunk.
 * carry_hidden: [B][4][d] bf16, the last 4 hidden rows before the chunk (their b-branch
 *               feeds entry 0), or NULL (entry 0 then pools its own block's a-branch
 *               alone). ratio 4 only.
 * W:            bf16 [(1+overlap)*2][c][d]: the projections as [out][in] matrices, in the
 *               order Wa_C, Wa_Z, Wb_C, Wb_Z (ratio 4) or Wa_C, Wa_Z (ratio 128).
 * logit_bias:   as csa_compress, or NULL.
 * out:          [B][n/ratio][c] in out_dt (F32 | BF16), batch stride out_bstride elements
 *               (0: (n/ratio)*c); a trailing partial block is not compressed.
 * Supported: (ratio, overlap) = (4, 1) or (128, 0); d % 32 == 0; n*d*2 and the weights
 * each under 4 GiB. Errors as csa_compress.
 */
int csa_compress_hidden(const void *hidden, const void *carry_hidden, const void *W, const float *logit_bias,
                        int B, int64_t n, int64_t d, int c, int ratio, int overlap, csa_dtype out_dt,
                        void *out, int64_t out_bstride, void *stream);

/*
 * csa_out_proj - grouped output projection after the attention (§4.2: the outputs are
 * aggregated per group and projected back to the model width; §7:
 * grouped_output_projection(inverse_rope(output))). The H heads form G groups of H/G
 * consecutive heads; group g's concatenated outputs are projected by its own matrix:
 *   y[t][g] = W_a[g] . concat_h o[t][g*H/G + h]            ([d_g], fp32 sums, bf16 y)
 * and, when W_b is given, the G results side by side are projected to the model width:
 *   out[t] = W_b . y[t]                                    ([d_model])
 * The inverse RoPE of §6/§7 comes first: csa_sparse_attn / hca_attn with rope_cs apply
 * it to their output, so o is passed as those calls return it.
 *
 * o:     [T][H][D] bf16.           W_a: [G][d_g][(H/G)*D] bf16 ([out][in] per group).
 * W_b:   [d_model][G*d_g] bf16, or NULL (then out = y, [T][G*d_g]).
 * out:   [T][d_model] (or [T][G*d_g]) in out_dt (F32 | BF16).
 * workspace: csa_out_proj_workspace_bytes(T, G, d_g) bytes for y (unused without W_b).
 * Supported: (H/G)*D and G*d_g multiples of 32. T may be 0.
 */
size_t csa_out_proj_workspace_bytes(int T, int G, int d_g);
int csa_out_proj(const void *o, int T, int H, int D, int G, const void *W_a, int d_g, const void *W_b,
                 int d_model, csa_dtype out_dt, void *out, void *workspace, size_t workspace_bytes,
                 void *stream);

/*
 * csa_index_scores - Lightning Indexer (§4.2):
 *   scores[t][i] = sum_h w[t][h] * ReLU(<q_I[t][h], k_I[q_seq[t]][i][h]>)
 * for every stored entry i with (i+1)*ratio <= q_pos[t]; -INFINITY otherwise.
 *
 * q_I:  [T][H_I][D_I] in dt.  For CSA_MXFP4: [T][H_I][D_I/2] bytes of E2M1 codes (even
 *       element in the low nibble) plus q_I_scale [T][H_I][D_I/32] E8M0 bytes (value =
 *       code * 2^(scale-127)), as in the MXFP4 checkpoints' indexer path.
 * w:    [T][H_I] fp32 query-dependent head weights (any sign).
 * k_I:  [B][N][k_heads][D_I] keys in dt (MXFP4: [B][N][k_heads][D_I/2] + k_I_scale
 *       [B][N][k_heads][D_I/32]). k_heads = H_I: one key per head (the formula's k_{i,h});
 *       k_heads = 1: one key shared by every head. q_I_scale / k_I_scale are ignored unless
 *       dt == CSA_MXFP4.
 * q_seq [T] int32 sequence of each query; q_pos [T] int64 absolute position.
 * scores: [T][N] fp32. Products and sums are fp32 (MXFP4 products are exact).
 * Supported: H_I == 64, D_I == 128 (the indexer of both model sizes), ratio >= 1; per-head
 * keys in F32 | BF16 | MXFP4, shared keys in BF16 (k_heads other than H_I or 1 is
 * CSA_EINVAL, a shared-key dtype other than BF16 CSA_EUNSUPPORTED). T, N may be 0 (nothing
 * is launched). MXFP4 per-head keys with B == 1 and T > 16 (a prefill chunk of one
 * sequence) run as matrix-core tiles of queries x entries over that one key store; every
 * other MXFP4 case (several sequences, or few queries) streams each query's own keys. Both
 * give the same scores.
 */
int csa_index_scores(const void *q_I, const uint8_t *q_I_scale, const float *w,
                     const void *k_I, const uint8_t *k_I_scale,
                     const int32_t *q_seq, const int64_t *q_pos,
                     int T, int B, int64_t N, int H_I, int D_I, int k_heads, int ratio,
                     csa_dtype dt, float *scores, void *stream);

/*
 * csa_index_topk - the MXFP4 decode scan fused with the top-k (§4.2: FP4 index scores of
 * every stored entry, then each query's k highest), with no [T][N] score array: the scores
 * of a 4,096-entry chunk stay in registers and only the chunk's k winners reach memory;
 * the top-k selection of csa_topk then runs over the winners. topk_idxs / topk_vals equal what
 * csa_topk returns for the scores csa_index_scores computes from the same arguments:
 * ascending index order, ties to the lower index, (-1, -INFINITY) padding past the visible
 * entries.
 *
 * q_I, q_I_scale, w, k_I, k_I_scale, q_seq, q_pos, T, B, N, ratio: as csa_index_scores with
 *       dt = CSA_MXFP4 and per-head keys ([B][N][64][64] codes, [B][N][64][4] scales).
 * topk_idxs: [T][k] int32 out.   topk_vals: [T][k] fp32 out, or NULL.
 * workspace: csa_index_topk_workspace_bytes(T, N, k) bytes (0 when N <= 4,096) for the
 *       chunk winners and the final selection.
 * Supported: H_I == 64, D_I == 128, 1 <= k <= 4096, T <= 65,535, N < 2^31. T may be 0;
 * with N == 0 (k_I and k_I_scale may then be NULL) every row is padding.
 */
size_t csa_index_topk_workspace_bytes(int T, int64_t N, int k);
int csa_index_topk(const uint8_t *q_I, const uint8_t *q_I_scale, const float *w,
                   const uint8_t *k_I, const uint8_t *k_I_scale,
                   const int32_t *q_seq, const int64_t *q_pos, int T, int B, int64_t N,
                   int H_I, int D_I, int ratio, int k, int32_t *topk_idxs, float *topk_vals,
                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * csa_index_rescore - Lightning Indexer scores (the formula of csa_index_scores) of a
 * per-query candidate list: the re-rank step after an FP4 scan has picked 2k candidates
 * (the indexer builds its candidates at twice the top-k, "DeepSeek-V4 混合注意力" §9).
 *
 * cand:   [T][M] int32 entry indices; a negative, >= N or not visible entry scores -inf.
 * q_I, w, k_I, q_seq, q_pos, ratio, dt: as csa_index_scores (per-head keys, F32 | BF16).
 * scores: [T][M] fp32 out, slot by slot.
 * Supported: H_I == 64, D_I == 128. T, M may be 0.
 */
int csa_index_rescore(const void *q_I, const float *w, const void *k_I, const int32_t *cand, int M,
                      const int32_t *q_seq, const int64_t *q_pos, int T, int B, int64_t N,
                      int H_I, int D_I, int ratio, csa_dtype dt, float *scores, void *stream);

/*
 * csa_quantize_mxfp4 - MXFP4 encoding of indexer operands, with the optional Hadamard
 * rotation that the DeepSeek-V4-Pro-MXFP4 page puts in front of the FP4 index dot
 * products (its Indexer section: the query goes through RoPE and a Hadamard rotation
 * before it is scored against the compressed keys). The rotation is orthonormal, so
 * rotating both q_I and k_I leaves every exact dot product unchanged; it spreads outlying
 * channels before the coarse FP4 grid sees them.
 *
 * x:      [rows][D] in dt (CSA_F32 or CSA_BF16).
 * hadamard != 0: y = H x with H the Sylvester-ordered Walsh-Hadamard matrix scaled by
 *         1/sqrt(D) (H[i][j] = (-1)^popcount(i & j) / sqrt(D)), computed in fp32 as
 *         log2(D) butterfly stages (a + b, a - b) on pairs (i, i + h), h = 1, 2, ..,
 *         D/2, then one multiply by the fp32 value of 1/sqrt(D). hadamard == 0: y = x.
 * codes:  [rows][D/2] out, E2M1 nibbles, even element in the low nibble.
 * scales: [rows][D/32] out, E8M0 (value = code * 2^(scale - 127)).
 * out_group_rows, out_group_stride: 0, 0 for the layout above; otherwise input row r is
 *         written to output row (r / out_group_rows) * out_group_stride + r % out_group_rows
 *         of codes and scales (e.g. one entry of 64 head rows per sequence straight into a
 *         [B][N][64] key cache: out_group_rows = 64, out_group_stride = 64 N).
 * Encoding (OCP Microscaling v1.0): per block of 32, scale exponent
 *   E = floor(log2(max |y|)) - 2 clamped to [-127, 127] (-127 for an all-zero block);
 *   each y / 2^E rounds to the nearest of {0, .5, 1, 1.5, 2, 3, 4, 6} (ties to the even
 *   code), saturating at 6, with the sign bit set for negative nonzero codes.
 * Supported: D in {128, 256, 512}. rows may be 0 (nothing is launched).
 */
int csa_quantize_mxfp4(const void *x, int64_t rows, int D, csa_dtype dt, int hadamard,
                       uint8_t *codes, uint8_t *scales, int64_t out_group_rows,
                       int64_t out_group_stride, void *stream);

/*
 * csa_quantize_kv8 - FP8 storage of compressed KV rows ("DeepSeek-V4 混合注意力" §4.2, last
 * paragraph: the RoPE-related dims of the compressed representation are kept in BF16 and
 * the rest is stored in FP8). Read as the OCP Microscaling v1.0 MXFP8 form for the non-RoPE
 * dims. A row of 512 dims (the last 64 the RoPE dims) becomes 592 bytes:
 *   bytes [0, 448)    E4M3 codes of dims 0..447 (OCP E4M3: bias 7, largest finite 448)
 *   bytes [448, 576)  dims 448..511 as bf16 (round to nearest even), little endian
 *   bytes [576, 590)  E8M0 scales, one per 32 codes (value 2^(s - 127))
 *   bytes [590, 592)  zero
 * Per block of 32: e = floor(log2(max |x|)) - 8, clamped to [-127, 127] (-127 for an
 * all-zero block); each code is the finite E4M3 value nearest to |x| / 2^e (ties to the
 * even code, everything above 448 becomes 448) with the sign of x unless it is 0. A row
 * decodes to code * 2^(e) for dims 0..447 and the bf16 values for 448..511.
 *
 * x:      [rows][512] in dt (CSA_F32 | CSA_BF16).
 * out:    [rows][592] bytes; with out_group_rows > 0, input row r goes to output row
 *         (r / out_group_rows) * out_group_stride + r % out_group_rows (e.g. one new entry
 *         per sequence into a [B][N][592] cache: out_group_rows = 1, out_group_stride = N).
 * Supported: rows >= 0 (0 launches nothing). x and out 16-byte aligned.
 */
int csa_quantize_kv8(const void *x, int64_t rows, csa_dtype dt, uint8_t *out, int64_t out_group_rows,
                     int64_t out_group_stride, void *stream);

/*
 * csa_rmsnorm_rope - RMSNorm of each row, then RoPE on its last R dims: the normalisation
 * that "DeepSeek-V4 混合注意力" §6 applies to the queries and to the compressed
 * representation (RMSNorm(x) = x / sqrt(mean(x^2) + eps) times a per-dim gain g), and the
 * partial RoPE of the same section (only the last 64 dims of a head rotate).
 *
 * x:      [rows][D] in dt_in (CSA_F32 | CSA_BF16).
 * g:      [D] fp32 gains.  eps: >= 0 (finite).
 * rope_cs: [ceil(rows / rope_group)][R] fp32, (cos, sin) of pair p at [2p], [2p + 1]; row r uses
 *         table row r / rope_group (rope_group = H for query rows [T][H][D] that share their
 *         token's angles, 1 for one entry per row). NULL when R == 0.
 * out:    [rows][D] in dt_out (CSA_F32 | CSA_BF16); may be x itself when dt_out == dt_in.
 *         x, out, g and rope_cs are 16-byte aligned (rows move as vector accesses).
 * Per row (fp32 arithmetic): y_d = x_d * g_d / sqrt(sum_e x_e^2 / D + eps), 0 when the
 *   denominator is 0; then for p < R/2 the pair (a, b) = (y[D-R+2p], y[D-R+2p+1]) becomes
 *   (a cos - b sin, a sin + b cos); bf16 output rounds to nearest even.
 * Supported: D in {128, 256, 512}; R even, 0 <= R <= D, and a multiple of D / 64 (R = 64
 *   for the pages' heads). rows may be 0 (nothing is launched).
 * Errors: CSA_EINVAL for a bad size, dtype, eps, R or rope_group, a NULL or misaligned
 *   tensor, or out == x with different dtypes; CSA_EUNSUPPORTED for another D or an R
 *   that is not a multiple of D / 64.
 */
int csa_rmsnorm_rope(const void *x, csa_dtype dt_in, int64_t rows, int D, const float *g, float eps,
                     const float *rope_cs, int R, int64_t rope_group, void *out, csa_dtype dt_out,
                     void *stream);

/*
 * csa_topk - per-query top-k selection over index scores (§4.2).
 *
 * scores: [T][N] fp32; -INFINITY (and NaN) entries are never selected.
 * topk_idxs: [T][k] int32 out: the indices of the k largest scores of each row, in
 *   ascending index order; ties at the k-th value go to the lower indices; when a row
 *   has fewer than k finite scores the remaining slots are -1.
 * topk_vals: [T][k] fp32 out (the scores of topk_idxs, -INFINITY for padding), or NULL.
 * workspace: device scratch of at least csa_topk_workspace_bytes(T, N, k) bytes
 *   (may be NULL when that query returns 0).
 * Supported: 1 <= k <= 4096.
 */
size_t csa_topk_workspace_bytes(int T, int64_t N, int k);
int csa_topk(const float *scores, int T, int64_t N, int k,
             int32_t *topk_idxs, float *topk_vals,
             void *workspace, size_t workspace_bytes, void *stream);

/*
 * csa_topk_noalloc - csa_topk without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). It takes the same arguments as csa_topk minus the workspace and
 * returns the same result (same kernels, bit-identical output).
 *
 * The chunk winners of the multi-level selection (rows longer than 32,768 scores) live in
 * a device array inside the library, 16 MiB per GPU, allocated when the library's code is
 * loaded on that GPU and held until the process ends; nothing is allocated per call. The
 * call needs csa_topk_workspace_bytes(T, N, k) <= 16 MiB (e.g. T <= 64 rows of 262,144
 * scores at k = 1,024); larger requests return CSA_EWORKSPACE and launch nothing.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU
 * (different streams, or threads without ordering) race and must not be issued; calls
 * ordered on one stream are safe. The array needs no clearing (each call writes what it
 * reads).
 */
int csa_topk_noalloc(const float *scores, int T, int64_t N, int k,
                     int32_t *topk_idxs, float *topk_vals, void *stream);

/*
 * csa_topk_ids - csa_topk over per-query candidate lists: row t of scores [T][M] scores
 * the entries ids [T][M]; topk_idxs [T][k] receives the entries of the k largest scores
 * in list order (ascending entry order for ascending lists, such as csa_topk's output),
 * ties to the earlier list position, -1 padded; topk_vals as csa_topk. An entry whose
 * score is -INFINITY (e.g. a -1 slot after csa_index_rescore) is never taken.
 * workspace: at least csa_topk_workspace_bytes(T, M, k) bytes. Supported: 1 <= k <= 4096.
 */
int csa_topk_ids(const float *scores, const int32_t *ids, int T, int64_t M, int k,
                 int32_t *topk_idxs, float *topk_vals, void *workspace,
                 size_t workspace_bytes, void *stream);


/*
 * csa_sparse_attn - shared-KV multi-query attention with an attention sink
 * (§4.2, §6; the sparse_attn(q, kv, attn_sink, topk_idxs, softmax_scale) call).
 *
 * For query t (sequence s = q_seq[t], position p = q_pos[t]) and head g the rows are
 *   kv[s][topk_idxs[t][j]] for every j with 0 <= topk_idxs[t][j] < N (others skipped),
 *   then swa_kv[s][r] for every position x in [max(0, p-window+1), p] with
 *   r = x - swa_pos0[s] in [0, swa_rows)   (the raw sliding-window rows, no dedup).
 * q' = q[t][g] with its last rope_dim dims rotated pairwise by rope_cs[t] (pair
 * (D-R+2i, D-R+2i+1) by (cos, sin)); z_j = softmax_scale * <q', row_j>;
 * o' = sum_j e^{z_j} row_j / (e^{attn_sink[g]} + sum_j e^{z_j});
 * out[t][g] = o' with its last rope_dim dims rotated back (by (cos, -sin));
 * lse[t][g] = log(e^{attn_sink[g]} + sum_j e^{z_j}).
 *
 * q: [T][H][D] dt; kv: [B][N][D] dt (already RoPE-rotated as stored in the cache);
 * attn_sink: [H] fp32 (not scaled); topk_idxs: [T][k] int32;
 * swa_kv: [B][swa_rows][D] dt or NULL (then window is ignored); swa_pos0: [B] int64;
 * rope_cs: [T][rope_dim/2][2] fp32 or NULL (rope_dim ignored); out: [T][H][D] dt;
 * lse: [T][H] fp32 or NULL; workspace: csa_attn_workspace_bytes(...) bytes, 16-byte aligned
 *      (CSA_EINVAL otherwise, when the query returns more than 0).
 * Supported: dt F32 | BF16, D <= 1024, D % 64 == 0, rope_dim even and <= D, 0 <= k <= 4096;
 * dt = CSA_KV8: kv rows [B][N][592] bytes in the format of csa_quantize_kv8 (q, swa_kv and
 * out bf16), D = 512 and H a multiple of 64.
 */
size_t csa_attn_workspace_bytes(int T, int H, int D, int64_t max_rows);
int csa_sparse_attn(const void *q, const void *kv, const float *attn_sink,
                    const int32_t *topk_idxs, int k, float softmax_scale,
                    const void *swa_kv, const int64_t *swa_pos0, int swa_rows, int window,
                    const int32_t *q_seq, const int64_t *q_pos,
                    const float *rope_cs, int rope_dim,
                    int T, int B, int64_t N, int H, int D, csa_dtype dt,
                    void *out, float *lse, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * hca_attn - HCA dense shared-KV MQA (§5, §6): csa_sparse_attn with the compressed rows
 * replaced by every summary i < N with (i+1)*ratio <= q_pos[t] (summ: [B][N][D] dt),
 * followed by the same SWA rows, sink, RoPE and outputs. max_rows for the workspace
 * query is N + window.
 */
int hca_attn(const void *q, const void *summ, const float *attn_sink, int ratio,
             float softmax_scale, const void *swa_kv, const int64_t *swa_pos0, int swa_rows,
             int window, const int32_t *q_seq, const int64_t *q_pos,
             const float *rope_cs, int rope_dim,
             int T, int B, int64_t N, int H, int D, csa_dtype dt,
             void *out, float *lse, void *workspace, size_t workspace_bytes, void *stream);

/* Static name of a status code. */
const char *csa_status_str(int status);
/* Detail string of the last non-OK return on the calling thread ("" if none). */
const char *csa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* CSA_H */
