/*
 * CPU oracle for the DeepSeek-V4 CSA / HCA attention hot path.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, fp64 definition of what
 * the path computes. Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load it; the GPU library never links, includes or calls it, and it
 * shares no header, helper or table with the GPU sources.
 *
 * Source: "DeepSeek-V4 混合注意力：从压缩记忆到百万上下文" (brenchcc notes):
 *   compress (ratio 4)    §4.1, equations for alpha_{i,:,j} and C^comp_{i,j}
 *   compress (ratio 128)  §5, equations for beta_{i,:,j} and C^hca_{i,j}
 *   index score           §4.2, equation for s_{t,i}
 *   top-k                 §2 table (Top-k 512 / 1,024) and §4.2
 *   sink softmax          §6, equation for p_i
 *   shared-KV MQA         §4.2 (one compressed vector is both K and V), §7 call chain
 *   SWA, partial RoPE     §6 (window 128, RoPE on the last 64 dims, inverse RoPE on o)
 *   MXFP4 operands        the MXFP4 model-card page (one E8M0 scale per 32 E2M1 values)
 *   Hadamard rotation     the same page's Indexer section (q rotated before FP4 scoring)
 *   RMSNorm               §6, equation for RMSNorm(x) (Q and the compressed entries)
 *   FP8 KV storage        §4.2 last paragraph (RoPE dims BF16, the rest FP8)
 *   projections           §4.1 (C^a, C^b, Z^a, Z^b formed from the hidden state H), §7
 *                         (Compressor.forward: project_a / project_b), §4.2 and §7
 *                         (outputs aggregated per group and projected to the model width)
 *
 * Every sum, dot product and softmax is accumulated in double precision and each
 * logit vector is materialised before it is normalised.
 *
 * Readings where the pages leave a step open:
 *  - the sum index r = 1..m of the compression equations is read as the same rows
 *    as the softmax slice, i.e. row (i-1)m + r - 1 (0-based);
 *  - a compression slot with no row (the b-branch of entry 0 without a carry) has
 *    weight zero;
 *  - a query at absolute position t sees compressed entry i iff (i+1)*ratio <= t;
 *  - the SWA rows of a query at t are positions max(0, t-window+1) .. t;
 *  - a RoPE pair is the interleaved pair (D-R+2p, D-R+2p+1), rotated by (cos, sin)
 *    of the caller's table; the output is rotated back with (cos, -sin);
 *  - top-k ties are broken by the lower entry index; -INF scores are never taken;
 *  - RMSNorm of an all-zero row with eps = 0 (0/0) is read as a zero row;
 *  - a projection is a plain linear map y = W x with W stored [out][in];
 *  - the grouped output projection: the H heads form G groups of H/G consecutive heads;
 *    group g's concatenated head outputs are mapped by its own W_a[g] to d_g values, and
 *    the G results side by side are mapped by W_b to the model width.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL 1

/* ---------------------------------------------------------------------------------
 * Compressor.  §4.1 (ratio 4, overlapped: the b-branch of block i-1 and the
 * a-branch of block i share one per-channel softmax over 2m slots) and §5
 * (ratio 128, non-overlapped: one softmax over the m' rows of block i).
 *
 * Ca, Za: [B][n][c]. Cb, Zb: [B][n][c] or NULL when overlap == 0.
 * carry_Cb, carry_Zb: [B][ratio][c] b-branch rows of the block before row 0, or NULL.
 * bias: [(1+overlap)*ratio][c] positional logit bias, or NULL.
 * out:  [B][n/ratio][c].
 * ------------------------------------------------------------------------------- */
int oracle_compress(const double *Ca, const double *Cb, const double *Za, const double *Zb,
                    const double *carry_Cb, const double *carry_Zb, const double *bias,
                    int B, int64_t n, int c, int ratio, int overlap, double *out)
{
    if (B < 0 || n < 0 || c <= 0 || ratio <= 0 || (overlap != 0 && overlap != 1)) return OR_EINVAL;
    if (overlap && (!Cb || !Zb)) return OR_EINVAL;
    const int64_t E = n / ratio;           /* a trailing partial block is not compressed */
    const int S = (1 + overlap) * ratio;   /* slots in one entry's receptive field */

#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b) {
        for (int64_t i = 0; i < E; ++i) {
            double *logit = (double *)malloc(sizeof(double) * S);
            double *val = (double *)malloc(sizeof(double) * S);
            int *has = (int *)malloc(sizeof(int) * S);
            for (int j = 0; j < c; ++j) {
                /* gather the receptive field of entry i, channel j */
                for (int s = 0; s < S; ++s) {
                    int is_b = overlap && s < ratio;
                    int r = is_b ? s : s - overlap * ratio;
                    has[s] = 1;
                    if (is_b) {
                        if (i >= 1) {
                            int64_t row = (i - 1) * ratio + r;
                            logit[s] = Zb[((int64_t)b * n + row) * c + j];
                            val[s] = Cb[((int64_t)b * n + row) * c + j];
                        } else if (carry_Cb && carry_Zb) {
                            logit[s] = carry_Zb[((int64_t)b * ratio + r) * c + j];
                            val[s] = carry_Cb[((int64_t)b * ratio + r) * c + j];
                        } else {
                            has[s] = 0;
                        }
                    } else {
                        int64_t row = i * ratio + r;
                        logit[s] = Za[((int64_t)b * n + row) * c + j];
                        val[s] = Ca[((int64_t)b * n + row) * c + j];
                    }
                    if (has[s] && bias) logit[s] += bias[(int64_t)s * c + j];
                }
                /* softmax over the present slots, then the weighted sum */
                double M = -INFINITY;
                for (int s = 0; s < S; ++s)
                    if (has[s] && logit[s] > M) M = logit[s];
                double den = 0.0, num = 0.0;
                for (int s = 0; s < S; ++s) {
                    if (!has[s]) continue;
                    double e = exp(logit[s] - M);
                    den += e;
                    num += e * val[s];
                }
                out[((int64_t)b * E + i) * c + j] = num / den;
            }
            free(logit);
            free(val);
            free(has);
        }
    }
    return OR_OK;
}

/* ---------------------------------------------------------------------------------
 * Projection Y = X W^T: Y[m][o] = sum_k X[m][k] W[o][k].  X: [M][K], W: [N][K], Y: [M][N].
 * ------------------------------------------------------------------------------- */
int oracle_matmul_nt(const double *X, const double *W, int64_t M, int64_t N, int64_t K, double *Y)
{
    if (M < 0 || N < 0 || K < 0) return OR_EINVAL;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t o = 0; o < N; ++o) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += X[m * K + k] * W[o * K + k];
            Y[m * N + o] = acc;
        }
    return OR_OK;
}

/* ---------------------------------------------------------------------------------
 * The compressor fed from hidden rows.  §4.1: C^a, C^b, Z^a, Z^b are formed from H;
 * §7: Compressor.forward projects the hidden rows (project_a, and project_b for the
 * overlapped ratio-4 compressor) and then pools.
 *
 * H: [B][n][d]; carry_H: [B][4][d] hidden rows before the chunk (ratio 4), or NULL;
 * W: [(1+overlap)*2][c][d] in the order W_Ca, W_Za (, W_Cb, W_Zb); bias as oracle_compress.
 * out: [B][n/ratio][c].
 * ------------------------------------------------------------------------------- */
int oracle_compress_hidden(const double *H, const double *carry_H, const double *W, const double *bias,
                           int B, int64_t n, int64_t d, int c, int ratio, int overlap, double *out)
{
    if (B < 0 || n < 0 || d <= 0 || c <= 0 || ratio <= 0 || (overlap != 0 && overlap != 1)) return OR_EINVAL;
    if (!overlap && carry_H) return OR_EINVAL;
    const int np = 2 * (1 + overlap);
    const int64_t plane = (int64_t)B * n * c;
    double *P = (double *)malloc(sizeof(double) * (size_t)(plane > 0 ? plane : 1) * np);
    double *cP = carry_H ? (double *)malloc(sizeof(double) * (size_t)B * ratio * c * 2) : NULL;
    for (int p = 0; p < np; ++p)           /* every hidden row through every projection */
        oracle_matmul_nt(H, W + (int64_t)p * c * d, (int64_t)B * n, c, d, P + (int64_t)p * plane);
    if (carry_H)                           /* the b-branch of the carry rows */
        for (int p = 0; p < 2; ++p)
            oracle_matmul_nt(carry_H, W + (int64_t)(2 + p) * c * d, (int64_t)B * ratio, c, d,
                             cP + (int64_t)p * B * ratio * c);
    int rc = oracle_compress(P, overlap ? P + 2 * plane : NULL, P + plane, overlap ? P + 3 * plane : NULL,
                             cP, cP ? cP + (int64_t)B * ratio * c : NULL, bias, B, n, c, ratio, overlap, out);
    free(P);
    free(cP);
    return rc;
}

/* ---------------------------------------------------------------------------------
 * Grouped output projection.  §4.2: the attention outputs are aggregated per group and
 * projected back to the model width; §7: grouped_output_projection(inverse_rope(o)).
 *
 * o: [T][H][D] (already rotated back); Wa: [G][d_g][(H/G)*D]; Wb: [d_model][G*d_g] or NULL.
 * out: [T][d_model], or [T][G*d_g] (the group results) when Wb is NULL.
 * ------------------------------------------------------------------------------- */
int oracle_out_proj(const double *o, int T, int H, int D, int G, const double *Wa, int d_g,
                    const double *Wb, int d_model, double *out)
{
    if (T < 0 || H <= 0 || D <= 0 || G <= 0 || d_g <= 0 || H % G != 0 || (Wb && d_model <= 0)) return OR_EINVAL;
    const int64_t K1 = (int64_t)(H / G) * D, GY = (int64_t)G * d_g;
    double *y = Wb ? (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * GY) : out;
#pragma omp parallel for collapse(2) schedule(static)
    for (int t = 0; t < T; ++t)
        for (int g = 0; g < G; ++g) {
            const double *x = o + (int64_t)t * H * D + (int64_t)g * K1;   /* group g's heads, side by side */
            for (int e = 0; e < d_g; ++e) {
                const double *wr = Wa + ((int64_t)g * d_g + e) * K1;
                double acc = 0.0;
                for (int64_t k = 0; k < K1; ++k) acc += wr[k] * x[k];
                y[(int64_t)t * GY + (int64_t)g * d_g + e] = acc;
            }
        }
    if (Wb) {
        oracle_matmul_nt(y, Wb, T, d_model, GY, out);
        free(y);
    }
    return OR_OK;
}

/* ---------------------------------------------------------------------------------
 * Lightning Indexer score.  §4.2:  s_{t,i} = sum_h w_{t,h} ReLU(<q^I_{t,h}, k^I_{i,h}>).
 *
 * qI: [T][H][Dh]; w: [T][H]; kI: [B][N][kh][Dh] with kh = H (per-head keys) or 1.
 * entry_ids: [N] absolute entry index of each stored key row (NULL: row i is entry i);
 * used to check a sample of a long key store without materialising all of it.
 * scores: [T][N]; -INF where the entry's block is not wholly before q_pos[t].
 * ------------------------------------------------------------------------------- */
int oracle_index_scores(const double *qI, const double *w, const double *kI,
                        const int32_t *q_seq, const int64_t *q_pos, const int64_t *entry_ids,
                        int T, int B, int64_t N, int H, int Dh, int kh, int ratio, double *scores)
{
    if (T < 0 || B <= 0 || N < 0 || H <= 0 || Dh <= 0 || (kh != H && kh != 1) || ratio <= 0)
        return OR_EINVAL;
#pragma omp parallel for collapse(2) schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int64_t i = 0; i < N; ++i) {
            const int s = q_seq[t];
            const int64_t e = entry_ids ? entry_ids[i] : i;
            double sc = -INFINITY;
            if (s >= 0 && s < B && (e + 1) * (int64_t)ratio <= q_pos[t]) {
                sc = 0.0;
                for (int h = 0; h < H; ++h) {
                    const double *q = qI + ((int64_t)t * H + h) * Dh;
                    const int hk = (kh == H) ? h : 0;
                    const double *k = kI + (((int64_t)s * N + i) * kh + hk) * Dh;
                    double dot = 0.0;
                    for (int d = 0; d < Dh; ++d) dot += q[d] * k[d];
                    sc += w[(int64_t)t * H + h] * (dot > 0.0 ? dot : 0.0);
                }
            }
            scores[(int64_t)t * N + i] = sc;
        }
    }
    return OR_OK;
}

/* ---------------------------------------------------------------------------------
 * Compressed-KV storage format.  §4.2 (last paragraph): the RoPE-related dims of the
 * compressed representation are kept in BF16 and the rest is stored in FP8. Read here as
 * the OCP Microscaling v1.0 MXFP8 form for the non-RoPE dims: E4M3 elements (bias 7,
 * largest finite 448, S.1111.111 is NaN) sharing one E8M0 scale per 32 elements; the last
 * R dims as bf16 (round to nearest even).
 *
 * Row of D dims with R RoPE dims (D - R a multiple of 32), in bytes:
 *   [0, D-R)              E4M3 codes of dims 0 .. D-R-1
 *   [D-R, D+R)            bf16 of dims D-R .. D-1 (little endian)
 *   [D+R, D+R+(D-R)/32)   E8M0 scales (value 2^(s-127)), one per 32 codes
 *   padding to a multiple of 16 bytes (zeros)
 * D = 512, R = 64: 448 + 128 + 14 (+2) = 592 bytes, against 1,024 in bf16.
 *
 * Encoding of a block of 32 (x as fp32): e = floor(log2(amax)) - 8 (8 = the largest E4M3
 * exponent), clamped to [-127, 127], -127 for an all-zero block; each element becomes the
 * finite E4M3 value nearest to |x| / 2^e (ties to the even code; beyond 448 saturates to
 * 448) with the sign of x unless the code is 0.
 * ------------------------------------------------------------------------------- */
static double or_e4m3(int code)
{
    const int e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    const double v = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return (code & 0x80) ? -v : v;
}

int oracle_kv8_row_bytes(int D, int R)
{
    if (D <= 0 || R < 0 || R > D || (D - R) % 32) return -1;
    const int raw = (D - R) + 2 * R + (D - R) / 32;
    return (raw + 15) / 16 * 16;
}

static uint16_t or_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

int oracle_kv8_encode(const float *x, int64_t rows, int D, int R, uint8_t *out)
{
    const int rb = oracle_kv8_row_bytes(D, R);
    if (rb < 0) return OR_EINVAL;
    const int nq = D - R;
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + r * D;
        uint8_t *o = out + r * rb;
        memset(o, 0, (size_t)rb);
        for (int b = 0; b < nq / 32; ++b) {
            double amax = 0.0;
            for (int i = 32 * b; i < 32 * b + 32; ++i)
                if (fabs((double)xr[i]) > amax) amax = fabs((double)xr[i]);
            int e = (amax > 0.0) ? (int)floor(log2(amax)) - 8 : -127;
            if (e < -127) e = -127;
            if (e > 127) e = 127;
            o[nq + 2 * R + b] = (uint8_t)(e + 127);
            for (int i = 32 * b; i < 32 * b + 32; ++i) {
                const double v = fabs((double)xr[i]) / ldexp(1.0, e);
                int best = 0;
                for (int c = 1; c < 127; ++c) {  /* the finite non-negative codes */
                    const double dc = fabs(v - or_e4m3(c)), db = fabs(v - or_e4m3(best));
                    if (dc < db || (dc == db && (c % 2 == 0) && (best % 2 != 0))) best = c;
                }
                o[i] = (uint8_t)((xr[i] < 0.0f && best != 0) ? (best | 0x80) : best);
            }
        }
        for (int i = 0; i < R; ++i) {
            const uint16_t h = or_bf16_rne(xr[nq + i]);
            o[nq + 2 * i] = (uint8_t)(h & 0xff);
            o[nq + 2 * i + 1] = (uint8_t)(h >> 8);
        }
    }
    return OR_OK;
}

int oracle_kv8_decode(const uint8_t *rows, int64_t nrows, int D, int R, double *out)
{
    const int rb = oracle_kv8_row_bytes(D, R);
    if (rb < 0) return OR_EINVAL;
    const int nq = D - R;
    for (int64_t r = 0; r < nrows; ++r) {
        const uint8_t *o = rows + r * rb;
        double *y = out + r * D;
        for (int i = 0; i < nq; ++i) {
            const uint8_t sc = o[nq + 2 * R + i / 32];
            y[i] = (sc == 255) ? NAN : or_e4m3(o[i]) * ldexp(1.0, (int)sc - 127);
        }
        for (int i = 0; i < R; ++i) {
            const uint32_t h = (uint32_t)o[nq + 2 * i] | ((uint32_t)o[nq + 2 * i + 1] << 8);
            const uint32_t u = h << 16;
            float f;
            memcpy(&f, &u, 4);
            y[nq + i] = f;
        }
    }
    return OR_OK;
}

/* the E4M3 value of each code (closed form above), for the pins */
int oracle_e4m3_table(double *out256)
{
    for (int c = 0; c < 256; ++c) out256[c] = or_e4m3(c);
    return OR_OK;
}

/* ---------------------------------------------------------------------------------
 * MXFP4 decode (the page on DeepSeek-V4-Pro-MXFP4: E2M1 values sharing one E8M0
 * scale per 32 elements). Value = sign * {0,.5,1,1.5,2,3,4,6}[code&7] * 2^(scale-127);
 * element 2m sits in the low nibble of byte m; scale byte 255 is NaN.
 * ------------------------------------------------------------------------------- */
int oracle_mxfp4_decode(const uint8_t *codes, const uint8_t *scales, int64_t nelem, double *out)
{
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    if (nelem % 32) return OR_EINVAL;
    for (int64_t e = 0; e < nelem; ++e) {
        uint8_t byte = codes[e / 2];
        int nib = (e & 1) ? (byte >> 4) : (byte & 15);
        uint8_t sc = scales[e / 32];
        double v = mag[nib & 7] * ldexp(1.0, (int)sc - 127);
        if (nib & 8) v = -v;
        out[e] = (sc == 255) ? NAN : v;
    }
    return OR_OK;
}

/* ---------------------------------------------------------------------------------
 * MXFP4 encode, with the optional Hadamard rotation in front (the DeepSeek-V4-Pro-MXFP4
 * page, Indexer: the query goes through RoPE and a Hadamard rotation before it is scored
 * in FP4).
 *
 * Rotation: y = H x with H = the Sylvester-ordered D x D Walsh-Hadamard matrix over
 * sqrt(D), taken as the textbook fast transform in single precision: stages h = 1, 2,
 * .., D/2 replace each pair (i, i + h) with bit h of i clear by (a + b, a - b); then
 * every element is multiplied by (float)(1/sqrt(D)). Which FP4 code a value gets
 * depends on its float rounding, so this side rounds at exactly these steps.
 *
 * Encoding (OCP Microscaling v1.0, E2M1 elements, one E8M0 scale per 32): block
 * exponent e = floor(log2(amax)) - 2 (2 = the largest E2M1 exponent), clamped to
 * [-127, 127], -127 for an all-zero block; each element becomes the E2M1 value nearest
 * to |y| / 2^e (ties to the even code; everything above 6 becomes 6) with the sign of
 * y unless the code is 0. Codes pack two per byte, element 2m in the low nibble.
 * ------------------------------------------------------------------------------- */
static void or_hadamard_row(float *y, int D)
{
    const float norm = (float)(1.0 / sqrt((double)D));
    for (int h = 1; h < D; h *= 2)
        for (int i = 0; i < D; ++i)
            if (!(i & h)) {
                const float a = y[i], b = y[i + h];
                y[i] = a + b;
                y[i + h] = a - b;
            }
    for (int i = 0; i < D; ++i) y[i] = y[i] * norm;
}

/* the rotation alone, row by row (D a power of two) */
int oracle_hadamard(const float *x, int64_t rows, int D, float *out)
{
    if (D <= 0 || (D & (D - 1))) return OR_EINVAL;
    for (int64_t r = 0; r < rows; ++r) {
        memcpy(out + r * D, x + r * D, (size_t)D * sizeof(float));
        or_hadamard_row(out + r * D, D);
    }
    return OR_OK;
}

int oracle_mxfp4_encode(const float *x, int64_t rows, int D, int hadamard, uint8_t *codes, uint8_t *scales)
{
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    if (D <= 0 || D % 32) return OR_EINVAL;
    if (hadamard && (D & (D - 1))) return OR_EINVAL;
    float *y = (float *)malloc((size_t)D * sizeof(float));
    if (!y) return OR_EINVAL;
    for (int64_t r = 0; r < rows; ++r) {
        memcpy(y, x + r * D, (size_t)D * sizeof(float));
        if (hadamard) or_hadamard_row(y, D);
        memset(codes + r * (D / 2), 0, (size_t)(D / 2));
        for (int b = 0; b < D / 32; ++b) {
            double amax = 0.0;
            for (int i = 32 * b; i < 32 * b + 32; ++i)
                if (fabs((double)y[i]) > amax) amax = fabs((double)y[i]);
            int e = (amax > 0.0) ? (int)floor(log2(amax)) - 2 : -127;
            if (e < -127) e = -127;
            if (e > 127) e = 127;
            scales[r * (D / 32) + b] = (uint8_t)(e + 127);
            for (int i = 32 * b; i < 32 * b + 32; ++i) {
                const double m = fabs((double)y[i]) / ldexp(1.0, e);
                int best = 0;
                for (int c = 1; c < 8; ++c) {
                    const double dc = fabs(m - mag[c]), db = fabs(m - mag[best]);
                    if (dc < db || (dc == db && (c % 2 == 0) && (best % 2 != 0))) best = c;
                }
                int nib = best;
                if (y[i] < 0.0f && best != 0) nib |= 8;
                codes[r * (D / 2) + i / 2] |= (uint8_t)((i & 1) ? (nib << 4) : nib);
            }
        }
    }
    free(y);
    return OR_OK;
}

/* ---------------------------------------------------------------------------------
 * RMSNorm of a row, then RoPE on its last R dims ("DeepSeek-V4 混合注意力" §6: RMSNorm
 * on Q and on the compressed representation, x / sqrt(mean(x^2) + eps) scaled per dim
 * by g; RoPE on the last 64 dims of each head):
 *   y_d = x_d / sqrt(eps + (1/D) sum_e x_e^2) * g_d
 *   (y_{D-R+2p}, y_{D-R+2p+1}) <- (y0 c - y1 s, y0 s + y1 c),  (c, s) = cs[r / group][p]
 * x, out: [rows][D]; g: [D]; cs: [rows / group][R/2][2] or NULL (R = 0).
 * ------------------------------------------------------------------------------- */
int oracle_rmsnorm_rope(const double *x, int64_t rows, int D, const double *g, double eps,
                        const double *cs, int R, int64_t group, double *out)
{
    if (D <= 0 || !(eps >= 0.0) || R < 0 || R % 2 || R > D || (R > 0 && !cs) || group < 1) return OR_EINVAL;
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * D;
        double *y = out + r * D;
        double ss = 0.0;
        for (int d = 0; d < D; ++d) ss += xr[d] * xr[d];
        const double den = sqrt(ss / D + eps);
        for (int d = 0; d < D; ++d) y[d] = (den > 0.0) ? xr[d] / den * g[d] : 0.0;
        const double *c = (R > 0) ? cs + (r / group) * R : NULL;
        for (int p = 0; p < R / 2; ++p) {
            const double y0 = y[D - R + 2 * p], y1 = y[D - R + 2 * p + 1];
            y[D - R + 2 * p] = y0 * c[2 * p] - y1 * c[2 * p + 1];
            y[D - R + 2 * p + 1] = y0 * c[2 * p + 1] + y1 * c[2 * p];
        }
    }
    return OR_OK;
}

/* ---------------------------------------------------------------------------------
 * Top-k: the k largest finite scores of each row, ties to the lower index,
 * padded with -1 (value -INF) when fewer than k are finite.
 * ------------------------------------------------------------------------------- */
typedef struct {
    double s;
    int64_t i;
} or_pair;

static int or_pair_cmp(const void *a, const void *b)
{
    const or_pair *x = (const or_pair *)a, *y = (const or_pair *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->i < y->i) ? -1 : (x->i > y->i);
}

int oracle_topk(const double *scores, int T, int64_t N, int k, int32_t *idx, double *vals)
{
    if (T < 0 || N < 0 || k <= 0) return OR_EINVAL;
#pragma omp parallel for schedule(dynamic)
    for (int t = 0; t < T; ++t) {
        or_pair *p = (or_pair *)malloc(sizeof(or_pair) * (N > 0 ? N : 1));
        int64_t cnt = 0;
        for (int64_t i = 0; i < N; ++i) {
            double s = scores[(int64_t)t * N + i];
            if (isfinite(s)) {
                p[cnt].s = s;
                p[cnt].i = i;
                ++cnt;
            }
        }
        qsort(p, (size_t)cnt, sizeof(or_pair), or_pair_cmp);
        for (int j = 0; j < k; ++j) {
            idx[(int64_t)t * k + j] = (j < cnt) ? (int32_t)p[j].i : -1;
            if (vals) vals[(int64_t)t * k + j] = (j < cnt) ? p[j].s : -INFINITY;
        }
        free(p);
    }
    return OR_OK;
}

/* ---------------------------------------------------------------------------------
 * Shared-KV MQA with a sink logit over an explicit row set (§4.2, §6).
 *   z_j = scale <q', row_j>;  p_j = e^{z_j} / (e^{sink} + sum_l e^{z_l});  o' = sum_j p_j row_j
 *   lse = log(e^{sink} + sum_j e^{z_j})
 * q' is q with its last R dims rotated forward, o is o' with its last R dims rotated back.
 * ------------------------------------------------------------------------------- */
static void mqa_rows(const double *qrow, const double *const *rows, int64_t L, double sink,
                     double scale, const double *cs, int R, int D, double *o, double *lse)
{
    double *qv = (double *)malloc(sizeof(double) * D);
    double *z = (double *)malloc(sizeof(double) * (L > 0 ? L : 1));
    memcpy(qv, qrow, sizeof(double) * D);
    if (cs) {
        for (int p = 0; p < R / 2; ++p) {
            double c = cs[2 * p], s = cs[2 * p + 1];
            double x0 = qv[D - R + 2 * p], x1 = qv[D - R + 2 * p + 1];
            qv[D - R + 2 * p] = x0 * c - x1 * s;
            qv[D - R + 2 * p + 1] = x0 * s + x1 * c;
        }
    }
    double M = sink;
    for (int64_t j = 0; j < L; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qv[d] * rows[j][d];
        z[j] = scale * dot;
        if (z[j] > M) M = z[j];
    }
    double den = exp(sink - M);
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t j = 0; j < L; ++j) {
        double e = exp(z[j] - M);
        den += e;
        for (int d = 0; d < D; ++d) o[d] += e * rows[j][d];
    }
    for (int d = 0; d < D; ++d) o[d] /= den;
    if (cs) {
        for (int p = 0; p < R / 2; ++p) {
            double c = cs[2 * p], s = cs[2 * p + 1];
            double x0 = o[D - R + 2 * p], x1 = o[D - R + 2 * p + 1];
            o[D - R + 2 * p] = x0 * c + x1 * s;
            o[D - R + 2 * p + 1] = -x0 * s + x1 * c;
        }
    }
    *lse = M + log(den);
    free(qv);
    free(z);
}

/* SWA rows of a query at t: positions max(0, t-window+1)..t present in swa[s]. */
static int64_t add_swa_rows(const double **rows, int64_t L, const double *swa, const int64_t *swa_pos0,
                            int swa_rows, int window, int s, int64_t t, int D)
{
    if (!swa || window <= 0) return L;
    int64_t lo = t - window + 1;
    if (lo < 0) lo = 0;
    for (int64_t p = lo; p <= t; ++p) {
        int64_t r = p - swa_pos0[s];
        if (r >= 0 && r < swa_rows) rows[L++] = swa + ((int64_t)s * swa_rows + r) * D;
    }
    return L;
}

/* q: [T][H][D]; kv: [B][N][D]; sink: [H]; topk_idxs: [T][k] (-1 or out of range: skipped);
 * swa: [B][swa_rows][D], row r of sequence s holds position swa_pos0[s] + r;
 * rope_cs: [T][R/2][2] or NULL; out: [T][H][D]; lse: [T][H] or NULL. */
int oracle_sparse_attn(const double *q, const double *kv, const double *sink,
                       const int32_t *topk_idxs, int k, double scale,
                       const double *swa, const int64_t *swa_pos0, int swa_rows, int window,
                       const int32_t *q_seq, const int64_t *q_pos, const double *rope_cs, int R,
                       int T, int B, int64_t N, int H, int D, double *out, double *lse)
{
    if (T < 0 || B <= 0 || N < 0 || H <= 0 || D <= 0 || k < 0 || window < 0) return OR_EINVAL;
    if (rope_cs && (R <= 0 || R % 2 || R > D)) return OR_EINVAL;
#pragma omp parallel for schedule(dynamic)
    for (int t = 0; t < T; ++t) {
        const int s = q_seq[t];
        const double **rows = (const double **)malloc(sizeof(double *) * ((size_t)k + window + 1));
        int64_t L = 0;
        for (int j = 0; j < k; ++j) {
            int32_t id = topk_idxs[(int64_t)t * k + j];
            if (id >= 0 && id < N) rows[L++] = kv + ((int64_t)s * N + id) * D;
        }
        L = add_swa_rows(rows, L, swa, swa_pos0, swa_rows, window, s, q_pos[t], D);
        for (int g = 0; g < H; ++g) {
            double l;
            mqa_rows(q + ((int64_t)t * H + g) * D, rows, L, sink[g], scale,
                     rope_cs ? rope_cs + (int64_t)t * R : NULL, R, D,
                     out + ((int64_t)t * H + g) * D, &l);
            if (lse) lse[(int64_t)t * H + g] = l;
        }
        free(rows);
    }
    return OR_OK;
}

/* HCA (§5): every summary i with (i+1)*ratio <= t, plus the SWA rows. summ: [B][N][D]. */
int oracle_hca_attn(const double *q, const double *summ, const double *sink, int ratio, double scale,
                    const double *swa, const int64_t *swa_pos0, int swa_rows, int window,
                    const int32_t *q_seq, const int64_t *q_pos, const double *rope_cs, int R,
                    int T, int B, int64_t N, int H, int D, double *out, double *lse)
{
    if (T < 0 || B <= 0 || N < 0 || H <= 0 || D <= 0 || ratio <= 0 || window < 0) return OR_EINVAL;
    if (rope_cs && (R <= 0 || R % 2 || R > D)) return OR_EINVAL;
#pragma omp parallel for schedule(dynamic)
    for (int t = 0; t < T; ++t) {
        const int s = q_seq[t];
        const double **rows = (const double **)malloc(sizeof(double *) * ((size_t)N + window + 1));
        int64_t L = 0;
        for (int64_t i = 0; i < N; ++i)
            if ((i + 1) * (int64_t)ratio <= q_pos[t]) rows[L++] = summ + ((int64_t)s * N + i) * D;
        L = add_swa_rows(rows, L, swa, swa_pos0, swa_rows, window, s, q_pos[t], D);
        for (int g = 0; g < H; ++g) {
            double l;
            mqa_rows(q + ((int64_t)t * H + g) * D, rows, L, sink[g], scale,
                     rope_cs ? rope_cs + (int64_t)t * R : NULL, R, D,
                     out + ((int64_t)t * H + g) * D, &l);
            if (lse) lse[(int64_t)t * H + g] = l;
        }
        free(rows);
    }
    return OR_OK;
}
