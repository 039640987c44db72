// Per-query top-k over index scores on gfx950 ("DeepSeek-V4 混合注意力" §4.2: each
// query keeps the k = 512 / 1,024 highest-scoring compressed entries).
//
// A workgroup (1024 lanes) owns one chunk of at most `cap` scores of one row and keeps
// it in LDS as order-preserving 32-bit keys (-inf / NaN map to 0 and are never taken):
//   1. three radix passes (digits of 11, 11 and 10 bits from the top) find the exact key
//      tau of the k-th largest element and how many elements equal to tau are to be
//      taken (ties go to the lower index); after the first pass the keys of the leading
//      bin are copied to a short LDS list when they fit, so the later passes scan only
//      that list; histogram increments are aggregated per wavefront for the common case
//      of a wave whose active lanes share one digit;
//   2. an ordered compaction (block scans over contiguous per-lane segments) writes the
//      selected (value, index) pairs in ascending index order.
// Rows longer than `cap` are cut into chunks; the exact top-k of the row is a subset of
// the union of the chunks' top-k sets, so the chunk winners (kept in index order) form a
// shorter row that the same kernel reduces again until one chunk remains.
#include "common.hpp"
#include "internal.hpp"

namespace csa {

namespace {

constexpr int NT = 1024;
constexpr int NW = NT / 64;
constexpr int kCand = 4096;  // LDS list of keys sharing the leading digit

__device__ __forceinline__ uint32_t order_key(float s) {
    if (!(s > -INFINITY)) return 0u;
    const uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// exclusive block scan of one int per thread (all NT threads must call it)
__device__ __forceinline__ int block_excl_scan(int v, int *wsum, int &total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    if (wv == 0) {
        int s = (lane < NW) ? wsum[lane] : 0;
#pragma unroll
        for (int o = 1; o < NW; o <<= 1) {
            const int y = __shfl_up(s, o);
            if (lane >= o) s += y;
        }
        if (lane < NW) wsum[NW + lane] = s;  // inclusive totals
    }
    __syncthreads();
    const int before = (wv > 0) ? wsum[NW + wv - 1] : 0;
    total = wsum[NW + NW - 1];
    __syncthreads();
    return before + x - v;
}

// Histogram of one radix digit (bits [shift, shift+nbits)) over the active keys, i.e.
// keys != 0 whose bits above the digit equal `prefix` (under `pmask`). Increments from
// lanes of a wavefront that share the first active lane's digit are merged into one
// atomic (the common case: scores concentrate in a few leading-digit bins).
__device__ __forceinline__ void digit_hist(const uint32_t *src, int n, uint32_t prefix, uint32_t pmask,
                                           int shift, uint32_t dmask, int *hist) {
    const int lane = threadIdx.x & 63;
    for (int base = 0; base < n; base += NT) {
        const int p = base + (int)threadIdx.x;
        const uint32_t key = (p < n) ? src[p] : 0u;
        const bool act = key != 0u && (key & pmask) == prefix;
        const int d = (int)((key >> shift) & dmask);
        const uint64_t am = __ballot(act);
        if (am) {
            const int lead = __ffsll((unsigned long long)am) - 1;
            const int dl = __shfl(d, lead);
            const uint64_t same = __ballot(act && d == dl);
            if (lane == lead) atomicAdd(&hist[dl], (int)__popcll(same));
            if (act && d != dl) atomicAdd(&hist[d], 1);
        }
    }
}

// Given a histogram of nbins digits and kr (how many of the active keys to keep, counted
// from the top), find the digit holding the kr-th largest and how many keys of that digit
// are still to be kept. Two bins per thread, scanned from the top digit down.
__device__ __forceinline__ void pick_digit(const int *hist, int nbins, int kr, int *wsum, int *sel) {
    const int tid = threadIdx.x;
    const int b0 = nbins - 1 - 2 * tid;  // the thread's two bins, top first: b0, b0 - 1
    const int h0 = (b0 >= 0) ? hist[b0] : 0;
    const int h1 = (b0 - 1 >= 0) ? hist[b0 - 1] : 0;
    int total;
    const int above = block_excl_scan(h0 + h1, wsum, total);  // keys in digits > b0
    if (b0 >= 0) {
        if (above < kr && above + h0 >= kr) {
            sel[0] = b0;
            sel[1] = kr - above;
        } else if (b0 - 1 >= 0 && above + h0 < kr && above + h0 + h1 >= kr) {
            sel[0] = b0 - 1;
            sel[1] = kr - above - h0;
        }
    }
    __syncthreads();
}

// vals_in/idx_in: rows of length L (row stride L); idx_in == nullptr means the index of
// position p is the position itself. The chunk of this block is positions
// [blockIdx.x * chunk, +chunk) of row blockIdx.y. Output slots [t][blockIdx.x*out_slots ...],
// row stride out_ld; exactly min(k, #valid) pairs are written in index order, the rest padded.
__global__ void __launch_bounds__(NT)
topk_select_kernel(const float *__restrict__ vals_in, const int32_t *__restrict__ idx_in, int64_t L,
                   int k, int chunk, float *__restrict__ vals_out, int32_t *__restrict__ idx_out,
                   int64_t out_ld, int out_slots)
{
    extern __shared__ __attribute__((aligned(16))) uint32_t keys[];
    __shared__ int hist[2048];
    __shared__ __attribute__((aligned(16))) uint32_t cand[kCand];
    __shared__ int wsum[2 * NW];
    __shared__ int sel[2];
    __shared__ int ncand;

    const int tid = threadIdx.x;
    const int64_t t = blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * chunk;
    const int n = (int)((L - c0 < chunk) ? (L - c0) : chunk);
    const float *vrow = vals_in + t * L + c0;
    const int32_t *irow = idx_in ? idx_in + t * L + c0 : nullptr;
    float *vo = vals_out ? vals_out + t * out_ld + (int64_t)blockIdx.x * out_slots : nullptr;
    int32_t *io = idx_out + t * out_ld + (int64_t)blockIdx.x * out_slots;

    // 1. keys into LDS (8 independent loads in flight per thread), count selectable ones
    int nvalid = 0;
    for (int base = 0; base < n; base += 8 * NT) {
        float x[8];
        int32_t ix[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int p = base + u * NT + tid;
            x[u] = (p < n) ? vrow[p] : -INFINITY;
            ix[u] = (irow != nullptr && p < n) ? irow[p] : 0;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int p = base + u * NT + tid;
            if (p < n) {
                const uint32_t key = (ix[u] < 0) ? 0u : order_key(x[u]);
                keys[p] = key;
                nvalid += key != 0u;
            }
        }
    }
    int total;
    block_excl_scan(nvalid, wsum, total);
    const int keff = total < k ? total : k;

    // 2. radix select: digits of 11, 11 and 10 bits from the top. tau = key of the keff-th
    //    largest, need_eq = how many keys equal to tau are kept (the lowest positions).
    uint32_t prefix = 0u, pmask = 0u;
    int kr = keff;
    if (keff > 0) {
        const int shifts[3] = {21, 10, 0};
        const int widths[3] = {11, 11, 10};
        const uint32_t *src = keys;
        int nsrc = n;
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = shifts[pass], nbins = 1 << widths[pass];
            const uint32_t dmask = (uint32_t)nbins - 1u;
            for (int i = tid; i < nbins; i += NT) hist[i] = 0;
            __syncthreads();
            digit_hist(src, nsrc, prefix, pmask, shift, dmask, hist);
            __syncthreads();
            pick_digit(hist, nbins, kr, wsum, sel);
            const int d = sel[0];
            kr = sel[1];
            prefix |= (uint32_t)d << shift;
            pmask |= dmask << shift;
            // after the first digit, keep only the keys of the chosen bin (when they fit),
            // so the later passes scan a short list
            if (pass == 0 && hist[d] <= kCand) {
                if (tid == 0) ncand = 0;
                __syncthreads();
                for (int p = tid; p < n; p += NT) {
                    const uint32_t key = keys[p];
                    if (key != 0u && (key & pmask) == prefix) cand[atomicAdd(&ncand, 1)] = key;
                }
                __syncthreads();
                src = cand;
                nsrc = ncand;
            }
            __syncthreads();
        }
    }
    const uint32_t tau = prefix;
    const int need_eq = kr;

    // 3. ordered compaction over contiguous per-thread segments (4 keys per LDS read)
    const int seg = (((n + NT - 1) / NT) + 3) & ~3;
    const int p0 = tid * seg;
    const int p1 = (p0 + seg < n) ? p0 + seg : n;
    int cgt = 0, ceq = 0;
    if (keff > 0)
        for (int p = p0; p < p1; p += 4) {
            const uint4 q4 = *reinterpret_cast<const uint4 *>(keys + p);
            const uint32_t kk[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (p + u < p1) {
                    cgt += kk[u] > tau;
                    ceq += kk[u] == tau;
                }
        }
    const int eq_before = block_excl_scan(ceq, wsum, total);
    int take_eq = need_eq - eq_before;
    take_eq = take_eq < 0 ? 0 : (take_eq > ceq ? ceq : take_eq);
    int pos = block_excl_scan(cgt + take_eq, wsum, total);
    if (keff > 0)
        for (int p = p0; p < p1; p += 4) {
            const uint4 q4 = *reinterpret_cast<const uint4 *>(keys + p);
            const uint32_t kk[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (p + u >= p1) break;
                bool take = kk[u] > tau;
                if (kk[u] == tau && take_eq > 0) {
                    take = true;
                    --take_eq;
                }
                if (take) {
                    io[pos] = irow ? irow[p + u] : (int32_t)(c0 + p + u);
                    if (vo) vo[pos] = vrow[p + u];
                    ++pos;
                }
            }
        }
    for (int j = keff + tid; j < out_slots; j += NT) {
        io[j] = -1;
        if (vo) vo[j] = -INFINITY;
    }
}

int g_cap = 0;

// largest power-of-two row chunk whose keys fit in LDS beside the static arrays
int topk_cap() {
    if (g_cap == 0) {
        int dev = 0, lds = 65536;
        if (hipGetDevice(&dev) == hipSuccess) {
            hipDeviceProp_t prop;
            if (hipGetDeviceProperties(&prop, dev) == hipSuccess) lds = (int)prop.sharedMemPerBlock;
        }
        const int fixed = 2048 * 4 + kCand * 4 + 1024;
        int cap = 32768;
        while (cap > 4096 && cap * 4 + fixed > lds) cap >>= 1;
        g_cap = cap;
    }
    return g_cap;
}

// first-level chunk of a row longer than the cap: about sqrt(N * k), so that the first
// level (one chunk per workgroup) and the second (nch * k survivors) are balanced
int first_chunk(int64_t N, int k, int cap) {
    int c = 4096;
    while (c < cap && (int64_t)c * c < N * (int64_t)k) c <<= 1;
    while (c < cap && ((N + c - 1) / c) * (int64_t)(k < c ? k : c) > cap) c <<= 1;
    return c;
}

}  // namespace

size_t topk_workspace_bytes(int T, int64_t N, int k) {
    const int cap = topk_cap();
    if (N <= cap) return 0;
    const int c1 = first_chunk(N, k, cap);
    const int64_t nch = (N + c1 - 1) / c1;
    const int64_t slots = k < c1 ? k : c1;
    // two ping-pong buffers of (value, index) pairs sized for the first reduction level
    return (size_t)2 * (size_t)T * (size_t)(nch * slots) * 8u;
}

int launch_topk(const float *scores, int T, int64_t N, int k, int32_t *idx, float *vals, void *ws,
                size_t ws_bytes, hipStream_t st) {
    if (T == 0) return CSA_OK;
    const int cap = topk_cap();
    const size_t need = topk_workspace_bytes(T, N, k);
    if (need > ws_bytes || (need > 0 && ws == nullptr))
        return fail(CSA_EWORKSPACE, "csa_topk: workspace smaller than csa_topk_workspace_bytes()");
    (void)hipFuncSetAttribute((const void *)topk_select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              cap * 4);
    const int64_t half = (int64_t)(need / 2);
    const float *vin = scores;
    const int32_t *iin = nullptr;
    int64_t L = N;
    int flip = 0;
    bool first = true;
    while (true) {
        if (L <= cap) {
            const size_t lds = (size_t)((L + 3) / 4 * 4 + 4) * 4;  // whole 16-byte groups for the vector reads
            hipLaunchKernelGGL(topk_select_kernel, dim3(1, T), dim3(NT), lds, st, vin, iin, L, k, cap, vals, idx,
                               (int64_t)k, k);
            return check_launch("topk_select_kernel");
        }
        const int chunk = first ? first_chunk(L, k, cap) : cap;
        const int64_t nch = (L + chunk - 1) / chunk;
        const int slots = k < chunk ? k : chunk;
        char *base = (char *)ws + (flip ? half : 0);
        float *vo = (float *)base;
        int32_t *io = (int32_t *)(base + (size_t)T * nch * slots * 4);
        hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)nch, T), dim3(NT), (size_t)chunk * 4, st, vin, iin,
                           L, k, chunk, vo, io, nch * slots, slots);
        int rc = check_launch("topk_select_kernel");
        if (rc != CSA_OK) return rc;
        vin = vo;
        iin = io;
        L = nch * slots;
        flip ^= 1;
        first = false;
    }
}

}  // namespace csa
