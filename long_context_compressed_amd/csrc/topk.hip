// Per-query top-k over index scores on gfx950 ("DeepSeek-V4 混合注意力" §4.2: each
// query keeps the k = 512 / 1,024 highest-scoring compressed entries).
//
// A workgroup (1024 lanes) owns one chunk of at most `cap` scores of one row and keeps
// it in LDS as order-preserving 32-bit keys (-inf / NaN map to 0 and are never taken):
//   1. four 8-bit radix passes over LDS find the exact key tau of the k-th largest
//      element and how many elements equal to tau are to be taken (ties go to the lower
//      index); histogram increments are aggregated per wavefront for the common case
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

// vals_in/idx_in: rows of length L (row stride L); idx_in == nullptr means the index of
// position p is the position itself. Output slots [t][chunk*out_slots ...], row stride
// out_ld; exactly min(k, #valid) pairs are written in index order, the rest padded.
__global__ void __launch_bounds__(NT)
topk_select_kernel(const float *__restrict__ vals_in, const int32_t *__restrict__ idx_in, int64_t L,
                   int k, int cap, float *__restrict__ vals_out, int32_t *__restrict__ idx_out,
                   int64_t out_ld, int out_slots)
{
    extern __shared__ uint32_t keys[];
    __shared__ int hist[256];
    __shared__ int wsum[2 * NW];
    __shared__ int sel[2];

    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t t = blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * cap;
    const int n = (int)((L - c0 < cap) ? (L - c0) : cap);
    const float *vrow = vals_in + t * L + c0;
    const int32_t *irow = idx_in ? idx_in + t * L + c0 : nullptr;
    float *vo = vals_out ? vals_out + t * out_ld + (int64_t)blockIdx.x * out_slots : nullptr;
    int32_t *io = idx_out + t * out_ld + (int64_t)blockIdx.x * out_slots;

    // 1. keys into LDS, count the selectable ones
    int nvalid = 0;
    for (int p = tid; p < n; p += NT) {
        uint32_t key = order_key(vrow[p]);
        if (irow && irow[p] < 0) key = 0u;
        keys[p] = key;
        nvalid += key != 0u;
    }
    int total;
    block_excl_scan(nvalid, wsum, total);
    const int keff = total < k ? total : k;

    // 2. radix passes: tau = key of the keff-th largest, need = how many == tau to take
    uint32_t prefix = 0u, pmask = 0u;
    int kr = keff;
    if (keff > 0) {
        for (int shift = 24; shift >= 0; shift -= 8) {
            if (tid < 256) hist[tid] = 0;
            __syncthreads();
            for (int base = 0; base < n; base += NT) {
                const int p = base + tid;
                const uint32_t key = (p < n) ? keys[p] : 0u;
                const bool act = key != 0u && (key & pmask) == prefix;
                const int d = (int)((key >> shift) & 255u);
                const uint64_t am = __ballot(act);
                if (am) {
                    const int lead = __ffsll((unsigned long long)am) - 1;
                    const int dl = __shfl(d, lead);
                    const uint64_t same = __ballot(act && d == dl);
                    if (lane == lead) atomicAdd(&hist[dl], (int)__popcll(same));
                    if (act && d != dl) atomicAdd(&hist[d], 1);
                }
            }
            __syncthreads();
            // suffix sums from the top digit down: thread r < 256 holds digit 255 - r
            int h = 0, x = 0;
            if (tid < 256) {
                h = hist[255 - tid];
                x = h;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int y = __shfl_up(x, o);
                    if (lane >= o) x += y;
                }
                if (lane == 63) wsum[tid >> 6] = x;
            }
            __syncthreads();
            if (tid < 256) {
                int off = 0;
                for (int w2 = 0; w2 < (tid >> 6); ++w2) off += wsum[w2];
                const int incl = x + off;  // elements whose digit is >= 255 - tid
                const int excl = incl - h; // elements whose digit is >  255 - tid
                if (incl >= kr && excl < kr) {
                    sel[0] = 255 - tid;
                    sel[1] = kr - excl;
                }
            }
            __syncthreads();
            prefix |= (uint32_t)sel[0] << shift;
            pmask |= 255u << shift;
            kr = sel[1];
            __syncthreads();
        }
    }
    const uint32_t tau = prefix;
    const int need_eq = kr;

    // 3. ordered compaction over contiguous per-thread segments
    const int seg = (n + NT - 1) / NT;
    const int p0 = tid * seg;
    const int p1 = (p0 + seg < n) ? p0 + seg : n;
    int cgt = 0, ceq = 0;
    if (keff > 0)
        for (int p = p0; p < p1; ++p) {
            const uint32_t key = keys[p];
            cgt += key > tau;
            ceq += key == tau;
        }
    const int eq_before = block_excl_scan(ceq, wsum, total);
    int take_eq = need_eq - eq_before;
    take_eq = take_eq < 0 ? 0 : (take_eq > ceq ? ceq : take_eq);
    int pos = block_excl_scan(cgt + take_eq, wsum, total);
    if (keff > 0)
        for (int p = p0; p < p1; ++p) {
            const uint32_t key = keys[p];
            bool take = key > tau;
            if (key == tau && take_eq > 0) {
                take = true;
                --take_eq;
            }
            if (take) {
                io[pos] = irow ? irow[p] : (int32_t)(c0 + p);
                if (vo) vo[pos] = vrow[p];
                ++pos;
            }
        }
    for (int j = keff + tid; j < out_slots; j += NT) {
        io[j] = -1;
        if (vo) vo[j] = -INFINITY;
    }
}

int g_cap = 0;

int topk_cap() {
    if (g_cap == 0) {
        int dev = 0, lds = 65536;
        if (hipGetDevice(&dev) == hipSuccess) {
            hipDeviceProp_t prop;
            if (hipGetDeviceProperties(&prop, dev) == hipSuccess) lds = (int)prop.sharedMemPerBlock;
        }
        int cap = 32768;
        while (cap > 4096 && cap * 4 + 4096 > lds) cap >>= 1;
        g_cap = cap;
    }
    return g_cap;
}

}  // namespace

size_t topk_workspace_bytes(int T, int64_t N, int k) {
    const int cap = topk_cap();
    if (N <= cap) return 0;
    const int64_t nch = (N + cap - 1) / cap;
    const int64_t slots = k < cap ? k : cap;
    // two ping-pong buffers of (value, index) pairs for the first reduction level
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
    while (true) {
        const int64_t nch = L > 0 ? (L + cap - 1) / cap : 1;
        const size_t lds = (size_t)(L < cap ? (L > 0 ? L : 1) : cap) * 4;
        if (nch == 1) {
            hipLaunchKernelGGL(topk_select_kernel, dim3(1, T), dim3(NT), lds, st, vin, iin, L, k, cap,
                               vals, idx, (int64_t)k, k);
            return check_launch("topk_select_kernel");
        }
        const int slots = k < cap ? k : cap;
        char *base = (char *)ws + (flip ? half : 0);
        float *vo = (float *)base;
        int32_t *io = (int32_t *)(base + (size_t)T * nch * slots * 4);
        hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)nch, T), dim3(NT), lds, st, vin, iin, L, k,
                           cap, vo, io, nch * slots, slots);
        int rc = check_launch("topk_select_kernel");
        if (rc != CSA_OK) return rc;
        vin = vo;
        iin = io;
        L = nch * slots;
        flip ^= 1;
    }
}

}  // namespace csa
