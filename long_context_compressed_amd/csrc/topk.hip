// Per-query top-k over index scores on gfx950 ("DeepSeek-V4 混合注意力" §4.2: each
// query keeps the k = 512 / 1,024 highest-scoring compressed entries).
//
// A workgroup (256 lanes, four wavefronts) owns one chunk of at most 256 * J scores of
// one row and keeps it in registers as order-preserving 32-bit keys (-inf / NaN map to 0
// and are never taken): lane `tid` holds the keys of positions j * 256 + tid, j < J, read
// with coalesced 4-byte loads. The LDS footprint is small (a 2,048-bin histogram and a
// few counters), so several workgroups share a compute unit and the barriers of one hide
// behind the arithmetic of the others.
//   1. three radix passes (digits of 11, 11 and 10 bits from the top) over the register
//      keys find the exact key tau of the k-th largest element and how many elements
//      equal to tau are to be taken (ties go to the lower index); histogram increments of
//      the lanes of a wavefront that share the first active lane's digit are merged into
//      one LDS atomic;
//   2. per (slot j, wavefront) counts of keys above and equal to tau, scanned in position
//      order, give every selected key its output slot, so the (value, index) pairs are
//      written in ascending index order. The value is recovered from the key.
// Rows longer than the chunk cap are cut into chunks; the exact top-k of the row is a
// subset of the union of the chunks' top-k sets, so the chunk winners (kept in index
// order, padded with (-inf, -1)) form a shorter row that the same kernel reduces again
// until one chunk remains.
#include "common.hpp"
#include "internal.hpp"

namespace csa {

namespace {

constexpr int kCap = 32768;  // longest chunk: 128 key registers per lane at 256 lanes

__device__ __forceinline__ uint32_t order_key(float s) {
    if (!(s > -INFINITY)) return 0u;
    const uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// An opaque copy: the compiler cannot prove it equal to the source, so comparisons made
// with it are not merged with (and kept live from) earlier ones.
template <typename T>
__device__ __forceinline__ T fresh(T v) {
    asm volatile("" : "+v"(v));
    return v;
}

__device__ __forceinline__ int wave_incl_scan(int x) {
    const int lane = fresh((int)(threadIdx.x & 63));
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    return x;
}

// exclusive scan of one int per lane over a workgroup of RT lanes; ws (RT / 64 ints) must
// not be read by a scan still in progress
template <int RT>
__device__ __forceinline__ int block_excl_scan(int v, int *ws, int &total) {
    constexpr int RW = RT / 64;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int x = wave_incl_scan(v);
    if (lane == 63) ws[wv] = x;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const int s = ws[i];
        before += (i < wv) ? s : 0;
        total += s;
    }
    return before + x - v;
}

// One radix pass: histogram of digit (key >> shift) & dmask over the active keys (bits
// above the digit equal to prefix under pmask), then the digit holding the kr-th largest
// active key; returns it and sets kr to how many keys of that digit are still to be kept.
// hist is zero on entry and is zero again on return. Zero keys (not selectable) are not
// filtered out: every selectable key is at least order_key(-FLT_MAX) = 0x00800000, so in
// the first pass they only fill bin 0, which is never picked (kr <= #selectable), and the
// later passes' prefixes exclude them.
template <int RT, int J>
__device__ __forceinline__ uint32_t radix_pass(const uint32_t (&key)[J], uint32_t prefix, uint32_t pmask, int shift,
                                               int nbins, int &kr, int *hist, int *ws, int *sel) {
    const int tid = threadIdx.x, lane = tid & 63;
    const uint32_t dmask = (uint32_t)nbins - 1u;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const uint32_t kk = key[j];
        const bool act = (kk & pmask) == prefix;
        const int d = (int)((kk >> shift) & dmask);
        const uint64_t am = __ballot(act);
        if (am) {
            const int lead = __ffsll((unsigned long long)am) - 1;
            const int dl = __builtin_amdgcn_readlane(d, lead);
            const uint64_t same = __ballot(act && d == dl);
            if (lane == lead) atomicAdd(&hist[dl], (int)__popcll(same));
            if (act && d != dl) atomicAdd(&hist[d], 1);
        }
    }
    __syncthreads();
    // bins per lane, top first: lane tid owns [nbins - bpt * (tid + 1), nbins - bpt * tid)
    const int bpt = nbins / RT;
    const int lo = nbins - bpt * (tid + 1);
    constexpr int kMaxBpt = 2048 / RT;
    int h[kMaxBpt], sum = 0;
#pragma unroll
    for (int i = 0; i < kMaxBpt; ++i) {
        h[i] = i < bpt ? hist[lo + i] : 0;
        sum += h[i];
    }
    int total;
    int above = block_excl_scan<RT>(sum, ws, total);
    // every lane has read its bins (the scan holds a barrier): clear them for the next pass
#pragma unroll
    for (int i = 0; i < kMaxBpt; ++i)
        if (i < bpt) hist[lo + i] = 0;
#pragma unroll
    for (int i = kMaxBpt - 1; i >= 0; --i) {  // bins lo + i, from the top
        if (i < bpt) {
            if (above < kr && above + h[i] >= kr) {
                sel[0] = lo + i;
                sel[1] = kr - above;
            }
            above += h[i];
        }
    }
    __syncthreads();
    kr = sel[1];
    return (uint32_t)sel[0];
}

// vals_in/idx_in: rows of length L (row stride L); idx_in == nullptr means the index of
// position p is the position itself, otherwise an entry with value -inf is padding. The
// chunk of this workgroup is positions [blockIdx.x * chunk, +chunk) of row blockIdx.y
// (chunk <= 256 * J). Output slots [t][blockIdx.x * out_slots ...], row stride out_ld;
// exactly min(k, #valid) pairs are written in index order, the rest padded.
template <int RT, int J>
__global__ void __launch_bounds__(RT)
topk_select_kernel(const float *__restrict__ vals_in, const int32_t *__restrict__ idx_in, int64_t L,
                   int k, int chunk, float *__restrict__ vals_out, int32_t *__restrict__ idx_out,
                   int64_t out_ld, int out_slots)
{
    constexpr int RW = RT / 64;
    __shared__ __attribute__((aligned(16))) int hist[2048];
    __shared__ int ws[6][RW];
    __shared__ int sel[2];
    __shared__ int cgt[J * RW], ceq[J * RW];  // per (slot, wavefront), in position order

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t t = blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * chunk;
    const int n = (int)((L - c0 < chunk) ? (L - c0) : chunk);
    const float *vrow = vals_in + t * L + c0;
    const int32_t *irow = idx_in ? idx_in + t * L + c0 : nullptr;
    float *vo = vals_out ? vals_out + t * out_ld + (int64_t)blockIdx.x * out_slots : nullptr;
    int32_t *io = idx_out + t * out_ld + (int64_t)blockIdx.x * out_slots;

    for (int i = tid; i < 2048; i += RT) hist[i] = 0;

    // 1. keys into registers: buffer reads bounded to the chunk (a read past it returns 0,
    //    and its key is set to 0; the whole offset is in the per-lane operand, which is the
    //    part the bounds check covers)
    uint32_t key[J];
    int nvalid = 0;
    {
        const uint64_t a = (uint64_t)(uintptr_t)vrow;
        const uint32_t alo = __builtin_amdgcn_readfirstlane((uint32_t)a);
        const uint32_t ahi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(((uint64_t)ahi << 32) | alo), 0, 4 * n, 0x00020000);
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int p = j * RT + tid;
            const float x = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, 4 * p, 0, 0));
            key[j] = order_key(x) & (0u - (uint32_t)(p < n));
            nvalid += key[j] != 0u;
        }
    }
    int total;
    block_excl_scan<RT>(nvalid, ws[0], total);
    const int keff = total < k ? total : k;

    if (keff > 0) {
        // 2. radix select: tau = key of the keff-th largest, need_eq = how many keys equal
        //    to tau are kept (the lowest positions)
        int kr = keff;
        uint32_t prefix = radix_pass<RT, J>(key, 0u, 0u, 21, 2048, kr, hist, ws[1], sel) << 21;
        prefix |= radix_pass<RT, J>(key, prefix, 0xffe00000u, 10, 2048, kr, hist, ws[2], sel) << 10;
        prefix |= radix_pass<RT, J>(key, prefix, 0xfffffc00u, 0, 1024, kr, hist, ws[3], sel);
        const uint32_t tau = prefix;
        const int need_eq = kr;

        // 3. counts of keys above / equal to tau per (slot, wavefront), then their
        //    exclusive scan in position order (slot-major, then wavefront)
        const uint32_t tau3 = fresh(tau);
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int a = (int)__popcll(__ballot(key[j] > tau3));
            const int e = (int)__popcll(__ballot(key[j] == tau3));
            if (lane == 0) {
                cgt[j * RW + wv] = a;
                ceq[j * RW + wv] = e;
            }
        }
        __syncthreads();
        {
            constexpr int EPT = (J * RW + RT - 1) / RT;  // entries per lane
            int a[EPT], e[EPT], sa = 0, se = 0;
#pragma unroll
            for (int i = 0; i < EPT; ++i) {
                const int x = EPT * tid + i;
                a[i] = x < J * RW ? cgt[x] : 0;
                e[i] = x < J * RW ? ceq[x] : 0;
                sa += a[i];
                se += e[i];
            }
            int ta, te;
            int pa = block_excl_scan<RT>(sa, ws[4], ta);
            int pe = block_excl_scan<RT>(se, ws[5], te);
#pragma unroll
            for (int i = 0; i < EPT; ++i) {
                const int x = EPT * tid + i;
                if (x < J * RW) {
                    cgt[x] = pa;
                    ceq[x] = pe;
                }
                pa += a[i];
                pe += e[i];
            }
        }
        __syncthreads();
        // the wavefront's scanned counts of slot j sit in lane j % 64 of (g|e)(j < 64 ? A : B)
        const int gA = lane < J ? cgt[lane * RW + wv] : 0, eA = lane < J ? ceq[lane * RW + wv] : 0;
        const int gB = lane + 64 < J ? cgt[(lane + 64) * RW + wv] : 0;
        const int eB = lane + 64 < J ? ceq[(lane + 64) * RW + wv] : 0;
        // 4. ordered output: the taken keys of a slot are consecutive output slots
        const uint64_t lt = (1ull << lane) - 1ull;
        const uint32_t tau4 = fresh(tau);
        const int tid4 = fresh(tid);  // positions recomputed here, not kept live from step 1
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const bool gt = key[j] > tau4, eq = key[j] == tau4;
            const uint64_t bg = __ballot(gt), be = __ballot(eq);
            if ((bg | be) == 0ull) continue;
            const int gtb = __builtin_amdgcn_readlane(j < 64 ? gA : gB, j & 63) + (int)__popcll(bg & lt);
            const int eqb = __builtin_amdgcn_readlane(j < 64 ? eA : eB, j & 63) + (int)__popcll(be & lt);
            if (gt || (eq && eqb < need_eq)) {
                const int pos = gtb + (eqb < need_eq ? eqb : need_eq);
                const int p = j * RT + tid4;
                io[pos] = irow ? irow[p] : (int32_t)(c0 + p);
                if (vo) vo[pos] = key_value(key[j]);
            }
        }
    }
    for (int i = keff + tid; i < out_slots; i += RT) {
        io[i] = -1;
        if (vo) vo[i] = -INFINITY;
    }
}

int topk_cap() { return kCap; }

// first-level chunk of a row longer than the cap: about sqrt(N * k), so that the first
// level (one chunk per workgroup) and the second (nch * k survivors) are balanced
int first_chunk(int64_t N, int k, int cap) {
    int c = 4096;
    while (c < cap && (int64_t)c * c < N * (int64_t)k) c <<= 1;
    while (c < cap && ((N + c - 1) / c) * (int64_t)(k < c ? k : c) > cap) c <<= 1;
    return c;
}

// one launch of the select kernel over chunks of at most `chunk` positions, with the
// register tile sized to the longest chunk: 256-lane workgroups when the grid has enough
// of them to keep several on every compute unit, else 1,024-lane ones (sixteen
// wavefronts share a chunk's work)
int launch_select(const float *vin, const int32_t *iin, int64_t L, int k, int chunk, int64_t nch, int T, float *vo,
                  int32_t *io, int64_t out_ld, int out_slots, hipStream_t st) {
    const int64_t longest = L < chunk ? L : chunk;
    const dim3 grid((unsigned)nch, (unsigned)T);
#define CSA_TOPK_LAUNCH(RR, JJ)                                                                               \
    if (longest <= (RR) * (JJ)) {                                                                            \
        hipLaunchKernelGGL((topk_select_kernel<RR, JJ>), grid, dim3(RR), 0, st, vin, iin, L, k, chunk, vo, io,  \
                           out_ld, out_slots);                                                               \
        return check_launch("topk_select_kernel");                                                           \
    }
    if (nch * T >= 4 * (int64_t)device_cu_count()) {
        CSA_TOPK_LAUNCH(256, 16)
        CSA_TOPK_LAUNCH(256, 32)
        CSA_TOPK_LAUNCH(256, 48)
        CSA_TOPK_LAUNCH(256, 64)
        CSA_TOPK_LAUNCH(256, 72)
        CSA_TOPK_LAUNCH(256, 80)
        CSA_TOPK_LAUNCH(256, 96)
        CSA_TOPK_LAUNCH(256, 128)
    } else {
        CSA_TOPK_LAUNCH(1024, 4)
        CSA_TOPK_LAUNCH(1024, 8)
        CSA_TOPK_LAUNCH(1024, 16)
        CSA_TOPK_LAUNCH(1024, 24)
        CSA_TOPK_LAUNCH(1024, 32)
    }
#undef CSA_TOPK_LAUNCH
    return fail(CSA_EUNSUPPORTED, "csa_topk: chunk longer than the register tile");
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
    const int64_t half = (int64_t)(need / 2);
    const float *vin = scores;
    const int32_t *iin = nullptr;
    int64_t L = N;
    int flip = 0;
    bool first = true;
    while (true) {
        if (L <= cap) return launch_select(vin, iin, L, k, cap, 1, T, vals, idx, (int64_t)k, k, st);
        const int chunk = first ? first_chunk(L, k, cap) : cap;
        const int64_t nch = (L + chunk - 1) / chunk;
        const int slots = k < chunk ? k : chunk;
        char *base = (char *)ws + (flip ? half : 0);
        float *vo = (float *)base;
        int32_t *io = (int32_t *)(base + (size_t)T * nch * slots * 4);
        const int rc = launch_select(vin, iin, L, k, chunk, nch, T, vo, io, nch * slots, slots, st);
        if (rc != CSA_OK) return rc;
        vin = vo;
        iin = io;
        L = nch * slots;
        flip ^= 1;
        first = false;
    }
}

}  // namespace csa
