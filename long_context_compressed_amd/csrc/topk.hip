// Per-query top-k over index scores on gfx950 ("DeepSeek-V4 混合注意力" §4.2: each
// query keeps the k = 512 / 1,024 highest-scoring compressed entries).
//
// A workgroup (256 or 1,024 lanes) owns one chunk of at most RT * J scores of one row and
// keeps it in registers as order-preserving 32-bit keys (-inf / NaN map to 0 and are
// never taken): lane `tid` holds the keys of positions j * RT + tid, j < J, read with
// coalesced buffer loads bounded to the chunk. LDS holds only a histogram, a list and a
// few counters (about 27 KB), so 256-lane workgroups share a compute unit four at a time
// and the barriers of one hide behind the arithmetic of the others; grids too small for
// that use 1,024-lane workgroups (sixteen wavefronts on one chunk).
//   1. Radix select with digits of 11, 11 and 10 bits from the top finds the exact key
//      tau of the k-th largest element and how many elements equal to tau are taken
//      (ties go to the lower position). The first pass histograms every register key;
//      the keys of the chosen leading bin are then compacted into an LDS list (each lane
//      writes its own scanned range) and the two later passes read only that list (the
//      register keys again when the bin is larger than the list).
//   2. Output: per (slot j, wavefront) counts of the taken keys, scanned in position
//      order, give every taken key its output slot, so the (value, index) pairs come out
//      in ascending position order; the value is recovered from the key. The pairs are
//      staged in the LDS list and written with coalesced stores.
// Rows longer than the chunk cap are cut into chunks; the exact top-k of the row is a
// subset of the union of the chunks' top-k sets, so the chunk winners (kept in position
// order, padded with (-inf, -1)) form a shorter row that the same kernel reduces again
// until one chunk remains. A row may come with an id per position (a candidate list):
// the ids are what is written out.
#include <mutex>
#include <string>

#include "common.hpp"
#include "internal.hpp"
#include "topk_select.hpp"

namespace csa {

namespace {

using namespace tksel;

constexpr int kCap = 32768;  // longest chunk: 128 key registers per lane at 256 lanes

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
    __shared__ SelectLds<RT, J> sm;
    const int tid = threadIdx.x;
    const int64_t t = blockIdx.y;
    const int64_t c0 = (int64_t)blockIdx.x * chunk;
    const int n = (int)((L - c0 < chunk) ? (L - c0) : chunk);
    const float *vrow = vals_in + t * L + c0;
    const int32_t *irow = idx_in ? idx_in + t * L + c0 : nullptr;
    float *vo = vals_out ? vals_out + t * out_ld + (int64_t)blockIdx.x * out_slots : nullptr;
    int32_t *io = idx_out + t * out_ld + (int64_t)blockIdx.x * out_slots;
    select_begin(sm);

    // keys into registers: buffer reads bounded to the chunk (a read past it returns 0,
    // and its key is set to 0; the whole offset goes in the per-lane operand, which the
    // bounds check covers), all issued before the first is converted
    uint32_t key[J];
    {
        const __amdgpu_buffer_rsrc_t rs = chunk_rsrc(vrow, n);
#pragma unroll
        for (int j = 0; j < J; ++j) key[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, fresh(4 * (j * RT + tid)), 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < J; ++j) key[j] = order_key(__uint_as_float(key[j])) & (0u - (uint32_t)(j * RT + tid < n));
    }
    select_chunk<RT, J>(key, n, k, irow, c0, vo, io, out_slots, sm);
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
    // rows go on grid.y (at most 65,535): more rows go out in slices, offset by whole rows
    constexpr int kMaxGridY = 65535;
#define CSA_TOPK_LAUNCH(RR, JJ)                                                                               \
    if (longest <= (RR) * (JJ)) {                                                                            \
        for (int t0 = 0; t0 < T; t0 += kMaxGridY) {                                                          \
            const int tn = (T - t0 < kMaxGridY) ? T - t0 : kMaxGridY;                                        \
            hipLaunchKernelGGL((topk_select_kernel<RR, JJ>), dim3((unsigned)nch, (unsigned)tn), dim3(RR), 0, st, \
                               vin + (int64_t)t0 * L, iin ? iin + (int64_t)t0 * L : nullptr, L, k, chunk,   \
                               vo ? vo + (int64_t)t0 * out_ld : nullptr, io + (int64_t)t0 * out_ld, out_ld,  \
                               out_slots);                                                                   \
        }                                                                                                    \
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

int launch_topk(const float *scores, const int32_t *ids, int T, int64_t N, int k, int32_t *idx, float *vals,
                void *ws, size_t ws_bytes, hipStream_t st) {
    if (T == 0) return CSA_OK;
    const int cap = topk_cap();
    const size_t need = topk_workspace_bytes(T, N, k);
    if (need > ws_bytes || (need > 0 && ws == nullptr))
        return fail(CSA_EWORKSPACE, "csa_topk: workspace smaller than csa_topk_workspace_bytes()");
    const int64_t half = (int64_t)(need / 2);
    const float *vin = scores;
    const int32_t *iin = ids;
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

// ======================================================================================
// Allocation-free variant: the chunk winners of multi-level selection live in a
// file-scope device array instead of a caller workspace. Every device the library runs on
// holds its own copy of the array for the life of the process; its device address is
// looked up once per device (with that device current) and kept here.
// ======================================================================================
namespace csa {

constexpr size_t kTopkScratchBytes = size_t{16} << 20;
static __device__ __align__(256) uint8_t scratch[kTopkScratchBytes];

size_t topk_scratch_bytes() { return kTopkScratchBytes; }

int topk_scratch_ptr(void **ptr) {
    constexpr int kMaxDev = 64;
    static std::mutex mu;
    static void *cached[kMaxDev] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev)
        return fail(CSA_EHIP, "csa_topk_noalloc: no current HIP device (or device id >= 64)");
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] == nullptr) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(CSA_EHIP, std::string("csa_topk_noalloc: hipGetSymbolAddress(scratch): ") +
                                      hipGetErrorString(e));
        cached[dev] = p;
    }
    *ptr = cached[dev];
    return CSA_OK;
}

}  // namespace csa
