// Exact top-k selection of one chunk held in registers, shared by the top-k kernel and the
// fused index-scan + top-k kernel ("DeepSeek-V4 混合注意力" §4.2: each query keeps the k
// highest-scoring compressed entries).
//
// A workgroup of RT lanes holds up to RT * J order-preserving 32-bit keys (-inf / NaN map to
// 0 and are never taken): lane `tid` holds the keys of positions j * RT + tid, j < J.
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
#pragma once

#include "common.hpp"

namespace csa {
namespace tksel {

constexpr int kList = 4096;      // LDS list of the keys that share the k-th key's leading digit
constexpr int kHistBins = 2048;  // bins of the widest digit; 64 words past them absorb idle adds

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

// inclusive scan over the 64 lanes of a wavefront with DPP moves: shifts of 1, 2, 4 and 8
// within each row of 16 lanes (a lane whose source falls outside the row adds 0), then
// lane 15 of rows 0 and 2 into rows 1 and 3, then lane 31 into rows 2 and 3
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
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

// Buffer resource over n 4-byte elements at p (a read at byte offset >= 4n returns 0;
// the bounds check covers the per-lane offset operand only, so callers pass the whole
// offset there).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void *p, int n) {
    const uint64_t a = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), 0, 4 * n, 0x00020000);
}

// Histogram increment of one key per lane (act: the key takes part, d: its digit).
// Increments of the lanes of a wavefront that share the first active lane's digit are
// merged into one (scores concentrate in a few leading-digit bins). Branch-free, so the
// compiler can interleave the keys of a lane: every lane issues one LDS add, and lanes
// with nothing to add (inactive, or merged into the leading lane's add) target a private
// word past the bins.
__device__ __forceinline__ void hist_add(bool act, int d, int *hist) {
    const int lane = threadIdx.x & 63;
    const uint64_t am = __ballot(act);
    const int lead = am ? __ffsll((unsigned long long)am) - 1 : 0;
    const int dl = __builtin_amdgcn_readlane(d, lead);
    const bool merged = act && d == dl;
    const uint64_t same = __ballot(merged);
    const bool own = act && !merged;
    const bool head = merged && lane == lead;
    const int addr = (own || head) ? (head ? dl : d) : kHistBins + lane;
    atomicAdd(&hist[addr], head ? (int)__popcll(same) : 1);
}

// Given the histogram of nbins digits (complete: the caller has synchronized) and kr (how
// many of the counted keys to keep, from the top), returns the digit holding the kr-th
// largest, sets kr to how many keys of that digit are still to be kept and bin to that
// digit's count. hist is zero again on return.
template <int RT>
__device__ __forceinline__ uint32_t pick_digit(int nbins, int &kr, int &bin, int *hist, int *ws, int *sel) {
    const int tid = threadIdx.x;
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
                sel[2] = h[i];
            }
            above += h[i];
        }
    }
    __syncthreads();
    kr = sel[1];
    bin = sel[2];
    return (uint32_t)sel[0];
}

// v[l] = x for one lane l (x and l wavefront-uniform)
__device__ __forceinline__ void lane_put(int &v, int x, int l) {
    asm("v_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(x), "i"(l));
}

template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};

// wavefront-exclusive count of the set bits of m below this lane
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}


// LDS of one selection (about 27 KB)
template <int RT, int J>
struct SelectLds {
    static constexpr int RW = RT / 64;
    __attribute__((aligned(16))) int hist[kHistBins + 64];
    int ws[7][RW];
    int sel[3];
    uint32_t list[kList];       // keys of the leading bin; later the staged output
    int cgt[J * RW], ceq[J * RW];  // per (slot, wavefront), in position order
};

// Clears the histogram of `sm` for select_chunk (after a barrier, so a previous selection
// with the same LDS has finished reading it).
template <int RT, int J>
__device__ __forceinline__ void select_begin(SelectLds<RT, J> &sm) {
    __syncthreads();
    for (int i = threadIdx.x; i < 2048; i += RT) sm.hist[i] = 0;
}

// Selects the min(k, #selectable) largest of the n keys (positions >= n must hold key 0)
// and writes them in ascending position order to io (index) and vo (value, when not
// null), padding the out_slots - keff slots after them with (-1, -inf). The index of
// position p is irow[p] (read from global memory) or, with irow null, c0 + p. Every
// thread of the workgroup calls it, after select_begin() on the same `sm` (which may
// come before the keys are loaded); the LDS of `sm` may be reused once it returns.
template <int RT, int J>
__device__ __forceinline__ void select_chunk(uint32_t (&key)[J], int n, int k, const int32_t *irow, int64_t c0,
                                             float *vo, int32_t *io, int out_slots, SelectLds<RT, J> &sm)
{
    constexpr int RW = RT / 64;
    int *const hist = sm.hist;
    auto &ws = sm.ws;
    int *const sel = sm.sel;
    uint32_t *const list = sm.list;
    int *const cgt = sm.cgt;
    int *const ceq = sm.ceq;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int nvalid = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) nvalid += key[j] != 0u;
    int total;
    block_excl_scan<RT>(nvalid, ws[0], total);
    const int keff = total < k ? total : k;

    if (keff > 0) {
        // 2. radix select: tau = key of the keff-th largest, need_eq = how many keys equal
        //    to tau are kept (the lowest positions). Zero keys (not selectable) are not
        //    filtered out: every selectable key is at least order_key(-FLT_MAX) =
        //    0x00800000, so in the first pass they only fill bin 0, which is never picked
        //    (kr <= #selectable), and the later prefixes exclude them.
        int kr = keff, bin;
#pragma unroll
        for (int j = 0; j < J; ++j) hist_add(true, (int)(key[j] >> 21), hist);
        __syncthreads();
        const uint32_t d0 = pick_digit<RT>(2048, kr, bin, hist, ws[1], sel);
        uint32_t prefix = d0 << 21;
        if (bin <= kList) {
            // the leading bin's keys fit the LDS list: the later passes read only those.
            // Each lane counts its keys of the bin; a scan of the counts gives every lane
            // its own range of the list (no atomics). The two sweeps compare with opaque
            // copies of the prefix, so the compiler keeps no per-key result between them.
            const uint32_t pa = fresh(prefix), pb = fresh(prefix);
            int mine = 0;
#pragma unroll
            for (int j = 0; j < J; ++j) mine += (key[j] ^ pa) < 0x00200000u;
            int off = wave_incl_scan(mine);
            if (lane == 63) ws[6][wv] = off;
            off -= mine;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < RW; ++i) off += (i < wv) ? ws[6][i] : 0;
#pragma unroll
            for (int j = 0; j < J; ++j)
                if ((key[j] ^ pb) < 0x00200000u) list[off++] = key[j];
            __syncthreads();
            const int nl = bin;  // list length
            for (int i = tid; i < nl; i += RT) hist_add(true, (int)((list[i] >> 10) & 2047u), hist);
            __syncthreads();
            prefix |= pick_digit<RT>(2048, kr, bin, hist, ws[2], sel) << 10;
            for (int i = tid; i < nl; i += RT) {
                const uint32_t kk = list[i];
                hist_add((kk & 0xfffffc00u) == prefix, (int)(kk & 1023u), hist);
            }
            __syncthreads();
            prefix |= pick_digit<RT>(1024, kr, bin, hist, ws[3], sel);
        } else {
            const uint32_t p1 = fresh(prefix);  // (keeps the compares of the two branches apart)
#pragma unroll
            for (int j = 0; j < J; ++j) hist_add((key[j] & 0xffe00000u) == p1, (int)((key[j] >> 10) & 2047u), hist);
            __syncthreads();
            prefix |= pick_digit<RT>(2048, kr, bin, hist, ws[2], sel) << 10;
#pragma unroll
            for (int j = 0; j < J; ++j) hist_add((key[j] & 0xfffffc00u) == prefix, (int)(key[j] & 1023u), hist);
            __syncthreads();
            prefix |= pick_digit<RT>(1024, kr, bin, hist, ws[3], sel);
        }
        const uint32_t tau = prefix;
        const int need_eq = kr;  // of the `bin` keys equal to tau

        // 3-4. Output. When every key equal to tau is taken (the usual case) the selected
        //    keys are those >= tau; otherwise keys above tau and the first need_eq keys
        //    equal to it, counted separately.
        auto emit = [&](auto split_tag) __attribute__((always_inline)) {
            constexpr bool kSplit = decltype(split_tag)::value;
            // 3. counts per (slot, wavefront), gathered into lane j % 64 of (g|e)(A|B),
            //    then scanned in position order (slot-major, then wavefront)
            const uint32_t tau3 = fresh(tau);
            int gA = 0, gB = 0, eA = 0, eB = 0;
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int a = (int)__popcll(__ballot(kSplit ? key[j] > tau3 : key[j] >= tau3));
                if (j < 64) lane_put(gA, a, j);
                else lane_put(gB, a, j - 64);
                if (kSplit) {
                    const int e = (int)__popcll(__ballot(key[j] == tau3));
                    if (j < 64) lane_put(eA, e, j);
                    else lane_put(eB, e, j - 64);
                }
            }
            if (lane < J) {
                cgt[lane * RW + wv] = gA;
                if (kSplit) ceq[lane * RW + wv] = eA;
            }
            if (lane + 64 < J) {
                cgt[(lane + 64) * RW + wv] = gB;
                if (kSplit) ceq[(lane + 64) * RW + wv] = eB;
            }
            __syncthreads();
            {
                constexpr int EPT = (J * RW + RT - 1) / RT;  // entries per lane
                int ca[EPT], ce[EPT], sa = 0, se = 0;
#pragma unroll
                for (int i = 0; i < EPT; ++i) {
                    const int x = EPT * tid + i;
                    ca[i] = x < J * RW ? cgt[x] : 0;
                    ce[i] = (kSplit && x < J * RW) ? ceq[x] : 0;
                    sa += ca[i];
                    se += ce[i];
                }
                int ta, te;
                int pa = block_excl_scan<RT>(sa, ws[4], ta);
                int pe = kSplit ? block_excl_scan<RT>(se, ws[5], te) : 0;
#pragma unroll
                for (int i = 0; i < EPT; ++i) {
                    const int x = EPT * tid + i;
                    if (x < J * RW) {
                        cgt[x] = pa;
                        if (kSplit) ceq[x] = pe;
                    }
                    pa += ca[i];
                    pe += ce[i];
                }
            }
            __syncthreads();
            gA = lane < J ? cgt[lane * RW + wv] : 0;
            gB = lane + 64 < J ? cgt[(lane + 64) * RW + wv] : 0;
            if (kSplit) {
                eA = lane < J ? ceq[lane * RW + wv] : 0;
                eB = lane + 64 < J ? ceq[(lane + 64) * RW + wv] : 0;
            }
            // 4. ordered output: the taken keys of a slot are consecutive output slots.
            //    Unstaged (k > 2,048), they are written with bounded buffer stores (a
            //    missing value output is a zero-length resource, whose stores are
            //    dropped); with input indices, the index reads of 8 slots are issued before
            //    their stores (a store waits for every older read and store of the
            //    wavefront).
            const __amdgpu_buffer_rsrc_t rso = chunk_rsrc(io, out_slots);
            const __amdgpu_buffer_rsrc_t rsv = chunk_rsrc(vo, vo ? out_slots : 0);
            const uint32_t tau4 = fresh(tau);
            const int tid4 = fresh(tid);  // positions recomputed here, not kept live from step 1
            auto slot = [&](int j, int &pos) __attribute__((always_inline)) -> bool {
                if (!kSplit) {
                    const bool ge = key[j] >= tau4;
                    const uint64_t bg = __ballot(ge);
                    if (bg == 0ull) return false;
                    pos = __builtin_amdgcn_readlane(j < 64 ? gA : gB, j & 63) + lanes_below(bg);
                    return ge;
                }
                const bool gt = key[j] > tau4, eq = key[j] == tau4;
                const uint64_t bg = __ballot(gt), be = __ballot(eq);
                if ((bg | be) == 0ull) return false;
                const int gtb = __builtin_amdgcn_readlane(j < 64 ? gA : gB, j & 63) + lanes_below(bg);
                const int eqb = __builtin_amdgcn_readlane(j < 64 ? eA : eB, j & 63) + lanes_below(be);
                pos = gtb + (eqb < need_eq ? eqb : need_eq);
                return gt || (eq && eqb < need_eq);
            };
            auto put = [&](int pos, uint32_t ix, uint32_t kk) __attribute__((always_inline)) {
                __builtin_amdgcn_raw_buffer_store_b32(ix, rso, 4 * pos, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(key_value(kk)), rsv, 4 * pos, 0, 0);
            };
            if (keff <= kList / 2) {
                // staged: (position, key) of every taken key into the LDS list (idle since
                // the last radix pass), then written out in order with coalesced stores
                uint32_t *sp = list, *sk = list + kList / 2;
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    int pos;
                    if (slot(j, pos)) {
                        sp[pos] = (uint32_t)(j * RT + tid4);
                        sk[pos] = key[j];
                    }
                }
                __syncthreads();
                for (int i0 = 0; i0 < keff; i0 += 4 * RT) {
                    int ix[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int i = i0 + u * RT + tid;
                        const int p = i < keff ? (int)sp[i] : 0;
                        ix[u] = irow ? irow[p] : (int)(c0 + p);
                    }
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int i = i0 + u * RT + tid;
                        if (i < keff) {
                            io[i] = ix[u];
                            if (vo) vo[i] = key_value(sk[i]);
                        }
                    }
                }
            } else if (irow == nullptr) {
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    int pos;
                    if (slot(j, pos)) put(pos, (uint32_t)(c0 + j * RT + tid4), key[j]);
                }
            } else {
                const __amdgpu_buffer_rsrc_t rsi = chunk_rsrc(irow, n);
#pragma unroll
                for (int j0 = 0; j0 < J; j0 += 8) {
                    int pos[8];
                    uint32_t ix[8];
                    bool take[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        // unconditional (bounded) reads, so their waits stay exact
                        ix[u] = j0 + u < J
                                    ? __builtin_amdgcn_raw_buffer_load_b32(rsi, fresh(4 * ((j0 + u) * RT + tid4)), 0, 0)
                                    : 0u;
                        take[u] = j0 + u < J && slot(j0 + u, pos[u]);
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        if (take[u]) put(pos[u], ix[u], key[j0 + u]);
                }
            }
        };
        if (need_eq == bin)
            emit(BoolTag<false>{});
        else
            emit(BoolTag<true>{});
    }
    for (int i = keff + tid; i < out_slots; i += RT) {
        io[i] = -1;
        if (vo) vo[i] = -INFINITY;
    }
}

}  // namespace tksel
}  // namespace csa
