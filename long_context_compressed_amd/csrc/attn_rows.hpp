// Row slots of one attention query, shared by the attention kernels.
//
// Slots [0, nmain) are the compressed rows (the query's top-k indices in sparse mode, or
// summaries 0..nvis-1 in dense mode); slots [nmain, nslots) are the SWA positions
// max(0, t-window+1)..t. A slot whose row the caller does not hold has no pointer.
#pragma once

#include "common.hpp"

namespace csa {

struct RowCtx {
    int64_t nmain;    // main slots
    int64_t nslots;   // main + window slots
    int64_t lo;       // first SWA position
    int s;
    int64_t pos;
    int64_t swa0;     // position held by SWA row 0 of the query's sequence
};

__device__ __forceinline__ RowCtx row_ctx(int t, const int32_t *q_seq, const int64_t *q_pos, int B,
                                          int64_t N, int k, int ratio, const void *swa,
                                          const int64_t *swa_pos0, int window) {
    RowCtx c;
    c.s = q_seq[t];
    c.pos = q_pos[t];
    c.swa0 = 0;
    if (c.s < 0 || c.s >= B || c.pos < 0) {
        c.nmain = c.nslots = 0;
        c.lo = 0;
        return c;
    }
    if (swa != nullptr) c.swa0 = swa_pos0[c.s];
    if (ratio > 0) {
        int64_t nv = c.pos / ratio;
        c.nmain = nv < N ? nv : N;
    } else {
        c.nmain = k;
    }
    c.lo = c.pos - window + 1;
    if (c.lo < 0) c.lo = 0;
    const int64_t nwin = (swa != nullptr && window > 0) ? (c.pos - c.lo + 1) : 0;
    c.nslots = c.nmain + nwin;
    return c;
}

template <typename ET>
__device__ __forceinline__ const ET *row_ptr(const RowCtx &c, int64_t j, int t, const ET *kv,
                                            const int32_t *idx, int k, int ratio, int64_t N,
                                            const ET *swa, const int64_t *swa_pos0, int swa_rows, int D) {
    if (j < 0 || j >= c.nslots) return nullptr;
    if (j < c.nmain) {
        int64_t id = j;
        if (ratio <= 0) {
            id = idx[(int64_t)t * k + j];
            if (id < 0 || id >= N) return nullptr;
        }
        return kv + ((int64_t)c.s * N + id) * D;
    }
    const int64_t x = c.lo + (j - c.nmain);
    const int64_t r = x - c.swa0;
    if (r < 0 || r >= swa_rows) return nullptr;
    return swa + ((int64_t)c.s * swa_rows + r) * D;
}

}  // namespace csa
