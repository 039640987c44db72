// Shared-KV MQA with an attention sink, 64 heads per workgroup, on gfx950 matrix cores.
//
// "DeepSeek-V4 混合注意力" §4.2 (one compressed vector is both K and V for every query head),
// §5 (HCA: every visible summary), §6 (SWA rows, sink softmax, partial RoPE / inverse RoPE).
//
// One workgroup = one query x 64 heads (x a range of row slots when split); wavefront w
// owns heads 16w..16w+15 over the full head dim D = 512. With 4 wavefronts (64 heads) two
// workgroups share a CU (256 registers and 78 KiB of LDS each), so one's softmax and
// barriers overlap the other's matrix and LDS work; with 8 (128 heads) a gathered row is
// fetched once for all heads of the query. Per 32-row tile:
//   - the rows (bf16, 1 KiB each) go from memory straight into LDS by buffer loads with
//     the LDS destination (one row per wave instruction, its address resolved in scalar
//     registers), into the other of two tile buffers while this tile is computed; rows are
//     padded to 1056 bytes so both read patterns below spread over the banks;
//   - S^T = K Q^T (rows x heads, MFMA 16x16x32 bf16): A = 16-byte row fragments from LDS,
//     B = the wavefront's q^T fragments, held in registers for the whole query;
//   - in the C layout of S^T every lane holds 8 rows of one head, which is exactly the
//     A-operand layout of P for O = P V, so P never leaves registers;
//   - V fragments (8 rows of one dim per lane) come from ds_read_b64_tr_b16 transposing
//     reads of the row-major tile; O (16 heads x 512 dims) accumulates in fp32 registers,
//     and one more matrix op per tile against a ones operand accumulates the softmax
//     denominators;
//   - online softmax with a lazy reference maximum: O and the denominators are rescaled
//     only when a head's running maximum grows by more than 2^16 (exponentials stay below
//     2^16), and the rescale itself runs on the matrix cores.
#include "attn_mfma.hpp"
#include "internal.hpp"

namespace csa {

namespace {

using namespace amfma;

constexpr int HPW = 16;     // heads per wavefront
// fragment chunks read ahead of the matrix ops (two workgroups per CU hide most of the
// LDS latency; deeper rings would not fit the 256 registers)
constexpr int SDA = 0;  // K fragments
constexpr int PVA = 2;  // V fragments

// NWV wavefronts per workgroup: 4 (64 heads; two workgroups share a CU) or 8 (128 heads,
// one workgroup per CU: every gathered row is loaded once for all 128 heads).
// KV8: the compressed rows are in the FP8 storage format (592 bytes: E4M3 codes with one
// E8M0 scale per 32, then the bf16 RoPE dims); each wavefront expands the rows it loaded to
// bf16 in place in LDS once they have landed, so the tile loop itself is unchanged.
template <int NWV, bool KV8>
__global__ void __launch_bounds__(64 * NWV, 8 / NWV)
attn_wide_kernel(const bf16_t *__restrict__ q, const bf16_t *__restrict__ kv, const float *__restrict__ sink,
                 const int32_t *__restrict__ idx, int k, int ratio, float scale_log2,
                 const bf16_t *__restrict__ swa, const int64_t *__restrict__ swa_pos0, int swa_rows,
                 int window, const int32_t *__restrict__ q_seq, const int64_t *__restrict__ q_pos,
                 const float *__restrict__ rope_cs, int R, int T, int B, int64_t N, int H,
                 bf16_t *__restrict__ out, float *__restrict__ lse, float *__restrict__ part,
                 int nsplit, int64_t split_slots)
{
    constexpr int WH = HPW * NWV;  // heads per workgroup
    constexpr int RPW = WR / NWV;  // tile rows loaded per wavefront
    __shared__ __attribute__((aligned(16))) bf16_t KV0[WR * WP];  // tile buffers (separate arrays,
    __shared__ __attribute__((aligned(16))) bf16_t KV1[WR * WP];  // see the row loads below)
    __shared__ int32_t sidx[kIdxCache];

    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;

    // XCD-aware placement: units (query, split, head group) are dealt to the 8 XCDs in
    // contiguous runs, so neighbouring queries (which share SWA rows and summaries) meet
    // in one L2
    const int HGN = H / WH;
    const int64_t U = (int64_t)T * nsplit * HGN;
    const int64_t per_xcd = (U + 7) / 8;
    const int64_t bid = blockIdx.x;
    const int64_t u = (bid & 7) * per_xcd + (bid >> 3);
    if ((bid >> 3) >= per_xcd || u >= U) return;
    const int hg = (int)(u % HGN);
    const int64_t tu = u / HGN;
    const int t = (int)(tu / nsplit), sp = (int)(tu % nsplit);
    const int head0 = hg * WH + HPW * w;  // first head of this wave

    const RowCtx c = row_ctx(t, q_seq, q_pos, B, N, k, ratio, swa, swa_pos0, window);
    const int64_t j0 = (int64_t)sp * split_slots;
    int64_t j1 = j0 + split_slots;
    if (j1 > c.nslots) j1 = c.nslots;

    // ---- q^T fragments (B operand of S^T): head head0 + l16, dims 32kk + 8g4 .. +7, with
    // RoPE applied to the last R dims (in fp32, rounded once to bf16)
    bf16x8 qf[KKN];
    {
        const bf16_t *qrow = q + ((int64_t)t * H + head0 + l16) * WD;
        const float *rope_t = rope_cs ? rope_cs + (int64_t)t * R : nullptr;
#pragma unroll
        for (int kk = 0; kk < KKN; ++kk) qf[kk] = q_fragment(qrow, kk, g4, rope_t, R);
    }

    // softmax state: m_ref of head head0 + l16 (replicated over the 4 lane groups); the
    // denominators live in the output layout (head head0 + 4g4 + r in component r of lacc)
    // and are accumulated by one extra matrix op per tile against a ones operand, so they
    // sum the same bf16 weights that enter O; the sink contributes 2^(m_ref - m_ref) = 1.
    const bool single = (nsplit == 1);
    float m_ref = single ? sink[head0 + l16] * kLog2e : -INFINITY;
    f32x4 lacc;
#pragma unroll
    for (int r = 0; r < 4; ++r) lacc[r] = (single && sink[head0 + 4 * g4 + r] != -INFINITY) ? 1.f : 0.f;
    f32x4 acc[NDN];
#pragma unroll
    for (int nd = 0; nd < NDN; ++nd) acc[nd] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The split's top-k indices (up to kIdxCache of them) are read once into LDS, so a
    // tile's row addresses cost no global round trip.
    const int64_t jm = (j1 < c.nmain) ? j1 : c.nmain;  // main slots of this split: [j0, jm)
    const int64_t ncache = (jm - j0 < kIdxCache) ? jm - j0 : kIdxCache;
    if (ratio <= 0)
        for (int64_t x = threadIdx.x; x < ncache; x += 64 * NWV) sidx[x] = idx[(int64_t)t * k + j0 + x];
    __syncthreads();
    // Rows without data read a valid stand-in address (this wave's own q rows) and are
    // masked out of the softmax, so every load is issued unconditionally.
    const bf16_t *standin = q + ((int64_t)t * H + head0) * WD;
    const int32_t *idx_t = (ratio > 0) ? nullptr : idx + (int64_t)t * k;
    // Row addresses of the tile at slot jt: lane r < 32 resolves slot jt + r to a byte
    // address (the stand-in when the slot has no row) and the tile's 32-bit validity mask
    // comes from a ballot.
    constexpr int64_t kKvRow = KV8 ? kKv8RowBytes / 2 : WD;  // bf16 elements per compressed row
    // (KV8) kvm: the tile's rows that are compressed rows (the rest are SWA rows, already
    // bf16, or stand-ins)
    auto tile_rows = [&](int64_t jt, uint64_t &addr, uint32_t &kvm) -> uint32_t {
        const int64_t j = jt + (lane & 31);
        const bf16_t *p = slot_row(c, j, j0, j1, ratio, sidx, idx_t, N, kv, swa, swa_rows, standin, kKvRow);
        addr = (uint64_t)(uintptr_t)p;
        kvm = KV8 ? (uint32_t)(__ballot(p != standin && j < c.nmain) & 0xffffffffull) : 0u;
        return (uint32_t)(__ballot(p != standin) & 0xffffffffull);
    };
    // Rows go from memory straight into LDS: wavefront w loads rows RPW*w .. RPW*w + RPW-1
    // of a tile, one 1 KiB row per buffer-load instruction (16 bytes per lane, LDS
    // destination). A load's row is the same for the whole wave, so its address is read
    // out of the resolving lane into scalar registers and wrapped in a buffer resource
    // over that row. The two tile buffers are separate LDS arrays and the loads are buffer
    // instructions, so the compiler can tell that loads into one buffer never alias reads
    // of the other and keeps the loads in flight across a whole tile.
    const int wu = __builtin_amdgcn_readfirstlane(w);
    // (the resource of an FP8-format row ends with the row: the rest of the 1 KiB load
    // reads zeros instead of the next row)
    auto dma_row = [&](bf16_t *buf, int i, uint64_t addr, uint32_t kvm) {
        const int row = RPW * wu + i;
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)addr, row);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(addr >> 32), row);
        const int bytes = (KV8 && ((kvm >> row) & 1u)) ? kKv8RowBytes : WD * 2;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), 0, bytes, kBufDword3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(buf + row * WP), 16,
                                                 lane * 16, 0, 0, 0);
    };
    // (KV8) the wave's compressed rows of a landed tile, expanded to bf16 in place, two rows
    // at a time (one per half-wavefront). In a half, lanes 0..27 turn 16 codes each into 32
    // bytes of bf16 (one scale per lane pair) with the scaled conversion (code x 2^e in one
    // instruction per two codes, exact), lanes 28..31 move 32 of the 128 bytes of bf16 RoPE
    // dims to dims 448..511. Every read of both rows is issued before the first write (LDS
    // serves one wavefront in order, and the compiler fence keeps the reads ahead), so a row
    // converts where it lies.
    auto kv8_expand = [&](bf16_t *buf, uint32_t kvm) {
        if constexpr (KV8) {
            static_assert(RPW % 2 == 0, "rows are expanded in pairs");
            const int hh = lane >> 5, l = lane & 31;
            const bool cv = l < 28;
            const int off = cv ? 16 * l : 448 + 32 * (l - 28);
#pragma unroll
            for (int i = 0; i < RPW; i += 2) {
                const int row = RPW * wu + i + hh;
                const bool act = (kvm >> row) & 1u;
                uint8_t *rb = reinterpret_cast<uint8_t *>(buf + row * WP);
                const uint4 r0 = *reinterpret_cast<const uint4 *>(rb + off);
                const uint4 r1 = *reinterpret_cast<const uint4 *>(rb + off + 16);
                const uint32_t sb = rb[576 + (cv ? (l >> 1) : 0)];
                asm volatile("" ::: "memory");
                if (act && cv) {
                    const uint32_t wd[4] = {r0.x, r0.y, r0.z, r0.w};
                    uint32_t o[8];
                    if (sb != 0u) {
                        const float sc = __builtin_bit_cast(float, sb << 23);  // 2^(sb - 127)
#pragma unroll
                        for (int qd = 0; qd < 4; ++qd) {
                            o[2 * qd] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd[qd], sc, false));
                            o[2 * qd + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd[qd], sc, true));
                        }
                    } else {
                        // e = -127 (2^-127 is no normal float): decode, then scale
#pragma unroll
                        for (int qd = 0; qd < 4; ++qd) {
                            const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(wd[qd], false);
                            const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(wd[qd], true);
                            o[2 * qd] = pack_bf16x2(__builtin_ldexpf(lo[0], -127), __builtin_ldexpf(lo[1], -127));
                            o[2 * qd + 1] = pack_bf16x2(__builtin_ldexpf(hi[0], -127), __builtin_ldexpf(hi[1], -127));
                        }
                    }
                    *reinterpret_cast<uint4 *>(rb + 32 * l) = make_uint4(o[0], o[1], o[2], o[3]);
                    *reinterpret_cast<uint4 *>(rb + 32 * l + 16) = make_uint4(o[4], o[5], o[6], o[7]);
                } else if (act) {
                    *reinterpret_cast<uint4 *>(rb + 896 + 32 * (l - 28)) = r0;
                    *reinterpret_cast<uint4 *>(rb + 896 + 32 * (l - 28) + 16) = r1;
                }
            }
        }
    };

    uint32_t valid = 0u, valid_next = 0u, kvm = 0u, kvm_next = 0u;
    uint64_t ra;  // row addresses of the next tile, resolved one tile ahead
    if (j0 < j1) {
        valid = tile_rows(j0, ra, kvm);
#pragma unroll
        for (int i = 0; i < RPW; ++i) dma_row(KV0, i, ra, kvm);
    }
    valid_next = tile_rows(j0 + WR, ra, kvm_next);
    // Every prologue load (Q fragments, first tile) has landed: without this the
    // loop's wait counters start pessimistic and stall the first matrix ops.
    __builtin_amdgcn_s_waitcnt(0);
    kv8_expand(KV0, kvm);
    __syncthreads();

    // One 32-row tile: compute from `tile`, load the next tile's rows into `nxt`. Past the
    // last tile every slot of the next tile resolves to the stand-in, so the loads need no
    // branch.
    auto tile_step = [&](const bf16_t *tile, bf16_t *nxt, int64_t jt, bool first) {
        uint64_t ra2;
        uint32_t valid_next2, kvm_next2;
        const uint32_t kvm_nxt = kvm_next;  // compressed rows of the tile loaded into nxt

#pragma unroll
        for (int i = 0; i < RPW; ++i) dma_row(nxt, i, ra, kvm_nxt);

        // ---- S^T = K Q^T (a ring keeps SDA chunks of K fragments in flight)
        f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        {
            bf16x8 ring[SDA + 1][2];
            const bf16_t *kb = tile + l16 * WP + g4 * 8;
#pragma unroll
            for (int cc = 0; cc < SDA; ++cc) {
                ring[cc][0] = ld_bf16x8(kb + 32 * cc);
                ring[cc][1] = ld_bf16x8(kb + 16 * WP + 32 * cc);
            }
#pragma unroll
            for (int kk = 0; kk < KKN; ++kk) {
                if (kk + SDA < KKN) {
                    ring[(kk + SDA) % (SDA + 1)][0] = ld_bf16x8(kb + 32 * (kk + SDA));
                    ring[(kk + SDA) % (SDA + 1)][1] = ld_bf16x8(kb + 16 * WP + 32 * (kk + SDA));
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    sacc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[kk % (SDA + 1)][m], qf[kk], sacc[m], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // rows of the tile after next: the index read and the address arithmetic overlap
        // the matrix ops still in flight
        valid_next2 = tile_rows(jt + 2 * WR, ra2, kvm_next2);

        // ---- online softmax with the lazy reference maximum
        // rows without data (only in a split's last tile or for padded / missing slots) are
        // masked to -inf; full tiles skip the mask
        if (valid != 0xffffffffu) {
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (!((valid >> (16 * m + 4 * g4 + r)) & 1u)) sacc[m][r] = -INFINITY;
        }
        // the scale is positive, so the max of the raw scores gives the max logit
        float smax = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                           fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
        {
            const auto x32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(smax), __float_as_uint(smax), false, false);
            smax = fmaxf(__uint_as_float(x32[0]), __uint_as_float(x32[1]));
            const auto x16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(smax), __float_as_uint(smax), false, false);
            smax = fmaxf(__uint_as_float(x16[0]), __uint_as_float(x16[1]));
        }
        const float tmax = smax * scale_log2;
        if (__ballot(tmax > m_ref + kLazy) != 0ull) {
            // rare: the accumulators are rescaled on the matrix cores, so they are only ever
            // touched by matrix ops; before the first P V product O is still zero
            const float mn = fmaxf(m_ref, tmax);
            const float alpha = (m_ref == -INFINITY || mn == -INFINITY) ? (mn == -INFINITY ? 1.f : 0.f)
                                                                        : exp2f(m_ref - mn);
            m_ref = mn;
            float ar[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ar[r] = (l16 == 4 * g4 + r) ? alpha : 0.f;
            lacc = scale_rows(lacc, ar);
            if (!first) {
#pragma unroll
                for (int nd = 0; nd < NDN; ++nd) acc[nd] = scale_rows(acc[nd], ar);
            }
        }
        // p = 2^(s * scale - m_ref) <= 2^kLazy, packed to bf16 in the A-operand layout of P.
        // v_exp_f32 flushes results below 2^-126 to zero, which only drops weights that
        // no bf16 sum could hold.
        bf16x8 pf;
        {
            const float nmu = (m_ref == -INFINITY) ? 0.f : -m_ref;
            uint32_t pk[4];
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int r = 0; r < 4; r += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[m][r], scale_log2, nmu));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[m][r + 1], scale_log2, nmu));
                    pk[2 * m + r / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{p0, p1}, bf16x2w));
                }
            pf = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
        }
        lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, ones_bf16x8(), lacc, 0, 0, 0);

        // ---- O += P V: V fragments (8 rows of one dim per lane, in the row order of the
        // C layout above) from transposing LDS reads, riding a register ring PVA ops ahead
        {
            const int s4 = l16 >> 2, sc = l16 & 3;
            const bf16_t *v0 = tile + (4 * g4 + s4) * WP + 4 * sc;
            const bf16_t *v1 = v0 + 16 * WP;
            bf16x4v vr[PVA + 1][2];
#pragma unroll
            for (int cc = 0; cc < PVA; ++cc) {
                vr[cc][0] = __builtin_bit_cast(bf16x4v, ld_tr(v0 + 16 * cc));
                vr[cc][1] = __builtin_bit_cast(bf16x4v, ld_tr(v1 + 16 * cc));
            }
#pragma unroll
            for (int nd = 0; nd < NDN; ++nd) {
                if (nd + PVA < NDN) {
                    vr[(nd + PVA) % (PVA + 1)][0] = __builtin_bit_cast(bf16x4v, ld_tr(v0 + 16 * (nd + PVA)));
                    vr[(nd + PVA) % (PVA + 1)][1] = __builtin_bit_cast(bf16x4v, ld_tr(v1 + 16 * (nd + PVA)));
                }
                __builtin_amdgcn_sched_barrier(0);
                const bf16x8 vf = __builtin_shufflevector(vr[nd % (PVA + 1)][0], vr[nd % (PVA + 1)][1], 0, 1, 2, 3,
                                                          4, 5, 6, 7);
                acc[nd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, vf, acc[nd], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        valid = valid_next;
        valid_next = valid_next2;
        kvm = kvm_next;
        kvm_next = kvm_next2;
        ra = ra2;
        // the next tile's rows have landed in `nxt` (this wave's own loads), and after the
        // barrier everyone's have (expanded, for FP8 rows) and nobody reads `tile` any more
        __builtin_amdgcn_s_waitcnt(0);
        kv8_expand(nxt, kvm_nxt);
        __syncthreads();
    };

    for (int64_t jt = j0; jt < j1;) {
        tile_step(KV0, KV1, jt, jt == j0);
        jt += WR;
        if (jt >= j1) break;
        tile_step(KV1, KV0, jt, false);
        jt += WR;
    }

    // ---- epilogue: O rows are heads head0 + 4g4 + r, columns dim 16nd + l16
    if (single) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int h = head0 + 4 * g4 + r;
            const float lv = lacc[r];
            const float mr = __shfl(m_ref, 4 * g4 + r);
            if (lse != nullptr && l16 == 0) {
                const float mu = (mr == -INFINITY) ? 0.f : mr;
                lse[(int64_t)t * H + h] = (lv > 0.f) ? (mu + log2f(lv)) * kLn2 : -INFINITY;
            }
            const float inv = lv > 0.f ? 1.f / lv : 0.f;
            bf16_t *orow = out + ((int64_t)t * H + h) * WD;
#pragma unroll
            for (int nd = 0; nd < NDN; ++nd) {
                const int d = 16 * nd + l16;
                float x = acc[nd][r] * inv;
                const float y = __shfl_xor(x, 1);
                if (rope_cs != nullptr && d >= WD - R) {
                    const int p = (d - (WD - R)) >> 1;
                    const float cs = rope_cs[((int64_t)t * (R / 2) + p) * 2];
                    const float sn = rope_cs[((int64_t)t * (R / 2) + p) * 2 + 1];
                    x = (d & 1) ? (x * cs - y * sn) : (x * cs + y * sn);
                }
                orow[d] = f32_to_bf16(x);
            }
        }
    } else {
        const int64_t pu = ((int64_t)t * nsplit + sp) * H + head0;
        float *pml = part;                                                               // [T][nsplit][H][2]
        bf16_t *pacc = reinterpret_cast<bf16_t *>(part + (int64_t)T * nsplit * H * 2);  // [T][nsplit][H][D]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float mr = __shfl(m_ref, 4 * g4 + r);
            if (l16 == 0) {
                pml[(pu + 4 * g4 + r) * 2] = mr;
                pml[(pu + 4 * g4 + r) * 2 + 1] = lacc[r];
            }
        }
        // bf16 pairs of adjacent dims: lanes l16 and l16 ^ 1 swap their values (DPP), then the
        // even lane of a pair stores heads 4g4 and 4g4 + 1 at dims (d, d + 1) and the odd lane
        // heads 4g4 + 2 and 4g4 + 3, so every lane issues two 4-byte stores per dim block
        const bool odd = (l16 & 1) != 0;
        const int ra = odd ? 2 : 0;
        const int dl = l16 & ~1;
#pragma unroll
        for (int nd = 0; nd < NDN; ++nd) {
            float nb[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                nb[r] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc[nd][r]), 0xB1, 0xF, 0xF, false));
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int r = ra + e;
                const float mine = odd ? acc[nd][2 + e] : acc[nd][e];
                const float other = odd ? nb[2 + e] : nb[e];
                const uint32_t w = odd ? pack_bf16x2(other, mine) : pack_bf16x2(mine, other);
                *reinterpret_cast<uint32_t *>(pacc + (pu + 4 * g4 + r) * WD + 16 * nd + dl) = w;
            }
        }
    }
}

}  // namespace

bool wide_attn_ok(csa_dtype dt, int H, int D) { return (dt == CSA_BF16 || dt == CSA_KV8) && D == WD && H % 64 == 0; }

int launch_attn_wide(const AttnArgs &a, float sl2, int nsplit, int64_t split_slots, hipStream_t st) {
    // many queries, one split each: 32 heads per wavefront, so every LDS fragment read
    // feeds two matrix ops (measured 16 % faster at the 4,096-query HCA prefill chunk and
    // 7 % at the 8,192-query sparse prefill chunk)
    if (w32_attn_ok(a.dt, a.H, a.D, a.N, a.swa_rows, a.ratio, a.k) && nsplit == 1 && (int64_t)a.T * (a.H / 128) >= 256)
        return launch_attn_w32(a, sl2, nsplit, split_slots, st);
    // many queries with gathered rows (sparse, 128-head multiples, no row split): one 8-wave
    // workgroup per 128 heads, so a row is fetched once per query (measured 5 % faster at
    // the Pro prefill chunk); otherwise 4-wave workgroups, two per CU (summaries sit in L2,
    // and few-query decode needs the extra workgroups)
    const bool wide8 = (a.ratio <= 0 && a.H % 128 == 0 && nsplit == 1);
    const int WH = wide8 ? 128 : 64;
    const int64_t U = (int64_t)a.T * nsplit * (a.H / WH);
    const int64_t blocks = ((U + 7) / 8) * 8;
#define CSA_WIDE_LAUNCH(NWV_, KV8_)                                                                            \
    hipLaunchKernelGGL((attn_wide_kernel<NWV_, KV8_>), dim3((unsigned)blocks), dim3(64 * NWV_), 0, st, (const bf16_t *)a.q, \
                       (const bf16_t *)a.kv, a.sink, a.idx, a.k, a.ratio, sl2, (const bf16_t *)a.swa, a.swa_pos0, \
                       a.swa_rows, a.window, a.q_seq, a.q_pos, a.rope_cs, a.rope_dim, a.T, a.B, a.N, a.H,        \
                       (bf16_t *)a.out, a.lse, (float *)a.ws, nsplit, split_slots);
    const bool kv8 = a.dt == CSA_KV8;
    if (wide8) {
        if (kv8) {
            CSA_WIDE_LAUNCH(8, true)
        } else {
            CSA_WIDE_LAUNCH(8, false)
        }
    } else {
        if (kv8) {
            CSA_WIDE_LAUNCH(4, true)
        } else {
            CSA_WIDE_LAUNCH(4, false)
        }
    }
#undef CSA_WIDE_LAUNCH
    return check_launch("attn_wide_kernel");
}

}  // namespace csa
