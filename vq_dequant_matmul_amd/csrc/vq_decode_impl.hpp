// vq_decode_impl.hpp -- bandwidth-bound VQ kernels for small token counts (gfx950).
//
// The decode step of a VQ MoE layer reads every routed expert's packed codes
// and scales once and does a handful of flops per byte, so it is bound by
// HBM bandwidth (the card "GLM-5.3-Flash-VQ-2.7bpw", section "Limitations",
// calls small-M decode the open frontier of the lineup; the card
// "Qwen3.8-Flash-Next-VQ-4.4bpw", changelog 2026-09, reports its Metal expert
// kernels being reworked for occupancy, direct activation reads and a SIMD
// reduction).  Layout of the work here:
//
//   * a wavefront is split into segments of S lanes (S = a power of two
//     >= the number of 64-column groups of a row, up to 64); a segment owns
//     one output row per iteration and each lane owns whole groups of it
//     (GPL groups per lane when a row has more than 64 groups);
//   * a lane's activations for its groups stay in registers for every row it
//     visits, as fp16 pairs scaled by a power of two chosen per (token,
//     group) so the conversion from bf16 is exact;
//   * codes are loaded as the few dwords that cover the lane's group and
//     shifted to bit 0 with v_alignbit; code t sits at the compile-time bit
//     t*b;  the tensor's codebook is staged once per workgroup in LDS;
//   * each code contributes dot2(codebook entry, x pair) in fp32 and the
//     group's fp16 scale is applied once per group (the scale factors out of
//     the group's sum);  the segment's partial sums meet in a butterfly.
//
// The same engine runs one expert (vq_expert_gemv), the routed gate+up
// projections with the SwiGLU product fused in the epilogue, and the routed
// down projection.  It is persistent: a few workgroups per CU each stage the
// codebooks and build the routing lists once (the (token, slot) pairs
// grouped by distinct expert, in slot order), then walk a contiguous range
// of work units.  A unit is (distinct expert, tile of rows, one of its
// pairs), ordered expert-major, so consecutive units of a workgroup share
// the pair's converted activations and usually the expert.
#pragma once
#include "vq_common.hpp"
#include "vq_internal.hpp"

namespace vq {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// a launch with bf16 activations and fewer units than this many per CU at
// two row passes per unit takes one pass per unit
constexpr int kRowsOnePassUnitsPerCu = 6;
constexpr int kRowsFourPassUnitsPerCu = 16;

struct RowsArgs {
    const uint32_t *codes[2];
    const uint16_t *scales[2];
    const int32_t *row_map[2];
    const uint16_t *codebook[2];
    int cb_dwords[2];
    int cb_offset[2];   // dword offset of each codebook in LDS (0 and cb1_offset())
    int list_offset;    // dword offset of the work lists in LDS
    int rows, groups, wpr;
    int S_log2;         // lanes per row segment
    int tile_rows;      // rows per work unit: waves * iters * rows per wave pass
    int tiles;          // tiles per expert
    int iters;          // row passes of a wave per unit (1 or 2: the kernel's ITERS)
    const void *act;
    int64_t act_stride;
    float *out;
    int64_t out_stride;
    int expert, n_act;  // one expert applied to n_act activation rows ...
    const int32_t *ids; // ... or routed pairs: pair q uses expert ids[q],
    int n_slots, act_div; // activation row q / act_div, output row q
};

// LDS layout of a workgroup (dwords, 16-byte aligned, nothing static):
//   [0, ...)             codebook of projection 0 (lookups address code*d/2)
//   [cb1_offset(), ...)  codebook of projection 1 (gate+up launches)
//   [list_offset, ...)   work lists (see build_lists)
// The second codebook sits at its largest possible size when that keeps
// the offset inside a ds_read immediate, so no lookup needs a base add.
// 8-bit codes with d = 2: the codebooks as 16 copies per entry.  Entry k of
// projection p owns bytes [128k + 64p, 128k + 64p + 64) of LDS and lane l
// reads copy l % 16, so of the 32 lanes an LDS pass serves only lanes l and
// l + 16 can meet in a bank (when their entries have equal parity), against
// a random spread over a single copy.  32 KiB for one or two projections.
template <int D, int BITS>
constexpr bool rows_banked() { return D == 2 && BITS == 8; }
constexpr int kBankedCbDwords = 8192;

template <int D, int BITS>
constexpr int cb1_fixed_dwords() { return (1 << BITS) * D / 2; }

template <int D, int BITS>
constexpr bool cb1_is_fixed() { return cb1_fixed_dwords<D, BITS>() * 4 <= 32768; }

template <int D, int BITS>
__device__ __forceinline__ int cb1_offset(const RowsArgs &a)
{
    if constexpr (cb1_is_fixed<D, BITS>())
        return cb1_fixed_dwords<D, BITS>();
    else
        return a.cb_offset[1];
}

template <int D>
struct Entry {
    uint32_t v[D / 2];
};

template <int D>
__device__ __forceinline__ Entry<D> fetch_entry(const uint32_t *__restrict__ cb, uint32_t code)
{
    Entry<D> e;
    if constexpr (D == 2) {
        e.v[0] = cb[code];
    } else if constexpr (D == 4) {
        const uint2 t = *reinterpret_cast<const uint2 *>(cb + 2 * code);
        e.v[0] = t.x;
        e.v[1] = t.y;
    } else {
        const uint4 t = *reinterpret_cast<const uint4 *>(cb + 4 * code);
        e.v[0] = t.x;
        e.v[1] = t.y;
        e.v[2] = t.z;
        e.v[3] = t.w;
    }
    return e;
}

// Code t of a group already shifted to bit 0 (t is a constant after unrolling).
template <int BITS, int NW>
__device__ __forceinline__ uint32_t extract(const uint32_t (&nw)[NW], int t)
{
    const int p = t * BITS;
    const int wi = p >> 5;
    const int sh = p & 31;
    const uint32_t mask = (1u << BITS) - 1u;
    if (sh + BITS <= 32)
        return __builtin_amdgcn_ubfe(nw[wi], sh, BITS);
    return __builtin_amdgcn_alignbit(nw[wi + 1], nw[wi], sh) & mask;
}

// Activations of one lane for one row: GPL groups x 32 fp16 pairs, plus the
// factor 2^-k that undoes each group's range scaling.
template <int GPL, bool HL>
struct XRegs {
    f16x2 hi[GPL][32];
    f16x2 lo[HL ? GPL : 1][HL ? 32 : 1];
    float m[GPL];
};

// Raw activations of one lane (bf16: 32 dwords per group, fp32: 64).
template <int GPL, bool F32>
struct XRaw {
    static constexpr int Q = F32 ? 16 : 8;   // uint4 per group
    uint4 q[GPL][Q];
};

template <int GPL, bool F32>
__device__ __forceinline__ void load_x_raw(const RowsArgs &a, int arow, int sl, int S,
                                           XRaw<GPL, F32> &xw)
{
    constexpr int Q = XRaw<GPL, F32>::Q;
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
        // lanes past the last group read the last group (their result is
        // discarded); every load is unconditional so all stay in flight
        const int g = min(sl + i * S, a.groups - 1);
        const int64_t off = (int64_t)arow * a.act_stride + 64 * g;
        const uint4 *p = F32 ? reinterpret_cast<const uint4 *>(static_cast<const float *>(a.act) + off)
                             : reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.act) + off);
#pragma unroll
        for (int j = 0; j < Q; ++j)
            xw.q[i][j] = p[j];
    }
}

// Raw activations -> range-scaled fp16 pairs, one dword (bf16 pair) or two
// floats at a time.  For bf16 the largest magnitude is found on the bit
// patterns (non-negative floats order like their integer encodings).
template <int GPL, bool HL, bool F32>
__device__ __forceinline__ void convert_x(const XRaw<GPL, F32> &xw, XRegs<GPL, HL> &xr)
{
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
        const uint4 *q = xw.q[i];
        if constexpr (F32) {
            float amax = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j)
                amax = fmaxf(fmaxf(amax, fmaxf(fabsf(__uint_as_float(q[j].x)),
                                               fabsf(__uint_as_float(q[j].y)))),
                             fmaxf(fabsf(__uint_as_float(q[j].z)), fabsf(__uint_as_float(q[j].w))));
            const int k = range_exponent(amax);
            const float up = ldexpf(1.0f, k);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float f[4] = {__uint_as_float(q[j].x) * up, __uint_as_float(q[j].y) * up,
                                    __uint_as_float(q[j].z) * up, __uint_as_float(q[j].w) * up};
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const f16x2 hp = pack_f16x2(f[2 * h], f[2 * h + 1]);
                    xr.hi[i][2 * j + h] = hp;
                    if constexpr (HL)
                        xr.lo[i][2 * j + h] = pack_f16x2(f[2 * h] - (float)hp.x, f[2 * h + 1] - (float)hp.y);
                }
            }
            xr.m[i] = ldexpf(1.0f, -k);
        } else {
            uint32_t mx = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t w4[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
                for (int h = 0; h < 4; ++h)
                    mx = max(mx, max(w4[h] & 0x7fffu, (w4[h] >> 16) & 0x7fffu));
            }
            const int k = range_exponent(__uint_as_float(mx << 16));
            const float up = ldexpf(1.0f, k);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t w4[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const float lo16 = __uint_as_float(w4[h] << 16) * up;
                    const float hi16 = __uint_as_float(w4[h] & 0xffff0000u) * up;
                    const f16x2 hp = pack_f16x2(lo16, hi16);
                    xr.hi[i][4 * j + h] = hp;
                    if constexpr (HL)
                        xr.lo[i][4 * j + h] = pack_f16x2(lo16 - (float)hp.x, hi16 - (float)hp.y);
                }
            }
            xr.m[i] = ldexpf(1.0f, -k);
        }
    }
}

template <int D, int BITS, int GPL, int NPROJ>
struct RowRegs {
    uint32_t w[NPROJ][GPL][Geom<D, BITS>::NW];
    uint32_t sc[NPROJ][GPL];
    int live;   // bit p: projection p's row is stored (not skip-zero)
};

// Issue the code and scale loads of this lane's rows (every load
// unconditional; rows past the end and dead rows read stored row 0 and are
// zeroed afterwards -- the host never launches for a tensor with no stored
// rows).  The stored-row lookup (row map) is one dependent load.
// MAP: some projection has a row map.  Without one no load depends on
// another, so nothing waits for loads issued earlier.
template <int D, int BITS, int GPL, int NPROJ, int ITERS, bool MAP>
__device__ __forceinline__ void load_rows_m(const RowsArgs &a, int e, int row0, int rpw, int seg,
                                            int sl, int S,
                                            RowRegs<D, BITS, GPL, NPROJ> (&rr)[ITERS])
{
    using GM = Geom<D, BITS>;
    constexpr int NW = GM::NW;
    int srow[ITERS][NPROJ];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int r = row0 + it * rpw + seg;
        const int64_t lin = (int64_t)e * a.rows + min(r, a.rows - 1);
#pragma unroll
        for (int p = 0; p < NPROJ; ++p)
            srow[it][p] = (MAP && a.row_map[p]) ? a.row_map[p][lin] : (int)lin;
    }
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int r = row0 + it * rpw + seg;
        rr[it].live = 0;
#pragma unroll
        for (int p = 0; p < NPROJ; ++p) {
            const bool live = (r < a.rows) && (srow[it][p] >= 0);
            rr[it].live |= live ? (1 << p) : 0;
            const int64_t sr = live ? srow[it][p] : 0;
            const uint32_t *row = a.codes[p] + sr * a.wpr;
#pragma unroll
            for (int i = 0; i < GPL; ++i) {
                const int g = min(sl + i * S, a.groups - 1);
                const int w0 = (g * GM::GB) >> 5;
                if constexpr (GM::CLAMP) {
#pragma unroll
                    for (int k = 0; k < NW; ++k)
                        rr[it].w[p][i][k] = row[min(w0 + k, a.wpr - 1)];
                } else {
                    // the group's words never leave its block: 16-byte loads
                    // (dword alignment suffices on gfx950)
                    __builtin_memcpy(rr[it].w[p][i], row + w0, NW * 4);
                }
                rr[it].sc[p][i] = a.scales[p][sr * a.groups + g];
            }
        }
    }
}

template <int D, int BITS, int GPL, int NPROJ, int ITERS>
__device__ __forceinline__ void load_rows(const RowsArgs &a, int e, int row0, int rpw, int seg,
                                          int sl, int S, RowRegs<D, BITS, GPL, NPROJ> (&rr)[ITERS])
{
    bool map = false;
#pragma unroll
    for (int p = 0; p < NPROJ; ++p)
        map = map || a.row_map[p] != nullptr;
    if (map)
        load_rows_m<D, BITS, GPL, NPROJ, ITERS, true>(a, e, row0, rpw, seg, sl, S, rr);
    else
        load_rows_m<D, BITS, GPL, NPROJ, ITERS, false>(a, e, row0, rpw, seg, sl, S, rr);
}

template <int D, int BITS, int GPL, int NPROJ, bool HL, int ITERS>
__device__ __forceinline__ void compute_rows(const RowsArgs &a, const uint32_t *__restrict__ lds,
                                             const RowRegs<D, BITS, GPL, NPROJ> (&rr)[ITERS],
                                             const XRegs<GPL, HL> &xr, int item, int S, int seg,
                                             int sl, int row0, int rpw)
{
    using GM = Geom<D, BITS>;
    constexpr int NW = GM::NW;
    constexpr int G = GM::G;
    constexpr int HP = D / 2;   // fp16 pairs per codebook entry

#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int r = row0 + it * rpw + seg;
        float part[NPROJ];
#pragma unroll
        for (int p = 0; p < NPROJ; ++p) {
            part[p] = 0.0f;
            const uint32_t *cb = lds + (p == 0 ? 0 : cb1_offset<D, BITS>(a));
            const uint32_t *cbk = lds + p * 16 + (threadIdx.x & 15);   // this lane's copies
#pragma unroll
            for (int i = 0; i < GPL; ++i) {
                const int g = sl + i * S;
                uint32_t nw[NW];
                shift_group_words<D, BITS>(g, rr[it].w[p][i], nw);
                float acc = 0.0f, accl = 0.0f;
#pragma unroll
                for (int t = 0; t < G; ++t) {
                    const uint32_t code = extract<BITS, NW>(nw, t);
                    Entry<D> en;
                    if constexpr (rows_banked<D, BITS>())
                        en.v[0] = cbk[code * 32];
                    else
                        en = fetch_entry<D>(cb, code);
#pragma unroll
                    for (int k = 0; k < HP; ++k) {
                        acc = dot2(en.v[k], xr.hi[i][t * HP + k], acc);
                        if constexpr (HL)
                            accl = dot2(en.v[k], xr.lo[i][t * HP + k], accl);
                    }
                }
                const float s = (g < a.groups) ? half_bits_to_float(rr[it].sc[p][i]) : 0.0f;
                part[p] += (HL ? acc + accl : acc) * (s * xr.m[i]);
                // keep one group's lookups in flight at a time (bounds registers)
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // segment reduction (S is uniform)
#pragma unroll
        for (int p = 0; p < NPROJ; ++p)
            part[p] = segment_sum_dpp(part[p], S);
        if (sl == 0 && r < a.rows) {
            float val;
            if constexpr (NPROJ == 2)
                val = (rr[it].live == 3) ? silu_mul(part[0], part[1]) : 0.0f;
            else
                val = (rr[it].live & 1) ? part[0] : 0.0f;
            a.out[(int64_t)item * a.out_stride + r] = val;
        }
    }
}

// Codebook staging (layout above).  Up to CbBatch
// uint4 per thread are loaded into registers together with everything else a
// workgroup needs, then written to LDS; larger codebooks finish with a
// looping pass.
template <int D, int BITS>
constexpr int cb_max_dwords() { return (1 << BITS) * D / 2; }

template <int D, int BITS>
constexpr int cb_batch()
{
    constexpr int per_thread = (cb_max_dwords<D, BITS>() / 4 + kThreads - 1) / kThreads;
    return per_thread < 4 ? per_thread : 4;
}

template <int D, int BITS, int NPROJ>
struct CbRegs {
    uint4 v[NPROJ][cb_batch<D, BITS>()];
};

// The first B*kThreads uint4 of a codebook, one slot per thread and batch.
template <int B>
__device__ __forceinline__ void cb_to_regs(const uint16_t *cb, int dwords, uint4 (&v)[B])
{
    const uint4 *src = reinterpret_cast<const uint4 *>(cb);
    const int n4 = dwords >> 2;
#pragma unroll
    for (int j = 0; j < B; ++j) {
        const int i = threadIdx.x + j * kThreads;
        v[j] = (i < n4) ? src[i] : make_uint4(0u, 0u, 0u, 0u);
    }
}

// The codebook into LDS at base: the register batches, then the rest
// (codebooks beyond B*16*kThreads bytes, and a tail of fewer than four
// dwords) straight from global memory.
template <int B>
__device__ __forceinline__ void cb_regs_to_lds(const uint16_t *cb, int dwords, const uint4 (&v)[B],
                                               uint32_t *__restrict__ base)
{
    uint4 *dst = reinterpret_cast<uint4 *>(base);
    const int n4 = dwords >> 2;
#pragma unroll
    for (int j = 0; j < B; ++j) {
        const int i = threadIdx.x + j * kThreads;
        if (i < n4)
            dst[i] = v[j];
    }
    const uint32_t *s32 = reinterpret_cast<const uint32_t *>(cb);
    for (int i = 4 * B * kThreads + threadIdx.x * 4; i + 3 < dwords; i += 4 * kThreads)
        *reinterpret_cast<uint4 *>(base + i) = *reinterpret_cast<const uint4 *>(s32 + i);
    for (int i = (n4 << 2) + threadIdx.x; i < dwords; i += kThreads)
        base[i] = s32[i];
}

template <int D, int BITS, int NPROJ>
__device__ __forceinline__ void load_codebooks(const RowsArgs &a, CbRegs<D, BITS, NPROJ> &cr)
{
    if constexpr (rows_banked<D, BITS>()) {
        // thread t holds entry t (one dword) of each projection
#pragma unroll
        for (int p = 0; p < NPROJ; ++p) {
            const int t = threadIdx.x;
            const uint32_t v =
                t < a.cb_dwords[p] ? reinterpret_cast<const uint32_t *>(a.codebook[p])[t] : 0u;
            cr.v[p][0] = make_uint4(v, v, v, v);
        }
    } else {
#pragma unroll
        for (int p = 0; p < NPROJ; ++p)
            cb_to_regs(a.codebook[p], a.cb_dwords[p], cr.v[p]);
    }
}

template <int D, int BITS, int NPROJ>
__device__ __forceinline__ void store_codebooks(const RowsArgs &a, const CbRegs<D, BITS, NPROJ> &cr,
                                                uint32_t *__restrict__ lds)
{
    if constexpr (rows_banked<D, BITS>()) {
        static_assert(kThreads == 256, "one thread per entry");
        // the 16 copies of entry t, 16 bytes at a time; neighbouring lanes
        // start at different chunks so a store's lanes spread over the banks
        char *row = reinterpret_cast<char *>(lds) + threadIdx.x * 128;
#pragma unroll
        for (int p = 0; p < NPROJ; ++p)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<uint4 *>(row + p * 64 + ((j + threadIdx.x) & 3) * 16) = cr.v[p][0];
    } else {
#pragma unroll
        for (int p = 0; p < NPROJ; ++p)
            cb_regs_to_lds(a.codebook[p], a.cb_dwords[p], cr.v[p],
                           lds + (p == 0 ? 0 : cb1_offset<D, BITS>(a)));
    }
}

// Work lists in LDS, from list_offset (P = number of pairs):
//   ids[P]      expert of each pair
//   first[P]    first pair with the same expert
//   rank[P]     position of the pair among its expert's pairs (slot order)
//   uidx[P]     index of the pair's expert among the distinct experts
//   ustart[P+1] start of each distinct expert's pairs in items[]
//   items[P]    pairs grouped by distinct expert (first-occurrence order)
//   uexp[P]     expert id of each distinct expert
//   U           number of distinct experts
// Everything is a deterministic function of the ids.
struct Lists {
    int *ids, *first, *rank, *uidx, *ustart, *items, *uexp, *U;
};

__device__ __forceinline__ Lists lists_at(uint32_t *lds, int offset, int P)
{
    Lists L;
    L.ids = reinterpret_cast<int *>(lds + offset);
    L.first = L.ids + P;
    L.rank = L.first + P;
    L.uidx = L.rank + P;
    L.ustart = L.uidx + P;
    L.items = L.ustart + P + 1;
    L.uexp = L.items + P;
    L.U = L.uexp + P;
    return L;
}

constexpr int list_dwords(int P) { return 7 * P + 2; }

// Lists of a single token's pairs: one "distinct expert" per pair (a
// repeated id is then simply streamed twice).  Called by every thread.
__device__ __forceinline__ void single_token_lists(const Lists &L, const int32_t *ids, int P)
{
    for (int q = threadIdx.x; q < P; q += kThreads) {
        const int id = ids[q];
        L.ids[q] = id;
        L.uexp[q] = id;
        L.items[q] = q;
        L.ustart[q] = q;
    }
    if (threadIdx.x == 0) {
        L.ustart[P] = P;
        *L.U = P;
    }
}

// The same with pair tid's expert id already in a register (P <= threads).
__device__ __forceinline__ void single_token_lists_held(const Lists &L, int id, int P)
{
    const int q = threadIdx.x;
    if (q < P) {
        L.ids[q] = id;
        L.uexp[q] = id;
        L.items[q] = q;
        L.ustart[q] = q;
    }
    if (q == 0) {
        L.ustart[P] = P;
        *L.U = P;
    }
}

// Called by every thread after L.ids is filled and a barrier.
__device__ __forceinline__ void build_lists(const Lists &L, int P)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    for (int q = tid; q < P; q += kThreads) {
        const int id = L.ids[q];
        int f = q, r = 0;
        for (int q2 = 0; q2 < q; ++q2)
            if (L.ids[q2] == id) {
                f = (r == 0) ? q2 : f;
                ++r;
            }
        L.first[q] = f;
        L.rank[q] = r;
    }
    for (int u = tid; u <= P; u += kThreads)
        L.ustart[u] = 0;
    __syncthreads();
    if (tid < 64) {   // distinct experts in first-occurrence order
        int base = 0;
        for (int c = 0; c < P; c += 64) {
            const int q = c + lane;
            const bool isf = (q < P) && (L.first[q] == q);
            const unsigned long long b = __ballot(isf);
            if (isf) {
                const int u = base + __popcll(b & ((1ull << lane) - 1ull));
                L.uidx[q] = u;
                L.uexp[u] = L.ids[q];
            }
            base += __popcll(b);
        }
        if (lane == 0)
            *L.U = base;
    }
    __syncthreads();
    for (int q = tid; q < P; q += kThreads)
        atomicAdd(&L.ustart[L.uidx[L.first[q]] + 1], 1);
    __syncthreads();
    if (tid < 64) {   // prefix sum of the counts
        const int U = *L.U;
        int run = 0;
        for (int c = 0; c < U; c += 64) {
            const int u = c + lane;
            int v = (u < U) ? L.ustart[u + 1] : 0;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int t = __shfl_up(v, o, 64);
                if (lane >= o)
                    v += t;
            }
            if (u < U)
                L.ustart[u + 1] = run + v;
            run += __shfl(v, 63, 64);
        }
    }
    __syncthreads();
    for (int q = tid; q < P; q += kThreads)
        L.items[L.ustart[L.uidx[L.first[q]]] + L.rank[q]] = q;
    __syncthreads();
}

template <int D, int BITS, int GPL, int NPROJ, bool HL, bool F32, int ITERS>
__global__ __launch_bounds__(kThreads) void k_rows(const RowsArgs a)
{
    // all LDS is dynamic so the first codebook starts at byte 0; 16-byte
    // alignment keeps the 8- and 16-byte codebook entries aligned (a
    // misaligned ds_read_b64 costs several times an aligned one)
    extern __shared__ __attribute__((aligned(16))) uint32_t lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // ---- this workgroup's contiguous range of units (expert, tile, pair) -----
    const int P = a.ids ? a.n_slots : a.n_act;
    const bool one_token = a.ids && a.act_div == a.n_slots;
    const int S = 1 << a.S_log2;
    const int rpw = 64 >> a.S_log2;
    const int seg = lane >> a.S_log2;
    const int sl = lane & (S - 1);
    const int64_t n_units = (int64_t)P * a.tiles;
    int64_t k = (int64_t)udiv_small((uint64_t)blockIdx.x * n_units, gridDim.x);
    const int64_t k_end = (int64_t)udiv_small((uint64_t)(blockIdx.x + 1) * n_units, gridDim.x);
    struct Unit {
        int item, e, row0;
    };
    // The setup's own loads go first (the codebooks, and with one token the
    // pairs' expert ids): loads return in issue order, so these arrive ahead
    // of the first unit's rows instead of behind them.
    CbRegs<D, BITS, NPROJ> cr;
    load_codebooks<D, BITS, NPROJ>(a, cr);
    const bool ids_held = one_token && P <= kThreads;
    const int my_id = (ids_held && tid < P) ? load_global(a.ids + tid) : 0;
    // With one expert, or one token's pairs, a unit's expert is known without
    // the lists: its rows are requested before the setup below, so that the
    // memory latency overlaps the codebook staging.
    RowRegs<D, BITS, GPL, NPROJ> A[ITERS], B[ITERS];
    Unit ua, ub;
    const bool direct = one_token || !a.ids;
    if (direct && k < k_end) {
        if (one_token) {
            ua.item = (int)udiv_small(k, a.tiles);
            ua.e = load_global(a.ids + ua.item);
            ua.row0 = (int)(k - (int64_t)ua.item * a.tiles) * a.tile_rows + wave * ITERS * rpw;
        } else {
            const int t = (int)udiv_small(k, P);
            ua.item = (int)(k - (int64_t)t * P);
            ua.e = a.expert;
            ua.row0 = t * a.tile_rows + wave * ITERS * rpw;
        }
        load_rows<D, BITS, GPL, NPROJ, ITERS>(a, ua.e, ua.row0, rpw, seg, sl, S, A);
    }

    // ---- setup: codebooks and work lists, once per workgroup -----------------
    const Lists L = lists_at(lds, a.list_offset, P);
    if (ids_held) {
        single_token_lists_held(L, my_id, P);
    } else if (one_token) {
        single_token_lists(L, a.ids, P);
    } else if (a.ids) {
        for (int q = tid; q < P; q += kThreads)
            L.ids[q] = a.ids[q];
    } else {
        for (int q = tid; q < P; q += kThreads) {
            L.items[q] = q;
            L.ids[q] = a.expert;
        }
        if (tid == 0) {
            L.ustart[0] = 0;
            L.ustart[1] = P;
            L.uexp[0] = a.expert;
            *L.U = 1;
        }
    }
    store_codebooks<D, BITS, NPROJ>(a, cr, lds);
    __syncthreads();
    if (a.ids && !one_token)
        build_lists(L, P);

    // Units are software-pipelined two deep: the rows of unit k+1 are in
    // flight while unit k is computed (buffers A and B alternate).
    // The current distinct expert's list entries are kept in (scalar)
    // registers: LDS is busy with the codebook lookups, so a unit of the same
    // expert reads it only to pick the pair when the expert serves several.
    int u = -1;
    int64_t u_end = 0;   // first unit past expert u
    int u0 = 0, nu = 1, ue = 0, uitem = 0;
    auto unit_at = [&](int64_t kk) {
        if (kk >= u_end) {
            do {
                ++u;
                u_end = (int64_t)L.ustart[u + 1] * a.tiles;
            } while (kk >= u_end);
            u0 = L.ustart[u];
            nu = L.ustart[u + 1] - u0;
            ue = L.uexp[u];
            uitem = L.items[u0];
        }
        const int64_t rel = kk - (int64_t)u0 * a.tiles;
        Unit un;
        un.e = ue;
        if (nu == 1) {
            un.item = uitem;
            un.row0 = (int)rel * a.tile_rows + wave * ITERS * rpw;
        } else {
            const int t = (int)udiv_small(rel, nu);
            un.item = L.items[u0 + (int)(rel - (int64_t)t * nu)];
            un.row0 = t * a.tile_rows + wave * ITERS * rpw;
        }
        return un;
    };
    int cur_item = -1;
    XRegs<GPL, HL> xr;
    auto run = [&](const Unit &un, const RowRegs<D, BITS, GPL, NPROJ>(&rr)[ITERS]) {
        if (un.item != cur_item) {
            XRaw<GPL, F32> xw;
            load_x_raw<GPL, F32>(a, un.item / a.act_div, sl, S, xw);
            convert_x<GPL, HL, F32>(xw, xr);
            cur_item = un.item;
        }
        compute_rows<D, BITS, GPL, NPROJ, HL, ITERS>(a, lds, rr, xr, un.item, S, seg, sl, un.row0,
                                                     rpw);
    };
    if (k >= k_end)
        return;
    if (!direct) {
        ua = unit_at(k);
        load_rows<D, BITS, GPL, NPROJ, ITERS>(a, ua.e, ua.row0, rpw, seg, sl, S, A);
    }
    for (;;) {
        const bool more_b = k + 1 < k_end;
        if (more_b) {
            ub = unit_at(k + 1);
            load_rows<D, BITS, GPL, NPROJ, ITERS>(a, ub.e, ub.row0, rpw, seg, sl, S, B);
        }
        run(ua, A);
        if (!more_b)
            break;
        ++k;
        const bool more_a = k + 1 < k_end;
        if (more_a) {
            ua = unit_at(k + 1);
            load_rows<D, BITS, GPL, NPROJ, ITERS>(a, ua.e, ua.row0, rpw, seg, sl, S, A);
        }
        run(ub, B);
        if (!more_a)
            break;
        ++k;
    }
}


// --------------------------------------------------------------------------------
// exact dequantize: one thread per (row, group)
// --------------------------------------------------------------------------------
template <int D, int BITS>
__global__ __launch_bounds__(256) void k_dequantize(const uint32_t *__restrict__ codes,
                                                    const uint16_t *__restrict__ scales,
                                                    const uint16_t *__restrict__ codebook,
                                                    const int32_t *__restrict__ row_map, int rows,
                                                    int groups, int wpr, int e, uint32_t kmax,
                                                    float *__restrict__ w)
{
    using GM = Geom<D, BITS>;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)rows * groups)
        return;
    const int r = (int)(i / groups);
    const int g = (int)(i % groups);
    float *out = w + (int64_t)r * groups * 64 + 64 * g;
    const int64_t s = stored_row(row_map, rows, e, r);
    if (s < 0) {
#pragma unroll
        for (int c = 0; c < 64; c += 4)
            *reinterpret_cast<float4 *>(out + c) = make_float4(0.f, 0.f, 0.f, 0.f);
        return;
    }
    uint32_t nw[GM::NW];
    load_group_words<D, BITS>(codes + s * wpr, g, nw);
    const float sc = half_bits_to_float(scales[s * groups + g]);
#pragma unroll
    for (int t = 0; t < GM::G; ++t) {
        // a code >= K (a precondition violation) reads entry K-1, never past
        // the codebook
        const uint32_t code = min(extract<BITS, GM::NW>(nw, t), kmax);
#pragma unroll
        for (int k = 0; k < D; ++k)
            out[t * D + k] = sc * half_bits_to_float(codebook[(int64_t)code * D + k]);
    }
}

// --------------------------------------------------------------------------------
// dispatch
// --------------------------------------------------------------------------------
template <int D, int BITS>
static hipError_t dequantize_db(const TensorDev &t, int e, float *w, hipStream_t stream)
{
    const int64_t n = (int64_t)t.rows * t.groups;
    const int blocks = (int)((n + 255) / 256);
    hipLaunchKernelGGL((k_dequantize<D, BITS>), dim3(blocks), dim3(256), 0, stream, t.codes,
                       t.scales, t.codebook, t.row_map, t.rows, t.groups, t.wpr, e,
                       (uint32_t)(t.K - 1), w);
    return hipGetLastError();
}

#define VQ_BITS_SWITCH(BITSV, FN, ...)                         \
    switch (BITSV) {                                           \
    case 8: return FN<8>(__VA_ARGS__);                         \
    case 9: return FN<9>(__VA_ARGS__);                         \
    case 10: return FN<10>(__VA_ARGS__);                       \
    case 11: return FN<11>(__VA_ARGS__);                       \
    case 12: return FN<12>(__VA_ARGS__);                       \
    case 13: return FN<13>(__VA_ARGS__);                       \
    default: return hipErrorInvalidValue;                      \
    }

template <int D>
struct DequantD {
    template <int BITS>
    static hipError_t run(const TensorDev &t, int e, float *w, hipStream_t s)
    {
        return dequantize_db<D, BITS>(t, e, w, s);
    }
};

template <int D>
hipError_t dequantize_d(const TensorDev &t, int e, float *w, hipStream_t s)
{
    VQ_BITS_SWITCH(t.bits, DequantD<D>::template run, t, e, w, s)
}

// --------------------------------------------------------------------------------
// down projection fused with the combine, for a few tokens, by output rows
// --------------------------------------------------------------------------------
// y[t][r] = sum over the (token, slot) pairs q of token t of
// w[q] * (W_down_{e_q} h_q)[r], added in a fixed order (distinct experts in
// first-occurrence order, then each expert's pairs in slot order).  A wave
// owns rpw output rows (one per segment of S lanes, each lane one 64-column
// group of the row, S >= groups) and walks the distinct routed experts: it
// streams each expert's rows once, with the next expert's words in flight,
// and applies them to every pair routed to that expert, adding the weighted
// products into per-(row, token) sums in LDS.  h is converted once per
// workgroup into range-scaled fp16 (a power of two per pair and group), the
// same activation format as the gate and up projections.
struct MixArgs {
    const uint32_t *codes;
    const uint16_t *scales;
    const int32_t *row_map;
    const uint16_t *codebook;
    int cb_dwords;
    int rows, groups, wpr;   // rows = hidden, groups = inter / 64
    int S_log2;
    const float *h;          // [P][inter]
    const int32_t *ids;      // [P]
    const float *w;          // [P]
    int n_tok, top_k;
    float *y;                // [n_tok][rows]
    int accumulate;          // 1: y += the combined sum (a residual stream)
    int list_offset, x_offset, m_offset, y_offset;   // LDS dword offsets
    int units;               // tiles of rpw rows
    int max_wgs;             // grid cap (a few workgroups per CU)
};

constexpr int kMixXStride = 36;   // dwords per (pair, group): 32 used, padded for ds_read_b128

// The engine of k_mix, in the pieces a caller runs in order: load_item(first)
// (optional, before the setup), the setup (stage_codebook, stage_lists,
// stage_h, finish_setup), then run().
//
// A workgroup walks tiles of rpw output rows (blockIdx.x, + gridDim.x,
// ...); its waves split the distinct experts into contiguous ranges of at
// most per = ceil(U / waves), taken CH (2 or 4) at a time: the launch picks
// the smaller when no wave has more than two experts, so no load slot of a
// batch is spent on a repeated expert.  Work item i of a
// wave is (tile i / nch, chunk i % nch); the words of item i+1 are in flight
// while item i is computed.  For a single token the experts are the ids
// themselves, so the first item can be requested before the setup and its
// memory latency overlaps it.
template <int D, int BITS, int CH>
struct MixEngine {
    static constexpr int kMixChunk = CH;   // experts whose rows are loaded together
    using GM = Geom<D, BITS>;
    static constexpr int NW = GM::NW;
    static constexpr int G = GM::G;
    static constexpr int HP = D / 2;
    struct Chunk {
        uint32_t wd[kMixChunk][NW];
        uint32_t sc[kMixChunk];
        int live;
    };

    const MixArgs &a;
    uint32_t *lds;
    int tid, lane, wave, P, S, rpw, seg, sl, g;
    bool gok, one;
    Lists L;
    int my_units;
    int ub = 0, ue = 0, nch = 1;

    __device__ __forceinline__ MixEngine(const MixArgs &args, uint32_t *l) : a(args), lds(l)
    {
        tid = threadIdx.x;
        lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: expert ids load as scalars
        P = a.n_tok * a.top_k;
        S = 1 << a.S_log2;
        rpw = 64 >> a.S_log2;
        seg = lane >> a.S_log2;
        sl = lane & (S - 1);
        g = min(sl, a.groups - 1);
        gok = sl < a.groups;
        one = a.n_tok == 1;
        L = lists_at(lds, a.list_offset, P);
        my_units = (int)blockIdx.x < a.units
                       ? (a.units - 1 - (int)blockIdx.x) / (int)gridDim.x + 1
                       : 0;
        if (one)
            wave_range(P);
    }

    __device__ __forceinline__ void wave_range(int U)
    {
        const int per = (U + kWaves - 1) / kWaves;
        ub = min(wave * per, U);
        ue = min(ub + per, U);
        nch = max(1, (per + kMixChunk - 1) / kMixChunk);   // the same for every wave
    }

    __device__ __forceinline__ int n_items() const { return my_units * nch; }

    // The experts of an item's chunk (entries past the wave's range repeat
    // its last expert and are skipped).
    __device__ __forceinline__ void experts_of(int item, int (&e)[kMixChunk]) const
    {
        const int u0 = ub + (item % nch) * kMixChunk;
#pragma unroll
        for (int c = 0; c < kMixChunk; ++c) {
            const int u = max(min(u0 + c, ue - 1), 0);
            e[c] = one ? load_global(a.ids + u) : L.uexp[u];
        }
    }

    __device__ __forceinline__ void load_item(Chunk &ck, int item) const
    {
        int e[kMixChunk];
        experts_of(item, e);
        load_item(ck, item, e);
    }

    __device__ __forceinline__ void load_item(Chunk &ck, int item, const int (&e)[kMixChunk]) const
    {
        if (a.row_map)
            load_item_m<true>(ck, item, e);
        else
            load_item_m<false>(ck, item, e);
    }

    // every load unconditional; MAP: the stored rows come from the row map
    // (without one no load waits for loads issued earlier)
    template <bool MAP>
    __device__ __forceinline__ void load_item_m(Chunk &ck, int item,
                                                const int (&e)[kMixChunk]) const
    {
        const int unit = blockIdx.x + (item / nch) * gridDim.x;
        const int r = unit * rpw + seg;
        const bool rok = r < a.rows;
        int64_t srow[kMixChunk];
#pragma unroll
        for (int c = 0; c < kMixChunk; ++c) {
            const int64_t lin = (int64_t)e[c] * a.rows + min(r, a.rows - 1);
            srow[c] = MAP ? a.row_map[lin] : lin;
        }
        ck.live = 0;
#pragma unroll
        for (int c = 0; c < kMixChunk; ++c) {
            const bool lv = rok && (srow[c] >= 0);
            ck.live |= lv ? (1 << c) : 0;
            const int64_t sr = lv ? srow[c] : 0;
            const uint32_t *row = a.codes + sr * a.wpr;
            const int w0 = (g * GM::GB) >> 5;
            if constexpr (GM::CLAMP) {
#pragma unroll
                for (int k = 0; k < NW; ++k)
                    ck.wd[c][k] = row[min(w0 + k, a.wpr - 1)];
            } else {
                __builtin_memcpy(ck.wd[c], row + w0, NW * 4);
            }
            ck.sc[c] = a.scales[sr * a.groups + g];
        }
    }

    // ---- setup: codebook, routing lists, h as range-scaled fp16 pairs ------------
    __device__ __forceinline__ void stage_codebook() const
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(a.codebook);
        const int n4 = a.cb_dwords >> 2;
        for (int i = tid; i < n4; i += kThreads)
            reinterpret_cast<uint4 *>(lds)[i] = src[i];
        const uint32_t *s32 = reinterpret_cast<const uint32_t *>(a.codebook);
        for (int i = (n4 << 2) + tid; i < a.cb_dwords; i += kThreads)
            lds[i] = s32[i];
    }

    __device__ __forceinline__ void stage_lists() const
    {
        if (one)
            single_token_lists(L, a.ids, P);
        else
            for (int q = tid; q < P; q += kThreads)
                L.ids[q] = a.ids[q];
    }

    // h as range-scaled fp16 pairs.  The 64 floats of a (pair, group) are
    // read by 16 consecutive lanes, 16 bytes each, their largest magnitude
    // found across those lanes, and each lane writes its four values as two
    // fp16 pairs.  Up to kHPasses passes of 16 (pair, group)s per workgroup
    // have their loads in flight together.
    static constexpr int kPerPass = kThreads / 16;
    static constexpr int kHPasses = 8;
    __device__ __forceinline__ int h_items() const { return P * a.groups; }
    __device__ __forceinline__ void h_load(int base, float4 (&v)[kHPasses]) const
    {
        const int n = h_items();   // (pair, group) items; item i is h[64 i, 64 i + 64)
        const int piece = tid & 15;
#pragma unroll
        for (int j = 0; j < kHPasses; ++j) {
            const int it = min(base + j * kPerPass + (tid >> 4), n - 1);
            const float4 *src = reinterpret_cast<const float4 *>(a.h) + (size_t)it * 16 + piece;
            v[j] = *src;
        }
    }
    __device__ __forceinline__ void h_store(int base, const float4 (&v)[kHPasses]) const
    {
        uint32_t *xs = lds + a.x_offset;                           // [P][groups][kMixXStride]
        float *xm = reinterpret_cast<float *>(lds + a.m_offset);   // [P][groups]
        const int n = h_items();
        const int piece = tid & 15;
#pragma unroll
        for (int j = 0; j < kHPasses; ++j) {
            const int it = base + j * kPerPass + (tid >> 4);
            const float m4 = fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)),
                                   fmaxf(fabsf(v[j].z), fabsf(v[j].w)));
            const int k = range_exponent(segment_max16_dpp(m4));
            const float up = ldexpf(1.0f, k);
            union { f16x2 h[2]; uint2 u; } o;
            o.h[0] = pack_f16x2(v[j].x * up, v[j].y * up);
            o.h[1] = pack_f16x2(v[j].z * up, v[j].w * up);
            if (it < n) {
                *reinterpret_cast<uint2 *>(xs + (size_t)it * kMixXStride + 2 * piece) = o.u;
                if (piece == 0)
                    xm[it] = ldexpf(1.0f, -k);
            }
        }
    }
    __device__ __forceinline__ void stage_h(int from = 0) const
    {
        for (int base = from; base < h_items(); base += kPerPass * kHPasses) {
            float4 v[kHPasses];
            h_load(base, v);
            h_store(base, v);
        }
    }

    // One token: the setup's loads (the codebook in up to kEarlyCb 16-byte
    // pieces a thread, the pairs' expert ids, the first pass of h) issued
    // before the first item's rows, so they return ahead of them (loads
    // return in issue order) and the setup is written while the rows are in
    // flight.
    static constexpr int kEarlyCb = 4;
    struct Early {
        uint4 cb[kEarlyCb];
        int id;
        float4 h[kHPasses];
    };
    __device__ __forceinline__ bool early_ok() const
    {
        return one && P <= kThreads && (a.cb_dwords & 3) == 0 &&
               (a.cb_dwords >> 2) <= kEarlyCb * kThreads;
    }
    __device__ __forceinline__ void early_load(Early &x) const
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(a.codebook);
        const int n4 = a.cb_dwords >> 2;
#pragma unroll
        for (int j = 0; j < kEarlyCb; ++j) {
            const int i = tid + j * kThreads;
            x.cb[j] = i < n4 ? src[i] : make_uint4(0u, 0u, 0u, 0u);
        }
        x.id = tid < P ? load_global(a.ids + tid) : 0;
        h_load(0, x.h);
    }
    __device__ __forceinline__ void early_store(const Early &x) const
    {
        const int n4 = a.cb_dwords >> 2;
#pragma unroll
        for (int j = 0; j < kEarlyCb; ++j) {
            const int i = tid + j * kThreads;
            if (i < n4)
                reinterpret_cast<uint4 *>(lds)[i] = x.cb[j];
        }
        single_token_lists_held(L, x.id, P);
        h_store(0, x.h);
        stage_h(kPerPass * kHPasses);
    }

    // After the stage_* calls: lists for several tokens and the waves' ranges.
    __device__ __forceinline__ void finish_setup()
    {
        __syncthreads();
        if (!one) {
            build_lists(L, P);
            wave_range(*L.U);
        }
    }

    // ---- the work items ----------------------------------------------------------------
    // yacc[w][row][t]: wave w's partial sums of the current tile, added in
    // wave order when the tile is done
    __device__ __forceinline__ void process(const Chunk &ck, int item) const
    {
        const uint32_t *xs = lds + a.x_offset;
        const float *xm = reinterpret_cast<const float *>(lds + a.m_offset);
        float *yall = reinterpret_cast<float *>(lds + a.y_offset);
        float *yacc = yall + wave * 64 * a.n_tok;
        const int tile = item / nch;
        const int ch = item - tile * nch;
        const int unit = blockIdx.x + tile * gridDim.x;
        const int u0 = ub + ch * kMixChunk;
        if (ch == 0)
            for (int t = sl; t < a.n_tok; t += S)
                yacc[seg * a.n_tok + t] = 0.0f;
#pragma unroll
        for (int c = 0; c < kMixChunk; ++c) {
            if (u0 + c >= ue)
                break;
            const int u = u0 + c;
            uint32_t nw[NW];
            shift_group_words<D, BITS>(g, ck.wd[c], nw);
            const bool lv = (ck.live >> c) & 1;
            const float sf = (lv && gok) ? half_bits_to_float(ck.sc[c]) : 0.0f;
            for (int i = L.ustart[u]; i < L.ustart[u + 1]; ++i) {
                const int q = L.items[i];
                const uint4 *xp =
                    reinterpret_cast<const uint4 *>(xs + (size_t)(q * a.groups + g) * kMixXStride);
                union { uint4 u[8]; f16x2 h[32]; } x;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    x.u[j] = xp[j];
                float acc = 0.0f;
#pragma unroll
                for (int t = 0; t < G; ++t) {
                    const uint32_t code = extract<BITS, NW>(nw, t);
                    const Entry<D> en = fetch_entry<D>(lds, code);
#pragma unroll
                    for (int k = 0; k < HP; ++k)
                        acc = dot2(en.v[k], x.h[t * HP + k], acc);
                }
                const float part = segment_sum_dpp(acc * (sf * xm[q * a.groups + g]), S);
                if (sl == 0 && lv)
                    yacc[seg * a.n_tok + q / a.top_k] += a.w[q] * part;
            }
        }
        if (ch == nch - 1) {
            __syncthreads();
            // wave order fixes the order of the sums
            for (int i = tid; i < rpw * a.n_tok; i += kThreads) {
                const int rr = unit * rpw + i / a.n_tok;
                const int t = i - (i / a.n_tok) * a.n_tok;
                float v = 0.0f;
#pragma unroll
                for (int w = 0; w < kWaves; ++w)
                    v += yall[w * 64 * a.n_tok + i];
                if (rr < a.rows) {
                    float *yp = a.y + (int64_t)t * a.rows + rr;
                    *yp = a.accumulate ? *yp + v : v;
                }
            }
            __syncthreads();
        }
    }

    // ca holds item 0 if preloaded; items alternate between ca and cb
    __device__ __forceinline__ void run(Chunk &ca, Chunk &cb, bool preloaded) const
    {
        const int n = n_items();
        if (n == 0)
            return;
        if (!preloaded)
            load_item(ca, 0);
        for (int i = 0; i < n; i += 2) {
            if (i + 1 < n)
                load_item(cb, i + 1);
            process(ca, i);
            if (i + 1 >= n)
                break;
            if (i + 2 < n)
                load_item(ca, i + 2);
            process(cb, i + 1);
        }
    }
};

template <int D, int BITS, int CH>
__global__ __launch_bounds__(kThreads) void k_mix(const MixArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
    MixEngine<D, BITS, CH> m(a, lds);
    typename MixEngine<D, BITS, CH>::Chunk ca, cb;
    const bool pre = m.one && m.my_units > 0;
    if (pre && m.early_ok()) {
        typename MixEngine<D, BITS, CH>::Early x;
        m.early_load(x);
        m.load_item(ca, 0);
        m.early_store(x);
    } else {
        if (pre)
            m.load_item(ca, 0);
        m.stage_codebook();
        m.stage_lists();
        m.stage_h();
    }
    m.finish_setup();
    m.run(ca, cb, pre);
}

template <int D, int BITS, int CH>
static hipError_t mix_dbc(const MixArgs &a, size_t lds, hipStream_t stream)
{
    auto kern = k_mix<D, BITS, CH>;
    if (lds > 65536) {
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess)
            return err;
    }
    // a few tiles per workgroup amortise staging h
    const int wgs = a.units < a.max_wgs ? a.units : a.max_wgs;
    hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
}

// Experts per load batch: two when one token's pairs leave every wave at
// most two experts, else four.
template <int D, int BITS>
static hipError_t mix_db(const MixArgs &a, size_t lds, hipStream_t stream)
{
    const int P = a.n_tok * a.top_k;
    if (a.n_tok == 1 && (P + kWaves - 1) / kWaves <= 2)
        return mix_dbc<D, BITS, 2>(a, lds, stream);
    return mix_dbc<D, BITS, 4>(a, lds, stream);
}

template <int D>
struct MixD {
    template <int BITS>
    static hipError_t run(const MixArgs &a, size_t lds, hipStream_t s)
    {
        return mix_db<D, BITS>(a, lds, s);
    }
};

template <int D>
hipError_t mix_d(int bits, const MixArgs &a, size_t lds, hipStream_t s)
{
    VQ_BITS_SWITCH(bits, MixD<D>::template run, a, lds, s)
}


// The persistent grid is as many workgroups as can be resident at once
// (occupancy of this instantiation at this LDS size, times the CU count),
// capped by the number of work units.
template <int D, int BITS, int GPL, int NPROJ, bool HL, bool F32, int ITERS>
static hipError_t rows_launch(const RowsArgs &a, int64_t units, int n_cu, size_t lds_bytes,
                              hipStream_t stream)
{
    auto kern = k_rows<D, BITS, GPL, NPROJ, HL, F32, ITERS>;
    if (lds_bytes > 65536) {
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)lds_bytes);
        if (err != hipSuccess)
            return err;
    }
    int per_cu = 0;
    hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void *>(kern), kThreads, lds_bytes);
    if (err != hipSuccess || per_cu < 1)
        per_cu = 1;
    const int64_t cap = (int64_t)per_cu * n_cu;
    const dim3 grid((unsigned)(units < cap ? units : cap));
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds_bytes, stream, a);
    return hipGetLastError();
}

// act: 0 bf16 activations; 1 fp32 ones, whose low bits ride along as a
// second fp16 term; 2 fp32 ones rounded once to fp16 (one projection: the
// down projection of h)
template <int D, int BITS, int GPL, int NPROJ, int ITERS>
static hipError_t rows_iters(const RowsArgs &a, int act, int64_t units, int n_cu, size_t lds,
                             hipStream_t s)
{
    if constexpr (NPROJ == 1) {
        if (act == 2)
            return rows_launch<D, BITS, GPL, NPROJ, false, true, ITERS>(a, units, n_cu, lds, s);
    }
    if (act != 0)
        return rows_launch<D, BITS, GPL, NPROJ, true, true, ITERS>(a, units, n_cu, lds, s);
    return rows_launch<D, BITS, GPL, NPROJ, false, false, ITERS>(a, units, n_cu, lds, s);
}

// one or two row passes per unit (a.iters)
template <int D, int BITS, int GPL, int NPROJ>
static hipError_t rows_act(const RowsArgs &a, int act, int64_t units, int n_cu, size_t lds,
                           hipStream_t s)
{
    if (a.iters == 1)
        return rows_iters<D, BITS, GPL, NPROJ, 1>(a, act, units, n_cu, lds, s);
    if constexpr (NPROJ == 1) {
        if (a.iters == 4)
            return rows_iters<D, BITS, GPL, NPROJ, 4>(a, act, units, n_cu, lds, s);
    }
    return rows_iters<D, BITS, GPL, NPROJ, 2>(a, act, units, n_cu, lds, s);
}

template <int D, int BITS>
static hipError_t rows_db(const RowsArgs &a, int gpl, int nproj, int act_f32, int64_t units,
                          int n_cu, size_t lds, hipStream_t s)
{
    if (gpl == 1)
        return nproj == 2 ? rows_act<D, BITS, 1, 2>(a, act_f32, units, n_cu, lds, s)
                          : rows_act<D, BITS, 1, 1>(a, act_f32, units, n_cu, lds, s);
    return nproj == 2 ? rows_act<D, BITS, 2, 2>(a, act_f32, units, n_cu, lds, s)
                      : rows_act<D, BITS, 2, 1>(a, act_f32, units, n_cu, lds, s);
}

template <int D>
struct RowsD {
    template <int BITS>
    static hipError_t run(const RowsArgs &a, int gpl, int nproj, int f32, int64_t units, int n_cu,
                          size_t lds, hipStream_t s)
    {
        return rows_db<D, BITS>(a, gpl, nproj, f32, units, n_cu, lds, s);
    }
};

template <int D>
hipError_t rows_d(int bits, const RowsArgs &a, int gpl, int nproj, int f32, int64_t units,
                  int n_cu, size_t lds, hipStream_t s)
{
    VQ_BITS_SWITCH(bits, RowsD<D>::template run, a, gpl, nproj, f32, units, n_cu, lds, s)
}

}  // namespace vq
