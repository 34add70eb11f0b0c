// vq_prefill_impl.hpp -- grouped MFMA GEMM over VQ expert weights (gfx950).
//
// For a batch of many tokens every routed expert sees a block of rows, and
// the expert matmul becomes a ragged grouped GEMM (the model cards' runtime
// dequantises in chunks before its prefill matmul: card
// "gemma-4-26b-a4b-it-VQ-6.2bpw", section "Runtime"; large codebooks get a
// dedicated kernel arm: card "Qwen3.5-397B-A17B-VQ-2.4bpw", changelog
// 2026-09-09).  Here:
//
//   * a workgroup owns one tile (expert, up to 32*MB of its grouped rows)
//     and 32 weight rows per wave; a wave's weight rows are of one
//     projection or of gate and up together (the SwiGLU product is formed in
//     the epilogue);
//   * the K loop walks 64-column groups through a ring of S stages in LDS,
//     filled by direct global->LDS loads (no register staging): the tile's
//     activation rows (fp16, already range-scaled) and every lane's own
//     packed-code window and scale.  A stage is issued S-1 groups ahead;
//   * the weights never exist as a dequantised tile: each lane decodes
//     exactly its own v_mfma_f32_32x32x16_f16 B operand from its code window
//     (codebook lookups in LDS, fp16 scale applied with packed multiplies),
//     one group ahead of the MFMAs that consume it;
//   * MFMA K order: in slice j of a group, lanes of half h supply columns
//     32h + 8j + [0, 8), so a lane's codes are one contiguous run of the row
//     (the same K permutation is applied to both operands, so the product
//     is unchanged);
//   * activation rows are 128 bytes per group in LDS with their 16-byte
//     chunks XOR-swizzled by row, so the fragment reads are conflict-free.
#pragma once

#include "vq_common.hpp"
#include "vq_internal.hpp"

#include <type_traits>

namespace vq {

constexpr int kLdsBudget = 160 * 1024;   // LDS of one gfx950 CU

typedef __attribute__((address_space(3))) void lds_void_t;

// Direct global -> LDS load of SIZE bytes per lane: lane l of the wave
// writes at lds_wave_base + l * SIZE, except that 12-byte loads keep a
// 16-byte lane stride (lds_wave_base must be wave-uniform).  Issued as inline assembly: the ring below tracks these loads with its own
// vmcnt waits, so the compiler must not add blanket waits of its own before
// every LDS read.  The instruction has no register results.
// The 32-bit LDS address of a pointer into LDS.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const lds_void_t *)p;
}

// lds_wave_base: a wave-uniform LDS address, best computed from uniform
// values only, so that it stays in scalar registers.
template <int SIZE>
__device__ __forceinline__ void dma(const void *src, uint32_t lds_wave_base)
{
    static_assert(SIZE == 4 || SIZE == 12 || SIZE == 16, "unsupported load size");
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_wave_base);
    if constexpr (SIZE == 16)
        asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(m0) : "memory");
    else if constexpr (SIZE == 12)
        asm volatile("global_load_lds_dwordx3 %0, off" : : "v"(src), "{m0}"(m0) : "memory");
    else
        asm volatile("global_load_lds_dword %0, off" : : "v"(src), "{m0}"(m0) : "memory");
}

// s_waitcnt vmcnt(N): at most N vector-memory operations of this wave are
// still outstanding (they complete in issue order).  The memory clobber
// keeps LDS reads below it.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt out of range");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// s_waitcnt lgkmcnt(0): this wave's LDS writes are done.
__device__ __forceinline__ void wait_lds()
{
    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
}

// Workgroup barrier with no implied memory waits (the waits above are
// explicit); the memory clobber keeps LDS accesses on their side of it.
__device__ __forceinline__ void barrier()
{
    asm volatile("s_barrier" : : : "memory");
}

// Calls f(integral_constant<int, i>) for i = 0 .. N-1.
template <int... I, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, I...>, F &&f)
{
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

// The packed-code window of one lane: codes CL*h + [0, CL) of a group
// (columns 32h + [0, 32)).
template <int D, int BITS>
struct BWin {
    static constexpr int G = 64 / D;          // codes per group
    static constexpr int CL = G / 2;          // codes per lane
    static constexpr int PER = 8 / D;         // codes per 16-column slice
    static constexpr int NBITS = CL * BITS;
    static constexpr int omax()
    {
        int m = 0;
        for (int g = 0; g < 32; ++g)
            for (int h = 0; h < 2; ++h) {
                const int o = (g * G * BITS + h * NBITS) & 31;
                m = o > m ? o : m;
            }
        return m;
    }
    static constexpr int NW = (omax() + NBITS + 31) / 32;   // words per window
    static constexpr int N16 = NW / 4;                      // 16-byte pieces
    static constexpr int TAIL = NW % 4;                     // words after them
    // direct loads per window: the 16-byte pieces, then one 12-byte or
    // single-word ones.  A 12-byte load still places lane l at 16*l.
    static constexpr int NDMA = N16 + (TAIL == 3 ? 1 : TAIL);
    static constexpr int LDS_BYTES = N16 * 16 + (TAIL == 3 ? 16 : 4 * TAIL);   // per lane
};

struct GemmArgs {
    const uint32_t *codes[2];
    const uint16_t *scales[2];
    const int32_t *row_map[2];     // with one projection, [1] may hold gate's map (split SwiGLU)
    const uint16_t *codebook[2];
    int cb_bytes[2];
    int rows, groups, wpr;
    const f16 *act;                // range-scaled fp16 activation rows
    int act_stride;                // halves between rows
    const int32_t *act_k;          // scaling exponent of each activation row
    const int32_t *perm;           // grouped position -> source index (NULL: identity)
    int act_div;                   // activation row = source index / act_div
    const int32_t *tiles;          // [n][3]: expert, first grouped position, rows
    const int32_t *n_tiles;
    int n_ntiles;                  // weight-row tiles per M tile
    const float *gate_in;          // split SwiGLU: gate outputs for this up projection
    float *out;
    int64_t out_stride;
};

template <int D, int BITS, int NPROJ, int MB, int WAVES>
struct GemmShape {
    static constexpr int NT = 64 * WAVES;
    // 32-row weight blocks per wave: two (each activation fragment read from
    // LDS then feeds 2*NPROJ MFMAs) unless the accumulators would not fit
    static constexpr int NN = (NPROJ * 2 * MB * 16 <= 256) ? 2 : 1;
    static constexpr int NPB = NPROJ * NN;                       // (projection, block) pairs
    static constexpr int WG_ROWS = 32 * NN * WAVES;              // weight rows per workgroup
    static constexpr int RPD = NT / 8;                           // tile rows per A load
    static constexpr int NDMA_A = (32 * MB + RPD - 1) / RPD;
    static constexpr int A_BYTES = NDMA_A * NT * 16;
    static constexpr int WIN = NT * (BWin<D, BITS>::LDS_BYTES + 4);   // one (projection, block)
    static constexpr int STAGE = A_BYTES + NPB * WIN;
    // vector-memory operations per stage and wave: scales, code windows, activations
    static constexpr int NOPS = NDMA_A + NPB * (BWin<D, BITS>::NDMA + 1);
    // LDS, one static array from address 0: a slot per codebook of the
    // largest size (64 KiB at most each), the tile's row factors, then the
    // ring; four stages when they fit
    static constexpr int CB_MAX = ((1 << BITS) * D * 2 < 65536) ? (1 << BITS) * D * 2 : 65536;
    static constexpr int KF_OFF = NPROJ * CB_MAX;
    static constexpr int FIXED = KF_OFF + 32 * MB * 4;   // a multiple of 16: the ring's offset
    static constexpr int S = (FIXED + 4 * STAGE <= kLdsBudget) ? 4 : 3;
    static constexpr bool FITS = FIXED + S * STAGE <= kLdsBudget;
};

// The K step's interleave: after each MFMA, up to this many LDS reads and
// VALU instructions (a sweep of 1-3 LDS reads and 2-4 VALU on the full-size
// gate+up layers put two and three ahead, by about 1 %).
constexpr int kSchedDs = 2;
constexpr int kSchedValu = 3;

template <int D, int BITS, int NPROJ, int MB, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_gemm(const GemmArgs a)
{
    using BW = BWin<D, BITS>;
    using SH = GemmShape<D, BITS, NPROJ, MB, WAVES>;
    constexpr int NT = SH::NT;
    constexpr int NW = BW::NW;
    constexpr int S = SH::S;
    constexpr int NN = SH::NN;
    constexpr int NPB = SH::NPB;
    if constexpr (SH::FITS) {
    // codebook slots and row factors, then the ring of S stages, in the
    // kernel's only LDS array: the slots sit at fixed addresses, which the
    // codebook reads carry as immediate offsets
    __shared__ __attribute__((aligned(16))) char smem[SH::FIXED + S * SH::STAGE];
    char *const lb = smem;
    char *const ring = smem + SH::FIXED;
    const uint32_t lb_l = lds_addr(lb);     // LDS addresses of the two regions
    const uint32_t ring_l = lds_addr(ring);
    auto cb_slot = [](int p) { return p == 0 ? 0 : SH::CB_MAX; };

    // Workgroup L runs on XCD L % 8 (round-robin dispatch); all weight-row
    // tiles of M tile t run on XCD t % 8 one after another, so the tile's
    // activation rows are fetched into that XCD's L2 once.
    const int L = blockIdx.x;
    const int slot = L >> 3;
    const int tile = (slot / a.n_ntiles) * 8 + (L & 7);
    const int ntile = slot - (slot / a.n_ntiles) * a.n_ntiles;
    if (tile >= *a.n_tiles)
        return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS bases in SGPRs
    const int h = lane >> 5;
    const int e = a.tiles[3 * tile + 0];
    const int m0 = a.tiles[3 * tile + 1];
    const int mlen = a.tiles[3 * tile + 2];
    const int nblk = (mlen + 31) >> 5;
    // weight row of block nb of this lane: nrow0 + 32 * nb
    const int nrow0 = ntile * SH::WG_ROWS + wave * 32 * NN + (lane & 31);
    const int G = a.groups;

    // ---- prologue: codebooks, row factors, per-lane sources ------------------------
#pragma unroll
    for (int p = 0; p < NPROJ; ++p) {
        const char *src = reinterpret_cast<const char *>(a.codebook[p]);
        char *dst = lb + cb_slot(p);
        const uint32_t dst_l = lb_l + (uint32_t)cb_slot(p);
        const int n16 = a.cb_bytes[p] >> 4;
        for (int i0 = 0; i0 < n16; i0 += NT)
            if (i0 + tid < n16)
                dma<16>(src + (size_t)(i0 + tid) * 16, dst_l + (uint32_t)(i0 + wave * 64) * 16u);
        for (int i = (n16 << 2) + tid; i < (a.cb_bytes[p] >> 2); i += NT)
            reinterpret_cast<uint32_t *>(dst)[i] = reinterpret_cast<const uint32_t *>(src)[i];
    }
    float *kf = reinterpret_cast<float *>(lb + SH::KF_OFF);
    for (int r = tid; r < 32 * MB; r += NT) {
        const int p = m0 + min(r, mlen - 1);
        const int row = a.perm ? a.perm[p] / a.act_div : p;
        kf[r] = ldexpf(1.0f, -a.act_k[row]);
    }
    // activation rows: thread tid of load q fills tile row q*RPD + tid/8,
    // LDS chunk tid%8 with global chunk (tid%8) ^ (row%8)
    uint32_t aoff[SH::NDMA_A];
#pragma unroll
    for (int q = 0; q < SH::NDMA_A; ++q) {
        const int r = q * SH::RPD + (tid >> 3);
        const int p = m0 + min(r, mlen - 1);
        const int row = a.perm ? a.perm[p] / a.act_div : p;
        const int chunk = (tid & 7) ^ ((tid >> 3) & 7);
        aoff[q] = (uint32_t)row * (uint32_t)a.act_stride * 2u + (uint32_t)chunk * 16u;
    }
    // weight rows, per (projection p, block nb): index pb = p * NN + nb
    const uint32_t *brow[NPB];
    const uint16_t *srow[NPB];
    int live = 0;
#pragma unroll
    for (int p = 0; p < NPROJ; ++p) {
#pragma unroll
        for (int nb = 0; nb < NN; ++nb) {
            const int n = nrow0 + 32 * nb;
            const int64_t lin = (int64_t)e * a.rows + min(n, a.rows - 1);
            const int s = a.row_map[p] ? a.row_map[p][lin] : (int)lin;
            bool lv = (n < a.rows) && (s >= 0);
            if (NPROJ == 1 && a.gate_in && a.row_map[1] && a.row_map[1][lin] < 0)
                lv = false;   // split SwiGLU: a dead gate row gives h = +0.0
            const int pb = p * NN + nb;
            live |= lv ? (1 << pb) : 0;
            const int64_t sr = lv ? s : 0;
            brow[pb] = a.codes[p] + sr * a.wpr;
            srow[pb] = a.scales[p] + sr * a.groups;
        }
    }

    // ---- loads of one stage, one instruction per unit: per (projection, block)
    // the scale and the code window, then the activation rows ---------------------------
    constexpr int PB = BW::NDMA + 1;                     // loads per (projection, block)
    auto dma_unit = [&](auto Q, int gg, uint32_t sb) {
        constexpr int q = decltype(Q)::value;
        if constexpr (q < NPB * PB) {
            constexpr int pb = q / PB, r = q % PB;
            const uint32_t bb = sb + SH::A_BYTES + pb * SH::WIN;
            if constexpr (r == 0) {
                // the aligned dword holding the scale (it never crosses a page)
                const uintptr_t sp = reinterpret_cast<uintptr_t>(srow[pb] + gg);
                dma<4>(reinterpret_cast<const void *>(sp & ~(uintptr_t)3), bb + wave * 64 * 4);
            } else {
                const int sbit = gg * BW::G * BITS + h * BW::NBITS;
                const int ws = min(sbit >> 5, a.wpr - NW);   // window kept inside the row
                const uint32_t *wp = brow[pb] + ws;
                constexpr int c = r - 1;
                if constexpr (c < BW::N16)
                    dma<16>(wp + 4 * c, bb + NT * 4 + c * NT * 16 + wave * 64 * 16);
                else if constexpr (BW::TAIL == 3)
                    dma<12>(wp + 4 * c, bb + NT * 4 + c * NT * 16 + wave * 64 * 16);
                else
                    dma<4>(wp + 4 * BW::N16 + (c - BW::N16),
                           bb + NT * 4 + BW::N16 * NT * 16 + (c - BW::N16) * NT * 4 + wave * 64 * 4);
            }
        } else {
            constexpr int qa = q - NPB * PB;
            dma<16>(reinterpret_cast<const char *>(a.act) + (size_t)gg * 128 + aoff[qa],
                    sb + qa * NT * 16 + wave * 1024);
        }
    };
    auto issue_all = [&](int gg, uint32_t sb) {
        static_for<SH::NOPS>([&](auto Q) { dma_unit(Q, gg, sb); });
    };

    // ---- decoding this lane's B operands, in pieces -----------------------------------
    struct Raw {
        uint32_t w[NW];
        uint32_t sw;
    };
    // raw: the scale dword and code words of (projection, block) pb
    auto read_raw = [&](int pb, const char *sb, Raw &rw) {
        const char *bb = sb + SH::A_BYTES + pb * SH::WIN;
        rw.sw = *reinterpret_cast<const uint32_t *>(bb + tid * 4);
        bb += NT * 4;
#pragma unroll
        for (int k = 0; k < BW::N16; ++k) {
            const uint4 v = *reinterpret_cast<const uint4 *>(bb + tid * 16);
            rw.w[4 * k] = v.x;
            rw.w[4 * k + 1] = v.y;
            rw.w[4 * k + 2] = v.z;
            rw.w[4 * k + 3] = v.w;
            bb += NT * 16;
        }
        if constexpr (BW::TAIL == 3) {
            const uint4 v = *reinterpret_cast<const uint4 *>(bb + tid * 16);
            rw.w[4 * BW::N16] = v.x;
            rw.w[4 * BW::N16 + 1] = v.y;
            rw.w[4 * BW::N16 + 2] = v.z;
        } else {
#pragma unroll
            for (int k = 0; k < BW::TAIL; ++k)
                rw.w[4 * BW::N16 + k] = *reinterpret_cast<const uint32_t *>(bb + tid * 4 + k * NT * 4);
        }
    };
    // shift: the words realigned so the lane's first code is at bit 0, and
    // the (s, s) multiplier (0 for a dead row)
    auto shift_raw = [&](int pb, int gg, const Raw &rw, uint32_t (&nw)[NW], f16x2 &s2) {
        const int sbit = gg * BW::G * BITS + h * BW::NBITS;
        const int w0 = sbit >> 5;
        const int delta = w0 - min(w0, a.wpr - NW);   // > 0 only near a row's end
        const int o = sbit & 31;
        uint32_t w[NW];
#pragma unroll
        for (int i = 0; i < NW; ++i)
            w[i] = rw.w[i];
        if (__builtin_expect(delta != 0, 0)) {
            // the window was pulled back to stay inside the row
            uint32_t t[NW];
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                uint32_t v = w[NW - 1];
#pragma unroll
                for (int d = NW - 1; d >= 1; --d)
                    if (i + d < NW)
                        v = (delta == d) ? w[i + d] : v;
                t[i] = v;
            }
#pragma unroll
            for (int i = 0; i < NW; ++i)
                w[i] = t[i];
        }
#pragma unroll
        for (int i = 0; i < NW; ++i)
            nw[i] = __builtin_amdgcn_alignbit(i + 1 < NW ? w[i + 1] : 0u, w[i], o);
        const bool hi = (reinterpret_cast<uintptr_t>(srow[pb] + gg) & 2) != 0;
        const uint32_t sc = (live >> pb & 1) ? (hi ? rw.sw >> 16 : rw.sw & 0xffffu) : 0u;
        union { uint32_t u; f16x2 h; } c2;
        c2.u = sc * 0x10001u;
        s2 = c2.h;
    };
    // lookup: the codebook entries of slice j (unscaled)
    auto lookup = [&](int p, int j, const uint32_t (&nw)[NW], f16x8 &o) {
        const uint32_t *cb = reinterpret_cast<const uint32_t *>(lb + cb_slot(p));
        constexpr uint32_t mask = (1u << BITS) - 1u;
        union { f16x8 v; uint32_t u[4]; } r;
#pragma unroll
        for (int c = 0; c < BW::PER; ++c) {
            const int t = j * BW::PER + c;
            const int pbit = t * BITS;
            const int wi = pbit >> 5, bsh = pbit & 31;
            const uint32_t code = (bsh + BITS <= 32)
                                      ? __builtin_amdgcn_ubfe(nw[wi], bsh, BITS)
                                      : (__builtin_amdgcn_alignbit(nw[wi + 1], nw[wi], bsh) & mask);
            if constexpr (D == 2) {
                r.u[c] = cb[code];
            } else if constexpr (D == 4) {
                const uint2 q = *reinterpret_cast<const uint2 *>(cb + 2 * code);
                r.u[2 * c] = q.x;
                r.u[2 * c + 1] = q.y;
            } else {
                const uint4 q = *reinterpret_cast<const uint4 *>(cb + 4 * code);
                r.u[0] = q.x;
                r.u[1] = q.y;
                r.u[2] = q.z;
                r.u[3] = q.w;
            }
        }
        o = r.v;
    };
    // scale: w = fp16(s * entry), v_pk_mul_f16
    auto scale = [&](f16x8 &o, f16x2 s2) {
        union { f16x8 v; f16x2 q[4]; } r;
        r.v = o;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            r.q[k] = r.q[k] * s2;
        o = r.v;
    };

    // A fragment of block b, slice j: tile row 32b + lane%32, columns
    // 32h + 8j + [0, 8) = chunk 4h + j, stored at chunk ^ (row % 8)
    int swz[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        swz[j] = (lane & 31) * 128 + (((4 * h + j) ^ (lane & 7)) << 4);

    // ---- the K loop for a tile of NB blocks ---------------------------------------------
    // Step g: wait until group g's activations and group g+1's codes have
    // landed (the later S-3 stages and group g+1's activations may still be
    // in flight), barrier (no wave still reads stage g-1), then slice by
    // slice: the MFMAs of group g's slice j, the codebook lookups of group
    // g+1's slice j into the registers those MFMAs just read, the scaling
    // of group g+1's slice j-1, and a quarter of the loads of group g+S-1
    // into stage g-1 (past the end: the last group again, never read).
    auto body = [&](auto NBc) {
        constexpr int NB = decltype(NBc)::value;
        f32x16 acc[NPB][NB];
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                acc[pb][b] = f32x16{};

        issue_all(0, ring_l);
        issue_all(min(1, G - 1), ring_l + SH::STAGE);
        if constexpr (S > 3)
            issue_all(min(2, G - 1), ring_l + 2 * SH::STAGE);
        // group 0's codes and scales (its activations and the later stages
        // may still be in flight); the barrier also publishes the codebooks
        // and the row factors
        wait_vm<SH::NDMA_A + (S - 2) * SH::NOPS>();
        wait_lds();
        barrier();
        f16x8 bf[NPB][4];
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb) {
            Raw rw;
            uint32_t nw[NW];
            f16x2 s2;
            read_raw(pb, ring, rw);
            shift_raw(pb, 0, rw, nw, s2);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                lookup(pb / NN, j, nw, bf[pb][j]);
                scale(bf[pb][j], s2);
            }
        }

        int st = 0;   // stage of group g
        for (int g = 0; g < G; ++g) {
            const int st_next = (st + 1 == S) ? 0 : st + 1;
            const int st_fill = (st == 0) ? S - 1 : st - 1;
            const char *sa = ring + st * SH::STAGE;
            const char *sn = ring + st_next * SH::STAGE;
            const uint32_t sf = ring_l + st_fill * SH::STAGE;
            const int gf = min(g + S - 1, G - 1);
            const int gn = min(g + 1, G - 1);
            wait_vm<SH::NDMA_A + (S - 3) * SH::NOPS>();
            barrier();

            Raw rw[NPB];
            uint32_t nw[NPB][NW];
            f16x2 s2[NPB];
            f16x8 af[2][NB];
#pragma unroll
            for (int pb = 0; pb < NPB; ++pb)
                read_raw(pb, sn, rw[pb]);
#pragma unroll
            for (int b = 0; b < NB; ++b)
                af[0][b] = *reinterpret_cast<const f16x8 *>(sa + b * 4096 + swz[0]);
            __builtin_amdgcn_sched_barrier(0);
            static_for<4>([&](auto J) {
                constexpr int j = decltype(J)::value;
                if constexpr (j < 3) {
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        af[(j + 1) & 1][b] =
                            *reinterpret_cast<const f16x8 *>(sa + b * 4096 + swz[j + 1]);
                }
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int pb = 0; pb < NPB; ++pb)
                        acc[pb][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[j & 1][b], bf[pb][j],
                                                                            acc[pb][b], 0, 0, 0);
                // a quarter of the next stage's loads
                constexpr int q0 = (j * SH::NOPS) / 4, q1 = ((j + 1) * SH::NOPS) / 4;
                static_for<q1 - q0>([&](auto Q) {
                    dma_unit(std::integral_constant<int, q0 + decltype(Q)::value>{}, gf, sf);
                });
                if constexpr (j == 0) {
#pragma unroll
                    for (int pb = 0; pb < NPB; ++pb)
                        shift_raw(pb, gn, rw[pb], nw[pb], s2[pb]);
                }
#pragma unroll
                for (int pb = 0; pb < NPB; ++pb)
                    lookup(pb / NN, j, nw[pb], bf[pb][j]);
                if constexpr (j > 0) {
#pragma unroll
                    for (int pb = 0; pb < NPB; ++pb)
                        scale(bf[pb][j - 1], s2[pb]);
                }
                // interleave the side work with the MFMAs of this slice
                static_for<NB * NPB>([&](auto) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, kSchedDs, 0);     // LDS reads
                    __builtin_amdgcn_sched_group_barrier(0x002, kSchedValu, 0);   // VALU
                });
                __builtin_amdgcn_sched_barrier(0);
            });
#pragma unroll
            for (int pb = 0; pb < NPB; ++pb)
                scale(bf[pb][3], s2[pb]);
            st = st_next;
        }
        // nothing may land in LDS after the workgroup ends
        wait_vm<0>();

        // ---- epilogue: lane holds D[8*(r/4) + 4*h + r%4][lane%32] of each block -----
#pragma unroll
        for (int nb = 0; nb < NN; ++nb) {
            const int n = nrow0 + 32 * nb;
            const bool colok = n < a.rows;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = 32 * b + 8 * (r / 4) + 4 * h + (r % 4);
                    if (!(colok && i < mlen))
                        continue;
                    const float f = kf[i];
                    const int64_t o = (int64_t)(m0 + i) * a.out_stride + n;
                    float v;
                    if constexpr (NPROJ == 2) {
                        v = ((live >> nb & 1) && (live >> (NN + nb) & 1))
                                ? silu_mul(acc[nb][b][r] * f, acc[NN + nb][b][r] * f)
                                : 0.0f;
                    } else {
                        if (a.gate_in)
                            v = (live >> nb & 1) ? silu_mul(a.gate_in[o], acc[nb][b][r] * f) : 0.0f;
                        else
                            v = (live >> nb & 1) ? acc[nb][b][r] * f : 0.0f;
                    }
                    a.out[o] = v;
                }
            }
        }
    };
    // one specialisation per block count keeps the step free of branches
    static_for<MB>([&](auto I) {
        constexpr int nb = decltype(I)::value + 1;
        if (nblk == nb)
            body(std::integral_constant<int, nb>{});
    });
    }
}

// ---- dispatch ------------------------------------------------------------------

constexpr int kGemmWaves = 4;

// hipErrorOutOfMemory: this geometry's codebooks leave no room for the ring
// (the caller then splits gate and up into two launches).
template <int D, int BITS, int NPROJ, int MB>
static hipError_t gemm_launch(GemmArgs a, int tile_cap, hipStream_t stream)
{
    constexpr int WAVES = kGemmWaves;
    using SH = GemmShape<D, BITS, NPROJ, MB, WAVES>;
    if constexpr (!SH::FITS) {
        return hipErrorOutOfMemory;
    } else {
        const void *kern = reinterpret_cast<const void *>(k_gemm<D, BITS, NPROJ, MB, WAVES>);
        a.n_ntiles = (a.rows + SH::WG_ROWS - 1) / SH::WG_ROWS;
        const int64_t wgs = (int64_t)((tile_cap + 7) / 8) * 8 * a.n_ntiles;
        if (wgs > 0x7fffffff)
            return hipErrorInvalidValue;
        void *args[] = {&a};
        return hipLaunchKernel(kern, dim3((unsigned)wgs), dim3(64 * WAVES), args, 0, stream);
    }
}

// Tile heights compiled: 32 * {2, 4, 5} rows.
template <int D, int BITS>
struct GemmD {
    static hipError_t run(int nproj, int mb, const GemmArgs &a, int cap, hipStream_t s)
    {
        if (nproj == 2) {
            switch (mb) {
            case 2: return gemm_launch<D, BITS, 2, 2>(a, cap, s);
            case 4: return gemm_launch<D, BITS, 2, 4>(a, cap, s);
            default: return gemm_launch<D, BITS, 2, 5>(a, cap, s);
            }
        }
        switch (mb) {
        case 2: return gemm_launch<D, BITS, 1, 2>(a, cap, s);
        case 4: return gemm_launch<D, BITS, 1, 4>(a, cap, s);
        default: return gemm_launch<D, BITS, 1, 5>(a, cap, s);
        }
    }
};

// Whether a launch of this geometry fits in LDS (host side of GemmShape::FITS).
template <int D, int BITS>
inline bool gemm_fits_db(int nproj, int mb)
{
    constexpr int W = kGemmWaves;
    if (nproj == 2)
        return mb == 2 ? GemmShape<D, BITS, 2, 2, W>::FITS
                       : (mb == 4 ? GemmShape<D, BITS, 2, 4, W>::FITS : GemmShape<D, BITS, 2, 5, W>::FITS);
    return mb == 2 ? GemmShape<D, BITS, 1, 2, W>::FITS
                   : (mb == 4 ? GemmShape<D, BITS, 1, 4, W>::FITS : GemmShape<D, BITS, 1, 5, W>::FITS);
}

template <int D>
inline bool gemm_fits_d(int bits, int nproj, int mb)
{
    switch (bits) {
    case 8: return gemm_fits_db<D, 8>(nproj, mb);
    case 9: return gemm_fits_db<D, 9>(nproj, mb);
    case 10: return gemm_fits_db<D, 10>(nproj, mb);
    case 11: return gemm_fits_db<D, 11>(nproj, mb);
    case 12: return gemm_fits_db<D, 12>(nproj, mb);
    case 13: return gemm_fits_db<D, 13>(nproj, mb);
    default: return false;
    }
}

inline bool gemm_fits(int d, int bits, int nproj, int mb)
{
    return d == 2 ? gemm_fits_d<2>(bits, nproj, mb)
                  : (d == 4 ? gemm_fits_d<4>(bits, nproj, mb) : gemm_fits_d<8>(bits, nproj, mb));
}

template <int D>
hipError_t gemm_d(int bits, int nproj, int mb, const GemmArgs &a, int cap, hipStream_t s)
{
    switch (bits) {
    case 8: return GemmD<D, 8>::run(nproj, mb, a, cap, s);
    case 9: return GemmD<D, 9>::run(nproj, mb, a, cap, s);
    case 10: return GemmD<D, 10>::run(nproj, mb, a, cap, s);
    case 11: return GemmD<D, 11>::run(nproj, mb, a, cap, s);
    case 12: return GemmD<D, 12>::run(nproj, mb, a, cap, s);
    case 13: return GemmD<D, 13>::run(nproj, mb, a, cap, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace vq
