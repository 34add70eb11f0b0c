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
template <int SIZE>
__device__ __forceinline__ void dma(const void *src, void *lds_wave_base)
{
    static_assert(SIZE == 4 || SIZE == 12 || SIZE == 16, "unsupported load size");
    const uint32_t m0 =
        __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t *)lds_wave_base);
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
    int cb_off[2];                 // LDS byte offsets of the codebooks
    int kf_off;                    // LDS byte offset of the tile's row factors
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
    static constexpr int RPD = NT / 8;                          // tile rows per A load
    static constexpr int NDMA_A = (32 * MB + RPD - 1) / RPD;
    static constexpr int A_BYTES = NDMA_A * NT * 16;
    static constexpr int B_BYTES = NPROJ * NT * (BWin<D, BITS>::LDS_BYTES + 4);
    static constexpr int STAGE = A_BYTES + B_BYTES;
    // vector-memory operations per stage and wave: scales, code windows, activations
    static constexpr int NOPS = NDMA_A + NPROJ * (BWin<D, BITS>::NDMA + 1);
};

// One lane's B operand of one projection for one group: 4 slices x 8 halves,
// w = fp16(scale * entry).
template <int D, int BITS>
__device__ __forceinline__ void decode_b(const uint32_t (&nw)[BWin<D, BITS>::NW], uint32_t sc,
                                         const uint32_t *__restrict__ cb, f16x8 (&bf)[4])
{
    using BW = BWin<D, BITS>;
    union { uint32_t u; f16x2 h; } s2;
    s2.u = sc * 0x10001u;
    constexpr uint32_t mask = (1u << BITS) - 1u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        union { f16x8 v; f16x2 p[4]; uint32_t u[4]; } o;
#pragma unroll
        for (int c = 0; c < BW::PER; ++c) {
            const int t = j * BW::PER + c;            // compile-time code position
            const int pb = t * BITS;
            const int wi = pb >> 5, bsh = pb & 31;
            const uint32_t code = (bsh + BITS <= 32)
                                      ? __builtin_amdgcn_ubfe(nw[wi], bsh, BITS)
                                      : (__builtin_amdgcn_alignbit(nw[wi + 1], nw[wi], bsh) & mask);
            if constexpr (D == 2) {
                o.u[c] = cb[code];
            } else if constexpr (D == 4) {
                const uint2 q = *reinterpret_cast<const uint2 *>(cb + 2 * code);
                o.u[2 * c] = q.x;
                o.u[2 * c + 1] = q.y;
            } else {
                const uint4 q = *reinterpret_cast<const uint4 *>(cb + 4 * code);
                o.u[0] = q.x;
                o.u[1] = q.y;
                o.u[2] = q.z;
                o.u[3] = q.w;
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k)
            o.p[k] = o.p[k] * s2.h;                   // v_pk_mul_f16: fp16(s * c)
        bf[j] = o.v;
    }
}

template <int D, int BITS, int NPROJ, int MB, int WAVES, int S>
__global__ __launch_bounds__(64 * WAVES) void k_gemm(const GemmArgs a)
{
    using BW = BWin<D, BITS>;
    using SH = GemmShape<D, BITS, NPROJ, MB, WAVES>;
    constexpr int NT = SH::NT;
    constexpr int NW = BW::NW;
    static_assert(S >= 3, "the ring needs three stages");
    // codebooks and row factors: dynamic LDS; the ring: one static array per
    // stage, so the compiler can tell a stage being filled from the stages
    // being read and waits only for the loads a read depends on
    extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
    char *const lb = reinterpret_cast<char *>(lds);
    __shared__ __attribute__((aligned(16))) char ring0[SH::STAGE];
    __shared__ __attribute__((aligned(16))) char ring1[SH::STAGE];
    __shared__ __attribute__((aligned(16))) char ring2[SH::STAGE];
    __shared__ __attribute__((aligned(16))) char ring3[S > 3 ? SH::STAGE : 16];
    auto ring = [&](auto K) -> char * {
        constexpr int k = decltype(K)::value;
        if constexpr (k == 0)
            return ring0;
        else if constexpr (k == 1)
            return ring1;
        else if constexpr (k == 2)
            return ring2;
        else
            return ring3;
    };

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
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const int e = a.tiles[3 * tile + 0];
    const int m0 = a.tiles[3 * tile + 1];
    const int mlen = a.tiles[3 * tile + 2];
    const int nblk = (mlen + 31) >> 5;
    const int n = ntile * (32 * WAVES) + 32 * wave + (lane & 31);   // this lane's weight row
    const int G = a.groups;

    // ---- prologue: codebooks, row factors, per-lane sources ------------------------
#pragma unroll
    for (int p = 0; p < NPROJ; ++p) {
        const char *src = reinterpret_cast<const char *>(a.codebook[p]);
        char *dst = lb + a.cb_off[p];
        const int n16 = a.cb_bytes[p] >> 4;
        for (int i0 = 0; i0 < n16; i0 += NT)
            if (i0 + tid < n16)
                dma<16>(src + (size_t)(i0 + tid) * 16, dst + (size_t)(i0 + wave * 64) * 16);
        for (int i = (n16 << 2) + tid; i < (a.cb_bytes[p] >> 2); i += NT)
            reinterpret_cast<uint32_t *>(dst)[i] = reinterpret_cast<const uint32_t *>(src)[i];
    }
    float *kf = reinterpret_cast<float *>(lb + a.kf_off);
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
    // weight rows
    const int64_t lin = (int64_t)e * a.rows + min(n, a.rows - 1);
    const uint32_t *brow[NPROJ];
    const uint16_t *srow[NPROJ];
    int live = 0;
#pragma unroll
    for (int p = 0; p < NPROJ; ++p) {
        const int s = a.row_map[p] ? a.row_map[p][lin] : (int)lin;
        const bool lv = (n < a.rows) && (s >= 0);
        live |= lv ? (1 << p) : 0;
        const int64_t sr = lv ? s : 0;
        brow[p] = a.codes[p] + sr * a.wpr;
        srow[p] = a.scales[p] + sr * a.groups;
    }
    if constexpr (NPROJ == 1) {
        if (a.gate_in && a.row_map[1] && a.row_map[1][lin] < 0)
            live = 0;   // split SwiGLU: a dead gate row gives h = +0.0
    }

    // ---- one stage of loads: scales and code windows, then activations -------------
    auto issue = [&](int gg, char *sb) {
        char *bb = sb + SH::A_BYTES;
        const int sbit = gg * BW::G * BITS + h * BW::NBITS;
        const int ws = min(sbit >> 5, a.wpr - NW);   // window start, kept inside the row
#pragma unroll
        for (int p = 0; p < NPROJ; ++p) {
            // the aligned dword holding the scale (it never crosses a page)
            const uintptr_t sp = reinterpret_cast<uintptr_t>(srow[p] + gg);
            dma<4>(reinterpret_cast<const void *>(sp & ~(uintptr_t)3), bb + wave * 64 * 4);
            bb += NT * 4;
            const uint32_t *wp = brow[p] + ws;
#pragma unroll
            for (int k = 0; k < BW::N16; ++k) {
                dma<16>(wp + 4 * k, bb + wave * 64 * 16);
                bb += NT * 16;
            }
            if constexpr (BW::TAIL == 3) {
                dma<12>(wp + 4 * BW::N16, bb + wave * 64 * 16);
                bb += NT * 16;
            } else {
#pragma unroll
                for (int k = 0; k < BW::TAIL; ++k) {
                    dma<4>(wp + 4 * BW::N16 + k, bb + wave * 64 * 4);
                    bb += NT * 4;
                }
            }
        }
        const char *ab = reinterpret_cast<const char *>(a.act) + (size_t)gg * 128;
#pragma unroll
        for (int q = 0; q < SH::NDMA_A; ++q)
            dma<16>(ab + aoff[q], sb + q * NT * 16 + wave * 1024);
    };

    // ---- this lane's B operands of group gg, from stage st --------------------------
    auto decode = [&](int gg, const char *sb, f16x8 (&bf)[NPROJ][4]) {
        const char *bb = sb + SH::A_BYTES;
        const int sbit = gg * BW::G * BITS + h * BW::NBITS;
        const int w0 = sbit >> 5;
        const int delta = w0 - min(w0, a.wpr - NW);   // > 0 only near a row's end
        const int o = sbit & 31;
#pragma unroll
        for (int p = 0; p < NPROJ; ++p) {
            const uint32_t sw = *reinterpret_cast<const uint32_t *>(bb + tid * 4);
            bb += NT * 4;
            const bool hi = (reinterpret_cast<uintptr_t>(srow[p] + gg) & 2) != 0;
            const uint32_t sc = (live >> p & 1) ? (hi ? sw >> 16 : sw & 0xffffu) : 0u;
            uint32_t w[NW];
#pragma unroll
            for (int k = 0; k < BW::N16; ++k) {
                const uint4 v = *reinterpret_cast<const uint4 *>(bb + tid * 16);
                w[4 * k] = v.x;
                w[4 * k + 1] = v.y;
                w[4 * k + 2] = v.z;
                w[4 * k + 3] = v.w;
                bb += NT * 16;
            }
            if constexpr (BW::TAIL == 3) {
                const uint4 v = *reinterpret_cast<const uint4 *>(bb + tid * 16);
                w[4 * BW::N16] = v.x;
                w[4 * BW::N16 + 1] = v.y;
                w[4 * BW::N16 + 2] = v.z;
                bb += NT * 16;
            } else {
#pragma unroll
                for (int k = 0; k < BW::TAIL; ++k) {
                    w[4 * BW::N16 + k] = *reinterpret_cast<const uint32_t *>(bb + tid * 4);
                    bb += NT * 4;
                }
            }
            if (__builtin_expect(delta != 0, 0)) {
                // the window was pulled back to stay inside the row: realign
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
            uint32_t nw[NW];
#pragma unroll
            for (int i = 0; i < NW; ++i)
                nw[i] = __builtin_amdgcn_alignbit(i + 1 < NW ? w[i + 1] : 0u, w[i], o);
            decode_b<D, BITS>(nw, sc, reinterpret_cast<const uint32_t *>(lb + a.cb_off[p]),
                              bf[p]);
        }
    };

    f32x16 acc[NPROJ][MB];
#pragma unroll
    for (int p = 0; p < NPROJ; ++p)
#pragma unroll
        for (int b = 0; b < MB; ++b)
            acc[p][b] = f32x16{};

    // A fragment of block b, slice j: tile row 32b + lane%32, columns
    // 32h + 8j + [0, 8) = chunk 4h + j, stored at chunk ^ (row % 8)
    int swz[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        swz[j] = (lane & 31) * 128 + (((4 * h + j) ^ (lane & 7)) << 4);

    auto mfmas = [&](const char *ab, const f16x8 (&bf)[NPROJ][4]) {
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            if (b < nblk) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f16x8 av = *reinterpret_cast<const f16x8 *>(ab + b * 4096 + swz[j]);
#pragma unroll
                    for (int p = 0; p < NPROJ; ++p)
                        acc[p][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bf[p][j], acc[p][b],
                                                                           0, 0, 0);
                }
            }
        }
    };

    // ---- the ring ---------------------------------------------------------------------
    issue(0, ring0);
    issue(min(1, G - 1), ring1);
    if constexpr (S > 3)
        issue(min(2, G - 1), ring2);
    // group 0's codes and scales (its activations and the later stages may
    // still be in flight); the barrier also publishes the codebooks and the
    // row factors
    wait_vm<SH::NDMA_A + (S - 2) * SH::NOPS>();
    wait_lds();
    barrier();

    f16x8 bfa[NPROJ][4], bfb[NPROJ][4];
    decode(0, ring0, bfa);
    // Group g: its activations and group g+1's codes must have landed (the
    // later S-3 stages and group g+1's activations may still be in flight).
    // After the barrier no wave still reads stage g-1, which is refilled with
    // group g+S-1 (past the end: the last group again, never read).  The loop
    // is unrolled so that stage and buffer indices are compile-time.
    constexpr int U = (S % 2 == 0) ? S : 2 * S;
    auto step = [&](auto K, int g) {
        constexpr int k = decltype(K)::value;
        constexpr int st = k % S, st_next = (k + 1) % S, st_fill = (k + S - 1) % S;
        wait_vm<SH::NDMA_A + (S - 3) * SH::NOPS>();
        barrier();
        issue(min(g + S - 1, G - 1), ring(std::integral_constant<int, st_fill>{}));
        if constexpr (k % 2 == 0) {
            if (g + 1 < G)
                decode(g + 1, ring(std::integral_constant<int, st_next>{}), bfb);
            mfmas(ring(std::integral_constant<int, st>{}), bfa);
        } else {
            if (g + 1 < G)
                decode(g + 1, ring(std::integral_constant<int, st_next>{}), bfa);
            mfmas(ring(std::integral_constant<int, st>{}), bfb);
        }
    };
    auto unrolled = [&](int g0, auto... K) { ((g0 + decltype(K)::value < G ? step(K, g0 + decltype(K)::value) : void()), ...); };
    for (int g0 = 0; g0 < G; g0 += U) {
        if constexpr (U == 4)
            unrolled(g0, std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{},
                     std::integral_constant<int, 2>{}, std::integral_constant<int, 3>{});
        else
            unrolled(g0, std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{},
                     std::integral_constant<int, 2>{}, std::integral_constant<int, 3>{},
                     std::integral_constant<int, 4>{}, std::integral_constant<int, 5>{});
    }
    // nothing may land in LDS after the workgroup ends
    wait_vm<0>();

    // ---- epilogue: lane holds D[8*(r/4) + 4*h + r%4][lane%32] of each block ---------
    const bool colok = n < a.rows;
#pragma unroll
    for (int b = 0; b < MB; ++b) {
        if (b >= nblk)
            continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 32 * b + 8 * (r / 4) + 4 * h + (r % 4);
            if (!(colok && i < mlen))
                continue;
            const float f = kf[i];
            const int64_t o = (int64_t)(m0 + i) * a.out_stride + n;
            float v;
            if constexpr (NPROJ == 2) {
                v = (live == 3) ? silu_mul(acc[0][b][r] * f, acc[1][b][r] * f) : 0.0f;
            } else {
                if (a.gate_in)
                    v = (live & 1) ? silu_mul(a.gate_in[o], acc[0][b][r] * f) : 0.0f;
                else
                    v = (live & 1) ? acc[0][b][r] * f : 0.0f;
            }
            a.out[o] = v;
        }
    }
}

// ---- dispatch ------------------------------------------------------------------

constexpr int kGemmWaves = 4;

// Dynamic LDS of one launch (codebooks, row factors); the ring of S stages is
// static.
template <int D, int BITS, int NPROJ, int MB, int S>
inline size_t gemm_layout(GemmArgs &a)
{
    using SH = GemmShape<D, BITS, NPROJ, MB, kGemmWaves>;
    size_t off = 0;
    for (int p = 0; p < NPROJ; ++p) {
        a.cb_off[p] = (int)off;
        off += ((size_t)a.cb_bytes[p] + 15) & ~(size_t)15;
    }
    a.kf_off = (int)off;
    off += (size_t)32 * MB * 4;
    return off;
}

// Returns hipErrorOutOfMemory when even a three-stage ring does not fit next
// to the codebooks (the caller then splits the projections).
template <int D, int BITS, int NPROJ, int MB>
static hipError_t gemm_launch(GemmArgs a, int tile_cap, hipStream_t stream)
{
    constexpr int WAVES = kGemmWaves;
    using SH = GemmShape<D, BITS, NPROJ, MB, WAVES>;
    const size_t lds = gemm_layout<D, BITS, NPROJ, MB, 4>(a);
    int S = 4;
    const void *kern = reinterpret_cast<const void *>(k_gemm<D, BITS, NPROJ, MB, WAVES, 4>);
    if (lds + 4 * (size_t)SH::STAGE > (size_t)kLdsBudget) {
        S = 3;
        kern = reinterpret_cast<const void *>(k_gemm<D, BITS, NPROJ, MB, WAVES, 3>);
    }
    if (lds + S * (size_t)SH::STAGE + 16 > (size_t)kLdsBudget)
        return hipErrorOutOfMemory;
    if (lds > 65536) {
        hipError_t err = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)lds);
        if (err != hipSuccess)
            return err;
    }
    a.n_ntiles = (a.rows + 32 * WAVES - 1) / (32 * WAVES);
    const int64_t wgs = (int64_t)((tile_cap + 7) / 8) * 8 * a.n_ntiles;
    if (wgs > 0x7fffffff)
        return hipErrorInvalidValue;
    void *args[] = {&a};
    return hipLaunchKernel(kern, dim3((unsigned)wgs), dim3(64 * WAVES), args, lds, stream);
}

// Tile heights compiled: 32 * {2, 3, 5} rows.
template <int D, int BITS>
struct GemmD {
    static hipError_t run(int nproj, int mb, const GemmArgs &a, int cap, hipStream_t s)
    {
        if (nproj == 2) {
            switch (mb) {
            case 2: return gemm_launch<D, BITS, 2, 2>(a, cap, s);
            case 3: return gemm_launch<D, BITS, 2, 3>(a, cap, s);
            default: return gemm_launch<D, BITS, 2, 5>(a, cap, s);
            }
        }
        switch (mb) {
        case 2: return gemm_launch<D, BITS, 1, 2>(a, cap, s);
        case 3: return gemm_launch<D, BITS, 1, 3>(a, cap, s);
        default: return gemm_launch<D, BITS, 1, 5>(a, cap, s);
        }
    }
};

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
