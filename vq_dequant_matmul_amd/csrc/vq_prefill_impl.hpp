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
//   * the K loop walks 64-column groups through rings in LDS filled by
//     direct global->LDS loads (no register staging): the tile's activation
//     rows (fp16, already range-scaled), the lanes' packed codes and their
//     scales.  Codes come as every lane's own window of one group (SC code
//     stages, SC-1 groups ahead), or, for 8-bit codes with d = 2, as
//     two-group chunks of 64 contiguous bytes per row; scales come four
//     groups a row at a time, a quarter of the rows per step.  The loads per
//     step are fixed, so every wait is a constant vmcnt;
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

// 8-bit codebooks as bank-private copies (1) or one plain copy (0)
#ifndef VQ_GEMM_BANKED_CB
#define VQ_GEMM_BANKED_CB 1
#endif
// a step's code-window loads all with its first slice (1) or spread over
// the four slices with the activation rows (0)
#ifndef VQ_GEMM_CODES_FIRST
#define VQ_GEMM_CODES_FIRST 1
#endif

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
    int tile_cap;                  // entries the tiles array holds
    const int32_t *n_tiles;
    int n_ntiles;                  // weight-row tiles per M tile
    const float *gate_in;          // split SwiGLU: gate outputs for this up projection
    float *out;
    int64_t out_stride;
    // one projection only: fp16 outputs in out_h (row stride out_stride, a
    // multiple of 64) with one power-of-two exponent per (tile, 64-column
    // chunk) repeated into out_e[row][chunk] (then out is unused)
    f16 *out_h;
    int8_t *out_e;
};

// Shape of one launch.  A workgroup has WAVES waves; each wave owns NN blocks
// of 32 weight rows of each of the NPROJ projections (NPB = NPROJ * NN
// (projection, block) pairs, all sharing every activation fragment it reads)
// for all MB row blocks of the tile.
template <int D, int BITS, int NPROJ, int MB, int NN_, int WAVES>
struct GemmShape {
    using BW = BWin<D, BITS>;
    static constexpr int NT = 64 * WAVES;
    static constexpr int NN = NN_;
    static constexpr int NPB = NPROJ * NN;
    // accumulators: all AGPRs at one wave per SIMD, half at two
    static constexpr bool ACC_OK = NPB * MB * 16 <= (WAVES >= 8 ? 128 : 256);
    static constexpr int WG_ROWS = 32 * NN * WAVES;             // weight rows per projection
    static constexpr int TR = 32 * MB;                          // tile rows
    static constexpr int RPD = NT / 8;                          // tile rows per A load
    static constexpr int NDMA_A = (TR + RPD - 1) / RPD;
    static constexpr int A_BYTES = TR * 128;                    // one activation stage
    // one (projection, block) of a code stage: every lane's code window
    static constexpr int WIN = NT * BW::LDS_BYTES;
    static constexpr int C_BYTES = NPB * WIN;                   // one code stage
    // scales: sw(SC) bytes per (projection, block) and wave.  With a multiple
    // of four groups per row they hold slots(SC) slots of four groups' scales
    // of the wave's 32 rows (dwords of groups 4c, 4c+1 for all rows, then of
    // 4c+2, 4c+3), a quarter of the rows loaded per step, so a load touches
    // eight rows' cache lines instead of 32; otherwise one dword per row and
    // code stage.  Three code stages need two slots, deeper rings three.
    static constexpr int slots(int sc) { return sc <= 3 ? 2 : 3; }
    static constexpr int sw(int sc) { return sc <= 3 ? 512 : 768; }
    static constexpr int sreg(int sc) { return NPB * WAVES * sw(sc); }
    // vector-memory operations per step and wave: per (projection, block) a
    // scale load and the code window, then the activations
    static constexpr int NOPS_C = NPB * (BW::NDMA + 1);
    static constexpr int NOPS_A = NDMA_A;
    static constexpr int NOPS = NOPS_C + NOPS_A;
    // Codebooks.  With 8-bit codes every entry gets a 256-byte row of
    // copies, one per lane position of an LDS bank pass (lanes are served 32
    // (d2), 16 (d4) or 8 (d8) at a time, and lane l reads copy l % COPIES),
    // so a wavefront's lookups never share a bank; the row of entry k starts
    // at byte k * 256 and, with two projections, the second projection's
    // copies fill the upper 128 bytes.  Wider codes keep one plain copy per
    // projection in a slot sized for 2^b entries.
    static constexpr int ES = 2 * D;                            // bytes per entry
    static constexpr bool BANKED = (BITS == 8) && VQ_GEMM_BANKED_CB;
    static constexpr int COPIES = (NPROJ == 2 ? 128 : 256) / ES;
    static constexpr int CB_SLOT = ((1 << BITS) * ES < 65536) ? (1 << BITS) * ES : 65536;
    static constexpr int CB_BYTES = BANKED ? 256 * 256 : NPROJ * CB_SLOT;
    static constexpr int KF_OFF = CB_BYTES;                     // row factors of the tile
    static constexpr int FIXED = KF_OFF + 32 * MB * 4;
    // Two-group code chunks (8-bit codes, d = 2, a multiple of four groups
    // per row): per (projection, block) and wave one slot of 32 rows x 64
    // bytes (groups 2j, 2j+1) and a three-slot scale ring, both inside the
    // code ring's bytes; the raw codebooks then arrive in the scale region.
    // A load fetches 16 rows x 64 contiguous bytes (16 cache lines, against
    // 32 for a one-group window of every row).  Even steps issue the scales
    // and activations (CH_E loads), odd steps also the next chunk (CH_O).
    static constexpr int CH_SLOT = 2048;
    static constexpr int CH_SW = 768;
    static constexpr int CH_CODES = NPB * WAVES * CH_SLOT;
    static constexpr int CH_REGION = CH_CODES + NPB * WAVES * CH_SW;
    static constexpr int CH_RAW = NPROJ * 256 * ES;             // raw 8-bit codebooks
    // Ring depths: code windows SC stages (loaded SC - 1 groups ahead), the
    // activation rows SA stages (SA - 1 ahead); the deepest pair that fits,
    // with SA >= SC - 1
    static constexpr bool fits(int sc, int sa)
    {
        return FIXED + sreg(sc) + sc * C_BYTES + sa * A_BYTES <= kLdsBudget;
    }
    // A layout for the chunk schedule alone (CHONLY), used where the general
    // one cannot keep loads in flight across steps (tall tiles): after the
    // codebooks and row factors only the raw codebooks, the chunk slots with
    // their scale ring, and the activation stages.  Such a launch needs a
    // multiple of four groups per row (the host checks).
    static constexpr bool fits_ch(int sa)
    {
        return FIXED + CH_RAW + CH_REGION + sa * A_BYTES <= kLdsBudget;
    }
    static constexpr bool CHONLY = BANKED && D == 2 && !fits(3, 3) && fits_ch(3);
    static constexpr int SC = CHONLY ? 3 : (fits(5, 4) ? 5 : (fits(4, 3) ? 4 : 3));
    static constexpr int SA = CHONLY ? (fits_ch(4) ? 4 : 3)
                                     : (fits(5, 4) ? 4 : (fits(4, 3) ? 3 : (fits(3, 3) ? 3 : 2)));
    // with fewer stages the top of every step waits for all loads of the
    // previous one (correct, but nothing stays in flight across steps)
    static constexpr bool DEEP = CHONLY || fits(3, 3);
    static constexpr int SLOTS = slots(SC);
    static constexpr int SW = sw(SC);
    static constexpr int SREG = CHONLY ? CH_RAW : sreg(SC);
    static constexpr int SRING = FIXED;
    static constexpr int CRING = FIXED + SREG;
    static constexpr int ARING = CRING + (CHONLY ? CH_REGION : SC * C_BYTES);
    static constexpr int LDS = ARING + SA * A_BYTES;
    // the 8-bit codebooks arrive through the last code stage before they are
    // copied out (through the scale region with chunks)
    static constexpr bool FITS =
        ACC_OK && (CHONLY ? fits_ch(SA)
                          : (fits(SC, SA) && (!BANKED || NPROJ * 256 * ES <= C_BYTES)));
    // vmcnt at the top of step g: activation rows of group g and the code
    // windows of group g + 1 have landed (every earlier step issued NOPS)
    static constexpr int W_TOP = ((SA - 2) * NOPS < NOPS_A + (SC - 3) * NOPS)
                                     ? (SA - 2) * NOPS : NOPS_A + (SC - 3) * NOPS;
    static_assert(SC * 128 <= SW, "one scale dword per row and code stage");
    static constexpr bool CHUNK = CHONLY || (BANKED && D == 2 && SA >= 3 &&
                                             CH_REGION <= SC * C_BYTES && CH_RAW <= SREG);
    static_assert(!CHONLY || (SA >= 3 && CH_RAW <= SREG), "chunk-only layout");
    static constexpr int CH_E = NPB + NDMA_A;
    static constexpr int CH_O = 3 * NPB + NDMA_A;
    static_assert(CH_O < 64, "vmcnt out of range");
};

// The K step's interleave: after each MFMA, up to this many LDS reads and
// VALU instructions.
constexpr int kSchedDs = 2;
constexpr int kSchedValu = 3;

template <int D, int BITS, int NPROJ, int MB, int NN, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_gemm(const GemmArgs a)
{
    using BW = BWin<D, BITS>;
    using SH = GemmShape<D, BITS, NPROJ, MB, NN, WAVES>;
    constexpr int NT = SH::NT;
    constexpr int NW = BW::NW;
    constexpr int SC = SH::SC;
    constexpr int SA = SH::SA;
    constexpr int NPB = SH::NPB;
    if constexpr (SH::FITS) {
    // codebooks and row factors, then the two rings, in the kernel's only LDS
    // array (at LDS address 0, so codebook reads carry fixed offsets)
    __shared__ __attribute__((aligned(16))) char smem[SH::LDS];
    const uint32_t smem_l = lds_addr(smem);
    const uint32_t cring_l = smem_l + SH::CRING;
    const uint32_t aring_l = smem_l + SH::ARING;
    auto cb_slot = [](int p) { return p * SH::CB_SLOT; };

    // Workgroup L runs on XCD L % 8 (round-robin dispatch); all weight-row
    // tiles of M tile t run on XCD t % 8 one after another, so the tile's
    // activation rows are fetched into that XCD's L2 once.
    const int L = blockIdx.x;
    const int slot = L >> 3;
    const int tile = (slot / a.n_ntiles) * 8 + (L & 7);
    const int ntile = slot - (slot / a.n_ntiles) * a.n_ntiles;
    // the tile's entry is read together with the tile count (one round trip
    // instead of two): the grid's last workgroups may name tiles past the
    // array, so the index is clamped to it and such a read is never used
    const int tl = min(tile, a.tile_cap - 1);
    const int e = a.tiles[3 * tl + 0];
    const int m0 = a.tiles[3 * tl + 1];
    const int mlen = a.tiles[3 * tl + 2];
    const int n_tiles = *a.n_tiles;
    // (the empty asm keeps the compiler from sinking the entry's loads below
    // the early return, behind the tile count's round trip)
    asm volatile("" : : "s"(e), "s"(m0), "s"(mlen), "s"(n_tiles));
    if (tile >= n_tiles)
        return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS bases in SGPRs
    const int h = lane >> 5;
    const int nblk = (mlen + 31) >> 5;
    // weight row of block nb of this lane: nrow0 + 32 * nb
    const int nrow0 = ntile * SH::WG_ROWS + wave * 32 * NN + (lane & 31);
    const int G = a.groups;

    // ---- prologue: codebooks (raw), row factors, per-lane sources -------------------------
    // 8-bit codebooks land in the last code stage (in the scale region with
    // two-group chunks) and are copied out below; wider ones go straight to
    // their slots
    const bool chunk = SH::CHUNK && (G & 3) == 0;
    const int raw_off = chunk ? SH::SRING : SH::CRING + (SC - 1) * SH::C_BYTES;
    const uint32_t raw_l = smem_l + (uint32_t)raw_off;
    char *const raw = smem + raw_off;
#pragma unroll
    for (int p = 0; p < NPROJ; ++p) {
        const char *src = reinterpret_cast<const char *>(a.codebook[p]);
        const uint32_t off = SH::BANKED ? (uint32_t)(p * 256 * SH::ES) : (uint32_t)cb_slot(p);
        const uint32_t dst_l = (SH::BANKED ? raw_l : smem_l) + off;
        char *dst = (SH::BANKED ? raw : smem) + off;
        const int n16 = a.cb_bytes[p] >> 4;
        for (int i0 = 0; i0 < n16; i0 += NT)
            if (i0 + tid < n16)
                dma<16>(src + (size_t)(i0 + tid) * 16, dst_l + (uint32_t)(i0 + wave * 64) * 16u);
        for (int i = (n16 << 2) + tid; i < (a.cb_bytes[p] >> 2); i += NT)
            reinterpret_cast<uint32_t *>(dst)[i] = reinterpret_cast<const uint32_t *>(src)[i];
    }
    // ---- the prologue's global loads -------------------------------------------------------
    // Every load below is issued before any of their results is used, and
    // none sits in a branch of its own (a load in a branch, or one whose
    // result the next branch tests, gets a wait right after it, and the
    // round trips then run one after another).  The grouped-position map
    // and the row maps are read through buffer resources based at the tile's
    // first position and at the expert's first row; a missing map gets an
    // empty resource, whose reads return 0 without an access, and a select
    // takes the identity instead.
    auto rsrc = [](const void *base, int bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes,
                                                 0x00020000);
    };
    const bool has_perm = a.perm != nullptr;
    const __amdgpu_buffer_rsrc_t r_perm =
        rsrc(has_perm ? a.perm + m0 : nullptr, has_perm ? mlen * 4 : 0);
    __amdgpu_buffer_rsrc_t r_map[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const bool hm = a.row_map[p] != nullptr;
        r_map[p] = rsrc(hm ? a.row_map[p] + (int64_t)e * a.rows : nullptr, hm ? a.rows * 4 : 0);
    }
    auto ld = [](const __amdgpu_buffer_rsrc_t &r, int i) {
        return (int)__builtin_amdgcn_raw_buffer_load_b32(r, i * 4, 0, 0);
    };
    // row factor of tile row tid (rows past the tile repeat its last row)
    const int kr = min(tid, mlen - 1);
    const int kperm = ld(r_perm, kr);
    // this thread's activation-row loads
    auto arow = [&](int q, int r) {
        constexpr int TR = SH::TR, RPD = SH::RPD;
        const int span = (TR - q * RPD < RPD) ? TR - q * RPD : RPD;
        return q * RPD + (r - q * RPD) % span;
    };
    int aperm[SH::NDMA_A];
#pragma unroll
    for (int q = 0; q < SH::NDMA_A; ++q)
        aperm[q] = ld(r_perm, min(arow(q, q * SH::RPD + (tid >> 3)), mlen - 1));
    // weight rows of this lane's blocks (and, split SwiGLU, gate's map)
    int rmap[NPB], gmap[NN];
#pragma unroll
    for (int p = 0; p < NPROJ; ++p)
#pragma unroll
        for (int nb = 0; nb < NN; ++nb)
            rmap[p * NN + nb] = ld(r_map[p], min(nrow0 + 32 * nb, a.rows - 1));
#pragma unroll
    for (int nb = 0; nb < NN; ++nb)
        gmap[nb] = NPROJ == 1 ? ld(r_map[1], min(nrow0 + 32 * nb, a.rows - 1)) : 0;
    // rows of this lane's two-group chunk pieces
    int cmap[SH::CHUNK ? NPB : 1][2];
    if constexpr (SH::CHUNK) {
#pragma unroll
        for (int p = 0; p < NPROJ; ++p)
#pragma unroll
            for (int nb = 0; nb < NN; ++nb)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    cmap[p * NN + nb][hh] = ld(
                        r_map[p], min(ntile * SH::WG_ROWS + wave * 32 * NN + 32 * nb + 16 * hh +
                                          (lane >> 2), a.rows - 1));
    }
    // the activation row's exponent (a second round trip when the rows are
    // gathered through perm)
    const int krow = has_perm ? kperm / a.act_div : m0 + kr;
    const int kexp = a.act_k[krow];

    float *kf = reinterpret_cast<float *>(smem + SH::KF_OFF);
    // activation rows: thread tid of load q fills tile row q*RPD + tid/8,
    // LDS chunk tid%8 with global chunk (tid%8) ^ (row%8).  Offsets fit 32
    // bits: the host keeps activation matrices below 4 GiB.
    // A load whose rows run past the tile (eight waves, three blocks) has
    // the waves past it repeat the rows of the first waves: the same bytes
    // to the same place, so every wave issues every load.
    uint32_t aoff[SH::NDMA_A];
#pragma unroll
    for (int q = 0; q < SH::NDMA_A; ++q) {
        const int r = arow(q, q * SH::RPD + (tid >> 3));
        const int row = has_perm ? aperm[q] / a.act_div : m0 + min(r, mlen - 1);
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
            const int s = a.row_map[p] ? rmap[p * NN + nb] : (int)lin;
            bool lv = (n < a.rows) && (s >= 0);
            if (NPROJ == 1 && a.gate_in && a.row_map[1] && gmap[nb] < 0)
                lv = false;   // split SwiGLU: a dead gate row gives h = +0.0
            const int pb = p * NN + nb;
            live |= lv ? (1 << pb) : 0;
            const int64_t sr = lv ? s : 0;
            brow[pb] = a.codes[p] + sr * a.wpr;
            srow[pb] = a.scales[p] + sr * a.groups;
        }
    }
    // 8-bit code windows: the lane's first word in group 0
    const uint32_t *wbase[NPB];
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb)
        wbase[pb] = brow[pb] + h * (BW::NBITS / 32);
    // two-group chunks: lane i of a load fetches 16 bytes of row 16*hh + i/4
    // of the wave's block, piece (i%4 - rot(i/4)) % 4, which lands in slot
    // i%4 of the row's 64 LDS bytes.  The rotation rot(r) = (r/2 + r/8) % 4
    // puts any 8 (16) consecutive rows' copies of one piece in distinct
    // 16-byte bank groups of a 128 (256) byte span, so the fragment reads
    // are conflict-free.
    auto chrot = [](int r) { return ((r >> 1) + (r >> 3)) & 3; };
    const uint32_t *cptr[SH::CHUNK ? NPB : 1][2];
    uint32_t croff[2];   // LDS offset of this lane's piece of an even / odd group
    if constexpr (SH::CHUNK) {
        const int r = lane >> 2;
        const int piece = ((lane & 3) - chrot(r)) & 3;
#pragma unroll
        for (int p = 0; p < NPROJ; ++p)
#pragma unroll
            for (int nb = 0; nb < NN; ++nb)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int n = ntile * SH::WG_ROWS + wave * 32 * NN + 32 * nb + 16 * hh + r;
                    const int64_t lin = (int64_t)e * a.rows + min(n, a.rows - 1);
                    const int sr = a.row_map[p] ? cmap[p * NN + nb][hh] : (int)lin;
                    // a dead or missing row reads row 0: its outputs are zeroed
                    cptr[p * NN + nb][hh] = a.codes[p] + (int64_t)max(sr, 0) * a.wpr + piece * 4;
                }
        const int n = lane & 31;
#pragma unroll
        for (int q = 0; q < 2; ++q)
            croff[q] = (uint32_t)((n >> 4) * 1024 + (n & 15) * 64 +
                                  ((((2 * q + h) + chrot(n & 15)) & 3) << 4));
    }
    // v_perm selectors that broadcast the scale's half of the loaded dword
    // (or zero, for a dead row) into both halves of the multiplier, for even
    // groups; odd groups take the other half (sel ^ sflip)
    const bool sring = (G & 3) == 0;   // scales four groups at a time (uniform)
    uint32_t ssel[NPB], sflip[NPB];
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) {
        const bool hi = !sring && ((reinterpret_cast<uintptr_t>(srow[pb]) >> 1) & 1u) != 0;
        const bool lv = (live >> pb & 1) != 0;
        ssel[pb] = !lv ? 0x0c0c0c0cu : (hi ? 0x03020302u : 0x01000100u);
        sflip[pb] = lv ? 0x02020202u : 0u;   // 0x01000100 <-> 0x03020302
    }

    static_assert(NT >= 32 * MB, "one row factor per thread");
    if (tid < 32 * MB)
        kf[tid] = ldexpf(1.0f, -kexp);

    // ---- the loads of one step g, one instruction per unit: per (projection,
    // block) a scale load and the code window of group gc into code stage cst
    // (code stage index csi), then the activation rows of group ga into
    // activation stage ast ---------------------------------------------------------------
    constexpr int PB = BW::NDMA + 1;                     // loads per (projection, block)
    // activation load qa of group ga into activation stage ast: this wave's
    // eight rows (wrapped as in aoff)
    auto a_load = [&](int qa, int ga, uint32_t ast) {
        const uint32_t r0 = (uint32_t)arow(qa, qa * SH::RPD + wave * 8);
        dma<16>(reinterpret_cast<const char *>(a.act) + (size_t)ga * 128 + aoff[qa], ast + r0 * 128);
    };
    const uint32_t sreg_l = smem_l + SH::SRING + (uint32_t)(wave * SH::SW);
    // the scale load of step g for (projection, block) pb.  Ring: rows
    // 8p .. 8p+7 (p = (g + SC + 2) mod 4) of the chunk of groups 4c .. 4c+3,
    // c = (g + SC + 2) / 4, into slot c mod SLOTS.  Chunk c is issued in
    // steps 4c-SC-2 .. 4c-SC+1, the last with the code windows of group 4c,
    // so the wait that publishes those before step 4c-1 covers it too; it is
    // read in steps 4c-1 .. 4c+2, and the next chunk of its slot comes from
    // step 4c+4*SLOTS-SC-2 > 4c+2 on.  Lane l < 32 loads groups 4c, 4c+1 of its row, lane
    // l + 32 groups 4c+2, 4c+3.  Otherwise lanes 0..31 load the dword holding
    // group gc's scale into the slot of its code stage csi.
    auto scale_load = [&](int pb, int g, int gc, int csi) {
        const uint32_t base = sreg_l + (uint32_t)(pb * WAVES * SH::SW);
        if (sring) {
            const int p = (g + SC + 2) & 3;
            const int c = min((g + SC + 2) >> 2, (G >> 2) - 1);
            const char *sp = reinterpret_cast<const char *>(srow[pb]) + c * 8 + h * 4;
            if (((lane & 31) >> 3) == p)
                dma<4>(sp, base + (uint32_t)((c % SH::SLOTS) * 256));
        } else {
            // the aligned dword holding the scale (it never crosses a page)
            const uintptr_t sp = reinterpret_cast<uintptr_t>(srow[pb] + gc);
            if (lane < 32)
                dma<4>(reinterpret_cast<const void *>(sp & ~(uintptr_t)3),
                       base + (uint32_t)(csi * 128));
        }
    };
    auto dma_unit = [&](auto Q, int g, int gc, uint32_t cst, int csi, int ga, uint32_t ast) {
        constexpr int q = decltype(Q)::value;
        if constexpr (q < SH::NOPS_C) {
            constexpr int pb = q / PB, r = q % PB;
            const uint32_t bb = cst + pb * SH::WIN;
            if constexpr (r == 0) {
                scale_load(pb, g, gc, csi);
            } else {
                const uint32_t *wp;
                if constexpr (SH::BANKED) {
                    // 8-bit windows never run past the row: a fixed stride per group
                    wp = wbase[pb] + gc * (BW::G * BITS / 32);
                } else {
                    const int sbit = gc * BW::G * BITS + h * BW::NBITS;
                    const int ws = min(sbit >> 5, a.wpr - NW);   // window kept inside the row
                    wp = brow[pb] + ws;
                }
                constexpr int c = r - 1;
                constexpr int cb0 = 0;
                if constexpr (c < BW::N16)
                    dma<16>(wp + 4 * c, bb + cb0 + c * NT * 16 + wave * 64 * 16);
                else if constexpr (BW::TAIL == 3)
                    dma<12>(wp + 4 * c, bb + cb0 + c * NT * 16 + wave * 64 * 16);
                else
                    dma<4>(wp + 4 * BW::N16 + (c - BW::N16),
                           bb + cb0 + BW::N16 * NT * 16 + (c - BW::N16) * NT * 4 + wave * 64 * 4);
            }
        } else {
            a_load(q - SH::NOPS_C, ga, ast);
        }
    };
    auto issue_step = [&](int g, int gc, uint32_t cst, int csi, int ga, uint32_t ast) {
        static_for<SH::NOPS>([&](auto Q) { dma_unit(Q, g, gc, cst, csi, ga, ast); });
    };
    auto cstage = [&](int s) { return cring_l + (uint32_t)(s * SH::C_BYTES); };
    auto astage = [&](int s) { return aring_l + (uint32_t)(s * SH::A_BYTES); };

    // ---- decoding this lane's B operands, in pieces -----------------------------------
    struct Raw {
        uint32_t w[NW];
        uint32_t sw;
    };
    // raw: the scale dword of group gn (code stage csi) and the code words of
    // (projection, block) pb
    auto read_raw = [&](int pb, const char *cs, int gn, int csi, Raw &rw) {
        const char *sb = smem + SH::SRING + (pb * WAVES + wave) * SH::SW + (lane & 31) * 4;
        const int soff = sring ? (((gn >> 2) % SH::SLOTS) * 256 + ((gn >> 1) & 1) * 128) : csi * 128;
        rw.sw = *reinterpret_cast<const uint32_t *>(sb + soff);
        const char *bb = cs + pb * SH::WIN;
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
    // the (s, s) multiplier (0 for a dead row).  8-bit windows always start
    // on a word boundary inside the row.
    auto shift_raw = [&](int pb, int gg, const Raw &rw, uint32_t (&nw)[NW], f16x2 &s2) {
        if constexpr (SH::BANKED) {
#pragma unroll
            for (int i = 0; i < NW; ++i)
                nw[i] = rw.w[i];
        } else {
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
        }
        union { uint32_t u; f16x2 h; } c2;
        const uint32_t odd = 0u - (uint32_t)(gg & 1);   // uniform: all ones for odd groups
        c2.u = __builtin_amdgcn_perm(rw.sw, rw.sw, ssel[pb] ^ (sflip[pb] & odd));
        s2 = c2.h;
    };
    // lookup: the codebook entries of slice j (unscaled)
    // 8-bit: the byte offset of code c's copy row is c * 256, and this lane's
    // copy sits at lane_off in it; v_perm puts the code byte above lane_off
    const uint32_t lane_off = (uint32_t)(lane % SH::COPIES) * SH::ES;
    auto lookup = [&](int p, int j, const uint32_t (&nw)[NW], f16x8 &o) {
        union { f16x8 v; uint32_t u[4]; } r;
        if constexpr (SH::BANKED) {
            const char *cb = smem + (NPROJ == 2 ? p * 128 : 0);
#pragma unroll
            for (int c = 0; c < BW::PER; ++c) {
                const int t = j * BW::PER + c;           // code t of the lane: byte t % 4 of word t / 4
                const uint32_t sel = 0x0c0c0000u | ((uint32_t)(4 + (t & 3)) << 8);
                const uint32_t off = __builtin_amdgcn_perm(nw[t >> 2], lane_off, sel);
                if constexpr (D == 2) {
                    r.u[c] = *reinterpret_cast<const uint32_t *>(cb + off);
                } else if constexpr (D == 4) {
                    const uint2 q = *reinterpret_cast<const uint2 *>(cb + off);
                    r.u[2 * c] = q.x;
                    r.u[2 * c + 1] = q.y;
                } else {
                    const uint4 q = *reinterpret_cast<const uint4 *>(cb + off);
                    r.u[0] = q.x;
                    r.u[1] = q.y;
                    r.u[2] = q.z;
                    r.u[3] = q.w;
                }
            }
        } else {
            const uint32_t *cb = reinterpret_cast<const uint32_t *>(smem + cb_slot(p));
            constexpr uint32_t mask = (1u << BITS) - 1u;
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

    // 8-bit codebooks: every raw entry copied into its row of copies: thread t
    // writes row k = t (NT >= 256 rows), chunk by chunk
    auto expand_cb = [&]() {
        // one 16-byte slot per thread and pass: the lanes of a wave fill the
        // consecutive slots of four entries (1 KiB), so their stores fall on
        // distinct banks; the 16 lanes of one entry read its raw bytes as a
        // broadcast
        for (int w = tid; w < 256 * 16; w += NT) {
            const int k = w >> 4, c = w & 15;
            const int p = (NPROJ == 2) ? (c >> 3) : 0;
            const int lim = (p == 0) ? a.cb_bytes[0] : a.cb_bytes[NPROJ - 1];
            const char *src = raw + p * 256 * SH::ES + k * SH::ES;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (k * SH::ES < lim) {
                if constexpr (D == 2) {
                    const uint32_t e = *reinterpret_cast<const uint32_t *>(src);
                    v = make_uint4(e, e, e, e);
                } else if constexpr (D == 4) {
                    const uint2 q = *reinterpret_cast<const uint2 *>(src);
                    v = make_uint4(q.x, q.y, q.x, q.y);
                } else {
                    v = *reinterpret_cast<const uint4 *>(src);
                }
            }
            *reinterpret_cast<uint4 *>(smem + k * 256 + c * 16) = v;
        }
    };

    // ---- epilogue: lane holds D[8*(r/4) + 4*h + r%4][lane%32] of each block --------------
    // Stores go through a buffer resource based at the tile's first output
    // row and sized to end at row mlen: the range check drops the rows past
    // the tile's end, and a lane past the last weight row takes an offset
    // beyond any size, so no store needs a branch.  The row factors come four
    // at a time from LDS.
    static_assert(SH::KF_OFF % 16 == 0, "row factors are read as float4");
    auto store_tile = [&](auto NBc, auto &acc) {
        constexpr int NB = decltype(NBc)::value;
        const uint32_t rs = (uint32_t)a.out_stride * 4u;   // bytes per output row
        const uint32_t nrec = (uint32_t)mlen * rs;
        const __amdgpu_buffer_rsrc_t ro =
            __builtin_amdgcn_make_buffer_rsrc(a.out + (int64_t)m0 * a.out_stride, (short)0,
                                              (int)nrec, 0x00020000);
        const bool split = NPROJ == 1 && a.gate_in != nullptr;
        __amdgpu_buffer_rsrc_t rg = ro;
        if (split)
            rg = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float *>(a.gate_in) + (int64_t)m0 * a.out_stride, (short)0,
                (int)nrec, 0x00020000);
#pragma unroll
        for (int nb = 0; nb < NN; ++nb) {
            const int n = nrow0 + 32 * nb;
            const bool lv = NPROJ == 2 ? ((live >> nb & 1) && (live >> (NN + nb) & 1))
                                       : (live >> nb & 1) != 0;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float4 f4[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    f4[q] = *reinterpret_cast<const float4 *>(kf + 32 * b + 8 * q + 4 * h);
                const uint32_t vb =
                    n < a.rows ? (uint32_t)(32 * b + 4 * h) * rs + (uint32_t)n * 4u : 0x80000000u;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float4 fq = f4[r / 4];
                    const float f = (r % 4 == 0) ? fq.x : (r % 4 == 1) ? fq.y : (r % 4 == 2) ? fq.z : fq.w;
                    const uint32_t off = vb + (uint32_t)(8 * (r / 4) + (r % 4)) * rs;
                    float v;
                    if constexpr (NPROJ == 2) {
                        v = silu_mul_fast(acc[nb][b][r] * f, acc[NN + nb][b][r] * f);
                    } else {
                        v = acc[nb][b][r] * f;
                        if (split)
                            v = silu_mul_fast(__builtin_bit_cast(
                                                  float, __builtin_amdgcn_raw_buffer_load_b32(rg, off, 0, 0)),
                                              v);
                    }
                    v = lv ? v : 0.0f;
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ro, off, 0, 0);
                }
            }
        }
    };

    // fp16 outputs (one projection; the routed FFN's down projection, whose
    // rows a combine reads back): per 64-column chunk of the wave (blocks 2c
    // and 2c + 1) every row of the tile is scaled by the one power of two 2^E
    // that puts the chunk's largest magnitude over the tile in [2^14, 2^15),
    // rounded to fp16, and E goes to out_e[row][chunk].  The activation rows
    // were range-scaled one by one, so the tile's rows have like magnitudes
    // and each value keeps fp16's relative precision; the row factor is not
    // applied here (a reader takes 2^-(E + k) with the row's exponent k).
    // Dead weight rows and lanes past the last weight row give +0.0.
    auto store_tile_h = [&](auto NBc, auto &acc) {
        constexpr int NB = decltype(NBc)::value;
        static_assert(NPROJ == 1 && NN % 2 == 0, "chunks are pairs of blocks of one projection");
        const int nch = (int)(a.out_stride >> 6);
        const uint32_t rs = (uint32_t)a.out_stride * 2u;   // bytes per output row
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
            a.out_h + (int64_t)m0 * a.out_stride, (short)0, (int)((uint32_t)mlen * rs), 0x00020000);
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
            a.out_e + (int64_t)m0 * nch, (short)0, mlen * nch, 0x00020000);
#pragma unroll
        for (int c = 0; c < NN / 2; ++c) {
            const int n0 = nrow0 + 64 * c, n1 = n0 + 32;
            // the chunk's first column (uniform); the row count is a multiple
            // of 64, so a chunk is wholly inside or wholly past the end
            const int cb = __builtin_amdgcn_readfirstlane(n0 - (lane & 31));
            if (cb >= a.rows)
                continue;
            const bool l0 = (live >> (2 * c) & 1) != 0, l1 = (live >> (2 * c + 1) & 1) != 0;
            float mx = 0.0f;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    mx = fmaxf(mx, fmaxf(l0 ? fabsf(acc[2 * c][b][r]) : 0.0f,
                                         l1 ? fabsf(acc[2 * c + 1][b][r]) : 0.0f));
            mx = segment_max16_dpp(mx);
            {
                const uint32_t u = __float_as_uint(mx);
                const auto q = __builtin_amdgcn_permlane16_swap(u, u, false, false);
                mx = fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
                const auto q2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx),
                                                                 __float_as_uint(mx), false, false);
                mx = fmaxf(__uint_as_float(q2[0]), __uint_as_float(q2[1]));
            }
            const int ex = range_exponent(mx);
            const float up = ldexpf(1.0f, ex);
            const int ch = cb >> 6;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const uint32_t v0 = n0 < a.rows ? (uint32_t)(32 * b + 4 * h) * rs + (uint32_t)n0 * 2u
                                                : 0x80000000u;
                const uint32_t v1 = n1 < a.rows ? (uint32_t)(32 * b + 4 * h) * rs + (uint32_t)n1 * 2u
                                                : 0x80000000u;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const uint32_t off = (uint32_t)(8 * (r / 4) + (r % 4)) * rs;
                    const f16 y0 = (f16)(l0 ? acc[2 * c][b][r] * up : 0.0f);
                    const f16 y1 = (f16)(l1 ? acc[2 * c + 1][b][r] * up : 0.0f);
                    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, y0), ro,
                                                          v0 + off, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, y1), ro,
                                                          v1 + off, 0, 0);
                }
                // the exponent of tile row 32b + lane (lanes 0..31)
                const uint32_t vx = lane < 32 ? (uint32_t)(32 * b + lane) * (uint32_t)nch + (uint32_t)ch
                                              : 0x80000000u;
                __builtin_amdgcn_raw_buffer_store_b8((unsigned char)(signed char)ex, rx, vx, 0, 0);
            }
        }
    };

    // ---- the K loop for a tile of NB blocks ---------------------------------------------
    // Step g reads the activation rows of group g from activation stage g % SA
    // and the code windows of group g + 1 from code stage (g + 1) % SC.  It
    // waits until both have landed (later groups' loads may still be in
    // flight), passes a barrier (no wave still reads what this step
    // overwrites), then slice by slice: the MFMAs of group g's slice j, the
    // codebook lookups of group g + 1's slice j into the registers those
    // MFMAs just read, the scaling of group g + 1's slice j - 1, and a quarter
    // of this step's loads: the code windows of group g + SC - 1 and the
    // activation rows of group g + SA - 1 (past the end: the last group again,
    // never read).  Every step, and each of the SC - 1 steps of the prologue,
    // issues NOPS loads, so the vmcnt waits are the same constants throughout.
    auto body = [&](auto NBc) {
        constexpr int NB = decltype(NBc)::value;
        f32x16 acc[NPB][NB];
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                acc[pb][b] = f32x16{};

        // the scales of groups 0..3 (ring: the quarters of chunk 0 that belong
        // to steps -SC-2 .. -SC), then prologue steps s = -(SC-1) .. -1:
        // code windows of group s + SC - 1, activation rows of group
        // max(s + SA - 1, 0) (a repeat of group 0 when negative: the same bytes
        // to the same place)
        if (sring) {
#pragma unroll
            for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
                for (int s = -SC - 2; s < -SC + 1; ++s)
                    scale_load(pb, s, 0, 0);
        }
#pragma unroll
        for (int s = -(SC - 1); s < 0; ++s) {
            const int gc = min(s + SC - 1, G - 1);
            const int ga = min(max(s + SA - 1, 0), G - 1);
            issue_step(s, gc, cstage(s + SC - 1), s + SC - 1, ga, astage(max(s + SA - 1, 0)));
        }
        if constexpr (SH::BANKED) {
            // the raw codebooks (issued before the prologue steps), then the
            // copies
            wait_vm<(SC - 1) * SH::NOPS>();
            wait_lds();
            barrier();
            expand_cb();
        }
        // group 0's code windows (issued by the first prologue step); the
        // barrier also publishes the codebooks and the row factors, and (with
        // 8-bit codes) keeps every wave's raw reads before step 0 refills the
        // last code stage
        wait_vm<SH::NOPS_A + (SC - 2) * SH::NOPS>();
        wait_lds();
        barrier();
        f16x8 bf[NPB][4];
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb) {
            Raw rw;
            uint32_t nw[NW];
            f16x2 s2;
            read_raw(pb, smem + SH::CRING, 0, 0, rw);
            shift_raw(pb, 0, rw, nw, s2);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                lookup(pb / NN, j, nw, bf[pb][j]);
                scale(bf[pb][j], s2);
            }
        }

        int sa = 0;   // activation stage of group g
        int sc = 0;   // code stage of group g
        for (int g = 0; g < G; ++g) {
            const int sa_fill = (sa == 0) ? SA - 1 : sa - 1;   // stage of group g + SA - 1
            const int sc_fill = (sc == 0) ? SC - 1 : sc - 1;   // stage of group g + SC - 1
            const int sc_next = (sc + 1 == SC) ? 0 : sc + 1;   // stage of group g + 1
            const char *as = smem + SH::ARING + sa * SH::A_BYTES;
            const char *cs = smem + SH::CRING + sc_next * SH::C_BYTES;
            const uint32_t cf = cstage(sc_fill), af = astage(sa_fill);
            const int gc = min(g + SC - 1, G - 1);
            const int ga = min(g + SA - 1, G - 1);
            const int gn = min(g + 1, G - 1);
            wait_vm<SH::W_TOP>();
            barrier();

            Raw rw[NPB];
            uint32_t nw[NPB][NW];
            f16x2 s2[NPB];
            f16x8 af2[2][NB];
#pragma unroll
            for (int pb = 0; pb < NPB; ++pb)
                read_raw(pb, cs, gn, sc_next, rw[pb]);
#pragma unroll
            for (int b = 0; b < NB; ++b)
                af2[0][b] = *reinterpret_cast<const f16x8 *>(as + b * 4096 + swz[0]);
            __builtin_amdgcn_sched_barrier(0);
            static_for<4>([&](auto J) {
                constexpr int j = decltype(J)::value;
                if constexpr (j < 3) {
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        af2[(j + 1) & 1][b] =
                            *reinterpret_cast<const f16x8 *>(as + b * 4096 + swz[j + 1]);
                }
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int pb = 0; pb < NPB; ++pb)
                        acc[pb][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af2[j & 1][b], bf[pb][j],
                                                                            acc[pb][b], 0, 0, 0);
                // this step's loads: the code windows (from HBM, the longest
                // wait) with the first slice, the activation rows spread over
                // the other three, in issue order
                constexpr int NA = SH::NOPS_A;
                constexpr int q0 = !VQ_GEMM_CODES_FIRST ? (j * SH::NOPS) / 4
                                   : ((j == 0) ? 0 : SH::NOPS_C + ((j - 1) * NA) / 3);
                constexpr int q1 = !VQ_GEMM_CODES_FIRST ? ((j + 1) * SH::NOPS) / 4
                                   : ((j == 0) ? SH::NOPS_C : SH::NOPS_C + (j * NA) / 3);
                static_for<q1 - q0>([&](auto Q) {
                    dma_unit(std::integral_constant<int, q0 + decltype(Q)::value>{}, g, gc, cf,
                             sc_fill, ga, af);
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
            sa = (sa + 1 == SA) ? 0 : sa + 1;
            sc = sc_next;
        }
        // nothing may land in LDS after the workgroup ends
        wait_vm<0>();

        if constexpr (NPROJ == 1 && NN % 2 == 0) {
            if (a.out_e) {
                store_tile_h(NBc, acc);
                return;
            }
        }
        store_tile(NBc, acc);
    };

    // ---- the K loop with two-group code chunks ------------------------------------------
    // Step g reads the activation rows of group g and decodes group g + 1 as
    // above, but the code words come in chunks of two groups: odd step 2j+1
    // reads chunk j+1 (groups 2j+2, 2j+3) from the wave's slot, keeps group
    // 2j+3's words in registers for step 2j+2, waits for those reads and
    // refills the slot with chunk j+2, which has two steps to land.  The top
    // of step g waits until everything issued up to step g-2 has landed (one
    // step's loads stay in flight), which covers the chunk, the activation
    // rows (issued SA-1 >= 2 steps ahead) and the scales (chunk c of the
    // scale ring in steps 4c-6 .. 4c-3, a quarter of the rows each, first read
    // in step 4c-1; slot c mod 3 takes chunk c+3 from step 4c+6 on, after its
    // last read in step 4c+2).  Past the end the last chunks and groups are
    // loaded again: the same bytes to the same place.
    auto body_ch = [&](auto NBc) {
        constexpr int NB = decltype(NBc)::value;
        constexpr int NA = SH::NDMA_A;
        f32x16 acc[NPB][NB];
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                acc[pb][b] = f32x16{};
        const int slot_w = (int)SH::CRING + wave * SH::CH_SLOT;                 // + pb * WAVES * CH_SLOT
        const int scal_w = (int)SH::CRING + SH::CH_CODES + wave * SH::CH_SW;    // + pb * WAVES * CH_SW
        auto scale_load_ch = [&](int pb, int g) {
            const int p = (g + 6) & 3;
            const int c = min((g + 6) >> 2, (G >> 2) - 1);
            const char *sp = reinterpret_cast<const char *>(srow[pb]) + c * 8 + h * 4;
            if (((lane & 31) >> 3) == p)
                dma<4>(sp, smem_l + (uint32_t)(scal_w + pb * WAVES * SH::CH_SW + (c % 3) * 256));
        };
        auto code_load_ch = [&](int j) {
            j = min(j, (G >> 1) - 1);
#pragma unroll
            for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    dma<16>(cptr[pb][hh] + j * 16,
                            smem_l + (uint32_t)(slot_w + pb * WAVES * SH::CH_SLOT + hh * 1024));
        };
        auto code_read_ch = [&](int pb, int q) {
            return *reinterpret_cast<const uint4 *>(smem + slot_w + pb * WAVES * SH::CH_SLOT + croff[q]);
        };
        auto scale_read_ch = [&](int pb, int gn) {
            return *reinterpret_cast<const uint32_t *>(
                smem + scal_w + pb * WAVES * SH::CH_SW + ((gn >> 2) % 3) * 256 + ((gn >> 1) & 1) * 128 +
                (lane & 31) * 4);
        };
        auto set_words = [](Raw &rw, const uint4 &v) {
            rw.w[0] = v.x;
            rw.w[1] = v.y;
            rw.w[2] = v.z;
            rw.w[3] = v.w;
        };

        // prologue: the scale quarters of steps -6 .. -1, chunk 0, the
        // activation rows of groups 0 .. SA-2; all landed, the codebooks copied
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
            for (int g = -6; g < 0; ++g)
                scale_load_ch(pb, g);
        code_load_ch(0);
#pragma unroll
        for (int i = 0; i < SA - 1; ++i)
#pragma unroll
            for (int qa = 0; qa < NA; ++qa)
                a_load(qa, min(i, G - 1), astage(i));
        wait_vm<0>();
        wait_lds();
        barrier();
        expand_cb();
        wait_lds();
        barrier();
        // group 0 decoded, group 1's words kept, then the slot takes chunk 1
        f16x8 bf[NPB][4];
        uint4 rnext[NPB];
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb) {
            Raw rw;
            uint32_t nw[NW];
            f16x2 s2;
            set_words(rw, code_read_ch(pb, 0));
            rnext[pb] = code_read_ch(pb, 1);
            rw.sw = scale_read_ch(pb, 0);
            shift_raw(pb, 0, rw, nw, s2);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                lookup(pb / NN, j, nw, bf[pb][j]);
                scale(bf[pb][j], s2);
            }
        }
        wait_lds();
        code_load_ch(1);

        int sa = 0;   // activation stage of group g
        auto step = [&](auto PARc, int g) {
            constexpr int PAR = decltype(PARc)::value;
            const int sa_fill = (sa == 0) ? SA - 1 : sa - 1;   // stage of group g + SA - 1
            const char *as = smem + SH::ARING + sa * SH::A_BYTES;
            const uint32_t af = astage(sa_fill);
            const int ga = min(g + SA - 1, G - 1);
            const int gn = min(g + 1, G - 1);
            if constexpr (PAR)
                wait_vm<SH::CH_E>();   // step g-1 was even
            else
                wait_vm<SH::CH_O>();
            barrier();

            Raw rw[NPB];
            uint32_t nw[NPB][NW];
            f16x2 s2[NPB];
            f16x8 af2[2][NB];
#pragma unroll
            for (int pb = 0; pb < NPB; ++pb) {
                if constexpr (PAR) {
                    set_words(rw[pb], code_read_ch(pb, 0));   // group g + 1 (even)
                    rnext[pb] = code_read_ch(pb, 1);          // group g + 2
                } else {
                    set_words(rw[pb], rnext[pb]);
                }
                rw[pb].sw = scale_read_ch(pb, gn);
            }
#pragma unroll
            for (int b = 0; b < NB; ++b)
                af2[0][b] = *reinterpret_cast<const f16x8 *>(as + b * 4096 + swz[0]);
            __builtin_amdgcn_sched_barrier(0);
            static_for<4>([&](auto J) {
                constexpr int j = decltype(J)::value;
                if constexpr (j < 3) {
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        af2[(j + 1) & 1][b] =
                            *reinterpret_cast<const f16x8 *>(as + b * 4096 + swz[j + 1]);
                }
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int pb = 0; pb < NPB; ++pb)
                        acc[pb][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af2[j & 1][b], bf[pb][j],
                                                                            acc[pb][b], 0, 0, 0);
                if constexpr (j == 0) {
#pragma unroll
                    for (int pb = 0; pb < NPB; ++pb)
                        scale_load_ch(pb, g);
#pragma unroll
                    for (int pb = 0; pb < NPB; ++pb)
                        shift_raw(pb, gn, rw[pb], nw[pb], s2[pb]);
                    if constexpr (PAR) {
                        // the slot's words are in registers: refill it
                        wait_lds();
                        code_load_ch((g + 3) >> 1);
                    }
                } else {
                    constexpr int q0 = ((j - 1) * NA) / 3, q1 = (j * NA) / 3;
#pragma unroll
                    for (int qa = q0; qa < q1; ++qa)
                        a_load(qa, ga, af);
                }
#pragma unroll
                for (int pb = 0; pb < NPB; ++pb)
                    lookup(pb / NN, j, nw[pb], bf[pb][j]);
                if constexpr (j > 0) {
#pragma unroll
                    for (int pb = 0; pb < NPB; ++pb)
                        scale(bf[pb][j - 1], s2[pb]);
                }
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
            sa = (sa + 1 == SA) ? 0 : sa + 1;
        };
        for (int g = 0; g < G; g += 2) {
            step(std::integral_constant<int, 0>{}, g);
            step(std::integral_constant<int, 1>{}, g + 1);
        }
        // nothing may land in LDS after the workgroup ends
        wait_vm<0>();

        if constexpr (NPROJ == 1 && NN % 2 == 0) {
            if (a.out_e) {
                store_tile_h(NBc, acc);
                return;
            }
        }
        store_tile(NBc, acc);
    };

    // one specialisation per block count keeps the step free of branches
    static_for<MB>([&](auto I) {
        constexpr int nb = decltype(I)::value + 1;
        if (nblk == nb) {
            if constexpr (SH::CHONLY) {
                if (chunk)   // always: the host launches this layout only then
                    body_ch(std::integral_constant<int, nb>{});
            } else if constexpr (SH::CHUNK) {
                if (chunk)
                    body_ch(std::integral_constant<int, nb>{});
                else
                    body(std::integral_constant<int, nb>{});
            } else {
                body(std::integral_constant<int, nb>{});
            }
        }
    });
    }
}

// ---- dispatch ------------------------------------------------------------------

// Waves per workgroup: with bank-private codebooks (8-bit codes) eight, two
// per SIMD, so one wave's waits are filled by the other's work (each wave then
// holds half the accumulators); otherwise four.
constexpr int gemm_waves(int bits) { return (bits == 8 && VQ_GEMM_BANKED_CB) ? 8 : 4; }

// Weight-row blocks per wave and projection: two projections take two each;
// one projection takes four (each activation fragment then feeds four MFMAs)
// unless the rows would leave most of a 512-row tile empty.
inline int gemm_nn(int nproj, int rows)
{
    if (nproj == 2)
        return 2;
    const int t4 = (rows + 511) / 512 * 512, t2 = (rows + 255) / 256 * 256;
    return (t4 - rows) * 8 <= t4 && t4 <= t2 + 256 ? 4 : 2;
}

// hipErrorOutOfMemory: this geometry's codebooks leave no room for the rings
// (the caller then splits gate and up into two launches).
template <int D, int BITS, int NPROJ, int MB, int NN>
static hipError_t gemm_launch(GemmArgs a, int tile_cap, hipStream_t stream)
{
    constexpr int WAVES = gemm_waves(BITS);
    using SH = GemmShape<D, BITS, NPROJ, MB, NN, WAVES>;
    if constexpr (!SH::FITS) {
        return hipErrorOutOfMemory;
    } else {
        if (SH::CHONLY && (a.groups & 3) != 0)
            return hipErrorInvalidValue;   // the chunk-only layout needs four groups a step
        const void *kern = reinterpret_cast<const void *>(k_gemm<D, BITS, NPROJ, MB, NN, WAVES>);
        a.n_ntiles = (a.rows + SH::WG_ROWS - 1) / SH::WG_ROWS;
        const int64_t wgs = (int64_t)((tile_cap + 7) / 8) * 8 * a.n_ntiles;
        if (wgs > 0x7fffffff)
            return hipErrorInvalidValue;
        void *args[] = {&a};
        return hipLaunchKernel(kern, dim3((unsigned)wgs), dim3(64 * WAVES), args, 0, stream);
    }
}

// Tile heights compiled: 32 * {2, 3, 4, 5} rows.
template <int D, int BITS>
struct GemmD {
    template <int NPROJ, int NN>
    static hipError_t by_mb(int mb, const GemmArgs &a, int cap, hipStream_t s)
    {
        return mb == 2 ? gemm_launch<D, BITS, NPROJ, 2, NN>(a, cap, s)
                       : (mb == 3 ? gemm_launch<D, BITS, NPROJ, 3, NN>(a, cap, s)
                                  : gemm_launch<D, BITS, NPROJ, 4, NN>(a, cap, s));
    }
    static hipError_t run(int nproj, int mb, const GemmArgs &a, int cap, hipStream_t s)
    {
        if constexpr (gemm_waves(BITS) == 8) {
            // two (projection, block) pairs per wave, up to four row blocks
            if (mb > 4)
                return hipErrorInvalidValue;
            return nproj == 2 ? by_mb<2, 1>(mb, a, cap, s) : by_mb<1, 2>(mb, a, cap, s);
        } else {
            // five 32-row blocks: two (projection, block) pairs per wave
            if (mb == 5)
                return nproj == 2 ? gemm_launch<D, BITS, 2, 5, 1>(a, cap, s)
                                  : gemm_launch<D, BITS, 1, 5, 2>(a, cap, s);
            if (nproj == 2)
                return by_mb<2, 2>(mb, a, cap, s);
            return gemm_nn(1, a.rows) == 4 ? by_mb<1, 4>(mb, a, cap, s)
                                           : by_mb<1, 2>(mb, a, cap, s);
        }
    }
};

// Host side of GemmShape: 0 = does not fit, 1 = fits, 2 = fits with loads in
// flight across steps.  The chunk-only layout takes rows of a multiple of
// four groups only.
template <int D, int BITS, int NPROJ, int NN>
inline int gemm_fit_level(int mb, int groups)
{
    constexpr int W = gemm_waves(BITS);
    using S2 = GemmShape<D, BITS, NPROJ, 2, NN, W>;
    using S3 = GemmShape<D, BITS, NPROJ, 3, NN, W>;
    using S4 = GemmShape<D, BITS, NPROJ, 4, NN, W>;
    const bool f = mb == 2 ? S2::FITS : (mb == 3 ? S3::FITS : S4::FITS);
    const bool d = mb == 2 ? S2::DEEP : (mb == 3 ? S3::DEEP : S4::DEEP);
    const bool co = mb == 2 ? S2::CHONLY : (mb == 3 ? S3::CHONLY : S4::CHONLY);
    if (co && (groups & 3) != 0)
        return 0;
    return f ? (d ? 2 : 1) : 0;
}

template <int D, int BITS>
inline int gemm_fit_db(int nproj, int mb, int rows, int groups)
{
    constexpr int W = gemm_waves(BITS);
    if constexpr (W == 8) {
        if (mb > 4)
            return 0;
        return nproj == 2 ? gemm_fit_level<D, BITS, 2, 1>(mb, groups)
                          : gemm_fit_level<D, BITS, 1, 2>(mb, groups);
    } else {
        if (mb == 5) {
            using S = GemmShape<D, BITS, 2, 5, 1, W>;
            using S1 = GemmShape<D, BITS, 1, 5, 2, W>;
            const bool f = nproj == 2 ? S::FITS : S1::FITS;
            const bool d = nproj == 2 ? S::DEEP : S1::DEEP;
            return f ? (d ? 2 : 1) : 0;
        }
        if (nproj == 2)
            return gemm_fit_level<D, BITS, 2, 2>(mb, groups);
        return gemm_nn(1, rows) == 4 ? gemm_fit_level<D, BITS, 1, 4>(mb, groups)
                                     : gemm_fit_level<D, BITS, 1, 2>(mb, groups);
    }
}

template <int D>
inline int gemm_fit_d(int bits, int nproj, int mb, int rows, int groups)
{
    switch (bits) {
    case 8: return gemm_fit_db<D, 8>(nproj, mb, rows, groups);
    case 9: return gemm_fit_db<D, 9>(nproj, mb, rows, groups);
    case 10: return gemm_fit_db<D, 10>(nproj, mb, rows, groups);
    case 11: return gemm_fit_db<D, 11>(nproj, mb, rows, groups);
    case 12: return gemm_fit_db<D, 12>(nproj, mb, rows, groups);
    case 13: return gemm_fit_db<D, 13>(nproj, mb, rows, groups);
    default: return 0;
    }
}

// rows, groups: the weight tensor's rows and 64-column groups per row
inline int gemm_fit(int d, int bits, int nproj, int mb, int rows, int groups)
{
    return d == 2 ? gemm_fit_d<2>(bits, nproj, mb, rows, groups)
                  : (d == 4 ? gemm_fit_d<4>(bits, nproj, mb, rows, groups)
                            : gemm_fit_d<8>(bits, nproj, mb, rows, groups));
}

inline bool gemm_fits(int d, int bits, int nproj, int mb, int rows, int groups)
{
    return gemm_fit(d, bits, nproj, mb, rows, groups) > 0;
}

template <int D>
hipError_t gemm_d(int bits, int nproj, int mb, const GemmArgs &a, int cap, hipStream_t s)
{
#ifdef VQ_GEMM_FAST_BUILD
    // timing builds: only the benchmarked widths (d2: 8 bits, d4: 11 bits)
    if constexpr (D == 2)
        return bits == 8 ? GemmD<D, 8>::run(nproj, mb, a, cap, s) : hipErrorInvalidValue;
    else if constexpr (D == 4)
        return bits == 11 ? GemmD<D, 11>::run(nproj, mb, a, cap, s) : hipErrorInvalidValue;
    else
        return hipErrorInvalidValue;
#else
    switch (bits) {
    case 8: return GemmD<D, 8>::run(nproj, mb, a, cap, s);
    case 9: return GemmD<D, 9>::run(nproj, mb, a, cap, s);
    case 10: return GemmD<D, 10>::run(nproj, mb, a, cap, s);
    case 11: return GemmD<D, 11>::run(nproj, mb, a, cap, s);
    case 12: return GemmD<D, 12>::run(nproj, mb, a, cap, s);
    case 13: return GemmD<D, 13>::run(nproj, mb, a, cap, s);
    default: return hipErrorInvalidValue;
    }
#endif
}

}  // namespace vq
