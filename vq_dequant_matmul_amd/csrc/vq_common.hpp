// vq_common.hpp -- device building blocks shared by the VQ kernels (gfx950).
//
// Storage format (model card "Qwen3.5-397B-A17B-VQ-2.6bpw", sections
// "Methodology" and "Sub-byte bit-packing"; "GLM-5.3-Flash-VQ-2.7bpw",
// section "Methodology"):
//   * one b-bit code per d consecutive input weights of an output row;
//   * codes packed LSB-first into row-local uint32 streams of 32-code blocks
//     (one block = exactly b words), rows padded to whole blocks;
//   * one fp16 scale per (row, 64 weights), i.e. per "group";
//   * one fp16 codebook [K][d] per tensor.
//
// A 64-column group holds G = 64/d codes = G*b bits.  Groups start at bit
// offsets that are multiples of G*b inside the row, so a group's first bit
// sits at an offset o in {0, gcd(G*b,32), ...} inside its first word.  The
// kernels give each lane whole groups: the lane loads the NW words that cover
// its group, shifts them so the group starts at bit 0 (v_alignbit), and then
// extracts code t at the compile-time bit position t*b.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vq {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int cgcd(int a, int b) { return b == 0 ? a : cgcd(b, a % b); }

// Compile-time facts about one (d, b) geometry.
template <int D, int BITS>
struct Geom {
    static_assert(D == 2 || D == 4 || D == 8, "d must be 2, 4 or 8");
    static_assert(BITS >= 1 && BITS <= 16, "code width out of range");
    static constexpr int G = 64 / D;                   // codes per group
    static constexpr int GB = G * BITS;                // bits per group
    static constexpr int GPB = 32 / G;                 // groups per 32-code block
    static constexpr int OSTEP = cgcd(GB, 32);         // spacing of start offsets
    static constexpr bool SHIFTED = (GB % 32) != 0;    // some groups start mid-word
    static constexpr int OMAX = SHIFTED ? 32 - OSTEP : 0;
    static constexpr int NW = (OMAX + GB + 31) / 32;   // words loaded per group
    static constexpr uint32_t MASK = (BITS == 32) ? 0xffffffffu : ((1u << BITS) - 1u);
    static constexpr int ENTRY_WORDS = D / 2;          // fp16 codebook entry, in dwords
    // true if the NW words of some group would run past the end of its
    // 32-code block (then the last row's loads must be clamped)
    static constexpr bool overruns()
    {
        for (int q = 0; q < GPB; ++q)
            if (((q * GB) >> 5) + NW > BITS)
                return true;
        return false;
    }
    static constexpr bool CLAMP = overruns();
};

// Word offset (inside the row) and bit offset of group g.
template <int D, int BITS>
__device__ __forceinline__ void group_origin(int g, int &w0, int &o, int &w_end)
{
    using GM = Geom<D, BITS>;
    const int bitpos = g * GM::GB;
    w0 = bitpos >> 5;
    o = bitpos & 31;
    // words of the group's 32-code block end here; loads never pass it
    w_end = (g / GM::GPB + 1) * BITS;
}

// Load the NW words covering group g of a stored row, zero beyond its block,
// and shift them so the group's first bit is bit 0 of nw[0].
template <int D, int BITS>
__device__ __forceinline__ void load_group_words(const uint32_t *__restrict__ row, int g,
                                                 uint32_t (&nw)[Geom<D, BITS>::NW])
{
    using GM = Geom<D, BITS>;
    int w0, o, w_end;
    group_origin<D, BITS>(g, w0, o, w_end);
    uint32_t w[GM::NW + 1];
#pragma unroll
    for (int i = 0; i < GM::NW; ++i)
        w[i] = (w0 + i < w_end) ? __builtin_nontemporal_load(row + w0 + i) : 0u;
    w[GM::NW] = 0u;
    if constexpr (GM::SHIFTED) {
#pragma unroll
        for (int i = 0; i < GM::NW; ++i)
            nw[i] = __builtin_amdgcn_alignbit(w[i + 1], w[i], o);
    } else {
#pragma unroll
        for (int i = 0; i < GM::NW; ++i)
            nw[i] = w[i];
    }
}

// Raw (unshifted) words of group g, for kernels that issue every load of a
// tile before touching any of them.
template <int D, int BITS>
__device__ __forceinline__ void load_group_raw(const uint32_t *__restrict__ row, int g,
                                               uint32_t (&w)[Geom<D, BITS>::NW])
{
    using GM = Geom<D, BITS>;
    int w0, o, w_end;
    group_origin<D, BITS>(g, w0, o, w_end);
#pragma unroll
    for (int i = 0; i < GM::NW; ++i)
        w[i] = (w0 + i < w_end) ? __builtin_nontemporal_load(row + w0 + i) : 0u;
}

template <int D, int BITS>
__device__ __forceinline__ void shift_group_words(int g, const uint32_t (&w)[Geom<D, BITS>::NW],
                                                  uint32_t (&nw)[Geom<D, BITS>::NW])
{
    using GM = Geom<D, BITS>;
    if constexpr (GM::SHIFTED) {
        const int o = (g * GM::GB) & 31;
#pragma unroll
        for (int i = 0; i < GM::NW; ++i)
            nw[i] = __builtin_amdgcn_alignbit(i + 1 < GM::NW ? w[i + 1] : 0u, w[i], o);
    } else {
#pragma unroll
        for (int i = 0; i < GM::NW; ++i)
            nw[i] = w[i];
    }
}

// Code t (compile-time) of a group whose bits start at bit 0 of nw[0].
template <int BITS, int T, int NW>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&nw)[NW])
{
    constexpr int p = T * BITS;
    constexpr int wi = p >> 5;
    constexpr int sh = p & 31;
    constexpr uint32_t mask = (1u << BITS) - 1u;
    if constexpr (sh + BITS <= 32) {
        return (nw[wi] >> sh) & mask;
    } else {
        return __builtin_amdgcn_alignbit(nw[wi + 1], nw[wi], sh) & mask;
    }
}

// ---- number formats ---------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b)
{
    return __uint_as_float(b << 16);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h)
{
    union { uint16_t u; f16 f; } v;
    v.u = (uint16_t)h;
    return (float)v.f;
}

// Power-of-two range scale for a block of activations: returns k such that
// max|x| * 2^k lies in [2^14, 2^15), so every scaled value is an fp16 normal
// (bf16 values then convert exactly); 0 for an all-zero block.  k is at most
// 126, so 2^k and 2^-k are both normal fp32 numbers: a block whose largest
// magnitude is below 2^-111 is scaled by 2^126 only (its small values then
// round in fp16 as subnormals instead of overflowing the scale).
__device__ __forceinline__ int range_exponent(float amax)
{
    if (!(amax > 0.0f))
        return 0;
    int ex;
    (void)frexpf(amax, &ex);   // amax = f * 2^ex, f in [0.5, 1)
    return min(15 - ex, 126);
}

__device__ __forceinline__ f16x2 pack_f16x2(float a, float b)
{
    f16x2 r;
    r.x = (f16)a;
    r.y = (f16)b;
    return r;
}

__device__ __forceinline__ float dot2(uint32_t cb_pair, f16x2 x, float acc)
{
    union { uint32_t u; f16x2 h; } c;
    c.u = cb_pair;
    return __builtin_amdgcn_fdot2(c.h, x, acc, false);
}

// ---- wavefront helpers ------------------------------------------------------

// v combined with lane (l ^ 1), (l ^ 2) (quad permutations), then across
// the halves of each 8-lane group and of each 16-lane row (half-mirror and
// mirror): DPP moves, so no LDS traffic.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}

// Sum over aligned segments of S lanes (S a power of two <= 64, uniform);
// every lane of a segment receives the segment's sum.  Steps inside a
// 16-lane row use DPP, wider ones a cross-lane permute.
__device__ __forceinline__ float segment_sum_dpp(float v, int S)
{
    if (S >= 2)
        v += dpp_move<0xb1>(v);    // quad_perm [1,0,3,2]
    if (S >= 4)
        v += dpp_move<0x4e>(v);    // quad_perm [2,3,0,1]
    if (S >= 8)
        v += dpp_move<0x141>(v);   // row_half_mirror
    if (S >= 16)
        v += dpp_move<0x140>(v);   // row_mirror
    // across 16-lane rows: v_permlane16_swap / v_permlane32_swap exchange
    // rows (halves) between two registers without going through LDS.  With
    // both operands v, the two results hold the pair's two rows (halves) in
    // every lane, so their sum is the same in all lanes.
    if (S >= 32) {
        const uint32_t u = __float_as_uint(v);
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    if (S >= 64) {
        const uint32_t u = __float_as_uint(v);
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return v;
}

// n / d for a 64-bit n that nearly always fits 32 bits: the 32-bit
// division is a short instruction sequence, the 64-bit one a long loop.
__device__ __forceinline__ uint64_t udiv_small(uint64_t n, uint32_t d)
{
    if (n <= 0xffffffffull)
        return (uint32_t)n / d;
    return n / d;
}

// A load through the global address space (a pointer the compiler cannot
// place would otherwise take a flat load, whose completion it tracks less
// precisely).
template <class T>
__device__ __forceinline__ T load_global(const T *p)
{
    return *(const __attribute__((address_space(1))) T *)p;
}

// Largest value over aligned segments of 16 lanes (every lane gets it).
__device__ __forceinline__ float segment_max16_dpp(float v)
{
    v = fmaxf(v, dpp_move<0xb1>(v));    // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp_move<0x4e>(v));    // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_move<0x141>(v));   // row_half_mirror
    v = fmaxf(v, dpp_move<0x140>(v));   // row_mirror
    return v;
}

// Stage a tensor's codebook (K*d fp16 = K*d/2 dwords) into LDS.
__device__ __forceinline__ void stage_codebook(uint32_t *__restrict__ lds,
                                               const uint16_t *__restrict__ cb, int n_dwords)
{
    const uint32_t *src = reinterpret_cast<const uint32_t *>(cb);
    for (int i = threadIdx.x; i < n_dwords; i += blockDim.x)
        lds[i] = src[i];
}

__device__ __forceinline__ int64_t stored_row(const int32_t *__restrict__ row_map, int rows,
                                              int e, int r)
{
    const int64_t lin = (int64_t)e * rows + r;
    return row_map ? (int64_t)row_map[lin] : lin;
}

__device__ __forceinline__ float silu_mul(float g, float u)
{
    return g / (1.0f + __expf(-g)) * u;
}

// The same with the hardware reciprocal (about 1 ulp) in place of the
// correctly rounded division.
__device__ __forceinline__ float silu_mul_fast(float g, float u)
{
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

}  // namespace vq
