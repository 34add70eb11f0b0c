// vq_prefill_impl.hpp -- grouped MFMA GEMM over VQ expert weights (gfx950).
//
// For a batch of many tokens every routed expert sees a block of rows, and
// the expert matmul becomes a ragged grouped GEMM (the model cards' runtime
// dequantises in chunks before its prefill matmul: card
// "gemma-4-26b-a4b-it-VQ-6.2bpw", section "Faster prefill"; its large
// codebooks get a dedicated kernel arm: card "Qwen3.5-397B-A17B-VQ-2.4bpw:
// Model Card", changelog 2026-09-09).  Here:
//
//   * a workgroup owns one tile (expert, up to 32*MB of its grouped rows)
//     and 128 consecutive weight rows; its four waves own 32 weight rows
//     each, of one projection or of gate and up together (so the SwiGLU
//     product is formed in the epilogue);
//   * the K loop walks 64-column groups.  The weights never pass through
//     LDS: each lane decodes exactly its own v_mfma_f32_32x32x16_f16 B
//     operand (8 consecutive columns of one weight row per 16-column slice)
//     from the code stream, looks the entries up in the LDS codebook and
//     scales them by the group's fp16 scale with packed fp16 multiplies;
//   * the activation rows of the tile are staged once per group into a
//     double-buffered LDS tile as fp16, each row multiplied by a power of
//     two chosen from its largest magnitude (exact for bf16 inputs); row
//     stride 72 halves keeps the 16-byte fragment reads free of bank
//     conflicts;
//   * the next group's code words and activations are loaded while the
//     current group's MFMAs run; one barrier per group.
#pragma once

#include "vq_common.hpp"
#include "vq_internal.hpp"

namespace vq {

constexpr int kGemmWaves = 4;
constexpr int kGemmThreads = 64 * kGemmWaves;
constexpr int kGemmN = 32 * kGemmWaves;     // weight rows per workgroup
constexpr int kAStride = 72;                // halves per staged activation row

struct GemmArgs {
    const uint32_t *codes[2];
    const uint16_t *scales[2];
    const int32_t *row_map[2];
    const uint16_t *codebook[2];
    int cb_dwords[2];
    int cb_offset1;        // LDS dword offset of codebook 1
    int a_offset;          // LDS dword offset of the activation tiles
    int rows, cols, groups, wpr;
    // activations: row of grouped position p is perm[p] / act_div (perm NULL:
    // p itself); amax[row] holds the bits of the row's largest magnitude
    const void *act;
    int64_t act_stride;
    const int32_t *perm;
    int act_div;
    const uint32_t *amax;
    // tiles: [n][3] = expert, first grouped position, row count
    const int32_t *tiles;
    const int32_t *n_tiles;
    // output rows are grouped positions
    float *out;
    int64_t out_stride;
    uint32_t *out_amax;    // swiglu: largest |h| of each output row (atomic max)
};

// Per-lane code pattern of the B operand.  In slice j (16 columns) lane l
// supplies columns 16j + 8*(l/32) + [0, 8) of its weight row, i.e. codes
// first(l) + j*SLICE + [0, PER) with:
template <int D, int BITS>
struct BFrag {
    static constexpr int PER = 8 / D;                 // codes per slice per lane
    static constexpr int SLICE = 16 / D;              // code stride between slices
    static constexpr int HOFF = 8 / D;                // first code of the upper half-wave
    static constexpr int SPAN = 3 * SLICE + PER;      // codes covered by one lane
    static constexpr int NWB = (31 + SPAN * BITS + 31) / 32;   // words loaded
};

template <int D, int BITS, int NPROJ>
struct BRaw {
    uint32_t w[NPROJ][BFrag<D, BITS>::NWB];
    uint32_t sc[NPROJ];
    int live;
};

// Load the code words this lane needs for group g of its weight row.
template <int D, int BITS, int NPROJ>
__device__ __forceinline__ void load_b(const GemmArgs &a, int e, int n, int h, int g,
                                       BRaw<D, BITS, NPROJ> &br)
{
    using BF = BFrag<D, BITS>;
    const int64_t lin = (int64_t)e * a.rows + min(n, a.rows - 1);
    br.live = 0;
#pragma unroll
    for (int p = 0; p < NPROJ; ++p) {
        const int s = a.row_map[p] ? a.row_map[p][lin] : (int)lin;
        const bool live = (n < a.rows) && (s >= 0);
        br.live |= live ? (1 << p) : 0;
        const int64_t sr = live ? s : 0;
        const uint32_t *row = a.codes[p] + sr * a.wpr;
        const int bit0 = g * (64 / D) * BITS + h * BF::HOFF * BITS;
        const int w0 = bit0 >> 5;
#pragma unroll
        for (int k = 0; k < BF::NWB; ++k)
            br.w[p][k] = row[min(w0 + k, a.wpr - 1)];
        br.sc[p] = a.scales[p][sr * a.groups + g];
    }
}

// Decode this lane's B operand for one projection: 4 slices x 8 halves.
template <int D, int BITS>
__device__ __forceinline__ void decode_b(const uint32_t (&w)[BFrag<D, BITS>::NWB], int shift,
                                         uint32_t sc_bits, bool live,
                                         const uint32_t *__restrict__ cb, f16x8 (&bf)[4])
{
    using BF = BFrag<D, BITS>;
    constexpr int NW = BF::NWB;
    uint32_t nw[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i)
        nw[i] = __builtin_amdgcn_alignbit(i + 1 < NW ? w[i + 1] : 0u, w[i], shift);
    union { uint32_t u; f16x2 h; } sc;
    sc.u = live ? (sc_bits & 0xffffu) * 0x10001u : 0u;   // (s, s), or 0 for a dead row
    constexpr uint32_t mask = (1u << BITS) - 1u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        union { f16x8 v; f16x2 p[4]; uint32_t u[4]; } o;
#pragma unroll
        for (int c = 0; c < BF::PER; ++c) {
            const int t = j * BF::SLICE + c;          // compile-time code position
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
            o.p[k] = o.p[k] * sc.h;                   // v_pk_mul_f16: fp16(s * c)
        bf[j] = o.v;
    }
}

// Activation staging: one 64-column group of the tile's rows.
template <int MB, bool AF32>
struct ARaw {
    // bf16: 8 threads per row (16 bytes each), 32 rows per pass;
    // fp32: 16 threads per row, 16 rows per pass
    static constexpr int TPR = AF32 ? 16 : 8;
    static constexpr int PASSES = 32 * MB / (kGemmThreads / TPR);
    uint4 q[PASSES];
    int k[PASSES];   // power-of-two exponent of each staged row
};

template <int MB, bool AF32>
__device__ __forceinline__ void load_a(const GemmArgs &a, int m0, int mlen, int g,
                                       ARaw<MB, AF32> &ar)
{
    using AR = ARaw<MB, AF32>;
    const int tid = threadIdx.x;
    const int sub = tid % AR::TPR;
#pragma unroll
    for (int ps = 0; ps < AR::PASSES; ++ps) {
        const int i = ps * (kGemmThreads / AR::TPR) + tid / AR::TPR;   // row of the tile
        const int p = m0 + min(i, mlen - 1);                            // grouped position
        const int row = a.perm ? a.perm[p] / a.act_div : p;
        const int64_t off = (int64_t)row * a.act_stride + 64 * g + (AF32 ? 4 : 8) * sub;
        ar.q[ps] = AF32 ? *reinterpret_cast<const uint4 *>(static_cast<const float *>(a.act) + off)
                        : *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.act) + off);
        ar.k[ps] = range_exponent(__uint_as_float(a.amax[row]));
    }
}

template <int MB, bool AF32>
__device__ __forceinline__ void store_a(const ARaw<MB, AF32> &ar, f16 *__restrict__ at)
{
    using AR = ARaw<MB, AF32>;
    const int tid = threadIdx.x;
    const int sub = tid % AR::TPR;
#pragma unroll
    for (int ps = 0; ps < AR::PASSES; ++ps) {
        const int i = ps * (kGemmThreads / AR::TPR) + tid / AR::TPR;
        const float up = ldexpf(1.0f, ar.k[ps]);
        const uint32_t w4[4] = {ar.q[ps].x, ar.q[ps].y, ar.q[ps].z, ar.q[ps].w};
        if constexpr (AF32) {
            union { f16x4 v; uint2 u; } o;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                o.v[c] = (f16)(__uint_as_float(w4[c]) * up);
            *reinterpret_cast<uint2 *>(at + i * kAStride + 4 * sub) = o.u;
        } else {
            union { f16x8 v; uint4 u; } o;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                o.v[2 * c] = (f16)(__uint_as_float(w4[c] << 16) * up);
                o.v[2 * c + 1] = (f16)(__uint_as_float(w4[c] & 0xffff0000u) * up);
            }
            *reinterpret_cast<uint4 *>(at + i * kAStride + 8 * sub) = o.u;
        }
    }
}

template <int D, int BITS, int NPROJ, int MB, bool AF32>
__global__ __launch_bounds__(kGemmThreads) void k_gemm(const GemmArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
    const int tile = blockIdx.y;
    if (tile >= *a.n_tiles)
        return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int e = a.tiles[3 * tile + 0];
    const int m0 = a.tiles[3 * tile + 1];
    const int mlen = a.tiles[3 * tile + 2];
    const int nblk = (mlen + 31) / 32;                 // active 32-row blocks (<= MB)
    const int n = blockIdx.x * kGemmN + 32 * wave + (lane & 31);   // this lane's weight row
    const int h = lane >> 5;

    // codebooks -> LDS (once)
#pragma unroll
    for (int p = 0; p < NPROJ; ++p) {
        uint32_t *dst = lds + (p == 0 ? 0 : a.cb_offset1);
        const uint4 *src = reinterpret_cast<const uint4 *>(a.codebook[p]);
        const int n4 = a.cb_dwords[p] >> 2;
        for (int i = tid; i < n4; i += kGemmThreads)
            reinterpret_cast<uint4 *>(dst)[i] = src[i];
        const uint32_t *s32 = reinterpret_cast<const uint32_t *>(a.codebook[p]);
        for (int i = (n4 << 2) + tid; i < a.cb_dwords[p]; i += kGemmThreads)
            dst[i] = s32[i];
    }
    f16 *abuf = reinterpret_cast<f16 *>(lds + a.a_offset);
    constexpr int ABUF = 32 * MB * kAStride;           // halves per buffer

    using BF = BFrag<D, BITS>;
    // lane-specific funnel shift of its code window
    const int G = a.groups;
    f32x16 accg[MB], accu[NPROJ == 2 ? MB : 1];
#pragma unroll
    for (int b = 0; b < MB; ++b) {
        accg[b] = f32x16{};
        if constexpr (NPROJ == 2)
            accu[b] = f32x16{};
    }

    BRaw<D, BITS, NPROJ> br;
    ARaw<MB, AF32> ar;
    load_b<D, BITS, NPROJ>(a, e, n, h, 0, br);
    load_a<MB, AF32>(a, m0, mlen, 0, ar);
    store_a<MB, AF32>(ar, abuf);
    __syncthreads();

    for (int g = 0; g < G; ++g) {
        const int shift = (g * (64 / D) * BITS + h * BF::HOFF * BITS) & 31;
        // B operands of this group from the words loaded last iteration
        f16x8 bg[4], bu[NPROJ == 2 ? 4 : 1];
        decode_b<D, BITS>(br.w[0], shift, br.sc[0], (br.live & 1) != 0, lds, bg);
        if constexpr (NPROJ == 2)
            decode_b<D, BITS>(br.w[1], shift, br.sc[1], (br.live & 2) != 0, lds + a.cb_offset1, bu);
        // next group's words and activations in flight during the MFMAs
        const bool more = g + 1 < G;
        if (more) {
            load_b<D, BITS, NPROJ>(a, e, n, h, g + 1, br);
            load_a<MB, AF32>(a, m0, mlen, g + 1, ar);
        }
        const f16 *at = abuf + (g & 1) * ABUF;
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            if (b < nblk) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f16x8 av = *reinterpret_cast<const f16x8 *>(
                        at + (32 * b + (lane & 31)) * kAStride + 16 * j + 8 * h);
                    accg[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bg[j], accg[b], 0, 0, 0);
                    if constexpr (NPROJ == 2)
                        accu[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bu[j], accu[b], 0, 0, 0);
                }
            }
        }
        if (more)
            store_a<MB, AF32>(ar, abuf + ((g + 1) & 1) * ABUF);
        __syncthreads();
    }

    // epilogue: lane holds D[8*(r/4) + 4*h + r%4][lane%32] of each block;
    // undo the activation row's power-of-two scaling, form silu(g)*u for
    // gate+up, write fp32, and (gate+up) fold each row's largest |h| into
    // out_amax so the next GEMM can scale that row into fp16
    const int col = n;
    const bool colok = col < a.rows;
#pragma unroll
    for (int b = 0; b < MB; ++b) {
        if (b >= nblk)
            continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = 32 * b + 8 * (r / 4) + 4 * h + (r % 4);
            const bool rowok = i < mlen;
            const int p = m0 + min(i, mlen - 1);
            const int row = a.perm ? a.perm[p] / a.act_div : p;
            const float down = ldexpf(1.0f, -range_exponent(__uint_as_float(a.amax[row])));
            float v;
            if constexpr (NPROJ == 2)
                v = (br.live == 3) ? silu_mul(accg[b][r] * down, accu[b][r] * down) : 0.0f;
            else
                v = (br.live & 1) ? accg[b][r] * down : 0.0f;
            if (colok && rowok)
                a.out[(int64_t)(m0 + i) * a.out_stride + col] = v;
            if constexpr (NPROJ == 2) {
                if (a.out_amax) {
                    // max over the 32 columns this half-wave holds for row i
                    float m = (colok && rowok) ? fabsf(v) : 0.0f;
#pragma unroll
                    for (int o = 16; o >= 1; o >>= 1)
                        m = fmaxf(m, __shfl_xor(m, o, 64));
                    if ((lane & 31) == 0 && rowok)
                        atomicMax(a.out_amax + (m0 + i), __float_as_uint(m));
                }
            }
        }
    }
}

// ---- dispatch ------------------------------------------------------------------

template <int D, int BITS, int NPROJ, int MB, bool AF32>
static hipError_t gemm_launch(const GemmArgs &a, dim3 grid, size_t lds, hipStream_t stream)
{
    auto kern = k_gemm<D, BITS, NPROJ, MB, AF32>;
    if (lds > 65536) {
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess)
            return err;
    }
    hipLaunchKernelGGL(kern, grid, dim3(kGemmThreads), lds, stream, a);
    return hipGetLastError();
}

template <int D, int BITS, int NPROJ>
static hipError_t gemm_np(int mb, bool af32, const GemmArgs &a, dim3 grid, size_t lds,
                          hipStream_t s)
{
    if (mb == 6)
        return af32 ? gemm_launch<D, BITS, NPROJ, 6, true>(a, grid, lds, s)
                    : gemm_launch<D, BITS, NPROJ, 6, false>(a, grid, lds, s);
    return af32 ? gemm_launch<D, BITS, NPROJ, 4, true>(a, grid, lds, s)
                : gemm_launch<D, BITS, NPROJ, 4, false>(a, grid, lds, s);
}

template <int D>
struct GemmD {
    template <int BITS>
    static hipError_t run(int nproj, int mb, bool af32, const GemmArgs &a, dim3 grid, size_t lds,
                          hipStream_t s)
    {
        return nproj == 2 ? gemm_np<D, BITS, 2>(mb, af32, a, grid, lds, s)
                          : gemm_np<D, BITS, 1>(mb, af32, a, grid, lds, s);
    }
};

template <int D>
hipError_t gemm_d(int bits, int nproj, int mb, bool af32, const GemmArgs &a, dim3 grid, size_t lds,
                  hipStream_t s)
{
    switch (bits) {
    case 8: return GemmD<D>::template run<8>(nproj, mb, af32, a, grid, lds, s);
    case 9: return GemmD<D>::template run<9>(nproj, mb, af32, a, grid, lds, s);
    case 10: return GemmD<D>::template run<10>(nproj, mb, af32, a, grid, lds, s);
    case 11: return GemmD<D>::template run<11>(nproj, mb, af32, a, grid, lds, s);
    case 12: return GemmD<D>::template run<12>(nproj, mb, af32, a, grid, lds, s);
    case 13: return GemmD<D>::template run<13>(nproj, mb, af32, a, grid, lds, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace vq
