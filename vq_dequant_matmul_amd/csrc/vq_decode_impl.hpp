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
// down projection.  Routed launches take one grid row per (token, slot)
// pair; a workgroup whose pair is not the first occurrence of its expert
// exits at once, the first occurrence serves every pair routed to that
// expert, so each expert's weights are streamed exactly once.
#pragma once
#include "vq_common.hpp"
#include "vq_internal.hpp"

namespace vq {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

struct RowsArgs {
    const uint32_t *codes[2];
    const uint16_t *scales[2];
    const int32_t *row_map[2];
    const uint16_t *codebook[2];
    int cb_dwords[2];
    int cb_offset[2];   // dword offset of each codebook in LDS
    int rows, groups, wpr;
    int S_log2;         // segment size
    int tile_rows;      // rows per workgroup
    const void *act;
    int64_t act_stride;
    float *out;
    int64_t out_stride;
    int expert, n_act;
    const int32_t *ids;
    int n_slots, act_div;
};

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

// Activations of one lane: NT rows x GPL groups x 32 fp16 pairs, plus the
// factor 2^-k that undoes each (row, group)'s range scaling.
template <int NT, int GPL, bool HL>
struct XRegs {
    f16x2 hi[NT][GPL][32];
    f16x2 lo[HL ? NT : 1][HL ? GPL : 1][HL ? 32 : 1];
    float m[NT][GPL];
};

template <bool F32>
__device__ __forceinline__ void load_act64(const void *base, int64_t off, float (&v)[64])
{
    if constexpr (F32) {
        const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const float *>(base) + off);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint4 q = p[i];
            v[4 * i + 0] = __uint_as_float(q.x);
            v[4 * i + 1] = __uint_as_float(q.y);
            v[4 * i + 2] = __uint_as_float(q.z);
            v[4 * i + 3] = __uint_as_float(q.w);
        }
    } else {
        const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + off);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint4 q = p[i];
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * i + 2 * j + 0] = __uint_as_float(w[j] << 16);
                v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
            }
        }
    }
}

// Scale 64 activations by a power of two so they are fp16 normals, and split
// into fp16 pairs (hi) plus, for fp32 sources, the fp16 residual (lo).
template <bool HL>
__device__ __forceinline__ float to_scaled_pairs(const float (&v)[64], f16x2 (&hi)[32],
                                                 f16x2 (&lo)[HL ? 32 : 1])
{
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i)
        amax = fmaxf(amax, fabsf(v[i]));
    const int k = range_exponent(amax);
    const float up = ldexpf(1.0f, k);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const float a = v[2 * i] * up, b = v[2 * i + 1] * up;
        hi[i] = pack_f16x2(a, b);
        if constexpr (HL)
            lo[i] = pack_f16x2(a - (float)hi[i].x, b - (float)hi[i].y);
    }
    return ldexpf(1.0f, -k);
}

template <int D, int BITS, int GPL, int NPROJ>
struct RowRegs {
    uint32_t w[NPROJ][GPL][Geom<D, BITS>::NW];
    uint32_t sc[NPROJ][GPL];
    int live;   // bit p: projection p's row is stored (not skip-zero)
};

// Wave-level: list of the pairs routed to this workgroup's expert, or an
// empty list when blockIdx.y is not the expert's first occurrence.
__device__ __forceinline__ void build_pair_list(const int *__restrict__ s_ids, int n_slots, int q,
                                                int *__restrict__ s_list, int *__restrict__ s_n)
{
    const int lane = threadIdx.x & 63;
    const int e = s_ids[q];
    bool dup = false;
    for (int i = lane; i < q; i += 64)
        dup |= (s_ids[i] == e);
    if (__ballot(dup) != 0ull) {
        if (lane == 0)
            *s_n = 0;
        return;
    }
    int n = 0;
    for (int base = q; base < n_slots; base += 64) {
        const int i = base + lane;
        const bool m = (i < n_slots) && (s_ids[i] == e);
        const unsigned long long b = __ballot(m);
        if (m)
            s_list[n + __popcll(b & ((1ull << lane) - 1ull))] = i;
        n += __popcll(b);
    }
    if (lane == 0)
        *s_n = n;
}

template <int D, int BITS, int GPL, int NPROJ, bool HL, bool F32, int ITERS, int NT>
__device__ __forceinline__ void compute_chunk(const RowsArgs &a, const uint32_t *__restrict__ lds,
                                              const RowRegs<D, BITS, GPL, NPROJ> (&rr)[ITERS],
                                              const int *__restrict__ list, int c0, int e, int S,
                                              int seg, int sl, int row0, int rpw)
{
    using GM = Geom<D, BITS>;
    constexpr int NW = GM::NW;
    constexpr int G = GM::G;
    constexpr int HP = D / 2;   // fp16 pairs per codebook entry
    (void)e;

    XRegs<NT, GPL, HL> xr;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int item = list ? list[c0 + n] : c0 + n;
        const int64_t arow = list ? (int64_t)(item / a.act_div) : (int64_t)item;
#pragma unroll
        for (int i = 0; i < GPL; ++i) {
            const int g = sl + i * S;
            if (g < a.groups) {
                float v[64];
                load_act64<F32>(a.act, arow * a.act_stride + 64 * g, v);
                xr.m[n][i] = to_scaled_pairs<HL>(v, xr.hi[n][i], xr.lo[HL ? n : 0][HL ? i : 0]);
            } else {
                xr.m[n][i] = 0.0f;
#pragma unroll
                for (int t = 0; t < 32; ++t) {
                    xr.hi[n][i][t] = f16x2{(f16)0.0f, (f16)0.0f};
                    if constexpr (HL)
                        xr.lo[n][i][t] = f16x2{(f16)0.0f, (f16)0.0f};
                }
            }
        }
    }

#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int r = row0 + it * rpw + seg;
        float part[NT][NPROJ];
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int p = 0; p < NPROJ; ++p)
                part[n][p] = 0.0f;
#pragma unroll
        for (int p = 0; p < NPROJ; ++p) {
            const uint32_t *cb = lds + a.cb_offset[p];
#pragma unroll
            for (int i = 0; i < GPL; ++i) {
                const int g = sl + i * S;
                uint32_t nw[NW];
                shift_group_words<D, BITS>(g, rr[it].w[p][i], nw);
                float acc[NT], accl[NT];
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    acc[n] = 0.0f;
                    accl[n] = 0.0f;
                }
#pragma unroll
                for (int t = 0; t < G; ++t) {
                    const uint32_t code = extract<BITS, NW>(nw, t);
                    const Entry<D> en = fetch_entry<D>(cb, code);
#pragma unroll
                    for (int n = 0; n < NT; ++n)
#pragma unroll
                        for (int k = 0; k < HP; ++k) {
                            acc[n] = dot2(en.v[k], xr.hi[n][i][t * HP + k], acc[n]);
                            if constexpr (HL)
                                accl[n] = dot2(en.v[k], xr.lo[n][i][t * HP + k], accl[n]);
                        }
                }
                const float s = half_bits_to_float(rr[it].sc[p][i]);
#pragma unroll
                for (int n = 0; n < NT; ++n)
                    part[n][p] += (HL ? acc[n] + accl[n] : acc[n]) * (s * xr.m[n][i]);
            }
        }
        // segment butterfly (S is uniform)
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int p = 0; p < NPROJ; ++p) {
                float v = part[n][p];
#pragma unroll
                for (int m = 32; m >= 1; m >>= 1)
                    if (m < S)
                        v += __shfl_xor(v, m, 64);
                part[n][p] = v;
            }
        if (sl == 0 && r < a.rows) {
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const int item = list ? list[c0 + n] : c0 + n;
                float val;
                if constexpr (NPROJ == 2)
                    val = (rr[it].live == 3) ? silu_mul(part[n][0], part[n][1]) : 0.0f;
                else
                    val = (rr[it].live & 1) ? part[n][0] : 0.0f;
                a.out[(int64_t)item * a.out_stride + r] = val;
            }
        }
    }
}

template <int D, int BITS, int GPL, int NPROJ, bool HL, bool F32, int ITERS, int NTM>
__global__ __launch_bounds__(kThreads) void k_rows(const RowsArgs a)
{
    using GM = Geom<D, BITS>;
    constexpr int NW = GM::NW;
    extern __shared__ uint32_t lds[];
    __shared__ int s_ids[kMaxSlots];
    __shared__ int s_list[kMaxSlots];
    __shared__ int s_n;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // ---- work list ---------------------------------------------------------
    int e, n_items;
    const int *list = nullptr;
    if (a.ids) {
        for (int i = tid; i < a.n_slots; i += kThreads)
            s_ids[i] = a.ids[i];
        __syncthreads();
        if (wave == 0)
            build_pair_list(s_ids, a.n_slots, blockIdx.y, s_list, &s_n);
        __syncthreads();
        n_items = s_n;
        if (n_items == 0)
            return;
        e = s_ids[blockIdx.y];
        list = s_list;
    } else {
        e = a.expert;
        n_items = a.n_act;
    }

    // ---- issue the loads of this wave's rows --------------------------------
    const int S = 1 << a.S_log2;
    const int rpw = 64 >> a.S_log2;
    const int seg = lane >> a.S_log2;
    const int sl = lane & (S - 1);
    const int row0 = blockIdx.x * a.tile_rows + wave * ITERS * rpw;

    RowRegs<D, BITS, GPL, NPROJ> rr[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int r = row0 + it * rpw + seg;
        rr[it].live = 0;
#pragma unroll
        for (int p = 0; p < NPROJ; ++p) {
            int64_t s = -1;
            if (r < a.rows)
                s = stored_row(a.row_map[p], a.rows, e, r);
            if (s >= 0)
                rr[it].live |= 1 << p;
#pragma unroll
            for (int i = 0; i < GPL; ++i) {
                const int g = sl + i * S;
                if (s >= 0 && g < a.groups) {
                    load_group_raw<D, BITS>(a.codes[p] + s * a.wpr, g, rr[it].w[p][i]);
                    rr[it].sc[p][i] = a.scales[p][s * a.groups + g];
                } else {
#pragma unroll
                    for (int k = 0; k < NW; ++k)
                        rr[it].w[p][i][k] = 0u;
                    rr[it].sc[p][i] = 0u;
                }
            }
        }
    }

    // ---- codebooks -> LDS ------------------------------------------------------
#pragma unroll
    for (int p = 0; p < NPROJ; ++p)
        stage_codebook(lds + a.cb_offset[p], a.codebook[p], a.cb_dwords[p]);
    __syncthreads();

    // ---- activations in chunks of up to NTM rows -------------------------------
    int c0 = 0;
    while (c0 < n_items) {
        const int left = n_items - c0;
        if (NTM >= 4 && left >= 4) {
            compute_chunk<D, BITS, GPL, NPROJ, HL, F32, ITERS, (NTM >= 4 ? 4 : 1)>(
                a, lds, rr, list, c0, e, S, seg, sl, row0, rpw);
            c0 += (NTM >= 4 ? 4 : 1);
        } else if (NTM >= 2 && left >= 2) {
            compute_chunk<D, BITS, GPL, NPROJ, HL, F32, ITERS, (NTM >= 2 ? 2 : 1)>(
                a, lds, rr, list, c0, e, S, seg, sl, row0, rpw);
            c0 += (NTM >= 2 ? 2 : 1);
        } else {
            compute_chunk<D, BITS, GPL, NPROJ, HL, F32, ITERS, 1>(a, lds, rr, list, c0, e, S,
                                                                   seg, sl, row0, rpw);
            c0 += 1;
        }
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
                                                    int groups, int wpr, int e,
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
        const uint32_t code = extract<BITS, GM::NW>(nw, t);
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
                       t.scales, t.codebook, t.row_map, t.rows, t.groups, t.wpr, e, w);
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

constexpr int kIters = 2;

template <int D, int BITS, int GPL, int NPROJ, bool HL, bool F32, int NTM>
static hipError_t rows_launch(const RowsArgs &a, dim3 grid, size_t lds_bytes, hipStream_t stream)
{
    auto kern = k_rows<D, BITS, GPL, NPROJ, HL, F32, kIters, NTM>;
    if (lds_bytes > 65536) {
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)lds_bytes);
        if (err != hipSuccess)
            return err;
    }
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds_bytes, stream, a);
    return hipGetLastError();
}

// Token-chunk width: 1 when every expert serves one activation row, else up
// to 4 rows per pass (fewer when the activations take more registers).
template <int D, int BITS, int GPL, int NPROJ>
static hipError_t rows_act(const RowsArgs &a, bool act_f32, bool multi, dim3 grid, size_t lds,
                           hipStream_t s)
{
    if (act_f32) {
        if (multi)
            return rows_launch<D, BITS, GPL, NPROJ, true, true, (GPL == 1 ? 2 : 1)>(a, grid, lds, s);
        return rows_launch<D, BITS, GPL, NPROJ, true, true, 1>(a, grid, lds, s);
    }
    if (multi)
        return rows_launch<D, BITS, GPL, NPROJ, false, false, (GPL == 1 ? 4 : 2)>(a, grid, lds, s);
    return rows_launch<D, BITS, GPL, NPROJ, false, false, 1>(a, grid, lds, s);
}

template <int D, int BITS>
static hipError_t rows_db(const RowsArgs &a, int gpl, int nproj, bool act_f32, bool multi,
                          dim3 grid, size_t lds, hipStream_t s)
{
    if (gpl == 1)
        return nproj == 2 ? rows_act<D, BITS, 1, 2>(a, act_f32, multi, grid, lds, s)
                          : rows_act<D, BITS, 1, 1>(a, act_f32, multi, grid, lds, s);
    return nproj == 2 ? rows_act<D, BITS, 2, 2>(a, act_f32, multi, grid, lds, s)
                      : rows_act<D, BITS, 2, 1>(a, act_f32, multi, grid, lds, s);
}

template <int D>
struct RowsD {
    template <int BITS>
    static hipError_t run(const RowsArgs &a, int gpl, int nproj, bool f32, bool multi, dim3 grid,
                          size_t lds, hipStream_t s)
    {
        return rows_db<D, BITS>(a, gpl, nproj, f32, multi, grid, lds, s);
    }
};

template <int D>
hipError_t rows_d(int bits, const RowsArgs &a, int gpl, int nproj, bool f32, bool multi,
                         dim3 grid, size_t lds, hipStream_t s)
{
    VQ_BITS_SWITCH(bits, RowsD<D>::template run, a, gpl, nproj, f32, multi, grid, lds, s)
}

}  // namespace vq
