// vq_decode.hip -- bandwidth-bound VQ kernels for small token counts (gfx950).
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
// This file holds the launch logic (grid sizing, LDS layout) for the
// persistent engine in vq_decode_impl.hpp, the slot-ordered combine and the
// fill kernel for tensors with no stored rows.
#include "vq_decode_impl.hpp"

namespace vq {

// Per-subvector-length instantiations live in vq_decode_d{2,4,8}.hip so they
// compile in parallel.
#define VQ_DECL_D(N)                                                                         \
    extern template hipError_t rows_d<N>(int, const RowsArgs &, int, int, int, int64_t, int, \
                                         size_t, hipStream_t);                                \
    extern template hipError_t dequantize_d<N>(const TensorDev &, int, float *, hipStream_t); \
    extern template hipError_t mix_d<N>(int, const MixArgs &, size_t, hipStream_t);
VQ_DECL_D(2)
VQ_DECL_D(4)
VQ_DECL_D(8)
#undef VQ_DECL_D

// --------------------------------------------------------------------------------
// combine: y[t][c] = sum over slots s (in order) of w[t][s] * z[t*k + s][c]
// --------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_combine(const float *__restrict__ z,
                                                 const float *__restrict__ w, int n_tok, int top_k,
                                                 int hidden, float *__restrict__ y, int accumulate)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t n4 = (int64_t)n_tok * hidden / 4;
    if (i >= n4)
        return;
    const int64_t t = (i * 4) / hidden;
    const int64_t c = (i * 4) % hidden;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    // unrolled so the slots' loads are in flight together
#pragma unroll 8
    for (int s = 0; s < top_k; ++s) {
        const float ws = w[t * top_k + s];
        const float4 v = *reinterpret_cast<const float4 *>(z + (t * top_k + s) * hidden + c);
        acc.x += ws * v.x;
        acc.y += ws * v.y;
        acc.z += ws * v.z;
        acc.w += ws * v.w;
    }
    float4 *yp = reinterpret_cast<float4 *>(y + t * hidden + c);
    if (accumulate) {
        const float4 old = *yp;
        acc = make_float4(old.x + acc.x, old.y + acc.y, old.z + acc.z, old.w + acc.w);
    }
    *yp = acc;
}


hipError_t launch_combine(const float *z, const float *w, int n_tok, int top_k, int hidden,
                          float *y, bool accumulate, hipStream_t stream)
{
    const int64_t n4 = (int64_t)n_tok * hidden / 4;
    if (n4 == 0)
        return hipSuccess;
    const int blocks = (int)((n4 + 255) / 256);
    hipLaunchKernelGGL(k_combine, dim3(blocks), dim3(256), 0, stream, z, w, n_tok, top_k, hidden, y,
                       accumulate ? 1 : 0);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_fill_rows(float *__restrict__ out, int n_rows, int cols,
                                                   int64_t stride)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < (int64_t)n_rows * cols)
        out[(i / cols) * stride + i % cols] = 0.0f;
}

static hipError_t launch_fill_rows(float *out, int n_rows, int cols, int64_t stride,
                                   hipStream_t stream)
{
    const int64_t n = (int64_t)n_rows * cols;
    hipLaunchKernelGGL(k_fill_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, out,
                       n_rows, cols, stride);
    return hipGetLastError();
}

// The device's CU count (queried once per device).
static int cu_count()
{
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// The engine's arguments and LDS layout for one launch: codebook 0 at dword
// 0; codebook 1 at 2^bits*d/2 dwords when that offset is at most 32 KiB (the
// kernel then uses it as a constant), else right after codebook 0; the work
// lists last.  Returns the LDS dwords.
static int rows_args(const RowsLaunch &L, RowsArgs &a, int &gpl, int iters)
{
    const TensorDev &t0 = L.t[0];
    gpl = (t0.groups + 63) / 64;
    const int per_lane = (t0.groups + gpl - 1) / gpl;
    int s_log2 = 0;
    while ((1 << s_log2) < per_lane)
        ++s_log2;
    const int rpw = 64 >> s_log2;
    a = RowsArgs{};
    for (int p = 0; p < L.nproj; ++p) {
        a.codes[p] = L.t[p].codes;
        a.scales[p] = L.t[p].scales;
        a.row_map[p] = L.t[p].row_map;
        a.codebook[p] = L.t[p].codebook;
        a.cb_dwords[p] = L.t[p].cb_dwords;
    }
    a.rows = t0.rows;
    a.groups = t0.groups;
    a.wpr = t0.wpr;
    a.S_log2 = s_log2;
    a.iters = iters;
    a.tile_rows = kWaves * iters * rpw;
    a.tiles = (t0.rows + a.tile_rows - 1) / a.tile_rows;
    a.act = L.act;
    a.act_stride = L.act_stride;
    a.out = L.out;
    a.out_stride = L.out_stride;
    a.expert = L.expert;
    a.n_act = L.n_act;
    a.ids = L.ids;
    a.n_slots = L.n_slots;
    a.act_div = (L.ids && L.act_div > 0) ? L.act_div : 1;
    const int P = L.ids ? L.n_slots : L.n_act;
    a.cb_offset[0] = 0;
    const int cb1_fixed = (1 << t0.bits) * t0.d / 2;
    a.cb_offset[1] = (cb1_fixed * 4 <= 32768) ? cb1_fixed : ((L.t[0].cb_dwords + 3) & ~3);
    int off = L.nproj == 2 ? a.cb_offset[1] + L.t[1].cb_dwords : L.t[0].cb_dwords;
    off = (off + 3) & ~3;
    if (t0.d == 2 && t0.bits == 8)   // copies of every entry (rows_banked)
        off = kBankedCbDwords;
    a.list_offset = off;
    return off + list_dwords(P);
}

hipError_t launch_rows(const RowsLaunch &L, hipStream_t stream)
{
    const TensorDev &t0 = L.t[0];
    if (t0.groups > kMaxGroupsDecode)
        return hipErrorInvalidValue;
    RowsArgs a;
    int gpl;
    size_t lds = (size_t)rows_args(L, a, gpl, 2) * 4;
    const int P = L.ids ? L.n_slots : L.n_act;
    if (P == 0 || t0.rows == 0)
        return hipSuccess;
    const int n_cu = cu_count();
    // Two row passes per unit amortise a unit's setup; with bf16 activations
    // and few units (about two per resident workgroup or fewer) one pass per
    // unit spreads the work more evenly over the chip.  (fp32 activations,
    // with their hi + lo terms, stay faster at two passes.)
    if (L.act_f32 == 0 && (int64_t)P * a.tiles < (int64_t)kRowsOnePassUnitsPerCu * n_cu)
        lds = (size_t)rows_args(L, a, gpl, 1) * 4;
    // one projection with many units (the down stage of a few tokens): four
    // row passes per unit, so a unit's fixed work covers twice the rows
    else if (L.nproj == 1 && (int64_t)P * a.tiles >= (int64_t)kRowsFourPassUnitsPerCu * n_cu)
        lds = (size_t)rows_args(L, a, gpl, 4) * 4;
    // a projection whose rows are all dead (skip-zero) stores nothing: every
    // output row it touches is exactly zero (for SwiGLU, silu(0)*u = 0 and
    // silu(g)*0 = 0 are written as +0.0)
    for (int p = 0; p < L.nproj; ++p)
        if (L.t[p].n_stored == 0)
            return launch_fill_rows(L.out, P, t0.rows, L.out_stride, stream);

    const int64_t units = (int64_t)P * a.tiles;
    switch (t0.d) {
    case 2: return rows_d<2>(t0.bits, a, gpl, L.nproj, L.act_f32, units, n_cu, lds, stream);
    case 4: return rows_d<4>(t0.bits, a, gpl, L.nproj, L.act_f32, units, n_cu, lds, stream);
    case 8: return rows_d<8>(t0.bits, a, gpl, L.nproj, L.act_f32, units, n_cu, lds, stream);
    default: return hipErrorInvalidValue;
    }
}

// The fused down projection and combine: everything but the LDS layout.
static void mix_args(const TensorDev &dn, int n_tok, int top_k, const float *h, const int32_t *ids,
                     const float *w, float *y, bool accumulate, MixArgs &a)
{
    int s_log2 = 0;
    while ((1 << s_log2) < dn.groups)
        ++s_log2;
    a.codes = dn.codes;
    a.scales = dn.scales;
    a.row_map = dn.row_map;
    a.codebook = dn.codebook;
    a.cb_dwords = dn.cb_dwords;
    a.rows = dn.rows;
    a.groups = dn.groups;
    a.wpr = dn.wpr;
    a.S_log2 = s_log2;
    a.h = h;
    a.ids = ids;
    a.w = w;
    a.n_tok = n_tok;
    a.top_k = top_k;
    a.y = y;
    a.accumulate = accumulate ? 1 : 0;
    const int rpw = 64 >> s_log2;
    a.units = (dn.rows + rpw - 1) / rpw;
    a.max_wgs = 2 * cu_count();
}

// Its LDS from dword list_off on (the codebook sits below, from dword 0):
// routing lists, staged h, h's factors, the waves' partial sums.  Returns the
// end in dwords (0: not applicable).
static int mix_layout(const TensorDev &dn, int n_tok, int top_k, int list_off, MixArgs &a)
{
    const int P = n_tok * top_k;
    if (dn.groups > 64 || n_tok > 16 || P > kMaxSlots)
        return 0;
    int off = list_off;
    a.list_offset = off;
    off += (list_dwords(P) + 3) & ~3;
    a.x_offset = off;
    off += P * dn.groups * kMixXStride;
    a.m_offset = off;
    off += (P * dn.groups + 3) & ~3;
    a.y_offset = off;
    off += kWaves * 64 * n_tok;
    return (size_t)off * 4 <= 65536 ? off : 0;
}

bool mix_supported(const TensorDev &dn, int n_tok, int top_k)
{
    MixArgs a = {};
    return mix_layout(dn, n_tok, top_k, (dn.cb_dwords + 3) & ~3, a) != 0;
}

hipError_t launch_mix(const TensorDev &dn, int n_tok, int top_k, const float *h,
                      const int32_t *ids, const float *w, float *y, bool accumulate,
                      hipStream_t stream)
{
    if (n_tok == 0 || dn.rows == 0)
        return hipSuccess;
    if (dn.n_stored == 0)   // every row dead: the sum is +0.0
        return accumulate ? hipSuccess : launch_fill_rows(y, n_tok, dn.rows, dn.rows, stream);
    MixArgs a = {};
    const int end = mix_layout(dn, n_tok, top_k, (dn.cb_dwords + 3) & ~3, a);
    if (end == 0)
        return hipErrorInvalidValue;
    mix_args(dn, n_tok, top_k, h, ids, w, y, accumulate, a);
    const size_t lds = (size_t)end * 4;
    switch (dn.d) {
    case 2: return mix_d<2>(dn.bits, a, lds, stream);
    case 4: return mix_d<4>(dn.bits, a, lds, stream);
    case 8: return mix_d<8>(dn.bits, a, lds, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dequantize(const TensorDev &t, int e, float *w, hipStream_t stream)
{
    if ((int64_t)t.rows * t.groups == 0)
        return hipSuccess;
    switch (t.d) {
    case 2: return dequantize_d<2>(t, e, w, stream);
    case 4: return dequantize_d<4>(t, e, w, stream);
    case 8: return dequantize_d<8>(t, e, w, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace vq
