// vq_prefill.hip -- routing, tiling and launch of the grouped MFMA GEMM path.
//
// A batch of many tokens is regrouped by expert (the routing of the model
// cards: 10 of 512 experts on "Qwen3.8-Flash-Next-VQ-4.4bpw", top-8 of 128 on
// "gemma-4-26b-a4b-it-VQ-6.2bpw"): counts per expert, an exclusive scan, and
// a scatter of every (token, slot) pair to its grouped position.  The order
// of pairs inside one expert's block is not fixed (atomic slots), but no
// output depends on it: every output row is computed on its own and the
// final combine sums each token's slots in slot order.
#include <algorithm>
#include <cmath>

#include "vq_prefill_impl.hpp"

namespace vq {

#define VQ_DECL_GEMM(N) \
    extern template hipError_t gemm_d<N>(int, int, int, const GemmArgs &, int, hipStream_t);
VQ_DECL_GEMM(2)
VQ_DECL_GEMM(4)
VQ_DECL_GEMM(8)
#undef VQ_DECL_GEMM

constexpr int kRouteThreads = 1024;
// ids per thread loaded together; a batch of up to kRouteThreads *
// kRouteBatch pairs stays in registers from the count to the scatter, so
// the single routing workgroup waits for the ids once instead of once per
// pass and batch (the rest of the chip is streaming activations meanwhile,
// so each round trip is long)
constexpr int kRouteBatch = 48;
constexpr int kMaxRouteExperts = 4096;

// Exclusive scan of v[0..n) in place (n <= 4 * kRouteThreads); returns the
// total.  Called by all threads of the block; uses 16 + 1 ints of scratch.
__device__ int block_exclusive_scan(int *v, int n, int *scratch)
{
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    constexpr int ITEMS = 4;
    int local[ITEMS];
    int sum = 0;
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
        const int i = tid * ITEMS + k;
        local[k] = (i < n) ? v[i] : 0;
        sum += local[k];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o, 64);
        if (lane >= o)
            incl += t;
    }
    if (lane == 63)
        scratch[wave] = incl;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int w = 0; w < kRouteThreads / 64; ++w) {
            const int t = scratch[w];
            scratch[w] = run;
            run += t;
        }
        scratch[16] = run;
    }
    __syncthreads();
    int run = scratch[wave] + incl - sum;
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
        const int i = tid * ITEMS + k;
        if (i < n)
            v[i] = run;
        run += local[k];
    }
    const int total = scratch[16];
    __syncthreads();
    return total;
}

// Tiles of at most mt rows per expert: full tiles, then the remainder
// (fewest 32-row blocks in total): tiles[t] = (expert, first grouped
// position, rows).  cnt, offs, toff: LDS arrays of E.
__device__ void build_tiles(const int *cnt, const int *offs, int *toff, int E, int mt,
                            int32_t *tiles, int32_t *n_tiles, int *scratch)
{
    for (int e = threadIdx.x; e < E; e += kRouteThreads)
        toff[e] = (cnt[e] + mt - 1) / mt;
    __syncthreads();
    const int total = block_exclusive_scan(toff, E, scratch);
    for (int e = threadIdx.x; e < E; e += kRouteThreads) {
        const int c = cnt[e];
        const int nt = (c + mt - 1) / mt;
        for (int j = 0; j < nt; ++j) {
            const int t = toff[e] + j;
            tiles[3 * t + 0] = e;
            tiles[3 * t + 1] = offs[e] + j * mt;
            tiles[3 * t + 2] = min(mt, c - j * mt);
        }
    }
    if (threadIdx.x == 0)
        *n_tiles = total;
}

// Route grouping for the MoE FFN: pairs q = t*top_k + s by expert; pos[q]
// receives the pair's grouped position (its inverse is k_invert_pos).
__device__ __forceinline__ void route_body(const int32_t *__restrict__ ids, int P, int E, int mt,
                                           int32_t *__restrict__ offs, int32_t *__restrict__ pos,
                                           int32_t *__restrict__ tiles,
                                           int32_t *__restrict__ n_tiles)
{
    extern __shared__ int s[];
    int *cnt = s, *base = s + E, *fill = s + 2 * E, *toff = s + 3 * E, *scratch = s + 4 * E;
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kRouteThreads) {
        cnt[e] = 0;
        fill[e] = 0;
    }
    __syncthreads();
    // the ids are read kRouteBatch per thread at a time, so their loads are
    // in flight together instead of one round trip per id; a single batch
    // is kept for the scatter below
    const bool held = P <= kRouteThreads * kRouteBatch;
    int id[kRouteBatch];
    for (int q0 = 0; q0 < P; q0 += kRouteThreads * kRouteBatch) {
#pragma unroll
        for (int k = 0; k < kRouteBatch; ++k) {
            const int q = q0 + k * kRouteThreads + tid;
            id[k] = q < P ? ids[q] : 0;
        }
#pragma unroll
        for (int k = 0; k < kRouteBatch; ++k)
            if (q0 + k * kRouteThreads + tid < P)
                atomicAdd(&cnt[id[k]], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += kRouteThreads)
        base[e] = cnt[e];
    __syncthreads();
    const int total = block_exclusive_scan(base, E, scratch);
    for (int e = tid; e < E; e += kRouteThreads)
        offs[e] = base[e];
    if (tid == 0)
        offs[E] = total;
    for (int q0 = 0; q0 < P; q0 += kRouteThreads * kRouteBatch) {
        if (!held) {
#pragma unroll
            for (int k = 0; k < kRouteBatch; ++k) {
                const int q = q0 + k * kRouteThreads + tid;
                id[k] = q < P ? ids[q] : 0;
            }
        }
#pragma unroll
        for (int k = 0; k < kRouteBatch; ++k) {
            const int q = q0 + k * kRouteThreads + tid;
            if (q < P) {
                const int p = base[id[k]] + atomicAdd(&fill[id[k]], 1);
                pos[q] = p;
            }
        }
    }
    __syncthreads();
    build_tiles(cnt, base, toff, E, mt, tiles, n_tiles, scratch);
}

// Tiles for a grouped GEMM whose rows are already grouped by expert.
__global__ __launch_bounds__(kRouteThreads) void k_tiles_from_offsets(
    const int32_t *__restrict__ expert_offsets, int E, int mt, int32_t *__restrict__ tiles,
    int32_t *__restrict__ n_tiles)
{
    extern __shared__ int s[];
    int *cnt = s, *base = s + E, *toff = s + 2 * E, *scratch = s + 3 * E;
    for (int e = threadIdx.x; e < E; e += kRouteThreads) {
        base[e] = expert_offsets[e];
        cnt[e] = max(0, expert_offsets[e + 1] - expert_offsets[e]);
    }
    __syncthreads();
    build_tiles(cnt, base, toff, E, mt, tiles, n_tiles, scratch);
}

// Each row scaled by a power of two that puts its largest magnitude in
// [2^14, 2^15) and converted to fp16 (exact for bf16 input in fp16's normal
// range, rounded to nearest for fp32); k[row] receives the exponent.  One
// wave per row.
// Rows of up to kRowRegs 16-byte chunks per lane are read once (the chunks
// stay in registers between the max and the conversion); longer rows read
// the rest again.
constexpr int kRowRegs = 8;

__device__ __forceinline__ void rowscale_row(const void *__restrict__ x, int f32, int rows,
                                             int cols, int64_t stride, f16 *__restrict__ out,
                                             int32_t *__restrict__ k, int row)
{
    const int lane = threadIdx.x & 63;
    if (row >= rows)
        return;
    f16 *o = out + (int64_t)row * cols;
    // elements per 16-byte chunk and per pass of the wave
    const int per = f32 ? 4 : 8;
    const int step = 64 * per;
    const char *p = static_cast<const char *>(x) + (int64_t)row * stride * (f32 ? 4 : 2);
    const int esz = f32 ? 4 : 2;
    auto absmax = [&](const uint4 &q) -> uint32_t {
        if (f32)
            return max(max(q.x & 0x7fffffffu, q.y & 0x7fffffffu),
                       max(q.z & 0x7fffffffu, q.w & 0x7fffffffu));
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            m = max(m, max((w[j] & 0x7fffu) << 16, (w[j] >> 16 & 0x7fffu) << 16));
        return m;
    };
    uint4 cache[kRowRegs];
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < kRowRegs; ++i) {
        const int c = lane * per + i * step;
        if (c < cols) {
            cache[i] = *reinterpret_cast<const uint4 *>(p + (int64_t)c * esz);
            mx = max(mx, absmax(cache[i]));
        }
    }
    for (int c = lane * per + kRowRegs * step; c < cols; c += step)
        mx = max(mx, absmax(*reinterpret_cast<const uint4 *>(p + (int64_t)c * esz)));
#pragma unroll
    for (int o2 = 32; o2 >= 1; o2 >>= 1)
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, o2, 64));
    const int ex = range_exponent(__uint_as_float(mx));
    const float up = ldexpf(1.0f, ex);
    auto convert = [&](const uint4 &q, int c) {
        if (f32) {
            union { f16x4 v; uint2 u; } h;
            h.v[0] = (f16)(__uint_as_float(q.x) * up);
            h.v[1] = (f16)(__uint_as_float(q.y) * up);
            h.v[2] = (f16)(__uint_as_float(q.z) * up);
            h.v[3] = (f16)(__uint_as_float(q.w) * up);
            *reinterpret_cast<uint2 *>(o + c) = h.u;
        } else {
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
            union { f16x8 v; uint4 u; } h;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                h.v[2 * j] = (f16)(__uint_as_float(w[j] << 16) * up);
                h.v[2 * j + 1] = (f16)(__uint_as_float(w[j] & 0xffff0000u) * up);
            }
            *reinterpret_cast<uint4 *>(o + c) = h.u;
        }
    };
#pragma unroll
    for (int i = 0; i < kRowRegs; ++i) {
        const int c = lane * per + i * step;
        if (c < cols)
            convert(cache[i], c);
    }
    for (int c = lane * per + kRowRegs * step; c < cols; c += step)
        convert(*reinterpret_cast<const uint4 *>(p + (int64_t)c * esz), c);
    if (lane == 0)
        k[row] = ex;
}

__global__ __launch_bounds__(256) void k_rowscale(const void *__restrict__ x, int f32, int rows,
                                                  int cols, int64_t stride, f16 *__restrict__ out,
                                                  int32_t *__restrict__ k)
{
    rowscale_row(x, f32, rows, cols, stride, out, k, blockIdx.x * 4 + (threadIdx.x >> 6));
}

// perm[pos[q]] = q: the grouped order's source pairs.  The routing
// workgroup writes pos only (in pair order, so its stores are coalesced);
// this scatter of one dword per pair to random lines is spread over many
// workgroups instead of queueing behind one CU's memory pipeline.
__global__ __launch_bounds__(256) void k_invert_pos(const int32_t *__restrict__ pos, int P,
                                                    int32_t *__restrict__ perm)
{
    const int q = blockIdx.x * 256 + threadIdx.x;
    if (q < P)
        perm[pos[q]] = q;
}

// The routing (workgroup 0) and the activation rows' scaling (the other
// workgroups, kRouteThreads / 64 rows each) in one launch: they are
// independent, and the routing alone leaves the rest of the chip idle.
__global__ __launch_bounds__(kRouteThreads) void k_route_rowscale(
    const int32_t *__restrict__ ids, int P, int E, int mt, int32_t *__restrict__ offs,
    int32_t *__restrict__ pos, int32_t *__restrict__ tiles,
    int32_t *__restrict__ n_tiles, const void *__restrict__ x, int f32, int rows, int cols,
    f16 *__restrict__ out, int32_t *__restrict__ k)
{
    if (blockIdx.x == 0) {
        route_body(ids, P, E, mt, offs, pos, tiles, n_tiles);
        return;
    }
    const int row = (blockIdx.x - 1) * (kRouteThreads / 64) + (threadIdx.x >> 6);
    rowscale_row(x, f32, rows, cols, (int64_t)cols, out, k, row);
}

// y[t][c] = sum over slots s (in order) of w[t][s] * z[pos[t*k + s]][c], with
// z the grouped GEMM's fp16 outputs and their exponents:
// z[p][c] = zh[p][c] * 2^-(ze[p][c/64] + hk[p]), hk the exponents of the
// down projection's activation rows.  Eight columns per thread.
__global__ __launch_bounds__(256) void k_combine_perm_h(const f16 *__restrict__ zh,
                                                        const int8_t *__restrict__ ze,
                                                        const int32_t *__restrict__ hk,
                                                        const int32_t *__restrict__ pos,
                                                        const float *__restrict__ w, int n_tok,
                                                        int top_k, int hidden,
                                                        float *__restrict__ y)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t n8 = (int64_t)n_tok * hidden / 8;
    if (i >= n8)
        return;
    const int64_t t = (i * 8) / hidden;
    const int c = (int)((i * 8) % hidden);
    const int nch = hidden >> 6;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int s = 0; s < top_k; ++s) {
        const float ws = w[t * top_k + s];
        const int64_t p = pos[t * top_k + s];
        const int ex = (int)ze[p * nch + (c >> 6)] + hk[p];
        union { uint4 u; f16 v[8]; } q;
        q.u = *reinterpret_cast<const uint4 *>(zh + p * hidden + c);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[j] += ws * ldexpf((float)q.v[j], -ex);
    }
    float4 *o = reinterpret_cast<float4 *>(y + t * hidden + c);
    o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// Zero fill (used when every row of a tensor is dead: the product is zero).
__global__ __launch_bounds__(256) void k_zero(float *__restrict__ p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = 0.0f;
}

// --------------------------------------------------------------------------------
// host side
// --------------------------------------------------------------------------------

static hipError_t launch_zero(float *p, int64_t n, hipStream_t stream)
{
    if (n <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

static hipError_t launch_rowscale(const void *x, int f32, int rows, int cols, f16 *out,
                                  int32_t *k, hipStream_t stream)
{
    if (rows <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_rowscale, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, x, f32,
                       rows, cols, (int64_t)cols, out, k);
    return hipGetLastError();
}

static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// How well the launches of a tile height fit in LDS: the lower of the grouped
// GEMMs' levels (gemm_fit: 0 = no, 1 = yes, 2 = with loads in flight across
// K steps).  For the FFN: gate and up together (or, failing that, apart) and
// the down projection.
static int mb_level(const TensorDev &t, bool ffn, const TensorDev *dn, int mb)
{
    int lv = gemm_fit(t.d, t.bits, ffn ? 2 : 1, mb, t.rows, t.groups);
    if (ffn && lv == 0)
        lv = gemm_fit(t.d, t.bits, 1, mb, t.rows, t.groups);
    if (dn)
        lv = std::min(lv, gemm_fit(dn->d, dn->bits, 1, mb, dn->rows, dn->groups));
    return lv;
}

// Tile height (32-row blocks): the smallest of 2 .. 5 that holds the
// expected largest expert block (mean + 2 standard deviations of a binomial
// count) in one tile, lowered while a smaller height keeps loads in flight
// across K steps and this one does not; larger blocks take several tiles.
static int pick_mb(int64_t rows, int E, const TensorDev &t, bool ffn, const TensorDev *dn)
{
    const double mean = (double)rows / E;
    const double big = mean + 2.0 * sqrt(mean);
    const int want = big <= 64.0 ? 2 : (big <= 96.0 ? 3 : (big <= 128.0 ? 4 : 5));
    for (int mb = want; mb >= 2; --mb)
        if (mb_level(t, ffn, dn, mb) == 2)
            return mb;
    for (int mb = want; mb >= 2; --mb)
        if (mb_level(t, ffn, dn, mb) >= 1)
            return mb;
    return 2;
}

static int64_t max_tiles(int64_t rows, int E, int mt)
{
    return rows / mt + (rows < E ? rows : E) + 1;
}

// gate and up in one launch unless their codebooks leave no room for the ring
static bool fused_gate_up(const TensorDev &g, int mb)
{
    return gemm_fits(g.d, g.bits, 2, mb, g.rows, g.groups);
}

static hipError_t launch_gemm(const TensorDev &t0, const TensorDev *t1, int mb, const f16 *act,
                              int act_stride, const int32_t *act_k, const int32_t *perm,
                              int act_div, const int32_t *tiles, const int32_t *n_tiles,
                              int64_t tile_cap, float *out, int64_t out_stride,
                              const float *gate_in, const int32_t *gate_map, hipStream_t stream,
                              f16 *out_h = nullptr, int8_t *out_e = nullptr)
{
    GemmArgs a = {};
    const TensorDev *ts[2] = {&t0, t1};
    const int nproj = t1 ? 2 : 1;
    for (int p = 0; p < nproj; ++p) {
        a.codes[p] = ts[p]->codes;
        a.scales[p] = ts[p]->scales;
        a.row_map[p] = ts[p]->row_map;
        a.codebook[p] = ts[p]->codebook;
        a.cb_bytes[p] = ts[p]->K * ts[p]->d * 2;
    }
    if (!t1)
        a.row_map[1] = gate_map;
    a.rows = t0.rows;
    a.groups = t0.groups;
    a.wpr = t0.wpr;
    a.act = act;
    a.act_stride = act_stride;
    a.act_k = act_k;
    a.perm = perm;
    a.act_div = act_div > 0 ? act_div : 1;
    a.tiles = tiles;
    a.n_tiles = n_tiles;
    a.gate_in = gate_in;
    a.out = out;
    a.out_stride = out_stride;
    a.out_h = out_h;
    a.out_e = out_e;
    if (out_e && (t1 || out_stride % 64 != 0 || out_stride != t0.rows))
        return hipErrorInvalidValue;
    if (tile_cap > 0x7fffffff || tile_cap < 1)
        return hipErrorInvalidValue;
    a.tile_cap = (int)tile_cap;
    switch (t0.d) {
    case 2: return gemm_d<2>(t0.bits, nproj, mb, a, (int)tile_cap, stream);
    case 4: return gemm_d<4>(t0.bits, nproj, mb, a, (int)tile_cap, stream);
    case 8: return gemm_d<8>(t0.bits, nproj, mb, a, (int)tile_cap, stream);
    default: return hipErrorInvalidValue;
    }
}

// ---- vq_expert_gemm ------------------------------------------------------------

struct GemmWs {
    size_t tiles, n_tiles, xs, xk, total;
    int mb;
    int64_t cap;
};

static GemmWs gemm_ws(const TensorDev &t, int n_x_rows)
{
    GemmWs w;
    w.mb = pick_mb(n_x_rows, t.n_experts, t, false, nullptr);
    w.cap = max_tiles(n_x_rows, t.n_experts, 32 * w.mb);
    size_t o = 0;
    w.tiles = o;
    o = align256(o + (size_t)w.cap * 12);
    w.n_tiles = o;
    o = align256(o + 4);
    w.xs = o;
    o = align256(o + (size_t)n_x_rows * t.cols * 2);
    w.xk = o;
    o = align256(o + (size_t)n_x_rows * 4);
    w.total = o;
    return w;
}

size_t gemm_workspace_bytes(const TensorDev &t, int n_x_rows)
{
    return gemm_ws(t, n_x_rows).total;
}

hipError_t launch_expert_gemm(const TensorDev &t, int n_x_rows, const void *x, int x_f32,
                              const int32_t *expert_offsets, float *y, void *ws,
                              hipStream_t stream)
{
    if (t.n_experts > kMaxRouteExperts)
        return hipErrorNotSupported;
    const GemmWs w = gemm_ws(t, n_x_rows);
    if (!gemm_fits(t.d, t.bits, 1, w.mb, t.rows, t.groups))
        return hipErrorNotSupported;
    char *base = static_cast<char *>(ws);
    int32_t *tiles = reinterpret_cast<int32_t *>(base + w.tiles);
    int32_t *n_tiles = reinterpret_cast<int32_t *>(base + w.n_tiles);
    f16 *xs = reinterpret_cast<f16 *>(base + w.xs);
    int32_t *xk = reinterpret_cast<int32_t *>(base + w.xk);
    const size_t lds_t = (size_t)(3 * t.n_experts + 17) * 4;
    hipLaunchKernelGGL(k_tiles_from_offsets, dim3(1), dim3(kRouteThreads), lds_t, stream,
                       expert_offsets, t.n_experts, 32 * w.mb, tiles, n_tiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (t.n_stored == 0) {
        // every row dead: the product is exactly zero
        return launch_zero(y, (int64_t)n_x_rows * t.rows, stream);
    }
    if ((e = launch_rowscale(x, x_f32, n_x_rows, t.cols, xs, xk, stream)) != hipSuccess)
        return e;
    const KernelEvents &ev = kernel_events();
    if (ev.start)
        (void)hipEventRecord(ev.start, stream);
    e = launch_gemm(t, nullptr, w.mb, xs, t.cols, xk, nullptr, 1, tiles, n_tiles, w.cap, y, t.rows,
                    nullptr, nullptr, stream);
    if (ev.stop)
        (void)hipEventRecord(ev.stop, stream);
    return e;
}

// ---- vq_moe_ffn, many tokens ---------------------------------------------------

struct FfnWs {
    size_t offs, perm, pos, tiles, n_tiles, xs, xk, g, h, hs, hk, zh, ze, total;
    int mb;
    bool fused;
    int64_t cap;
};

static FfnWs ffn_ws(const TensorDev &g, const TensorDev &dn, int n_tok, int top_k)
{
    FfnWs w;
    const int64_t P = (int64_t)n_tok * top_k;
    w.mb = pick_mb(P, g.n_experts, g, true, &dn);
    w.cap = max_tiles(P, g.n_experts, 32 * w.mb);
    w.fused = fused_gate_up(g, w.mb);
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align256(o + bytes);
        return at;
    };
    w.offs = take((size_t)(g.n_experts + 1) * 4);
    w.perm = take((size_t)P * 4);
    w.pos = take((size_t)P * 4);
    w.tiles = take((size_t)w.cap * 12);
    w.n_tiles = take(4);
    w.xs = take((size_t)n_tok * g.cols * 2);
    w.xk = take((size_t)n_tok * 4);
    w.g = take(w.fused ? 0 : (size_t)P * g.rows * 4);
    w.h = take((size_t)P * g.rows * 4);
    w.hs = take((size_t)P * g.rows * 2);
    w.hk = take((size_t)P * 4);
    w.zh = take((size_t)P * dn.rows * 2);
    w.ze = take((size_t)P * (dn.rows / 64));
    w.total = o;
    return w;
}

size_t moe_prefill_workspace_bytes(const TensorDev &g, const TensorDev &, const TensorDev &dn,
                                   int n_tok, int top_k)
{
    return ffn_ws(g, dn, n_tok, top_k).total;
}

hipError_t launch_moe_prefill(const TensorDev &g, const TensorDev &u, const TensorDev &dn,
                              int n_tok, int top_k, const void *x, int x_f32, const int32_t *ids,
                              const float *wts, float *y, void *ws, hipStream_t stream)
{
    if (g.n_experts > kMaxRouteExperts)
        return hipErrorNotSupported;
    const FfnWs w = ffn_ws(g, dn, n_tok, top_k);
    if (!gemm_fits(g.d, g.bits, 1, w.mb, g.rows, g.groups) ||
        !gemm_fits(dn.d, dn.bits, 1, w.mb, dn.rows, dn.groups))
        return hipErrorNotSupported;
    char *base = static_cast<char *>(ws);
    int32_t *offs = reinterpret_cast<int32_t *>(base + w.offs);
    int32_t *perm = reinterpret_cast<int32_t *>(base + w.perm);
    int32_t *pos = reinterpret_cast<int32_t *>(base + w.pos);
    int32_t *tiles = reinterpret_cast<int32_t *>(base + w.tiles);
    int32_t *n_tiles = reinterpret_cast<int32_t *>(base + w.n_tiles);
    f16 *xs = reinterpret_cast<f16 *>(base + w.xs);
    int32_t *xk = reinterpret_cast<int32_t *>(base + w.xk);
    float *gbuf = reinterpret_cast<float *>(base + w.g);
    float *h = reinterpret_cast<float *>(base + w.h);
    f16 *hs = reinterpret_cast<f16 *>(base + w.hs);
    int32_t *hk = reinterpret_cast<int32_t *>(base + w.hk);
    f16 *zh = reinterpret_cast<f16 *>(base + w.zh);
    int8_t *ze = reinterpret_cast<int8_t *>(base + w.ze);
    const int P = n_tok * top_k;
    const int E = g.n_experts;

    // routing and the activation rows' scaling in one launch
    const size_t lds_r = (size_t)(4 * E + 17) * 4;
    const int rs_wgs = (n_tok + kRouteThreads / 64 - 1) / (kRouteThreads / 64);
    hipLaunchKernelGGL(k_route_rowscale, dim3((unsigned)(1 + rs_wgs)), dim3(kRouteThreads), lds_r,
                       stream, ids, P, E, 32 * w.mb, offs, pos, tiles, n_tiles, x, x_f32,
                       n_tok, g.cols, xs, xk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_invert_pos, dim3((unsigned)((P + 255) / 256)), dim3(256), 0, stream, pos,
                       P, perm);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    if (g.n_stored == 0 || u.n_stored == 0 || dn.n_stored == 0)
        return launch_zero(y, (int64_t)n_tok * dn.rows, stream);
    const KernelEvents &ev = kernel_events();
    if (ev.start)
        (void)hipEventRecord(ev.start, stream);
    if (w.fused) {
        e = launch_gemm(g, &u, w.mb, xs, g.cols, xk, perm, top_k, tiles, n_tiles, w.cap, h, g.rows,
                        nullptr, nullptr, stream);
    } else {
        // codebooks too large for one launch: gate first, then up with SwiGLU
        e = launch_gemm(g, nullptr, w.mb, xs, g.cols, xk, perm, top_k, tiles, n_tiles, w.cap, gbuf,
                        g.rows, nullptr, nullptr, stream);
        if (e == hipSuccess)
            e = launch_gemm(u, nullptr, w.mb, xs, g.cols, xk, perm, top_k, tiles, n_tiles, w.cap,
                            h, g.rows, gbuf, g.row_map, stream);
    }
    if (ev.stop)
        (void)hipEventRecord(ev.stop, stream);
    if (e != hipSuccess)
        return e;
    if ((e = launch_rowscale(h, 1, P, g.rows, hs, hk, stream)) != hipSuccess)
        return e;
    // the down projection's outputs in fp16 with exponents per (tile, 64
    // columns): half the bytes of fp32 written here and read by the combine
    e = launch_gemm(dn, nullptr, w.mb, hs, g.rows, hk, nullptr, 1, tiles, n_tiles, w.cap, nullptr,
                    dn.rows, nullptr, nullptr, stream, zh, ze);
    if (e != hipSuccess)
        return e;
    const int64_t n8 = (int64_t)n_tok * dn.rows / 8;
    hipLaunchKernelGGL(k_combine_perm_h, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                       zh, ze, hk, pos, wts, n_tok, top_k, dn.rows, y);
    return hipGetLastError();
}

}  // namespace vq
