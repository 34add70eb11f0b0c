// vq_fit.hip -- fitting the format: scales, k-means / Lloyd over the weight
// subvectors, fp16 codebook, encode and pack.
//
// The cards fit their codebooks data-free by k-means / Lloyd over the weight
// subvectors from a seeded or unseeded subsample, with an fp16 scale per
// (row, 64 weights) and the codes packed sub-byte ("Methodology" sections of
// the Qwen3.5-397B-A17B 2.6bpw and 2.4bpw, Qwen3.8-Flash-Next and
// GLM-5.3-Flash cards).  Where they are silent this follows one reading,
// chosen so that every integer decision (a nearest centroid, a code) is a
// function of the inputs alone, whatever the thread order:
//   - scale = fp16 (nearest even) of the group's max |w|; v = w / s in fp32
//     with IEEE division; a group with s == 0 normalises to zeros;
//   - the fit set (subsample) and the K initial subvectors are inputs;
//   - distance = sum over t in order of (v_t - c_t)^2, every fp32 operation
//     rounded on its own (no fused multiply-add); ties go to the lower index;
//   - a centroid is the mean of its members: coordinates rounded to nearest
//     even on a 2^-30 grid and summed as 64-bit integers (integer atomics
//     are order-independent), the sum divided by the count in fp64; a
//     centroid without members keeps its value;
//   - the codebook is the centroids in fp16, and every subvector of the
//     tensor is coded to its nearest fp16 entry and packed LSB-first into
//     row-local 32-code blocks.
// All of it is ALU work on small data: nearest-centroid searches against a
// codebook held in LDS (K*d fp32 values), K*d subtract-multiply-add triples
// per subvector; the weights are read once, coalesced.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "vq_common.hpp"
#include "vq_internal.hpp"

// Every fp32 and fp64 operation in this file rounds on its own (no fused
// multiply-add forms), as the decisions above require.
#pragma clang fp contract(off)

namespace vq {
namespace {

constexpr int kFitThreads = 256;

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint16_t float_to_half_bits(float f)
{
    const f16 h = (f16)f;   // v_cvt_f16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

// Distance of x to entry c, every operation rounded: no contraction.
template <int D>
__device__ __forceinline__ float dist2(const float (&x)[D], const float *c)
{
    float acc = 0.0f;
#pragma unroll
    for (int t = 0; t < D; ++t) {
        const float diff = x[t] - c[t];
        const float sq = diff * diff;
        acc = acc + sq;
    }
    return acc;
}

// Index of the nearest of the K entries in LDS (first minimum).
template <int D>
__device__ __forceinline__ uint32_t nearest(const float (&x)[D], const float *C, int K)
{
    float best = dist2<D>(x, C);
    uint32_t bk = 0;
    for (int k = 1; k < K; ++k) {
        const float dk = dist2<D>(x, C + k * D);
        if (dk < best) {
            best = dk;
            bk = (uint32_t)k;
        }
    }
    return bk;
}

// Normalised subvector i = r * n_sub + j.
template <int D>
__device__ __forceinline__ void subvector(const uint16_t *__restrict__ w,
                                          const uint16_t *__restrict__ scales, int cols,
                                          int64_t n_sub, int64_t i, float (&v)[D])
{
    const int64_t r = i / n_sub, j = i - r * n_sub;
    const float s = half_bits_to_float(scales[r * (cols / 64) + (j * D) / 64]);
    const uint16_t *src = w + r * cols + j * D;
#pragma unroll
    for (int t = 0; t < D; ++t)
        v[t] = s == 0.0f ? 0.0f : bf16_bits_to_float(src[t]) / s;
}

// scales[r][g] = fp16(max |w| over the group): one thread per (row, group).
__global__ __launch_bounds__(kFitThreads) void k_fit_scales(const uint16_t *__restrict__ w,
                                                            int64_t n_groups, int groups,
                                                            uint16_t *__restrict__ scales)
{
    const int64_t i = (int64_t)blockIdx.x * kFitThreads + threadIdx.x;
    if (i >= n_groups)
        return;
    const uint4 *src = reinterpret_cast<const uint4 *>(w + (i / groups) * groups * 64 +
                                                       (i % groups) * 64);
    uint32_t m = 0;   // largest |w| as bf16 magnitude bits (order-preserving)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const uint4 u = src[q];
        const uint32_t p[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            m = max(m, p[k] & 0x7fffu);
            m = max(m, (p[k] >> 16) & 0x7fffu);
        }
    }
    scales[i] = float_to_half_bits(bf16_bits_to_float(m));
}

// The fit set's vectors (xs) and the initial centroids (C).  Indices are
// clamped into the tensor (a precondition; the clamp keeps reads in bounds).
template <int D>
__global__ __launch_bounds__(kFitThreads) void k_fit_vectors(
    const uint16_t *__restrict__ w, const uint16_t *__restrict__ scales, int cols, int64_t N,
    const int64_t *__restrict__ sample, int64_t n_sample, const int64_t *__restrict__ init, int K,
    float *__restrict__ xs, float *__restrict__ C)
{
    const int64_t i = (int64_t)blockIdx.x * kFitThreads + threadIdx.x;
    if (i >= n_sample + K)
        return;
    const bool is_init = i >= n_sample;
    int64_t idx = is_init ? init[i - n_sample] : sample[i];
    idx = idx < 0 ? 0 : (idx >= N ? N - 1 : idx);
    float v[D];
    subvector<D>(w, scales, cols, cols / D, idx, v);
    float *dst = is_init ? C + (i - n_sample) * D : xs + i * D;
#pragma unroll
    for (int t = 0; t < D; ++t)
        dst[t] = v[t];
}

__device__ __forceinline__ void stage_centroids(const float *__restrict__ C, int n, float *lds)
{
    for (int i = threadIdx.x; i < n; i += kFitThreads)
        lds[i] = C[i];
    __syncthreads();
}

// One assignment pass: every fit-set vector to its nearest centroid, its
// coordinates added (as integers on the 2^-30 grid) to that centroid's sums.
// LOCAL: the workgroup first adds into its own sums in LDS (after the
// centroids) and then adds those to the global ones, one atomic per
// non-zero sum, so a hot centroid costs each workgroup one global atomic
// instead of one per member.  Either way the sums are exact integers, so the
// result is the same.
template <int D, bool LOCAL>
__global__ __launch_bounds__(kFitThreads) void k_lloyd_assign(const float *__restrict__ xs,
                                                              int64_t n_sample,
                                                              const float *__restrict__ C, int K,
                                                              unsigned long long *__restrict__ sums,
                                                              unsigned long long *__restrict__ cnt)
{
    extern __shared__ float cl[];
    unsigned long long *ls = reinterpret_cast<unsigned long long *>(cl + ((K * D + 1) & ~1));
    unsigned long long *lc = ls + K * D;
    if constexpr (LOCAL)
        for (int i = threadIdx.x; i < K * D + K; i += kFitThreads)
            ls[i] = 0ull;
    stage_centroids(C, K * D, cl);   // ends with a barrier
    unsigned long long *ts = LOCAL ? ls : sums;
    unsigned long long *tc = LOCAL ? lc : cnt;
    for (int64_t i = (int64_t)blockIdx.x * kFitThreads + threadIdx.x; i < n_sample;
         i += (int64_t)gridDim.x * kFitThreads) {
        float x[D];
#pragma unroll
        for (int t = 0; t < D; ++t)
            x[t] = xs[i * D + t];
        const uint32_t k = nearest<D>(x, cl, K);
        atomicAdd(tc + k, 1ull);
#pragma unroll
        for (int t = 0; t < D; ++t) {
            const long long q = (long long)rint((double)x[t] * 0x1p30);
            atomicAdd(ts + (int64_t)k * D + t, (unsigned long long)q);
        }
    }
    if constexpr (LOCAL) {
        __syncthreads();
        for (int i = threadIdx.x; i < K * D + K; i += kFitThreads) {
            const unsigned long long v = ls[i];
            if (v != 0ull)
                atomicAdd(i < K * D ? sums + i : cnt + (i - K * D), v);
        }
    }
}

// Centroid update from the sums (members' mean; none: unchanged), then the
// sums are cleared for the next pass.
__global__ __launch_bounds__(kFitThreads) void k_lloyd_update(float *__restrict__ C, int K, int d,
                                                              unsigned long long *__restrict__ sums,
                                                              unsigned long long *__restrict__ cnt)
{
    const int k = blockIdx.x * kFitThreads + threadIdx.x;
    if (k >= K)
        return;
    const unsigned long long n = cnt[k];
    for (int t = 0; t < d; ++t) {
        if (n != 0) {
            const long long s = (long long)sums[(int64_t)k * d + t];
            C[(int64_t)k * d + t] = (float)(((double)s / (double)n) * 0x1p-30);
        }
        sums[(int64_t)k * d + t] = 0ull;
    }
    cnt[k] = 0ull;
}

__global__ __launch_bounds__(kFitThreads) void k_fit_clear(unsigned long long *__restrict__ p,
                                                           int n)
{
    const int i = blockIdx.x * kFitThreads + threadIdx.x;
    if (i < n)
        p[i] = 0ull;
}

// codebook = fp16(C); C is then replaced by the fp16 values, which the
// encode pass searches.
__global__ __launch_bounds__(kFitThreads) void k_fit_codebook(float *__restrict__ C, int n,
                                                              uint16_t *__restrict__ codebook)
{
    const int i = blockIdx.x * kFitThreads + threadIdx.x;
    if (i >= n)
        return;
    const uint16_t h = float_to_half_bits(C[i]);
    codebook[i] = h;
    C[i] = half_bits_to_float(h);
}

// Encode and pack.  A workgroup takes kEncBlocks consecutive 32-code blocks
// (in row-major block order, which is also the order of their words in
// memory); thread t codes subvector t % 32 of block t / 32, so a wavefront
// reads its blocks' weights contiguously.  The codes meet in LDS, and one
// thread per output word then gathers the codes overlapping its 32 bits,
// so the blocks' words are written contiguously too.
constexpr int kEncBlocks = kFitThreads / 32;

template <int D>
__global__ __launch_bounds__(kFitThreads) void k_fit_encode(
    const uint16_t *__restrict__ w, const uint16_t *__restrict__ scales, int64_t n_rows,
    int cols, int bits, const float *__restrict__ C, int K, uint32_t *__restrict__ codes)
{
    extern __shared__ float cl[];
    __shared__ uint32_t cs[kFitThreads];
    stage_centroids(C, K * D, cl);
    const int64_t n_sub = cols / D;
    const int n_blk = (int)((n_sub + 31) / 32);
    const int64_t n_blocks = n_rows * n_blk;
    const int64_t b0 = (int64_t)blockIdx.x * kEncBlocks;
    const int t = threadIdx.x;
    const int64_t bi = b0 + t / 32;          // this thread's block (row-major)
    uint32_t code = 0;                       // padding codes past the row's end are zero
    if (bi < n_blocks) {
        const int64_t r = bi / n_blk;
        const int64_t j = (bi - r * n_blk) * 32 + (t & 31);
        if (j < n_sub) {
            float v[D];
            subvector<D>(w, scales, cols, n_sub, r * n_sub + j, v);
            code = nearest<D>(v, cl, K);
        }
    }
    cs[t] = code;
    __syncthreads();
    // word q of local block lb holds stream bits [32q, 32q + 32) of that
    // block: codes floor(32q/bits) .. floor((32q+31)/bits)
    const int64_t nb = min((int64_t)kEncBlocks, n_blocks - b0);
    for (int o = t; o < nb * bits; o += kFitThreads) {
        const int lb = o / bits, q = o - lb * bits;
        const uint32_t *bc = cs + lb * 32;
        uint32_t word = 0;
        for (int c = (32 * q) / bits; c < 32 && c * bits < 32 * q + 32; ++c) {
            const int sh = c * bits - 32 * q;   // code c's offset from this word's bit 0
            word |= sh >= 0 ? bc[c] << sh : bc[c] >> -sh;
        }
        codes[b0 * bits + o] = word;
    }
}

int device_cus()
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

unsigned grid_for(int64_t n) { return (unsigned)std::max<int64_t>(1, (n + kFitThreads - 1) / kFitThreads); }

template <int D>
hipError_t fit_d(const FitArgs &f, hipStream_t s)
{
    const int64_t N = f.n_rows * (f.cols / D);
    const int groups = f.cols / 64;
    const int kd = f.K * D;
    const size_t lds = (size_t)kd * 4;
    hipLaunchKernelGGL(k_fit_scales, dim3(grid_for(f.n_rows * groups)), dim3(kFitThreads), 0, s,
                       f.w, f.n_rows * groups, groups, f.scales);
    hipLaunchKernelGGL(k_fit_vectors<D>, dim3(grid_for(f.n_sample + f.K)), dim3(kFitThreads), 0,
                       s, f.w, f.scales, f.cols, N, f.sample, f.n_sample, f.init, f.K, f.xs, f.C);
    hipLaunchKernelGGL(k_fit_clear, dim3(grid_for(kd + f.K)), dim3(kFitThreads), 0, s, f.sums,
                       kd + f.K);
    // per-workgroup sums in LDS when they fit beside the centroids (then a
    // few workgroups per CU, each with many members); else global atomics
    const size_t lds_local = (size_t)((kd + 1) & ~1) * 4 + (size_t)(kd + f.K) * 8;
    const bool local = lds_local <= 65536;
    const unsigned assign_grid = (unsigned)std::min<int64_t>(
        grid_for(f.n_sample), local ? 2 * (int64_t)device_cus() : 8 * 256);
    for (int it = 0; it < f.iters; ++it) {
        if (f.n_sample > 0) {
            if (local)
                hipLaunchKernelGGL((k_lloyd_assign<D, true>), dim3(assign_grid), dim3(kFitThreads),
                                   lds_local, s, f.xs, f.n_sample, f.C, f.K, f.sums, f.sums + kd);
            else
                hipLaunchKernelGGL((k_lloyd_assign<D, false>), dim3(assign_grid), dim3(kFitThreads),
                                   lds, s, f.xs, f.n_sample, f.C, f.K, f.sums, f.sums + kd);
        }
        hipLaunchKernelGGL(k_lloyd_update, dim3(grid_for(f.K)), dim3(kFitThreads), 0, s, f.C,
                           f.K, D, f.sums, f.sums + kd);
    }
    hipLaunchKernelGGL(k_fit_codebook, dim3(grid_for(kd)), dim3(kFitThreads), 0, s, f.C, kd,
                       f.codebook);
    const int n_blk = (int)((f.cols / D + 31) / 32);
    const int64_t enc_grid = (f.n_rows * n_blk + kEncBlocks - 1) / kEncBlocks;
    if (enc_grid > 0x7fffffff)
        return hipErrorInvalidValue;
    const KernelEvents &ev = kernel_events();
    if (ev.start)
        (void)hipEventRecord(ev.start, s);
    hipLaunchKernelGGL(k_fit_encode<D>, dim3((unsigned)enc_grid), dim3(kFitThreads), lds, s, f.w,
                       f.scales, f.n_rows, f.cols, f.bits, f.C, f.K, f.codes);
    const hipError_t e = hipGetLastError();
    if (ev.stop)
        (void)hipEventRecord(ev.stop, s);
    return e;
}

}  // namespace

size_t fit_workspace_bytes(int d, int K, int64_t n_sample, FitArgs *f, void *ws)
{
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    const size_t xs = up((size_t)n_sample * d * 4);
    const size_t c = up((size_t)K * d * 4);
    const size_t sums = up(((size_t)K * d + K) * 8);
    if (f) {
        char *p = static_cast<char *>(ws);
        f->xs = reinterpret_cast<float *>(p);
        f->C = reinterpret_cast<float *>(p + xs);
        f->sums = reinterpret_cast<unsigned long long *>(p + xs + c);
    }
    return xs + c + sums;
}

hipError_t launch_fit(const FitArgs &f, hipStream_t stream)
{
    switch (f.d) {
    case 2: return fit_d<2>(f, stream);
    case 4: return fit_d<4>(f, stream);
    case 8: return fit_d<8>(f, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace vq
