// vq_probe.hip -- ceiling probes for the rooflines (gfx950).
//
// Two kernels that bound what the hot path can reach on the device it runs
// on, independent of the VQ format:
//
//   * k_probe_read: a streaming read of a large buffer, every lane loading
//     16 bytes per load with four loads in flight, workgroups striding over
//     the buffer so the chip reads one contiguous window at a time (the best
//     case for HBM);
//   * k_probe_mfma: v_mfma_f32_32x32x16_f16 on register operands only, four
//     independent accumulator chains per wave, no memory traffic (the best
//     case for the matrix cores at the clock the chip holds under that load).
#include "vq_common.hpp"
#include "vq_internal.hpp"

namespace vq {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;

__global__ __launch_bounds__(kProbeThreads) void k_probe_read(const uint4 *__restrict__ p,
                                                              size_t n16, uint32_t *__restrict__ out)
{
    const size_t tid = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
    const size_t nth = (size_t)gridDim.x * kProbeThreads;
    uint32_t acc = 0;
    size_t base = 0;
    for (; base + kProbeUnroll * nth <= n16; base += kProbeUnroll * nth) {
        uint4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u)
            v[u] = p[base + (size_t)u * nth + tid];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // the tail, one load at a time
    for (size_t i = base + tid; i < n16; i += nth) {
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    out[tid] = acc;
}

__global__ __launch_bounds__(kProbeThreads) void k_probe_mfma(int iters, float *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    f16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(0.001f * (float)((lane + i) & 15));
        b[i] = (_Float16)(0.002f * (float)((lane * 3 + i) & 7));
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r)
        s += c0[r] + c1[r] + c2[r] + c3[r];
    out[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

hipError_t launch_probe_read(const void *p, size_t bytes, uint32_t *out, int n_wg,
                             hipStream_t stream)
{
    k_probe_read<<<n_wg, kProbeThreads, 0, stream>>>(static_cast<const uint4 *>(p), bytes / 16,
                                                     out);
    return hipGetLastError();
}

hipError_t launch_probe_mfma(int n_wg, int iters, float *out, hipStream_t stream)
{
    k_probe_mfma<<<n_wg, kProbeThreads, 0, stream>>>(iters, out);
    return hipGetLastError();
}

}  // namespace vq
