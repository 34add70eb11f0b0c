// vq_gather.hip -- row gather from a stacked VQ tensor.
//
// Model card "Qwen3.8-Flash-Next-VQ-4.4bpw" (opening summary; changelog
// 2026-10-04): the per-layer n-gram embedding tables are VQ tensors in the
// experts' format (d=2/K=256) and are read one hashed row per lookup.  The
// tables of a stacked tensor are its experts; id = e*rows + r names logical
// row r of table e, and the output row is that row decoded exactly in fp32
// (fp16 scale x fp16 entry fits fp32).  The hash producing the ids belongs
// to the model and is not done here.
//
// The output dominates the traffic (4 bytes per weight written against about
// half a byte read at d=2/K=256), so the kernel is shaped around the stores:
// the output is a flat sequence of 16-byte chunks (4 columns), consecutive
// lanes own consecutive chunks, and every store of a wavefront covers 1 KiB of
// contiguous memory.  A chunk needs the row's id, one or two code words and
// one scale; each thread takes kUnroll chunks at a time so their dependent
// loads (id -> row map -> codes and scale) overlap.  The codebook is staged in
// LDS once per workgroup.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "vq_common.hpp"
#include "vq_internal.hpp"

namespace vq {
namespace {

constexpr int kThreadsG = 256;


struct GatherArgs {
    const uint32_t *codes;
    const uint16_t *scales;
    const uint32_t *codebook;  // fp16 [K][d] read as dwords (pairs of entries' halves)
    const int32_t *row_map;    // NULL = dense
    const int64_t *ids;
    float *y;
    uint64_t n_chunks;         // n * cols / 4
    int64_t n_rows;            // n_experts * rows: valid ids are below
    int wpr;                   // words per stored row
    int groups;                // cols / 64
    int cq;                    // chunks per output row (cols / 4)
    int cb_dwords;             // K * d / 2
    uint32_t kmax;             // K - 1
};

// One output chunk: columns [4*c4, 4*c4 + 4) of the row named by ids[j].
// D=2 takes two codes, D=4 one, D=8 one half of a code's 8-vector.
template <int D, int BITS, int kUnroll>
__global__ __launch_bounds__(kThreadsG) void k_gather(GatherArgs a)
{
    constexpr int NC = D == 2 ? 2 : 1;      // codes per chunk
    constexpr int NB = NC * BITS;           // their bits, contiguous in the stream
    // chunk c4 starts at stream bit (4*c4/D)*BITS, a multiple of NB for
    // D <= 4 and of BITS for D = 8, so the bits never cross a word when NB
    // divides 32
    constexpr bool ONE_WORD = (32 % NB) == 0;
    constexpr uint32_t MASK = (1u << BITS) - 1u;

    // codebook -> LDS, eight loads in flight per thread (a 64 KiB codebook
    // takes eight rounds); the index is clamped so every load is in bounds
    extern __shared__ uint32_t cb[];
    for (int i0 = threadIdx.x; i0 < a.cb_dwords; i0 += 8 * kThreadsG) {
        uint32_t v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            v[k] = load_global(a.codebook + min(i0 + k * kThreadsG, a.cb_dwords - 1));
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (i0 + k * kThreadsG < a.cb_dwords)
                cb[i0 + k * kThreadsG] = v[k];
    }
    __syncthreads();

    // Loads are issued for every chunk of a batch before any is used; lanes
    // with nothing to read (past the end, a bad id, a dead row) read element
    // 0 of the same array instead of branching, so the batch's loads stay in
    // flight together.  The host guarantees n_chunks < 2^31.
    const uint32_t n_chunks = (uint32_t)a.n_chunks;
    const uint32_t stride = gridDim.x * kThreadsG;
    for (uint32_t q0 = blockIdx.x * kThreadsG + threadIdx.x; q0 < n_chunks;
         q0 += stride * kUnroll) {
        bool live[kUnroll];
        uint32_t c4[kUnroll];
        int64_t s[kUnroll];  // stored row; -1 dead row, -2 id out of range

#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t q = q0 + u * stride;
            live[u] = q < n_chunks;
            const uint32_t j = q / (uint32_t)a.cq;
            c4[u] = q - j * (uint32_t)a.cq;
            s[u] = load_global(a.ids + (live[u] ? j : 0u));
        }
        bool ok[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            ok[u] = s[u] >= 0 && s[u] < a.n_rows;
            s[u] = ok[u] ? s[u] : 0;
        }
        if (a.row_map) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                s[u] = load_global(a.row_map + s[u]);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            s[u] = ok[u] ? s[u] : -2;

        uint32_t w0[kUnroll], w1[kUnroll], off[kUnroll];
        uint16_t sc[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t j0 = (4u * c4[u]) / D;          // first code of the chunk
            const uint32_t p = j0 * BITS;                  // its stream bit
            off[u] = p & 31u;
            const bool have = s[u] >= 0;
            int64_t w = have ? s[u] * a.wpr + (p >> 5) : 0;
            int64_t g = have ? s[u] * a.groups + (c4[u] >> 4) : 0;
            // opaque to the optimizer, which would otherwise split each
            // selected address into a branch around two loads
            asm volatile("" : "+v"(w), "+v"(g));
            w0[u] = __builtin_nontemporal_load(a.codes + w);
            // when the chunk's bits cross into the next word, that word holds
            // bits of this chunk and so lies inside the row (rows are padded
            // to whole 32-code blocks)
            if constexpr (!ONE_WORD)
                w1[u] = __builtin_nontemporal_load(a.codes + w + (have && off[u] + NB > 32u));
            else
                w1[u] = 0u;
            sc[u] = load_global(a.scales + g);
        }

#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t bits =
                ONE_WORD ? (w0[u] >> off[u]) : __builtin_amdgcn_alignbit(w1[u], w0[u], off[u]);
            const float scale = half_bits_to_float(sc[u]);
            uint32_t e0, e1;
            if constexpr (D == 2) {
                // codes above K-1 are clamped so the lookup stays in the table
                e0 = cb[min(bits & MASK, a.kmax)];
                e1 = cb[min((bits >> BITS) & MASK, a.kmax)];
            } else {
                const uint32_t k = min(bits & MASK, a.kmax);
                // D=4: the entry's two dwords; D=8: the chunk's half of four
                const uint32_t base = D == 4 ? 2u * k : 4u * k + 2u * (c4[u] & 1u);
                const uint2 e = *reinterpret_cast<const uint2 *>(cb + base);
                e0 = e.x;
                e1 = e.y;
            }
            f32x4 v;
            v[0] = scale * half_bits_to_float(e0 & 0xffffu);
            v[1] = scale * half_bits_to_float(e0 >> 16);
            v[2] = scale * half_bits_to_float(e1 & 0xffffu);
            v[3] = scale * half_bits_to_float(e1 >> 16);
            if (s[u] < 0) {
                const float f = s[u] == -1 ? 0.f : __builtin_nanf("");
                v = f32x4{f, f, f, f};
            }
            // chunk q covers output floats [4q, 4q + 4)
            if (live[u])
                __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(a.y) + q0 + u * stride);
        }
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

template <int D, int BITS, int U>
hipError_t gather_launch(const GatherArgs &a, hipStream_t stream)
{
    const size_t lds = (size_t)a.cb_dwords * 4;
    // Small codebooks: one batch of U chunks per thread, workgroups queued
    // in output order (a measured few per cent ahead of a resident grid).
    // Codebooks over 4 KiB: as many resident workgroups as the LDS allows,
    // up to 8 per CU, and a grid-stride loop, so that each stages its
    // codebook once for many chunks.
    const int per_cu = lds == 0 ? 8 : (int)std::max<size_t>(1, std::min<size_t>(8, 163840 / lds));
    const uint64_t want = (a.n_chunks + (uint64_t)kThreadsG * U - 1) / ((uint64_t)kThreadsG * U);
    const uint64_t cap = lds <= 4096 ? want : (uint64_t)per_cu * device_cus();
    const unsigned blocks = (unsigned)std::max<uint64_t>(1, std::min(want, cap));
    hipLaunchKernelGGL((k_gather<D, BITS, U>), dim3(blocks), dim3(kThreadsG), lds, stream, a);
    return hipGetLastError();
}

// Eight chunks per thread keep enough loads in flight on large gathers; a
// gather too small to fill the chip with such batches (a token's lookups)
// takes one chunk per thread, which shortens each thread's chain.
template <int D, int BITS>
hipError_t gather_db(const GatherArgs &a, hipStream_t stream)
{
    if (a.n_chunks < (uint64_t)kThreadsG * 8 * device_cus())
        return gather_launch<D, BITS, 1>(a, stream);
    return gather_launch<D, BITS, 8>(a, stream);
}

template <int D>
hipError_t gather_d(int bits, const GatherArgs &a, hipStream_t stream)
{
    switch (bits) {
    case 8: return gather_db<D, 8>(a, stream);
    case 9: return gather_db<D, 9>(a, stream);
    case 10: return gather_db<D, 10>(a, stream);
    case 11: return gather_db<D, 11>(a, stream);
    case 12: return gather_db<D, 12>(a, stream);
    case 13: return gather_db<D, 13>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gather(const TensorDev &t, int64_t n, const int64_t *ids, float *y,
                         hipStream_t stream)
{
    GatherArgs a;
    // A tensor with no stored rows may have empty code and scale arrays;
    // every row is then dead and the kernel's placeholder reads (element 0)
    // go to the codebook, which always holds at least one entry.
    const bool empty = t.n_stored == 0;
    a.codes = empty ? reinterpret_cast<const uint32_t *>(t.codebook) : t.codes;
    a.scales = empty ? t.codebook : t.scales;
    a.codebook = reinterpret_cast<const uint32_t *>(t.codebook);
    a.row_map = t.row_map;
    a.cq = t.cols / 4;
    a.n_rows = (int64_t)t.n_experts * t.rows;
    a.wpr = t.wpr;
    a.groups = t.groups;
    a.cb_dwords = t.cb_dwords;
    a.kmax = (uint32_t)(t.K - 1);
    // chunk indices are 32-bit in the kernel: launch slices of output rows
    const int64_t rows_per_launch = ((int64_t)1 << 31) / a.cq - 1;
    for (int64_t i0 = 0; i0 < n; i0 += rows_per_launch) {
        const int64_t m = std::min(rows_per_launch, n - i0);
        a.ids = ids + i0;
        a.y = y + i0 * t.cols;
        a.n_chunks = (uint64_t)m * (uint64_t)a.cq;
        hipError_t e = hipErrorInvalidValue;
        switch (t.d) {
        case 2: e = gather_d<2>(t.bits, a, stream); break;
        case 4: e = gather_d<4>(t.bits, a, stream); break;
        case 8: e = gather_d<8>(t.bits, a, stream); break;
        }
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace vq
