// vq_api.cpp -- the C ABI: argument validation, workspace sizing, dispatch.
//
// Errors follow the convention of the card "gemma-4-26b-a4b-it-VQ-6.2bpw"
// (section "Multi-machine (exo) note"): a misuse fails loudly with an
// explanatory message instead of producing plausible garbage.  Every check
// here is on host-visible values; device-resident contents are documented
// preconditions in vq.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/vq.h"
#include "vq_internal.hpp"

#define VQ_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

vq_status fail(vq_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

vq_status fail(vq_status st, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

vq_status ok()
{
    g_last_error.clear();
    return VQ_OK;
}

vq_status hip_fail(hipError_t e, const char *what)
{
    return fail(VQ_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t words_per_row(const vq_tensor &t)
{
    const int64_t n_sub = t.cols / t.d;
    return ((n_sub + 31) / 32) * (int64_t)t.bits;
}

vq_status check_tensor(const vq_tensor *t, const char *name)
{
    if (!t)
        return fail(VQ_ERR_INVALID_ARGUMENT, "%s: descriptor is NULL", name);
    if (t->rows < 1)
        return fail(VQ_ERR_INVALID_ARGUMENT, "%s.rows = %d: must be >= 1", name, t->rows);
    if (t->cols < 64 || t->cols % 64 != 0)
        return fail(VQ_ERR_INVALID_ARGUMENT,
                    "%s.cols = %d: must be a positive multiple of 64 (one fp16 scale per 64 weights)",
                    name, t->cols);
    if (t->d != 2 && t->d != 4 && t->d != 8)
        return fail(VQ_ERR_UNSUPPORTED, "%s.d = %d: supported subvector lengths are 2, 4 and 8",
                    name, t->d);
    if (t->bits < 8 || t->bits > 13)
        return fail(VQ_ERR_UNSUPPORTED, "%s.bits = %d: supported code widths are 8..13", name,
                    t->bits);
    if (t->K < 1 || (int64_t)t->K > ((int64_t)1 << t->bits))
        return fail(VQ_ERR_INVALID_ARGUMENT, "%s.K = %d: need 1 <= K <= 2^bits = %lld", name,
                    t->K, (long long)(1LL << t->bits));
    if ((int64_t)t->K * t->d * 2 > vq::kMaxCodebookBytes)
        return fail(VQ_ERR_UNSUPPORTED,
                    "%s: codebook of %lld bytes exceeds the %d-byte LDS budget per tensor", name,
                    (long long)t->K * t->d * 2, vq::kMaxCodebookBytes);
    if (t->n_experts < 1)
        return fail(VQ_ERR_INVALID_ARGUMENT, "%s.n_experts = %d: must be >= 1", name,
                    t->n_experts);
    if (!t->codebook || !t->codes || !t->scales)
        return fail(VQ_ERR_INVALID_ARGUMENT, "%s: codebook, codes and scales must be non-NULL",
                    name);
    if (!aligned(t->codebook, 4) || !aligned(t->codes, 4) || !aligned(t->scales, 2) ||
        !aligned(t->row_map, 4))
        return fail(VQ_ERR_INVALID_ARGUMENT,
                    "%s: codebook/codes/row_map must be 4-byte and scales 2-byte aligned", name);
    const int64_t full = (int64_t)t->n_experts * t->rows;
    if (!t->row_map && t->n_stored != full)
        return fail(VQ_ERR_INVALID_ARGUMENT,
                    "%s.n_stored = %lld: a dense tensor (row_map NULL) stores n_experts*rows = %lld rows",
                    name, (long long)t->n_stored, (long long)full);
    if (t->row_map && (t->n_stored < 0 || t->n_stored > full))
        return fail(VQ_ERR_INVALID_ARGUMENT, "%s.n_stored = %lld: must be in [0, n_experts*rows]",
                    name, (long long)t->n_stored);
    if (words_per_row(*t) * t->n_stored > ((int64_t)1 << 40))
        return fail(VQ_ERR_UNSUPPORTED, "%s: tensor too large", name);
    return VQ_OK;
}

vq_status check_dtype(vq_dtype dt)
{
    if (dt != VQ_F32 && dt != VQ_BF16)
        return fail(VQ_ERR_INVALID_ARGUMENT, "x_dtype = %d: must be VQ_F32 or VQ_BF16", (int)dt);
    return VQ_OK;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct DecodeWs {
    size_t h_off, z_off, total;
};

DecodeWs decode_ws(const vq_tensor &g, const vq_tensor &dn, int n_tok, int top_k)
{
    DecodeWs w;
    const size_t pairs = (size_t)n_tok * top_k;
    w.h_off = 0;
    w.z_off = align_up(pairs * g.rows * sizeof(float), 256);
    w.total = w.z_off + align_up(pairs * dn.rows * sizeof(float), 256);
    return w;
}

constexpr int kDecodeMaxTokens = 16;
constexpr int kGemvMaxTokens = 64;

// Past kDecodeMaxTokens tokens the routed FFN stays on the decode kernels
// while the batch has at most max(kDecodeMaxPairs, 3/4 of the experts)
// routed pairs.  The decode kernels cost about the same per pair at any
// batch size (every pair streams its expert's rows), while the grouped GEMM
// reads an expert once per tile of its pairs but pays a fixed cost per call
// (routing, row scaling, the combine, tiles that small batches leave mostly
// empty); its cost grows with the distinct experts a batch touches, so the
// crossover moves out with the expert count.  Measured: on the 512-expert
// top-10 layer (6.3 MB per routed expert) decode 0.56 ms against 0.60 at
// 320 pairs, 1.10 against 0.86 at 640 (the two meet near 380); on the
// 128-expert top-8 one (1.3 MB) near 240, decode 0.187 ms against 0.179 at
// 256 pairs.
#ifndef VQ_DECODE_MAX_PAIRS
#define VQ_DECODE_MAX_PAIRS 176
#endif
constexpr int kDecodeMaxPairs = VQ_DECODE_MAX_PAIRS;

static int64_t decode_pair_limit(const vq_tensor &gate)
{
    return std::max<int64_t>(kDecodeMaxPairs, (int64_t)gate.n_experts * 3 / 4);
}

}  // namespace

namespace vq {

KernelEvents &kernel_events()
{
    thread_local KernelEvents ev = {nullptr, nullptr};
    return ev;
}

TensorDev to_dev(const vq_tensor &t)
{
    TensorDev d;
    d.codes = t.codes;
    d.scales = t.scales;
    d.codebook = t.codebook;
    d.row_map = t.row_map;
    d.rows = t.rows;
    d.cols = t.cols;
    d.d = t.d;
    d.bits = t.bits;
    d.K = t.K;
    d.n_experts = t.n_experts;
    d.n_stored = t.n_stored;
    d.groups = t.cols / 64;
    d.wpr = (int)words_per_row(t);
    d.cb_dwords = t.K * t.d / 2;
    return d;
}

}  // namespace vq

// ------------------------------------------------------------------------------------
// housekeeping
// ------------------------------------------------------------------------------------

VQ_EXPORT int32_t vq_abi_version(void) { return VQ_ABI_VERSION; }

VQ_EXPORT const char *vq_status_string(vq_status s)
{
    switch (s) {
    case VQ_OK: return "VQ_OK";
    case VQ_ERR_INVALID_ARGUMENT: return "VQ_ERR_INVALID_ARGUMENT";
    case VQ_ERR_UNSUPPORTED: return "VQ_ERR_UNSUPPORTED";
    case VQ_ERR_WORKSPACE: return "VQ_ERR_WORKSPACE";
    case VQ_ERR_HIP: return "VQ_ERR_HIP";
    }
    return "VQ_ERR_UNKNOWN";
}

VQ_EXPORT const char *vq_last_error(void) { return g_last_error.c_str(); }

VQ_EXPORT vq_status vq_probe_read(const void *buf, size_t bytes, int32_t n_workgroups,
                                  uint32_t *out, void *stream)
{
    if (!buf || !aligned(buf, 16) || bytes % 16 != 0 || bytes == 0)
        return fail(VQ_ERR_INVALID_ARGUMENT,
                    "buf: must be a non-NULL, 16-byte aligned device buffer of a multiple of 16 "
                    "bytes (got %zu bytes at %p)", bytes, buf);
    if (n_workgroups < 1 || n_workgroups > 65536 || !out)
        return fail(VQ_ERR_INVALID_ARGUMENT,
                    "n_workgroups = %d: must be in [1, 65536], with out non-NULL", n_workgroups);
    const hipError_t e = vq::launch_probe_read(buf, bytes, out, n_workgroups,
                                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "vq_probe_read");
}

VQ_EXPORT vq_status vq_probe_mfma(int32_t n_workgroups, int32_t iters, float *out, void *stream)
{
    if (n_workgroups < 1 || n_workgroups > 65536 || iters < 1 || !out)
        return fail(VQ_ERR_INVALID_ARGUMENT,
                    "n_workgroups = %d, iters = %d: need n_workgroups in [1, 65536], iters >= 1 "
                    "and out non-NULL", n_workgroups, iters);
    const hipError_t e = vq::launch_probe_mfma(n_workgroups, iters, out,
                                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "vq_probe_mfma");
}

VQ_EXPORT vq_status vq_set_kernel_events(void *start, void *stop)
{
    if ((start == nullptr) != (stop == nullptr))
        return fail(VQ_ERR_INVALID_ARGUMENT, "start and stop must both be set or both be NULL");
    vq::kernel_events().start = static_cast<hipEvent_t>(start);
    vq::kernel_events().stop = static_cast<hipEvent_t>(stop);
    return ok();
}

VQ_EXPORT vq_status vq_validate(const vq_tensor *W)
{
    vq_status st = check_tensor(W, "W");
    return st != VQ_OK ? st : ok();
}

// ------------------------------------------------------------------------------------
// dequantize
// ------------------------------------------------------------------------------------

VQ_EXPORT vq_status vq_dequantize(const vq_tensor *W, int32_t expert, float *w, void *stream)
{
    vq_status st = check_tensor(W, "W");
    if (st != VQ_OK)
        return st;
    if (expert < 0 || expert >= W->n_experts)
        return fail(VQ_ERR_INVALID_ARGUMENT, "expert = %d: must be in [0, %d)", expert,
                    W->n_experts);
    if (!w || !aligned(w, 16))
        return fail(VQ_ERR_INVALID_ARGUMENT, "w: must be a non-NULL, 16-byte aligned device pointer");
    hipError_t e = vq::launch_dequantize(vq::to_dev(*W), expert, w, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "vq_dequantize");
}

// ------------------------------------------------------------------------------------
// fitting the format
// ------------------------------------------------------------------------------------

constexpr int64_t kFitMaxSample = (int64_t)1 << 22;   // keeps the integer sums below 2^53

static vq_status check_fit(int64_t n_rows, int32_t cols, int32_t d, int32_t bits, int32_t K,
                           int64_t n_sample, int32_t iters)
{
    if (n_rows < 1)
        return fail(VQ_ERR_INVALID_ARGUMENT, "n_rows = %lld: must be >= 1", (long long)n_rows);
    if (cols < 64 || cols % 64 != 0)
        return fail(VQ_ERR_INVALID_ARGUMENT, "cols = %d: must be a positive multiple of 64", cols);
    if (d != 2 && d != 4 && d != 8)
        return fail(VQ_ERR_UNSUPPORTED, "d = %d: supported subvector lengths are 2, 4 and 8", d);
    if (bits < 8 || bits > 13)
        return fail(VQ_ERR_UNSUPPORTED, "bits = %d: supported code widths are 8..13", bits);
    if (K < 1 || (int64_t)K > ((int64_t)1 << bits))
        return fail(VQ_ERR_INVALID_ARGUMENT, "K = %d: need 1 <= K <= 2^bits", K);
    if ((int64_t)K * d > 16384)
        return fail(VQ_ERR_UNSUPPORTED,
                    "K*d = %lld: the fit keeps K*d <= 16384 fp32 centroid values in LDS",
                    (long long)K * d);
    if (n_sample < 0 || n_sample > kFitMaxSample)
        return fail(VQ_ERR_INVALID_ARGUMENT, "n_sample = %lld: must be in [0, %lld]",
                    (long long)n_sample, (long long)kFitMaxSample);
    if (iters < 0)
        return fail(VQ_ERR_INVALID_ARGUMENT, "iters = %d: must be >= 0", iters);
    if (n_rows > ((int64_t)1 << 40) / cols)
        return fail(VQ_ERR_UNSUPPORTED, "n_rows = %lld: tensor too large", (long long)n_rows);
    return VQ_OK;
}

VQ_EXPORT size_t vq_fit_workspace_size(int32_t d, int32_t K, int64_t n_sample)
{
    if (d < 1 || K < 1 || n_sample < 0)
        return 0;
    return vq::fit_workspace_bytes(d, K, n_sample, nullptr, nullptr);
}

VQ_EXPORT vq_status vq_fit(int64_t n_rows, int32_t cols, int32_t d, int32_t bits, int32_t K,
                           const uint16_t *w, int64_t n_sample, const int64_t *sample,
                           const int64_t *init, int32_t iters, uint16_t *codebook,
                           uint16_t *scales, uint32_t *codes, void *workspace,
                           size_t workspace_bytes, void *stream)
{
    vq_status st = check_fit(n_rows, cols, d, bits, K, n_sample, iters);
    if (st != VQ_OK)
        return st;
    if (!w || !aligned(w, 16))
        return fail(VQ_ERR_INVALID_ARGUMENT, "w: must be a non-NULL, 16-byte aligned device pointer");
    if (!init || !aligned(init, 8) || (n_sample > 0 && (!sample || !aligned(sample, 8))))
        return fail(VQ_ERR_INVALID_ARGUMENT,
                    "init (and sample when n_sample > 0) must be non-NULL, 8-byte aligned");
    if (!codebook || !scales || !codes || !aligned(codebook, 2) || !aligned(scales, 2) ||
        !aligned(codes, 4))
        return fail(VQ_ERR_INVALID_ARGUMENT,
                    "codebook, scales (2-byte aligned) and codes (4-byte aligned) must be non-NULL");
    const size_t need = vq::fit_workspace_bytes(d, K, n_sample, nullptr, nullptr);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return fail(VQ_ERR_WORKSPACE,
                    "workspace: need %zu bytes, 256-byte aligned (got %zu bytes at %p)", need,
                    workspace_bytes, workspace);
    vq::FitArgs f;
    f.n_rows = n_rows;
    f.cols = cols;
    f.d = d;
    f.bits = bits;
    f.K = K;
    f.w = w;
    f.n_sample = n_sample;
    f.sample = sample;
    f.init = init;
    f.iters = iters;
    f.codebook = codebook;
    f.scales = scales;
    f.codes = codes;
    vq::fit_workspace_bytes(d, K, n_sample, &f, workspace);
    hipError_t e = vq::launch_fit(f, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "vq_fit");
}

// ------------------------------------------------------------------------------------
// row gather
// ------------------------------------------------------------------------------------

VQ_EXPORT vq_status vq_row_gather(const vq_tensor *W, int64_t n, const int64_t *ids, float *y,
                                  void *stream)
{
    vq_status st = check_tensor(W, "W");
    if (st != VQ_OK)
        return st;
    if (n < 0)
        return fail(VQ_ERR_INVALID_ARGUMENT, "n = %lld: must be >= 0", (long long)n);
    if (n == 0)
        return ok();
    if (n > ((int64_t)1 << 40) / W->cols)
        return fail(VQ_ERR_UNSUPPORTED, "n = %lld: output too large", (long long)n);
    if (!ids || !aligned(ids, 8))
        return fail(VQ_ERR_INVALID_ARGUMENT,
                    "ids: must be a non-NULL, 8-byte aligned device pointer");
    if (!y || !aligned(y, 16))
        return fail(VQ_ERR_INVALID_ARGUMENT, "y: must be a non-NULL, 16-byte aligned device pointer");
    hipError_t e = vq::launch_gather(vq::to_dev(*W), n, ids, y, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "vq_row_gather");
}

// ------------------------------------------------------------------------------------
// decode: one expert
// ------------------------------------------------------------------------------------

VQ_EXPORT vq_status vq_expert_gemv(const vq_tensor *W, int32_t expert, int32_t n_tokens,
                                   const void *x, vq_dtype x_dtype, float *y, void *stream)
{
    vq_status st = check_tensor(W, "W");
    if (st != VQ_OK)
        return st;
    if ((st = check_dtype(x_dtype)) != VQ_OK)
        return st;
    if (expert < 0 || expert >= W->n_experts)
        return fail(VQ_ERR_INVALID_ARGUMENT, "expert = %d: must be in [0, %d)", expert,
                    W->n_experts);
    if (n_tokens < 0 || n_tokens > kGemvMaxTokens)
        return fail(VQ_ERR_INVALID_ARGUMENT, "n_tokens = %d: must be in [0, %d]", n_tokens,
                    kGemvMaxTokens);
    if (W->cols / 64 > vq::kMaxGroupsDecode)
        return fail(VQ_ERR_UNSUPPORTED, "W.cols = %d: the decode kernels take at most %d columns",
                    W->cols, 64 * vq::kMaxGroupsDecode);
    if (n_tokens == 0)
        return ok();
    if (!x || !aligned(x, 16))
        return fail(VQ_ERR_INVALID_ARGUMENT, "x: must be a non-NULL, 16-byte aligned device pointer");
    if (!y || !aligned(y, 4))
        return fail(VQ_ERR_INVALID_ARGUMENT, "y: must be a non-NULL, 4-byte aligned device pointer");
    vq::RowsLaunch L = {};
    L.t[0] = vq::to_dev(*W);
    L.nproj = 1;
    L.act = x;
    L.act_f32 = x_dtype == VQ_F32;
    L.act_stride = W->cols;
    L.out = y;
    L.out_stride = W->rows;
    L.expert = expert;
    L.n_act = n_tokens;
    hipError_t e = vq::launch_rows(L, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "vq_expert_gemv");
}

// ------------------------------------------------------------------------------------
// prefill: grouped GEMM
// ------------------------------------------------------------------------------------

VQ_EXPORT size_t vq_expert_gemm_workspace_size(const vq_tensor *W, int32_t n_x_rows)
{
    if (check_tensor(W, "W") != VQ_OK || n_x_rows < 0)
        return 0;
    return vq::gemm_workspace_bytes(vq::to_dev(*W), n_x_rows);
}

VQ_EXPORT vq_status vq_expert_gemm(const vq_tensor *W, int32_t n_x_rows, const void *x,
                                   vq_dtype x_dtype, const int32_t *expert_offsets, float *y,
                                   void *workspace, size_t workspace_bytes, void *stream)
{
    vq_status st = check_tensor(W, "W");
    if (st != VQ_OK)
        return st;
    if ((st = check_dtype(x_dtype)) != VQ_OK)
        return st;
    if (n_x_rows < 0)
        return fail(VQ_ERR_INVALID_ARGUMENT, "n_x_rows = %d: must be >= 0", n_x_rows);
    if (n_x_rows == 0)
        return ok();
    if (!x || !aligned(x, 16))
        return fail(VQ_ERR_INVALID_ARGUMENT, "x: must be a non-NULL, 16-byte aligned device pointer");
    if (!y || !aligned(y, 16))
        return fail(VQ_ERR_INVALID_ARGUMENT, "y: must be a non-NULL, 16-byte aligned device pointer");
    if (!expert_offsets)
        return fail(VQ_ERR_INVALID_ARGUMENT, "expert_offsets: must be non-NULL");
    if ((int64_t)n_x_rows * W->cols * 2 >= vq::kMaxGemmActBytes)
        return fail(VQ_ERR_UNSUPPORTED,
                    "x of %d x %d fp16 values reaches %lld bytes, the grouped GEMM's limit",
                    n_x_rows, W->cols, (long long)vq::kMaxGemmActBytes);
    const vq::TensorDev td = vq::to_dev(*W);
    const size_t need = vq::gemm_workspace_bytes(td, n_x_rows);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
        return fail(VQ_ERR_WORKSPACE,
                    "workspace: need %zu bytes, 256-byte aligned (got %zu bytes at %p)", need,
                    workspace_bytes, workspace);
    hipError_t e = vq::launch_expert_gemm(td, n_x_rows, x, x_dtype == VQ_F32, expert_offsets, y,
                                          workspace, static_cast<hipStream_t>(stream));
    if (e == hipErrorNotSupported)
        return fail(VQ_ERR_UNSUPPORTED, "vq_expert_gemm: geometry not supported by the MFMA path");
    return e == hipSuccess ? ok() : hip_fail(e, "vq_expert_gemm");
}

// ------------------------------------------------------------------------------------
// routed SwiGLU FFN
// ------------------------------------------------------------------------------------

static vq_status check_decode_sizes(const vq_tensor &a, const vq_tensor &b, int32_t n_tokens,
                                    int32_t top_k)
{
    if (n_tokens < 0)
        return fail(VQ_ERR_INVALID_ARGUMENT, "n_tokens = %d: must be >= 0", n_tokens);
    if (a.cols / 64 > vq::kMaxGroupsDecode || b.cols / 64 > vq::kMaxGroupsDecode)
        return fail(VQ_ERR_UNSUPPORTED, "the decode kernels take at most %d columns",
                    64 * vq::kMaxGroupsDecode);
    if ((int64_t)n_tokens * top_k > vq::kMaxSlots)
        return fail(VQ_ERR_UNSUPPORTED, "n_tokens * top_k = %lld exceeds %d",
                    (long long)n_tokens * top_k, vq::kMaxSlots);
    return VQ_OK;
}

static hipError_t launch_gate_up(const vq::TensorDev &g, const vq::TensorDev &u, int n_tokens,
                                 int top_k, const void *x, bool x_f32, const int32_t *ids,
                                 float *h, hipStream_t s)
{
    vq::RowsLaunch L = {};
    L.t[0] = g;
    L.t[1] = u;
    L.nproj = 2;
    L.act = x;
    L.act_f32 = x_f32;
    L.act_stride = g.cols;
    L.out = h;
    L.out_stride = g.rows;
    L.ids = ids;
    L.n_slots = n_tokens * top_k;
    L.act_div = top_k;
    L.multi_per_expert = n_tokens > 1;
    const vq::KernelEvents &ev = vq::kernel_events();
    if (ev.start)
        (void)hipEventRecord(ev.start, s);
    const hipError_t e = vq::launch_rows(L, s);
    if (ev.stop)
        (void)hipEventRecord(ev.stop, s);
    return e;
}

static hipError_t launch_down(const vq::TensorDev &dn, int n_tokens, int top_k, const float *h,
                              const int32_t *ids, float *z, hipStream_t s)
{
    vq::RowsLaunch L = {};
    L.t[0] = dn;
    L.nproj = 1;
    L.act = h;
    L.act_f32 = 2;   // h rounded once to fp16, as in the fused down+combine kernel
    L.act_stride = dn.cols;
    L.out = z;
    L.out_stride = dn.rows;
    L.ids = ids;
    L.n_slots = n_tokens * top_k;
    L.act_div = 1;
    L.multi_per_expert = n_tokens > 1;
    return vq::launch_rows(L, s);
}

static vq_status check_ffn(const vq_tensor *gate, const vq_tensor *up, const vq_tensor *down,
                           int32_t n_tokens, int32_t top_k)
{
    vq_status st;
    if ((st = check_tensor(gate, "gate")) != VQ_OK || (st = check_tensor(up, "up")) != VQ_OK ||
        (st = check_tensor(down, "down")) != VQ_OK)
        return st;
    if (up->rows != gate->rows || up->cols != gate->cols)
        return fail(VQ_ERR_INVALID_ARGUMENT, "up is %dx%d but gate is %dx%d", up->rows, up->cols,
                    gate->rows, gate->cols);
    if (down->rows != gate->cols || down->cols != gate->rows)
        return fail(VQ_ERR_INVALID_ARGUMENT,
                    "down is %dx%d: must be hidden x inter = %dx%d", down->rows, down->cols,
                    gate->cols, gate->rows);
    if (up->n_experts != gate->n_experts || down->n_experts != gate->n_experts)
        return fail(VQ_ERR_INVALID_ARGUMENT, "gate/up/down must have the same n_experts");
    if (up->d != gate->d || up->bits != gate->bits)
        return fail(VQ_ERR_UNSUPPORTED,
                    "gate and up must share d and bits (they run in one fused kernel)");
    if (n_tokens < 0)
        return fail(VQ_ERR_INVALID_ARGUMENT, "n_tokens = %d: must be >= 0", n_tokens);
    if (top_k < 1 || top_k > gate->n_experts)
        return fail(VQ_ERR_INVALID_ARGUMENT, "top_k = %d: must be in [1, n_experts = %d]", top_k,
                    gate->n_experts);
    return VQ_OK;
}

// Which engine runs the routed FFN (arguments already checked): the decode
// kernels for up to kDecodeMaxTokens tokens (whose size limits then apply),
// and for larger batches of at most decode_pair_limit() routed pairs whose
// columns fit the decode kernels; otherwise the grouped MFMA GEMM.
static bool ffn_uses_decode(const vq_tensor &gate, const vq_tensor &down, int32_t n_tokens,
                            int32_t top_k)
{
    if (n_tokens <= kDecodeMaxTokens)
        return true;
    const int64_t pairs = (int64_t)n_tokens * top_k;
    return pairs <= decode_pair_limit(gate) && pairs <= vq::kMaxSlots &&
           gate.cols / 64 <= vq::kMaxGroupsDecode && down.cols / 64 <= vq::kMaxGroupsDecode;
}

// Size limits of the grouped-GEMM path: routed pairs are counted in int32,
// and every activation matrix the GEMM reads (x rows, then one h row per
// routed pair) is indexed in 32-bit bytes.
static vq_status check_prefill_sizes(const vq_tensor &gate, int32_t n_tokens, int32_t top_k)
{
    const int64_t pairs = (int64_t)n_tokens * top_k;
    if (pairs > vq::kMaxPrefillPairs)
        return fail(VQ_ERR_UNSUPPORTED, "n_tokens * top_k = %lld exceeds %lld routed pairs",
                    (long long)pairs, (long long)vq::kMaxPrefillPairs);
    if ((int64_t)n_tokens * gate.cols * 2 >= vq::kMaxGemmActBytes ||
        pairs * gate.rows * 2 >= vq::kMaxGemmActBytes)
        return fail(VQ_ERR_UNSUPPORTED,
                    "activations of %lld x %d or h of %lld x %d fp16 values reach %lld bytes, "
                    "the grouped GEMM's limit", (long long)n_tokens, gate.cols, (long long)pairs,
                    gate.rows, (long long)vq::kMaxGemmActBytes);
    return VQ_OK;
}

// The small-batch FFN: gate+up+SwiGLU -> down -> slot-ordered combine, into y
// (accumulate: added to y).  Sizes and the workspace are checked by the caller.
static vq_status run_decode_ffn(const vq::TensorDev &g, const vq::TensorDev &u,
                                const vq::TensorDev &dn, int n_tokens, int top_k, const void *x,
                                bool x_f32, const int32_t *ids, const float *w, float *y,
                                bool accumulate, const DecodeWs &ws, void *workspace,
                                hipStream_t s, const char *what)
{
    float *h = reinterpret_cast<float *>(static_cast<char *>(workspace) + ws.h_off);
    float *z = reinterpret_cast<float *>(static_cast<char *>(workspace) + ws.z_off);
    hipError_t e = launch_gate_up(g, u, n_tokens, top_k, x, x_f32, ids, h, s);
    if (e != hipSuccess)
        return hip_fail(e, what);
    if (vq::mix_supported(dn, n_tokens, top_k)) {
        // down projection and combine in one pass over the output rows
        e = vq::launch_mix(dn, n_tokens, top_k, h, ids, w, y, accumulate, s);
        return e == hipSuccess ? ok() : hip_fail(e, what);
    }
    e = launch_down(dn, n_tokens, top_k, h, ids, z, s);
    if (e != hipSuccess)
        return hip_fail(e, what);
    e = vq::launch_combine(z, w, n_tokens, top_k, dn.rows, y, accumulate, s);
    return e == hipSuccess ? ok() : hip_fail(e, what);
}

VQ_EXPORT size_t vq_moe_ffn_workspace_size(const vq_tensor *gate, const vq_tensor *up,
                                           const vq_tensor *down, int32_t n_tokens, int32_t top_k)
{
    if (check_ffn(gate, up, down, n_tokens, top_k) != VQ_OK)
        return 0;
    if (ffn_uses_decode(*gate, *down, n_tokens, top_k))
        return decode_ws(*gate, *down, n_tokens, top_k).total;
    if (check_prefill_sizes(*gate, n_tokens, top_k) != VQ_OK)
        return 0;
    return vq::moe_prefill_workspace_bytes(vq::to_dev(*gate), vq::to_dev(*up), vq::to_dev(*down),
                                           n_tokens, top_k);
}

VQ_EXPORT vq_status vq_moe_ffn_engine(const vq_tensor *gate, const vq_tensor *up,
                                      const vq_tensor *down, int32_t n_tokens, int32_t top_k,
                                      int32_t *engine)
{
    vq_status st = check_ffn(gate, up, down, n_tokens, top_k);
    if (st != VQ_OK)
        return st;
    if (!engine)
        return fail(VQ_ERR_INVALID_ARGUMENT, "engine must be non-NULL");
    *engine = ffn_uses_decode(*gate, *down, n_tokens, top_k) ? VQ_ENGINE_DECODE : VQ_ENGINE_MFMA;
    return ok();
}

VQ_EXPORT vq_status vq_moe_ffn(const vq_tensor *gate, const vq_tensor *up, const vq_tensor *down,
                               int32_t n_tokens, int32_t top_k, const void *x, vq_dtype x_dtype,
                               const int32_t *topk_ids, const float *topk_weights, float *y,
                               void *workspace, size_t workspace_bytes, void *stream)
{
    vq_status st = check_ffn(gate, up, down, n_tokens, top_k);
    if (st != VQ_OK)
        return st;
    if ((st = check_dtype(x_dtype)) != VQ_OK)
        return st;
    if (n_tokens == 0)
        return ok();
    if (!x || !aligned(x, 16))
        return fail(VQ_ERR_INVALID_ARGUMENT, "x: must be a non-NULL, 16-byte aligned device pointer");
    if (!topk_ids || !topk_weights)
        return fail(VQ_ERR_INVALID_ARGUMENT, "topk_ids and topk_weights must be non-NULL");
    if (!y || !aligned(y, 16))
        return fail(VQ_ERR_INVALID_ARGUMENT, "y: must be a non-NULL, 16-byte aligned device pointer");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const vq::TensorDev g = vq::to_dev(*gate), u = vq::to_dev(*up), dn = vq::to_dev(*down);

    if (!ffn_uses_decode(*gate, *down, n_tokens, top_k)) {
        if ((st = check_prefill_sizes(*gate, n_tokens, top_k)) != VQ_OK)
            return st;
        const size_t need = vq::moe_prefill_workspace_bytes(g, u, dn, n_tokens, top_k);
        if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
            return fail(VQ_ERR_WORKSPACE,
                        "workspace: need %zu bytes, 256-byte aligned (got %zu bytes at %p)", need,
                        workspace_bytes, workspace);
        hipError_t e = vq::launch_moe_prefill(g, u, dn, n_tokens, top_k, x, x_dtype == VQ_F32,
                                              topk_ids, topk_weights, y, workspace, s);
        if (e == hipErrorNotSupported)
            return fail(VQ_ERR_UNSUPPORTED, "vq_moe_ffn: geometry not supported by the MFMA path");
        return e == hipSuccess ? ok() : hip_fail(e, "vq_moe_ffn (prefill)");
    }

    // ---- decode: gate+up+SwiGLU -> down -> slot-ordered combine ------------------
    if ((st = check_decode_sizes(*gate, *down, n_tokens, top_k)) != VQ_OK)
        return st;
    const DecodeWs ws = decode_ws(*gate, *down, n_tokens, top_k);
    if (!workspace || workspace_bytes < ws.total || !aligned(workspace, 256))
        return fail(VQ_ERR_WORKSPACE,
                    "workspace: need %zu bytes, 256-byte aligned (got %zu bytes at %p)", ws.total,
                    workspace_bytes, workspace);
    return run_decode_ffn(g, u, dn, n_tokens, top_k, x, x_dtype == VQ_F32, topk_ids,
                          topk_weights, y, false, ws, workspace, s, "vq_moe_ffn (decode)");
}

// ------------------------------------------------------------------------------------
// the routed FFN without allocation: its workspace is a static device array
// ------------------------------------------------------------------------------------

// One copy per GPU, created with the code object and held until the process
// ends.  Host code never passes `scratch` itself to a kernel or a copy (on the
// host the name is only a stand-in): it uses the address looked up below.
static __device__ __align__(256) unsigned char scratch[VQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of each GPU's `scratch` (null: not yet)

// This GPU's address of `scratch`, looked up on the first call with the
// device current and kept per device.
hipError_t scratch_address(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

VQ_EXPORT vq_status vq_moe_ffn_noalloc(const vq_tensor *gate, const vq_tensor *up,
                                       const vq_tensor *down, int32_t n_tokens, int32_t top_k,
                                       const void *x, vq_dtype x_dtype, const int32_t *topk_ids,
                                       const float *topk_weights, float *y, void *stream)
{
    vq_status st = check_ffn(gate, up, down, n_tokens, top_k);
    if (st != VQ_OK)
        return st;
    if (n_tokens == 0)
        return ok();
    if (!ffn_uses_decode(*gate, *down, n_tokens, top_k) &&
        (st = check_prefill_sizes(*gate, n_tokens, top_k)) != VQ_OK)
        return st;
    const size_t need = vq_moe_ffn_workspace_size(gate, up, down, n_tokens, top_k);
    if (need > (size_t)VQ_NOALLOC_SCRATCH_BYTES)
        return fail(VQ_ERR_UNSUPPORTED,
                    "vq_moe_ffn_noalloc: %d tokens x top-%d need %zu bytes of workspace; the "
                    "static scratch array holds %zu (call vq_moe_ffn with a workspace instead)",
                    n_tokens, top_k, need, (size_t)VQ_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess)
        return hip_fail(e, "vq_moe_ffn_noalloc: address of the scratch array");
    return vq_moe_ffn(gate, up, down, n_tokens, top_k, x, x_dtype, topk_ids, topk_weights, y, ws,
                      (size_t)VQ_NOALLOC_SCRATCH_BYTES, stream);
}

// ------------------------------------------------------------------------------------
// a stack of MoE layers on a residual stream (small batches)
// ------------------------------------------------------------------------------------

static vq_status check_stack(const vq_moe_layer *layers, int32_t n_layers, int32_t n_tokens,
                             int32_t top_k)
{
    if (n_layers < 0 || (n_layers > 0 && !layers))
        return fail(VQ_ERR_INVALID_ARGUMENT, "n_layers = %d: must be >= 0 with a layer array",
                    n_layers);
    if (n_tokens < 0 || n_tokens > kDecodeMaxTokens)
        return fail(VQ_ERR_UNSUPPORTED, "n_tokens = %d: the layer stack takes 0..%d tokens",
                    n_tokens, kDecodeMaxTokens);
    for (int32_t l = 0; l < n_layers; ++l) {
        const vq_moe_layer &L = layers[l];
        vq_status st = check_ffn(L.gate, L.up, L.down, n_tokens, top_k);
        if (st != VQ_OK)
            return fail(st, "layer %d: %s", l, vq_last_error());
        if (L.gate->cols != layers[0].gate->cols)
            return fail(VQ_ERR_INVALID_ARGUMENT,
                        "layer %d: hidden size %d differs from layer 0's %d", l, L.gate->cols,
                        layers[0].gate->cols);
        if ((st = check_decode_sizes(*L.gate, *L.down, n_tokens, top_k)) != VQ_OK)
            return fail(st, "layer %d: %s", l, vq_last_error());
        if (n_tokens > 0 && (!L.topk_ids || !L.topk_weights))
            return fail(VQ_ERR_INVALID_ARGUMENT, "layer %d: topk_ids and topk_weights must be non-NULL",
                        l);
    }
    return VQ_OK;
}

VQ_EXPORT size_t vq_moe_stack_workspace_size(const vq_moe_layer *layers, int32_t n_layers,
                                             int32_t n_tokens, int32_t top_k)
{
    if (check_stack(layers, n_layers, n_tokens, top_k) != VQ_OK)
        return 0;
    size_t need = 256;
    for (int32_t l = 0; l < n_layers; ++l)
        need = std::max(need, decode_ws(*layers[l].gate, *layers[l].down, n_tokens, top_k).total);
    return need;
}

VQ_EXPORT vq_status vq_moe_stack(const vq_moe_layer *layers, int32_t n_layers, int32_t n_tokens,
                                 int32_t top_k, float *hidden, void *workspace,
                                 size_t workspace_bytes, void *stream)
{
    vq_status st = check_stack(layers, n_layers, n_tokens, top_k);
    if (st != VQ_OK)
        return st;
    if (n_tokens == 0 || n_layers == 0)
        return ok();
    if (!hidden || !aligned(hidden, 16))
        return fail(VQ_ERR_INVALID_ARGUMENT,
                    "hidden: must be a non-NULL, 16-byte aligned device pointer");
    const size_t need = vq_moe_stack_workspace_size(layers, n_layers, n_tokens, top_k);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return fail(VQ_ERR_WORKSPACE,
                    "workspace: need %zu bytes, 256-byte aligned (got %zu bytes at %p)", need,
                    workspace_bytes, workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int32_t l = 0; l < n_layers; ++l) {
        const vq_moe_layer &L = layers[l];
        const vq::TensorDev g = vq::to_dev(*L.gate), u = vq::to_dev(*L.up),
                            dn = vq::to_dev(*L.down);
        // hidden is read by gate+up and then updated in place by the combine,
        // which runs after it on the same stream
        st = run_decode_ffn(g, u, dn, n_tokens, top_k, hidden, true, L.topk_ids, L.topk_weights,
                            hidden, true, decode_ws(*L.gate, *L.down, n_tokens, top_k), workspace,
                            s, "vq_moe_stack");
        if (st != VQ_OK)
            return st;
    }
    return ok();
}

VQ_EXPORT vq_status vq_moe_gate_up(const vq_tensor *gate, const vq_tensor *up, int32_t n_tokens,
                                   int32_t top_k, const void *x, vq_dtype x_dtype,
                                   const int32_t *topk_ids, float *h, void *stream)
{
    vq_status st;
    if ((st = check_tensor(gate, "gate")) != VQ_OK || (st = check_tensor(up, "up")) != VQ_OK)
        return st;
    if (up->rows != gate->rows || up->cols != gate->cols || up->n_experts != gate->n_experts)
        return fail(VQ_ERR_INVALID_ARGUMENT, "up must match gate's shape and n_experts");
    if (up->d != gate->d || up->bits != gate->bits)
        return fail(VQ_ERR_UNSUPPORTED,
                    "gate and up must share d and bits (they run in one fused kernel)");
    if ((st = check_dtype(x_dtype)) != VQ_OK)
        return st;
    if (top_k < 1 || top_k > gate->n_experts)
        return fail(VQ_ERR_INVALID_ARGUMENT, "top_k = %d: must be in [1, n_experts = %d]", top_k,
                    gate->n_experts);
    if ((st = check_decode_sizes(*gate, *gate, n_tokens, top_k)) != VQ_OK)
        return st;
    if (n_tokens == 0)
        return ok();
    if (!x || !aligned(x, 16) || !topk_ids || !h || !aligned(h, 4))
        return fail(VQ_ERR_INVALID_ARGUMENT,
                    "x (16-byte aligned), topk_ids and h must be non-NULL device pointers");
    hipError_t e = launch_gate_up(vq::to_dev(*gate), vq::to_dev(*up), n_tokens, top_k, x,
                                  x_dtype == VQ_F32, topk_ids, h, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "vq_moe_gate_up");
}

VQ_EXPORT vq_status vq_moe_down(const vq_tensor *down, int32_t n_tokens, int32_t top_k,
                                const float *h, const int32_t *topk_ids, float *z, void *stream)
{
    vq_status st;
    if ((st = check_tensor(down, "down")) != VQ_OK)
        return st;
    if (top_k < 1 || top_k > down->n_experts)
        return fail(VQ_ERR_INVALID_ARGUMENT, "top_k = %d: must be in [1, n_experts = %d]", top_k,
                    down->n_experts);
    if ((st = check_decode_sizes(*down, *down, n_tokens, top_k)) != VQ_OK)
        return st;
    if (n_tokens == 0)
        return ok();
    if (!h || !aligned(h, 16) || !topk_ids || !z || !aligned(z, 4))
        return fail(VQ_ERR_INVALID_ARGUMENT,
                    "h (16-byte aligned), topk_ids and z must be non-NULL device pointers");
    hipError_t e = launch_down(vq::to_dev(*down), n_tokens, top_k, h, topk_ids, z,
                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "vq_moe_down");
}

VQ_EXPORT vq_status vq_moe_combine(int32_t n_tokens, int32_t top_k, int32_t hidden, const float *z,
                                   const float *topk_weights, float *y, void *stream)
{
    if (n_tokens < 0 || top_k < 1 || hidden < 0 || hidden % 4 != 0)
        return fail(VQ_ERR_INVALID_ARGUMENT,
                    "n_tokens = %d, top_k = %d, hidden = %d: need n_tokens >= 0, top_k >= 1, "
                    "hidden a multiple of 4", n_tokens, top_k, hidden);
    if (n_tokens == 0 || hidden == 0)
        return ok();
    if (!z || !aligned(z, 16) || !y || !aligned(y, 16) || !topk_weights)
        return fail(VQ_ERR_INVALID_ARGUMENT,
                    "z and y (16-byte aligned) and topk_weights must be non-NULL device pointers");
    hipError_t e = vq::launch_combine(z, topk_weights, n_tokens, top_k, hidden, y, false,
                                      static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ok() : hip_fail(e, "vq_moe_combine");
}
