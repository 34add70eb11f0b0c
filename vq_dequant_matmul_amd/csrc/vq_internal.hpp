// vq_internal.hpp -- host-side interface between the C ABI layer and the
// kernel launchers.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/vq.h"

namespace vq {

// A tensor's device pointers and derived sizes.
struct TensorDev {
    const uint32_t *codes;
    const uint16_t *scales;
    const uint16_t *codebook;
    const int32_t *row_map;
    int rows, cols, d, bits, K, n_experts;
    int64_t n_stored;
    int groups;      // cols / 64
    int wpr;         // words per stored row
    int cb_dwords;   // K * d / 2
};

TensorDev to_dev(const vq_tensor &t);

// Decode-engine work description (one launch).
struct RowsLaunch {
    TensorDev t[2];        // one or two projections (gate, up)
    int nproj;             // 1 or 2 (2 = SwiGLU of t[0] (gate) and t[1] (up))
    const void *act;       // activations: rows of t[0].cols elements
    int act_f32;           // 0: bf16 bit patterns; 1: fp32 activations (hi + lo fp16
                           // terms); 2: fp32 activations rounded once to fp16
    int64_t act_stride;    // elements between activation rows
    float *out;            // output rows
    int64_t out_stride;    // elements between output rows
    // work list: either one expert applied to n_act activation rows ...
    int expert;
    int n_act;
    // ... or routed slots: pair q (< n_slots) uses expert ids[q]; its
    // activation row is q / act_div (act_div = top_k for token inputs, 1
    // for per-pair inputs) and its output row is q.
    const int32_t *ids;
    int n_slots;
    int act_div;
    // set when one expert may serve several pairs of the list (more than one
    // token, or repeated ids within a token); selects the multi-row kernel
    int multi_per_expert;
};

hipError_t launch_rows(const RowsLaunch &L, hipStream_t stream);

// y[t][c] = sum_s w[t][s] * z[t*k + s][c], slot order (accumulate: y[t][c] +=
// that sum).
// ceiling probes (vq_probe.hip)
hipError_t launch_probe_read(const void *p, size_t bytes, uint32_t *out, int n_wg,
                             hipStream_t stream);
hipError_t launch_probe_mfma(int n_wg, int iters, float *out, hipStream_t stream);

hipError_t launch_combine(const float *z, const float *w, int n_tok, int top_k, int hidden,
                          float *y, bool accumulate, hipStream_t stream);

hipError_t launch_dequantize(const TensorDev &t, int expert, float *w, hipStream_t stream);

// Fitting the format (scales, Lloyd iterations, fp16 codebook, encode).
struct FitArgs {
    int64_t n_rows;
    int cols, d, bits, K;
    const uint16_t *w;          // bf16 [n_rows][cols]
    int64_t n_sample;
    const int64_t *sample;      // [n_sample] subvector indices (the fit set)
    const int64_t *init;        // [K] subvector indices (initial centroids)
    int iters;
    uint16_t *codebook;         // fp16 [K][d] out
    uint16_t *scales;           // fp16 [n_rows][cols/64] out
    uint32_t *codes;            // [n_rows][wpr] out
    float *xs;                  // workspace: fit-set vectors [n_sample][d]
    float *C;                   // workspace: centroids [K][d]
    unsigned long long *sums;   // workspace: [K*d] sums, then [K] counts
};
// Workspace bytes; with f set, also places f's workspace pointers in ws.
size_t fit_workspace_bytes(int d, int K, int64_t n_sample, FitArgs *f, void *ws);
hipError_t launch_fit(const FitArgs &f, hipStream_t stream);

// y[i] = logical row ids[i] (= e*rows + r) of the stacked tensor, fp32.
hipError_t launch_gather(const TensorDev &t, int64_t n, const int64_t *ids, float *y,
                         hipStream_t stream);

// Down projection fused with the slot-ordered combine for a few tokens:
// y[t] = sum_s w[t][s] * W_down_{e[t][s]} h[t*top_k + s] (accumulate: y[t] +=
// that sum).  mix_supported() tells whether the shapes fit the fused kernel.
bool mix_supported(const TensorDev &dn, int n_tok, int top_k);
hipError_t launch_mix(const TensorDev &dn, int n_tok, int top_k, const float *h,
                      const int32_t *ids, const float *w, float *y, bool accumulate,
                      hipStream_t stream);

// Prefill (MFMA) path.
struct GemmLaunch;
size_t gemm_workspace_bytes(const TensorDev &t, int n_x_rows);
hipError_t launch_expert_gemm(const TensorDev &t, int n_x_rows, const void *x, int x_f32,
                              const int32_t *expert_offsets, float *y, void *ws,
                              hipStream_t stream);
size_t moe_prefill_workspace_bytes(const TensorDev &g, const TensorDev &u, const TensorDev &dn,
                                   int n_tok, int top_k);
hipError_t launch_moe_prefill(const TensorDev &g, const TensorDev &u, const TensorDev &dn,
                              int n_tok, int top_k, const void *x, int x_f32,
                              const int32_t *ids, const float *w, float *y, void *ws,
                              hipStream_t stream);

// Events the caller asked to record around the dominant kernel of the next
// calls on this thread (both null = off).
struct KernelEvents {
    hipEvent_t start, stop;
};
KernelEvents &kernel_events();

// Limits of the decode engine.
constexpr int kMaxSlots = 1024;      // n_tokens * top_k in one routed launch
constexpr int kMaxGroupsDecode = 128; // cols <= 8192
constexpr int kMaxCodebookBytes = 65536;

// Limits of the grouped-GEMM path (routed pairs are int32; activation
// matrices are addressed in 32-bit bytes).
constexpr int64_t kMaxPrefillPairs = 0x7fffffff;
constexpr int64_t kMaxGemmActBytes = (int64_t)1 << 32;

}  // namespace vq
