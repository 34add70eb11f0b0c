/*
 * vq.h -- C ABI of the vector-quantized MoE expert matmul for MI355X (gfx950).
 *
 * The weight format is the one described on the VQ model cards:
 *   - "Qwen3.5-397B-A17B-VQ-2.6bpw", section "Methodology": each d-weight
 *     subvector of a row stores one b-bit index into a per-tensor fp16
 *     codebook of K d-vectors, with an fp16 scale per (row, 64 weights);
 *     section "Sub-byte bit-packing": codes are packed into uint32 words,
 *     row-local, in 32-code blocks.
 *   - "GLM-5.3-Flash-VQ-2.7bpw", section "Methodology": 9-bit codes at
 *     K=512 and 11-bit codes at K=2048, sub-byte packed into uint32 words.
 *   - "Qwen3.8-Flash-Next-VQ-4.4bpw": d=2/K=256 experts with d=2/K=1024
 *     (10-bit packed) layers.
 *   - "Qwen3.5-397B-A17B-VQ-2.4bpw: Model Card", changelog 2026-10-01
 *     ("vq-skipzero"): dead output rows have no codes or scales and output
 *     exact zeros.
 *
 * Layout of one tensor (one projection of one MoE layer, all experts):
 *   logical weight of expert e:  W_e[rows][cols]  (out x in), y = W_e x
 *   n_sub  = cols / d            codes per row
 *   wpr    = ceil(n_sub/32)*bits uint32 words per stored row
 *   code j of a stored row = stream bits [j*bits, j*bits+bits), where stream
 *          bit q is bit (q mod 32) of word q/32 of that row (LSB first); the
 *          tail of the last 32-code block is zero padding
 *   W_e[r][j*d+t] = scale[s][(j*d)/64] * codebook[code_j][t],
 *          s = the stored row of logical row r of expert e
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers; descriptors are host structs
 *     read during the call and not retained.  The caller owns every buffer;
 *     the library never allocates, frees or synchronizes in these calls.
 *     Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and the call returns without waiting.
 *   - Host-visible arguments are validated; a bad one returns a non-zero
 *     vq_status and sets a thread-local message naming the field
 *     (vq_last_error).  Device-resident contents (codes >= K, row-map
 *     entries, expert ids out of range, non-finite values) cannot be checked
 *     without a synchronization and are preconditions: violating them gives
 *     undefined output but never an out-of-bounds access for codes (the
 *     kernels' codebook lookups stay inside the LDS copy of the codebook, and
 *     the exact dequantisation reads entry K-1 for a code >= K) -- ids and
 *     row maps must be in range.
 *   - A HIP launch error returns VQ_ERR_HIP with the runtime's message.
 *   - Results are bit-reproducible run to run (no floating-point atomics).
 *   - One codebook per tensor, shared by all its experts: codebooks are
 *     replicated, never sliced ("gemma-4-26b-a4b-it-VQ-6.2bpw", section
 *     "Multi-machine (exo) note").
 */
#ifndef VQ_H
#define VQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VQ_ABI_VERSION 1

typedef enum vq_status {
    VQ_OK = 0,
    VQ_ERR_INVALID_ARGUMENT = 1, /* a null pointer, a negative size, mismatched shapes */
    VQ_ERR_UNSUPPORTED = 2,      /* a geometry or size the kernels do not handle      */
    VQ_ERR_WORKSPACE = 3,        /* workspace missing or smaller than required        */
    VQ_ERR_HIP = 4               /* the HIP runtime reported an error                 */
} vq_status;

typedef enum vq_dtype {
    VQ_F32 = 0,  /* IEEE binary32 activations                     */
    VQ_BF16 = 1  /* bfloat16 activations (bit patterns, uint16)   */
} vq_dtype;

/* One VQ linear tensor stacked over experts. */
typedef struct vq_tensor {
    int32_t rows;             /* logical out features per expert, >= 1          */
    int32_t cols;             /* in features, a positive multiple of 64         */
    int32_t d;                /* subvector length: 2, 4 or 8                    */
    int32_t bits;             /* code width: 8..13                              */
    int32_t K;                /* codebook entries: 1 <= K <= 2^bits, and the
                                 fp16 codebook (K*d*2 bytes) must fit 64 KiB   */
    int32_t n_experts;        /* >= 1 (1 for a plain linear layer)              */
    int64_t n_stored;         /* stored rows in codes/scales; == n_experts*rows
                                 when row_map is NULL                          */
    const uint16_t *codebook; /* fp16 bits [K][d]                               */
    const uint32_t *codes;    /* [n_stored][wpr]                                */
    const uint16_t *scales;   /* fp16 bits [n_stored][cols/64]                  */
    const int32_t *row_map;   /* [n_experts*rows]: stored row of logical row r
                                 of expert e at [e*rows + r], or -1 when the row
                                 is dead (skip-zero); NULL = dense, stored row
                                 e*rows + r                                      */
} vq_tensor;

/* ---- housekeeping ---------------------------------------------------- */

int32_t vq_abi_version(void);
const char *vq_status_string(vq_status s);
/* Message of the last failed call on this thread ("" if none). */
const char *vq_last_error(void);

/* Host-only checks of a descriptor (no GPU work). */
vq_status vq_validate(const vq_tensor *W);

/* ---- dequantize (exact) ---------------------------------------------- */

/* w[r][c] = W_e[r][c] as fp32 for expert `expert`, dead rows +0.0.
   The fp16 x fp16 product is exact in fp32, so the result is bit-identical
   to any exact decode.  w: device [rows][cols] fp32. */
vq_status vq_dequantize(const vq_tensor *W, int32_t expert, float *w, void *stream);

/* ---- row gather (VQ embedding tables) -------------------------------- */

/* Card "Qwen3.8-Flash-Next-VQ-4.4bpw" (opening summary; changelog
   2026-10-04): the per-layer n-gram embedding tables are stored in this same
   format (d=2/K=256 there) and read one hashed row per lookup.  Here the
   tables are the experts of W: id = e*rows + r names logical row r of table
   e, and
     y[i][c] = W_e[r][c] as fp32 for i < n (exact, as vq_dequantize),
   a dead row giving +0.0 and an id outside [0, n_experts*rows) a row of NaN
   (a bad id shows in the output; nothing outside the tensor is read).  The
   hash that turns tokens into ids is the model's and not part of this call.
   ids: device int64 [n], 8-byte aligned; y: device fp32 [n][cols], 16-byte
   aligned.  n = 0 is a no-op.  Bandwidth-bound (HBM roofline, dominated by
   the fp32 output). */
vq_status vq_row_gather(const vq_tensor *W, int64_t n, const int64_t *ids, float *y,
                        void *stream);

/* ---- decode: one expert, a few tokens ---------------------------------- */

/* Card "Qwen3.8-Flash-Next-VQ-4.4bpw", changelog entry "2026-09 — bundle
   refresh": the runtime's decode-time expert kernels read an expert's packed
   codes straight from memory, with the activations read directly and a
   SIMD-wide sum; card "GLM-5.3-Flash-VQ-2.7bpw", Limitations: small-batch
   decode is where the format's kernels are least settled.
     y[n][r] = sum_c W_e[r][c] * x[n][c] for n < n_tokens (0..64), fp32 out.
   x: [n_tokens][cols] in x_dtype; y: [n_tokens][rows] fp32.  Dead rows
   write +0.0.  Bandwidth-bound path (HBM roofline). */
vq_status vq_expert_gemv(const vq_tensor *W, int32_t expert, int32_t n_tokens,
                         const void *x, vq_dtype x_dtype, float *y, void *stream);

/* ---- prefill: grouped GEMM over experts ---------------------------------- */

/* Card "gemma-4-26b-a4b-it-VQ-6.2bpw", section "Faster prefill (optional)":
   for long prompts the runtime turns the experts' codes into weights a chunk
   at a time before its matmul; card "Qwen3.8-Flash-Next-VQ-4.4bpw",
   changelog 2026-09-09: prefill kernel arms are chosen per geometry (large
   codebooks, d = 8).  Here one launch serves every expert of a batch.
   Rows of x are grouped by expert: rows [expert_offsets[e], expert_offsets[e+1])
   use expert e.  y[i][r] = sum_c W_e[r][c] * x[i][c], fp32, dead rows +0.0.
   expert_offsets: device int32 [n_experts+1], non-decreasing, from 0 to
   n_x_rows.  x: [n_x_rows][cols]; y: [n_x_rows][rows].  MFMA path with
   dequantised fp16 tiles.  workspace: device, at least
   vq_expert_gemm_workspace_size() bytes, 256-byte aligned. */
size_t vq_expert_gemm_workspace_size(const vq_tensor *W, int32_t n_x_rows);
vq_status vq_expert_gemm(const vq_tensor *W, int32_t n_x_rows, const void *x, vq_dtype x_dtype,
                         const int32_t *expert_offsets, float *y,
                         void *workspace, size_t workspace_bytes, void *stream);

/* ---- the routed SwiGLU expert FFN ----------------------------------------- */

/* The models on the cards are mixture-of-experts transformers whose routed
   experts are the VQ tensors (card "gemma-4-26b-a4b-it-VQ-6.2bpw", section
   "How it was built": the experts hold most of the language model's bytes
   and are the vector-quantized part; card "Qwen3.8-Flash-Next-VQ-4.4bpw",
   changelog 2026-09 memory notes: a token touches only its routed experts).
   The pages do not spell out the expert MLP or how routed outputs combine;
   this call takes the plainest reading, a gated (SwiGLU) MLP per expert and
   a weighted sum over the token's top_k routed experts:
   For each token t and slot s < top_k with expert e = topk_ids[t][s]:
     g = W_gate_e x_t,  u = W_up_e x_t,  h = silu(g) * u  (silu(z) = z/(1+e^-z)),
     y[t] = sum_s topk_weights[t][s] * (W_down_e h).
   Shapes: gate, up: rows = inter, cols = hidden; down: rows = hidden,
   cols = inter; all three share n_experts.  x: [n_tokens][hidden] in
   x_dtype; topk_ids int32 and topk_weights fp32 [n_tokens][top_k];
   y: [n_tokens][hidden] fp32.  The bandwidth-bound decode kernels (the
   three stages below, in order) run every batch of up to 16 tokens, and
   larger batches of at most max(176, 3*n_experts/4) routed pairs
   (n_tokens*top_k) with hidden
   and inter at most 8192; other batches run the grouped MFMA GEMM
   (vq_moe_ffn_engine says which); that path carries x, h and the down
   projection's outputs in fp16 with power-of-two range scaling and
   accumulates in fp32.  workspace: device, at least
   vq_moe_ffn_workspace_size() bytes, 256-byte aligned. */
size_t vq_moe_ffn_workspace_size(const vq_tensor *gate, const vq_tensor *up,
                                 const vq_tensor *down, int32_t n_tokens, int32_t top_k);
vq_status vq_moe_ffn(const vq_tensor *gate, const vq_tensor *up, const vq_tensor *down,
                     int32_t n_tokens, int32_t top_k, const void *x, vq_dtype x_dtype,
                     const int32_t *topk_ids, const float *topk_weights, float *y,
                     void *workspace, size_t workspace_bytes, void *stream);

/* The engine vq_moe_ffn runs for these arguments: *engine = VQ_ENGINE_DECODE
   (the three small-batch stages) or VQ_ENGINE_MFMA (the grouped GEMM).  Host
   only: no device work, no device pointers.  Errors as vq_moe_ffn's
   argument checks. */
#define VQ_ENGINE_DECODE 0
#define VQ_ENGINE_MFMA 1
vq_status vq_moe_ffn_engine(const vq_tensor *gate, const vq_tensor *up, const vq_tensor *down,
                            int32_t n_tokens, int32_t top_k, int32_t *engine);

/* vq_moe_ffn for callers that cannot allocate device memory (code under HIP
   graph capture, tight serving loops, harnesses that forbid hipMalloc): the
   same computation and kernels as vq_moe_ffn, bit for bit, with the
   workspace taken from a static device array of VQ_NOALLOC_SCRATCH_BYTES
   (64 MiB) that every GPU the library runs on holds from the library's load
   until the process ends.  Nothing is allocated or freed in the call.  A
   call whose vq_moe_ffn_workspace_size() exceeds the array returns
   VQ_ERR_UNSUPPORTED (that covers every batch on the decode kernels up to
   1024 routed pairs of hidden + inter <= 16384, and batches on the grouped
   GEMM of a few thousand routed pairs: 4400 at hidden 4096 and inter 1024,
   6320 at 2816 and 704).  All calls on one GPU share its array: calls that
   overlap on that GPU (several streams or threads at once) race and give
   undefined output; calls in order on one stream are safe.  The array's
   address is looked up on the first call on each device (with that device
   current); `stream` must belong to the current device. */
#define VQ_NOALLOC_SCRATCH_BYTES (64u << 20)
vq_status vq_moe_ffn_noalloc(const vq_tensor *gate, const vq_tensor *up, const vq_tensor *down,
                             int32_t n_tokens, int32_t top_k, const void *x, vq_dtype x_dtype,
                             const int32_t *topk_ids, const float *topk_weights, float *y,
                             void *stream);

/* ---- the three stages of the small-batch FFN, callable one by one -------- */

/* Stage 1 (gate, up, SwiGLU): for pair q = t*top_k + s with e = topk_ids[t][s],
     h[q][r] = silu(g) * u,  g = (W_gate_e x_t)[r],  u = (W_up_e x_t)[r];
   a row dead in gate or in up gives h = +0.0.  Each routed expert's weights
   are read once however many pairs it serves.  n_tokens*top_k <= 1024;
   h: device fp32 [n_tokens*top_k][inter]. */
vq_status vq_moe_gate_up(const vq_tensor *gate, const vq_tensor *up, int32_t n_tokens,
                         int32_t top_k, const void *x, vq_dtype x_dtype,
                         const int32_t *topk_ids, float *h, void *stream);

/* Stage 2 (down): z[q][c] = sum_r W_down_e[c][r] * h[q][r] for every pair q;
   dead rows of down give +0.0.  h enters the products rounded once to
   fp16, scaled by a power of two per (pair, 64-column group), as the
   grouped GEMM's h does.  h: device fp32 [n_tokens*top_k][inter];
   z: device fp32 [n_tokens*top_k][hidden]. */
vq_status vq_moe_down(const vq_tensor *down, int32_t n_tokens, int32_t top_k, const float *h,
                      const int32_t *topk_ids, float *z, void *stream);

/* Stage 3 (combine): y[t][c] = sum over s in slot order of
   topk_weights[t][s] * z[t*top_k + s][c].  z, y: device fp32, 16-byte
   aligned; hidden a multiple of 4. */
vq_status vq_moe_combine(int32_t n_tokens, int32_t top_k, int32_t hidden, const float *z,
                         const float *topk_weights, float *y, void *stream);

/* ---- a stack of MoE layers on a residual stream (small batches) ---------- */

/* Decode through several MoE layers in one call.  Layers may differ in
   geometry (d, bits, K) and in inter size, as the promoted layers do on
   the cards "GLM-5.3-Flash-VQ-2.7bpw" (opening summary: eight layers at
   d=4/K=2048 among d=4/K=512 ones) and "Qwen3.8-Flash-Next-VQ-4.4bpw"
   (opening summary: seven layers at d=2/K=1024 among d=2/K=256 ones); they
   share hidden size and top_k.  Each
   layer brings its own routing (topk_ids, topk_weights: device
   [n_tokens][top_k], as for vq_moe_ffn).  For l = 0 .. n_layers-1, in order:
     hidden[t] <- hidden[t] + FFN_l(hidden[t])      (FFN_l as in vq_moe_ffn)
   hidden: device fp32 [n_tokens][hidden size], 16-byte aligned, read and
   updated in place.  The router, attention and norms between the MoE blocks
   are not part of this call.  n_tokens <= 16 (the decode kernels, two
   launches per layer; capture the call in a HIP graph to replay a step).
   workspace: device, at least vq_moe_stack_workspace_size() bytes, 256-byte
   aligned; shared by the layers in turn. */
typedef struct vq_moe_layer {
    const vq_tensor *gate;       /* rows = inter, cols = hidden size        */
    const vq_tensor *up;         /* same shape, d and bits as gate           */
    const vq_tensor *down;       /* rows = hidden size, cols = inter         */
    const int32_t *topk_ids;     /* device int32 [n_tokens][top_k]           */
    const float *topk_weights;   /* device fp32 [n_tokens][top_k]            */
} vq_moe_layer;

size_t vq_moe_stack_workspace_size(const vq_moe_layer *layers, int32_t n_layers,
                                   int32_t n_tokens, int32_t top_k);
vq_status vq_moe_stack(const vq_moe_layer *layers, int32_t n_layers, int32_t n_tokens,
                       int32_t top_k, float *hidden, void *workspace, size_t workspace_bytes,
                       void *stream);

/* ---- fitting the format ------------------------------------------------------- */

/* The step before the path: produce codebook, scales and packed codes from
   bf16 weights.  The cards fit "data-free" by k-means / Lloyd over the
   weight subvectors from a seeded or unseeded subsample, with an fp16 scale
   per (row, 64 weights) ("Methodology" sections of the Qwen3.5-397B-A17B
   2.6bpw and 2.4bpw, Qwen3.8-Flash-Next and GLM-5.3-Flash cards).  Here:
     scales[r][g] = fp16 (nearest even) of max |w| over the group;
     subvector i = r*(cols/d) + j is v = w[r][j*d .. j*d+d) / s in fp32
       (a group with s == 0 gives zeros);
     centroids start at the subvectors init[0..K); each of `iters` Lloyd
       passes assigns every subvector named in sample[0..n_sample) to its
       nearest centroid and moves each centroid with members to their mean
       (distances: fp32 sums of rounded squares in coordinate order, ties to
       the lower index; means: exact integer sums on a 2^-30 grid divided
       in fp64), so the result does not depend on thread order;
     codebook = the centroids in fp16; every subvector of the tensor is
       coded to its nearest codebook entry and packed as in the layout above.
   The outputs form a dense vq_tensor with rows = n_rows (no row map).
   w: device bf16 [n_rows][cols], 16-byte aligned; sample, init: device
   int64 subvector indices (in range: a precondition; out-of-range values
   are clamped), n_sample <= 2^22; codebook: device fp16 [K][d]; scales:
   device fp16 [n_rows][cols/64]; codes: device uint32 [n_rows][wpr].
   K*d <= 16384 (the centroids are searched from LDS as fp32).  Weights must
   be finite with |w| <= 65504.  workspace: at least vq_fit_workspace_size()
   bytes, 256-byte aligned. */
size_t vq_fit_workspace_size(int32_t d, int32_t K, int64_t n_sample);
vq_status vq_fit(int64_t n_rows, int32_t cols, int32_t d, int32_t bits, int32_t K,
                 const uint16_t *w, int64_t n_sample, const int64_t *sample,
                 const int64_t *init, int32_t iters, uint16_t *codebook, uint16_t *scales,
                 uint32_t *codes, void *workspace, size_t workspace_bytes, void *stream);

/* ---- measurement -------------------------------------------------------------- */

/* Until cleared (NULL, NULL), every vq_moe_ffn / vq_moe_gate_up /
   vq_expert_gemm / vq_fit call made on this thread records `start` (a
   hipEvent_t) on its stream right before its dominant kernel (the fused
   gate+up launch; the GEMM for vq_expert_gemm; the encode pass for vq_fit)
   and `stop` right after it, so a caller can
   time that one kernel with hipEventElapsedTime.  The events are owned by
   the caller. */
vq_status vq_set_kernel_events(void *start, void *stop);

/* ---- ceiling probes (measurement only) ---------------------------------- */

/* Streaming read of buf (device, 16-byte aligned, bytes a multiple of 16)
   by n_workgroups workgroups of 256 lanes, each lane loading 16 bytes per
   load with four loads in flight; out: device uint32 [n_workgroups*256]
   receives an xor of what each lane read.  Times the best-case HBM read
   rate of the device, the ceiling beside the 8 TB/s published peak. */
vq_status vq_probe_read(const void *buf, size_t bytes, int32_t n_workgroups, uint32_t *out,
                        void *stream);

/* iters x 4 dependent-chain-free v_mfma_f32_32x32x16_f16 per wave on
   register operands (32768 flops each), n_workgroups workgroups of four
   waves, no memory traffic; out: device fp32 [n_workgroups*256].  Times the
   fp16 matrix-core rate the device holds, the ceiling beside the
   2.5 PFLOP/s published dense peak. */
vq_status vq_probe_mfma(int32_t n_workgroups, int32_t iters, float *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* VQ_H */
