/*
 * vq_oracle.h -- plain CPU oracle for the vector-quantized MoE expert matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this code; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code with the HIP
 * library (no headers, helpers, tables or constants) and never touches a GPU.
 *
 * What it computes is the plain definition of the method described on the
 * model cards "Qwen3.5-397B-A17B-VQ-2.6bpw" (section "Methodology": one b-bit
 * index per d-weight subvector into a per-tensor fp16 codebook, an fp16 scale
 * per (row, 64 weights); "Sub-byte bit-packing": codes packed into uint32
 * words, row-local, 32-code blocks), "Qwen3.5-397B-A17B-VQ-2.4bpw: Model
 * Card" (Changelog 2026-10-01 "vq-skipzero": dead rows have no codes or
 * scales and output exact zeros) and "GLM-5.3-Flash-VQ-2.7bpw" (section
 * "Methodology": 9-bit codes at K=512, 11-bit at K=2048, fp16 scale per
 * (row, 64 weights)):
 *
 *   1. unpack   code j of a stored row occupies stream bits [j*b, j*b+b);
 *               stream bit q is bit (q mod 32) of word q/32 (LSB first);
 *               each row starts on a word boundary and is padded to whole
 *               32-code blocks (b words per block).
 *   2. decode   W[r][j*d+t] = scale[s][(j*d)/64] * codebook[code][t]; the
 *               product of two fp16 values is exact in fp32.  Dead rows
 *               (row_map[r] < 0) are all zero.
 *   3. matmul   y[n][r] = sum_c W[r][c] * x[n][c], accumulated in fp64.
 *   4. FFN      g = Wg x, u = Wu x, h = silu(g) * u, z = Wd h, and
 *               y[t] = sum_s w[t][s] * z_{ids[t][s]}(t), all in fp64.
 *
 * Each function below cites the passage it follows.  Where the pages are
 * silent (bit order, padding, map format, SwiGLU form) the reading used is
 * the one stated in the repository's design notes; every such reading is
 * listed there.
 */
#ifndef VQ_ORACLE_H
#define VQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One VQ linear tensor, stacked over experts.  All pointers are host memory. */
typedef struct vqo_tensor {
    int32_t rows;             /* logical output features per expert        */
    int32_t cols;             /* input features; a multiple of 64          */
    int32_t d;                /* subvector length: 1, 2, 4 or 8           */
    int32_t bits;             /* code width b, 0..16                       */
    int32_t K;                /* codebook entries, 1 <= K <= 2^b           */
    int32_t n_experts;        /* >= 1                                      */
    int64_t n_stored;         /* stored (live) rows in codes / scales      */
    const uint16_t *codebook; /* fp16 bit patterns, [K][d]                 */
    const uint32_t *codes;    /* [n_stored][words_per_row]                 */
    const uint16_t *scales;   /* fp16 bit patterns, [n_stored][cols/64]    */
    const int32_t *row_map;   /* [n_experts*rows]: stored row or -1 (dead);
                                 NULL means dense: stored = e*rows + r      */
} vqo_tensor;

enum { VQO_OK = 0, VQO_EBADARG = 1, VQO_ECODE = 2, VQO_EMAP = 3, VQO_ENOMEM = 4 };
enum { VQO_X_F32 = 0, VQO_X_BF16 = 1, VQO_X_F64 = 2 };

/* IEEE 754 binary16 bit pattern -> value (exact). */
double vqo_half_to_double(uint16_t h);
/* bfloat16 bit pattern (the upper half of a binary32) -> value (exact). */
double vqo_bf16_to_double(uint16_t h);

/* Words per stored row: ceil(n_sub / 32) * bits, n_sub = cols / d. */
int64_t vqo_words_per_row(int32_t cols, int32_t d, int32_t bits);

/* Code j of a row's bit stream (step 1). */
uint32_t vqo_code(const uint32_t *row_words, int32_t bits, int64_t j);

/* Unpack the first n codes of one row (step 1). */
void vqo_unpack_row(const uint32_t *row_words, int32_t bits, int64_t n, uint32_t *out);

/* Check a descriptor and every code / map entry it references.
   Returns VQO_OK or an error code. */
int vqo_check(const vqo_tensor *T);

/* Decode expert e to dense fp32 W[rows][cols] (step 2). */
int vqo_decode(const vqo_tensor *T, int32_t e, float *W);

/* Y[i][:] = logical row ids[i] of the stacked tensor (id = e*rows + r), fp32,
   for i < n; dead rows are zero, ids outside [0, n_experts*rows) give NaN
   rows.  Y: [n][cols]. */
int vqo_gather(const vqo_tensor *T, int64_t n, const int64_t *ids, float *Y);

/* y[n][r] = sum_c W_e[r][c] * x[n][c] in fp64 (step 3).  x holds n_tok rows
   of cols values in x_dtype (VQO_X_F32 / VQO_X_BF16 bit patterns or
   VQO_X_F64 values); y is [n_tok][rows]. */
int vqo_linear(const vqo_tensor *T, int32_t e, int32_t n_tok,
               const void *x, int32_t x_dtype, double *y);

/* Routed SwiGLU expert FFN (step 4) for the tokens listed in `tokens`
   (n_sel entries, each in [0, n_tok)); y is [n_sel][hidden] in fp64.
   ids and w are [n_tok][top_k]; x is [n_tok][hidden] in x_dtype. */
int vqo_moe_ffn(const vqo_tensor *gate, const vqo_tensor *up, const vqo_tensor *down,
                int32_t n_tok, int32_t top_k, const void *x, int32_t x_dtype,
                const int32_t *ids, const float *w,
                int32_t n_sel, const int32_t *tokens, double *y);

/* SwiGLU activation product silu(g) * u with silu(z) = z / (1 + exp(-z)). */
double vqo_swiglu(double g, double u);

/* A stack of MoE layers (step 5): h <- h + FFN_l(h) for l = 0..n_layers-1,
   FFN_l as in vqo_moe_ffn over all tokens, with layer l's tensors and
   routing (ids[l], w[l]: [n_tok][top_k]).  h: [n_tok][hidden] fp64, in
   place. */
int vqo_moe_stack(int32_t n_layers, const vqo_tensor *const *gate,
                  const vqo_tensor *const *up, const vqo_tensor *const *down,
                  int32_t n_tok, int32_t top_k, const int32_t *const *ids,
                  const float *const *w, double *h);

/* ---- Step 0: fitting the format (test infrastructure for the fit) ---- */

/* fp32 -> fp16 bits, round to nearest even. */
uint16_t vqo_float_to_half(float f);

/* scales[r][g] = fp16(max |w[r][64g .. 64g+63]|); w: bf16 bits [n_rows][cols]. */
int vqo_fit_scales(int64_t n_rows, int32_t cols, const uint16_t *w, uint16_t *scales);

/* Lloyd's k-means on the normalised subvectors named by sample[0..n_sample)
   (subvector i = r*(cols/d) + j), from the K subvectors named by init, for
   iters iterations; C: fp32 [K][d] out.  n_sample <= 2^22. */
int vqo_kmeans(int64_t n_rows, int32_t cols, int32_t d, int32_t K, const uint16_t *w,
               const uint16_t *scales, int64_t n_sample, const int64_t *sample,
               const int64_t *init, int32_t iters, float *C);

/* Every subvector coded to its nearest fp16 codebook entry and packed:
   codes [n_rows][words_per_row]. */
int vqo_encode(int64_t n_rows, int32_t cols, int32_t d, int32_t bits, int32_t K,
               const uint16_t *w, const uint16_t *scales, const uint16_t *codebook,
               uint32_t *codes);

/* scales, k-means, fp16 codebook, encode: the whole fit. */
int vqo_fit(int64_t n_rows, int32_t cols, int32_t d, int32_t bits, int32_t K, const uint16_t *w,
            int64_t n_sample, const int64_t *sample, const int64_t *init, int32_t iters,
            uint16_t *codebook, uint16_t *scales, uint32_t *codes);

/* OpenMP threads of the loops above (n > 0), and the current count. */
void vqo_set_threads(int32_t n);
int32_t vqo_threads(void);

#ifdef __cplusplus
}
#endif
#endif /* VQ_ORACLE_H */
