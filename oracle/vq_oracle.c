/*
 * vq_oracle.c -- plain CPU oracle for the vector-quantized MoE expert matmul.
 *
 * TEST INFRASTRUCTURE ONLY (see vq_oracle.h): used by the test suite, the
 * smoke check and the benchmark's CPU-baseline leg, never by the product path.
 *
 * Written for clarity, not speed: codes are unpacked one bit at a time,
 * weights are decoded to a dense fp32 matrix, and every dot product is a
 * straight fp64 loop with the column index ascending.  OpenMP only splits
 * independent output rows across threads; it does not change any sum.
 */
#include "vq_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads of the OpenMP loops below (they only split independent output
   rows; no sum depends on the count).  Used to time the oracle at one
   thread and at all host cores. */
void vqo_set_threads(int32_t n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int32_t vqo_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------- */
/* Number formats                                                          */
/* ---------------------------------------------------------------------- */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
   bits.  Normal: (-1)^s * 2^(e-15) * (1 + f/1024).  Subnormal (e == 0):
   (-1)^s * 2^-14 * (f/1024).  e == 31: infinity (f == 0) or NaN.
   The model cards store codebooks and scales in this format ("fp16"). */
double vqo_half_to_double(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);               /* f/1024 * 2^-14 */
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + f), e - 25);   /* (1+f/1024) * 2^(e-15) */
    return s ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
   Normal: (-1)^s * 2^(e-127) * (1 + f/128).  Subnormal: (-1)^s * 2^-126 *
   (f/128).  e == 255: infinity or NaN.  Activations arrive in this format
   ("bf16 I/O" on the Qwen3.8-Flash-Next-VQ-4.4bpw card, changelog 2026-09-17). */
double vqo_bf16_to_double(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int f = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);              /* f/128 * 2^-126 */
    else if (e == 255)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(128 + f), e - 134);   /* (1+f/128) * 2^(e-127) */
    return s ? -v : v;
}

static double x_value(const void *x, int32_t dtype, int64_t i)
{
    if (dtype == VQO_X_F32) {
        float f;
        memcpy(&f, (const char *)x + 4 * i, 4);
        return (double)f;
    }
    if (dtype == VQO_X_BF16)
        return vqo_bf16_to_double(((const uint16_t *)x)[i]);
    return ((const double *)x)[i];
}

/* ---------------------------------------------------------------------- */
/* Step 1: the packed code stream                                          */
/* ---------------------------------------------------------------------- */

/* Model card "Qwen3.5-397B-A17B-VQ-2.6bpw", section "Sub-byte bit-packing":
   codes are packed into uint32 words, row-local, in 32-code blocks.  32 codes
   of b bits fill exactly b words, so a row of n_sub = cols/d codes takes
   ceil(n_sub/32) blocks = ceil(n_sub/32) * b words (the tail of the last
   block is padding). */
int64_t vqo_words_per_row(int32_t cols, int32_t d, int32_t bits)
{
    int64_t n_sub = cols / d;
    return ((n_sub + 31) / 32) * (int64_t)bits;
}

/* Code j = stream bits [j*b, j*b + b), least significant bit first; stream
   bit q is bit (q mod 32) of word q / 32.  Assembled one bit at a time. */
uint32_t vqo_code(const uint32_t *row_words, int32_t bits, int64_t j)
{
    uint32_t code = 0;
    for (int32_t i = 0; i < bits; ++i) {
        int64_t q = j * (int64_t)bits + i;
        uint32_t bit = (row_words[q / 32] >> (q % 32)) & 1u;
        code |= bit << i;
    }
    return code;
}

void vqo_unpack_row(const uint32_t *row_words, int32_t bits, int64_t n, uint32_t *out)
{
    for (int64_t j = 0; j < n; ++j)
        out[j] = vqo_code(row_words, bits, j);
}

/* ---------------------------------------------------------------------- */
/* Descriptor checks                                                       */
/* ---------------------------------------------------------------------- */

static int64_t stored_row(const vqo_tensor *T, int32_t e, int32_t r)
{
    if (T->row_map == NULL)
        return (int64_t)e * T->rows + r;
    return T->row_map[(int64_t)e * T->rows + r];
}

int vqo_check(const vqo_tensor *T)
{
    if (!T || T->rows < 0 || T->cols < 0 || T->n_experts < 1)
        return VQO_EBADARG;
    if (T->d != 1 && T->d != 2 && T->d != 4 && T->d != 8)
        return VQO_EBADARG;
    if (T->cols % 64 != 0 || T->bits < 0 || T->bits > 16)
        return VQO_EBADARG;
    if (T->K < 1 || (int64_t)T->K > ((int64_t)1 << T->bits))
        return VQO_EBADARG;
    if (T->row_map == NULL && T->n_stored != (int64_t)T->n_experts * T->rows)
        return VQO_EMAP;
    /* Every stored row referenced at most once, every index in range. */
    if (T->row_map != NULL) {
        char *seen = (char *)calloc((size_t)(T->n_stored > 0 ? T->n_stored : 1), 1);
        if (!seen)
            return VQO_ENOMEM;
        for (int64_t i = 0; i < (int64_t)T->n_experts * T->rows; ++i) {
            int32_t s = T->row_map[i];
            if (s < -1 || s >= T->n_stored || (s >= 0 && seen[s])) {
                free(seen);
                return VQO_EMAP;
            }
            if (s >= 0)
                seen[s] = 1;
        }
        free(seen);
    }
    int64_t wpr = vqo_words_per_row(T->cols, T->d, T->bits);
    int64_t n_sub = T->cols / T->d;
    for (int64_t s = 0; s < T->n_stored; ++s)
        for (int64_t j = 0; j < n_sub; ++j)
            if (vqo_code(T->codes + s * wpr, T->bits, j) >= (uint32_t)T->K)
                return VQO_ECODE;
    return VQO_OK;
}

/* ---------------------------------------------------------------------- */
/* Step 2: decode to dense weights                                         */
/* ---------------------------------------------------------------------- */

/* Model card "Qwen3.5-397B-A17B-VQ-2.6bpw", section "Methodology": each
   d-weight subvector stores one index into a per-tensor fp16 codebook, with
   an fp16 scale per (row, 64 weights).  Subvector j of row r covers columns
   [j*d, j*d + d); its scale is the one of group (j*d)/64.  The product of
   two fp16 numbers has at most 22 significant bits and an exponent well
   inside fp32's range, so computing it in double and storing it as float is
   exact.  Skip-zero ("Qwen3.5-397B-A17B-VQ-2.4bpw: Model Card", changelog
   2026-10-01): a dead row has no codes or scales and is exactly zero.

   One logical row: s is its stored row (-1 = dead); writes cols floats. */
static int decode_row(const vqo_tensor *T, int64_t s, float *wr)
{
    if (s < 0) {
        for (int32_t c = 0; c < T->cols; ++c)
            wr[c] = 0.0f;
        return VQO_OK;
    }
    if (s >= T->n_stored)
        return VQO_EMAP;
    const int64_t wpr = vqo_words_per_row(T->cols, T->d, T->bits);
    const int64_t groups = T->cols / 64;
    const int64_t n_sub = T->cols / T->d;
    const uint32_t *words = T->codes + s * wpr;
    const uint16_t *srow = T->scales + s * groups;
    int err = VQO_OK;
    for (int64_t j = 0; j < n_sub; ++j) {
        uint32_t code = vqo_code(words, T->bits, j);
        if (code >= (uint32_t)T->K) {
            err = VQO_ECODE;
            code = 0;
        }
        double scale = vqo_half_to_double(srow[(j * T->d) / 64]);
        for (int32_t t = 0; t < T->d; ++t) {
            double c = vqo_half_to_double(T->codebook[(int64_t)code * T->d + t]);
            wr[j * T->d + t] = (float)(scale * c);
        }
    }
    return err;
}

int vqo_decode(const vqo_tensor *T, int32_t e, float *W)
{
    if (!T || e < 0 || e >= T->n_experts || !W)
        return VQO_EBADARG;
    int err = VQO_OK;

#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < T->rows; ++r) {
        int rc = decode_row(T, stored_row(T, e, r), W + (int64_t)r * T->cols);
        if (rc != VQO_OK) {
#pragma omp atomic write
            err = rc;
        }
    }
    return err;
}

/* Row gather.  Model card "Qwen3.8-Flash-Next-VQ-4.4bpw" (opening summary
   and changelog 2026-10-04): the per-layer n-gram embedding (PLE) tables are
   stored in the same VQ format (d=2/K=256) and read one hashed row per
   lookup.  The tables of a stacked tensor are its experts: id = e*rows + r
   names logical row r of table e, and Y[i] = W_e[r] in fp32 (exact, as in
   decode_row).  The hash that produces the ids is the model's and is not
   part of this: ids are given.  An id outside [0, n_experts*rows) has no
   row; its output row is NaN so that the error shows. */
int vqo_gather(const vqo_tensor *T, int64_t n, const int64_t *ids, float *Y)
{
    if (!T || n < 0 || (n > 0 && (!ids || !Y)))
        return VQO_EBADARG;
    const int64_t total = (int64_t)T->n_experts * T->rows;
    int err = VQO_OK;

#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float *yr = Y + i * T->cols;
        const int64_t id = ids[i];
        if (id < 0 || id >= total) {
            for (int32_t c = 0; c < T->cols; ++c)
                yr[c] = NAN;
            continue;
        }
        int rc = decode_row(T, stored_row(T, (int32_t)(id / T->rows), (int32_t)(id % T->rows)),
                            yr);
        if (rc != VQO_OK) {
#pragma omp atomic write
            err = rc;
        }
    }
    return err;
}

/* ---------------------------------------------------------------------- */
/* Step 3: the matmul                                                      */
/* ---------------------------------------------------------------------- */

/* y = W x with W [out][in] (the subvector runs along the input dimension of
   one output row, as in "an fp16 scale per (row, 64 weights)").  Every sum
   is an fp64 loop over ascending columns. */
static void matvec_f64(const float *W, int32_t rows, int32_t cols,
                       const double *x, double *y)
{
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < rows; ++r) {
        const float *wr = W + (int64_t)r * cols;
        double acc = 0.0;
        for (int32_t c = 0; c < cols; ++c)
            acc += (double)wr[c] * x[c];
        y[r] = acc;
    }
}

int vqo_linear(const vqo_tensor *T, int32_t e, int32_t n_tok,
               const void *x, int32_t x_dtype, double *y)
{
    if (!T || n_tok < 0 || (n_tok > 0 && (!x || !y)))
        return VQO_EBADARG;
    if (x_dtype != VQO_X_F32 && x_dtype != VQO_X_BF16 && x_dtype != VQO_X_F64)
        return VQO_EBADARG;
    float *W = (float *)malloc(sizeof(float) * (size_t)T->rows * (size_t)T->cols + 1);
    double *xv = (double *)malloc(sizeof(double) * (size_t)T->cols + 1);
    if (!W || !xv) {
        free(W);
        free(xv);
        return VQO_ENOMEM;
    }
    int err = vqo_decode(T, e, W);
    for (int32_t n = 0; n < n_tok && err == VQO_OK; ++n) {
        for (int32_t c = 0; c < T->cols; ++c)
            xv[c] = x_value(x, x_dtype, (int64_t)n * T->cols + c);
        matvec_f64(W, T->rows, T->cols, xv, y + (int64_t)n * T->rows);
    }
    free(W);
    free(xv);
    return err;
}

/* ---------------------------------------------------------------------- */
/* Step 4: the routed SwiGLU expert FFN                                    */
/* ---------------------------------------------------------------------- */

/* SwiGLU: h = silu(gate) * up with silu(z) = z * sigmoid(z) = z / (1 + e^-z). */
double vqo_swiglu(double g, double u)
{
    return g / (1.0 + exp(-g)) * u;
}

/* Each token t is routed to top_k experts ids[t][0..k) with gate weights
   w[t][0..k) (the Qwen3.8-Flash-Next card: 10 of 512 experts; the gemma-4
   card: 128 experts, top-8).  Expert e applies gate, up and down projections
   of its own; the token's output is the gate-weighted sum over its slots,
   taken in slot order. */
int vqo_moe_ffn(const vqo_tensor *gate, const vqo_tensor *up, const vqo_tensor *down,
                int32_t n_tok, int32_t top_k, const void *x, int32_t x_dtype,
                const int32_t *ids, const float *w,
                int32_t n_sel, const int32_t *tokens, double *y)
{
    if (!gate || !up || !down || n_tok < 0 || top_k < 1 || n_sel < 0)
        return VQO_EBADARG;
    if (n_sel > 0 && (!x || !ids || !w || !tokens || !y))
        return VQO_EBADARG;
    if (x_dtype != VQO_X_F32 && x_dtype != VQO_X_BF16 && x_dtype != VQO_X_F64)
        return VQO_EBADARG;
    const int32_t hidden = gate->cols, inter = gate->rows;
    const int32_t E = gate->n_experts;
    if (up->cols != hidden || up->rows != inter || down->cols != inter ||
        down->rows != hidden || up->n_experts != E || down->n_experts != E)
        return VQO_EBADARG;
    for (int32_t i = 0; i < n_sel; ++i)
        if (tokens[i] < 0 || tokens[i] >= n_tok)
            return VQO_EBADARG;
    for (int32_t i = 0; i < n_sel; ++i)
        for (int32_t s = 0; s < top_k; ++s) {
            int32_t e = ids[(int64_t)tokens[i] * top_k + s];
            if (e < 0 || e >= E)
                return VQO_EBADARG;
        }

    const size_t nz = (size_t)n_sel * top_k * hidden;
    double *z = (double *)calloc(nz + 1, sizeof(double));
    float *Wg = (float *)malloc(sizeof(float) * (size_t)inter * hidden + 1);
    float *Wu = (float *)malloc(sizeof(float) * (size_t)inter * hidden + 1);
    float *Wd = (float *)malloc(sizeof(float) * (size_t)hidden * inter + 1);
    double *xv = (double *)malloc(sizeof(double) * (size_t)hidden + 1);
    double *g = (double *)malloc(sizeof(double) * (size_t)inter + 1);
    double *u = (double *)malloc(sizeof(double) * (size_t)inter + 1);
    double *h = (double *)malloc(sizeof(double) * (size_t)inter + 1);
    int err = (z && Wg && Wu && Wd && xv && g && u && h) ? VQO_OK : VQO_ENOMEM;

    /* Decode each expert once, then apply it to every selected (token, slot)
       routed to it; z[i][s] holds that slot's down-projection output. */
    for (int32_t e = 0; e < E && err == VQO_OK; ++e) {
        int used = 0;
        for (int32_t i = 0; i < n_sel && !used; ++i)
            for (int32_t s = 0; s < top_k; ++s)
                if (ids[(int64_t)tokens[i] * top_k + s] == e)
                    used = 1;
        if (!used)
            continue;
        err = vqo_decode(gate, e, Wg);
        if (err == VQO_OK)
            err = vqo_decode(up, e, Wu);
        if (err == VQO_OK)
            err = vqo_decode(down, e, Wd);
        for (int32_t i = 0; i < n_sel && err == VQO_OK; ++i) {
            int32_t t = tokens[i];
            for (int32_t s = 0; s < top_k; ++s) {
                if (ids[(int64_t)t * top_k + s] != e)
                    continue;
                for (int32_t c = 0; c < hidden; ++c)
                    xv[c] = x_value(x, x_dtype, (int64_t)t * hidden + c);
                matvec_f64(Wg, inter, hidden, xv, g);
                matvec_f64(Wu, inter, hidden, xv, u);
                for (int32_t r = 0; r < inter; ++r)
                    h[r] = vqo_swiglu(g[r], u[r]);
                matvec_f64(Wd, hidden, inter, h, z + ((size_t)i * top_k + s) * hidden);
            }
        }
    }
    /* y[t] = sum over slots, in slot order, of w[t][s] * z[t][s]. */
    for (int32_t i = 0; i < n_sel && err == VQO_OK; ++i) {
        int32_t t = tokens[i];
        for (int32_t c = 0; c < hidden; ++c) {
            double acc = 0.0;
            for (int32_t s = 0; s < top_k; ++s)
                acc += (double)w[(int64_t)t * top_k + s] * z[((size_t)i * top_k + s) * hidden + c];
            y[(int64_t)i * hidden + c] = acc;
        }
    }
    free(z);
    free(Wg);
    free(Wu);
    free(Wd);
    free(xv);
    free(g);
    free(u);
    free(h);
    return err;
}

/* ---------------------------------------------------------------------- */
/* Step 5: a stack of MoE layers                                           */
/* ---------------------------------------------------------------------- */

/* Layers in sequence, each applying its own routed FFN (step 4) to the
   running hidden state and adding the result to it:
       h <- h + FFN_l(h)   for l = 0, 1, ..., n_layers-1.
   The cards build models whose expert layers differ in geometry (promoted
   layers: "GLM-5.3-Flash-VQ-2.7bpw" and "Qwen3.8-Flash-Next-VQ-4.4bpw",
   opening summaries); a layer's FFN is computed exactly as in step 4, from
   the fp64 state.  The residual form is the standard place of an MoE block
   in a decoder layer (the cards do not describe the block); the attention,
   norms and router between the blocks are not modelled.  h: [n_tok][hidden]
   fp64, updated in place. */
int vqo_moe_stack(int32_t n_layers, const vqo_tensor *const *gate,
                  const vqo_tensor *const *up, const vqo_tensor *const *down,
                  int32_t n_tok, int32_t top_k, const int32_t *const *ids,
                  const float *const *w, double *h)
{
    if (n_layers < 0 || n_tok < 0 || (n_layers > 0 && (!gate || !up || !down || !ids || !w)))
        return VQO_EBADARG;
    if (n_layers == 0 || n_tok == 0)
        return VQO_OK;
    if (!h)
        return VQO_EBADARG;
    const int32_t hidden = gate[0]->cols;
    int32_t *tokens = (int32_t *)malloc(sizeof(int32_t) * (size_t)n_tok);
    double *y = (double *)malloc(sizeof(double) * (size_t)n_tok * hidden);
    int err = (tokens && y) ? VQO_OK : VQO_ENOMEM;
    for (int32_t t = 0; t < n_tok && tokens; ++t)
        tokens[t] = t;
    for (int32_t l = 0; l < n_layers && err == VQO_OK; ++l) {
        if (!gate[l] || gate[l]->cols != hidden) {
            err = VQO_EBADARG;
            break;
        }
        err = vqo_moe_ffn(gate[l], up[l], down[l], n_tok, top_k, h, VQO_X_F64, ids[l], w[l],
                          n_tok, tokens, y);
        for (int64_t i = 0; i < (int64_t)n_tok * hidden && err == VQO_OK; ++i)
            h[i] += y[i];
    }
    free(tokens);
    free(y);
    return err;
}

/* ---------------------------------------------------------------------- */
/* Step 0: fitting the format (the step before the path)                   */
/* ---------------------------------------------------------------------- */

/* The cards fit codebooks "data-free" by k-means / Lloyd over the weight
   subvectors, from a subsample drawn unseeded or with seed 1234, with an
   fp16 scale per (row, 64 weights) and the codes packed sub-byte
   ("Qwen3.5-397B-A17B-VQ-2.6bpw", "Methodology"; "Qwen3.5-397B-A17B-VQ-2.4bpw:
   Model Card", "Methodology"; "Qwen3.8-Flash-Next-VQ-4.4bpw" and
   "GLM-5.3-Flash-VQ-2.7bpw", "Methodology").  They do not say how a
   scale is chosen, how the fit is initialised or how many iterations run.
   The readings taken here:
     - scale s[r][g] = fp16 (round to nearest even) of max |w| over the
       group; a subvector is normalised as v_t = w_t / s in fp32 (IEEE
       division), and a group with s == 0 normalises to zeros;
     - the fit runs on a given set of subvector indices (the subsample) from
       K given initial subvectors (the seeded draw is an input) for a given
       number of Lloyd iterations;
     - distance = sum over t, in order, of (v_t - c_t)^2 in fp32 with every
       operation rounded (no fused multiply-add); ties go to the lower index;
     - a centroid is the mean of its members, summed exactly as integers in
       units of 2^-30 (each coordinate rounded to nearest even into that
       grid) and divided in fp64; a centroid with no members keeps its value;
     - the codebook is the centroids rounded to fp16, and every subvector of
       the tensor is then coded to its nearest fp16 entry (same distance).
   With these, a result is a function of its inputs alone, independent of
   the order in which members are visited. */

/* Built with -ffp-contract=off: every fp32 operation below rounds on its own. */

/* fp32 -> fp16 bits, round to nearest, ties to even (IEEE 754 conversion):
   scale |f| onto the 11-bit significand grid of its binade (the subnormal
   grid below 2^-14) in fp64, where the scaling is exact, and round there. */
uint16_t vqo_float_to_half(float f)
{
    if (isnan(f))
        return 0x7e00;
    const uint16_t sign = signbit(f) ? 0x8000 : 0;
    const double a = fabs((double)f);
    if (a >= 65520.0)            /* at or above the midpoint past 65504 */
        return sign | 0x7c00;
    int e;
    frexp(a, &e);                /* a in [2^(e-1), 2^e) */
    int ex = e - 1;
    if (ex < -14)
        ex = -14;                /* subnormal grid: 2^-24 */
    double q = nearbyint(ldexp(a, 10 - ex));
    if (q >= 2048.0) {           /* rounded up into the next binade */
        ex += 1;
        q = 1024.0;
    }
    if (q < 1024.0)              /* subnormal or zero */
        return sign | (uint16_t)q;
    return sign | (uint16_t)(((ex + 15) << 10) | ((int)q - 1024));
}

static float bf16_to_float(uint16_t h)
{
    return (float)vqo_bf16_to_double(h);   /* exact: bf16 is a prefix of fp32 */
}

int vqo_fit_scales(int64_t n_rows, int32_t cols, const uint16_t *w, uint16_t *scales)
{
    if (n_rows < 0 || cols <= 0 || cols % 64 || (n_rows > 0 && (!w || !scales)))
        return VQO_EBADARG;
    const int32_t groups = cols / 64;
    for (int64_t r = 0; r < n_rows; ++r)
        for (int32_t g = 0; g < groups; ++g) {
            float m = 0.0f;
            for (int32_t c = 0; c < 64; ++c) {
                float a = fabsf(bf16_to_float(w[r * cols + 64 * g + c]));
                if (a > m)
                    m = a;
            }
            scales[r * groups + g] = vqo_float_to_half(m);
        }
    return VQO_OK;
}

/* Normalised subvector i = r*(cols/d) + j of the tensor. */
static void subvector(const uint16_t *w, const uint16_t *scales, int32_t cols, int32_t d,
                      int64_t i, float *v)
{
    const int64_t n_sub = cols / d;
    const int64_t r = i / n_sub, j = i % n_sub;
    const float s = (float)vqo_half_to_double(scales[r * (cols / 64) + (j * d) / 64]);
    for (int32_t t = 0; t < d; ++t)
        v[t] = (s == 0.0f) ? 0.0f : bf16_to_float(w[r * cols + j * d + t]) / s;
}

static float dist2(const float *x, const float *c, int32_t d)
{
    float acc = 0.0f;
    for (int32_t t = 0; t < d; ++t) {
        const float diff = x[t] - c[t];
        const float sq = diff * diff;
        acc = acc + sq;
    }
    return acc;
}

static int32_t nearest(const float *x, const float *C, int32_t K, int32_t d)
{
    int32_t best = 0;
    float bd = dist2(x, C, d);
    for (int32_t k = 1; k < K; ++k) {
        const float dk = dist2(x, C + (int64_t)k * d, d);
        if (dk < bd) {
            bd = dk;
            best = k;
        }
    }
    return best;
}

#define VQO_FIT_MAX_SAMPLE (1 << 22)   /* keeps every integer sum below 2^53 */

int vqo_kmeans(int64_t n_rows, int32_t cols, int32_t d, int32_t K, const uint16_t *w,
               const uint16_t *scales, int64_t n_sample, const int64_t *sample,
               const int64_t *init, int32_t iters, float *C)
{
    const int64_t N = n_rows * (cols / (d > 0 ? d : 1));
    if (n_rows < 1 || cols <= 0 || cols % 64 || (d != 2 && d != 4 && d != 8) || K < 1 ||
        n_sample < 0 || n_sample > VQO_FIT_MAX_SAMPLE || iters < 0 || !w || !scales || !init ||
        !C || (n_sample > 0 && !sample))
        return VQO_EBADARG;
    for (int32_t k = 0; k < K; ++k)
        if (init[k] < 0 || init[k] >= N)
            return VQO_EBADARG;
    for (int64_t i = 0; i < n_sample; ++i)
        if (sample[i] < 0 || sample[i] >= N)
            return VQO_EBADARG;
    for (int32_t k = 0; k < K; ++k)
        subvector(w, scales, cols, d, init[k], C + (int64_t)k * d);

    int64_t *sum = (int64_t *)calloc((size_t)K * d + 1, sizeof(int64_t));
    int64_t *cnt = (int64_t *)calloc((size_t)K + 1, sizeof(int64_t));
    if (!sum || !cnt) {
        free(sum);
        free(cnt);
        return VQO_ENOMEM;
    }
    float v[8];
    for (int32_t it = 0; it < iters; ++it) {
        memset(sum, 0, sizeof(int64_t) * (size_t)K * d);
        memset(cnt, 0, sizeof(int64_t) * (size_t)K);
        for (int64_t i = 0; i < n_sample; ++i) {
            subvector(w, scales, cols, d, sample[i], v);
            const int32_t k = nearest(v, C, K, d);
            cnt[k] += 1;
            for (int32_t t = 0; t < d; ++t)
                sum[(int64_t)k * d + t] += llrint(ldexp((double)v[t], 30));
        }
        for (int32_t k = 0; k < K; ++k) {
            if (cnt[k] == 0)
                continue;
            for (int32_t t = 0; t < d; ++t)
                C[(int64_t)k * d + t] =
                    (float)ldexp((double)sum[(int64_t)k * d + t] / (double)cnt[k], -30);
        }
    }
    free(sum);
    free(cnt);
    return VQO_OK;
}

int vqo_encode(int64_t n_rows, int32_t cols, int32_t d, int32_t bits, int32_t K,
               const uint16_t *w, const uint16_t *scales, const uint16_t *codebook,
               uint32_t *codes)
{
    if (n_rows < 0 || cols <= 0 || cols % 64 || (d != 2 && d != 4 && d != 8) || K < 1 ||
        bits < 1 || bits > 16 || (int64_t)K > ((int64_t)1 << bits) ||
        (n_rows > 0 && (!w || !scales || !codebook || !codes)))
        return VQO_EBADARG;
    float *C = (float *)malloc(sizeof(float) * (size_t)K * d);
    if (!C)
        return VQO_ENOMEM;
    for (int64_t i = 0; i < (int64_t)K * d; ++i)
        C[i] = (float)vqo_half_to_double(codebook[i]);
    const int64_t n_sub = cols / d, wpr = vqo_words_per_row(cols, d, bits);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_rows; ++r) {
        uint32_t *row = codes + r * wpr;
        float v[8];
        for (int64_t q = 0; q < wpr; ++q)
            row[q] = 0;
        /* code j occupies stream bits [j*bits, j*bits + bits), LSB first */
        for (int64_t j = 0; j < n_sub; ++j) {
            subvector(w, scales, cols, d, r * n_sub + j, v);
            const uint32_t code = (uint32_t)nearest(v, C, K, d);
            for (int32_t b = 0; b < bits; ++b)
                if ((code >> b) & 1u) {
                    const int64_t q = j * bits + b;
                    row[q / 32] |= 1u << (q % 32);
                }
        }
    }
    free(C);
    return VQO_OK;
}

int vqo_fit(int64_t n_rows, int32_t cols, int32_t d, int32_t bits, int32_t K, const uint16_t *w,
            int64_t n_sample, const int64_t *sample, const int64_t *init, int32_t iters,
            uint16_t *codebook, uint16_t *scales, uint32_t *codes)
{
    if (!codebook || (int64_t)K > ((int64_t)1 << (bits > 0 && bits < 31 ? bits : 0)))
        return VQO_EBADARG;
    int err = vqo_fit_scales(n_rows, cols, w, scales);
    if (err != VQO_OK)
        return err;
    float *C = (float *)malloc(sizeof(float) * (size_t)(K > 0 ? K : 1) * 8);
    if (!C)
        return VQO_ENOMEM;
    err = vqo_kmeans(n_rows, cols, d, K, w, scales, n_sample, sample, init, iters, C);
    if (err == VQO_OK) {
        for (int64_t i = 0; i < (int64_t)K * d; ++i)
            codebook[i] = vqo_float_to_half(C[i]);
        err = vqo_encode(n_rows, cols, d, bits, K, w, scales, codebook, codes);
    }
    free(C);
    return err;
}
