/*
 * q8o.h -- CPU oracle for the Q8_0 quantized matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  This header and q8o.c are a plain, slow
 * restatement of what the GPU path computes (optionally on several OpenMP
 * threads over independent outputs).  Only the tests,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or helper with the HIP library.
 *
 * Sources (ds4-learning pages):
 *   - "Part 3: 模型架构", section 2 (量化与矩阵运算), the Q8_K row quantizer
 *     snippet: per block amax = max|x|, scale = amax/127, q = (int8)roundf(x/scale).
 *   - "Part 6: 代码走读", trace 3 (GPU matmul 与 matvec): Q8_0 weights times
 *     Q8_0 activations, in_dim must be a multiple of 32 (the Q8_0 block size).
 *   - "Part 3: 模型架构", section 2, item 4 (矩阵-向量乘法): y = x @ W.
 *   - "Part 6: 代码走读", trace 5 (GPU MoE): each token's selected expert list
 *     drives one matmul per (token, expert slot).
 *
 * Block format (one Q8_0 block = 32 values, 34 bytes):
 *   bytes 0..1  binary16 scale d, little-endian
 *   bytes 2..33 int8 quants q[0..31]
 * A matrix of shape [rows][k] is rows*(k/32) consecutive blocks, row-major.
 */
#ifndef Q8O_H
#define Q8O_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* OpenMP threads for the loops over independent outputs (default 1).  The
 * results do not depend on it: every output is computed by the same code in
 * the same order. */
void q8o_set_threads(int n);
int q8o_get_threads(void);

/* IEEE 754 binary16 conversions, written from the format definition. */
uint16_t q8o_f16_from_f32(float f);   /* round to nearest, ties to even */
double q8o_f16_to_f64(uint16_t h);    /* exact */

/* Quantize x[n_rows][k] (fp32) into n_rows*(k/32) Q8_0 blocks.
 * Returns 0, or -1 if k is not a multiple of 32 or a size is negative. */
int q8o_quantize(const float *x, int64_t n_rows, int64_t k, uint8_t *blocks);

/* out[t][o] = sum_b f16(d_w[o][b]) * f16(d_x[t][b]) * S_b[t][o], where
 * S_b = sum_i qw[o][b][i] * qx[t][b][i] is an exact integer.  Terms and the
 * sum are formed in double, ascending b; out is the double rounded to fp32.
 * mag[t][o] (optional) = sum_b |term_b|; blocksums[t][o][b] (optional) = S_b.
 * Returns 0, or -1 on a bad size. */
int q8o_matmul(const uint8_t *w, int64_t in_dim, int64_t out_dim,
               const uint8_t *xq, int64_t n_tok,
               float *out, double *mag, int32_t *blocksums);

/* Grouped expert matmul: for each token t and slot j, e = selected[t][j] and
 * out[t][j][:] = matmul(expert_w[e], x row), where the x row is xq row t
 * (x_rows == 0) or xq row t*n_used + j (x_rows == 1).  A pair whose expert id
 * lies outside [0, n_expert) gets a row of NaN.  Returns the number of such
 * pairs (>= 0), or -1 on a bad size. */
int q8o_moe_grouped(const uint8_t *const *expert_w, int32_t n_expert,
                    int64_t in_dim, int64_t out_dim,
                    const int32_t *selected, int32_t n_used,
                    const uint8_t *xq, int32_t x_rows, int64_t n_tok,
                    float *out, double *mag);

/* Expert FFN activation, SwiGLU ("Part 3: 模型架构", section 4, SwiGLU
 * activation): for each i, g = gate[i] and u = up[i]; when clamp > 0 the
 * 2-bit path's limits apply first (g > clamp -> clamp; u > clamp -> clamp;
 * u < -clamp -> -clamp; NaN passes through); then
 * mid[i] = silu(g) * u with silu(g) = g * sigmoid(g) = g / (1 + exp(-g)),
 * evaluated in double and rounded once to fp32.  clamp <= 0: no clamp. */
void q8o_swiglu(const float *gate, const float *up, int64_t n, float clamp, float *mid);

/* Weighted combine of the experts' outputs ("Part 6: 代码走读", trace 5, the
 * routed MoE's last step): out[t][o] = sum over j = 0..n_used-1 of
 * weights[t][j] * y[t][j][o], in double in ascending j, rounded once to fp32;
 * mag[t][o] (optional) = sum_j |weights[t][j] * y[t][j][o]|. */
void q8o_moe_combine(const float *y, const float *weights, int64_t n_tok, int32_t n_used,
                     int64_t dim, float *out, double *mag);

#ifdef __cplusplus
}
#endif

#endif /* Q8O_H */
