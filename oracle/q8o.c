/*
 * q8o.c -- CPU oracle for the Q8_0 quantized matmul.
 *
 * TEST INFRASTRUCTURE ONLY: a plain, slow, obviously correct restatement of
 * the method, used by the tests, the smoke check and the benchmark's CPU
 * baseline.  Nothing here is shared with the GPU library.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -fopenmp -fPIC
 * -shared (no fast-math, no FMA contraction: every float operation is the
 * IEEE one that the source code spells out).
 *
 * Threads: q8o_set_threads(n) lets the loops over independent outputs (rows
 * of the quantizer, (token, output) pairs of the matmul, (token, slot) pairs
 * of the grouped call) run on n OpenMP threads with a static partition.  Each
 * output is computed by exactly the same code in the same order whatever the
 * thread count, so results are bit-identical to the single-threaded run
 * (tested).  The default is one thread.
 *
 * Readings of the pages taken here (the pages show a Q8_K snippet only; see
 * "Part 3: 模型架构", section 2, the ds4_quantize_row_q8_K listing):
 *   - The same amax/127 + roundf rule is applied per 32-value block, and the
 *     scale is stored as binary16 (Q8_0 instead of Q8_K's 256-value block and
 *     fp32 scale).
 *   - q is computed by fp32 IEEE division of x by the fp32 scale d32, then C
 *     roundf (halves away from zero); the stored scale is binary16(d32),
 *     rounded to nearest even.
 *   - A block whose amax is 0, or whose fp32 scale d32 underflows to 0, is a
 *     zero block: scale bits 0x0000, all q = 0 (the snippet would divide by 0).
 *   - q is clamped to [-127, 127].  For a normal d32 the quotient never leaves
 *     [-127, 127] after rounding, so the clamp only acts when d32 is an fp32
 *     subnormal that lost precision.
 *   - A block holding a NaN or an infinity, or whose d32 is too large for
 *     binary16 (d32 >= 65520), is marked: scale bits 0x7E00 (a NaN), all
 *     q = 0.  Every output that uses such a block is NaN.
 * Parity of this file is pinned by tests/test_oracle_*.py against closed
 * forms, library conversions, brute force and invariants.
 */
#include "q8o.h"

#include <math.h>
#include <string.h>

#define QK 32          /* values per Q8_0 block */
#define BLOCK_BYTES 34 /* 2-byte binary16 scale + 32 int8 quants */

static int g_threads = 1;

void q8o_set_threads(int n) { g_threads = n < 1 ? 1 : n; }
int q8o_get_threads(void) { return g_threads; }

/* ---- binary16 ---------------------------------------------------------- */

double q8o_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0x1F) {
        v = m ? NAN : INFINITY;
    } else if (e == 0) {
        v = ldexp((double)m, -24);              /* subnormal: m units of 2^-24 */
    } else {
        v = ldexp((double)(1024 + m), e - 25);  /* (1 + m/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

uint16_t q8o_f16_from_f32(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(f)) return (uint16_t)(sign | 0x7E00u);
    if (isinf(f)) return (uint16_t)(sign | 0x7C00u);
    double a = fabs((double)f);
    if (a == 0.0) return sign;

    /* a lies in [2^e, 2^(e+1)).  Within that binade binary16 values are spaced
     * by 2^(max(e, -14) - 10); below 2^-14 the spacing stays 2^-24. */
    int e;
    frexp(a, &e);
    e -= 1;
    int ulp_exp = (e < -14 ? -14 : e) - 10;
    double n = ldexp(a, -ulp_exp);  /* a in units of that spacing; exact */
    double fl = floor(n);
    double frac = n - fl;
    double r = fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) r = fl + 1.0;
    double v = ldexp(r, ulp_exp);   /* rounded magnitude */

    if (v >= 65536.0) return (uint16_t)(sign | 0x7C00u);     /* overflow */
    if (v < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)r); /* subnormal */
    frexp(v, &e);
    e -= 1;
    uint16_t mant = (uint16_t)(ldexp(v, -e) * 1024.0 - 1024.0);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | mant);
}

/* ---- quantizer --------------------------------------------------------- */

static void quantize_block(const float *v, uint8_t *blk) {
    int finite = 1;
    float amax = 0.0f;
    for (int i = 0; i < QK; i++) {
        if (!isfinite(v[i])) {
            finite = 0;
        } else if (fabsf(v[i]) > amax) {
            amax = fabsf(v[i]);
        }
    }

    uint16_t dh = 0;
    int8_t q[QK];
    memset(q, 0, sizeof q);

    if (!finite) {
        dh = 0x7E00;
    } else if (amax > 0.0f) {
        float d = amax / 127.0f;
        if (d > 0.0f) {
            dh = q8o_f16_from_f32(d);
            if ((dh & 0x7FFFu) == 0x7C00u) {
                dh = 0x7E00;  /* scale does not fit binary16 */
            } else {
                for (int i = 0; i < QK; i++) {
                    float r = v[i] / d;
                    float qr = roundf(r);
                    if (qr > 127.0f) qr = 127.0f;
                    if (qr < -127.0f) qr = -127.0f;
                    q[i] = (int8_t)qr;
                }
            }
        }
    }

    blk[0] = (uint8_t)(dh & 0xFF);
    blk[1] = (uint8_t)(dh >> 8);
    memcpy(blk + 2, q, QK);
}

int q8o_quantize(const float *x, int64_t n_rows, int64_t k, uint8_t *blocks) {
    if (n_rows < 0 || k < 0 || k % QK != 0) return -1;
    int64_t nb = k / QK;
    #pragma omp parallel for collapse(2) schedule(static) num_threads(g_threads)
    for (int64_t t = 0; t < n_rows; t++) {
        for (int64_t b = 0; b < nb; b++) {
            quantize_block(x + t * k + b * QK, blocks + (t * nb + b) * BLOCK_BYTES);
        }
    }
    return 0;
}

/* ---- matmul ------------------------------------------------------------ */

static uint16_t block_scale_bits(const uint8_t *blk) {
    return (uint16_t)(blk[0] | ((uint16_t)blk[1] << 8));
}

int q8o_matmul(const uint8_t *w, int64_t in_dim, int64_t out_dim,
               const uint8_t *xq, int64_t n_tok,
               float *out, double *mag, int32_t *blocksums) {
    if (in_dim < 0 || out_dim < 0 || n_tok < 0 || in_dim % QK != 0) return -1;
    int64_t nb = in_dim / QK;
    #pragma omp parallel for collapse(2) schedule(static) num_threads(g_threads)
    for (int64_t t = 0; t < n_tok; t++) {
        for (int64_t o = 0; o < out_dim; o++) {
            double acc = 0.0;
            double m = 0.0;
            for (int64_t b = 0; b < nb; b++) {
                const uint8_t *wb = w + (o * nb + b) * BLOCK_BYTES;
                const uint8_t *xb = xq + (t * nb + b) * BLOCK_BYTES;
                int32_t s = 0;
                for (int i = 0; i < QK; i++) {
                    s += (int32_t)(int8_t)wb[2 + i] * (int32_t)(int8_t)xb[2 + i];
                }
                /* 11-bit x 11-bit x 20-bit significands: exact in double */
                double term = q8o_f16_to_f64(block_scale_bits(wb)) *
                              q8o_f16_to_f64(block_scale_bits(xb)) * (double)s;
                acc += term;
                m += fabs(term);
                if (blocksums) blocksums[(t * out_dim + o) * nb + b] = s;
            }
            out[t * out_dim + o] = (float)acc;
            if (mag) mag[t * out_dim + o] = m;
        }
    }
    return 0;
}

/* ---- grouped experts --------------------------------------------------- */

int q8o_moe_grouped(const uint8_t *const *expert_w, int32_t n_expert,
                    int64_t in_dim, int64_t out_dim,
                    const int32_t *selected, int32_t n_used,
                    const uint8_t *xq, int32_t x_rows, int64_t n_tok,
                    float *out, double *mag) {
    if (n_expert < 1 || n_used < 1 || n_tok < 0 || in_dim < 0 || out_dim < 0 ||
        in_dim % QK != 0 || (x_rows != 0 && x_rows != 1)) {
        return -1;
    }
    int64_t row_bytes = (in_dim / QK) * BLOCK_BYTES;
    int invalid = 0;
    /* Pairs are independent; the matmul inside runs single-threaded there
     * (nested parallel regions get one thread). */
    #pragma omp parallel for collapse(2) schedule(static) num_threads(g_threads) reduction(+:invalid)
    for (int64_t t = 0; t < n_tok; t++) {
        for (int32_t j = 0; j < n_used; j++) {
            int64_t pair = t * n_used + j;
            int32_t e = selected[pair];
            float *orow = out + pair * out_dim;
            double *mrow = mag ? mag + pair * out_dim : NULL;
            if (e < 0 || e >= n_expert) {
                for (int64_t o = 0; o < out_dim; o++) {
                    orow[o] = NAN;
                    if (mrow) mrow[o] = NAN;
                }
                invalid++;
                continue;
            }
            const uint8_t *xrow = xq + (x_rows == 0 ? t : pair) * row_bytes;
            q8o_matmul(expert_w[e], in_dim, out_dim, xrow, 1, orow, mrow, NULL);
        }
    }
    return invalid;
}

void q8o_swiglu(const float *gate, const float *up, int64_t n, float clamp, float *mid) {
  for (int64_t i = 0; i < n; ++i) {
    float g = gate[i], u = up[i];
    if (clamp > 0.0f) {
      if (g > clamp) g = clamp;
      if (u > clamp) u = clamp;
      if (u < -clamp) u = -clamp;
    }
    const double gd = (double)g;
    const double silu = gd / (1.0 + exp(-gd));
    mid[i] = (float)(silu * (double)u);
  }
}

void q8o_moe_combine(const float *y, const float *weights, int64_t n_tok, int32_t n_used,
                     int64_t dim, float *out, double *mag) {
  for (int64_t t = 0; t < n_tok; ++t) {
    for (int64_t o = 0; o < dim; ++o) {
      double acc = 0.0, m = 0.0;
      for (int32_t j = 0; j < n_used; ++j) {
        const double term = (double)weights[t * n_used + j] * (double)y[(t * n_used + j) * dim + o];
        acc += term;
        m += fabs(term);
      }
      out[t * dim + o] = (float)acc;
      if (mag) mag[t * dim + o] = m;
    }
  }
}
