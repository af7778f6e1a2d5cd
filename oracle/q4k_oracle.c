/*
 * Q4_K CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow, obviously correct statement of what the Q4_K
 * dequantize-and-multiply path computes.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load it.  The product library never
 * links, loads or calls it, and shares no source with it.
 *
 * What is computed, and where it comes from:
 *  - "Struct WgslForwardPass" (trueno docs), method upload_q4k_weight: weights
 *    are kept as raw Q4K bytes and multiplied by a fused dequant+GEMV.
 *  - "qualia_core_db/inference/cuda_lane/mod.rs", module docs, "Honest limits":
 *    the fallback to a fused kernel is to dequantize once to dense f32; this
 *    oracle is exactly that fallback, with the dot product accumulated in f64.
 *  - "@simulatte/doppler 0.1.7 -> 0.1.8", matmul.d.ts, MatmulOptions.transposeB:
 *    the weight matrix B is stored [N,K], row n holding its K weights.
 *  - The Q4_K super-block layout is not printed on the pages; the model files
 *    they use are Q4_K_M GGUF files (issue #3346, measured 0.8B inventory) and
 *    the missing kernel is called llama.cpp-class (cuda_lane module docs).  The
 *    layout used is therefore the public GGUF k-quant Q4_K block:
 *        bytes 0-1    d      IEEE binary16, little-endian
 *        bytes 2-3    dmin   IEEE binary16, little-endian
 *        bytes 4-15   scales 8 six-bit scales sc_j and 8 six-bit mins m_j
 *        bytes 16-143 qs     256 four-bit codes
 *    sub-block j (32 weights, j = 0..7) uses scale d*sc_j and min dmin*m_j.
 *
 * Precision (fixed by the method's statement of the oracle): f16 -> f32 exact,
 * dl = d*sc and ml = dmin*m in f32, w = f32(f32(dl*q) - ml) with no fused
 * multiply-add, then y = sum_k (double)w * (double)x in f64 in k order.
 * Build with -ffp-contract=off so no step is fused.
 *
 * Every row-range function works on rows [r0, r1) of a matrix with `k`
 * columns (k % 256 == 0), whose row n starts at byte n * (k/256) * 144.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define Q4K_BLOCK_BYTES 144
#define Q4K_BLOCK_WEIGHTS 256

/* IEEE 754 binary16 -> binary32, written from the format definition:
 * sign bit, 5-bit exponent with bias 15, 10-bit fraction; exponent 0 is
 * zero/subnormal (fraction * 2^-24), exponent 31 is infinity/NaN. */
float q4k_oracle_f16_to_f32(uint16_t h) {
    const int sign = (h >> 15) & 1;
    const int exponent = (h >> 10) & 0x1f;
    const int fraction = h & 0x3ff;
    double v;
    if (exponent == 0) {
        v = ldexp((double)fraction, -24);
    } else if (exponent == 31) {
        v = fraction ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + fraction), exponent - 25);
    }
    return (float)(sign ? -v : v);
}

/* Six-bit scale and min of sub-block j (0..7) from the 12 packed bytes.
 * Sub-blocks 0-3 keep their values in the low six bits of bytes j (scale) and
 * j+4 (min).  Sub-blocks 4-7 take their low four bits from byte j+4 (scale in
 * the low nibble, min in the high nibble) and their top two bits from the
 * spare top bits of bytes j-4 (scale) and j (min). */
void q4k_oracle_scale_min(const uint8_t *scales, int j, int *sc, int *m) {
    if (j < 4) {
        *sc = scales[j] & 63;
        *m = scales[j + 4] & 63;
    } else {
        *sc = (scales[j + 4] & 15) | ((scales[j - 4] >> 6) << 4);
        *m = (scales[j + 4] >> 4) | ((scales[j] >> 6) << 4);
    }
}

/* Four-bit code of weight e (0..255) of a block: the 128 code bytes form four
 * groups of 32; weight 64g+l is the low nibble of byte 32g+l and weight
 * 64g+32+l is the high nibble of the same byte. */
static int q4k_oracle_code(const uint8_t *qs, int e) {
    const int g = e / 64;
    const int r = e % 64;
    const uint8_t byte = qs[32 * g + (r % 32)];
    return r < 32 ? (byte & 15) : (byte >> 4);
}

/* Dequantize one 144-byte super-block into 256 f32 weights. */
void q4k_oracle_dequant_block(const uint8_t *blk, float *out) {
    const float d = q4k_oracle_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
    const float dmin = q4k_oracle_f16_to_f32((uint16_t)(blk[2] | (blk[3] << 8)));
    const uint8_t *scales = blk + 4;
    const uint8_t *qs = blk + 16;
    for (int e = 0; e < Q4K_BLOCK_WEIGHTS; ++e) {
        const int j = e / 32; /* sub-block */
        int sc, m;
        q4k_oracle_scale_min(scales, j, &sc, &m);
        const float dl = d * (float)sc;
        const float ml = dmin * (float)m;
        const float t = dl * (float)q4k_oracle_code(qs, e);
        out[e] = t - ml;
    }
}

/* W[r, :] as f32 for rows [r0, r1); out is [(r1-r0), k] row-major. */
void q4k_oracle_dequant_rows(const uint8_t *w, int64_t k, int64_t r0, int64_t r1, float *out) {
    const int64_t nb = k / Q4K_BLOCK_WEIGHTS;
    for (int64_t r = r0; r < r1; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            q4k_oracle_dequant_block(w + (r * nb + b) * Q4K_BLOCK_BYTES,
                                     out + (r - r0) * k + b * Q4K_BLOCK_WEIGHTS);
        }
    }
}

/* One row's dot product with x, in f64, k order; also sum_k |w x|. */
static void q4k_oracle_row_dot(const uint8_t *row, int64_t k, const float *x, double *y, double *a) {
    const int64_t nb = k / Q4K_BLOCK_WEIGHTS;
    float wblk[Q4K_BLOCK_WEIGHTS];
    double acc = 0.0, mag = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
        q4k_oracle_dequant_block(row + b * Q4K_BLOCK_BYTES, wblk);
        for (int e = 0; e < Q4K_BLOCK_WEIGHTS; ++e) {
            const double p = (double)wblk[e] * (double)x[b * Q4K_BLOCK_WEIGHTS + e];
            acc += p;
            mag += fabs(p);
        }
    }
    *y = acc;
    *a = mag;
}

/* GEMV, rows [r0, r1): y[r-r0] = sum_k W[r,k] x[k]; a[r-r0] = sum_k |W[r,k] x[k]|. */
void q4k_gemv_oracle_into(const uint8_t *w, const float *x, int64_t k, int64_t r0, int64_t r1,
                          double *y, double *a) {
    const int64_t row_bytes = (k / Q4K_BLOCK_WEIGHTS) * Q4K_BLOCK_BYTES;
    for (int64_t r = r0; r < r1; ++r) {
        q4k_oracle_row_dot(w + r * row_bytes, k, x, &y[r - r0], &a[r - r0]);
    }
}

/* Batched: X is [m, k] row-major (one activation row per token); Y and A are
 * [m, r1-r0] row-major: Y[t, r-r0] = sum_k W[r,k] X[t,k]. */
void q4k_gemv_batched_oracle_into(const uint8_t *w, const float *xs, int64_t m, int64_t k,
                                  int64_t r0, int64_t r1, double *y, double *a) {
    const int64_t row_bytes = (k / Q4K_BLOCK_WEIGHTS) * Q4K_BLOCK_BYTES;
    const int64_t nr = r1 - r0;
    for (int64_t t = 0; t < m; ++t) {
        for (int64_t r = r0; r < r1; ++r) {
            q4k_oracle_row_dot(w + r * row_bytes, k, xs + t * k, &y[t * nr + (r - r0)],
                               &a[t * nr + (r - r0)]);
        }
    }
}

/* SwiGLU over two Q4_K matrices of the same shape ("Struct WgslForwardPass",
 * silu_mul_shader; cuda_lane exports try_q4k_soa_fused_swiglu):
 * g = Wg x, u = Wu x, h = silu(g) * u with silu(t) = t / (1 + exp(-t)), all f64.
 * Also returns g, u and their magnitude sums for the error bound. */
void q4k_fused_swiglu_oracle_into(const uint8_t *wg, const uint8_t *wu, const float *x, int64_t k,
                                  int64_t r0, int64_t r1, double *h, double *g, double *u,
                                  double *ag, double *au) {
    const int64_t row_bytes = (k / Q4K_BLOCK_WEIGHTS) * Q4K_BLOCK_BYTES;
    for (int64_t r = r0; r < r1; ++r) {
        const int64_t i = r - r0;
        q4k_oracle_row_dot(wg + r * row_bytes, k, x, &g[i], &ag[i]);
        q4k_oracle_row_dot(wu + r * row_bytes, k, x, &u[i], &au[i]);
        h[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
    }
}

/* GEMV with a residual added ("qualia_core_db/inference/cuda_lane/mod.rs"
 * exports try_q4k_soa_ffn_block_residual: the down projection whose result is
 * added to the residual stream), rows [r0, r1):
 * y[r-r0] = sum_k W[r,k] x[k] + res[r], the sum in f64 and then the residual
 * added in f64; a[r-r0] = sum_k |W[r,k] x[k]| + |res[r]|. */
void q4k_gemv_residual_oracle_into(const uint8_t *w, const float *x, const float *res, int64_t k, int64_t r0,
                                   int64_t r1, double *y, double *a) {
    const int64_t row_bytes = (k / Q4K_BLOCK_WEIGHTS) * Q4K_BLOCK_BYTES;
    for (int64_t r = r0; r < r1; ++r) {
        double dot, mag;
        q4k_oracle_row_dot(w + r * row_bytes, k, x, &dot, &mag);
        y[r - r0] = dot + (double)res[r];
        a[r - r0] = mag + fabs((double)res[r]);
    }
}

/* ------------------------------------------------------------------ Q8_0
 * The second block format of the decode path ("qualia_core_db/inference/
 * cuda_lane/mod.rs" re-exports q8_0_gemv_oracle_into, try_q8_0_cuda_gemv,
 * Q8_0_BLOCK_BYTES and Q8_0_BLOCK_ELEMS from its q8 module).  The block layout
 * is not printed on the pages; as for Q4_K the public GGUF block is used:
 *     bytes 0-1    d   IEEE binary16, little-endian
 *     bytes 2-33   q   32 signed bytes (two's complement)
 * and weight e of the block is f32(d) * q[e] (exact in f32: 11 x 8 bits).
 * A row of k weights (k % 32 == 0) is k/32 consecutive blocks. */
#define Q8_0_BLOCK_BYTES 34
#define Q8_0_BLOCK_WEIGHTS 32

/* Dequantize one 34-byte block into 32 f32 weights. */
void q8_0_oracle_dequant_block(const uint8_t *blk, float *out) {
    const float d = q4k_oracle_f16_to_f32((uint16_t)((blk[1] << 8) | blk[0]));
    for (int e = 0; e < Q8_0_BLOCK_WEIGHTS; ++e) {
        const int q = (int)(int8_t)blk[2 + e];
        out[e] = d * (float)q;
    }
}

/* W[r, :] as f32 for rows [r0, r1); out is [(r1-r0), k] row-major. */
void q8_0_oracle_dequant_rows(const uint8_t *w, int64_t k, int64_t r0, int64_t r1, float *out) {
    const int64_t nb = k / Q8_0_BLOCK_WEIGHTS;
    const int64_t row_bytes = nb * Q8_0_BLOCK_BYTES;
    for (int64_t r = r0; r < r1; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            q8_0_oracle_dequant_block(w + r * row_bytes + b * Q8_0_BLOCK_BYTES,
                                      out + (r - r0) * k + b * Q8_0_BLOCK_WEIGHTS);
        }
    }
}

/* GEMV, rows [r0, r1): y[r-r0] = sum_k W[r,k] x[k] in f64, k order;
 * a[r-r0] = sum_k |W[r,k] x[k]|. */
void q8_0_gemv_oracle_into(const uint8_t *w, const float *x, int64_t k, int64_t r0, int64_t r1, double *y,
                           double *a) {
    const int64_t nb = k / Q8_0_BLOCK_WEIGHTS;
    const int64_t row_bytes = nb * Q8_0_BLOCK_BYTES;
    float wblk[Q8_0_BLOCK_WEIGHTS];
    for (int64_t r = r0; r < r1; ++r) {
        double acc = 0.0, mag = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            q8_0_oracle_dequant_block(w + r * row_bytes + b * Q8_0_BLOCK_BYTES, wblk);
            for (int e = 0; e < Q8_0_BLOCK_WEIGHTS; ++e) {
                const double p = (double)wblk[e] * (double)x[b * Q8_0_BLOCK_WEIGHTS + e];
                acc += p;
                mag += p < 0.0 ? -p : p;
            }
        }
        y[r - r0] = acc;
        a[r - r0] = mag;
    }
}
