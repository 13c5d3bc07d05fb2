/*
 * kvc_delta.c - plain CPU reference of token-delta ("change-based") coding
 * with anchors: the step before quantization in the CacheGen write-up
 * ([CG] 1.2 point 1: neighbouring tokens' K/V are close, so differences
 * rather than raw values are coded, which lowers their spread; [CG] 2.3
 * step 1 names the anchor-based form, which the walked-through code skips).
 *
 * TEST INFRASTRUCTURE ONLY, like kvc_oracle.c.  Parity unpinned by the
 * pages (they print no formula); the readings below are this build's.
 *
 * Readings (the pages leave every detail open):
 *   - anchors are the tokens at chunk-relative positions 0, G, 2G, ...
 *     (G = anchor_tokens >= 1), so every chunk still stands alone;
 *   - token t of a chunk starting at t0 has anchor a = t0 + G*floor((t-t0)/G);
 *   - the reference is the anchor's own reconstruction xa_hat: the codec's
 *     quantization of the anchor row (layer's bins) dequantized to fp16, the
 *     values a decoder holds, so an anchor's error does not carry into its
 *     tokens;
 *   - forward: an anchor row is kept; any other row becomes
 *       d = fp16(sat(fp32(x) - fp32(xa_hat)))  (fp32 subtraction, then fp16)
 *     and the delta tensor goes through the unchanged codec;
 *   - inverse, on the decoded fp16 tensor y (whose anchor rows are xa_hat):
 *       x_hat = fp16(sat(fp32(y) + fp32(y_anchor))) for every non-anchor row;
 *   - sat() clamps to [-65504, 65504], the finite fp16 range: a delta of two
 *     finite fp16 values can reach twice that, and a clamped delta is a
 *     coding error like any other (the inverse then lands at most
 *     |delta| - 65504 away); only a non-finite input is an error.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "kvc_oracle.h"

static float sat(float v) { return v > 65504.0f ? 65504.0f : (v < -65504.0f ? -65504.0f : v); }

static int64_t anchor_of(int64_t t, int32_t Tc, int32_t G)
{
    int64_t t0 = (t / Tc) * Tc;
    return t0 + ((t - t0) / G) * G;
}

/* The codec's reconstruction of one row x [C] at bins nb, through the
 * oracle's own quantizer and dequantizer (a one-layer, one-token tensor). */
static int reconstruct_row(const uint16_t *x, int32_t C, int32_t nb, uint16_t *xhat)
{
    uint16_t *kv = calloc((size_t)2 * C, sizeof(uint16_t));
    uint8_t *sym = malloc((size_t)2 * C);
    uint16_t max1[2];
    uint16_t *y = malloc((size_t)2 * C * sizeof(uint16_t));
    int32_t bins[2] = {nb, nb};
    int rc = ORC_ERR_ARG;
    if (kv && sym && y) {
        memcpy(kv, x, (size_t)C * sizeof(uint16_t)); /* the K slot; V stays zero */
        rc = orc_quantize(1, C, 1, bins, kv, sym, max1);
        if (rc == ORC_OK) rc = orc_dequantize(1, C, 1, bins, sym, max1, y, 0);
        if (rc == ORC_OK) memcpy(xhat, y, (size_t)C * sizeof(uint16_t));
    }
    free(kv);
    free(sym);
    free(y);
    return rc;
}

int orc_delta_forward(int32_t L, int32_t C, int64_t T, int32_t Tc, int32_t G, const int32_t *bins,
                      const uint16_t *kv, uint16_t *out)
{
    if (L < 1 || C < 1 || T < 0 || Tc < 1 || G < 1 || !bins) return ORC_ERR_ARG;
    uint16_t *xa = malloc((size_t)C * sizeof(uint16_t));
    if (!xa) return ORC_ERR_ARG;
    int rc = ORC_OK;
    for (int32_t l = 0; l < L && rc == ORC_OK; ++l) {
        for (int kvi = 0; kvi < 2 && rc == ORC_OK; ++kvi) {
            const int64_t base = ((int64_t)l * 2 + kvi) * T;
            for (int64_t t = 0; t < T; ++t) {
                const int64_t a = anchor_of(t, Tc, G);
                const uint16_t *x = kv + (base + t) * C;
                uint16_t *d = out + (base + t) * C;
                if (t == a) {
                    rc = reconstruct_row(x, C, bins[l * 2 + kvi], xa);
                    if (rc != ORC_OK) break;
                    memcpy(d, x, (size_t)C * sizeof(uint16_t));
                    continue;
                }
                for (int32_t c = 0; c < C; ++c) {
                    const float xv = orc_half_to_float(x[c]);
                    if (!isfinite(xv)) {
                        rc = ORC_ERR_NONFINITE;
                        break;
                    }
                    d[c] = orc_float_to_half(sat(xv - orc_half_to_float(xa[c])));
                }
                if (rc != ORC_OK) break;
            }
        }
    }
    free(xa);
    return rc;
}

int orc_delta_inverse(int32_t L, int32_t C, int64_t T, int32_t Tc, int32_t G, uint16_t *y)
{
    if (L < 1 || C < 1 || T < 0 || Tc < 1 || G < 1) return ORC_ERR_ARG;
    for (int64_t r = 0; r < (int64_t)L * 2; ++r) {
        const int64_t base = r * T;
        for (int64_t t = 0; t < T; ++t) {
            const int64_t a = anchor_of(t, Tc, G);
            if (t == a) continue;
            const uint16_t *ya = y + (base + a) * C; /* anchors are never rewritten */
            uint16_t *yt = y + (base + t) * C;
            for (int32_t c = 0; c < C; ++c)
                yt[c] = orc_float_to_half(sat(orc_half_to_float(yt[c]) + orc_half_to_float(ya[c])));
        }
    }
    return ORC_OK;
}
