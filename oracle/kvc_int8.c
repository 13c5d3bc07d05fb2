/*
 * kvc_int8.c - plain CPU reference of the 8-bit KV quantization that the
 * codec is compared against: the per-channel INT8 quantizer
 * (KVQuantizationCache.quantize_key / dequantize_key) of the page
 * "大模型推理的KV Cache管理：从内存碎片到前缀缓存的优化实战" (KV cache management for LLM
 * inference), section 四 (KV cache quantization), cited as [KVM] 四.  It
 * stands for the 8-bit baseline of the CacheGen page's results table ([CG]
 * 1.3).
 *
 * TEST INFRASTRUCTURE ONLY, like kvc_oracle.c.
 *
 * For every group of g contiguous channels of a (layer, K|V, token) row (g =
 * head_dim: the page reduces over the last axis of a [heads][tokens]
 * [head_dim] tensor), in fp32 with every operation rounded on its own and
 * rint() rounding half to even:
 *   mn, mx     = min, max of the group
 *   scale      = (mx - mn) / 255
 *   zero_point = clamp(round(-mn / scale), 0, 255)          (u8)
 *   q          = clamp(round((x - mn) / scale), 0, 255)     (u8)
 *   y          = (q - zero_point) * scale
 * The page's dequantizer returns that product as float32 (it converts q and
 * the zero point with .float() and multiplies by the float scale), so fp32 is
 * the output that follows it; an fp16 output is the fp32 value rounded to
 * nearest even (and overflows to Inf where |y| passes 65504).
 * A constant group has scale 0, where the printed formula divides 0 by 0:
 * here it stores q = 0, zero_point = 0 and decodes to 0.
 */
#include <math.h>
#include <stdint.h>

#include "kvc_oracle.h"

static float clamp255(float r) { return r < 0.0f ? 0.0f : (r > 255.0f ? 255.0f : r); }

int orc_int8_quantize(int32_t L, int32_t C, int64_t T, int32_t g, const uint16_t *kv, uint8_t *q,
                      float *scale, uint8_t *zp)
{
    if (L < 1 || C < 1 || T < 0 || g < 1 || C % g != 0) return ORC_ERR_ARG;
    const int64_t n_rows = 2 * (int64_t)L * T;
    const int32_t G = C / g;
    for (int64_t row = 0; row < n_rows; ++row) {
        for (int32_t k = 0; k < G; ++k) {
            const uint16_t *x = kv + row * C + (int64_t)k * g;
            uint8_t *qq = q + row * C + (int64_t)k * g;
            float mn = orc_half_to_float(x[0]), mx = mn;
            for (int32_t i = 0; i < g; ++i) {
                const float v = orc_half_to_float(x[i]);
                if (!isfinite(v)) return ORC_ERR_NONFINITE;
                if (v < mn) mn = v;
                if (v > mx) mx = v;
            }
            const float range = mx - mn;
            const float s = range / 255.0f;
            const int64_t gi = row * G + k;
            scale[gi] = s;
            if (s == 0.0f) {
                zp[gi] = 0;
                for (int32_t i = 0; i < g; ++i) qq[i] = 0;
                continue;
            }
            const float z = -mn / s;
            zp[gi] = (uint8_t)(int)clamp255(rintf(z));
            for (int32_t i = 0; i < g; ++i) {
                const float d = orc_half_to_float(x[i]) - mn;
                const float u = d / s;
                qq[i] = (uint8_t)(int)clamp255(rintf(u));
            }
        }
    }
    return ORC_OK;
}

int orc_int8_dequantize(int32_t L, int32_t C, int64_t T, int32_t g, const uint8_t *q,
                        const float *scale, const uint8_t *zp, void *out, int32_t out_fp32)
{
    if (L < 1 || C < 1 || T < 0 || g < 1 || C % g != 0) return ORC_ERR_ARG;
    const int64_t n_rows = 2 * (int64_t)L * T;
    const int32_t G = C / g;
    for (int64_t row = 0; row < n_rows; ++row) {
        for (int32_t c = 0; c < C; ++c) {
            const int64_t gi = row * G + c / g;
            const float d = (float)((int32_t)q[row * C + c] - (int32_t)zp[gi]);
            const float y = d * scale[gi];
            if (out_fp32)
                ((float *)out)[row * C + c] = y;
            else
                ((uint16_t *)out)[row * C + c] = orc_float_to_half(y);
        }
    }
    return ORC_OK;
}
