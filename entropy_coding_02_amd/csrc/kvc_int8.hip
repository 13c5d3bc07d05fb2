// kvc_int8.hip - the 8-bit KV quantizer the codec is compared with: the
// per-channel INT8 quantizer of the page "大模型推理的KV Cache管理：从内存碎片到前缀缓存的
// 优化实战" (KV cache management for LLM inference), section 四, cited [KVM] 四.
//
// Per group of g contiguous channels of a (layer, K|V, token) row, in fp32
// with every operation rounded on its own (rint: half to even):
//   scale = (max - min) / 255,  zero_point = clamp(rint(-min / scale), 0, 255),
//   q = clamp(rint((x - min) / scale), 0, 255),  y = fp16((q - zero_point) * scale).
// A constant group (scale 0, where the printed formula divides 0 by 0) stores
// q = 0 and zero_point = 0, and decodes to 0.
#include "kvc_common.h"
#include "kvc_kernels.h"

namespace {

__device__ __forceinline__ float clamp255(float r) { return r < 0.0f ? 0.0f : (r > 255.0f ? 255.0f : r); }

__device__ __forceinline__ uint32_t q8(float x, float mn, float s)
{
    const float d = x - mn;
    const float u = d / s;
    return (uint32_t)clamp255(__builtin_rintf(u));
}

// One wavefront per row, C % 8 == 0, C <= 1024, 16-byte aligned buffers; a
// group is LPG = g / 8 consecutive lanes (a power of two up to 64), so its
// min and max are a segmented shuffle reduction.
template <int LPG>
__global__ __launch_bounds__(256) void k_int8_quant_rows(const uint16_t *__restrict__ kv,
                                                         uint8_t *__restrict__ q,
                                                         float *__restrict__ scale,
                                                         uint8_t *__restrict__ zp, int64_t n_rows,
                                                         int C, int32_t *status)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const int C8 = C / 8, G = C / (8 * LPG);
    for (int64_t row = wave; row < n_rows; row += nwaves) {
        const uint16_t *x = kv + row * C;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int pi = lane + 64 * k;  // uniform per LPG-lane segment
            if (k * 64 >= C8) break;
            const bool on = pi < C8;
            const u32x4 v = on ? *(const u32x4 *)(x + 8 * pi) : u32x4{0, 0, 0, 0};
            float f[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) f[i] = kvc_h2f((v[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
            float mn = f[0], mx = f[0];
            uint32_t bad = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                mn = fminf(mn, f[i]);
                mx = fmaxf(mx, f[i]);
                bad |= ((v[i >> 1] >> (16 * (i & 1))) & 0x7C00u) == 0x7C00u;
            }
#pragma unroll
            for (int off = 1; off < LPG; off <<= 1) {
                mn = fminf(mn, __shfl_xor(mn, off, 64));
                mx = fmaxf(mx, __shfl_xor(mx, off, 64));
            }
            if (on && bad) kvc_flag(status, KVC_DEV_NONFINITE);
            const float range = mx - mn;
            const float s = range / 255.0f;
            uint32_t b[2] = {0, 0};
            if (s != 0.0f) {
#pragma unroll
                for (int i = 0; i < 8; ++i) b[i >> 2] |= q8(f[i], mn, s) << (8 * (i & 3));
            }
            if (on) {
                *(uint2 *)(q + row * C + 8 * pi) = make_uint2(b[0], b[1]);
                if ((pi & (LPG - 1)) == 0) {
                    const int64_t gi = row * G + pi / LPG;
                    scale[gi] = s;
                    zp[gi] = s != 0.0f ? (uint8_t)clamp255(__builtin_rintf(-mn / s)) : (uint8_t)0;
                }
            }
        }
    }
}

// Any shape: one thread per group.
__global__ __launch_bounds__(256) void k_int8_quant_groups(const uint16_t *__restrict__ kv,
                                                           uint8_t *__restrict__ q,
                                                           float *__restrict__ scale,
                                                           uint8_t *__restrict__ zp,
                                                           int64_t n_groups, int g, int32_t *status)
{
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gi < n_groups; gi += step) {
        const uint16_t *x = kv + gi * g;
        float mn = kvc_h2f(x[0]), mx = mn;
        bool bad = false;
        for (int i = 0; i < g; ++i) {
            const float f = kvc_h2f(x[i]);
            mn = fminf(mn, f);
            mx = fmaxf(mx, f);
            bad |= (x[i] & 0x7C00u) == 0x7C00u;
        }
        if (bad) kvc_flag(status, KVC_DEV_NONFINITE);
        const float range = mx - mn;
        const float s = range / 255.0f;
        scale[gi] = s;
        zp[gi] = s != 0.0f ? (uint8_t)clamp255(__builtin_rintf(-mn / s)) : (uint8_t)0;
        for (int i = 0; i < g; ++i) q[gi * g + i] = s != 0.0f ? (uint8_t)q8(kvc_h2f(x[i]), mn, s) : 0;
    }
}

// y = (q - zero_point) * scale, as fp32 (F32) or rounded to fp16, one
// element per thread.
template <bool F32>
__global__ __launch_bounds__(256) void k_int8_dequant(const uint8_t *__restrict__ q,
                                                      const float *__restrict__ scale,
                                                      const uint8_t *__restrict__ zp,
                                                      void *__restrict__ out, int64_t n_el, int g)
{
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n_el; e += step) {
        const int64_t gi = e / g;
        const float d = (float)((int32_t)q[e] - (int32_t)zp[gi]);
        const float y = d * scale[gi];
        if constexpr (F32)
            ((float *)out)[e] = y;
        else
            ((uint16_t *)out)[e] = (uint16_t)kvc_f2h(y);
    }
}

// The same for g % 8 == 0 and aligned buffers: 8 elements (one group) per
// thread, an 8-byte load and one 16-byte (fp16) or two (fp32) stores.
template <bool F32>
__global__ __launch_bounds__(256) void k_int8_dequant8(const uint8_t *__restrict__ q,
                                                       const float *__restrict__ scale,
                                                       const uint8_t *__restrict__ zp,
                                                       void *__restrict__ out, int64_t n8, int g8)
{
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n8; e += step) {
        const int64_t gi = e / g8;
        const uint2 v = ((const uint2 *)q)[e];
        const int32_t z = zp[gi];
        const float s = scale[gi];
        float y[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t w = i < 4 ? v.x : v.y;
            y[i] = (float)((int32_t)((w >> (8 * (i & 3))) & 0xFFu) - z) * s;
        }
        if constexpr (F32) {
            ((float4 *)out)[2 * e] = make_float4(y[0], y[1], y[2], y[3]);
            ((float4 *)out)[2 * e + 1] = make_float4(y[4], y[5], y[6], y[7]);
        } else {
            ((uint4 *)out)[e] = make_uint4(kvc_f2h2(y[0], y[1]), kvc_f2h2(y[2], y[3]), kvc_f2h2(y[4], y[5]),
                                           kvc_f2h2(y[6], y[7]));
        }
    }
}

unsigned grid_cap(int64_t blocks)
{
    return (unsigned)(blocks < 1 ? 1 : (blocks > 262144 ? 262144 : blocks));
}

}  // namespace

hipError_t launch_int8_quantize(const uint16_t *kv, uint8_t *q, float *scale, uint8_t *zp,
                                int64_t n_rows, int C, int g, bool vec, int32_t *status,
                                hipStream_t stream)
{
    if (n_rows == 0) return hipSuccess;
    const int lpg = g / 8;
    const bool rows = vec && g % 8 == 0 && C % 8 == 0 && C <= 1024 && lpg >= 1 && lpg <= 64 &&
                      (lpg & (lpg - 1)) == 0;
    if (rows) {
        const dim3 grid(grid_cap((n_rows + 3) / 4)), block(256);
#define KVC_I8(N)                                                                                    \
    case N:                                                                                          \
        hipLaunchKernelGGL(k_int8_quant_rows<N>, grid, block, 0, stream, kv, q, scale, zp, n_rows, C, \
                           status);                                                                  \
        break;
        switch (lpg) {
            KVC_I8(1) KVC_I8(2) KVC_I8(4) KVC_I8(8) KVC_I8(16) KVC_I8(32) KVC_I8(64)
        }
#undef KVC_I8
    } else {
        const int64_t n_groups = n_rows * (C / g);
        hipLaunchKernelGGL(k_int8_quant_groups, dim3(grid_cap((n_groups + 255) / 256)), dim3(256), 0,
                           stream, kv, q, scale, zp, n_groups, g, status);
    }
    return hipGetLastError();
}

hipError_t launch_int8_dequantize(const uint8_t *q, const float *scale, const uint8_t *zp, void *out,
                                  bool f32, int64_t n_el, int g, hipStream_t stream)
{
    if (n_el == 0) return hipSuccess;
    if (g % 8 == 0 && ((uintptr_t)q & 7) == 0 && ((uintptr_t)out & 15) == 0) {
        const int64_t n8 = n_el / 8;
        const dim3 grid(grid_cap((n8 + 255) / 256)), block(256);
        if (f32)
            hipLaunchKernelGGL(k_int8_dequant8<true>, grid, block, 0, stream, q, scale, zp, out, n8, g / 8);
        else
            hipLaunchKernelGGL(k_int8_dequant8<false>, grid, block, 0, stream, q, scale, zp, out, n8, g / 8);
    } else {
        const dim3 grid(grid_cap((n_el + 255) / 256)), block(256);
        if (f32)
            hipLaunchKernelGGL(k_int8_dequant<true>, grid, block, 0, stream, q, scale, zp, out, n_el, g);
        else
            hipLaunchKernelGGL(k_int8_dequant<false>, grid, block, 0, stream, q, scale, zp, out, n_el, g);
    }
    return hipGetLastError();
}
