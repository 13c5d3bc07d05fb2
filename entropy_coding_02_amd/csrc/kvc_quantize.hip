// kvc_quantize.hip - group max-abs quantization ([CG] 2.3 step 1).
//
// One wavefront per (layer, K|V, token) row.  For finite fp16, |x| orders
// like its bit pattern with the sign cleared, so the row max is an integer
// max of (bits & 0x7FFF): exact, and it detects Inf/NaN (>= 0x7C00) for free.
// The quantizer runs in fp32 with one rounding per operation (the library is
// built with -ffp-contract=off): factor = MAX / m by IEEE division,
// p = x * factor, p = p + MAX, q = rint(p) (round half to even).
#include "kvc_common.h"
#include "kvc_kernels.h"

namespace {

__device__ __forceinline__ uint32_t quant1(uint32_t bits, float factor, float M)
{
    float p = kvc_h2f(bits) * factor;
    p = p + M;
    float r = __builtin_rintf(p);
    r = r < 0.0f ? 0.0f : (r > 255.0f ? 255.0f : r);  // only non-finite rows get here
    return (uint32_t)r;
}

// VEC = fp16 elements per lane access: 8 (16-byte loads, C % 8 == 0 and
// 16-byte aligned buffers) or 1 (any C).
template <int VEC>
__global__ __launch_bounds__(256) void k_quantize_rows(const uint16_t *__restrict__ kv,
                                                       uint8_t *__restrict__ sym,
                                                       uint16_t *__restrict__ max1, KParams p,
                                                       int32_t *status)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const int C = p.C;
    for (int64_t row = wave; row < p.n_rows; row += nwaves) {
        const uint16_t *x = kv + row * C;
        uint8_t *q = sym + row * C;
        uint32_t mx = 0;
        // rows of up to 1024 channels stay in registers (two 16-byte pieces per lane)
        constexpr int KREG = VEC == 8 ? 2 : 1;
        u32x4 reg[KREG];
        if constexpr (VEC == 8) {
#pragma unroll
            for (int k = 0; k < KREG; ++k) {
                const int c = (lane + 64 * k) * 8;
                reg[k] = c < C ? *(const u32x4 *)(x + c) : u32x4{0, 0, 0, 0};
            }
            for (int c = (lane + 64 * KREG) * 8; c < C; c += 64 * 8) {
                const u32x4 v = *(const u32x4 *)(x + c);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t a = v[i] & 0x7FFF7FFFu;
                    mx = max(mx, max(a & 0xFFFFu, a >> 16));
                }
            }
#pragma unroll
            for (int k = 0; k < KREG; ++k)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t a = reg[k][i] & 0x7FFF7FFFu;
                    mx = max(mx, max(a & 0xFFFFu, a >> 16));
                }
        } else {
            for (int c = lane; c < C; c += 64) mx = max(mx, (uint32_t)(x[c] & 0x7FFFu));
        }
        mx = wave_max_u32(mx);
        const int32_t lk = (int32_t)(row / p.T);
        const float M = (float)p.maxq[lk];
        const float m = kvc_h2f(mx);
        const float factor = (mx != 0) ? M / m : 0.0f;
        if (mx >= 0x7C00u && lane == 0) kvc_flag(status, KVC_DEV_NONFINITE);
        if (lane == 0) max1[row] = (uint16_t)mx;
        if constexpr (VEC == 8) {
            auto put = [&](int c, const u32x4 &v) {
                uint32_t b[2] = {0, 0};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t q0 = quant1(v[i] & 0xFFFFu, factor, M);
                    const uint32_t q1 = quant1(v[i] >> 16, factor, M);
                    b[i >> 1] |= (q0 | (q1 << 8)) << ((i & 1) * 16);
                }
                *(uint2 *)(q + c) = make_uint2(b[0], b[1]);
            };
#pragma unroll
            for (int k = 0; k < KREG; ++k) {
                const int c = (lane + 64 * k) * 8;
                if (c < C) put(c, reg[k]);
            }
            for (int c = (lane + 64 * KREG) * 8; c < C; c += 64 * 8) put(c, *(const u32x4 *)(x + c));
        } else {
            for (int c = lane; c < C; c += 64) q[c] = (uint8_t)quant1(x[c], factor, M);
        }
    }
}

}  // namespace

hipError_t launch_quantize_rows(const uint16_t *kv, uint8_t *sym, uint16_t *max1, const KParams &p,
                                int32_t *status, bool vec8, hipStream_t stream)
{
    if (p.n_rows == 0) return hipSuccess;
    int64_t blocks = (p.n_rows + 3) / 4;  // one wave per row, 4 waves per block
    const int64_t cap = 256 * 1024;
    if (blocks > cap) blocks = cap;
    if (vec8)
        hipLaunchKernelGGL(k_quantize_rows<8>, dim3((unsigned)blocks), dim3(256), 0, stream, kv, sym,
                           max1, p, status);
    else
        hipLaunchKernelGGL(k_quantize_rows<1>, dim3((unsigned)blocks), dim3(256), 0, stream, kv, sym,
                           max1, p, status);
    return hipGetLastError();
}
