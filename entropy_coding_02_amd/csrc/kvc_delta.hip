// kvc_delta.hip - token-delta ("change-based") coding with anchors, the step
// before quantization in the CacheGen write-up ([CG] 1.2 point 1: the K/V of
// neighbouring tokens are close, so differences rather than raw values are
// coded; [CG] 2.3 step 1 names the anchor-based form).
//
// Anchors are the tokens at chunk-relative positions 0, G, 2G, ... (G =
// anchor_tokens), so every chunk stands alone.  Forward: an anchor row is
// kept; another row x becomes d = fp16(sat(fp32(x) - fp32(xa_hat))), where
// xa_hat is the codec's reconstruction of its anchor row (the group max-abs
// quantizer at the layer's bins, dequantized to fp16: the values a decoder
// holds).  Inverse, on the decoded fp16 tensor y: every non-anchor row
// becomes fp16(sat(fp32(y) + fp32(y_anchor))).  sat() clamps to the finite
// fp16 range [-65504, 65504] (a difference of two finite fp16 values can
// reach twice that; the clamp is a coding error like any other), so only a
// non-finite input raises KVC_DEV_NONFINITE.  Both are HBM-bound streaming
// passes: one wave per anchor group, the anchor row (reconstructed once) in
// registers.
#include "kvc_common.h"
#include "kvc_kernels.h"

namespace {

__device__ __forceinline__ uint32_t d_quant1(uint32_t bits, float factor, float M)
{
    float p = kvc_h2f(bits) * factor;
    p = p + M;
    float r = __builtin_rintf(p);
    r = r < 0.0f ? 0.0f : (r > 255.0f ? 255.0f : r);  // only non-finite rows get here
    return (uint32_t)r;
}

// The codec's reconstruction of one element: fp16(fp32(q - MAX) / MAX * m),
// each operation rounded on its own (the decoder's table entry times max1).
__device__ __forceinline__ uint32_t recon1(uint32_t bits, float factor, float M, int Mi, float m)
{
    const uint32_t q = d_quant1(bits, factor, M);
    const float u = (float)((int)q - Mi) / (float)Mi;
    return kvc_f2h(u * m);
}

__device__ __forceinline__ float dsat(float v) { return __builtin_fminf(__builtin_fmaxf(v, -65504.0f), 65504.0f); }
__device__ __forceinline__ uint32_t dsub(uint32_t x, uint32_t a) { return kvc_f2h(dsat(kvc_h2f(x) - kvc_h2f(a))); }
__device__ __forceinline__ uint32_t dadd(uint32_t y, uint32_t a) { return kvc_f2h(dsat(kvc_h2f(y) + kvc_h2f(a))); }
// Inf or NaN in either half of a packed pair.
__device__ __forceinline__ bool nonfinite2(uint32_t x)
{
    return (x & 0x7C00u) == 0x7C00u || (x & 0x7C000000u) == 0x7C000000u;
}

struct Groups {
    int64_t per_lk;  // groups per (layer, K|V)
    int32_t gpc;     // groups per full chunk
    int32_t G;
};

__host__ __device__ inline Groups make_groups(const KParams &p, int G)
{
    Groups g;
    g.G = G;
    g.gpc = (p.Tc + G - 1) / G;
    g.per_lk = (int64_t)(p.NC - 1) * g.gpc + (p.last_nj + G - 1) / G;
    return g;
}

// Group gid -> its (layer, K|V) row block, first row (the anchor) and row count.
__device__ __forceinline__ void group_rows(const KParams &p, const Groups &gr, int64_t gid, int64_t &row0,
                                           int &nrows)
{
    const int64_t lk = gid / gr.per_lk;
    const int64_t rem = gid - lk * gr.per_lk;
    int64_t j = rem / gr.gpc;
    if (j > p.NC - 1) j = p.NC - 1;
    const int64_t g = rem - j * gr.gpc;
    const int nj = (j == p.NC - 1) ? p.last_nj : p.Tc;
    row0 = lk * p.T + j * p.Tc + g * gr.G;
    nrows = min(gr.G, nj - (int)(g * gr.G));
}

__device__ __forceinline__ uint32_t dpp_max(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// One wavefront per anchor group; C % 8 == 0, C <= 512 * KREG, 16-byte
// aligned buffers.  kv and out may be the same buffer.
template <int KREG>
__global__ __launch_bounds__(256) void k_delta_fwd(const uint16_t *kv, uint16_t *out, KParams p, Groups gr,
                                                   int64_t n_groups, int32_t *status)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const int C = p.C, C8 = C / 8;
    for (int64_t gid = wave; gid < n_groups; gid += nwaves) {
        int64_t row0;
        int nrows;
        group_rows(p, gr, gid, row0, nrows);
        const int lk = (int)(row0 / p.T);
        u32x4 a[KREG];
        uint32_t mx = 0;
#pragma unroll
        for (int k = 0; k < KREG; ++k) {
            const int pi = lane + 64 * k;
            a[k] = pi < C8 ? *(const u32x4 *)(kv + row0 * C + 8 * pi) : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t v = a[k][i] & 0x7FFF7FFFu;
                mx = max(mx, max(v & 0xFFFFu, v >> 16));
            }
        }
        mx = dpp_max(mx);
        bool bad = mx >= 0x7C00u;
        const int Mi = p.maxq[lk];
        const float M = (float)Mi, m = kvc_h2f(mx);
        const float factor = (mx != 0) ? M / m : 0.0f;
        u32x4 ah[KREG];  // the anchor's reconstruction
#pragma unroll
        for (int k = 0; k < KREG; ++k) {
            const int pi = lane + 64 * k;
            if (pi >= C8) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t lo = recon1(a[k][i] & 0xFFFFu, factor, M, Mi, m);
                const uint32_t hi = recon1(a[k][i] >> 16, factor, M, Mi, m);
                ah[k][i] = lo | (hi << 16);
            }
            if (out != kv) *(u32x4 *)(out + row0 * C + 8 * pi) = a[k];
        }
        for (int r = 1; r < nrows; ++r) {
            const int64_t row = row0 + r;
#pragma unroll
            for (int k = 0; k < KREG; ++k) {
                const int pi = lane + 64 * k;
                if (pi >= C8) continue;
                const u32x4 x = *(const u32x4 *)(kv + row * C + 8 * pi);
                u32x4 d;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t lo = dsub(x[i] & 0xFFFFu, ah[k][i] & 0xFFFFu);
                    const uint32_t hi = dsub(x[i] >> 16, ah[k][i] >> 16);
                    bad |= nonfinite2(x[i]);
                    d[i] = lo | (hi << 16);
                }
                *(u32x4 *)(out + row * C + 8 * pi) = d;
            }
        }
        if (bad) kvc_flag(status, KVC_DEV_NONFINITE);
    }
}

template <int KREG>
__global__ __launch_bounds__(256) void k_delta_inv(uint16_t *y, KParams p, Groups gr, int64_t n_groups)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const int C = p.C, C8 = C / 8;
    for (int64_t gid = wave; gid < n_groups; gid += nwaves) {
        int64_t row0;
        int nrows;
        group_rows(p, gr, gid, row0, nrows);
        u32x4 a[KREG];
#pragma unroll
        for (int k = 0; k < KREG; ++k) {
            const int pi = lane + 64 * k;
            a[k] = pi < C8 ? *(const u32x4 *)(y + row0 * C + 8 * pi) : u32x4{0, 0, 0, 0};
        }
        for (int r = 1; r < nrows; ++r) {
            const int64_t row = row0 + r;
#pragma unroll
            for (int k = 0; k < KREG; ++k) {
                const int pi = lane + 64 * k;
                if (pi >= C8) continue;
                u32x4 v = *(const u32x4 *)(y + row * C + 8 * pi);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    v[i] = dadd(v[i] & 0xFFFFu, a[k][i] & 0xFFFFu) | (dadd(v[i] >> 16, a[k][i] >> 16) << 16);
                *(u32x4 *)(y + row * C + 8 * pi) = v;
            }
        }
    }
}

// Any shape: one 64-thread block (one wave) per group, the anchor's
// reconstruction in LDS (C fp16 values).
__global__ __launch_bounds__(64) void k_delta_fwd_any(const uint16_t *kv, uint16_t *out, KParams p, Groups gr,
                                                      int64_t n_groups, int32_t *status)
{
    extern __shared__ uint16_t xa[];
    const int lane = threadIdx.x;
    const int C = p.C;
    for (int64_t gid = blockIdx.x; gid < n_groups; gid += gridDim.x) {
        int64_t row0;
        int nrows;
        group_rows(p, gr, gid, row0, nrows);
        const int lk = (int)(row0 / p.T);
        uint32_t mx = 0;
        for (int c = lane; c < C; c += 64) mx = max(mx, (uint32_t)(kv[row0 * C + c] & 0x7FFFu));
        mx = dpp_max(mx);
        bool bad = mx >= 0x7C00u;
        const int Mi = p.maxq[lk];
        const float M = (float)Mi, m = kvc_h2f(mx);
        const float factor = (mx != 0) ? M / m : 0.0f;
        __syncthreads();  // the previous group's readers are done with xa
        for (int c = lane; c < C; c += 64) {
            const uint32_t x = kv[row0 * C + c];
            xa[c] = (uint16_t)recon1(x, factor, M, Mi, m);
            if (out != kv) out[row0 * C + c] = (uint16_t)x;
        }
        __syncthreads();
        for (int r = 1; r < nrows; ++r) {
            const int64_t row = row0 + r;
            for (int c = lane; c < C; c += 64) {
                const uint32_t x = kv[row * C + c];
                bad |= nonfinite2(x);
                out[row * C + c] = (uint16_t)dsub(x, xa[c]);
            }
        }
        if (bad) kvc_flag(status, KVC_DEV_NONFINITE);
    }
}

__device__ __forceinline__ int64_t anchor_row(const KParams &p, const Groups &gr, int64_t row)
{
    const int64_t lk = row / p.T;
    const int64_t t = row - lk * p.T;
    const int64_t j = t / p.Tc;
    return lk * p.T + j * p.Tc + ((t - j * p.Tc) / gr.G) * gr.G;
}

__global__ __launch_bounds__(256) void k_delta_inv_any(uint16_t *y, KParams p, Groups gr)
{
    const int64_t n = p.n_rows * p.C;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += step) {
        const int64_t row = e / p.C, c = e - row * p.C;
        const int64_t arow = anchor_row(p, gr, row);
        if (row != arow) y[e] = (uint16_t)dadd(y[e], y[arow * p.C + c]);
    }
}

unsigned grid_of(int64_t blocks)
{
    return (unsigned)(blocks < 1 ? 1 : (blocks > 262144 ? 262144 : blocks));
}

}  // namespace

int64_t delta_groups(const KParams &p, int G) { return p.n_rows == 0 ? 0 : 2 * (int64_t)p.L * make_groups(p, G).per_lk; }

hipError_t launch_delta_forward(const uint16_t *kv, uint16_t *out, const KParams &p, int G, bool vec,
                                int32_t *status, hipStream_t stream)
{
    if (p.n_rows == 0) return hipSuccess;
    const Groups gr = make_groups(p, G);
    const int64_t ng = delta_groups(p, G);
    if (vec) {
        const dim3 grid(grid_of((ng + 3) / 4)), block(256);
        if (p.C <= 512)
            hipLaunchKernelGGL(k_delta_fwd<1>, grid, block, 0, stream, kv, out, p, gr, ng, status);
        else
            hipLaunchKernelGGL(k_delta_fwd<2>, grid, block, 0, stream, kv, out, p, gr, ng, status);
    } else {
        hipLaunchKernelGGL(k_delta_fwd_any, dim3(grid_of(ng)), dim3(64), (size_t)p.C * sizeof(uint16_t), stream,
                           kv, out, p, gr, ng, status);
    }
    return hipGetLastError();
}

hipError_t launch_delta_inverse(uint16_t *y, const KParams &p, int G, bool vec, hipStream_t stream)
{
    if (p.n_rows == 0) return hipSuccess;
    const Groups gr = make_groups(p, G);
    const int64_t ng = delta_groups(p, G);
    if (vec) {
        const dim3 grid(grid_of((ng + 3) / 4)), block(256);
        if (p.C <= 512)
            hipLaunchKernelGGL(k_delta_inv<1>, grid, block, 0, stream, y, p, gr, ng);
        else
            hipLaunchKernelGGL(k_delta_inv<2>, grid, block, 0, stream, y, p, gr, ng);
    } else {
        hipLaunchKernelGGL(k_delta_inv_any, dim3(grid_of((p.n_rows * p.C + 255) / 256)), dim3(256), 0, stream, y,
                           p, gr);
    }
    return hipGetLastError();
}
