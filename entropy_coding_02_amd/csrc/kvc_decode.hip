// kvc_decode.hip - parallel range decoding with fused dequantization
// ([CG] 2.4 steps 1-2), and dequantization on its own.
//
// k_decode: one lane per stream, 256 tokens of one slab per block.  The block
// finds its streams' payload offsets (slab offset + exclusive scan of the
// stream lengths), builds the slab's dequantization table
//     lut[q] = fp32(q - MAX) / MAX        (one IEEE division per entry)
// in LDS, and each lane then decodes its C symbols: a binary search of the
// channel's CDF row for the largest k with r*cdf_k <= code, the interval
// update, byte refill, and y = lut[s] * max1 written as fp16 or fp32.
// Because fl(fl(q - MAX) / MAX) is exactly the table entry, the fused output
// equals the separate dequantization bit for bit.
#include "kvc_common.h"
#include "kvc_kernels.h"
#include "lane_coder.h"

namespace {

enum { ODT_F16 = 0, ODT_F32 = 1, ODT_NONE = 2 };

template <bool VEC, int ODT>
__global__ __launch_bounds__(256) void k_decode(const uint8_t *__restrict__ payload,
                                                int64_t payload_bytes,
                                                const uint64_t *__restrict__ slab_off,
                                                const uint16_t *__restrict__ stream_len,
                                                const uint16_t *__restrict__ cdf,
                                                const uint16_t *__restrict__ max1,
                                                uint8_t *__restrict__ sym_out, void *__restrict__ out,
                                                KParams p, int32_t *status)
{
    __shared__ float lut[256];
    __shared__ uint32_t s_red[4];
    const int bps = (p.Tc + 255) / 256;
    const int64_t slab = blockIdx.x / bps;
    const int tb = (int)(blockIdx.x - slab * bps);
    const int t = tb * 256 + (int)threadIdx.x;
    const SlabGeom g = slab_geom(p, slab);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int C = p.C, A = p.A;

    // bytes of the slab's streams before this block (only when chunk_tokens > 256)
    uint32_t pre = 0;
    const int n_before = min(tb * 256, g.nj);
    for (int i = threadIdx.x; i < n_before; i += 256) pre += stream_len[g.sid0 + i];
    pre = wave_sum_u32(pre);
    if (lane == 0) s_red[wid] = pre;
    __syncthreads();
    pre = s_red[0] + s_red[1] + s_red[2] + s_red[3];
    __syncthreads();
    // exclusive scan of this block's lengths
    const uint32_t len = t < g.nj ? stream_len[g.sid0 + t] : 0u;
    uint32_t incl = len;
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t o = (uint32_t)__shfl_up((int)incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) s_red[wid] = incl;
    if (threadIdx.x < (unsigned)A) {
        const int M = p.maxq[g.lk];
        lut[threadIdx.x] = (float)((int)threadIdx.x - M) / (float)M;
    }
    __syncthreads();
    uint32_t wbase = 0;
    for (int i = 0; i < wid; ++i) wbase += s_red[i];
    if (t >= g.nj) return;  // no barriers below

    const int64_t row = g.row0 + t;
    const uint64_t off = slab_off[slab] + pre + wbase + incl - len;
    StreamIn in;
    in.init(payload, off, len, (uint64_t)payload_bytes);
    DecState d;
    dec_init(d, in);
    const uint16_t *rows = cdf + slab * C * A;
    const float m = (ODT != ODT_NONE) ? kvc_h2f(max1[row]) : 0.0f;
    const uint32_t step0 = dec_step0((uint32_t)A);
    uint32_t bad = 0;
    uint8_t *so = sym_out ? sym_out + row * C : nullptr;

    auto decode1 = [&](int c) -> uint32_t {
        return dec_symbol(d, rows + c * A, (uint32_t)A, step0, in, &bad);
    };

    if constexpr (VEC) {
        // C % 16 == 0: 16 symbols per round, written with 16-byte stores
        for (int c0 = 0; c0 < C; c0 += 16) {
            uint32_t sw[4] = {0, 0, 0, 0};
            uint32_t hw[8];
            float fw[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                uint32_t s = decode1(c0 + i);
                sw[i >> 2] |= s << (8 * (i & 3));
                if constexpr (ODT != ODT_NONE) {
                    float y = lut[s] * m;
                    if constexpr (ODT == ODT_F16) {
                        if (i & 1)
                            hw[i >> 1] |= kvc_f2h(y) << 16;
                        else
                            hw[i >> 1] = kvc_f2h(y);
                    } else {
                        fw[i] = y;
                    }
                }
            }
            if (so) *(uint4 *)(so + c0) = make_uint4(sw[0], sw[1], sw[2], sw[3]);
            if constexpr (ODT == ODT_F16) {
                uint4 *o = (uint4 *)((uint16_t *)out + row * C + c0);
                o[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
                o[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
            } else if constexpr (ODT == ODT_F32) {
                float4 *o = (float4 *)((float *)out + row * C + c0);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    o[i] = make_float4(fw[4 * i], fw[4 * i + 1], fw[4 * i + 2], fw[4 * i + 3]);
            }
        }
    } else {
        for (int c = 0; c < C; ++c) {
            uint32_t s = decode1(c);
            if (so) so[c] = (uint8_t)s;
            if constexpr (ODT != ODT_NONE) {
                float y = lut[s] * m;
                if constexpr (ODT == ODT_F16)
                    ((uint16_t *)out)[row * C + c] = (uint16_t)kvc_f2h(y);
                else
                    ((float *)out)[row * C + c] = y;
            }
        }
    }
    if (bad) kvc_flag(status, KVC_DEV_CORRUPT);
}

// Dequantization alone: one wavefront per row; each wave keeps the table of
// its current (layer, K|V) in its own LDS slice.
template <int ODT>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t *__restrict__ sym,
                                                 const uint16_t *__restrict__ max1,
                                                 void *__restrict__ out, KParams p)
{
    __shared__ float lut[4][256];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const int C = p.C;
    int cur = -1;
    for (int64_t row = wave; row < p.n_rows; row += nwaves) {
        const int lk = (int)(row / p.T);
        if (lk != cur) {
            const int M = p.maxq[lk];
            for (int q = lane; q < 256; q += 64) lut[wid][q] = (float)(q - M) / (float)M;
            cur = lk;
        }
        const float m = kvc_h2f(max1[row]);
        const uint8_t *q = sym + row * C;
        for (int c = lane; c < C; c += 64) {
            float y = lut[wid][q[c]] * m;
            if constexpr (ODT == ODT_F16)
                ((uint16_t *)out)[row * C + c] = (uint16_t)kvc_f2h(y);
            else
                ((float *)out)[row * C + c] = y;
        }
    }
}

}  // namespace

hipError_t launch_decode(const uint8_t *payload, int64_t payload_bytes, const uint64_t *slab_off,
                         const uint16_t *stream_len, const uint16_t *cdf, const uint16_t *max1,
                         uint8_t *sym_out, void *out, int out_dtype, const KParams &p,
                         int32_t *status, bool vec, hipStream_t stream)
{
    if (p.n_slabs == 0) return hipSuccess;
    const int64_t bps = (p.Tc + 255) / 256;
    dim3 grid((unsigned)(bps * p.n_slabs)), block(256);
    const int odt = out ? out_dtype : ODT_NONE;
#define KVC_DEC(V, O)                                                                            \
    hipLaunchKernelGGL((k_decode<V, O>), grid, block, 0, stream, payload, payload_bytes, slab_off, \
                       stream_len, cdf, max1, sym_out, out, p, status)
    if (vec) {
        if (odt == ODT_F16) KVC_DEC(true, ODT_F16);
        else if (odt == ODT_F32) KVC_DEC(true, ODT_F32);
        else KVC_DEC(true, ODT_NONE);
    } else {
        if (odt == ODT_F16) KVC_DEC(false, ODT_F16);
        else if (odt == ODT_F32) KVC_DEC(false, ODT_F32);
        else KVC_DEC(false, ODT_NONE);
    }
#undef KVC_DEC
    return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t *sym, const uint16_t *max1, void *out, int out_dtype,
                             const KParams &p, bool vec, hipStream_t stream)
{
    (void)vec;
    if (p.n_rows == 0) return hipSuccess;
    int64_t blocks = (p.n_rows + 3) / 4;
    if (blocks > 256 * 1024) blocks = 256 * 1024;
    if (out_dtype == KVC_F16)
        hipLaunchKernelGGL(k_dequant<ODT_F16>, dim3((unsigned)blocks), dim3(256), 0, stream, sym,
                           max1, out, p);
    else
        hipLaunchKernelGGL(k_dequant<ODT_F32>, dim3((unsigned)blocks), dim3(256), 0, stream, sym,
                           max1, out, p);
    return hipGetLastError();
}
