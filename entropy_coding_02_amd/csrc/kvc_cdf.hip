// kvc_cdf.hip - per-(chunk, layer, K|V, channel) symbol histograms turned into
// 16-bit CDFs ([CG] 2.3 steps 2-3).
//
// One block per (slab, tile of CT channels).  The tile's histograms live in
// LDS as CT rows of A+1 counters: the odd row stride puts neighbouring
// channels in different banks, so the atomics of a wave (one channel per
// lane, all counting the modal symbols) do not collide.  Each thread then
// turns its channel's row into cdf_k = k + floor(C_k * (65536 - A) / N_j)
// in place (kvc_cdf_entry), and the block writes the tile's [CT][A] uint16 rows, which are
// contiguous in the output, with coalesced stores.
#include "kvc_common.h"
#include "kvc_kernels.h"

namespace {

__global__ __launch_bounds__(256) void k_cdf(const uint8_t *__restrict__ sym,
                                             uint16_t *__restrict__ cdf, KParams p, int CT,
                                             int32_t *status)
{
    extern __shared__ uint32_t hist[];
    const int A = p.A, stride = A + 1, C = p.C;
    const int ntile = (p.C + CT - 1) / CT;
    const int64_t slab = blockIdx.x / ntile;
    const SlabGeom g = slab_geom(p, slab);
    const int c0 = (int)(blockIdx.x - slab * ntile) * CT;
    const int cl = threadIdx.x % CT, tg = threadIdx.x / CT, tstep = blockDim.x / CT;
    const int c = c0 + cl;

    for (int i = threadIdx.x; i < CT * stride; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    uint32_t bad = 0;
    if (c < C) {
        const uint8_t *col = sym + g.row0 * C + c;
        uint32_t *h = hist + cl * stride;
        for (int t = tg; t < g.nj; t += tstep) {
            uint32_t v = col[(int64_t)t * C];
            bad |= v >= (uint32_t)A ? 1u : 0u;
            v = v < (uint32_t)A ? v : (uint32_t)(A - 1);
            atomicAdd(&h[v], 1u);
        }
    }
    if (bad) kvc_flag(status, KVC_DEV_BAD_SYMBOL);
    __syncthreads();
    if (tg == 0 && c < C) {
        uint32_t *h = hist + cl * stride;
        const uint32_t K = 65536u - (uint32_t)A;
        uint32_t Ck = 0;
        for (int k = 0; k < A; ++k) {
            uint32_t n = h[k];
            h[k] = kvc_cdf_entry((uint32_t)k, Ck, K, g.rn);
            Ck += n;
        }
    }
    __syncthreads();
    const int nch = min(CT, C - c0);
    uint16_t *dst = cdf + (slab * C + c0) * A;
    for (int e = threadIdx.x; e < nch * A; e += blockDim.x) {
        int r = e / A, k = e - r * A;
        dst[e] = (uint16_t)hist[r * stride + k];
    }
}

// Wide variant for C % 4 == 0 and A <= 64: a block covers 256 channels of a
// slab (4 consecutive channels per lane, so a wave reads 256 contiguous
// symbol bytes of a token with one dword load per lane); wave w of the NW
// takes the tokens t = w (mod NW): 4, or 16 on launches of few slabs, where
// the 16 waves each walk a quarter of the tokens.  Counters are 16-bit halves of LDS words, word
// (c, s) at c*W + (c >> 2) + s/2 with W = A/2 + 1: at each of a lane's four
// steps the lanes' channels are 4 apart, and the (c >> 2) skew makes the word
// stride between lanes odd, so equal symbols fall in distinct banks.  Each
// thread then turns one channel's counts into its CDF row.
template <int NW>
__global__ __launch_bounds__(64 * NW) void k_cdf_wide(const uint8_t *__restrict__ sym,
                                                      uint16_t *__restrict__ cdf, KParams p,
                                                      int32_t *status)
{
    extern __shared__ uint32_t hist[];
    const int A = p.A, W = A / 2 + 1, C = p.C;
    const int ntile = (C + 255) / 256;
    const int64_t slab = blockIdx.x / ntile;
    const SlabGeom g = slab_geom(p, slab);
    const int c0 = (int)(blockIdx.x - slab * ntile) * 256;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int nwords = 256 * W + 64;
    for (int i = threadIdx.x; i < nwords; i += 64 * NW) hist[i] = 0;
    __syncthreads();
    const int cq = c0 + 4 * lane;  // this lane's first channel
    uint32_t bad = 0;
    if (cq < C) {
        const uint8_t *col = sym + g.row0 * C + cq;
        const int cl = 4 * lane;
        // 8 tokens per step, loaded before any is counted, so 8 loads are in flight
        for (int t0 = wid; t0 < g.nj; t0 += 8 * NW) {
            uint32_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int t = t0 + NW * u;
                v[u] = t < g.nj ? *(const uint32_t *)(col + (int64_t)t * C) : 0u;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) bad |= kvc_bytes_ge(v[u], (uint32_t)A);  // missing tokens read 0
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (t0 + NW * u >= g.nj) break;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint32_t s = (v[u] >> (8 * k)) & 0xFFu;
                    s = s < (uint32_t)A ? s : (uint32_t)(A - 1);
                    const int c = cl + k;
                    atomicAdd(&hist[c * W + (c >> 2) + (int)(s >> 1)], 1u << (16 * (s & 1u)));
                }
            }
        }
    }
    if (bad) kvc_flag(status, KVC_DEV_BAD_SYMBOL);
    __syncthreads();
    const int c = c0 + (int)threadIdx.x;
    if (threadIdx.x < 256 && c < C) {
        const int cl = (int)threadIdx.x;
        const uint32_t *h = hist + cl * W + (cl >> 2);
        const uint32_t K = 65536u - (uint32_t)A;
        uint16_t *dst = cdf + (slab * C + c) * A;
        uint32_t Ck = 0;
        for (int k = 0; k < A; k += 2) {
            const uint32_t w = h[k >> 1];
            const uint32_t lo = kvc_cdf_entry((uint32_t)k, Ck, K, g.rn);
            Ck += w & 0xFFFFu;
            const uint32_t hi = kvc_cdf_entry((uint32_t)(k + 1), Ck, K, g.rn);
            Ck += w >> 16;
            *(uint32_t *)(dst + k) = lo | (hi << 16);  // A even, rows 4-byte aligned
        }
    }
}

}  // namespace

// Launches of at most this many 256-channel tiles take 16 waves per block.
constexpr int64_t KVC_CDF_WIDE_TALL_MAX_BLOCKS = 1024;

hipError_t launch_cdf(const uint8_t *sym, uint16_t *cdf, const KParams &p, int32_t *status,
                      hipStream_t stream)
{
    if (p.n_slabs == 0) return hipSuccess;
    // k_cdf_wide counts in 16-bit halves: tables of at most 65535 tokens
    if (p.Tc <= 65535 && p.C % 4 == 0 && p.A <= 64 && ((uintptr_t)sym & 3) == 0 && ((uintptr_t)cdf & 3) == 0) {
        const size_t lds = sizeof(uint32_t) * (256 * (size_t)(p.A / 2 + 1) + 64);
        dim3 grid((unsigned)(((p.C + 255) / 256) * p.n_slabs));
        if (grid.x <= KVC_CDF_WIDE_TALL_MAX_BLOCKS)
            hipLaunchKernelGGL(k_cdf_wide<16>, grid, dim3(1024), lds, stream, sym, cdf, p, status);
        else
            hipLaunchKernelGGL(k_cdf_wide<4>, grid, dim3(256), lds, stream, sym, cdf, p, status);
        return hipGetLastError();
    }
    const int CT = p.A <= 128 ? 64 : 32;
    const size_t lds = (size_t)CT * (p.A + 1) * sizeof(uint32_t);
    dim3 grid((unsigned)(((p.C + CT - 1) / CT) * p.n_slabs));
    hipLaunchKernelGGL(k_cdf, grid, dim3(256), lds, stream, sym, cdf, p, CT, status);
    return hipGetLastError();
}
