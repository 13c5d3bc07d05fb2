// kvc_cdf.hip - per-(chunk, layer, K|V, channel) symbol histograms turned into
// 16-bit CDFs ([CG] 2.3 steps 2-3).
//
// One block per (slab, tile of CT channels).  The tile's histograms live in
// LDS as CT rows of A+1 counters: the odd row stride puts neighbouring
// channels in different banks, so the atomics of a wave (one channel per
// lane, all counting the modal symbols) do not collide.  Each thread then
// turns its channel's row into cdf_k = k + floor(C_k * (65536 - A) / N_j)
// in place, and the block writes the tile's [CT][A] uint16 rows, which are
// contiguous in the output, with coalesced stores.
#include "kvc_common.h"
#include "kvc_kernels.h"

namespace {

__global__ __launch_bounds__(256) void k_cdf(const uint8_t *__restrict__ sym,
                                             uint16_t *__restrict__ cdf, KParams p, int CT)
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
    if (c < C) {
        const uint8_t *col = sym + g.row0 * C + c;
        uint32_t *h = hist + cl * stride;
        for (int t = tg; t < g.nj; t += tstep) {
            uint32_t v = col[(int64_t)t * C];
            v = v < (uint32_t)A ? v : (uint32_t)(A - 1);
            atomicAdd(&h[v], 1u);
        }
    }
    __syncthreads();
    if (tg == 0 && c < C) {
        uint32_t *h = hist + cl * stride;
        const uint32_t K = 65536u - (uint32_t)A, N = (uint32_t)g.nj;
        uint32_t Ck = 0;
        for (int k = 0; k < A; ++k) {
            uint32_t n = h[k];
            h[k] = (uint32_t)k + (Ck * K) / N;  // Ck * K < 2^32 since Ck <= N <= 65535
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

}  // namespace

hipError_t launch_cdf(const uint8_t *sym, uint16_t *cdf, const KParams &p, hipStream_t stream)
{
    if (p.n_slabs == 0) return hipSuccess;
    const int CT = p.A <= 128 ? 64 : 32;
    const size_t lds = (size_t)CT * (p.A + 1) * sizeof(uint32_t);
    dim3 grid((unsigned)(((p.C + CT - 1) / CT) * p.n_slabs));
    hipLaunchKernelGGL(k_cdf, grid, dim3(256), lds, stream, sym, cdf, p, CT);
    return hipGetLastError();
}
