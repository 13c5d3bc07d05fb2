// kvc_encode.hip - range coding of every stream, then packing ([CG] 2.1
// ac_enc; 2.3 step 3 for the chunking).
//
// k_encode:    one lane per stream (chunk, layer, K|V, token), 256 tokens of
//              one slab per block; the lane walks its C channel symbols and
//              codes each with its channel's CDF row (all lanes of a wave read
//              the same row at the same step).  Bytes go to the lane's own
//              scratch slot as aligned dwords; the length to stream_len.
// k_slab_sum:  per-slab sum of the stream lengths.
// k_scan:      exclusive scan of the slab sums -> slab_off (one block).
// k_pack:      per slab, an exclusive scan of its stream lengths, then each
//              wave copies streams from their slots to the payload.
#include "kvc_common.h"
#include "kvc_kernels.h"
#include "lane_coder.h"
#include "pair_tile.h"

namespace {

// One lane per stream, 256 tokens of one slab per block.  The slab's CDF is
// walked in tiles of CT channels (CT * A = 2048 pairs, 8 KB), double-buffered
// in LDS: while a tile is coded, the next one is in flight in registers.
// All lanes of a wave read the same tile row at the same step, so a pair
// lookup is a broadcast or a distinct bank.
template <bool VEC16>
__global__ __launch_bounds__(256) void k_encode(const uint8_t *__restrict__ sym,
                                                const uint16_t *__restrict__ cdf,
                                                uint8_t *__restrict__ slots,
                                                uint16_t *__restrict__ stream_len, KParams p, int CT)
{
    extern __shared__ uint32_t lds[];
    const int bps = (p.Tc + 255) / 256;
    const int64_t slab = blockIdx.x / bps;
    const int t = (int)(blockIdx.x - slab * bps) * 256 + (int)threadIdx.x;
    const SlabGeom g = slab_geom(p, slab);
    const int C = p.C, A = p.A;
    const bool active = t < g.nj;
    const int64_t sid = g.sid0 + t;
    const uint8_t *q = sym + (g.row0 + (active ? t : 0)) * C;
    const uint16_t *rows = cdf + slab * C * A;
    lds_u32 *const tiles = (lds_u32 *)lds;
    const int ntiles = (C + CT - 1) / CT;

    PairTile pt;
    pt.load(rows, 0, CT, C, A);
    pt.store(tiles, CT, A);
    __syncthreads();

    SlotOut out{(uint32_t *)(slots + (active ? sid : 0) * p.slot_bytes)};
    EncState e;
    enc_init(e);
    for (int it = 0; it < ntiles; ++it) {
        const int c0 = it * CT, c1 = min(C, c0 + CT);
        if (it + 1 < ntiles) pt.load(rows, c0 + CT, CT, C, A);
        const lds_u32 *tile = tiles + (it & 1) * CT * A;
        if (active) {
            if constexpr (VEC16) {
                for (int cg = c0; cg < c1; cg += 16) {
                    const uint4 v = *(const uint4 *)(q + cg);
                    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
                    const lds_u32 *trow = tile + (cg - c0) * A;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        uint32_t s = (wv[i >> 2] >> (8 * (i & 3))) & 0xFFu;
                        s = s < (uint32_t)A ? s : (uint32_t)(A - 1);
                        enc_pair(e, trow[i * A + s], out);
                    }
                }
            } else {
                for (int c = c0; c < c1; ++c) {
                    uint32_t s = q[c];
                    s = s < (uint32_t)A ? s : (uint32_t)(A - 1);
                    enc_pair(e, tile[(c - c0) * A + s], out);
                }
            }
        }
        if (it + 1 < ntiles) pt.store(tiles + ((it + 1) & 1) * CT * A, CT, A);
        __syncthreads();
    }
    if (active) stream_len[sid] = (uint16_t)enc_finish(e, out);
}

__global__ __launch_bounds__(256) void k_slab_sum(const uint16_t *__restrict__ stream_len,
                                                  uint64_t *__restrict__ slab_total, KParams p)
{
    __shared__ uint32_t part[4];
    const SlabGeom g = slab_geom(p, blockIdx.x);
    uint32_t acc = 0;
    for (int t = threadIdx.x; t < g.nj; t += blockDim.x) acc += stream_len[g.sid0 + t];
    acc = wave_sum_u32(acc);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) slab_total[blockIdx.x] = (uint64_t)part[0] + part[1] + part[2] + part[3];
}

// Exclusive scan of 1024 per-thread values held in registers; returns the
// thread's prefix and writes the block total to *total.
__device__ uint64_t block_excl_scan_1024(uint64_t v, uint64_t *sh, uint64_t *total)
{
    const int tid = threadIdx.x;
    sh[tid] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        uint64_t add = tid >= off ? sh[tid - off] : 0;
        __syncthreads();
        sh[tid] += add;
        __syncthreads();
    }
    uint64_t incl = sh[tid];
    *total = sh[1023];
    __syncthreads();
    return incl - v;
}

__global__ __launch_bounds__(1024) void k_scan(const uint64_t *__restrict__ slab_total,
                                               uint64_t *__restrict__ slab_off, int64_t n,
                                               int64_t payload_cap, int32_t *status)
{
    __shared__ uint64_t sh[1024];
    const int64_t per = (n + 1023) / 1024;
    const int64_t b = threadIdx.x * per, e = min(n, b + per);
    uint64_t local = 0;
    for (int64_t i = b; i < e; ++i) local += slab_total[i];
    uint64_t total;
    uint64_t run = block_excl_scan_1024(local, sh, &total);
    for (int64_t i = b; i < e; ++i) {
        slab_off[i] = run;
        run += slab_total[i];
    }
    if (threadIdx.x == 0) {
        slab_off[n] = total;
        if (total > (uint64_t)payload_cap) kvc_flag(status, KVC_DEV_PAYLOAD_OVERFLOW);
    }
}

__global__ __launch_bounds__(256) void k_pack(const uint8_t *__restrict__ slots,
                                              const uint16_t *__restrict__ stream_len,
                                              const uint64_t *__restrict__ slab_off,
                                              uint8_t *__restrict__ payload, int64_t payload_cap,
                                              KParams p)
{
    __shared__ uint32_t s_len[256];
    __shared__ uint32_t s_off[256];
    __shared__ uint32_t s_wave[4];
    const SlabGeom g = slab_geom(p, blockIdx.x);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    uint64_t base = slab_off[blockIdx.x];
    for (int t0 = 0; t0 < g.nj; t0 += 256) {
        const int t = t0 + (int)threadIdx.x;
        uint32_t len = t < g.nj ? stream_len[g.sid0 + t] : 0u;
        // block exclusive scan of len
        uint32_t incl = len;
        for (int off = 1; off < 64; off <<= 1) {
            uint32_t o = (uint32_t)__shfl_up((int)incl, off, 64);
            if (lane >= off) incl += o;
        }
        if (lane == 63) s_wave[wid] = incl;
        __syncthreads();
        uint32_t wbase = 0;
        for (int i = 0; i < wid; ++i) wbase += s_wave[i];
        s_len[threadIdx.x] = len;
        s_off[threadIdx.x] = wbase + incl - len;
        const uint32_t round_total = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
        __syncthreads();
        // wave wid copies the streams of its own 64 lanes, one after another
        for (int k = 0; k < 64; ++k) {
            const int idx = wid * 64 + k;
            const int tk = t0 + idx;
            if (tk >= g.nj) break;
            const uint32_t n = s_len[idx];
            const uint8_t *src = slots + (g.sid0 + tk) * p.slot_bytes;
            const uint64_t dst = base + s_off[idx];
            for (uint32_t i = lane; i < n; i += 64)
                if (dst + i < (uint64_t)payload_cap) payload[dst + i] = src[i];
        }
        base += round_total;
        __syncthreads();
    }
}

__global__ void k_zero_u64(uint64_t *dst) { *dst = 0; }

}  // namespace

// Channels per LDS tile: 2048 pairs (8 KB) per buffer; at least 16 channels.
static int enc_tile_channels(int A) { return A <= 128 ? 2048 / A : 16; }

hipError_t launch_zero_u64(uint64_t *dst, hipStream_t stream)
{
    hipLaunchKernelGGL(k_zero_u64, dim3(1), dim3(1), 0, stream, dst);
    return hipGetLastError();
}

hipError_t launch_encode(const uint8_t *sym, const uint16_t *cdf, uint8_t *slots,
                         uint64_t *slab_total, uint16_t *stream_len, uint64_t *slab_off,
                         uint8_t *payload, int64_t payload_cap, const KParams &p, int32_t *status,
                         bool vec16, hipStream_t stream)
{
    if (p.n_slabs == 0) return launch_zero_u64(slab_off, stream);
    const int64_t bps = (p.Tc + 255) / 256;
    dim3 grid((unsigned)(bps * p.n_slabs));
    const int CT = enc_tile_channels(p.A);
    const size_t lds = 2 * (size_t)CT * p.A * sizeof(uint32_t);
    if (vec16 && CT % 16 == 0)
        hipLaunchKernelGGL(k_encode<true>, grid, dim3(256), lds, stream, sym, cdf, slots, stream_len, p, CT);
    else
        hipLaunchKernelGGL(k_encode<false>, grid, dim3(256), lds, stream, sym, cdf, slots, stream_len, p, CT);
    hipLaunchKernelGGL(k_slab_sum, dim3((unsigned)p.n_slabs), dim3(256), 0, stream, stream_len,
                       slab_total, p);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, stream, slab_total, slab_off, p.n_slabs,
                       payload_cap, status);
    hipLaunchKernelGGL(k_pack, dim3((unsigned)p.n_slabs), dim3(256), 0, stream, slots, stream_len,
                       slab_off, payload, payload_cap, p);
    return hipGetLastError();
}
