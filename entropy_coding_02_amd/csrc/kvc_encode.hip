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

// One lane per stream, 256 tokens of one slab per block.  The slab is walked
// in tiles of CT channels: at each tile boundary the block stages the tile's
// CDF rows as packed (start, frequency) pairs and, when C % 16 == 0, the
// tile's symbols of its 256 tokens (coalesced 16-byte loads) in LDS.  The
// coding loop then reads only LDS: 16 symbols per ds_read_b128, pair lookups
// in batches of 8.  All lanes of a wave read the same pair row at the same
// step (broadcast or distinct banks); the symbol rows have a 16-byte-padded
// stride that spreads lanes over all banks.  Without global loads in the
// loop, the lanes' byte stores never make it wait.
template <bool VEC16>
__global__ __launch_bounds__(256) void k_encode(const uint8_t *__restrict__ sym,
                                                const uint16_t *__restrict__ cdf,
                                                uint8_t *__restrict__ slots,
                                                uint16_t *__restrict__ stream_len, KParams p, int CT)
{
    // LDS: pairs [CT][A] u32 | symbols [256][CT + 16] u8 (VEC16 only)
    extern __shared__ uint32_t lds[];
    const int bps = (p.Tc + 255) / 256;
    const int64_t slab = blockIdx.x / bps;
    const int tb = (int)(blockIdx.x - slab * bps);
    const int t = tb * 256 + (int)threadIdx.x;
    const SlabGeom g = slab_geom(p, slab);
    const int C = p.C, A = p.A;
    const bool active = t < g.nj;
    const int64_t sid = g.sid0 + t;
    const uint8_t *q = sym + (g.row0 + (active ? t : 0)) * C;
    const uint16_t *rows = cdf + slab * C * A;
    lds_u32 *const pairs = (lds_u32 *)lds;
    const int sstride = CT + 16;
    lds_u8 *const stile = (lds_u8 *)(pairs + CT * A);
    const int ntiles = (C + CT - 1) / CT;

    // slot dword k of this lane: block region + (k * 256 + lane) dwords
    SlotOut out{(uint32_t *)(slots + (int64_t)blockIdx.x * p.slot_bytes * 256) + threadIdx.x, 256u};
    EncState e;
    enc_init(e);
    for (int it = 0; it < ntiles; ++it) {
        const int c0 = it * CT, c1 = min(C, c0 + CT);
        __syncthreads();  // every wave is done with the previous tile
        {
            PairTile pt;
            pt.load(rows, c0, CT, C, A);
            pt.store(pairs, CT, A);
        }
        if constexpr (VEC16) {
            const int per_row = CT / 16;
            for (int ch = threadIdx.x; ch < 256 * per_row; ch += 256) {
                const int r = ch / per_row, part = ch - r * per_row;
                const int tok = tb * 256 + r, cc = c0 + part * 16;
                if (tok < g.nj && cc < C) {
                    const u32x4 v = *(const u32x4 *)(sym + (g.row0 + tok) * C + cc);
                    *(lds_u32x4 *)(stile + r * sstride + part * 16) = v;
                }
            }
        }
        __syncthreads();
        if (!active) continue;
        if constexpr (VEC16) {
            const lds_u8 *my = stile + threadIdx.x * sstride;
            for (int cg = c0; cg < c1; cg += 16) {
                const u32x4 v = *(const lds_u32x4 *)(my + (cg - c0));
                const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
                const lds_u32 *trow = pairs + (cg - c0) * A;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    uint32_t pv[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int k = h * 8 + i;
                        uint32_t s = (wv[k >> 2] >> (8 * (k & 3))) & 0xFFu;
                        s = s < (uint32_t)A ? s : (uint32_t)(A - 1);
                        pv[i] = trow[k * A + s];
                    }
#pragma unroll
                    for (int i = 0; i < 8; ++i) enc_pair(e, pv[i], out);
                }
            }
        } else {
            for (int c = c0; c < c1; ++c) {
                uint32_t s = q[c];
                s = s < (uint32_t)A ? s : (uint32_t)(A - 1);
                enc_pair(e, pairs[(c - c0) * A + s], out);
            }
        }
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

// Per encoder block (256 streams of a slab): the streams' payload offsets
// (slab offset + the lengths before them), then rounds of 64 bytes per
// stream: the block stages dwords [16r, 16r+16) of every lane's interleaved
// slot in LDS (loads coalesced across lanes), and each wave copies its 64
// streams' 64-byte pieces to their places in the payload, a stream at a time
// with one byte per lane.
__global__ __launch_bounds__(256) void k_pack(const uint8_t *__restrict__ slots,
                                              const uint16_t *__restrict__ stream_len,
                                              const uint64_t *__restrict__ slab_off,
                                              uint8_t *__restrict__ payload, int64_t payload_cap,
                                              KParams p)
{
    __shared__ uint32_t stage[256 * 17];
    __shared__ uint32_t s_len[256];
    __shared__ uint32_t s_red[4];
    __shared__ uint32_t s_max[4];
    const int bps = (p.Tc + 255) / 256;
    const int64_t slab = blockIdx.x / bps;
    const int tb = (int)(blockIdx.x - slab * bps);
    const SlabGeom g = slab_geom(p, slab);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int t = tb * 256 + (int)threadIdx.x;
    const bool active = t < g.nj;

    uint32_t pre = 0;
    const int n_before = min(tb * 256, g.nj);
    for (int i = threadIdx.x; i < n_before; i += 256) pre += stream_len[g.sid0 + i];
    pre = wave_sum_u32(pre);
    if (lane == 0) s_red[wid] = pre;
    __syncthreads();
    pre = s_red[0] + s_red[1] + s_red[2] + s_red[3];
    __syncthreads();
    const uint32_t len = active ? stream_len[g.sid0 + t] : 0u;
    uint32_t incl = len;
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t o = (uint32_t)__shfl_up((int)incl, off, 64);
        if (lane >= off) incl += o;
    }
    const uint32_t mx = wave_max_u32(len);
    if (lane == 63) s_red[wid] = incl;
    if (lane == 0) s_max[wid] = mx;
    s_len[threadIdx.x] = len;
    __syncthreads();
    uint32_t wbase = 0;
    for (int i = 0; i < wid; ++i) wbase += s_red[i];
    const uint64_t my_off = slab_off[slab] + pre + wbase + incl - len;
    const uint32_t maxlen = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
    const uint32_t *region = (const uint32_t *)(slots + (int64_t)blockIdx.x * p.slot_bytes * 256);

    for (uint32_t r0 = 0; r0 < maxlen; r0 += 64) {
        // stage dwords [r0/4, r0/4 + 16) of every lane's slot
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t k = r0 / 4 + (uint32_t)j;
            stage[threadIdx.x * 17 + j] = (4u * k < len) ? region[(int64_t)k * 256 + threadIdx.x] : 0u;
        }
        __syncthreads();
        // wave wid copies bytes [r0, r0+64) of streams wid*64 .. wid*64+63
        for (int k = 0; k < 64; ++k) {
            const int idx = wid * 64 + k;
            const uint32_t n = s_len[idx];
            const uint32_t b = r0 + (uint32_t)lane;
            const uint64_t o = __shfl(my_off, k, 64) + b;
            if (b < n && o < (uint64_t)payload_cap)
                payload[o] = (uint8_t)(stage[idx * 17 + lane / 4] >> (8 * (lane & 3)));
        }
        __syncthreads();
    }
}

__global__ void k_zero_u64(uint64_t *dst) { *dst = 0; }

}  // namespace

// Channels per tile: 1024 pairs (4 KB), between 16 and 64 channels (a
// multiple of 16, so symbol tiles are whole 16-byte pieces).
static int enc_tile_channels(int A)
{
    const int ct = 1024 / A;
    return ct < 16 ? 16 : (ct > 64 ? 64 : ct);
}

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
    const size_t lds_pairs = (size_t)CT * p.A * sizeof(uint32_t);
    if (vec16)
        hipLaunchKernelGGL(k_encode<true>, grid, dim3(256), lds_pairs + 256 * (size_t)(CT + 16), stream,
                           sym, cdf, slots, stream_len, p, CT);
    else
        hipLaunchKernelGGL(k_encode<false>, grid, dim3(256), lds_pairs, stream, sym, cdf, slots,
                           stream_len, p, CT);
    hipLaunchKernelGGL(k_slab_sum, dim3((unsigned)p.n_slabs), dim3(256), 0, stream, stream_len,
                       slab_total, p);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, stream, slab_total, slab_off, p.n_slabs,
                       payload_cap, status);
    hipLaunchKernelGGL(k_pack, grid, dim3(256), 0, stream, slots, stream_len,
                       slab_off, payload, payload_cap, p);
    return hipGetLastError();
}
