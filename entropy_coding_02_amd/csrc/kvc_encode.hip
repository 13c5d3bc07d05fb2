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
template <bool VEC16, int PER>
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
    // A tile's pairs and symbols arrive in registers while the previous tile
    // is coded, and go into LDS between two barriers.  Symbol pieces: 16 bytes
    // of a token row; CT <= 64 gives at most 4 per thread.
    PairTile<PER> pt;
    u32x4 sv[4];
    const int per_row = CT / 16;
    auto load_syms = [&](int c0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ch = (int)threadIdx.x + 256 * i;
            const int r = ch / per_row, part = ch - r * per_row;
            const int tok = tb * 256 + r, cc = c0 + part * 16;
            sv[i] = (ch < 256 * per_row && tok < g.nj && cc < C)
                        ? *(const u32x4 *)(sym + (g.row0 + tok) * C + cc)
                        : u32x4{0, 0, 0, 0};
        }
    };
    auto store_syms = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ch = (int)threadIdx.x + 256 * i;
            if (ch < 256 * per_row) {
                const int r = ch / per_row, part = ch - r * per_row;
                *(lds_u32x4 *)(stile + r * sstride + part * 16) = sv[i];
            }
        }
    };
    pt.load(rows, 0, CT, C, A);
    if constexpr (VEC16) load_syms(0);
    for (int it = 0; it < ntiles; ++it) {
        const int c0 = it * CT, c1 = min(C, c0 + CT);
        __syncthreads();  // every wave is done with the previous tile
        pt.store(pairs, CT, A);
        if constexpr (VEC16) store_syms();
        __syncthreads();
        if (it + 1 < ntiles) {
            pt.load(rows, c0 + CT, CT, C, A);
            if constexpr (VEC16) load_syms(c0 + CT);
        }
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

// Per encoder block (256 streams of a slab), one lane per stream: the
// stream's payload offset o (slab offset + the lengths before it), then its
// bytes go out as whole aligned dwords wherever a destination dword lies
// inside [o, o + len), each the funnel shift of two consecutive slot dwords
// (slot loads are coalesced: lanes read their k-th dwords together); the up
// to 3 + 3 bytes at either end, which share a dword with the neighbouring
// streams, are written one byte at a time.  Nothing is written at or past
// payload_cap.
__global__ __launch_bounds__(256) void k_pack(const uint8_t *__restrict__ slots,
                                              const uint16_t *__restrict__ stream_len,
                                              const uint64_t *__restrict__ slab_off,
                                              uint8_t *__restrict__ payload, int64_t payload_cap,
                                              KParams p)
{
    __shared__ uint32_t s_red[4];
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
    if (lane == 63) s_red[wid] = incl;
    __syncthreads();
    uint32_t wbase = 0;
    for (int i = 0; i < wid; ++i) wbase += s_red[i];
    if (!active || len == 0) return;  // no barriers below
    const uint64_t o = slab_off[slab] + pre + wbase + incl - len;
    const uint64_t e = o + len;
    const uint32_t *src = (const uint32_t *)(slots + (int64_t)blockIdx.x * p.slot_bytes * 256) + threadIdx.x;
    const uint64_t cap = (uint64_t)payload_cap;
    // byte i of the stream is byte (i & 3) of slot dword i >> 2 (bytes in memory order)
    auto byte_at = [&](uint32_t i) -> uint32_t { return (src[(i >> 2) * 256u] >> (8u * (i & 3u))) & 0xFFu; };
    const uint64_t d0 = (o + 3u) & ~(uint64_t)3;  // first whole destination dword
    const uint64_t d1 = e & ~(uint64_t)3;         // end of the whole destination dwords
    if (d0 >= d1) {
        for (uint32_t i = 0; i < len; ++i)
            if (o + i < cap) payload[o + i] = (uint8_t)byte_at(i);
        return;
    }
    for (uint64_t b = o; b < d0; ++b)
        if (b < cap) payload[b] = (uint8_t)byte_at((uint32_t)(b - o));
    for (uint64_t b = d1; b < e; ++b)
        if (b < cap) payload[b] = (uint8_t)byte_at((uint32_t)(b - o));
    // whole dwords: destination dword at b takes stream bytes [b - o, b - o + 4)
    const uint32_t i0 = (uint32_t)(d0 - o);  // 0..3
    const uint32_t sh = 8u * (i0 & 3u);
    uint32_t k = i0 >> 2;  // 0
    uint32_t lo = src[(uint64_t)k * 256u];
    for (uint64_t b = d0; b < d1; b += 4) {
        const uint32_t hi = (b - o + 4u <= len) || sh ? src[(uint64_t)(k + 1) * 256u] : 0u;
        const uint32_t v = sh ? (lo >> sh) | (hi << (32u - sh)) : lo;
        if (b + 4u <= cap) {
            *(uint32_t *)(payload + b) = v;
        } else {
            for (uint32_t j = 0; j < 4; ++j)
                if (b + j < cap) payload[b + j] = (uint8_t)(v >> (8u * j));
        }
        lo = hi;
        ++k;
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
    const int per = (CT * (p.A / 2) + 255) / 256;  // pairs staged per thread
#define KVC_ENC(V, P, L)                                                                             \
    hipLaunchKernelGGL((k_encode<V, P>), grid, dim3(256), L, stream, sym, cdf, slots, stream_len, p, CT)
    const size_t lds_syms = lds_pairs + 256 * (size_t)(CT + 16);
    if (vec16) {
        if (per <= 2) KVC_ENC(true, 2, lds_syms);
        else KVC_ENC(true, 8, lds_syms);
    } else {
        if (per <= 2) KVC_ENC(false, 2, lds_pairs);
        else KVC_ENC(false, 8, lds_pairs);
    }
#undef KVC_ENC
    hipLaunchKernelGGL(k_slab_sum, dim3((unsigned)p.n_slabs), dim3(256), 0, stream, stream_len,
                       slab_total, p);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, stream, slab_total, slab_off, p.n_slabs,
                       payload_cap, status);
    hipLaunchKernelGGL(k_pack, grid, dim3(256), 0, stream, slots, stream_len,
                       slab_off, payload, payload_cap, p);
    return hipGetLastError();
}
