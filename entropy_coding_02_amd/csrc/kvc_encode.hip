// kvc_encode.hip - range coding of every stream, then packing ([CG] 2.1
// ac_enc; 2.3 step 3 for the chunking).
//
// k_encode:    one lane per stream (chunk, layer, K|V, token), 16 or 64 streams
//              per wave, 256 tokens of one slab per slot region; the lane
//              walks its C channel symbols and
//              codes each with its channel's CDF row (all lanes of a wave read
//              the same row at the same step).  Bytes go to the lane's own
//              scratch slot as aligned dwords; the length to stream_len.
// k_slab_sum:  per-slab sum of the stream lengths.
// k_scan:      exclusive scan of the slab sums -> slab_off (one block).
// k_pack:      per 16 or 64 streams, their payload offsets, then the wave copies
//              them from their slots to the payload through an LDS window
//              (whole slot dwords as unaligned dword stores).
#include "kvc_common.h"
#include "kvc_kernels.h"
#include "lane_coder.h"
#include "pair_tile.h"

namespace {

// One lane per stream; the 256 tokens of a slab that share a slot region are
// coded by 256 / (4 SPW) blocks of four waves, SPW streams per wave (the
// other lanes only help stage tiles).  SPW = 64 keeps every lane coding;
// launches of few streams take SPW = 16, which fills four times as many
// SIMDs with waves whose branch to write out a finished dword is taken only
// when one of 16 lanes, not one of 64, has one (at a bit or two per symbol
// some lane of 64 nearly always has).  The slab is walked
// in tiles of CT channels: at each tile boundary the block stages the tile's
// CDF rows as packed (start, frequency) pairs in LDS.  When C % 16 == 0 the
// symbols of the block's tokens are staged too, in tiles of SW channels
// (coalesced 16-byte loads; SW is a multiple of CT): 64, so a 128-byte line
// of a token row is fetched in two halves rather than in 32-byte pieces, or
// 128 (whole lines) for launches of few streams, where the LDS it takes
// costs no occupancy that matters.  The coding loop then reads only LDS: 16 symbols per
// ds_read_b128, pair lookups in batches of 8.  All lanes of a wave read the
// same pair row at the same step (broadcast or distinct banks); the symbol
// rows have a 16-byte-padded stride that spreads lanes over all banks.
// Without global loads in the loop, the lanes' byte stores never make it
// wait.
//
// PRE4 (staged symbols, A a power of two up to 64): a byte is out of range
// when it has a bit at or above log2 A, one and-or per 16 staged bytes; the
// bytes are then staged as 4 * (s & (A - 1)), the byte offset of the pair
// within its row, so each lookup address is one byte-select add, and an
// out-of-range byte (flagged) still reads inside its row.
//
// A launch covers the slabs of (layer, K|V) pairs lk0 .. lk0 + nlk - 1 (of
// every chunk, in slab order) and stages the first A_st entries of each CDF
// row (A_st < A only where every symbol of those layers lies below A_st - 1):
// a symbol at or past A_st then sets KVC_DEV_INTERNAL_REDO, not
// KVC_DEV_BAD_SYMBOL.  A guard launch (guard != 0) returns unless that bit is
// set.
template <bool VEC16, int PER, int ENC_SW, int SPW, bool PRE4 = false>
__global__ __launch_bounds__(256) void k_encode(const uint8_t *__restrict__ sym,
                                                const uint16_t *__restrict__ cdf,
                                                uint8_t *__restrict__ slots,
                                                uint16_t *__restrict__ stream_len, KParams p, int CT,
                                                int32_t *status, int A_st, int lk0, int nlk, int guard)
{
    if (guard && (__atomic_load_n(status, __ATOMIC_RELAXED) & KVC_DEV_INTERNAL_REDO) == 0) return;
    static_assert(SPW == 16 || SPW == 32 || SPW == 64, "16, 32 or 64 streams per wave");
    constexpr int SPB = 4 * SPW;   // streams (token rows) per block
    constexpr int GB = 256 / SPB;  // blocks per 256-token slot region
    // LDS: pairs [CT][A] u32 | symbols [SPB][SW + 16] u8 (VEC16 only)
    extern __shared__ uint32_t lds[];
    const int bps = (p.Tc + 255) / 256;
    const int64_t bl = xcd_block(blockIdx.x, gridDim.x);  // a slab's blocks share an XCD
    const int64_t grl = bl / GB;  // 256 tokens of one of the launch's slabs
    const int sub = (int)(bl - grl * GB);
    const int64_t ql = grl / bps;  // the launch's slab ql: chunk ql / nlk, (layer, K|V) lk0 + ql % nlk
    const int tb = (int)(grl - ql * bps);
    const int64_t slab = (ql / nlk) * (2 * (int64_t)p.L) + lk0 + ql % nlk;
    const int64_t grp = slab * bps + tb;  // slot region
    const SlabGeom g = slab_geom(p, slab);
    const int r0 = tb * 256 + sub * SPB;  // the block's first token
    if (r0 >= g.nj) return;               // uniform: the whole block is past the slab
    const int lane = (int)threadIdx.x & 63;
    const int j = ((int)threadIdx.x >> 6) * SPW + lane;  // stream within the block (lane < SPW)
    const int t = r0 + j;
    const int C = p.C, A = A_st, AR = p.A;  // staged entries per row; the table's row length
    const bool active = lane < SPW && t < g.nj;
    const int64_t sid = g.sid0 + t;
    const uint8_t *q = sym + (g.row0 + (active ? t : 0)) * C;
    const uint16_t *rows = cdf + g.tab * C * AR;
    lds_u32 *const pairs = (lds_u32 *)lds;
    constexpr int sstride = ENC_SW + 16;
    lds_u8 *const stile = (lds_u8 *)(pairs + CT * A);
    const int ntiles = (C + CT - 1) / CT;

    // slot dword k of this lane: region + (k * 256 + stream within the region) dwords
    SlotOut out{(uint32_t *)(slots + grp * p.slot_bytes * 256), (uint32_t)(sub * SPB + j), 256u};
    EncState e;
    enc_init(e);
    // Tiles arrive in registers while the previous ones are coded, and go
    // into LDS between two barriers.  Symbol pieces: 16 bytes of a token row,
    // SW / 16 per row, SPB rows over 256 threads.
    PairTile<PER> pt;
    constexpr int per_row = ENC_SW / 16;
    constexpr int NP = SPB * per_row / 256;  // pieces per thread
    static_assert(NP >= 1 && SPB * per_row == 256 * NP, "whole pieces per thread");
    u32x4 sv[NP];
    uint32_t badsym = 0;  // some staged symbol byte is >= A
    auto load_syms = [&](int s0) {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int ch = (int)threadIdx.x + 256 * i;
            const int r = ch / per_row, part = ch - r * per_row;
            const int tok = r0 + r, cc = s0 + part * 16;
            sv[i] = (tok < g.nj && cc < C) ? *(const u32x4 *)(sym + (g.row0 + tok) * C + cc)
                                           : u32x4{0, 0, 0, 0};
        }
        if constexpr (PRE4) {
            const uint32_t hi = (0x100u - (uint32_t)A) * 0x01010101u, lo = ((uint32_t)A - 1u) * 0x01010101u;
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                badsym |= (sv[i].x | sv[i].y | sv[i].z | sv[i].w) & hi;
                sv[i] = u32x4{(sv[i].x & lo) << 2, (sv[i].y & lo) << 2, (sv[i].z & lo) << 2, (sv[i].w & lo) << 2};
            }
        } else {
#pragma unroll
            for (int i = 0; i < NP; ++i)
                badsym |= kvc_bytes_ge(sv[i].x, (uint32_t)A) | kvc_bytes_ge(sv[i].y, (uint32_t)A) |
                          kvc_bytes_ge(sv[i].z, (uint32_t)A) | kvc_bytes_ge(sv[i].w, (uint32_t)A);
        }
    };
    auto store_syms = [&]() {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int ch = (int)threadIdx.x + 256 * i;
            const int r = ch / per_row, part = ch - r * per_row;
            *(lds_u32x4 *)(stile + r * sstride + part * 16) = sv[i];
        }
    };
    pt.load(rows, 0, CT, C, A, AR);
    if constexpr (VEC16) load_syms(0);
    for (int it = 0; it < ntiles; ++it) {
        const int c0 = it * CT, c1 = min(C, c0 + CT);
        const int s0 = c0 - c0 % ENC_SW;  // the symbol tile holding [c0, c1)
        const bool new_stile = c0 == s0;
        __syncthreads();  // every wave is done with the previous tile
        pt.store(pairs, CT, A);
        if constexpr (VEC16) {
            if (new_stile) store_syms();
        }
        __syncthreads();
        if (it + 1 < ntiles) pt.load(rows, c0 + CT, CT, C, A, AR);
        if constexpr (VEC16) {
            if (new_stile && s0 + ENC_SW < C) load_syms(s0 + ENC_SW);
        }
        if (!active) continue;
        if constexpr (VEC16) {
            const lds_u8 *my = stile + j * sstride;
            for (int cg = c0; cg < c1; cg += 16) {
                const u32x4 v = *(const lds_u32x4 *)(my + (cg - s0));
                const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
                const lds_u32 *trow = pairs + (cg - c0) * A;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    uint32_t pv[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int k = h * 8 + i;
                        const uint32_t b = (wv[k >> 2] >> (8 * (k & 3))) & 0xFFu;
                        if constexpr (PRE4)  // b = 4 * symbol, a byte offset in row k
                            pv[i] = *(const lds_u32 *)((const lds_u8 *)(trow + k * A) + b);
                        else
                            pv[i] = trow[k * A + min(b, (uint32_t)A - 1u)];
                    }
#pragma unroll
                    for (int i = 0; i < 8; ++i) enc_pair(e, pv[i], out);
                }
            }
        } else {
            for (int c = c0; c < c1; ++c) {
                uint32_t s = q[c];
                badsym |= s >= (uint32_t)A ? 1u : 0u;
                s = min(s, (uint32_t)A - 1u);
                enc_pair(e, pairs[(c - c0) * A + s], out);
            }
        }
    }
    if (active) stream_len[sid] = (uint16_t)enc_finish(e, out);
    if (badsym) kvc_flag(status, A < AR ? KVC_DEV_INTERNAL_REDO : KVC_DEV_BAD_SYMBOL);
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
// thread's prefix and writes the block total to *total.  Each wave scans its
// 64 values with shuffles, wave 0 scans the 16 wave totals, and every thread
// adds its wave's offset: three barriers.
__device__ uint64_t block_excl_scan_1024(uint64_t v, uint64_t *sh, uint64_t *total)
{
    const int lane = (int)threadIdx.x & 63, wid = (int)threadIdx.x >> 6;
    uint64_t incl = v;
    for (int off = 1; off < 64; off <<= 1) {
        const uint64_t o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) sh[wid] = incl;
    __syncthreads();
    if (wid == 0) {
        uint64_t w = lane < 16 ? sh[lane] : 0u;
        for (int off = 1; off < 16; off <<= 1) {
            const uint64_t o = __shfl_up(w, off, 64);
            if (lane >= off) w += o;
        }
        if (lane < 16) sh[16 + lane] = w;  // inclusive prefix of the wave totals
    }
    __syncthreads();
    const uint64_t base = wid > 0 ? sh[16 + wid - 1] : 0u;
    *total = sh[31];
    __syncthreads();
    return base + incl - v;
}

// slab_total and slab_off may be the same array (each thread reads its own
// range before the scan and rewrites it element by element after).  With
// `expect`, a total different from *expect sets KVC_DEV_BAD_CONTAINER;
// otherwise a total above payload_cap sets KVC_DEV_PAYLOAD_OVERFLOW.
// Totals per thread k_scan keeps in registers (launches of up to 32768 slabs).
constexpr int SCAN_REG = 32;

__global__ __launch_bounds__(1024) void k_scan(const uint64_t *slab_total, uint64_t *slab_off,
                                               int64_t n, int64_t payload_cap,
                                               const uint64_t *expect, int32_t *status)
{
    __shared__ uint64_t sh[32];
    const int64_t per = (n + 1023) / 1024;
    const int64_t b = threadIdx.x * per, e = min(n, b + per);
    uint64_t total;
    if (per <= SCAN_REG) {
        // the thread's totals all requested at once and kept in registers for
        // the second pass (a loop waits for each load in turn)
        uint64_t v[SCAN_REG];
        uint64_t local = 0;
#pragma unroll
        for (int k = 0; k < SCAN_REG; ++k) {
            v[k] = b + k < e ? slab_total[b + k] : 0u;
            local += v[k];
        }
        uint64_t run = block_excl_scan_1024(local, sh, &total);
#pragma unroll
        for (int k = 0; k < SCAN_REG; ++k)
            if (b + k < e) {
                slab_off[b + k] = run;
                run += v[k];
            }
    } else {
        uint64_t local = 0;
        for (int64_t i = b; i < e; ++i) local += slab_total[i];
        uint64_t run = block_excl_scan_1024(local, sh, &total);
        for (int64_t i = b; i < e; ++i) {
            const uint64_t v = slab_total[i];
            slab_off[i] = run;
            run += v;
        }
    }
    if (threadIdx.x == 0) {
        // the encoder's guard launch has run: its redo bit is done with
        if (status) atomicAnd(status, ~(int32_t)KVC_DEV_INTERNAL_REDO);
        slab_off[n] = total;
        if (expect) {
            if (total != *expect) kvc_flag(status, KVC_DEV_BAD_CONTAINER);
        } else if (total > (uint64_t)payload_cap) {
            kvc_flag(status, KVC_DEV_PAYLOAD_OVERFLOW);
        }
    }
}

// One wavefront per SPW consecutive streams of a slot region (256 tokens of
// one slab): 64, or 16 for launches of few streams, where four times as many
// waves each walk a quarter of the streams.  Lane i < SPW first finds stream
// i's payload offset o (slab offset + the lengths before it).  The wave then
// walks its streams' slot dwords in rounds of 64: it stages slot dwords
// [64r, 64r + 64) of its SPW streams in LDS (coalesced loads: the slots are
// interleaved, stream i's k-th dword next to stream i + 1's), then writes the
// round's (stream, dword) pairs enumerated flat over the lanes (a prefix of
// the streams' dword counts, each lane finding its stream by a binary search
// of it), so a round takes about sum(dwords) / 64 store passes rather than
// one pass per stream: most streams hold a few dwords.  A slot
// dword holds 4 stream bytes in stream order, so every whole one goes out as
// one dword store at byte offset o + 4j, unaligned (gfx9 global stores take
// any byte address and write only the 4 bytes), and the last len % 4 bytes
// as byte stores; a store instruction thus covers up to 256 contiguous
// payload bytes and no byte of a neighbouring stream is touched.  Nothing is
// written at or past payload_cap.
// slot dwords per stream and round: 32 keeps the window small enough for
// about twice the waves per CU of 64 (the copy is latency-bound), and covers
// most streams of the larger workloads in one round
constexpr int PACK_W = 32;

template <int SPW>
__global__ __launch_bounds__(64) void k_pack(const uint8_t *__restrict__ slots,
                                             const uint16_t *__restrict__ stream_len,
                                             const uint64_t *__restrict__ slab_off,
                                             uint8_t *__restrict__ payload, int64_t payload_cap,
                                             KParams p)
{
    static_assert(SPW == 16 || SPW == 64, "16 or 64 streams per wave");
    constexpr int WPR = 256 / SPW;  // waves per slot region
    constexpr int PPR = SPW / 4;    // 16-byte pieces per staged slot row
    constexpr int RPL = 64 / PPR;   // slot rows per wave-wide load
    __shared__ uint32_t win[SPW * (PACK_W + 1)];  // [stream][PACK_W + 1] staged slot dwords
    __shared__ uint32_t pfx[SPW];                 // the round's flat start of each stream
    __shared__ uint32_t s_len[SPW], s_olo[SPW], s_ohi[SPW];  // each stream's length and payload offset
    const int bps = (p.Tc + 255) / 256;
    const int64_t eb = blockIdx.x / WPR;  // slot region
    const int wq = (int)(blockIdx.x - eb * WPR);
    const int64_t slab = eb / bps;
    const int tb = (int)(eb - slab * bps);
    const SlabGeom g = slab_geom(p, slab);
    const int lane = (int)threadIdx.x;
    const int t0 = tb * 256 + wq * SPW;
    if (t0 >= g.nj) return;  // the whole wave is past the slab's streams
    const int t = t0 + lane;
    const bool active = lane < SPW && t < g.nj;

    uint32_t pre = 0;  // bytes of the slab's streams before this wave's
    for (int i = lane; i < t0; i += 64) pre += stream_len[g.sid0 + i];
    pre = wave_sum_u32(pre);
    const uint32_t len = active ? stream_len[g.sid0 + t] : 0u;
    uint32_t incl = len;
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t v = (uint32_t)__shfl_up((int)incl, off, 64);
        if (lane >= off) incl += v;
    }
    const uint64_t o = slab_off[slab] + pre + incl - len;
    const int ndw = (int)((len + 3u) >> 2);  // slot dwords holding the stream
    const int ndw_max = (int)wave_max_u32((uint32_t)ndw);
    const int rounds = (ndw_max + PACK_W - 1) / PACK_W;
    // slot dword k of stream wq * SPW + i is dword k * 256 + wq * SPW + i of the region's slots
    const uint32_t *srcw = (const uint32_t *)(slots + eb * p.slot_bytes * 256) + wq * SPW;
    const uint32_t olo = (uint32_t)o, ohi = (uint32_t)(o >> 32);
    const uint64_t cap = (uint64_t)payload_cap;
    // staging: lane l loads 16 bytes = dword k of streams 4m .. 4m + 3 (m = l % PPR) for
    // k = k0 + RPL q + l / PPR, so one wave-wide load covers RPL slot rows
    const int sg = lane / PPR, sm = lane % PPR;
    // a load covers streams 4 sm .. 4 sm + 3: only their longest needs slot row k
    int ndw4 = max(ndw, __shfl_xor(ndw, 1, 64));
    ndw4 = max(ndw4, __shfl_xor(ndw4, 2, 64));
    const int ndw_grp = __shfl(ndw4, 4 * sm, 64);

    for (int r = 0; r < rounds; ++r) {
        const int k0 = r * PACK_W;
        u32x4 v4[PACK_W / RPL];
#pragma unroll
        for (int q = 0; q < PACK_W / RPL; ++q) {
            const int k = k0 + RPL * q + sg;
            v4[q] = k < ndw_grp ? *(const u32x4 *)(srcw + (int64_t)k * 256 + 4 * sm) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int q = 0; q < PACK_W / RPL; ++q) {
            const int u = RPL * q + sg;
#pragma unroll
            for (int e = 0; e < 4; ++e) win[(4 * sm + e) * (PACK_W + 1) + u] = v4[q][e];
        }
        // the round's (stream, slot dword) pairs, enumerated flat over the lanes:
        // stream i has n_i = clamp(ndw_i - k0, 0, PACK_W) of them, from flat index P_i on
        const uint32_t n_me = active ? (uint32_t)min(max(ndw - k0, 0), PACK_W) : 0u;
        uint32_t pin = n_me;  // inclusive prefix of n over the wave's streams
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t v = (uint32_t)__shfl_up((int)pin, off, 64);
            if (lane >= off) pin += v;
        }
        if (lane < SPW) {
            pfx[lane] = pin - n_me;
            s_len[lane] = len;
            s_olo[lane] = olo;
            s_ohi[lane] = ohi;
        }
        const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)pin, 63);
        __syncthreads();
        if (total >= 16u * SPW) {
            // long streams (16 dwords or more on average in this round): one
            // stream at a time, lane j < PACK_W taking its slot dword k0 + j,
            // with no search
            const uint32_t j = (uint32_t)(k0 + lane);
            for (int i = 0; i < SPW; ++i) {
                const uint32_t len_i = s_len[i];
                if ((uint32_t)k0 * 4u >= len_i) continue;  // uniform: stream i is done
                if (lane >= PACK_W || 4u * j >= len_i) continue;
                const uint64_t o_i = ((uint64_t)s_ohi[i] << 32) | s_olo[i];
                const uint32_t v = win[i * (PACK_W + 1) + lane];
                const uint64_t b = o_i + 4u * j;
                const uint32_t nb = min(len_i - 4u * j, 4u);
                if (nb == 4u && b + 4u <= cap) {
                    __builtin_memcpy(payload + b, &v, 4);
                } else {
                    for (uint32_t q = 0; q < nb; ++q)
                        if (b + q < cap) payload[b + q] = (uint8_t)(v >> (8u * q));
                }
            }
            __syncthreads();
            continue;
        }
        for (uint32_t f = (uint32_t)lane; f < total; f += 64u) {
            // stream i: the last with P_i <= f (P non-decreasing; streams of no dwords share a P)
            uint32_t i = 0;
#pragma unroll
            for (uint32_t b = SPW / 2; b >= 1; b >>= 1)
                if (pfx[i + b] <= f) i += b;
            const uint32_t jr = f - pfx[i];  // slot dword within the round
            const uint32_t j = (uint32_t)k0 + jr;
            const uint32_t len_i = s_len[i];  // (from LDS: a lane-to-lane read would see 0 from lanes
            const uint64_t o_i = ((uint64_t)s_ohi[i] << 32) | s_olo[i];  //  already out of this loop)
            const uint32_t v = win[i * (PACK_W + 1) + jr];
            const uint64_t b = o_i + 4u * j;  // stream bytes [4j, 4j + 4) go here
            const uint32_t nb = min(len_i - 4u * j, 4u);
            if (nb == 4u && b + 4u <= cap) {
                __builtin_memcpy(payload + b, &v, 4);
            } else {
                for (uint32_t q = 0; q < nb; ++q)
                    if (b + q < cap) payload[b + q] = (uint8_t)(v >> (8u * q));
            }
        }
        __syncthreads();
    }
}

// SplitOut for a lane of k_encode_split's phase B: the per-symbol dword
// store is a raw buffer store over the block's 64 slots, and a store that must
// not happen gets an offset past the buffer's range, which the hardware
// drops (no write, no fault), so no lane mask has to be set up for it.
struct SplitOutBuf : SplitOut {
    __amdgpu_buffer_rsrc_t rsrc;  // the block's slots, uniform
    uint32_t lbase;               // this lane's slot within them (bytes)
    __device__ void store_if(bool p, uint32_t i, uint32_t v) const
    {
        __builtin_amdgcn_raw_buffer_store_b32(v, rsrc, p ? lbase + off + 4u * i : 0x80000000u, 0, 0);
    }
    __device__ bool any(bool p) const { return __ballot(p) != 0; }
    // out of line, so the common path is one uniform branch over the call
    __device__ __noinline__ void carry(bool p, uint32_t w) const
    {
        if (p) enc_carry_into_written(*this, w);
    }
};

// floor(x / d) as a multiply-high, with m = 0xFFFFFFFF / d + 1 (d >= 2):
// m = 2^32 / d + eps with 0 <= eps < 1, so x m / 2^32 exceeds x / d by less
// than x / 2^32, which is below 1 / d when x d < 2^32 -- too little to
// carry x / d (whose fraction is at most (d - 1) / d) past an integer.
__device__ __forceinline__ uint32_t div_by_mulhi(uint32_t x, uint32_t m) { return __umulhi(x, m); }

// In B the four lanes of a quad read rows of four blocks a multiple of 32
// dwords apart, which would put equal symbols in one LDS bank: the table's
// four runs are set this many dwords apart.
#define KVC_SPLIT_SKEW 8

// A chunk of k_encode_split's pair table in registers.  With A even a CDF
// row is A / 2 dwords, each one (start, next start) pair, so pair e of a
// chunk is a dword of the table: chunk m < NA is dwords [m P, m P + P) (P =
// CH A / 2, channels [m CH, m CH + CH)); chunk NA + m is four runs of Q = P
// / 4 dwords, run b starting at channel b B + m CQ (local channel lc is block
// lc / CQ).  A thread's pairs are e = threadIdx.x + 256 i; bit i of last
// marks a pair that ends its row (its successor start is 65536), the same
// for every chunk.
template <int PERC>
struct ChunkPairs {
    uint32_t w[PERC], nx[PERC];

    // Every load is issued (pairs past the chunk read its first dword, and
    // a row's last pair reads its own start again), so none waits on a branch.
    __device__ void load(const uint32_t *rows, int m, int NA, int P, int B2, uint32_t last)
    {
        const int Q = P >> 2;
#pragma unroll
        for (int i = 0; i < PERC; ++i) {
            const int e = (int)threadIdx.x + 256 * i;
            int d;
            if (m < NA) {
                d = m * P + e;
            } else {
                const int b = (e >= Q) + (e >= 2 * Q) + (e >= 3 * Q);
                d = b * B2 + (m - NA) * Q + (e - b * Q);
            }
            d = e < P ? d : (m < NA ? m * P : (m - NA) * Q);
            w[i] = rows[d];
            nx[i] = ((const uint16_t *)rows)[2 * d + (((last >> i) & 1u) ? 0 : 2)];
        }
    }
    // run b of the chunk goes b * skew dwords further on
    __device__ void store(lds_u32 *ptab, int P, uint32_t last, int skew) const
    {
        const int Q = P >> 2;
#pragma unroll
        for (int i = 0; i < PERC; ++i) {
            const int e = (int)threadIdx.x + 256 * i;
            if (e < P) {
                lds_u32 *const dst = ptab + ((e >= Q) + (e >= 2 * Q) + (e >= 3 * Q)) * skew;
                // the loaded values are used from here only: nothing may be
                // computed from them (and so wait for them) at the load
                uint32_t wv = w[i], nv = nx[i];
                __asm__ volatile("" : "+v"(wv), "+v"(nv));
                const uint32_t st0 = wv & 0xFFFFu, st1 = wv >> 16;
                const uint32_t n2 = ((last >> i) & 1u) ? 65536u : nv;
                dst[2 * e] = cdf_pair(st0, st1);
                dst[2 * e + 1] = cdf_pair(st1, n2);
            }
        }
    }
};

// One stream coded by a quad of lanes (lane_coder.h, "one stream coded by G
// lanes"), for launches of few streams: 64 streams per block, 16 per wave,
// a slot region's 256 tokens over four blocks.  C splits into 4 blocks of B
// = C / 4 channels.  The block stages the symbols of all its 64 streams in
// LDS once, and the CDF pairs in chunks of CH channels (64 KB or less), so
// each phase waits on memory C / CH times, not once per small tile.
//  A. Every lane follows its stream's range chain over all C channels,
//     recording the range at its own block's start and the shift totals at
//     every block boundary.
//  B. Lane q codes channels [q B, q B + B) with the full coder from low = 0,
//     its shifted-out bytes going straight to their stream positions in the
//     stream's slot (contiguous here, one unaligned dword store per flush).
//     A chunk holds CH / 4 channels of each of the four blocks.
//  C. After a barrier, lane 0 of the quad adds the blocks' lows and the final
//     0xFFFFFF and trims: the stream's bytes and length are those of k_encode.
// Slots: stream j of slot region grp at slots + (grp * 256 + j) * slot_bytes.
// Needs A even, C % CH == 0, CH % 64 == 0, CH * A / 2 <= 256 * PERC.
template <int PERC>
__global__ __launch_bounds__(256) void k_encode_split(const uint8_t *__restrict__ sym,
                                                      const uint16_t *__restrict__ cdf,
                                                      uint8_t *__restrict__ slots,
                                                      uint16_t *__restrict__ stream_len, KParams p, int CH,
                                                      int32_t *status)
{
    constexpr int SPB = 64;  // streams per block
    constexpr int GB = 4;    // blocks per slot region
    extern __shared__ uint32_t lds[];
    __shared__ uint32_t s_tot[4];
    const int bps = (p.Tc + 255) / 256;
    const int64_t bl = xcd_block(blockIdx.x, gridDim.x);  // a slab's blocks share an XCD
    const int64_t grp = bl / GB;
    const int sub = (int)(bl - grp * GB);
    const int64_t slab = grp / bps;
    const int tb = (int)(grp - slab * bps);
    const SlabGeom g = slab_geom(p, slab);
    const int r0 = tb * 256 + sub * SPB;  // the block's first token
    // the block's payload bytes go to the last 4 bytes of its first stream's
    // slot, which no stream reaches (at most 2C + 4 of round_up(2C + 16, 16))
    uint32_t *const btot =
        (uint32_t *)(slots + ((int64_t)grp * 256 + sub * SPB + 1) * p.slot_bytes - 4);
    if (r0 >= g.nj) {  // uniform
        if (threadIdx.x == 0) *btot = 0;
        return;
    }
    const int lane = (int)threadIdx.x & 63, wid = (int)threadIdx.x >> 6;
    const int qd = lane & 3;                // this lane's block of channels
    const int jj = wid * 16 + (lane >> 2);  // stream within the block
    const int t = r0 + jj;
    const bool active = t < g.nj;
    const int C = p.C, A = p.A, B = C / 4, CQ = CH / 4, half = A / 2;
    const uint32_t *rows = (const uint32_t *)(cdf + g.tab * C * A);  // A even: rows of A / 2 dwords
    const int P = CH * half, B2 = B * half;                           // pairs per chunk, per block
    uint8_t *const myslot = slots + ((int64_t)grp * 256 + sub * SPB + jj) * p.slot_bytes;
    const int sst = C + 16;  // symbol row stride (bytes)
    lds_u8 *const stab = (lds_u8 *)lds;                        // [64][C + 16] symbols
    lds_u32 *const ptab = (lds_u32 *)lds + 16 * sst;           // [CH][A] (start, frequency) pairs

    // chunks of CH channels of pairs, each loaded into registers one chunk
    // ahead of its use and stored to the table between two barriers
    const int NA = C / CH, NM = 2 * NA;
    uint32_t last = 0;  // pair e = threadIdx.x + 256 i ends its row: (e + 1) % half == 0
    {
        const int step = 256 % half;
        int rem = ((int)threadIdx.x + 1) % half;
#pragma unroll
        for (int i = 0; i < PERC; ++i) {
            last |= (rem == 0 ? 1u : 0u) << i;
            rem += step;
            rem -= rem >= half ? half : 0;
        }
    }
    ChunkPairs<PERC> cp;
    // the symbols of the block's 64 streams, 16-byte pieces, 16 per thread in
    // flight, with the first pair chunk
    uint32_t badsym = 0;  // some staged symbol byte is >= A
    {
        // the block's rows are contiguous in sym: piece k is bytes [16 k, 16 k
        // + 16) from its first row, row k / per_row of the table
        const int per_row = C / 16, npieces = SPB * per_row;
        const int nvalid = (g.nj - r0 < SPB ? g.nj - r0 : SPB) * per_row;
        const uint32_t mrow = 0xFFFFFFFFu / (uint32_t)per_row + 1u;  // npieces * per_row < 2^32
        const uint8_t *src = sym + (g.row0 + r0) * C;
        cp.load(rows, 0, NA, P, B2, last);
        for (int base = 0; base < npieces; base += 256 * 16) {
            u32x4 v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int k = base + (int)threadIdx.x + 256 * i;
                v[i] = k < nvalid ? *(const u32x4 *)(src + (int64_t)k * 16) : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int k = base + (int)threadIdx.x + 256 * i;
                const int r = (int)div_by_mulhi((uint32_t)k, mrow);
                if (k < npieces) *(lds_u32x4 *)(stab + k * 16 + r * 16) = v[i];
            }
#pragma unroll
            for (int i = 0; i < 16; ++i)
                badsym |= kvc_bytes_ge(v[i].x, (uint32_t)A) |
                          kvc_bytes_ge(v[i].y, (uint32_t)A) | kvc_bytes_ge(v[i].z, (uint32_t)A) |
                          kvc_bytes_ge(v[i].w, (uint32_t)A);
        }
    }
    // This lane's symbols [c, c + n) (c, n multiples of 16) and their pairs
    // from the table rows at trow, 8 at a time: the next 8 lookups (and the
    // symbols two groups of 16 ahead) are in flight while `use` runs on the
    // current 8, so the coder waits on LDS only at a run's start.  grp(g) runs before the
    // symbols [c + g, c + g + 16) are used.
    const lds_u8 *my = stab + jj * sst;
    const uint32_t amax = (uint32_t)A - 1u;
    auto look8 = [&](uint32_t lo, uint32_t hi, const lds_u32 *t, uint32_t(&pv)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t sy = min(((i < 4 ? lo : hi) >> (8 * (i & 3))) & 0xFFu, amax);
            pv[i] = t[i * A + sy];
        }
    };
    auto run_pairs = [&](int c, int n, const lds_u32 *trow, auto &&grp, auto &&use) {
        u32x4 s0 = *(const lds_u32x4 *)(my + c);
        u32x4 s1 = *(const lds_u32x4 *)(my + c + (16 < n ? 16 : 0));
        uint32_t pa[8], pb[8];
        look8(s0.x, s0.y, trow, pa);
        for (int g = 0; g < n; g += 16) {
            // groups past the run read its last group again
            const int gn = g + 16 < n ? g + 16 : g, gnn = g + 32 < n ? g + 32 : n - 16;
            const u32x4 s2 = *(const lds_u32x4 *)(my + c + gnn);
            look8(s0.z, s0.w, trow + (g + 8) * A, pb);
            // the lookups above are issued before any use of pa[] below
            __asm__ volatile("" : "+v"(pa[0])::"memory");
            grp(g);
#pragma unroll
            for (int i = 0; i < 8; ++i) use(pa[i]);
            look8(s1.x, s1.y, trow + gn * A, pa);
            __asm__ volatile("" : "+v"(pb[0])::"memory");
#pragma unroll
            for (int i = 0; i < 8; ++i) use(pb[i]);
            s0 = s1;
            s1 = s2;
        }
    };

    // ---- A: the range chain up to the last block's start (the last block's
    // own chain runs inside its coder in B)
    const int CA = 3 * B, NAA = (CA + CH - 1) / CH;  // channels, chunks
    uint32_t range = 0xFFFFFFFFu, S = 0, rq = 0, S1 = 0, S2 = 0;
    for (int m = 0; m < NAA; ++m) {
        const int c0 = m * CH;
        __syncthreads();  // every wave is done with the previous chunk
        cp.store(ptab, P, last, 0);
        __syncthreads();
        cp.load(rows, m + 1 < NAA ? m + 1 : NA, NA, P, B2, last);
        if (active)
            run_pairs(
                c0, CA - c0 < CH ? CA - c0 : CH, ptab,
                [&](int g) {
                    // block boundaries fall on multiples of 16 channels
                    const int cg = c0 + g;
                    if (cg == B) S1 = S;
                    if (cg == 2 * B) S2 = S;
                    rq = cg == qd * B ? range : rq;
                },
                [&](uint32_t pr) { S += enc_range_step(range, pr >> 16); });
    }
    const uint32_t S3 = S;
    rq = qd == 3 ? range : rq;

    // ---- B: each lane codes its block
    EncState e;
    enc_init(e);
    e.range = rq;
    const uint32_t Sg = qd == 0 ? 0u : qd == 1 ? S1 : qd == 2 ? S2 : S3;
    uint8_t *const bslots = slots + ((int64_t)grp * 256 + sub * SPB) * p.slot_bytes;
    const SplitOutBuf out{{myslot, Sg / 8u},
                          __builtin_amdgcn_make_buffer_rsrc(bslots, (short)0, (int)(SPB * p.slot_bytes), 0x00020000),
                          (uint32_t)(jj * p.slot_bytes)};
    for (int m = NA; m < NM; ++m) {
        const int j0 = (m - NA) * CQ;
        __syncthreads();
        cp.store(ptab, P, last, KVC_SPLIT_SKEW);
        __syncthreads();
        if (m + 1 < NM) cp.load(rows, m + 1, NA, P, B2, last);
        if (active)
            run_pairs(qd * B + j0, CQ, ptab + qd * (CQ * A + KVC_SPLIT_SKEW), [](int) {},
                      [&](uint32_t pr) { enc_pair_nb(e, pr, out); });
    }
    // the bits shifted out of the whole stream: those before the last block
    // and those the last block's coder shifted (its written dwords and
    // pending bits)
    const uint32_t SC = (uint32_t)__shfl((int)(Sg + 32u * e.w + e.kb), (lane & ~3) + 3, 64);
    if (active) {
        enc_block_end(e, out);
        if (qd == 3)
            for (uint32_t b = 0; b < 4u; ++b) *out.byte(SC / 8u + b) = (uint8_t)(e.lo >> (24u - 8u * b));
    }
    // ---- C: the lows added, 0xFFFFFF added, the tail trimmed (lane 0 of the quad)
    const int qbase = lane & ~3;
    const uint32_t lo0 = (uint32_t)__shfl((int)e.lo, qbase, 64);
    const uint32_t lo1 = (uint32_t)__shfl((int)e.lo, qbase + 1, 64);
    const uint32_t lo2 = (uint32_t)__shfl((int)e.lo, qbase + 2, 64);
    __syncthreads();  // every block's bytes are in the slot
    uint32_t len = 0;
    if (active && qd == 0) {
        split_add(out, S1 / 8u, lo0, 4);
        split_add(out, S2 / 8u, lo1, 4);
        split_add(out, S3 / 8u, lo2, 4);
        const uint32_t nt = SC / 8u + 4u;
        split_add(out, nt - 3u, 0xFFFFFFu, 3);
        len = split_trim(out, nt - 3u);
        stream_len[g.sid0 + t] = (uint16_t)len;
    }
    len = wave_sum_u32(len);
    if (lane == 0) s_tot[wid] = len;
    __syncthreads();
    if (threadIdx.x == 0) *btot = s_tot[0] + s_tot[1] + s_tot[2] + s_tot[3];
    if (badsym) kvc_flag(status, KVC_DEV_BAD_SYMBOL);
}

// k_pack for slots holding each stream contiguously (k_encode_split): a wave
// per 16 streams of a slot region finds their payload offsets as k_pack does,
// then copies them in rounds of 64 dwords: lane j first loads dword j of all
// 16 streams (aligned loads, all in flight at once), then stores them one
// stream after the other at their byte offsets (unaligned dword stores; the
// last len % 4 bytes as byte stores).  Nothing is written at or past
// payload_cap.
template <bool FUSED>
__global__ __launch_bounds__(64) void k_pack_flat(const uint8_t *__restrict__ slots,
                                                  const uint16_t *__restrict__ stream_len,
                                                  uint64_t *__restrict__ slab_off,
                                                  uint8_t *__restrict__ payload, int64_t payload_cap,
                                                  KParams p, int32_t *status)
{
    constexpr int SPW = 16, WPR = 256 / SPW;
    const int bps = (p.Tc + 255) / 256;
    const int64_t eb = blockIdx.x / WPR;  // slot region
    const int wq = (int)(blockIdx.x - eb * WPR);
    const int64_t slab = eb / bps;
    const int tb = (int)(eb - slab * bps);
    const SlabGeom g = slab_geom(p, slab);
    const int lane = (int)threadIdx.x;
    const int t0 = tb * 256 + wq * SPW;
    if (t0 >= g.nj) return;
    const int t = t0 + lane;
    const bool active = lane < SPW && t < g.nj;
    uint32_t pre = 0;
    for (int i = lane; i < t0; i += 64) pre += stream_len[g.sid0 + i];
    pre = wave_sum_u32(pre);
    const uint32_t len = active ? stream_len[g.sid0 + t] : 0u;
    uint32_t incl = len;
    for (int off = 1; off < 64; off <<= 1) {
        uint32_t v = (uint32_t)__shfl_up((int)incl, off, 64);
        if (lane >= off) incl += v;
    }
    uint64_t base;  // the slab's first payload byte
    if constexpr (FUSED) {
        // the totals k_encode_split left per encoder block (4 per slot region, in
        // payload order): those of earlier slabs; the wave of block 0 also writes
        // the grand total and checks it against the capacity
        auto btot = [&](int64_t b) {
            return (uint64_t) * (const uint32_t *)(slots + ((b >> 2) * 256 + (b & 3) * 64 + 1) * p.slot_bytes - 4);
        };
        uint64_t acc = 0;
        for (int64_t b = lane; b < slab * bps * 4; b += 64) acc += btot(b);
        base = wave_sum_u64(acc);
        if (tb == 0 && wq == 0 && lane == 0) slab_off[slab] = base;
        if (blockIdx.x == 0) {
            uint64_t all = 0;
            for (int64_t b = lane; b < p.n_slabs * bps * 4; b += 64) all += btot(b);
            all = wave_sum_u64(all);
            if (lane == 0) {
                slab_off[p.n_slabs] = all;
                if (all > (uint64_t)payload_cap) kvc_flag(status, KVC_DEV_PAYLOAD_OVERFLOW);
            }
        }
    } else {
        base = slab_off[slab];
    }
    const uint64_t o = base + pre + incl - len;
    const uint32_t olo = (uint32_t)o, ohi = (uint32_t)(o >> 32);
    const uint64_t cap = (uint64_t)payload_cap;
    const uint8_t *src0 = slots + ((int64_t)eb * 256 + wq * SPW) * p.slot_bytes;
    const int ndw_max = (int)((wave_max_u32(len) + 3u) >> 2);
    // rounds of 64 dwords: each lane loads dword 64r + lane of all SPW streams first
    for (int k0 = 0; k0 < ndw_max; k0 += 64) {
        const uint32_t j = (uint32_t)(k0 + lane);
        uint32_t v[SPW];
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const uint32_t len_i = (uint32_t)__builtin_amdgcn_readlane((int)len, i);
            v[i] = 4u * j < len_i ? ((const uint32_t *)(src0 + (int64_t)i * p.slot_bytes))[j] : 0u;
        }
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const uint32_t len_i = (uint32_t)__builtin_amdgcn_readlane((int)len, i);
            if (4u * j >= len_i) continue;
            const uint64_t o_i = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)ohi, i) << 32) |
                                 (uint32_t)__builtin_amdgcn_readlane((int)olo, i);
            const uint64_t b = o_i + 4u * j;
            const uint32_t nb = min(len_i - 4u * j, 4u);
            if (nb == 4u && b + 4u <= cap) {
                __builtin_memcpy(payload + b, &v[i], 4);
            } else {
                for (uint32_t q = 0; q < nb; ++q)
                    if (b + q < cap) payload[b + q] = (uint8_t)(v[i] >> (8u * q));
            }
        }
    }
}

__global__ void k_zero_u64(uint64_t *dst) { *dst = 0; }

}  // namespace

// Launches of at most this many streams stage wider CDF tiles.
constexpr int64_t KVC_ENC_WIDE_MAX_STREAMS = 32768;
// Launches of at most this many streams code 16 streams per wave, others 64.
constexpr int64_t KVC_ENC_SPARSE_MAX_STREAMS = 16384;
// Launches of at most this many streams pack 16 streams per wave, others 64.
constexpr int64_t KVC_PACK_SPARSE_MAX_STREAMS = 16384;

// Runs of (layer, K|V) pairs encoded with only the first entries of each CDF
// row staged take at least this many blocks, else they stage whole rows.
constexpr int64_t KVC_ENC_RUN_MIN_BLOCKS = 4096;

// Depth n (rows staged to 2^n entries) for (layer, K|V) lk: that of its bins,
// at least 3 and at most the table's (nfull); nfull when may_cut is false.
static int enc_run_nstep(const KParams &p, int lk, int nfull, bool may_cut)
{
    if (!may_cut) return nfull;
    const int bins = 2 * ((int)p.maxq[lk] + 1);
    int n = (int)cdf_nstep((uint32_t)bins);
    if (n < 3) n = 3;
    return n < nfull ? n : nfull;
}

// Symbol tile width: 128 channels, the whole 128-byte line of each token row
// of 1024 channels, so every line of the symbols is read from memory once.
// (64-channel tiles read each line twice, its halves a tile apart with the
// first copy gone from L2 in between: 16.4 GB read for 9.8 GB of symbols and
// tables at the 34B 80K shape, against 9.8 GB now.)
constexpr int ENC_SYMBOL_TILE = 128;

// Streams coded per wave.
static int enc_streams_per_wave(int64_t n_streams) { return n_streams <= KVC_ENC_SPARSE_MAX_STREAMS ? 16 : 64; }

// Launches of at most this many streams code each stream with a quad of lanes
// (k_encode_split) where the shape allows it.
constexpr int64_t KVC_ENC_SPLIT_MAX_STREAMS = 16384;

// Split launches of at most this many encoder blocks take their slab offsets
// from k_pack_flat (each pack wave sums the block totals before its slab)
// instead of k_slab_sum and k_scan.
constexpr int64_t KVC_PACK_FUSED_MAX_BLOCKS = 1024;

// k_encode_split's pair chunk (channels) and dynamic LDS for this shape, or
// 0 when the shape does not take it: C % 64 == 0, A <= 64, a power-of-two
// chunk of at least 64 channels dividing C with at most 32 KB of pairs, and
// the 64 streams' symbols plus one chunk within the device's LDS per block.
static int enc_split_chunk(const KParams &p, size_t *lds)
{
    if (p.C % 64 != 0 || p.A > 64 || p.A % 2 != 0) return 0;
    int ch = 64;
    while (2 * ch <= p.C / 2 && 2 * ch * p.A * 4 <= 32768 && p.C % (2 * ch) == 0) ch *= 2;
    if (p.C % ch != 0 || ch * p.A * 4 > 32768) return 0;
    const size_t bytes = 64 * (size_t)(p.C + 16) + ((size_t)ch * p.A + 3 * KVC_SPLIT_SKEW) * sizeof(uint32_t);
    int dev = 0, lim = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        bytes > (size_t)lim)
        return 0;
    *lds = bytes;
    return ch;
}

// Channels per tile (a power of two, 16 to the symbol tile width).  With few
// streams a tile of 16 channels is coded in less time than its successor's
// rows take to arrive from memory, so small launches stage up to 128
// channels (up to 8 pairs per thread); large ones keep the tile at one or two
// pairs per thread.
static int enc_tile_channels(int A, int64_t n_streams)
{
    const int sw = ENC_SYMBOL_TILE;
    int ct = 16;
    if (n_streams <= KVC_ENC_WIDE_MAX_STREAMS)
        while (ct < sw && 2 * ct * (A / 2) <= 8 * 256) ct *= 2;
    else
        while (ct < sw && 2 * ct * A <= 1024) ct *= 2;
    return ct;
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
    const int64_t regions = bps * p.n_slabs;  // slot regions: 256 tokens of one slab
    const int spw = enc_streams_per_wave(p.n_streams);
    size_t lds_split = 0;
    const int ch = (vec16 && p.n_streams <= KVC_ENC_SPLIT_MAX_STREAMS) ? enc_split_chunk(p, &lds_split) : 0;
    if (ch > 0) {
        const void *fn = (const void *)k_encode_split<16>;
        if (lds_split > 65536) {
            const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)lds_split);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL((k_encode_split<16>), dim3((unsigned)(regions * 4)), dim3(256), lds_split, stream,
                           sym, cdf, slots, stream_len, p, ch, status);
        if (regions * 4 <= KVC_PACK_FUSED_MAX_BLOCKS) {
            // the slab offsets come out of the pack itself, from the encoder's block totals
            hipLaunchKernelGGL(k_pack_flat<true>, dim3((unsigned)(regions * 16)), dim3(64), 0, stream, slots,
                               stream_len, slab_off, payload, payload_cap, p, status);
        } else {
            hipLaunchKernelGGL(k_slab_sum, dim3((unsigned)p.n_slabs), dim3(256), 0, stream, stream_len,
                               slab_total, p);
            hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, stream, slab_total, slab_off, p.n_slabs,
                               payload_cap, (const uint64_t *)nullptr, status);
            hipLaunchKernelGGL(k_pack_flat<false>, dim3((unsigned)(regions * 16)), dim3(64), 0, stream, slots,
                               stream_len, slab_off, payload, payload_cap, p, status);
        }
        return hipGetLastError();
    }
    // One launch per run of (layer, K|V) pairs whose symbols fit the same
    // power-of-two prefix of the CDF rows, as in the decoder: a run of layers
    // with fewer bins than the table's rows stages only the first 2^n entries
    // of each row (symbols of b bins run to b - 2), so that its tiles hold more
    // channels in the same LDS and fewer barriers pass per symbol.  A symbol at
    // or past the staged entries sets the redo bit; a guard launch over whole
    // rows follows any cut run and encodes everything again when the bit is set
    // (k_scan clears it).  Without a status word, or for runs of fewer than
    // KVC_ENC_RUN_MIN_BLOCKS blocks, whole rows.
    const int LK = 2 * p.L;
    const int nfull = (int)cdf_nstep((uint32_t)p.A);
    int run_n[2 * KVC_MAX_LAYERS];  // each (layer, K|V)'s depth
    for (int lk = 0; lk < LK;) {
        const int n = enc_run_nstep(p, lk, nfull, status != nullptr);
        int lk1 = lk + 1;
        while (lk1 < LK && enc_run_nstep(p, lk1, nfull, status != nullptr) == n) ++lk1;
        const bool small = (int64_t)(lk1 - lk) * p.NC * bps * (64 / spw) < KVC_ENC_RUN_MIN_BLOCKS;
        for (int k = lk; k < lk1; ++k) run_n[k] = small ? nfull : n;
        lk = lk1;
    }
    bool cut = false;
    for (int lk0 = 0; lk0 <= LK;) {
        const bool guard_pass = lk0 == LK;  // after the runs: the guard launch
        if (guard_pass && !cut) break;
        const int n0 = guard_pass ? nfull : run_n[lk0];
        int lk1 = guard_pass ? LK + 1 : lk0 + 1;
        while (lk1 < LK && run_n[lk1] == n0) ++lk1;
        const int A_st = n0 < nfull ? (1 << n0) : p.A;  // entries staged per row
        cut = cut || A_st < p.A;
        const int nlk = guard_pass ? LK : lk1 - lk0, lkb = guard_pass ? 0 : lk0, guard = guard_pass ? 1 : 0;
        const int CT = enc_tile_channels(A_st, p.n_streams);
        const size_t lds_pairs = (size_t)CT * A_st * sizeof(uint32_t);
        const int per = (CT * (A_st / 2) + 255) / 256;  // pairs staged per thread
        const dim3 grid((unsigned)(bps * (int64_t)nlk * p.NC * (64 / spw)));
        const bool pre4 = (A_st & (A_st - 1)) == 0 && A_st <= 64;  // symbols staged as pair byte offsets
#define KVC_ENC(V, P, S, W, L)                                                                       \
    hipLaunchKernelGGL((k_encode<V, P, S, W>), grid, dim3(256), L, stream, sym, cdf, slots, stream_len, \
                       p, CT, status, A_st, lkb, nlk, guard)
#define KVC_ENC4(P, S, W, L)                                                                         \
    hipLaunchKernelGGL((k_encode<true, P, S, W, true>), grid, dim3(256), L, stream, sym, cdf, slots,    \
                       stream_len, p, CT, status, A_st, lkb, nlk, guard)
#define KVC_ENC_S(S, W)                                                                              \
    {                                                                                                \
        const size_t lds_syms = lds_pairs + 4 * W * (size_t)(S + 16);                                \
        if (vec16 && pre4) {                                                                         \
            if (per <= 2) KVC_ENC4(2, S, W, lds_syms);                                               \
            else KVC_ENC4(8, S, W, lds_syms);                                                        \
        } else if (vec16) {                                                                          \
            if (per <= 2) KVC_ENC(true, 2, S, W, lds_syms);                                          \
            else KVC_ENC(true, 8, S, W, lds_syms);                                                   \
        } else {                                                                                     \
            if (per <= 2) KVC_ENC(false, 2, S, W, lds_pairs);                                        \
            else KVC_ENC(false, 8, S, W, lds_pairs);                                                 \
        }                                                                                            \
    }
        if (spw == 16)
            KVC_ENC_S(ENC_SYMBOL_TILE, 16)
        else
            KVC_ENC_S(ENC_SYMBOL_TILE, 64)
#undef KVC_ENC_S
#undef KVC_ENC4
#undef KVC_ENC
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        lk0 = lk1;
    }
    hipLaunchKernelGGL(k_slab_sum, dim3((unsigned)p.n_slabs), dim3(256), 0, stream, stream_len,
                       slab_total, p);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, stream, slab_total, slab_off, p.n_slabs,
                       payload_cap, (const uint64_t *)nullptr, status);
    if (p.n_streams <= KVC_PACK_SPARSE_MAX_STREAMS)
        hipLaunchKernelGGL(k_pack<16>, dim3((unsigned)(regions * 16)), dim3(64), 0, stream, slots,
                           stream_len, slab_off, payload, payload_cap, p);
    else
        hipLaunchKernelGGL(k_pack<64>, dim3((unsigned)(regions * 4)), dim3(64), 0, stream, slots,
                           stream_len, slab_off, payload, payload_cap, p);
    return hipGetLastError();
}

hipError_t launch_slab_offsets(const uint16_t *stream_len, uint64_t *slab_off, const KParams &p,
                               const uint64_t *expect, int32_t *status, hipStream_t stream)
{
    if (p.n_slabs == 0) return launch_zero_u64(slab_off, stream);
    // the slab totals go into slab_off itself, then are scanned in place
    hipLaunchKernelGGL(k_slab_sum, dim3((unsigned)p.n_slabs), dim3(256), 0, stream, stream_len,
                       slab_off, p);
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, stream, slab_off, slab_off, p.n_slabs,
                       (int64_t)0, expect, status);
    return hipGetLastError();
}
