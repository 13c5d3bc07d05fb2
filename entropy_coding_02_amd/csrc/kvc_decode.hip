// kvc_decode.hip - parallel range decoding with fused dequantization
// ([CG] 2.4 steps 1-2), and dequantization on its own.
//
// k_decode: one lane per stream, 256 tokens of one slab per block.  The block
// finds its streams' payload offsets (slab offset + exclusive scan of the
// stream lengths), builds the slab's dequantization table
//     lut[q] = fp32(q - MAX) / MAX        (one IEEE division per entry)
// in LDS, and each lane then decodes its C symbols: a binary search of the
// channel's CDF row for the largest k with r*cdf_k <= code, the interval
// update, byte refill, and y = lut[s] * max1 written as fp16 or fp32 (lut[s]
// is staged next to each (start, frequency) pair, so one read gives both).
// Because fl(fl(q - MAX) / MAX) is exactly the table entry, the fused output
// equals the separate dequantization bit for bit.
//
// k_decode_group: launches of few streams, G lanes per stream splitting each
// symbol's search over rows of (start, frequency) keys (comment at the kernel).
#include <mutex>

#include "kvc_common.h"
#include "kvc_kernels.h"
#include "lane_coder.h"
#include "pair_tile.h"

// Launches of at most this many streams decode with a group of lanes per
// stream (k_decode_group), for rows of 8 to 64 entries.
constexpr int64_t KVC_DEC_GROUP_MAX_STREAMS = 16384;
// Lanes per stream there for rows of 16 or 32 entries (4 or 8; 64-entry rows use 8).
constexpr int64_t KVC_DEC_GROUP_LANES = 4;

// Record dwords per channel of k_decode_mode: ModeRec and the block heads.
#define DEC_MODE_RS(NSTEP) ((NSTEP) <= 5 ? 8 : 12)
// Pairs each thread stages per tile of k_decode_mode: the tile's CT * A / 2
// pairs over 256 threads (CT = dec_mode_tile_channels: CT * P2 = 1024, and
// 32 channels of 64-entry rows).
#define DEC_MODE_PER(NSTEP) ((NSTEP) == 6 ? 4 : 2)

namespace {

enum { ODT_F16 = 0, ODT_F32 = 1 };

// A lane's 17 byte-ring slots for WinIn in k_decode_mode, slot i at
// p[(16 - i) * 256] (p: the lane's slot 16): the block's 256 lanes keep slot i
// side by side, so a wave's reads of any mix of slots fall in distinct banks,
// and slot i + 1 lies just below slot i, so one two-dword read (lower address
// first) returns (slot i + 1, slot i): the window's 64 bits already in
// register order.
struct LaneRing {
    lds_u32 *p;
    __device__ lds_u32 &operator[](uint32_t i) const { return p[(16u - i) * 256u]; }
};
// what k_decode writes: a compile-time set, so every store in the symbol loop
// is unconditional and the loads of the byte feed never wait for them
enum { OUT_F16 = 1, OUT_F32 = 2, OUT_SYM = 4 };

// BLK: the two-level table search (two dependent LDS reads per symbol
// instead of NSTEP, a few more VALU operations).
template <bool VEC, int OUT, int NSTEP, bool BLK, bool PAD = true>
__global__ __launch_bounds__(256) void k_decode(const uint8_t *__restrict__ payload,
                                                int64_t payload_bytes,
                                                const uint64_t *__restrict__ slab_off,
                                                const uint16_t *__restrict__ stream_len,
                                                const uint16_t *__restrict__ cdf,
                                                const uint16_t *__restrict__ max1,
                                                uint8_t *__restrict__ sym_out, void *__restrict__ out,
                                                KParams p, int32_t *status, int CT)
{
    // LDS: lut[256] f32 | ring[256][17] u32 | rows16 [CT][P2] u16 | (pair, lut) [CT][A] u32x2
    extern __shared__ uint32_t lds[];
    __shared__ uint32_t s_red[4];
    constexpr uint32_t P2 = 1u << NSTEP;  // search row length: A padded to a power of two
    const int C = p.C, A = p.A;
    float *lut = (float *)lds;
    lds_u32 *const ring = (lds_u32 *)(lds + 256) + threadIdx.x * 17u;
    const int n16 = (CT * (int)P2 + 1) / 2;
    lds_u32 *const tile = (lds_u32 *)(lds + 256 + 256 * 17);
    lds_u16 *const r16 = (lds_u16 *)tile;
    lds_u32 *const pr = tile + n16;

    const int bps = (p.Tc + 255) / 256;
    const int64_t slab = blockIdx.x / bps;
    const int tb = (int)(blockIdx.x - slab * bps);
    const int t = tb * 256 + (int)threadIdx.x;
    const SlabGeom g = slab_geom(p, slab);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const bool active = t < g.nj;

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
    const uint32_t len = active ? stream_len[g.sid0 + t] : 0u;
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
    // padding of the search rows (never rewritten by the tile stores)
    if (P2 > (uint32_t)A)
        for (int e = threadIdx.x; e < CT * (int)P2; e += 256)
            if ((uint32_t)(e & (P2 - 1)) >= (uint32_t)A) r16[e] = 0xFFFFu;
    __syncthreads();
    uint32_t wbase = 0;
    for (int i = 0; i < wid; ++i) wbase += s_red[i];

    const int64_t row = g.row0 + (active ? t : 0);
    const uint64_t off = active ? slab_off[slab] + pre + wbase + incl - len : 0;
    RingIn<lds_u32 *> in;
    in.init(payload, off, len, (uint64_t)payload_bytes, ring);
    DecState d;
    dec_init(d, in);
    constexpr int ODT = (OUT & OUT_F16) ? ODT_F16 : (OUT & OUT_F32) ? ODT_F32 : -1;
    constexpr int PER = NSTEP >= 7 ? 8 : 2;  // pairs staged per thread: CT * A / 2 / 256
    const float m = (ODT >= 0) ? kvc_h2f(max1[row]) : 0.0f;
    uint32_t bad = 0;
    uint8_t *so = (OUT & OUT_SYM) ? sym_out + row * C : nullptr;
    const uint16_t *srows = cdf + g.tab * C * A;
    const int ntiles = (C + CT - 1) / CT;
    // search the row, then one 8-byte read: the symbol's (start, frequency) and
    // its dequantization value lv
    auto decode1 = [&](int cl, float &lv) -> uint32_t {
        const uint32_t r = d.range >> 16;
        uint32_t s;
        if constexpr (BLK) {
            const lds_u16 *rowp = r16 + cl * P2;
            auto piece = [&](uint32_t b) -> kvc_u32x4 { return *(const lds_u32x4 *)(rowp + 8u * b); };
            s = cdf_search_blocks<NSTEP, PAD>(rowp, piece, (uint32_t)A, r, d.code);
        } else {
            s = cdf_search<NSTEP>(r16 + cl * P2, (uint32_t)A, r, d.code);
        }
        const lds_u32 *prow = pr + 2 * cl * A;  // uniform: the address is one shift-add of s
        const u32x2 e = *(const lds_u32x2 *)(prow + 2 * s);
        bad |= dec_advance(d, r, e.x & 0xFFFFu, e.x >> 16);
        lv = __uint_as_float(e.y);
        return s;
    };

    // the tile's rows arrive in registers while the previous tile is decoded,
    // and go into LDS between two barriers
    PairTile<PER> pt;
    // fp16 output of a 32-channel block (VEC path)
    uint32_t hw[16];
    auto put_f16 = [&](int cb, int nb) {
        uint4 *o = (uint4 *)((uint16_t *)out + row * C + cb);
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
            if (gi * 8 < nb) o[gi] = make_uint4(hw[4 * gi], hw[4 * gi + 1], hw[4 * gi + 2], hw[4 * gi + 3]);
    };
    pt.load(srows, 0, CT, C, A);
    for (int it = 0; it < ntiles; ++it) {
        const int c0 = it * CT, c1 = min(C, c0 + CT);
        __syncthreads();  // all waves are done with the previous tile
        pt.store_with(pr, CT, A, r16, (int)P2, (const uint32_t *)lut);
        __syncthreads();
        if (it + 1 < ntiles) pt.load(srows, c0 + CT, CT, C, A);
        if (!active) continue;
        if constexpr (VEC) {
            // C % 16 == 0 and CT % 16 == 0: groups of 8 symbols; the fp16 output of
            // up to 32 channels (64 bytes of the row) is collected in registers and
            // written with back-to-back 16-byte stores, so whole 64-byte pieces of
            // a line reach L2 together instead of 16-byte fragments.
            for (int cb = c0; cb < c1; cb += 32) {
                const int nb = min(32, c1 - cb);  // 16 or 32
                float fw[8];
#pragma unroll
                for (int gi = 0; gi < 4; ++gi) {
                    if (gi * 8 >= nb) break;
                    const int cg = cb + gi * 8;
                    in.group();
                    uint32_t sw[2] = {0, 0};
                    float ylo = 0.0f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        if ((i & 1) == 0) dec_refill(d, in);
                        float lv;
                        const uint32_t s = decode1(cg - c0 + i, lv);
                        sw[i >> 2] |= s << (8 * (i & 3));
                        if constexpr (ODT >= 0) {
                            const float y = lv * m;
                            if constexpr (ODT == ODT_F16) {
                                if (i & 1)
                                    hw[gi * 4 + (i >> 1)] = kvc_f2h2(ylo, y);
                                else
                                    ylo = y;
                            } else {
                                fw[i] = y;
                            }
                        }
                    }
                    if constexpr ((OUT & OUT_SYM) != 0) *(uint2 *)(so + cg) = make_uint2(sw[0], sw[1]);
                    if constexpr (ODT == ODT_F32) {
                        float4 *o = (float4 *)((float *)out + row * C + cg);
                        o[0] = make_float4(fw[0], fw[1], fw[2], fw[3]);
                        o[1] = make_float4(fw[4], fw[5], fw[6], fw[7]);
                    }
                }
                if constexpr (ODT == ODT_F16) put_f16(cb, nb);
            }
        } else {
            for (int c = c0; c < c1; ++c) {
                if ((c & 7) == 0) in.group();
                if ((c & 1) == 0) dec_refill(d, in);
                float lv;
                const uint32_t s = decode1(c - c0, lv);
                if constexpr ((OUT & OUT_SYM) != 0) so[c] = (uint8_t)s;
                if constexpr (ODT >= 0) {
                    const float y = lv * m;
                    if constexpr (ODT == ODT_F16)
                        ((uint16_t *)out)[row * C + c] = (uint16_t)kvc_f2h(y);
                    else
                        ((float *)out)[row * C + c] = y;
                }
            }
        }
    }

    if (active && bad) kvc_flag(status, KVC_DEV_CORRUPT);
}

// Mode-first decoding, one lane per stream (256 tokens of one slab per
// block), for rows of 8 to 64 entries.  Each tile's CDF rows are staged as
// (start, frequency) pairs and search rows, plus a record per channel
// (PairTile::store_mode): the row's one symbol of frequency above
// 65536 - KVC_MODE_SPAN, if it has one, with its start, frequency and
// dequantization value, and the row's block heads.  All 64 lanes of a wave
// decode the same channel at each step, so the record is one broadcast read.
// Every lane first tries the record's symbol: one multiply-add, one multiply
// and a compare, and if all lanes land inside its interval with no
// renormalisation due, that is the symbol (the row's only qualifying one on a
// non-decreasing row).  In most chunks of long contexts most channels hardly
// vary, so most symbols end there.  Otherwise the wave takes the exact
// two-level search with the heads from the record.  Renormalisation takes
// its bits from a 32-bit window at the stream's byte position (WinIn): no bit
// buffer to count or top up.
//
// Output: a lane writes its own token row.  The fp16 values of two 32-channel
// halves are collected in registers (the older half moved down as the next
// one starts) and stored as one 128-byte line, which keeps the HBM writes of
// ~250K concurrently written rows efficient.  Vector memory operations
// complete in order, so a load issued after a store cannot be waited for
// before the store is acknowledged: each half's first byte-feed load is
// issued before its stores, and the next tile's CDF rows are requested
// before them as well.
template <bool VEC, int OUT, int NSTEP, bool PAD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NSTEP <= 5 ? 4 : 3))) void k_decode_mode(
    const uint8_t *__restrict__ payload, int64_t payload_bytes, const uint64_t *__restrict__ slab_off,
    const uint16_t *__restrict__ stream_len, const uint16_t *__restrict__ cdf,
    const uint16_t *__restrict__ max1, uint8_t *__restrict__ sym_out, void *__restrict__ out, KParams p,
    int32_t *status, int CT, int A_st, int64_t sb0, int guard)
{
    // LDS: lut[256] f32 | ring[17][256] u32 | rec[2][CT][RS] u32 | rows16 [CT][P2] u16 |
    //      pairs [CT][A] u32 | output staging [4 waves][16 rows][36] u32
    extern __shared__ uint32_t lds[];
    __shared__ uint32_t s_red[4];
    constexpr uint32_t P2 = 1u << NSTEP;
    constexpr int NB = 1 << (NSTEP - 3);
    constexpr int RS = DEC_MODE_RS(NSTEP);
    constexpr int PER = DEC_MODE_PER(NSTEP);  // pairs staged per thread: CT * A / 2 / 256
    // A: the entries staged and searched per row; AR: the table's row length
    // (A < AR only on a launch over slabs whose symbols all lie below A - 1)
    const int C = p.C, A = A_st, AR = p.A;
    // the guard launch (after launches with A < AR) decodes only when one of
    // them found a stream inconsistent with its tables
    if (guard && (__atomic_load_n(status, __ATOMIC_RELAXED) & KVC_DEV_CORRUPT) == 0) return;
    float *lut = (float *)lds;
    const lds_u32 *const lutw = (const lds_u32 *)lds;
    const LaneRing ring{(lds_u32 *)(lds + 256) + threadIdx.x};  // slot i at [(16 - i) * 256]
    lds_u32 *const recs = (lds_u32 *)(lds + 256 + 256 * 17);
    lds_u32 *const tile = recs + 2 * CT * RS;
    const int n16 = (CT * (int)P2 + 1) / 2;
    lds_u16 *const r16 = (lds_u16 *)tile;
    lds_u32 *const pr = tile + n16;
    lds_u32 *const xs = pr + CT * A;  // output staging: per wave 16 rows of 36 dwords

    // blocks in memory order: consecutive blocks take consecutive chunks of one
    // (layer, K|V), whose output rows lie back to back, not the 2L slabs of one
    // chunk, which lie a whole (layer, K|V) apart: the rows written at the same
    // time then share DRAM pages
    const int bps = (p.Tc + 255) / 256;
    const int64_t sbl = blockIdx.x / bps;  // slab of the launch's range
    const int tb = (int)(blockIdx.x - sbl * bps);
    const int64_t sb = sb0 + sbl;
    const int64_t slab = (sb % p.NC) * (2 * (int64_t)p.L) + sb / p.NC;
    const int t = tb * 256 + (int)threadIdx.x;
    const SlabGeom g = slab_geom(p, slab);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const bool active = t < g.nj;

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
    const uint32_t len = active ? stream_len[g.sid0 + t] : 0u;
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
    // padding of the search rows and of the record heads (never rewritten by
    // the tile stores), and both record buffers' frequency words
    if (P2 > (uint32_t)A)
        for (int e = threadIdx.x; e < CT * (int)P2; e += 256)
            if ((uint32_t)(e & (P2 - 1)) >= (uint32_t)A) r16[e] = 0xFFFFu;
    for (int i = threadIdx.x; i < 2 * CT; i += 256) {
        recs[i * RS + 2] = 0u;
        for (int b = 1; b < NB; ++b)
            if (8 * b >= A) recs[i * RS + 3 + b] = 0xFFFFu;
    }
    __syncthreads();
    uint32_t wbase = 0;
    for (int i = 0; i < wid; ++i) wbase += s_red[i];

    const int64_t row = g.row0 + (active ? t : 0);
    const uint64_t off = active ? slab_off[slab] + pre + wbase + incl - len : 0;
    WinIn<LaneRing> in;
    uint32_t code = in.init(payload, off, len, (uint64_t)payload_bytes, ring);
    uint32_t range = 0xFFFFFFFFu;
    constexpr int ODT = (OUT & OUT_F16) ? ODT_F16 : (OUT & OUT_F32) ? ODT_F32 : -1;
    const float m = (ODT >= 0) ? kvc_h2f(max1[row]) : 0.0f;
    BadMask bad;
    uint8_t *so = (OUT & OUT_SYM) ? sym_out + row * C : nullptr;
    const uint16_t *srows = cdf + g.tab * C * AR;
    const int ntiles = (C + CT - 1) / CT;
    const lds_u32 *rec = recs;
    // the mode part of tile channel cl's record (a broadcast read: every lane
    // the same address), loaded one symbol ahead of its use
    using Rec = u32x4;
    auto load_rec = [&](int cl) -> Rec { return *(const lds_u32x4 *)(rec + cl * RS); };
    // one symbol of tile channel cl with its record's mode part ra; lvb
    // receives its dequantization value
    auto decode1 = [&](int cl, const lds_u32 *rc, const Rec &ra, uint32_t &lvb) -> uint32_t {  // rc: cl's record
        auto heads = [&](uint32_t *hd) {  // the exact path's block heads
            hd[0] = 0u;
            if constexpr (NB >= 2) {
                const u32x4 rb = *(const lds_u32x4 *)(rc + 4);
                hd[1] = rb.x;
                if constexpr (NB >= 4) {
                    hd[2] = rb.y;
                    hd[3] = rb.z;
                }
                if constexpr (NB >= 8) {
                    const u32x4 rd = *(const lds_u32x4 *)(rc + 8);
                    hd[4] = rb.w;
                    hd[5] = rd.x;
                    hd[6] = rd.y;
                    hd[7] = rd.z;
                }
            }
        };
        const ModeRec mr{ra.x, (int32_t)ra.y, ra.z, ra.w};
        const lds_u16 *rowp = r16 + cl * P2;
        auto piece = [&](uint32_t b) -> kvc_u32x4 { return *(const lds_u32x4 *)(rowp + 8u * b); };
        const lds_u32 *prow = pr + cl * A;  // uniform: the pair address is one shift-add of s
        auto ent = [&](uint32_t s) -> kvc_u32x2 { return kvc_u32x2{prow[s], lutw[s]}; };
        uint32_t fast;
        return dec_symbol_mode<NSTEP, PAD>(code, range, in, mr, heads, piece, ent, (uint32_t)A, bad, &fast,
                                           &lvb);
    };

    PairTile<PER> pt;
    // fp16 output: hw[0..15] the previous 32-channel half, hw[16..31] the
    // current one.  A pair of halves (128 bytes of each of the wave's 64 rows)
    // goes out through the wave's LDS slice, 16 rows at a time: those rows'
    // lanes write their pieces to LDS, then every lane stores one 16-byte piece,
    // 8 lanes per row, so each store writes 8 whole 128-byte lines (stored
    // straight from the lanes, one instruction would touch 64 lines, one L2
    // request each).  Every lane of the wave takes part, so lanes past the
    // slab's end decode too (an empty stream) and only rows before it are stored.
    uint32_t hw[32];
    const int wid_u = __builtin_amdgcn_readfirstlane(wid);  // uniform: the slice and rows live in SGPRs
    lds_u32 *const xw = xs + wid_u * 576;
    const int nact = __builtin_popcountll(__builtin_amdgcn_ballot_w64(active));  // active lanes: a prefix
    uint16_t *const wout = (uint16_t *)out + (g.row0 + (int64_t)tb * 256 + wid_u * 64) * C;  // the wave's first row
    auto put_rows = [&](auto piece, int npc, int cs, int nch) {  // pieces piece(q), q < npc; channels [cs, cs + nch)
#pragma unroll
        for (int pass = 0; pass < 4; ++pass) {
            if ((lane >> 4) == pass) {
                lds_u32 *const d = xw + (lane & 15) * 36;
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    if (q < npc) *(lds_u32x4 *)(d + 4 * q) = piece(q);
            }
            __asm__ volatile("" ::: "memory");  // a wave's LDS operations run in order: the reads see the writes
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int r = 8 * k + (lane >> 3), pc = lane & 7;
                const u32x4 v = *(const lds_u32x4 *)(xw + r * 36 + 4 * pc);
                const int wr = 16 * pass + r;
                if (wr < nact && pc * 8 < nch)
                    *(uint4 *)(wout + (uint32_t)(wr * C + cs + 8 * pc)) = make_uint4(v.x, v.y, v.z, v.w);
            }
            __asm__ volatile("" ::: "memory");  // the slice is read before the next pass writes it
        }
    };
    auto put_pair = [&](int cs, int nch) {  // channels [cs, cs + nch) from hw[0 ..]
        put_rows([&](int q) { return u32x4{hw[4 * q], hw[4 * q + 1], hw[4 * q + 2], hw[4 * q + 3]}; }, 8, cs, nch);
    };
    auto put_half = [&](int cs, int nch) {  // channels [cs, cs + nch) from hw[16 ..]
        put_rows([&](int q) { return u32x4{hw[16 + 4 * q], hw[17 + 4 * q], hw[18 + 4 * q], hw[19 + 4 * q]}; }, 4,
                 cs, nch);
    };
    const bool wave_on = nact > 0;
    pt.load(srows, 0, CT, C, A, AR);
    for (int it = 0; it < ntiles; ++it) {
        const int c0 = it * CT, c1 = min(C, c0 + CT);
        lds_u32 *const rnow = recs + (it & 1) * CT * RS;
        __syncthreads();  // all waves are done with the previous tile
        pt.store_mode(pr, CT, A, r16, (int)P2, (const uint32_t *)lut, rnow, recs + ((it + 1) & 1) * CT * RS, RS);
        __syncthreads();
        rec = rnow;
        if (it + 1 < ntiles) pt.load(srows, c0 + CT, CT, C, A, AR);
        if (!wave_on) continue;
        if constexpr (VEC) {
            // halves of 32 channels (CT is a multiple of 32; C of 16)
            for (int cb = c0; cb < c1; cb += 32) {
                const int nb = min(32, c1 - cb);  // 16 or 32
                in.group();                       // before the stores below
                if constexpr (ODT == ODT_F16) {
                    if ((cb & 63) == 0 && cb >= 64) put_pair(cb - 64, 64);
#pragma unroll
                    for (int q = 0; q < 16; ++q) hw[q] = hw[16 + q];
                }
                float fw[8];
#pragma unroll
                for (int gi = 0; gi < 4; ++gi) {
                    if (gi * 8 >= nb) break;
                    const int cg = cb + gi * 8;
                    if (gi) in.group();
                    uint32_t sw[2] = {0, 0};
                    float ylo = 0.0f;
                    // the group's records from one address held in a VGPR (their
                    // offsets are immediates), not rebuilt from a scalar per read
                    const lds_u32 *rg = rec + (cg - c0) * RS;
                    __asm__("" : "+v"(rg));
                    Rec rq = *(const lds_u32x4 *)rg;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const Rec rn = *(const lds_u32x4 *)(rg + (i < 7 ? i + 1 : i) * RS);
                        uint32_t lvb;
                        const uint32_t s = decode1(cg - c0 + i, rg + i * RS, rq, lvb);
                        rq = rn;
                        sw[i >> 2] |= s << (8 * (i & 3));
                        if constexpr (ODT >= 0) {
                            const float y = __uint_as_float(lvb) * m;
                            if constexpr (ODT == ODT_F16) {
                                if (i & 1)
                                    hw[16 + gi * 4 + (i >> 1)] = kvc_f2h2(ylo, y);
                                else
                                    ylo = y;
                            } else {
                                fw[i] = y;
                            }
                        }
                    }
                    if constexpr ((OUT & OUT_SYM) != 0)
                        if (active) *(uint2 *)(so + cg) = make_uint2(sw[0], sw[1]);
                    if constexpr (ODT == ODT_F32) {
                        if (active) {
                            float4 *o = (float4 *)((float *)out + row * C + cg);
                            o[0] = make_float4(fw[0], fw[1], fw[2], fw[3]);
                            o[1] = make_float4(fw[4], fw[5], fw[6], fw[7]);
                        }
                    }
                }
            }
        } else {
            for (int c = c0; c < c1; ++c) {
                if ((c & 7) == 0) in.group();
                uint32_t lvb;
                const uint32_t s = decode1(c - c0, rec + (c - c0) * RS, load_rec(c - c0), lvb);
                if (!active) continue;
                if constexpr ((OUT & OUT_SYM) != 0) so[c] = (uint8_t)s;
                if constexpr (ODT >= 0) {
                    const float y = __uint_as_float(lvb) * m;
                    if constexpr (ODT == ODT_F16)
                        ((uint16_t *)out)[row * C + c] = (uint16_t)kvc_f2h(y);
                    else
                        ((float *)out)[row * C + c] = y;
                }
            }
        }
    }
    // the row's last half or pair of halves
    if constexpr (VEC && ODT == ODT_F16) {
        if (wave_on && C > 0) {
            const int hl = (C - 1) >> 5;  // index of the last half
            if (hl & 1)
                put_pair(32 * (hl - 1), C - 32 * (hl - 1));
            else
                put_half(32 * hl, C - 32 * hl);
        }
    }
    if (active && bad.mine()) kvc_flag(status, KVC_DEV_CORRUPT);
}

// Maximum of v over each aligned group of G lanes (G = 2, 4 or 8), in every
// lane of the group: DPP swaps within quads, then the half-row mirror (every
// source lane exists, so bound_ctrl loses nothing and saves setting the old
// value).
template <int G>
__device__ __forceinline__ uint32_t group_max(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));
    if constexpr (G >= 4) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true));
    if constexpr (G >= 8) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, true));
    return v;
}

// The last key of k[0, E) with r * (key >> 16) <= code, k[0] taken to
// qualify (the qualifying keys a prefix); its index in idx.
template <int E>
__device__ __forceinline__ uint32_t slice_last_key(const uint32_t *k, uint32_t r, uint32_t code,
                                                   uint32_t &idx)
{
    if constexpr (E == 1) {
        idx = 0;
        return k[0];
    } else {
        const bool a = r * (k[E / 2] >> 16) <= code;
        uint32_t h[E / 2];
#pragma unroll
        for (int i = 0; i < E / 2; ++i) h[i] = a ? k[E / 2 + i] : k[i];
        uint32_t sub;
        const uint32_t v = slice_last_key<E / 2>(h, r, code, sub);
        idx = (a ? (uint32_t)(E / 2) : 0u) + sub;
        return v;
    }
}

// Decoding with G lanes per stream, for launches with few streams.  A stream's
// symbols are a chain of dependent steps, so with one lane per stream a small
// launch leaves most of the chip idle while each step waits on its table
// reads.  Here the G lanes of a group carry identical coder state and byte
// feeds (each its own ring).  A tile's CDF rows are staged as rows of P2 keys
// start << 16 | frequency (PairTile::store_keys: entries past A repeat entry
// A - 1, entry 0's start is 0), and at each symbol lane q searches its slice
// [q E, q E + E) of the channel's row (E = P2 / G) over registers for the
// last key with r * start <= code (a prefix of the slice on a non-decreasing
// row).  On such a row the keys grow with the index, so the maximum over the
// group of the lanes' keys (a lane whose first key does not qualify offers
// 0) is the key of the largest qualifying k, the symbol the one-lane
// searches find: its interval comes out of the search itself, with no table
// read after it, and the symbol, needed only for the output, is the maximum
// of the lanes' q E + index.  The slice reads do not depend on the coder
// state and are issued a group of 8 channels ahead.  The outputs of a stream
// are split over its lanes.  Block: 256 / G streams of one slab.
template <bool VEC, int OUT, int NSTEP, int G, bool PAD>
__global__ __launch_bounds__(256) void k_decode_group(const uint8_t *__restrict__ payload,
                                                      int64_t payload_bytes,
                                                      const uint64_t *__restrict__ slab_off,
                                                      const uint16_t *__restrict__ stream_len,
                                                      const uint16_t *__restrict__ cdf,
                                                      const uint16_t *__restrict__ max1,
                                                      uint8_t *__restrict__ sym_out,
                                                      void *__restrict__ out, KParams p,
                                                      int32_t *status, int CT)
{
    extern __shared__ uint32_t lds[];
    __shared__ uint32_t s_red[4];
    constexpr uint32_t P2 = 1u << NSTEP;
    constexpr int E = (int)P2 / G;  // slice entries per lane: 2, 4, 8 or 16
    static_assert(E >= 2 && E <= 16 && (E & (E - 1)) == 0, "slices of 2 to 16 entries");
    constexpr int SPB = 256 / G;     // streams per block
    const int C = p.C, A = p.A;
    float *lut = (float *)lds;
    lds_u32 *const ring = (lds_u32 *)(lds + 256) + threadIdx.x * 17u;
    lds_u32 *const tile = (lds_u32 *)(lds + 256 + 256 * 17);
    lds_u32 *const keys = tile;  // [CT][P2] keys start << 16 | frequency
    constexpr int SW = E;        // dwords of a lane's slice

    const int q = (int)threadIdx.x % G;   // lane within the stream's group
    const int sl = (int)threadIdx.x / G;  // stream within the block
    const int bps = (p.Tc + SPB - 1) / SPB;
    const int64_t bl = xcd_block(blockIdx.x, gridDim.x);  // the slab's blocks share an XCD
    const int64_t slab = bl / bps;
    const int tb = (int)(bl - slab * bps);
    const int t = tb * SPB + sl;
    const SlabGeom g = slab_geom(p, slab);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const bool active = t < g.nj;

    // bytes of the slab's streams before this block
    uint32_t pre = 0;
    const int n_before = min(tb * SPB, g.nj);
    for (int i = threadIdx.x; i < n_before; i += 256) pre += stream_len[g.sid0 + i];
    pre = wave_sum_u32(pre);
    if (lane == 0) s_red[wid] = pre;
    __syncthreads();
    pre = s_red[0] + s_red[1] + s_red[2] + s_red[3];
    __syncthreads();
    // exclusive scan over the block's streams: lane 0 of each group adds its length
    const uint32_t len = active ? stream_len[g.sid0 + t] : 0u;
    uint32_t incl = q == 0 ? len : 0u;
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

    const int64_t row = g.row0 + (active ? t : 0);
    const uint64_t off = active ? slab_off[slab] + pre + wbase + incl - len : 0;
    RingIn<lds_u32 *> in;
    in.init(payload, off, len, (uint64_t)payload_bytes, ring);
    DecState d;
    dec_init(d, in);
    constexpr int ODT = (OUT & OUT_F16) ? ODT_F16 : (OUT & OUT_F32) ? ODT_F32 : -1;
    const float m = (ODT >= 0) ? kvc_h2f(max1[row]) : 0.0f;
    uint32_t bad = 0;
    uint8_t *so = (OUT & OUT_SYM) ? sym_out + row * C : nullptr;
    const uint16_t *srows = cdf + g.tab * C * A;
    const int ntiles = (C + CT - 1) / CT;
    const uint32_t amax = (uint32_t)A - 1u;
    // this lane's slice of the key row of tile channel cl: keys [q E, q E + E)
    auto load_slice = [&](int cl, uint32_t(&ks)[SW]) {
        const lds_u32 *sp = keys + cl * (int)P2 + q * E;
        if constexpr (E == 2) {
            const u32x2 v = *(const lds_u32x2 *)sp;
            ks[0] = v.x;
            ks[1] = v.y;
        } else {
#pragma unroll
            for (int h = 0; h < E / 4; ++h) {
                const u32x4 v = *(const lds_u32x4 *)(sp + 4 * h);
                ks[4 * h] = v.x;
                ks[4 * h + 1] = v.y;
                ks[4 * h + 2] = v.z;
                ks[4 * h + 3] = v.w;
            }
        }
    };
    // The slice's last qualifying key (r * start <= code; a prefix of a slice
    // whose key 0 qualifies) by binary search over registers, its index in
    // ki.  Keys of qualifying entries grow with the index, so the group's
    // maximum over lanes whose key 0 qualifies is the key of the symbol: its
    // interval is known without a table read that waits on the search.  The
    // symbol itself (for the output) is the maximum of the lanes' q E + ki.
    auto decode1 = [&](int cl, const uint32_t(&ks)[SW], float &lv) -> uint32_t {
        const uint32_t r = d.range >> 16;
        uint32_t ki;
        uint32_t key = slice_last_key<E>(ks, r, d.code, ki);
        __asm__("" : "+v"(key), "+v"(ki));
        const bool q0 = r * (ks[0] >> 16) <= d.code;  // lane 0: start 0, always
        key = q0 ? key : 0u;
        uint32_t s = q0 ? (uint32_t)(q * E) + ki : 0u;
        key = group_max<G>(key);
        s = group_max<G>(s);
        if constexpr (PAD) s = min(s, amax);  // padding repeats entry A - 1
        bad |= dec_advance(d, r, key >> 16, key & 0xFFFFu);
        lv = lut[s];
        return s;
    };
    PairTile<2> pt;
    uint32_t hw[16];
    // slices of 8 consecutive channels, loaded one such group ahead of their
    // decoding (the groups of a tile alternate between the two buffers)
    uint32_t sa[8][SW], sb[8][SW];
    auto load_group = [&](int cl0, uint32_t(&buf)[8][SW]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) load_slice(cl0 + i, buf[i]);
    };
    pt.load(srows, 0, CT, C, A);
    for (int it = 0; it < ntiles; ++it) {
        const int c0 = it * CT, c1 = min(C, c0 + CT);
        __syncthreads();
        pt.store_keys(keys, CT, A, (int)P2);
        __syncthreads();
        if (it + 1 < ntiles) pt.load(srows, c0 + CT, CT, C, A);
        if (!active) continue;
        if constexpr (VEC) {
            // C % 16 == 0, CT % 16 == 0: blocks of 32 channels (64 fp16 bytes per
            // row), lane q writing 64 / G bytes of each; 8-symbol groups of
            // symbols or fp32 values by lane gi % G.  A block has an even number
            // of groups, so group gi of every block decodes from buffer gi % 2.
            load_group(0, sa);
            for (int cb = c0; cb < c1; cb += 32) {
                const int nb = min(32, c1 - cb);  // 16 or 32
#pragma unroll
                for (int gi = 0; gi < 4; ++gi) {
                    if (gi * 8 >= nb) break;
                    const int cg = cb + gi * 8;
                    uint32_t(&cur)[8][SW] = (gi & 1) ? sb : sa;
                    // the next group of the tile (the last group reloads itself, so the
                    // loads need no branch); the barrier keeps them ahead of this
                    // group's decoding
                    load_group(min(cg + 8, c1 - 8) - c0, (gi & 1) ? sa : sb);
                    __asm__ volatile("" ::: "memory");
                    in.group();
                    uint32_t sw[2] = {0, 0};
                    float fw[8];
                    float ylo = 0.0f;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        if ((i & 1) == 0) dec_refill(d, in);
                        float lv;
                        const uint32_t s = decode1(cg - c0 + i, cur[i], lv);
                        sw[i >> 2] |= s << (8 * (i & 3));
                        if constexpr (ODT >= 0) {
                            const float y = lv * m;
                            if constexpr (ODT == ODT_F16) {
                                if (i & 1)
                                    hw[gi * 4 + (i >> 1)] = kvc_f2h2(ylo, y);
                                else
                                    ylo = y;
                            } else {
                                fw[i] = y;
                            }
                        }
                    }
                    if (q == gi % G) {
                        if constexpr ((OUT & OUT_SYM) != 0) *(uint2 *)(so + cg) = make_uint2(sw[0], sw[1]);
                        if constexpr (ODT == ODT_F32) {
                            float4 *o = (float4 *)((float *)out + row * C + cg);
                            o[0] = make_float4(fw[0], fw[1], fw[2], fw[3]);
                            o[1] = make_float4(fw[4], fw[5], fw[6], fw[7]);
                        }
                    }
                }
                if constexpr (ODT == ODT_F16) {
                    constexpr int NW = 16 / G;  // dwords per lane
                    uint32_t wv[NW];
#pragma unroll
                    for (int k = 0; k < NW; ++k) {
                        wv[k] = hw[k];
#pragma unroll
                        for (int j = 1; j < G; ++j)
                            if (q == j) wv[k] = hw[j * NW + k];
                    }
                    if (q * 2 * NW < nb) {
                        uint32_t *o = (uint32_t *)((uint16_t *)out + row * C + cb) + q * NW;
                        if constexpr (NW == 8) {
                            ((uint4 *)o)[0] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
                            ((uint4 *)o)[1] = make_uint4(wv[4], wv[5], wv[6], wv[7]);
                        } else if constexpr (NW == 4) {
                            *(uint4 *)o = make_uint4(wv[0], wv[1], wv[2], wv[3]);
                        } else {
                            *(uint2 *)o = make_uint2(wv[0], wv[1]);
                        }
                    }
                }
            }
        } else {
            for (int c = c0; c < c1; ++c) {
                if ((c & 7) == 0) in.group();
                if ((c & 1) == 0) dec_refill(d, in);
                float lv;
                uint32_t e2[SW];
                load_slice(c - c0, e2);
                const uint32_t s = decode1(c - c0, e2, lv);
                if (q == c % G) {
                    if constexpr ((OUT & OUT_SYM) != 0) so[c] = (uint8_t)s;
                    if constexpr (ODT >= 0) {
                        const float y = lv * m;
                        if constexpr (ODT == ODT_F16)
                            ((uint16_t *)out)[row * C + c] = (uint16_t)kvc_f2h(y);
                        else
                            ((float *)out)[row * C + c] = y;
                    }
                }
            }
        }
    }

    if (active && bad && q == 0) kvc_flag(status, KVC_DEV_CORRUPT);
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

// Channels per LDS tile: search rows of P2 entries, CT * P2 = 1024, at least 16
// (12.8 KB of LDS per block at A = 32, so 8 blocks fit on a CU).
static int dec_tile_channels(int A)
{
    int P2 = 1;
    while (P2 < A) P2 <<= 1;
    return P2 <= 64 ? 1024 / P2 : 16;
}

static size_t dec_lds_bytes(int A, int CT)
{
    int P2 = 1;
    while (P2 < A) P2 <<= 1;
    const size_t n16 = ((size_t)CT * P2 + 1) / 2;
    return sizeof(uint32_t) * (256 + 256 * 17 + n16 + 2 * (size_t)CT * A);
}

// k_decode_mode's tile: as k_decode's (CT * P2 = 1024), but at least one
// 32-channel half of its output.
static int dec_mode_tile_channels(int nstep)
{
    const int ct = 1024 >> nstep;
    return ct < 32 ? 32 : ct;
}

// k_decode_mode: the table, the rings, two buffers of CT records, the search
// rows and the (start, frequency) pairs.
static size_t dec_mode_lds_bytes(int A, int CT, int nstep)
{
    const size_t P2 = (size_t)1 << nstep;
    const size_t n16 = ((size_t)CT * P2 + 1) / 2;
    return sizeof(uint32_t) * (256 + 256 * 17 + 2 * (size_t)CT * DEC_MODE_RS(nstep) + n16 + (size_t)CT * A +
                               4 * 576);
}

int decode_lanes_per_stream(const KParams &p)
{
    const int nstep = (int)cdf_nstep((uint32_t)p.A);
    if (nstep < 3 || nstep > 6 || p.n_streams > KVC_DEC_GROUP_MAX_STREAMS) return 1;
    return (nstep == 6 || (nstep >= 4 && KVC_DEC_GROUP_LANES == 8)) ? 8 : 4;
}

// k_decode_group: 4 lanes per stream (8 for 64-entry rows, so a lane's slice is 8 entries).
static hipError_t launch_decode_group(const uint8_t *payload, int64_t payload_bytes,
                                      const uint64_t *slab_off, const uint16_t *stream_len,
                                      const uint16_t *cdf, const uint16_t *max1, uint8_t *sym_out,
                                      void *out, int mode, const KParams &p, int32_t *status, bool vec,
                                      int CT, size_t lds, int nstep, hipStream_t stream)
{
    const int G = decode_lanes_per_stream(p);
    const int64_t bps = (p.Tc + 256 / G - 1) / (256 / G);
    dim3 grid((unsigned)(bps * p.n_slabs)), block(256);
#define KVC_DECG(V, O, N, GG)                                                                        \
    if (p.A == (1 << N))                                                                             \
        hipLaunchKernelGGL((k_decode_group<V, O, N, GG, false>), grid, block, lds, stream, payload,   \
                           payload_bytes, slab_off, stream_len, cdf, max1, sym_out, out, p, status, CT); \
    else                                                                                             \
        hipLaunchKernelGGL((k_decode_group<V, O, N, GG, true>), grid, block, lds, stream, payload,    \
                           payload_bytes, slab_off, stream_len, cdf, max1, sym_out, out, p, status, CT)
#define KVC_DECG_N(V, O)                                                                             \
    switch (nstep) {                                                                                 \
    case 3: KVC_DECG(V, O, 3, 4); break;                                                             \
    case 4: KVC_DECG(V, O, 4, KVC_DEC_GROUP_LANES); break;                                           \
    case 5: KVC_DECG(V, O, 5, KVC_DEC_GROUP_LANES); break;                                           \
    default: KVC_DECG(V, O, 6, 8); break;                                                            \
    }
#define KVC_DECG_M(V)                                                                                \
    switch (mode) {                                                                                  \
    case OUT_F16: KVC_DECG_N(V, OUT_F16) break;                                                      \
    case OUT_F32: KVC_DECG_N(V, OUT_F32) break;                                                      \
    case OUT_SYM: KVC_DECG_N(V, OUT_SYM) break;                                                      \
    case OUT_F16 | OUT_SYM: KVC_DECG_N(V, OUT_F16 | OUT_SYM) break;                                  \
    case OUT_F32 | OUT_SYM: KVC_DECG_N(V, OUT_F32 | OUT_SYM) break;                                  \
    default: break;                                                                                  \
    }
    (void)G;
    if (vec) {
        KVC_DECG_M(true)
    } else {
        KVC_DECG_M(false)
    }
#undef KVC_DECG_M
#undef KVC_DECG_N
#undef KVC_DECG
    return hipGetLastError();
}

// KVC_DEC_N(V, O) over the output modes and vector forms (kvc_decode rejects
// a call with nothing to write)
#define KVC_DEC_DISPATCH                                                                             \
    {                                                                                                \
        if (vec) {                                                                                   \
            switch (mode) {                                                                          \
            case OUT_F16: KVC_DEC_N(true, OUT_F16) break;                                            \
            case OUT_F32: KVC_DEC_N(true, OUT_F32) break;                                            \
            case OUT_SYM: KVC_DEC_N(true, OUT_SYM) break;                                            \
            case OUT_F16 | OUT_SYM: KVC_DEC_N(true, OUT_F16 | OUT_SYM) break;                        \
            case OUT_F32 | OUT_SYM: KVC_DEC_N(true, OUT_F32 | OUT_SYM) break;                        \
            default: break;                                                                          \
            }                                                                                        \
        } else {                                                                                     \
            switch (mode) {                                                                          \
            case OUT_F16: KVC_DEC_N(false, OUT_F16) break;                                           \
            case OUT_F32: KVC_DEC_N(false, OUT_F32) break;                                           \
            case OUT_SYM: KVC_DEC_N(false, OUT_SYM) break;                                           \
            case OUT_F16 | OUT_SYM: KVC_DEC_N(false, OUT_F16 | OUT_SYM) break;                       \
            case OUT_F32 | OUT_SYM: KVC_DEC_N(false, OUT_F32 | OUT_SYM) break;                       \
            default: break;                                                                          \
            }                                                                                        \
        }                                                                                            \
    }

// Streams on which launch_decode runs the mode-first decoder's runs after the
// first one, concurrently with it, and the events that fork them from the
// caller's stream and join them back before the guard launch: made on first
// use on each device, at the default priority.  g_run_mu is held from the fork
// to the join, so that calls from several host threads do not interleave
// their records and waits on the shared events.
constexpr int kRunStreams = 3;
constexpr int kRunDevices = 64;
struct RunStreams {
    hipStream_t s[kRunStreams];
    hipEvent_t fork, join[kRunStreams];
};
static std::mutex g_run_mu;
static RunStreams *g_runs[kRunDevices];

// The current device's streams (g_run_mu held), or NULL if they cannot be made
// (the runs then go one after the other on the caller's stream).
static RunStreams *run_streams()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kRunDevices) return nullptr;
    if (!g_runs[dev]) {
        RunStreams r{};
        bool ok = hipEventCreateWithFlags(&r.fork, hipEventDisableTiming) == hipSuccess;
        for (int i = 0; ok && i < kRunStreams; ++i)
            ok = hipStreamCreateWithFlags(&r.s[i], hipStreamNonBlocking) == hipSuccess &&
                 hipEventCreateWithFlags(&r.join[i], hipEventDisableTiming) == hipSuccess;
        if (!ok) return nullptr;
        g_runs[dev] = new RunStreams(r);
    }
    return g_runs[dev];
}

// Runs of (layer, K|V) pairs decoded with a shallower search than the
// table's rows need take at least this many blocks (four times what the chip
// holds at once), else they search whole rows with their neighbours.
constexpr int64_t KVC_DEC_RUN_MIN_BLOCKS = 4096;

// Search depth of the mode-first decoder for (layer, K|V) lk: that of its
// bins, at least nmin and at most the table's (nstep).
static int dec_run_nstep(const KParams &p, int lk, int nstep, int nmin)
{
    const int bins = 2 * ((int)p.maxq[lk] + 1);
    int n = (int)cdf_nstep((uint32_t)bins);
    if (n < nmin) n = nmin;
    return n < nstep ? n : nstep;
}

hipError_t launch_decode(const uint8_t *payload, int64_t payload_bytes, const uint64_t *slab_off,
                         const uint16_t *stream_len, const uint16_t *cdf, const uint16_t *max1,
                         uint8_t *sym_out, void *out, int out_dtype, const KParams &p,
                         int32_t *status, bool vec, hipStream_t stream)
{
    if (p.n_slabs == 0) return hipSuccess;
    const int64_t bps = (p.Tc + 255) / 256;
    dim3 grid((unsigned)(bps * p.n_slabs)), block(256);
    const int mode = (out ? (out_dtype == KVC_F16 ? OUT_F16 : OUT_F32) : 0) | (sym_out ? OUT_SYM : 0);
    const int CT = dec_tile_channels(p.A);
    const size_t lds = dec_lds_bytes(p.A, CT);
    vec = vec && (CT % 16 == 0);
    const int nstep = (int)cdf_nstep((uint32_t)p.A);
    if (decode_lanes_per_stream(p) > 1)
        return launch_decode_group(payload, payload_bytes, slab_off, stream_len, cdf, max1, sym_out, out,
                                   mode, p, status, vec, CT, lds, nstep, stream);
    // Rows of 8 to 64 entries take the mode-first decoder (its exact path is
    // the two-level search, measured faster than binary lifting at every
    // launch size since its searches run over registers); 4-entry and 128-
    // or 256-entry rows binary lifting.
    if (nstep >= 3 && nstep <= 6) {
        // One launch per run of consecutive (layer, K|V) pairs whose symbols
        // need the same search depth: a run of layers with fewer bins than the
        // table's rows stages and searches only the first 2^n entries of each
        // row (n = its depth), every symbol of theirs lying below entry 2^n - 1
        // (symbols of b bins run to b - 2), with fewer levels, wider tiles and,
        // below 64 entries, more waves per SIMD.  In memory order block sb
        // takes (layer, K|V) sb / NC, so a run's blocks are one range of sb.
        //
        // Such a run decodes as the full search does until a search lands
        // past its staged entries, which only a stream inconsistent with its
        // tables can make happen, and the step that does flags the stream
        // (its code lies past the last staged interval).  So when any run was
        // cut short, a guard launch of the full search over every slab follows;
        // its blocks return at once unless a stream was flagged, and otherwise
        // decode everything again, so that the outputs are always the full
        // search's.
        // (Without a status word nothing could tell the guard, so then every
        // run searches whole rows.)  Launches on one stream run one after the
        // other, so a run of fewer than KVC_DEC_RUN_MIN_BLOCKS blocks, which
        // could not fill the chip for long, searches whole rows too and joins
        // its neighbours that do.
        const int LK = 2 * p.L;
        const int nmin = status ? 3 : nstep;  // the shallowest depth a run may take
        int run_n[2 * KVC_MAX_LAYERS];  // each (layer, K|V)'s depth
        for (int lk = 0; lk < LK;) {
            const int n = dec_run_nstep(p, lk, nstep, nmin);
            int lk1 = lk + 1;
            while (lk1 < LK && dec_run_nstep(p, lk1, nstep, nmin) == n) ++lk1;
            const bool small = bps * (int64_t)(lk1 - lk) * p.NC < KVC_DEC_RUN_MIN_BLOCKS;
            for (int k = lk; k < lk1; ++k) run_n[k] = small ? nstep : n;
            lk = lk1;
        }
        int n_runs = 0;
        for (int lk = 0; lk < LK; ++lk) n_runs += lk == 0 || run_n[lk] != run_n[lk - 1];
        // The runs after the first go on streams of their own, concurrently
        // with it (each run's last, partly filled wave of blocks then overlaps
        // another run's), joined back before the guard.
        std::unique_lock<std::mutex> run_lock(g_run_mu, std::defer_lock);
        RunStreams *rs = nullptr;
        if (n_runs > 1) {
            run_lock.lock();
            rs = run_streams();
            if (rs && hipEventRecord(rs->fork, stream) != hipSuccess) return hipErrorLaunchFailure;
        }
        bool cut = false;
        int run = 0;
        for (int lk0 = 0; lk0 <= LK;) {
            const bool guard_pass = lk0 == LK;  // after the runs: the guard launch
            if (guard_pass && rs) {
                for (int i = 0; i < kRunStreams && i < n_runs - 1; ++i)
                    if (hipEventRecord(rs->join[i], rs->s[i]) != hipSuccess ||
                        hipStreamWaitEvent(stream, rs->join[i], 0) != hipSuccess)
                        return hipErrorLaunchFailure;
            }
            if (guard_pass && !cut) break;
            const int n0 = guard_pass ? nstep : run_n[lk0];
            int lk1 = guard_pass ? LK + 1 : lk0 + 1;
            while (lk1 < LK && run_n[lk1] == n0) ++lk1;
            hipStream_t st = stream;  // this launch's stream
            if (rs && !guard_pass && run > 0) {
                st = rs->s[(run - 1) % kRunStreams];
                if (run <= kRunStreams && hipStreamWaitEvent(st, rs->fork, 0) != hipSuccess)
                    return hipErrorLaunchFailure;
            }
            run += guard_pass ? 0 : 1;
            const int A_st = n0 < nstep ? (1 << n0) : p.A;  // entries staged per row
            const bool pad = A_st != (1 << n0);
            cut = cut || A_st < p.A;
            const int CT_mode = dec_mode_tile_channels(n0);
            const size_t lds_mode = dec_mode_lds_bytes(A_st, CT_mode, n0);
            // the staging covers DEC_MODE_PER(n) pairs per thread: never launch a
            // tile it would stage only in part
            if (CT_mode * (A_st / 2) > 256 * DEC_MODE_PER(n0)) return hipErrorInvalidValue;
            const int64_t nlk = guard_pass ? LK : lk1 - lk0;
            const dim3 grid_run((unsigned)(bps * nlk * p.NC));
            const int64_t sb0 = guard_pass ? 0 : (int64_t)lk0 * p.NC;
            const int guard = guard_pass ? 1 : 0;
#define KVC_DECM(V, O, N, PD)                                                                        \
    hipLaunchKernelGGL((k_decode_mode<V, O, N, PD>), grid_run, block, lds_mode, st, payload,     \
                       payload_bytes, slab_off, stream_len, cdf, max1, sym_out, out, p, status, CT_mode, \
                       A_st, sb0, guard)
#define KVC_DECB(V, O, N)                                                                            \
    if (pad) KVC_DECM(V, O, N, true);                                                                \
    else KVC_DECM(V, O, N, false)
#define KVC_DEC_N(V, O)                                                                              \
    switch (n0) {                                                                                    \
    case 3: KVC_DECB(V, O, 3); break;                                                                \
    case 4: KVC_DECB(V, O, 4); break;                                                                \
    case 5: KVC_DECB(V, O, 5); break;                                                                \
    default: KVC_DECB(V, O, 6); break;                                                               \
    }
            KVC_DEC_DISPATCH
#undef KVC_DEC_N
#undef KVC_DECB
#undef KVC_DECM
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            lk0 = lk1;
        }
        return hipSuccess;
    }
#define KVC_DEC(V, O, N, B)                                                                          \
    hipLaunchKernelGGL((k_decode<V, O, N, B>), grid, block, lds, stream, payload, payload_bytes,     \
                       slab_off, stream_len, cdf, max1, sym_out, out, p, status, CT)
#define KVC_DEC_N(V, O)                                                                              \
    switch (nstep) {                                                                                 \
    case 2: KVC_DEC(V, O, 2, false); break;                                                          \
    case 7: KVC_DEC(V, O, 7, false); break;                                                          \
    default: KVC_DEC(V, O, 8, false); break;                                                         \
    }
    KVC_DEC_DISPATCH
#undef KVC_DEC_N
#undef KVC_DEC
    return hipGetLastError();
}
#undef KVC_DEC_DISPATCH

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
