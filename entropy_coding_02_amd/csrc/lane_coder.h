// lane_coder.h - one range-coder stream per GPU lane.
//
// The CacheGen write-up (LMCache, "1.2 Core challenges and solutions", design
// point 3, and "2.1 Core components": ac_enc / ac_dec) codes the quantized
// symbols with GPU-parallel arithmetic coding; the stream unit here is one
// (chunk, layer, K|V, token) row of C channel symbols.  The coder is a 32-bit
// range coder over 16-bit cumulative frequencies with byte renormalisation:
//
//   r = range >> 16;  low += r * cdf_s;  range = r * f_s;  scale by 256 while range < 2^24
//   finish: round low up to a multiple of 2^24; the stream is the number
//   written in base 256 with its (always zero) first byte and its trailing
//   zero bytes removed.  A decoder reads zeros past the end.
//
// The byte sequence is fully fixed by those rules; how a lane buffers bytes
// and resolves carries is free, and this file does it without a byte loop:
//   * the renormalisation shift count is clz(range) & 24 (0, 8 or 16 bits),
//     applied to a 96-bit shift register {pb (64 bits), lo (32 bits)};
//   * pb holds k <= 7 pending bytes; a carry out of lo is added to pb, and
//     integer addition ripples it through pending 0xFF bytes by itself.  A
//     carry that runs past all k pending bytes sets bit 8k of pb: it belongs
//     to bytes already written, and is added to them (a rare path);
//   * when k reaches 6, the 4 oldest pending bytes go out as one aligned
//     big-endian dword, so at least 2 bytes always stay pending (the state
//     counts pending bits, 8k).
// All arithmetic is 32/64-bit integer; this header is compiled both for the
// GPU kernels and, in the tests, for the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define KVC_HD __host__ __device__ __forceinline__

typedef uint32_t kvc_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t kvc_u32x2 __attribute__((ext_vector_type(2)));

KVC_HD uint32_t kvc_bswap32(uint32_t v) { return __builtin_bswap32(v); }

// a * b for a, b < 2^24 (one full-rate 24-bit multiply on the GPU, where a
// 32-bit multiply whose operands the compiler cannot bound is quarter rate).
KVC_HD uint32_t kvc_umul24(uint32_t a, uint32_t b)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __umul24(a, b);
#else
    return (a & 0xFFFFFFu) * (b & 0xFFFFFFu);
#endif
}

// Shift count (bits) that brings range back to >= 2^24; range must be >= 2^8.
KVC_HD uint32_t kvc_renorm_bits(uint32_t range) { return (uint32_t)__builtin_clz(range) & 24u; }

// ----------------------------------------------------------------- encoder

struct EncState {
    uint32_t lo;     // low 32 bits of the coding interval's lower end
    uint32_t range;  // interval width, >= 2^24 between symbols
    uint64_t pb;     // k pending bytes (newest lowest) + carry indicator at bit 8k
    uint32_t kb;     // pending bits, 8k
    uint32_t w;      // dwords already written to the stream slot
};

// A stream slot: dword-addressable memory owned by one lane; dword i of the
// stream is at base[i * stride + lane] (the kernels interleave the slots of a
// block's lanes, stride = lanes per block, so lanes writing their k-th dwords
// at about the same time fill the same cache lines).  base is the same for
// the whole block and a slot region stays below 4 GiB, so an address is the
// uniform base plus a 32-bit offset.
struct SlotOut {
    uint32_t *base;
    uint32_t lane;
    uint32_t stride;
    KVC_HD uint32_t *at(uint32_t i) const
    {
        return (uint32_t *)((char *)base + (size_t)((i * stride + lane) * 4u));
    }
    KVC_HD uint32_t load(uint32_t i) const { return *at(i); }
    KVC_HD void store(uint32_t i, uint32_t v) const { *at(i) = v; }
};

KVC_HD void enc_init(EncState &e)
{
    e.lo = 0;
    e.range = 0xFFFFFFFFu;
    e.pb = 0;
    e.kb = 0;
    e.w = 0;
}

// Add one to the big-endian number held in dwords [0, w) of the slot.
template <class Out>
__host__ __device__ __noinline__ void enc_carry_into_written(const Out &out, uint32_t w)
{
    for (int32_t i = (int32_t)w - 1; i >= 0; --i) {
        uint32_t v = kvc_bswap32(out.load((uint32_t)i)) + 1u;
        out.store((uint32_t)i, kvc_bswap32(v));
        if (v != 0) break;
    }
}

// Code one symbol with cumulative frequency st and frequency fr (1 <= fr,
// st + fr <= 65536).
template <class Out>
KVC_HD void enc_put(EncState &e, uint32_t st, uint32_t fr, const Out &out)
{
    uint32_t r = e.range >> 16;
    uint32_t add = r * st;
    uint32_t lo2 = e.lo + add;
    e.pb += (lo2 < add) ? 1u : 0u;
    e.range = r * fr;
    uint32_t n = kvc_renorm_bits(e.range);
    e.range <<= n;
    uint64_t wide = (uint64_t)lo2 << n;
    e.pb = (e.pb << n) | (wide >> 32);
    e.lo = (uint32_t)wide;
    e.kb += n;
    if (e.kb >= 48u) {
        // k = 6 or 7: bytes k-1 .. k-4 go out, 16 or 24 bits stay; the carry
        // indicator (bit 8k) is bit sh of the high dword
        const uint32_t sh = e.kb - 32u;
        const uint32_t word = (uint32_t)(e.pb >> sh);
        if (((uint32_t)(e.pb >> 32) >> sh) != 0) enc_carry_into_written(out, e.w);
        out.store(e.w, kvc_bswap32(word));
        e.w += 1;
        e.pb = (uint64_t)((uint32_t)e.pb & ((1u << sh) - 1u));
        e.kb -= 32u;
    }
}

// Flush and write the tail; returns the stream length in bytes (trailing
// zero bytes removed).  At most 4*w + 8 bytes of the slot are touched.
template <class Out>
KVC_HD uint32_t enc_finish(EncState &e, const Out &out)
{
    uint32_t lo2 = e.lo + 0xFFFFFFu;
    e.pb += (lo2 < 0xFFFFFFu) ? 1u : 0u;
    uint32_t top = lo2 >> 24;  // the byte kept after rounding up to a multiple of 2^24
    const uint32_t kb = e.kb;
    if ((e.pb >> kb) != 0) {
        enc_carry_into_written(out, e.w);
        e.pb &= ((uint64_t)1 << kb) - 1u;
    }
    uint64_t tail = (e.pb << 8) | top;  // k + 1 bytes, oldest first
    uint32_t nt = kb / 8u + 1u;
    while (nt > 0 && (tail & 0xFFu) == 0) {
        tail >>= 8;
        nt -= 1;
    }
    if (nt > 0) {
        uint64_t t = tail << (64u - 8u * nt);  // left-align
        out.store(e.w, kvc_bswap32((uint32_t)(t >> 32)));
        if (nt > 4) out.store(e.w + 1u, kvc_bswap32((uint32_t)t));
        return 4u * e.w + nt;
    }
    // the tail is all zero: the stream ends inside the written dwords
    for (int32_t i = (int32_t)e.w - 1; i >= 0; --i) {
        uint32_t v = kvc_bswap32(out.load((uint32_t)i));
        if (v != 0) return 4u * (uint32_t)i + 4u - ((uint32_t)__builtin_ctz(v) >> 3);
    }
    return 0;
}

// ------------------------------------------- one stream coded by G lanes
//
// The interval arithmetic splits: the range never depends on low, and low is
// a sum.  With r_i = range_i >> 16, S_i the bits shifted out before symbol i
// (S_0 = 0) and S at the end, the coder's final low is
//     X = sum_i r_i * cdf_{s_i} * 2^(S - S_i)
// (each term is added, then shifted with everything after it).  Cut the
// symbols into consecutive blocks.  Block g coded alone, from low = 0 and the
// range the whole chain has at its start, gives P_g = sum over its symbols of
// r_i * cdf_{s_i} * 2^(E_g - S_i) (E_g = S at its end) as (E_g - S_g)/8
// shifted-out bytes followed by its 4-byte low, and X = sum_g P_g * 2^(S - E_g).
// In stream byte positions P_g starts at S_g / 8, so consecutive blocks
// overlap only where P_g's low meets P_{g+1}'s first 4 bytes.  The stream is
// the first S/8 + 1 bytes of X + 0xFFFFFF written in S/8 + 4 bytes, trailing
// zeros removed: what enc_finish writes.
//
// Hence G lanes can code one stream: each follows the range chain over the
// whole stream (no low, no bytes: a few operations a symbol), then codes its
// own block with the full coder, writing its shifted-out bytes straight to
// their stream positions; a last step adds every block's low (and the
// 0xFFFFFF) at its position, the carry running into the bytes before it,
// and trims.

// One range-chain step: the interval width after a symbol of frequency fr,
// renormalised; returns the bits shifted.
KVC_HD uint32_t enc_range_step(uint32_t &range, uint32_t fr)
{
    range = (range >> 16) * fr;
    const uint32_t n = kvc_renorm_bits(range);
    range <<= n;
    return n;
}

// A stream slot holding the stream's bytes contiguously, viewed from one
// block whose first byte is at stream position off.  load/store move the
// block's dword i (its bytes 4i .. 4i + 3, the first in the low byte, as
// SlotOut does) as one unaligned 4-byte access.
struct SplitOut {
    uint8_t *base;
    uint32_t off;
    KVC_HD uint8_t *byte(uint32_t pos) const { return base + pos; }
    KVC_HD uint32_t load(uint32_t i) const
    {
        uint32_t v;
        __builtin_memcpy(&v, base + off + 4u * i, 4);
        return v;
    }
    KVC_HD void store(uint32_t i, uint32_t v) const { __builtin_memcpy(base + off + 4u * i, &v, 4); }
    KVC_HD void store_if(bool p, uint32_t i, uint32_t v) const
    {
        if (p) store(i, v);
    }
    KVC_HD bool any(bool p) const { return p; }
    KVC_HD void carry(bool p, uint32_t w) const
    {
        if (p) enc_carry_into_written(*this, w);
    }
};

// End of a block: resolve a carry past the pending bytes, then write them
// after the block's dwords.  Returns the number of pending bytes; the low
// stays in e.lo.
template <class Out>
KVC_HD uint32_t enc_block_end(EncState &e, const Out &out)
{
    const uint32_t kb = e.kb;  // < 48
    if ((e.pb >> kb) != 0) {
        enc_carry_into_written(out, e.w);
        e.pb &= ((uint64_t)1 << kb) - 1u;
    }
    const uint32_t k = kb >> 3;
    for (uint32_t i = 0; i < k; ++i) *out.byte(out.off + 4u * e.w + i) = (uint8_t)(e.pb >> (8u * (k - 1u - i)));
    return k;
}

// Add the nb-byte (<= 4) big-endian value v at stream positions [pos, pos + nb)
// of the stream f addresses (f.off unused), the carry running into the bytes
// before pos.
KVC_HD void split_add(const SplitOut &f, uint32_t pos, uint32_t v, uint32_t nb)
{
    uint32_t carry = 0;
    for (uint32_t b = nb; b-- > 0;) {
        uint8_t *q = f.byte(pos + b);
        const uint32_t t = (uint32_t)*q + ((v >> (8u * (nb - 1u - b))) & 0xFFu) + carry;
        *q = (uint8_t)t;
        carry = t >> 8;
    }
    for (uint32_t q = pos; carry != 0 && q-- > 0;) {
        uint8_t *c = f.byte(q);
        const uint32_t t = (uint32_t)*c + 1u;
        *c = (uint8_t)t;
        carry = t >> 8;
    }
}

// Stream length once every byte of positions [0, n) is in place: n without
// its trailing zero bytes.
KVC_HD uint32_t split_trim(const SplitOut &f, uint32_t n)
{
    while (n > 0 && *f.byte(n - 1u) == 0) --n;
    return n;
}

// ----------------------------------------------------------------- decoder

// Funnel shift: bits [sh, sh + 32) of the 64-bit value hi:lo (sh < 32).
KVC_HD uint32_t kvc_alignbit(uint32_t hi, uint32_t lo, uint32_t sh)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_alignbit(hi, lo, sh);
#else
    return sh ? (lo >> sh) | (hi << (32u - sh)) : lo;
#endif
}

// True if `c` holds on every active lane of the wavefront (on the host: c).
KVC_HD bool kvc_all(bool c)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_ballot_w64(c) == __builtin_amdgcn_read_exec();
#else
    return c;
#endif
}

// Byte feed of one stream through a 16-dword per-lane ring in LDS.
//
// The stream [start, start+len) of a buffer of `cap` bytes (a multiple of 4,
// at least 16) is fetched as aligned raw dwords from a0 = start & ~3.
// Stream dword j (bytes start+4j .. start+4j+3) is funnel-shifted out of raw
// dwords j and j+1, byte-swapped to big-endian and, past the end of the
// stream, masked to zero when it enters the ring, so a reader refill is one
// LDS read.  Every group of 8 symbols (at most 16 bytes = 4 stream dwords)
// the lane commits the 4 raw dwords it asked for one group earlier, if any,
// and, while at most 8 stream dwords are unread, asks for the next 4 with
// one 16-byte load.  That keeps at least 5 unread dwords at every group
// start and never overwrites an unread one.  Near the end of the buffer the 16-byte
// piece is moved back to end at `cap`, and the commit shifts its dwords into
// place (dwords it cannot supply lie past the buffer, so past the stream,
// and are masked).  The reader keeps one ring dword ahead in a register.
template <class Ring>
struct RingIn {
    const uint8_t *p;  // base + a0
    Ring ring;         // this lane's 16 ring dwords (stream dword j at ring[j & 15])
    uint32_t len;      // stream length in bytes
    int32_t lim16;     // largest offset from p at which a 16-byte piece may be loaded (>= -12)
    uint32_t sh;       // (start & 3) * 8
    uint32_t w;        // stream dwords in the ring: [0, w), a multiple of 4
    uint32_t rd;       // next stream dword to read from the ring
    uint32_t nxt;      // stream dword rd - 1, read ahead
    uint32_t last;     // raw dword w: the low part of stream dword w
    kvc_u32x4 st;      // the piece in flight: raw dwords w+1 .. w+4, moved back by `back` bytes
    uint32_t back;     // how far the piece was moved back (0 unless near the buffer end)
    uint32_t want;     // a piece is in flight

    KVC_HD void issue()
    {
        const int32_t off = 4 * (int32_t)(w + 1u);
        const int32_t at = off < lim16 ? off : lim16;
        __builtin_memcpy(&st, p + at, 16);
        back = (uint32_t)(off - at);
    }
    KVC_HD void commit()
    {
        kvc_u32x4 r = st;
        if (!kvc_all(back == 0u)) {
            // raw dword w+1+k is piece dword k + back/4 (none when that is >= 4)
            const uint32_t d = back >> 2;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t i = (uint32_t)k + d;
                r[k] = i == 1u ? st[1] : i == 2u ? st[2] : i == 3u ? st[3] : (i == 0u ? st[0] : 0u);
            }
        }
        uint32_t v[4];
        v[0] = kvc_bswap32(kvc_alignbit(r[0], last, sh));
        v[1] = kvc_bswap32(kvc_alignbit(r[1], r[0], sh));
        v[2] = kvc_bswap32(kvc_alignbit(r[2], r[1], sh));
        v[3] = kvc_bswap32(kvc_alignbit(r[3], r[2], sh));
        if (!kvc_all(4u * w + 16u <= len)) {
            // bytes at or past len read as zero
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t pos = 4u * (w + (uint32_t)k);
                const uint32_t keep = len > pos ? len - pos : 0u;
                v[k] = keep >= 4u ? v[k] : (keep == 0u ? 0u : v[k] & ~(0xFFFFFFFFu >> (8u * keep)));
            }
        }
        const uint32_t b = w & 12u;
#pragma unroll
        for (int k = 0; k < 4; ++k) ring[b + (uint32_t)k] = v[k];
        last = r[3];
        w += 4u;
    }
    KVC_HD void init(const uint8_t *base, uint64_t start, uint64_t length, uint64_t capacity, Ring rg)
    {
        uint64_t a0 = start & ~(uint64_t)3;
        sh = (uint32_t)(start & 3u) * 8u;
        len = (uint32_t)length;
        if (a0 + 4u > capacity) {  // only an empty stream at the very end of the buffer
            a0 = capacity - 4u;
            len = 0;
        }
        p = base + a0;
        const uint64_t room = capacity - 16u;  // the last piece starts here
        lim16 = a0 > room ? -(int32_t)(a0 - room) : (room - a0 > 0x7FFFFFF0u ? 0x7FFFFFF0 : (int32_t)(room - a0));
        ring = rg;
        w = 0;
        last = *(const uint32_t *)p;
        issue();
        commit();
        issue();
        commit();  // stream dwords 0..7 in the ring
        issue();   // raw dwords 9..12 in flight
        want = 1;
        nxt = ring[0];
        rd = 1;
    }
    // Once per group of 8 symbols.
    KVC_HD void group()
    {
        if (want) commit();
        want = w - rd <= 8u ? 1u : 0u;
        if (want) issue();
    }
    // The next 4 stream bytes as a big-endian dword.
    KVC_HD uint32_t next()
    {
        const uint32_t v = nxt;
        nxt = ring[rd & 15u];
        rd += 1u;
        return v;
    }
    // next() if take, else 0 and nothing consumed.  Branch-free: the ring is
    // read either way (without take, stream dword rd - 1 again: it is still
    // in the ring), so no path waits for that read before the next refill.
    KVC_HD uint32_t next_if(bool take)
    {
        const uint32_t v = take ? nxt : 0u;
        const uint32_t idx = take ? rd : rd - 1u;
        nxt = ring[idx & 15u];
        rd = idx + 1u;
        return v;
    }
};

struct DecState {
    uint32_t code;
    uint32_t range;
    uint64_t bb;  // upcoming stream bits, most significant first
    uint32_t nb;  // valid bits in bb
};

template <class In>
KVC_HD void dec_init(DecState &d, In &in)
{
    d.code = in.next();
    d.bb = (uint64_t)in.next() << 32;
    d.nb = 32;
    d.range = 0xFFFFFFFFu;
}

// After the symbol with cumulative frequency st and frequency fr was found
// for r = range >> 16: narrow the interval and renormalise, taking the new
// bits from bb.  Returns 1 if the stream is inconsistent with the CDF (code
// outside the new interval).  A symbol consumes at most 16 bits (range >=
// 2^8 after narrowing), so bb must hold at least 16 valid bits.
KVC_HD uint32_t dec_advance(DecState &d, uint32_t r, uint32_t st, uint32_t fr)
{
    d.code -= r * st;
    d.range = r * fr;
    uint32_t bad = d.code >= d.range ? 1u : 0u;
    uint32_t n = kvc_renorm_bits(d.range);
    d.range <<= n;
    uint64_t t = (((uint64_t)d.code << 32) | (d.bb >> 32)) << n;
    d.code = (uint32_t)(t >> 32);
    d.bb <<= n;
    d.nb -= n;
    return bad;
}

// Top bb up to at least 32 valid bits: enough for the next two symbols.
// Without a branch (In::next_if), so a wave does not stall on the byte feed.
template <class In>
KVC_HD void dec_refill(DecState &d, In &in)
{
    const bool need = d.nb < 32u;
    const uint32_t v = in.next_if(need);  // 0 unless need, and then 32 - nb is in [1, 32]
    d.bb |= (uint64_t)v << ((32u - d.nb) & 63u);
    d.nb += need ? 32u : 0u;
}

// ------------------------------------------------- per-symbol table lookups

// The (start, frequency) pair of symbol s of a CDF row with A entries
// (cdf_A = 65536 implicit), packed as start | frequency << 16.  A
// non-increasing row gets frequency 1, so malformed tables cannot stall or
// overrun the coder.
KVC_HD uint32_t cdf_pair(uint32_t st, uint32_t nx)
{
    uint32_t fr = nx > st ? nx - st : 1u;
    return st | (fr << 16);
}

// Code symbol s whose packed pair is p.
template <class Out>
KVC_HD void enc_pair(EncState &e, uint32_t p, const Out &out)
{
    enc_put(e, p & 0xFFFFu, p >> 16, out);
}

// enc_put with no branch that depends on the lane: the flush is computed on
// every symbol and selected, the dword goes out through out.store_if(flush,
// ...), and only a carry past the pending bytes (when out.any() sees one in
// any lane) takes a branch, to out.carry().  Same state, same bytes as enc_put.  Where lanes
// run in lockstep this trades a few selects for the two masked blocks
// enc_put's flush needs on nearly every symbol.
template <class Out>
KVC_HD void enc_put_nb(EncState &e, uint32_t st, uint32_t fr, const Out &out)
{
    const uint32_t r = e.range >> 16;
    const uint32_t add = r * st;
    const uint32_t lo2 = e.lo + add;
    uint64_t pb = e.pb + ((lo2 < add) ? 1u : 0u);
    e.range = r * fr;
    const uint32_t n = kvc_renorm_bits(e.range);
    e.range <<= n;
    const uint64_t wide = (uint64_t)lo2 << n;
    pb = (pb << n) | (wide >> 32);
    e.lo = (uint32_t)wide;
    const uint32_t kb = e.kb + n;
    // k = 6 or 7 pending bytes: bytes k-1 .. k-4 go out (see enc_put)
    const bool fl = kb >= 48u;
    const uint32_t sh = (kb - 32u) & 31u;  // 16 or 24 when fl
    const bool ci = fl && (((uint32_t)(pb >> 32) >> sh) != 0);
    if (__builtin_expect(out.any(ci), 0)) out.carry(ci, e.w);
    out.store_if(fl, e.w, kvc_bswap32((uint32_t)(pb >> sh)));
    e.w += fl ? 1u : 0u;
    e.pb = fl ? (uint64_t)((uint32_t)pb & ((1u << sh) - 1u)) : pb;
    e.kb = fl ? kb - 32u : kb;
}

template <class Out>
KVC_HD void enc_pair_nb(EncState &e, uint32_t p, const Out &out)
{
    enc_put_nb(e, p & 0xFFFFu, p >> 16, out);
}

// Largest k in [0, A) with r * row[k] <= code, where `row` holds the A
// cumulative frequencies padded with 0xFFFF up to 2^NSTEP entries: binary
// lifting over the padded row, then a clamp to A - 1 (a padding entry can
// only be chosen when every real entry qualifies, and then A - 1 is right).
template <int NSTEP, class Row>
KVC_HD uint32_t cdf_search(const Row &row, uint32_t A, uint32_t r, uint32_t code)
{
    uint32_t s = 0;
#pragma unroll
    for (int i = NSTEP - 1; i >= 0; --i) {
        const uint32_t k = s + (1u << i);
        if (r * (uint32_t)row[k] <= code) s = k;
    }
    return s < A - 1u ? s : A - 1u;
}

// Index of the last qualifying entry (r * e <= code) of a non-decreasing run
// of E entries (E a power of two, 2 to 16) packed two per dword (entry 2j in
// the low half of d[j]), given that entry 0 qualifies, appended to idx: the
// result is idx * E + that index.  A binary search over values already in
// registers: log2 E compares, each halving the run with selects and adding
// one bit (idx = 2 idx + bit, one add with carry).
template <int E>
KVC_HD uint32_t piece_last(uint32_t idx, const uint32_t *d, uint32_t r, uint32_t code)
{
    if constexpr (E == 2) {
        return 2u * idx + (r * (d[0] >> 16) <= code ? 1u : 0u);
    } else {
        constexpr int H = E / 4;  // dwords in each half
        const bool a = r * (d[H] & 0xFFFFu) <= code;  // entry E / 2
        uint32_t h[H];
#pragma unroll
        for (int k = 0; k < H; ++k) h[k] = a ? d[H + k] : d[k];
        return piece_last<E / 2>(2u * idx + (a ? 1u : 0u), h, r, code);
    }
}

// The same over NB values one per register (h[0] is taken to qualify).
template <int NB>
KVC_HD uint32_t heads_last(uint32_t idx, const uint32_t *h, uint32_t r, uint32_t code)
{
    if constexpr (NB == 1) {
        return idx;
    } else {
        const bool a = kvc_umul24(r, h[NB / 2]) <= code;
        uint32_t g[NB / 2];
#pragma unroll
        for (int k = 0; k < NB / 2; ++k) g[k] = a ? h[NB / 2 + k] : h[k];
        return heads_last<NB / 2>(2u * idx + (a ? 1u : 0u), g, r, code);
    }
}

// Two-level form of cdf_search for rows padded to 2^NSTEP = 8 * NB entries
// (NSTEP 3 .. 6): b = the last block head row[8b] that qualifies (row[0] is
// taken to), then the last qualifying entry of row[8b .. 8b + 7], those 8
// entries read as one 16-byte piece (piece(b) returns them two per dword,
// the lower index in the low half); both searches run over registers.  On a
// non-decreasing padded row the qualifying entries form a prefix, so this is
// the k binary lifting finds, with two dependent table reads instead of NSTEP.
// PAD: the row has padding (A < 2^NSTEP), so the result is clamped to A - 1.
template <int NSTEP, bool PAD, class Row, class Piece>
KVC_HD uint32_t cdf_search_blocks(const Row &row, const Piece &piece, uint32_t A, uint32_t r,
                                  uint32_t code)
{
    static_assert(NSTEP >= 3 && NSTEP <= 6, "rows of 8 to 64 entries");
    constexpr int NB = 1 << (NSTEP - 3);
    uint32_t hd[NB];
    hd[0] = 0u;  // row[0]: not compared
#pragma unroll
    for (int i = 1; i < NB; ++i) hd[i] = (uint32_t)row[8 * i];
    const uint32_t b = heads_last<NB>(0u, hd, r, code);
    const kvc_u32x4 v = piece(b);
    const uint32_t dv[4] = {v[0], v[1], v[2], v[3]};
    const uint32_t s = piece_last<8>(b, dv, r, code);
    if constexpr (PAD) return s < A - 1u ? s : A - 1u;
    return s;
}

// Decode one symbol: search `row` (padded cumulative frequencies), take its
// packed pair from `pairs`, narrow the interval.  *bad |= 1 when the stream
// left its interval.  The caller refills bb (dec_refill) before every second
// symbol.
template <int NSTEP, class Row, class Pairs>
KVC_HD uint32_t dec_symbol(DecState &d, const Row &row, const Pairs &pairs, uint32_t A,
                           uint32_t *bad)
{
    const uint32_t r = d.range >> 16;
    const uint32_t s = cdf_search<NSTEP>(row, A, r, d.code);
    const uint32_t p = pairs[s];
    *bad |= dec_advance(d, r, p & 0xFFFFu, p >> 16);
    return s;
}

// dec_symbol with the two-level search (cdf_search_blocks).
template <int NSTEP, bool PAD, class Row, class Piece, class Pairs>
KVC_HD uint32_t dec_symbol_blocks(DecState &d, const Row &row, const Piece &piece, const Pairs &pairs,
                                  uint32_t A, uint32_t *bad)
{
    const uint32_t r = d.range >> 16;
    const uint32_t s = cdf_search_blocks<NSTEP, PAD>(row, piece, A, r, d.code);
    const uint32_t p = pairs[s];
    *bad |= dec_advance(d, r, p & 0xFFFFu, p >> 16);
    return s;
}

// Binary-lifting steps for an alphabet of A symbols: log2 of the next power of two.
KVC_HD uint32_t cdf_nstep(uint32_t A)
{
    uint32_t n = 0;
    while ((1u << n) < A) ++n;
    return n;
}

// ------------------------------------ decoder fed by a byte-position window
//
// Renormalisation shifts code left by n = 0, 8 or 16 bits (a whole number of
// bytes) and brings in the next n stream bits.  WinIn keeps posb, the stream
// position (in bits, a multiple of 8) of the first bit not yet in code, and
// hands out the 32 stream bits from there as one window: ring dwords
// posb/32 and posb/32 + 1 funnel-shifted by posb mod 32.  Narrowing and
// renormalising are then code = the high half of ((code - r*st) : window)
// << n and posb += n: no bit buffer to count and top up per symbol.
//
// The ring holds 16 stream dwords per lane (dword j at slot j mod 16) and a
// 17th slot with a copy of slot 0, so a window read at slot 15 needs no
// wrap.  The ring starts full (stream dwords 0..15), so a stream of up to 64
// bytes needs no further loads.  Feeding is RingIn's: a 16-byte piece (4
// stream dwords) is fetched one group of 8 symbols before it is committed;
// pieces past the stream's end are written as zeros without a load.  At a
// group start, after the commit, w - posb/32 >= 6 holds: the group consumes
// at most 16 bytes (4 dwords) and a window needs 2 dwords, and a piece is
// asked for whenever w - posb/32 <= 10, so the next group starts with at
// least 6 again.  A commit overwrites the slots of dwords w - 16 .. w - 13,
// none of which is still needed (w - posb/32 <= 10 when the piece was asked
// for).
template <class Ring>
struct WinIn {
    const uint8_t *p;  // base + a0
    Ring ring;         // this lane's 17 ring slots
    uint32_t len;      // stream length in bytes
    int32_t lim16;     // largest offset from p at which a 16-byte piece may be loaded (>= -12)
    uint32_t sh;       // (start & 3) * 8
    uint32_t w;        // stream dwords committed: [0, w), a multiple of 4
    uint32_t posb;     // stream bit position of the next bit not yet in code
    uint32_t last;     // raw dword w: the low part of stream dword w
    kvc_u32x4 st;      // the piece in flight: raw dwords w+1 .. w+4, moved back by `back` bytes
    uint32_t back;     // how far the piece was moved back (0 unless near the buffer end)
    uint32_t want;     // a piece is in flight

    KVC_HD void issue()
    {
        const int32_t off = 4 * (int32_t)(w + 1u);
        const int32_t at = off < lim16 ? off : lim16;
        __builtin_memcpy(&st, p + at, 16);
        back = (uint32_t)(off - at);
    }
    // Stream dwords w .. w+3, big-endian, zero past the stream, into the ring.
    KVC_HD void commit()
    {
        kvc_u32x4 r = st;
        if (!kvc_all(back == 0u)) {
            const uint32_t d = back >> 2;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t i = (uint32_t)k + d;
                r[k] = i == 1u ? st[1] : i == 2u ? st[2] : i == 3u ? st[3] : (i == 0u ? st[0] : 0u);
            }
        }
        uint32_t v[4];
        v[0] = kvc_bswap32(kvc_alignbit(r[0], last, sh));
        v[1] = kvc_bswap32(kvc_alignbit(r[1], r[0], sh));
        v[2] = kvc_bswap32(kvc_alignbit(r[2], r[1], sh));
        v[3] = kvc_bswap32(kvc_alignbit(r[3], r[2], sh));
        if (!kvc_all(4u * w + 16u <= len)) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t pos = 4u * (w + (uint32_t)k);
                const uint32_t keep = len > pos ? len - pos : 0u;
                v[k] = keep >= 4u ? v[k] : (keep == 0u ? 0u : v[k] & ~(0xFFFFFFFFu >> (8u * keep)));
            }
        }
        const uint32_t b = w & 12u;
#pragma unroll
        for (int k = 0; k < 4; ++k) ring[b + (uint32_t)k] = v[k];
        if (b == 0u) ring[16] = v[0];
        last = r[3];
        w += 4u;
    }
    // Returns the first 4 stream bytes (the decoder's initial code).
    KVC_HD uint32_t init(const uint8_t *base, uint64_t start, uint64_t length, uint64_t capacity, Ring rg)
    {
        uint64_t a0 = start & ~(uint64_t)3;
        sh = (uint32_t)(start & 3u) * 8u;
        len = (uint32_t)length;
        if (a0 + 4u > capacity) {  // only an empty stream at the very end of the buffer
            a0 = capacity - 4u;
            len = 0;
        }
        p = base + a0;
        const uint64_t room = capacity - 16u;  // the last piece starts here
        lim16 = a0 > room ? -(int32_t)(a0 - room) : (room - a0 > 0x7FFFFFF0u ? 0x7FFFFFF0 : (int32_t)(room - a0));
        ring = rg;
        last = *(const uint32_t *)p;
        // the whole ring, stream dwords 0..15, from four pieces requested
        // together (a piece wholly past the stream is not fetched: commit
        // zeroes every byte past the stream); nothing is in flight after it
        kvc_u32x4 pc[4];
        uint32_t bk[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            w = 4u * (uint32_t)k;
            if (k < 2 || 4u * w < len) {
                issue();
            } else {
                st = kvc_u32x4{0u, 0u, 0u, 0u};
                back = 0u;
            }
            pc[k] = st;
            bk[k] = back;
        }
        w = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            st = pc[k];
            back = bk[k];
            commit();
        }
        want = 0;
        posb = 32;
        return ring[0];
    }
    // Stream dwords w .. w+3 when all of them lie past the stream: zeros,
    // written without a load.
    KVC_HD void zeros()
    {
        const uint32_t b = w & 12u;
#pragma unroll
        for (int k = 0; k < 4; ++k) ring[b + (uint32_t)k] = 0u;
        if (b == 0u) ring[16] = 0u;
        w += 4u;
    }
    // Once per group of 8 symbols.  Pieces wholly past the stream are not
    // fetched: the ring gets zeros instead, so a lane whose stream is all in
    // the ring issues no more loads (and waits for none), which is most lanes
    // where a stream takes a few dozen bytes.
    KVC_HD void group()
    {
        if (want) commit();
        const bool need = w - (posb >> 5) <= 10u;
        want = need && 4u * w < len ? 1u : 0u;
        if (want) issue();
        else if (need) zeros();
    }
    // The 32 stream bits from posb on.
    KVC_HD uint32_t window() const
    {
        const uint32_t j = (posb >> 5) & 15u;
        const uint64_t two = ((uint64_t)ring[j] << 32) | ring[j + 1u];
        return (uint32_t)((two << (posb & 31u)) >> 32);
    }
};

// code - r * st as r * (-st) + code (a 24-bit signed multiply-add on the GPU:
// r < 2^16 and -st >= -65535 both fit 24 signed bits).
KVC_HD uint32_t kvc_mul_nst(uint32_t r, int32_t nst)
{
#if defined(__HIP_DEVICE_COMPILE__)
    return (uint32_t)__mul24((int)r, nst);
#else
    return (uint32_t)((int64_t)r * nst);
#endif
}
KVC_HD uint32_t kvc_mad_nst(uint32_t r, int32_t nst, uint32_t code) { return kvc_mul_nst(r, nst) + code; }

// Narrow to the interval [st, st + fr) found for r = range >> 16 and
// renormalise from the window.  Returns 1 if code left the interval.
template <class In>
KVC_HD uint32_t dec_step_win(uint32_t &code, uint32_t &range, In &in, uint32_t r, uint32_t st,
                             uint32_t fr)
{
    const uint32_t win = in.window();
    const uint32_t c2 = code - r * st;
    const uint32_t rn = r * fr;
    const uint32_t bad = c2 >= rn ? 1u : 0u;
    const uint32_t n = kvc_renorm_bits(rn);
    range = rn << n;
    code = (uint32_t)(((((uint64_t)c2) << 32) | win) << n >> 32);
    in.posb += n;
    return bad;
}

// A CDF row's mode record for the mode-first decoder: the row's one symbol
// whose frequency exceeds 65536 - KVC_MODE_SPAN (there is at most one), or
// none.  Rows of chunks where a channel's symbol hardly varies (most rows of
// the larger workloads) have one; for them every lane of a wave first tries
// that symbol: one multiply-add and one multiply, and a check that every
// lane's code lies in its interval with no renormalisation due.  A row
// without one has frequency 0 in its record, so the check fails for every
// lane and the exact search runs (no separate branch on the kind).
#define KVC_MODE_SPAN 1024u
struct ModeRec {
    uint32_t md;   // the symbol
    int32_t nst;   // -(start of md)
    uint32_t fr;   // frequency of md, or 0 when the row has no such symbol
    uint32_t lv;   // dequantization value of md (fp32 bits)
};

// The two-level search of cdf_search_blocks with its NB block heads given
// (hd[0] = 0; the heads are row[8b], uniform over a wave in the kernels).
template <int NSTEP, bool PAD, class Piece>
KVC_HD uint32_t cdf_search_heads(const uint32_t *hd, const Piece &piece, uint32_t A, uint32_t r,
                                 uint32_t code)
{
    static_assert(NSTEP >= 3 && NSTEP <= 6, "rows of 8 to 64 entries");
    constexpr int NB = 1 << (NSTEP - 3);
    const uint32_t b = heads_last<NB>(0u, hd, r, code);
    const kvc_u32x4 v = piece(b);
    const uint32_t dv[4] = {v[0], v[1], v[2], v[3]};
    const uint32_t s = piece_last<8>(b, dv, r, code);
    if constexpr (PAD) return s < A - 1u ? s : A - 1u;
    return s;
}

// Flags of streams that left their interval, as dec_symbol_mode collects
// them: one lane's flag (BadFlag), or on the GPU a whole wave's as a lane
// mask (BadMask: one compare into a scalar register pair per check, no
// per-lane select and or).
struct BadFlag {
    uint32_t f = 0;
    KVC_HD void add(bool b) { f |= b ? 1u : 0u; }
};
struct BadMask {
    uint64_t m = 0;
#if defined(__HIP_DEVICE_COMPILE__)
    __device__ void add(bool b) { m |= __builtin_amdgcn_ballot_w64(b); }
    __device__ bool mine() const { return ((m >> __lane_id()) & 1u) != 0u; }
#else
    void add(bool b) { m |= b ? 1u : 0u; }
    bool mine() const { return m != 0u; }
#endif
};

// One symbol of the mode-first decoder: the mode record's symbol when every
// lane lands in its interval without renormalising (*fast = 1), else the
// exact two-level search, with the block heads heads(hd) loads (only then:
// the fast path needs none) and pieces of the padded row; ent(s) gives
// symbol s's (start | frequency << 16) pair and its dequantization value
// (fp32 bits), and *lv receives the chosen symbol's.  Returns the symbol;
// bad.add(true) when the stream left its interval.
template <int NSTEP, bool PAD, class Heads, class Piece, class Ent, class In, class Bad>
KVC_HD uint32_t dec_symbol_mode(uint32_t &code, uint32_t &range, In &in, const ModeRec &m,
                                const Heads &heads, const Piece &piece, const Ent &ent, uint32_t A,
                                Bad &bad, uint32_t *fast, uint32_t *lv)
{
    const uint32_t r = range >> 16;
    // The mode's step is taken into code and range at once, so the state
    // needs no copies on the common path; the exact path gets the code back
    // by subtracting the same product (exact modulo 2^32, whatever the
    // record's start word holds) and recomputes both.
    const uint32_t d = kvc_mad_nst(r, m.nst, code);
    const uint32_t rn = kvc_umul24(r, m.fr);
    const bool hit = d < rn && rn >= (1u << 24);
    code = d;
    range = rn;
    *lv = m.lv;
    *fast = 1;
    if (kvc_all(hit)) return m.md;
    *fast = 0;
    code = d - kvc_mul_nst(r, m.nst);
    constexpr int NB = 1 << (NSTEP - 3);
    uint32_t hd[NB];
    heads(hd);
    const uint32_t s = cdf_search_heads<NSTEP, PAD>(hd, piece, A, r, code);
    const kvc_u32x2 e = ent(s);
    bad.add(dec_step_win(code, range, in, r, e[0] & 0xFFFFu, e[0] >> 16) != 0u);
    *lv = e[1];
    return s;
}
