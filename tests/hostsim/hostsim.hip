// hostsim.hip - the GPU lane coder (entropy_coding_02_amd/csrc/lane_coder.h)
// compiled for the host, so CPU tests can compare it with the oracle stream
// by stream before any kernel runs.  Test infrastructure only.
#include <stdint.h>
#include <string.h>
#include <vector>

#include "../../entropy_coding_02_amd/csrc/kvc_common.h"
#include "../../entropy_coding_02_amd/csrc/lane_coder.h"

extern "C" {

// The kernels' XCD-aware block renumbering (kvc_common.h).
int64_t hostsim_xcd_block(int64_t b, int64_t nb) { return xcd_block(b, nb); }

// The kernels' packed test for symbol bytes >= A (kvc_common.h).
uint32_t hostsim_bytes_ge(uint32_t w, uint32_t A) { return kvc_bytes_ge(w, A); }

// Encode one stream into `slot` (>= round_up(2C+16, 16) bytes); returns its length.
int64_t hostsim_encode_stream(const uint8_t *q, int32_t C, int32_t A, const uint16_t *cdf_rows,
                              uint8_t *slot)
{
    EncState e;
    enc_init(e);
    SlotOut out{(uint32_t *)slot, 0, 1};
    for (int32_t c = 0; c < C; ++c) {
        const uint16_t *row = cdf_rows + (int64_t)c * A;
        uint32_t s = q[c] < (uint32_t)A ? q[c] : (uint32_t)A - 1u;
        uint32_t nx = s + 1 < (uint32_t)A ? row[s + 1] : 65536u;
        enc_pair(e, cdf_pair(row[s], nx), out);
    }
    return enc_finish(e, out);
}

// Encode one stream the way the split encoder kernel does with G lanes
// (lane_coder.h, "one stream coded by G lanes"): the range chain over the
// whole stream, then each block of ceil(C/G) channels coded alone with its
// bytes written at their stream positions, then the blocks' lows and
// 0xFFFFFF added and the tail trimmed.  Same slot and result as
// hostsim_encode_stream.
int64_t hostsim_encode_stream_split(const uint8_t *q, int32_t C, int32_t A, const uint16_t *cdf_rows,
                                    uint8_t *slot, int32_t G)
{
    auto pair_of = [&](int32_t c) {
        const uint16_t *row = cdf_rows + (int64_t)c * A;
        const uint32_t s = q[c] < (uint32_t)A ? q[c] : (uint32_t)A - 1u;
        return cdf_pair(row[s], s + 1 < (uint32_t)A ? row[s + 1] : 65536u);
    };
    const int32_t B = (C + G - 1) / G;
    std::vector<uint32_t> r0(G), s0(G + 1);
    uint32_t range = 0xFFFFFFFFu, S = 0;
    for (int32_t c = 0; c < C; ++c) {
        if (c % B == 0) {
            r0[c / B] = range;
            s0[c / B] = S;
        }
        S += enc_range_step(range, pair_of(c) >> 16);
    }
    for (int32_t g = (C + B - 1) / B; g < G; ++g) {  // blocks past the last channel
        r0[g] = range;
        s0[g] = S;
    }
    s0[G] = S;
    const SplitOut f{slot, 0};
    std::vector<uint32_t> lo(G);
    for (int32_t g = 0; g < G; ++g) {
        EncState e;
        enc_init(e);
        e.range = r0[g];
        const SplitOut out{slot, s0[g] / 8u};
        for (int32_t c = g * B; c < C && c < (g + 1) * B; ++c) enc_pair_nb(e, pair_of(c), out);
        enc_block_end(e, out);
        lo[g] = e.lo;
    }
    for (uint32_t b = 0; b < 4u; ++b) *f.byte(S / 8u + b) = (uint8_t)(lo[G - 1] >> (24u - 8u * b));
    for (int32_t g = 0; g + 1 < G; ++g) split_add(f, s0[g + 1] / 8u, lo[g], 4);
    const uint32_t nt = S / 8u + 4u;
    split_add(f, nt - 3u, 0xFFFFFFu, 3);
    return split_trim(f, nt - 3u);
}

// Decode the stream at [off, off+len) of a buffer of `cap` bytes (a multiple
// of 4, at least 4); returns the corrupt flag.
// search 0: binary lifting; 1: the two-level search where the padded row has
// 8 to 64 entries (binary lifting otherwise); 2: the mode-first decoder with
// the window feed there (fast_count, if not NULL, counts its fast symbols).
int hostsim_decode_stream_n(const uint8_t *buf, int64_t cap, int64_t off, int64_t len, int32_t C,
                            int32_t A, const uint16_t *cdf_rows, uint8_t *q, int32_t search,
                            int64_t *fast_count)
{
    uint32_t ring[16], ring2[17];
    RingIn<uint32_t *> in;
    in.init(buf, (uint64_t)off, (uint64_t)len, (uint64_t)cap, ring);
    DecState d;
    dec_init(d, in);
    WinIn<uint32_t *> win;  // the mode-first decoder's feed (search 2)
    uint32_t wcode = win.init(buf, (uint64_t)off, (uint64_t)len, (uint64_t)cap, ring2), wrange = 0xFFFFFFFFu;
    uint32_t bad = 0, nstep = cdf_nstep((uint32_t)A), P2 = 1u << nstep;
    BadFlag wbad;  // the mode-first decoder's flag
    std::vector<uint16_t> padded(P2);
    std::vector<uint32_t> pairs(A);
    for (int32_t c = 0; c < C; ++c) {
        if ((c & 7) == 0) in.group();
        if ((c & 7) == 0) win.group();
        if ((c & 1) == 0) dec_refill(d, in);
        const uint16_t *row = cdf_rows + (int64_t)c * A;
        for (uint32_t k = 0; k < P2; ++k) padded[k] = k < (uint32_t)A ? row[k] : 0xFFFFu;
        for (int32_t k = 0; k < A; ++k) pairs[k] = cdf_pair(row[k], k + 1 < A ? row[k + 1] : 65536u);
        auto piece = [&](uint32_t b) {
            kvc_u32x4 v;
            memcpy(&v, padded.data() + 8 * b, 16);
            return v;
        };
        uint32_t sym;
        if (search == 2 && nstep >= 3 && nstep <= 6) {
            // the mode-first decoder (lane_coder.h dec_symbol_mode), its record
            // and block heads built from the row as the kernel's staging does
            ModeRec m{0u, 0, 0u, 0u};
            for (int32_t k = 0; k < A; ++k) {
                const uint32_t pr = pairs[k];
                if ((pr >> 16) > 65536u - KVC_MODE_SPAN)
                    m = ModeRec{(uint32_t)k, -(int32_t)(pr & 0xFFFFu), pr >> 16, 0u};
            }
            auto hd = [&](uint32_t *h) {
                h[0] = 0u;
                for (uint32_t b = 1; b < (P2 >> 3); ++b) h[b] = padded[8 * b];
            };
            uint32_t fast = 0;
            auto pa = [&](uint32_t k) { return kvc_u32x2{pairs[k], 0u}; };
            uint32_t lvv = 0;
            switch (nstep) {
            case 3: sym = (uint32_t)A < 8u ? dec_symbol_mode<3, true>(wcode, wrange, win, m, hd, piece, pa, (uint32_t)A, wbad, &fast, &lvv) : dec_symbol_mode<3, false>(wcode, wrange, win, m, hd, piece, pa, (uint32_t)A, wbad, &fast, &lvv); break;
            case 4: sym = (uint32_t)A < 16u ? dec_symbol_mode<4, true>(wcode, wrange, win, m, hd, piece, pa, (uint32_t)A, wbad, &fast, &lvv) : dec_symbol_mode<4, false>(wcode, wrange, win, m, hd, piece, pa, (uint32_t)A, wbad, &fast, &lvv); break;
            case 5: sym = (uint32_t)A < 32u ? dec_symbol_mode<5, true>(wcode, wrange, win, m, hd, piece, pa, (uint32_t)A, wbad, &fast, &lvv) : dec_symbol_mode<5, false>(wcode, wrange, win, m, hd, piece, pa, (uint32_t)A, wbad, &fast, &lvv); break;
            default: sym = (uint32_t)A < 64u ? dec_symbol_mode<6, true>(wcode, wrange, win, m, hd, piece, pa, (uint32_t)A, wbad, &fast, &lvv) : dec_symbol_mode<6, false>(wcode, wrange, win, m, hd, piece, pa, (uint32_t)A, wbad, &fast, &lvv); break;
            }
            q[c] = (uint8_t)sym;
            if (fast_count) *fast_count += fast;
            continue;
        }
        if (search == 1 && nstep >= 3 && nstep <= 6) {
            switch (nstep) {
            case 3: sym = (uint32_t)A < (1u << 3) ? dec_symbol_blocks<3, true>(d, padded.data(), piece, pairs.data(), (uint32_t)A, &bad) : dec_symbol_blocks<3, false>(d, padded.data(), piece, pairs.data(), (uint32_t)A, &bad); break;
            case 4: sym = (uint32_t)A < (1u << 4) ? dec_symbol_blocks<4, true>(d, padded.data(), piece, pairs.data(), (uint32_t)A, &bad) : dec_symbol_blocks<4, false>(d, padded.data(), piece, pairs.data(), (uint32_t)A, &bad); break;
            case 5: sym = (uint32_t)A < (1u << 5) ? dec_symbol_blocks<5, true>(d, padded.data(), piece, pairs.data(), (uint32_t)A, &bad) : dec_symbol_blocks<5, false>(d, padded.data(), piece, pairs.data(), (uint32_t)A, &bad); break;
            default: sym = (uint32_t)A < 64u ? dec_symbol_blocks<6, true>(d, padded.data(), piece, pairs.data(), (uint32_t)A, &bad) : dec_symbol_blocks<6, false>(d, padded.data(), piece, pairs.data(), (uint32_t)A, &bad); break;
            }
            q[c] = (uint8_t)sym;
            continue;
        }
        switch (nstep) {
        case 1: sym = dec_symbol<1>(d, padded.data(), pairs.data(), (uint32_t)A, &bad); break;
        case 2: sym = dec_symbol<2>(d, padded.data(), pairs.data(), (uint32_t)A, &bad); break;
        case 3: sym = dec_symbol<3>(d, padded.data(), pairs.data(), (uint32_t)A, &bad); break;
        case 4: sym = dec_symbol<4>(d, padded.data(), pairs.data(), (uint32_t)A, &bad); break;
        case 5: sym = dec_symbol<5>(d, padded.data(), pairs.data(), (uint32_t)A, &bad); break;
        case 6: sym = dec_symbol<6>(d, padded.data(), pairs.data(), (uint32_t)A, &bad); break;
        case 7: sym = dec_symbol<7>(d, padded.data(), pairs.data(), (uint32_t)A, &bad); break;
        default: sym = dec_symbol<8>(d, padded.data(), pairs.data(), (uint32_t)A, &bad); break;
        }
        q[c] = (uint8_t)sym;
    }
    return (int)(bad | wbad.f);
}

int hostsim_decode_stream(const uint8_t *buf, int64_t cap, int64_t off, int64_t len, int32_t C,
                          int32_t A, const uint16_t *cdf_rows, uint8_t *q, int32_t search)
{
    return hostsim_decode_stream_n(buf, cap, off, len, C, A, cdf_rows, q, search, nullptr);
}

}  // extern "C"
