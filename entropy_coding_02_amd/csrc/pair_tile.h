// pair_tile.h - staging of CDF rows into LDS as packed (start, frequency)
// pairs, shared by the encoder and the decoder kernels.
#pragma once

#include "kvc_common.h"
#include "lane_coder.h"

// Stage CDF rows [c0, c0+CT) of a slab as packed (start, frequency) pairs.
// Thread i handles the entry pairs (2j, 2j+1) with index i, i+256, ...: one
// 4-byte load of cdf[2j], cdf[2j+1] plus cdf[2j+2] for the second frequency
// (A is even, so rows and pairs are 4-byte aligned).  load() stages the first
// A entries of rows AR entries long (AR >= A, even; AR = A when omitted): the
// last staged entry's frequency then comes from the row's entry A.
template <int kMaxPer>  // pairs per thread: CT * A / 2 / 256 rounded up
struct PairTile {
    uint32_t w[kMaxPer], n2[kMaxPer];

    __device__ void load(const uint16_t *rows, int c0, int CT, int C, int A, int AR = 0)
    {
        if (AR < A) AR = A;
        const int npairs = CT * (A >> 1);
#pragma unroll
        for (int i = 0; i < kMaxPer; ++i) {
            const int e = (int)threadIdx.x + i * 256;
            w[i] = 0;
            n2[i] = 65536u;
            if (e < npairs) {
                const int cl = e / (A >> 1), k = (e - cl * (A >> 1)) * 2;
                if (c0 + cl < C) {
                    const uint16_t *row = rows + (int64_t)(c0 + cl) * AR;
                    w[i] = *(const uint32_t *)(row + k);
                    if (k + 2 < AR) n2[i] = row[k + 2];
                }
            }
        }
    }
    // The decoder's form: entry k of row cl as the 8-byte (pair, lut[k]) at
    // dst[2 (cl A + k)], so one read gives a symbol's interval and its
    // dequantization value; and the starts as rows of P2 uint16 (the search),
    // entry 0 written as 0, so that it qualifies as on a well-formed row
    // (cdf_0 = 0) and every search finds a k in [0, A).
    template <class D32, class D16, class LUT>
    __device__ void store_with(D32 dst, int CT, int A, D16 dst16, int P2, const LUT &lut) const
    {
        const int npairs = CT * (A >> 1);
#pragma unroll
        for (int i = 0; i < kMaxPer; ++i) {
            const int e = (int)threadIdx.x + i * 256;
            if (e < npairs) {
                const int cl = e / (A >> 1), k = (e - cl * (A >> 1)) * 2;
                const uint32_t st0 = w[i] & 0xFFFFu, st1 = w[i] >> 16;
                *(lds_u32x4 *)(dst + 4 * e) =
                    u32x4{cdf_pair(st0, st1), lut[k], cdf_pair(st1, n2[i]), lut[k + 1]};
                dst16[cl * P2 + k] = (uint16_t)(k == 0 ? 0u : st0);
                dst16[cl * P2 + k + 1] = (uint16_t)st1;
            }
        }
    }
    // The mode-first decoder's form: the (start, frequency) pairs, entry k of
    // row cl at dst[cl A + k] (its dequantization value is read from the
    // slab's table), the starts as rows of P2 uint16 (the search; entry 0
    // written as 0, as in store_with), and a record of RS dwords per channel
    // in rec: ModeRec (dwords 0-3), then the block heads row[8b], b >= 1, as
    // dwords 3 + b.  A head is written by the thread holding entry 8b; the
    // ModeRec only by a thread holding an entry whose frequency exceeds
    // 65536 - KVC_MODE_SPAN (a row has at most one), so a row without one
    // keeps the zero frequency word the staging of the tile before wrote:
    // records alternate between two buffers, and each staging clears the
    // frequency words of the other one (rec_clear), which every wave finished
    // reading before this staging.
    template <class D32, class D16, class LUT>
    __device__ void store_mode(D32 dst, int CT, int A, D16 dst16, int P2, const LUT &lut, D32 rec,
                               D32 rec_clear, int RS) const
    {
        const int npairs = CT * (A >> 1);
#pragma unroll
        for (int i = 0; i < kMaxPer; ++i) {
            const int e = (int)threadIdx.x + i * 256;
            if (e < npairs) {
                const int cl = e / (A >> 1), k = (e - cl * (A >> 1)) * 2;
                const uint32_t st0 = w[i] & 0xFFFFu, st1 = w[i] >> 16;
                const uint32_t p0 = cdf_pair(st0, st1), p1 = cdf_pair(st1, n2[i]);
                *(lds_u32x2 *)(dst + 2 * e) = u32x2{p0, p1};
                *(lds_u32 *)(dst16 + cl * P2 + k) = (k == 0 ? 0u : st0) | (st1 << 16);
                if ((k & 7) == 0 && k > 0) rec[cl * RS + 3 + (k >> 3)] = st0;
                if ((p0 >> 16) > 65536u - KVC_MODE_SPAN)
                    *(lds_u32x4 *)(rec + cl * RS) = u32x4{(uint32_t)k, 0u - st0, p0 >> 16, lut[k]};
                if ((p1 >> 16) > 65536u - KVC_MODE_SPAN)
                    *(lds_u32x4 *)(rec + cl * RS) = u32x4{(uint32_t)(k + 1), 0u - st1, p1 >> 16, lut[k + 1]};
            }
        }
        if ((int)threadIdx.x < CT) rec_clear[(int)threadIdx.x * RS + 2] = 0u;
    }
    // The group decoder's form: row cl as P2 keys start << 16 | frequency (a
    // pair with its halves swapped, so that on a non-decreasing row the keys
    // grow with k), entry 0's start taken as 0 (as on a well-formed row), and
    // entries [A, P2) repeating entry A - 1.
    template <class D32>
    __device__ void store_keys(D32 dst, int CT, int A, int P2) const
    {
        const int npairs = CT * (A >> 1);
#pragma unroll
        for (int i = 0; i < kMaxPer; ++i) {
            const int e = (int)threadIdx.x + i * 256;
            if (e < npairs) {
                const int cl = e / (A >> 1), k = (e - cl * (A >> 1)) * 2;
                const uint32_t st0 = k == 0 ? 0u : (w[i] & 0xFFFFu), st1 = w[i] >> 16;
                const uint32_t p0 = cdf_pair(st0, st1), p1 = cdf_pair(st1, n2[i]);
                const uint32_t k0 = (p0 << 16) | (p0 >> 16), k1 = (p1 << 16) | (p1 >> 16);
                *(lds_u32x2 *)(dst + cl * P2 + k) = u32x2{k0, k1};
                if (k + 2 == A)
                    for (int kk = A; kk < P2; ++kk) dst[cl * P2 + kk] = k1;
            }
        }
    }
    // Also writes the starts as rows of P2 uint16 (for the decoder's search).
    template <class D32, class D16 = lds_u16 *>
    __device__ void store(D32 dst, int CT, int A, D16 dst16 = nullptr, int P2 = 0) const
    {
        const int npairs = CT * (A >> 1);
#pragma unroll
        for (int i = 0; i < kMaxPer; ++i) {
            const int e = (int)threadIdx.x + i * 256;
            if (e < npairs) {
                const uint32_t st0 = w[i] & 0xFFFFu, st1 = w[i] >> 16;
                dst[2 * e] = cdf_pair(st0, st1);
                dst[2 * e + 1] = cdf_pair(st1, n2[i]);
                if (dst16) {
                    const int cl = e / (A >> 1), k = (e - cl * (A >> 1)) * 2;
                    dst16[cl * P2 + k] = (uint16_t)w[i];
                    dst16[cl * P2 + k + 1] = (uint16_t)(w[i] >> 16);
                }
            }
        }
    }
};

