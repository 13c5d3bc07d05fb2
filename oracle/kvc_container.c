/*
 * kvc_container.c - plain CPU reference of the codec's byte container: the
 * one buffer a serializer hands to storage or the network ([CG] 2.1, the
 * CacheGenSerializer entry; 3.2, to_bytes of a KV tensor), with the CDF
 * tables compacted to each layer's own alphabet.
 *
 * TEST INFRASTRUCTURE ONLY, like kvc_oracle.c: nothing in the product path
 * includes, links, loads or calls it.
 *
 * Format, version 1 (every integer little-endian, every section starting at a
 * multiple of 16 bytes, padding bytes zero):
 *   header   64 bytes: u32 magic 0x3143564B ("KVC1"), u32 version 1, u32 L,
 *            u32 C, u64 T, u32 Tc, u32 A, u64 payload_bytes, u64 total_bytes,
 *            u32 S (chunks per CDF table, 1 .. NC; 1 when there are no chunks),
 *            12 zero bytes
 *   bins     u8 [L][2], the bin count of each (layer, K|V)
 *   cdf      for each table (group g of S chunks, layer l, K|V) in that
 *            order, for each channel c: entries 1 .. b-2 of the table's row c
 *            as u16, where b = bins[l][kv].  The other entries are implied:
 *            entry 0 is 0, and a quantizer with b bins never emits a symbol
 *            above b-2 (2*MAX), so every k >= b-1 has C_k = N_g and entry k
 *            equals k + (65536 - A).  A table without that form is refused.
 *   max1     u16 [L][2][T]
 *   lengths  u16 [n_streams], stream order
 *   payload  payload_bytes bytes, the section padded to at least 16 bytes
 *            (the decoder reads whole 16-byte pieces)
 */
#include <stdint.h>
#include <string.h>

#include "kvc_oracle.h"

#define KVC_MAGIC 0x3143564Bu

static int64_t round16(int64_t x) { return (x + 15) / 16 * 16; }

static void put_u32(uint8_t *p, uint32_t v)
{
    for (int i = 0; i < 4; ++i) p[i] = (uint8_t)(v >> (8 * i));
}

static void put_u64(uint8_t *p, uint64_t v)
{
    for (int i = 0; i < 8; ++i) p[i] = (uint8_t)(v >> (8 * i));
}

static uint32_t get_u32(const uint8_t *p)
{
    uint32_t v = 0;
    for (int i = 0; i < 4; ++i) v |= (uint32_t)p[i] << (8 * i);
    return v;
}

static uint64_t get_u64(const uint8_t *p)
{
    uint64_t v = 0;
    for (int i = 0; i < 8; ++i) v |= (uint64_t)p[i] << (8 * i);
    return v;
}

/* Chunks per table as stored: tab_chunks, at most NC, 1 when NC = 0. */
static int64_t stored_tab_chunks(int64_t T, int32_t Tc, int32_t tab_chunks)
{
    const int64_t NC = (T + Tc - 1) / Tc;
    return tab_chunks < NC ? tab_chunks : (NC > 0 ? NC : 1);
}

/* Section offsets: [0] bins, [1] cdf, [2] max1, [3] lengths, [4] payload, [5] end. */
static int layout(int32_t L, int32_t C, int64_t T, int32_t Tc, int32_t tab_chunks, const int32_t *bins,
                  int64_t payload_bytes, int64_t off[6])
{
    if (L < 1 || C < 1 || T < 0 || Tc < 1 || tab_chunks < 1 || !bins || payload_bytes < 0) return ORC_ERR_ARG;
    const int64_t NC = (T + Tc - 1) / Tc, S = stored_tab_chunks(T, Tc, tab_chunks);
    const int64_t NG = (NC + S - 1) / S;
    int64_t per_chunk = 0; /* compact CDF entries of one table */
    for (int32_t i = 0; i < 2 * L; ++i) {
        if (bins[i] < 4 || bins[i] > 256 || (bins[i] & 1)) return ORC_ERR_ARG;
        per_chunk += (int64_t)C * (bins[i] - 2);
    }
    off[0] = 64;
    off[1] = round16(off[0] + 2 * (int64_t)L);
    off[2] = round16(off[1] + 2 * NG * per_chunk);
    off[3] = round16(off[2] + 2 * (2 * (int64_t)L * T));
    off[4] = round16(off[3] + 2 * (2 * (int64_t)L * T));
    off[5] = off[4] + round16(payload_bytes < 16 ? 16 : payload_bytes);
    return ORC_OK;
}

int64_t orc_container_bytes(int32_t L, int32_t C, int64_t T, int32_t Tc, int32_t tab_chunks,
                            const int32_t *bins, int64_t payload_bytes)
{
    int64_t off[6];
    int rc = layout(L, C, T, Tc, tab_chunks, bins, payload_bytes, off);
    return rc == ORC_OK ? off[5] : rc;
}

int64_t orc_container_payload_offset(int32_t L, int32_t C, int64_t T, int32_t Tc, int32_t tab_chunks,
                                     const int32_t *bins)
{
    int64_t off[6];
    int rc = layout(L, C, T, Tc, tab_chunks, bins, 0, off);
    return rc == ORC_OK ? off[4] : rc;
}

static int32_t max_bins(int32_t L, const int32_t *bins)
{
    int32_t A = 0;
    for (int32_t i = 0; i < 2 * L; ++i) A = bins[i] > A ? bins[i] : A;
    return A;
}

int64_t orc_serialize(int32_t L, int32_t C, int64_t T, int32_t Tc, int32_t tab_chunks,
                      const int32_t *bins, const uint16_t *cdf, const uint16_t *max1,
                      const uint16_t *stream_len, const uint8_t *payload, int64_t payload_bytes,
                      uint8_t *out, int64_t out_cap)
{
    int64_t off[6];
    int rc = layout(L, C, T, Tc, tab_chunks, bins, payload_bytes, off);
    if (rc != ORC_OK) return rc;
    if (out_cap < off[5]) return ORC_ERR_CAPACITY;
    const int32_t A = max_bins(L, bins);
    const uint32_t K = 65536u - (uint32_t)A;
    const int64_t NC = (T + Tc - 1) / Tc, S = stored_tab_chunks(T, Tc, tab_chunks);
    const int64_t NG = (NC + S - 1) / S;
    memset(out, 0, (size_t)off[5]);

    put_u32(out + 0, KVC_MAGIC);
    put_u32(out + 4, 1);
    put_u32(out + 8, (uint32_t)L);
    put_u32(out + 12, (uint32_t)C);
    put_u64(out + 16, (uint64_t)T);
    put_u32(out + 24, (uint32_t)Tc);
    put_u32(out + 28, (uint32_t)A);
    put_u64(out + 32, (uint64_t)payload_bytes);
    put_u64(out + 40, (uint64_t)off[5]);
    put_u32(out + 48, (uint32_t)S);
    for (int32_t i = 0; i < 2 * L; ++i) out[off[0] + i] = (uint8_t)bins[i];

    uint8_t *p = out + off[1];
    for (int64_t g = 0; g < NG; ++g) {
        for (int32_t lk = 0; lk < 2 * L; ++lk) {
            const int32_t b = bins[lk];
            const int64_t slab = g * 2 * L + lk;
            for (int32_t c = 0; c < C; ++c) {
                const uint16_t *row = cdf + (slab * C + c) * A;
                if (row[0] != 0) return ORC_ERR_ARG;
                for (int32_t k = b - 1; k < A; ++k)
                    if (row[k] != (uint32_t)k + K) return ORC_ERR_ARG;
                for (int32_t k = 1; k <= b - 2; ++k) {
                    p[0] = (uint8_t)row[k];
                    p[1] = (uint8_t)(row[k] >> 8);
                    p += 2;
                }
            }
        }
    }
    const int64_t n_rows = 2 * (int64_t)L * T;
    for (int64_t i = 0; i < n_rows; ++i) {
        out[off[2] + 2 * i] = (uint8_t)max1[i];
        out[off[2] + 2 * i + 1] = (uint8_t)(max1[i] >> 8);
        out[off[3] + 2 * i] = (uint8_t)stream_len[i];
        out[off[3] + 2 * i + 1] = (uint8_t)(stream_len[i] >> 8);
    }
    if (payload_bytes > 0) memcpy(out + off[4], payload, (size_t)payload_bytes);
    return off[5];
}

int orc_deserialize(int32_t L, int32_t C, int64_t T, int32_t Tc, int32_t tab_chunks,
                    const int32_t *bins, const uint8_t *in, int64_t in_bytes, uint16_t *cdf,
                    uint16_t *max1, uint16_t *stream_len, uint64_t *slab_off, int64_t *payload_bytes)
{
    int64_t off[6];
    int rc = layout(L, C, T, Tc, tab_chunks, bins, 0, off);
    if (rc != ORC_OK || in_bytes < 64) return ORC_ERR_ARG;
    const int32_t A = max_bins(L, bins);
    const uint32_t K = 65536u - (uint32_t)A;
    const int64_t S = stored_tab_chunks(T, Tc, tab_chunks);
    if (get_u32(in) != KVC_MAGIC || get_u32(in + 4) != 1 || get_u32(in + 8) != (uint32_t)L ||
        get_u32(in + 12) != (uint32_t)C || get_u64(in + 16) != (uint64_t)T ||
        get_u32(in + 24) != (uint32_t)Tc || get_u32(in + 28) != (uint32_t)A ||
        get_u32(in + 48) != (uint32_t)S)
        return ORC_ERR_ARG;
    const int64_t pb = (int64_t)get_u64(in + 32);
    rc = layout(L, C, T, Tc, tab_chunks, bins, pb, off);
    if (rc != ORC_OK || (int64_t)get_u64(in + 40) != off[5] || in_bytes < off[5]) return ORC_ERR_ARG;
    for (int32_t i = 0; i < 2 * L; ++i)
        if (in[off[0] + i] != (uint8_t)bins[i]) return ORC_ERR_ARG;

    const int64_t NC = (T + Tc - 1) / Tc, NG = (NC + S - 1) / S;
    const uint8_t *p = in + off[1];
    for (int64_t g = 0; g < NG; ++g) {
        for (int32_t lk = 0; lk < 2 * L; ++lk) {
            const int32_t b = bins[lk];
            const int64_t slab = g * 2 * L + lk;
            for (int32_t c = 0; c < C; ++c) {
                uint16_t *row = cdf + (slab * C + c) * A;
                row[0] = 0;
                for (int32_t k = 1; k <= b - 2; ++k) {
                    row[k] = (uint16_t)(p[0] | (p[1] << 8));
                    p += 2;
                }
                for (int32_t k = b - 1; k < A; ++k) row[k] = (uint16_t)((uint32_t)k + K);
            }
        }
    }
    const int64_t n_rows = 2 * (int64_t)L * T;
    for (int64_t i = 0; i < n_rows; ++i) {
        max1[i] = (uint16_t)(in[off[2] + 2 * i] | (in[off[2] + 2 * i + 1] << 8));
        stream_len[i] = (uint16_t)(in[off[3] + 2 * i] | (in[off[3] + 2 * i + 1] << 8));
    }
    /* slab offsets: running sum of the stream lengths, slab by slab */
    uint64_t run = 0;
    int64_t sid = 0;
    for (int64_t j = 0; j < NC; ++j) {
        const int64_t Nj = (T - j * Tc < Tc) ? (T - j * Tc) : Tc;
        for (int32_t lk = 0; lk < 2 * L; ++lk) {
            slab_off[j * 2 * L + lk] = run;
            for (int64_t t = 0; t < Nj; ++t) run += stream_len[sid++];
        }
    }
    slab_off[NC * 2 * L] = run;
    if ((int64_t)run != pb) return ORC_ERR_CORRUPT;
    *payload_bytes = pb;
    return ORC_OK;
}
