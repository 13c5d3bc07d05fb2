/*
 * kvc_oracle.c - plain, slow, single-threaded CPU reference of the
 * CacheGen-style KV-cache codec (the parity authority for the HIP library).
 *
 * TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the bench's
 * CPU-baseline leg may load it.  It shares no code with the HIP path.
 *
 * Source of each step: the page "CacheGen technical deep dive: efficient
 * compression and streaming of the KV cache" (LMCache write-up of the
 * SIGCOMM'24 CacheGen paper), cited below as [CG] with its section.
 *   quantize    [CG] 2.3 Encoder pipeline, step 1 (vectorized adaptive quantization)
 *   bins/layer  [CG] 2.2 CacheGenConfig, and 2.3 step 1 (layer-wise configuration)
 *   histogram   [CG] 2.3 step 2 (CDF of the quantized symbols, width = max bins)
 *   chunks      [CG] 2.3 step 3 (256-token chunks)
 *   coder       [CG] 1.2 design point 3 and 2.1 (arithmetic coding); the exact
 *               coder is not on the page: a 32-bit range coder with 16-bit
 *               totals, byte renormalisation and a carry cache is taken.
 *   decode      [CG] 2.4 Decoder pipeline, step 1
 *   dequantize  [CG] 2.4 step 2 (undo offset, normalise by MAX, scale by max)
 *
 * Floating point: IEEE binary32, round to nearest even, every operation rounded
 * on its own (built with -ffp-contract=off), denormals kept.
 */
#include "kvc_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ fp16 */

/* IEEE binary16 -> binary32, exact. */
float orc_half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -24); /* zero or subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexpf((float)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* IEEE binary32 -> binary16, round to nearest, ties to even. */
uint16_t orc_float_to_half(float f)
{
    uint16_t sign = signbit(f) ? 0x8000u : 0u;
    float a = fabsf(f);
    if (isnan(f)) return (uint16_t)(sign | 0x7E00u);
    if (a >= 65520.0f) return (uint16_t)(sign | 0x7C00u); /* 65504 + half an ulp rounds to inf */
    if (a < 0x1.0p-14f) {
        /* subnormal range: a multiple of 2^-24; rint uses the current (nearest-even) mode */
        double q = rint((double)a * 16777216.0);
        return (uint16_t)(sign | (uint16_t)q); /* q == 1024 is the smallest normal */
    }
    int e;
    frexpf(a, &e); /* a = fr * 2^e, fr in [0.5, 1) */
    /* 11 significant bits: mantissa integer in [1024, 2048) */
    double q = rint(ldexp((double)a, 11 - e));
    int biased = e - 1 + 15;
    uint32_t bits = ((uint32_t)biased << 10) + (uint32_t)q - 1024u; /* q == 2048 carries into e */
    return (uint16_t)(sign | bits);
}

/* --------------------------------------------------------- a2 + a3: quantize */

/*
 * One group is one (layer, K|V, token) row of C channels ([CG] 2.3 step 1: the
 * max-abs reduction runs over the last axis of the per-layer grouped tensor).
 *   MAX    = bins/2 - 1
 *   max1   = max_c |x_c|
 *   factor = MAX / max1          (one IEEE division; 0 when max1 == 0)
 *   q      = round(x * factor + MAX)   in [0, 2*MAX]
 */
int orc_quantize(int32_t L, int32_t C, int64_t T, const int32_t *bins, const uint16_t *kv,
                 uint8_t *sym, uint16_t *max1)
{
    if (L < 1 || C < 1 || T < 0 || !bins) return ORC_ERR_ARG;
    for (int32_t l = 0; l < L; ++l) {
        for (int kvi = 0; kvi < 2; ++kvi) {
            int32_t nb = bins[l * 2 + kvi];
            if (nb < 4 || nb > 256 || (nb & 1)) return ORC_ERR_ARG;
            int32_t MAX = nb / 2 - 1;
            float M = (float)MAX;
            for (int64_t t = 0; t < T; ++t) {
                int64_t row = ((int64_t)l * 2 + kvi) * T + t;
                const uint16_t *x = kv + row * C;
                uint8_t *q = sym + row * C;

                float m = 0.0f;
                for (int32_t c = 0; c < C; ++c) {
                    float a = fabsf(orc_half_to_float(x[c]));
                    if (!isfinite(a)) return ORC_ERR_NONFINITE;
                    if (a > m) m = a;
                }
                max1[row] = orc_float_to_half(m); /* exact: m is one of the inputs */

                float factor = (m > 0.0f) ? M / m : 0.0f;
                for (int32_t c = 0; c < C; ++c) {
                    float v = orc_half_to_float(x[c]);
                    float p = v * factor;
                    p = p + M;
                    float r = rintf(p);
                    if (r < 0.0f || r > 2.0f * M) return ORC_ERR_ARG; /* cannot happen */
                    q[c] = (uint8_t)(int)r;
                }
            }
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------ a4 + a5: CDF */

/*
 * Per table, layer, K|V and channel c.  A table serves S consecutive chunks
 * (S = tab_chunks, taken as at most NC): table g covers tokens
 * [g*S*Tc, min((g+1)*S*Tc, T)), N_g of them.  S = 1 is the page's reading,
 * one table per chunk ([CG] 2.3 steps 2-3); S > 1 shares one table between
 * the chunks of a group, which the page's per-chunk tables leave open.
 *   n_s   = number of the table's tokens whose symbol in channel c is s, s in [0, A)
 *   C_k   = n_0 + ... + n_{k-1}
 *   cdf_k = k + floor(C_k * (65536 - A) / N_g),   k = 0..A  (cdf_A = 65536)
 * Every symbol keeps a frequency cdf_{s+1} - cdf_s >= 1.
 */
static int64_t eff_tab_chunks(int64_t T, int32_t Tc, int32_t tab_chunks)
{
    const int64_t NC = (T + Tc - 1) / Tc;
    return tab_chunks < NC ? tab_chunks : (NC > 0 ? NC : 1);
}

int orc_cdf(int32_t L, int32_t C, int64_t T, int32_t Tc, int32_t tab_chunks, int32_t A,
            const uint8_t *sym, uint16_t *cdf)
{
    if (L < 1 || C < 1 || T < 0 || Tc < 1 || Tc > 65535 || tab_chunks < 1 || A < 2 || A > 256)
        return ORC_ERR_ARG;
    const int64_t S = eff_tab_chunks(T, Tc, tab_chunks);
    const int64_t span = S * Tc; /* tokens of a full table */
    const int64_t NG = (T + span - 1) / span;
    uint64_t *n = (uint64_t *)malloc(sizeof(uint64_t) * (size_t)A);
    if (!n) return ORC_ERR_ARG;
    const uint64_t K = 65536u - (uint64_t)A;
    for (int64_t g = 0; g < NG; ++g) {
        int64_t t0 = g * span;
        int64_t Ng = (T - t0 < span) ? (T - t0) : span;
        for (int32_t l = 0; l < L; ++l) {
            for (int kvi = 0; kvi < 2; ++kvi) {
                int64_t tab = (g * L + l) * 2 + kvi;
                for (int32_t c = 0; c < C; ++c) {
                    memset(n, 0, sizeof(uint64_t) * (size_t)A);
                    for (int64_t t = t0; t < t0 + Ng; ++t) {
                        uint8_t s = sym[(((int64_t)l * 2 + kvi) * T + t) * C + c];
                        if (s >= A) {
                            free(n);
                            return ORC_ERR_ARG;
                        }
                        n[s] += 1;
                    }
                    uint16_t *row = cdf + (tab * C + c) * A;
                    uint64_t Ck = 0;
                    for (int32_t k = 0; k < A; ++k) {
                        row[k] = (uint16_t)((uint64_t)k + (Ck * K) / (uint64_t)Ng);
                        Ck += n[k];
                    }
                }
            }
        }
    }
    free(n);
    return ORC_OK;
}

/* ----------------------------------------------------------- a6: range coder */

/*
 * Range encoder state (integer arithmetic only):
 *   low   : 33 live bits (bit 32 is a pending carry)
 *   range : 32 bits, kept >= 2^24 between symbols
 *   cache : the last byte shifted out that a carry could still change
 *   pend  : 1 + number of 0xFF bytes waiting behind `cache`
 * Symbol s of a row with cumulative counts cdf (total 65536):
 *   r = range >> 16;  low += r*cdf_s;  range = r*(cdf_{s+1} - cdf_s)
 *   while range < 2^24: range <<= 8 and shift one byte out of low.
 * Finish: round low up to a multiple of 2^24, shift out two more bytes.
 * The first byte out is always 0 and is dropped; trailing 0 bytes are
 * dropped too (the decoder reads zeros past the end of a stream).
 */
typedef struct {
    uint64_t low;
    uint32_t range;
    uint32_t cache;
    uint64_t pend;
    uint8_t *buf;
    int64_t n, cap;
} orc_enc;

static void enc_put(orc_enc *e, uint32_t byte)
{
    if (e->n < e->cap) e->buf[e->n] = (uint8_t)byte;
    e->n += 1;
}

static void enc_shift_low(orc_enc *e)
{
    uint32_t carry = (uint32_t)(e->low >> 32);
    if ((uint32_t)e->low < 0xFF000000u || carry != 0) {
        enc_put(e, (e->cache + carry) & 0xFFu);
        while (e->pend > 1) {
            enc_put(e, (0xFFu + carry) & 0xFFu);
            e->pend -= 1;
        }
        e->pend = 0;
        e->cache = (uint32_t)(e->low >> 24) & 0xFFu;
    }
    e->pend += 1;
    e->low = (e->low & 0x00FFFFFFu) << 8;
}

static uint32_t cdf_at(const uint16_t *row, int32_t A, int32_t k)
{
    return (k >= A) ? 65536u : (uint32_t)row[k];
}

/* Encode one stream: symbol c uses CDF row c (cdf_rows + c*A).  Writes at most
 * `cap` bytes and returns the stream length, or a negative error. */
int64_t orc_encode_stream(const uint8_t *q, int32_t C, int32_t A, const uint16_t *cdf_rows,
                          uint8_t *out, int64_t cap)
{
    if (C < 0 || A < 2 || A > 256) return ORC_ERR_ARG;
    int64_t bufcap = 2 * (int64_t)C + 8;
    uint8_t *buf = (uint8_t *)malloc((size_t)bufcap);
    if (!buf) return ORC_ERR_ARG;
    orc_enc e = {0, 0xFFFFFFFFu, 0, 1, buf, 0, bufcap};
    for (int32_t c = 0; c < C; ++c) {
        const uint16_t *row = cdf_rows + (int64_t)c * A;
        int32_t s = q[c];
        if (s >= A) {
            free(buf);
            return ORC_ERR_ARG;
        }
        uint32_t lo = cdf_at(row, A, s), hi = cdf_at(row, A, s + 1);
        if (hi <= lo) {
            free(buf);
            return ORC_ERR_ARG; /* zero-frequency symbol: not a valid CDF */
        }
        uint32_t r = e.range >> 16;
        e.low += (uint64_t)r * lo;
        e.range = r * (hi - lo);
        while (e.range < (1u << 24)) {
            e.range <<= 8;
            enc_shift_low(&e);
        }
    }
    e.low = (e.low + 0xFFFFFFu) & ~(uint64_t)0xFFFFFFu;
    enc_shift_low(&e);
    enc_shift_low(&e);
    if (e.n > bufcap || e.n < 1 || buf[0] != 0) {
        free(buf);
        return ORC_ERR_ARG; /* impossible by construction */
    }
    int64_t len = e.n - 1;
    while (len > 0 && buf[len] == 0) --len; /* bytes are buf[1..len] */
    if (len > cap) {
        free(buf);
        return ORC_ERR_CAPACITY;
    }
    memcpy(out, buf + 1, (size_t)len);
    free(buf);
    return len;
}

/* ----------------------------------------------------------- a8: range decoder */

/*
 * code = next 4 bytes (big-endian), range = 2^32-1.  Per channel:
 *   r = range >> 16;  s = the largest k with r*cdf_k <= code
 *   code -= r*cdf_s;  range = r*(cdf_{s+1} - cdf_s);  refill bytes while range < 2^24
 * Bytes at or past `len` read as 0.  Returns 1 if the stream was inconsistent
 * with the CDFs (code fell outside the coded interval), else 0.
 */
int orc_decode_stream(const uint8_t *in, int64_t len, int32_t C, int32_t A,
                      const uint16_t *cdf_rows, uint8_t *q)
{
    int64_t pos = 0;
    uint32_t code = 0, range = 0xFFFFFFFFu;
    int corrupt = 0;
    for (int i = 0; i < 4; ++i) {
        code = (code << 8) | (pos < len ? in[pos] : 0u);
        ++pos;
    }
    for (int32_t c = 0; c < C; ++c) {
        const uint16_t *row = cdf_rows + (int64_t)c * A;
        uint32_t r = range >> 16;
        int32_t s = 0;
        for (int32_t k = 1; k < A; ++k)
            if ((uint64_t)r * row[k] <= code) s = k;
        uint32_t lo = cdf_at(row, A, s), hi = cdf_at(row, A, s + 1);
        code -= r * lo;
        range = r * (hi - lo);
        if (code >= range) corrupt = 1;
        while (range < (1u << 24)) {
            range <<= 8;
            code = (code << 8) | (pos < len ? in[pos] : 0u);
            ++pos;
        }
        q[c] = (uint8_t)s;
    }
    return corrupt;
}

/* --------------------------------------------------------- a6 + a7: all streams */

static int64_t chunk_tokens_of(int64_t T, int32_t Tc, int64_t j)
{
    int64_t left = T - j * Tc;
    return left < Tc ? left : Tc;
}

/*
 * Streams in (chunk, layer, K|V, token) order; stream (j, l, kv, t) codes the
 * symbols of token j*Tc+t of (l, kv) with the CDF rows of table
 * (floor(j / S), l, kv), S = chunks per table (orc_cdf).
 * slab_off[s] = bytes of all streams of the slabs before slab s.  Returns the
 * payload size, or a negative error (ORC_ERR_CAPACITY if it exceeds the cap).
 */
int64_t orc_encode(int32_t L, int32_t C, int64_t T, int32_t Tc, int32_t tab_chunks, int32_t A,
                   const uint8_t *sym, const uint16_t *cdf, uint16_t *stream_len, uint64_t *slab_off,
                   uint8_t *payload, int64_t payload_cap)
{
    if (L < 1 || C < 1 || T < 0 || Tc < 1 || Tc > 65535 || tab_chunks < 1 || A < 2 || A > 256)
        return ORC_ERR_ARG;
    int64_t NC = (T + Tc - 1) / Tc;
    const int64_t S = eff_tab_chunks(T, Tc, tab_chunks);
    int64_t tmpcap = 2 * (int64_t)C + 8;
    uint8_t *tmp = (uint8_t *)malloc((size_t)tmpcap);
    if (!tmp) return ORC_ERR_ARG;
    int64_t off = 0, sid = 0, slab = 0;
    int overflow = 0;
    for (int64_t j = 0; j < NC; ++j) {
        int64_t Nj = chunk_tokens_of(T, Tc, j);
        for (int32_t l = 0; l < L; ++l) {
            for (int kvi = 0; kvi < 2; ++kvi, ++slab) {
                slab_off[slab] = (uint64_t)off;
                const int64_t tab = (j / S) * 2 * L + (int64_t)l * 2 + kvi;
                const uint16_t *rows = cdf + tab * C * (int64_t)A;
                for (int64_t t = 0; t < Nj; ++t, ++sid) {
                    const uint8_t *q = sym + (((int64_t)l * 2 + kvi) * T + j * Tc + t) * C;
                    int64_t n = orc_encode_stream(q, C, A, rows, tmp, tmpcap);
                    if (n < 0) {
                        free(tmp);
                        return n;
                    }
                    stream_len[sid] = (uint16_t)n;
                    if (off + n <= payload_cap)
                        memcpy(payload + off, tmp, (size_t)n);
                    else
                        overflow = 1;
                    off += n;
                }
            }
        }
    }
    slab_off[slab] = (uint64_t)off;
    free(tmp);
    return overflow ? ORC_ERR_CAPACITY : off;
}

/* Decode every stream back to symbols [L][2][T][C].  Returns ORC_OK, or
 * ORC_ERR_CORRUPT if any stream was inconsistent. */
int orc_decode(int32_t L, int32_t C, int64_t T, int32_t Tc, int32_t tab_chunks, int32_t A,
               const uint8_t *payload, const uint64_t *slab_off, const uint16_t *stream_len,
               const uint16_t *cdf, uint8_t *sym)
{
    if (L < 1 || C < 1 || T < 0 || Tc < 1 || Tc > 65535 || tab_chunks < 1 || A < 2 || A > 256)
        return ORC_ERR_ARG;
    int64_t NC = (T + Tc - 1) / Tc;
    const int64_t S = eff_tab_chunks(T, Tc, tab_chunks);
    int64_t sid = 0, slab = 0;
    int corrupt = 0;
    for (int64_t j = 0; j < NC; ++j) {
        int64_t Nj = chunk_tokens_of(T, Tc, j);
        for (int32_t l = 0; l < L; ++l) {
            for (int kvi = 0; kvi < 2; ++kvi, ++slab) {
                const int64_t tab = (j / S) * 2 * L + (int64_t)l * 2 + kvi;
                const uint16_t *rows = cdf + tab * C * (int64_t)A;
                uint64_t off = slab_off[slab];
                for (int64_t t = 0; t < Nj; ++t, ++sid) {
                    uint8_t *q = sym + (((int64_t)l * 2 + kvi) * T + j * Tc + t) * C;
                    corrupt |= orc_decode_stream(payload + off, stream_len[sid], C, A, rows, q);
                    off += stream_len[sid];
                }
            }
        }
    }
    return corrupt ? ORC_ERR_CORRUPT : ORC_OK;
}

/* -------------------------------------------------------------- a9: dequantize */

/*
 * [CG] 2.4 step 2, in the page's order:
 *   t = q - MAX;  t = float(t) / MAX;  y = t * max1
 * Output fp32, or fp16 rounded to nearest even from that fp32 value.
 */
int orc_dequantize(int32_t L, int32_t C, int64_t T, const int32_t *bins, const uint8_t *sym,
                   const uint16_t *max1, void *out, int32_t out_fp32)
{
    if (L < 1 || C < 1 || T < 0 || !bins) return ORC_ERR_ARG;
    for (int32_t l = 0; l < L; ++l) {
        for (int kvi = 0; kvi < 2; ++kvi) {
            int32_t nb = bins[l * 2 + kvi];
            if (nb < 4 || nb > 256 || (nb & 1)) return ORC_ERR_ARG;
            int32_t MAX = nb / 2 - 1;
            for (int64_t t = 0; t < T; ++t) {
                int64_t row = ((int64_t)l * 2 + kvi) * T + t;
                float m = orc_half_to_float(max1[row]);
                for (int32_t c = 0; c < C; ++c) {
                    int32_t d = (int32_t)sym[row * C + c] - MAX;
                    float u = (float)d / (float)MAX;
                    float y = u * m;
                    if (out_fp32)
                        ((float *)out)[row * C + c] = y;
                    else
                        ((uint16_t *)out)[row * C + c] = orc_float_to_half(y);
                }
            }
        }
    }
    return ORC_OK;
}
