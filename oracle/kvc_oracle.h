/*
 * kvc_oracle.h - plain, slow, single-threaded CPU reference of the
 * CacheGen-style KV-cache codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code: only the tests, the smoke check and the bench's CPU
 * baseline leg use it.  It shares no code with the HIP library.
 *
 * Layouts (all row-major):
 *   kv, out      [L][2][T][C]    fp16 bits (or fp32 for out), (layer, K|V, token, channel)
 *   sym          [L][2][T][C]    uint8 symbols in [0, bins-2]
 *   max1         [L][2][T]       fp16 bits, per-row max |x|
 *   cdf          [NG][L][2][C][A] uint16, one table per S = tab_chunks chunks (S = 1:
 *                per chunk), NG = ceil(NC / S), NC = ceil(T/Tc); cdf[A] = 65536 is implicit
 *   stream_len   [NC][L][2][Nj]  uint16, Nj = tokens of chunk j
 *   slab_off     [NC*L*2 + 1]    uint64 byte offset of each (chunk, layer, K|V) slab
 *   payload      bytes of all streams, in stream order (chunk, layer, K|V, token)
 */
#ifndef KVC_ORACLE_H
#define KVC_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    ORC_OK = 0,
    ORC_ERR_ARG = -1,
    ORC_ERR_NONFINITE = -2,
    ORC_ERR_CAPACITY = -3,
    ORC_ERR_CORRUPT = -4
};

float orc_half_to_float(uint16_t h);
uint16_t orc_float_to_half(float f);

int orc_quantize(int32_t L, int32_t C, int64_t T, const int32_t *bins, const uint16_t *kv,
                 uint8_t *sym, uint16_t *max1);
int orc_cdf(int32_t L, int32_t C, int64_t T, int32_t Tc, int32_t tab_chunks, int32_t A,
            const uint8_t *sym, uint16_t *cdf);
int64_t orc_encode_stream(const uint8_t *q, int32_t C, int32_t A, const uint16_t *cdf_rows,
                          uint8_t *out, int64_t cap);
int orc_decode_stream(const uint8_t *in, int64_t len, int32_t C, int32_t A,
                      const uint16_t *cdf_rows, uint8_t *q);
int64_t orc_encode(int32_t L, int32_t C, int64_t T, int32_t Tc, int32_t tab_chunks, int32_t A,
                   const uint8_t *sym, const uint16_t *cdf, uint16_t *stream_len, uint64_t *slab_off,
                   uint8_t *payload, int64_t payload_cap);
int orc_decode(int32_t L, int32_t C, int64_t T, int32_t Tc, int32_t tab_chunks, int32_t A,
               const uint8_t *payload, const uint64_t *slab_off, const uint16_t *stream_len,
               const uint16_t *cdf, uint8_t *sym);
int orc_dequantize(int32_t L, int32_t C, int64_t T, const int32_t *bins, const uint8_t *sym,
                   const uint16_t *max1, void *out, int32_t out_fp32);

/* Byte container with compact CDF tables (kvc_container.c). */
int64_t orc_container_bytes(int32_t L, int32_t C, int64_t T, int32_t Tc, int32_t tab_chunks,
                            const int32_t *bins, int64_t payload_bytes);
int64_t orc_container_payload_offset(int32_t L, int32_t C, int64_t T, int32_t Tc, int32_t tab_chunks,
                                     const int32_t *bins);
int64_t orc_serialize(int32_t L, int32_t C, int64_t T, int32_t Tc, int32_t tab_chunks,
                      const int32_t *bins, const uint16_t *cdf, const uint16_t *max1,
                      const uint16_t *stream_len, const uint8_t *payload, int64_t payload_bytes,
                      uint8_t *out, int64_t out_cap);
int orc_deserialize(int32_t L, int32_t C, int64_t T, int32_t Tc, int32_t tab_chunks,
                    const int32_t *bins, const uint8_t *in, int64_t in_bytes, uint16_t *cdf,
                    uint16_t *max1, uint16_t *stream_len, uint64_t *slab_off, int64_t *payload_bytes);

/* 8-bit comparator quantizer, [KVM] 四 (kvc_int8.c): groups of g channels. */
/* Token-delta coding with anchors every G chunk-relative tokens (kvc_delta.c). */
int orc_delta_forward(int32_t L, int32_t C, int64_t T, int32_t Tc, int32_t G, const int32_t *bins,
                      const uint16_t *kv, uint16_t *out);
int orc_delta_inverse(int32_t L, int32_t C, int64_t T, int32_t Tc, int32_t G, uint16_t *y);

int orc_int8_quantize(int32_t L, int32_t C, int64_t T, int32_t g, const uint16_t *kv, uint8_t *q,
                      float *scale, uint8_t *zp);
int orc_int8_dequantize(int32_t L, int32_t C, int64_t T, int32_t g, const uint8_t *q,
                        const float *scale, const uint8_t *zp, void *out, int32_t out_fp32);

#ifdef __cplusplus
}
#endif
#endif
