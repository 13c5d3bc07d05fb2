/*
 * kvc.h - C ABI of libkvc.so, a CacheGen-style KV-cache codec for AMD
 * MI355X (gfx950), written as HIP kernels.
 *
 * The method is the one the page "CacheGen technical deep dive: efficient
 * compression and streaming of the KV cache" (an LMCache write-up of the
 * SIGCOMM'24 CacheGen paper) describes, cited below as [CG]:
 *   - layer-wise adaptive group quantization of fp16 K/V ([CG] 1.2 point 2,
 *     2.2 CacheGenConfig, 2.3 step 1),
 *   - per-(layer, channel) symbol statistics turned into CDFs ([CG] 1.2 point 3,
 *     2.3 step 2),
 *   - parallel arithmetic coding of independent streams in 256-token chunks
 *     ([CG] 2.1, 2.3 step 3),
 *   - parallel decode and dequantization ([CG] 2.4 steps 1-2).
 *
 * Data layout in device memory (row-major):
 *   kv, out      [L][2][T][C]      fp16 (out: fp16 or fp32), (layer, K|V, token, channel)
 *                                   i.e. the kv_shape (layers, 2, tokens, kv_heads, head_dim)
 *                                   of [CG] 3.2 with C = kv_heads * head_dim
 *   sym          [L][2][T][C]      uint8 symbols, in [0, bins-2]
 *   max1         [L][2][T]         fp16 bits: max |x| of each (layer, K|V, token) row
 *   cdf          [NG][L][2][C][A]  uint16 cumulative frequencies out of 65536;
 *                                   cdf[0] = 0, cdf[A] = 65536 is implicit; one table
 *                                   per S consecutive chunks (S = 1: per chunk),
 *                                   NG = ceil(NC / S)
 *   stream_len   [n_streams]       uint16 byte length of each stream
 *   slab_off     [n_slabs + 1]     uint64 payload offset of each slab's first stream
 *   payload      bytes of all streams back to back
 * with A = max bins, NC = ceil(T / chunk_tokens) chunks, a slab = (chunk j,
 * layer l, K|V), slabs in (j, l, kv) order, n_slabs = 2*L*NC, and one stream
 * per (chunk, layer, K|V, token) in that order, n_streams = 2*L*T.  Stream
 * (j, l, kv, t) codes the C symbols of token j*chunk_tokens + t of (l, kv),
 * channel 0 first, with the CDF rows of table (floor(j / S), l, kv).
 *
 * Conventions:
 *   - The caller allocates every buffer.  The library allocates no memory and
 *     keeps no state between calls, except the streams and events kvc_decode
 *     makes on first use on a device (kept until the process ends); calls are
 *     re-entrant.
 *   - Every compute call is asynchronous on `stream` (a hipStream_t; NULL is
 *     the default stream).  Outputs are valid once the stream is synchronised.
 *   - Errors the host can see return a negative kvc_status at once and launch
 *     nothing.  Errors found on the device are OR-ed as KVC_DEV_* bits into
 *     *dev_status (a device int32 the caller zeroes), which may be NULL.
 *   - Pointers to device buffers must be 4-byte aligned (16-byte alignment
 *     enables the vectorised paths); `desc->bins` is a host pointer.
 *   - A descriptor is rejected (KVC_ERR_ARG) when its 1-D launches would not
 *     fit 32-bit grids: 2^29 or more blocks of 256 streams (n_slabs times
 *     ceil(chunk_tokens / 256)), or 2^31 or more blocks of 64 channels.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_VERSION 1

enum kvc_status {
    KVC_OK = 0,
    KVC_ERR_ARG = -1,      /* null/misaligned pointer, bad bins, size out of range */
    KVC_ERR_CAPACITY = -2, /* a caller buffer is smaller than the call needs */
    KVC_ERR_HIP = -3       /* a HIP launch failed */
};

/* device-side findings, OR-ed into *dev_status */
#define KVC_DEV_NONFINITE 1        /* a row max was Inf or NaN (kvc_quantize) */
#define KVC_DEV_CORRUPT 2          /* a stream left its coding interval (kvc_decode) */
#define KVC_DEV_PAYLOAD_OVERFLOW 4 /* the packed payload did not fit (kvc_encode, kvc_serialize) */
#define KVC_DEV_BAD_CDF 8          /* a CDF row the container cannot carry (kvc_serialize) */
#define KVC_DEV_BAD_CONTAINER 16   /* a container that does not match the descriptor (kvc_deserialize) */
#define KVC_DEV_BAD_SYMBOL 32      /* a symbol >= A, outside every CDF row (kvc_cdf, kvc_encode) */
/* Bit 30 is used within a kvc_encode call (set and cleared on its stream); no
 * call leaves it set. */

enum kvc_dtype { KVC_F16 = 0, KVC_F32 = 1 };

typedef struct kvc_desc {
    int32_t n_layers;     /* L, 1..256 */
    int32_t n_channels;   /* C = kv_heads * head_dim, 1..16384 */
    int64_t n_tokens;     /* T >= 0 */
    int32_t chunk_tokens; /* tokens per chunk, 1..65535 ([CG] 2.3 step 3 uses 256) */
    int32_t cdf_chunks;   /* S, chunks sharing one CDF table: 0 or 1 = a table per chunk
                             (the page's reading); S > 1 = groups of S consecutive chunks;
                             S >= NC = one table per (layer, K|V, channel).  Taken as at
                             most NC; a table may count at most 2^21 tokens
                             (min(S * chunk_tokens, T) <= 2^21) */
    const int32_t *bins;  /* HOST [L][2] (K, V) bin counts, even, 4..256 ([CG] 2.2) */
} kvc_desc;

/* Library version (KVC_VERSION). */
int kvc_version(void);

/* Static text for a kvc_status value. */
const char *kvc_status_string(int status);

/* Sizes.  Each returns a negative kvc_status if the descriptor is invalid.
 *   kvc_alphabet          A = max over layers and K|V of bins ([CG] 2.3 step 2
 *                         sizes the CDF by the largest bins value)
 *   kvc_scratch_bytes     device scratch kvc_encode needs: a slot of
 *                         round_up(2C+16, 16) bytes for each of the 256 token
 *                         rows of every slab's ceil(chunk_tokens/256) slot
 *                         regions, plus 8 bytes per slab
 *   kvc_max_payload_bytes an upper bound of the payload: n_streams * (2C+1) */
int32_t kvc_alphabet(const kvc_desc *desc);
int64_t kvc_n_chunks(const kvc_desc *desc);
int64_t kvc_n_slabs(const kvc_desc *desc);
int64_t kvc_n_streams(const kvc_desc *desc);
/* Lanes per stream kvc_decode launches with for this shape: 4 (8 for rows of
 * 33 to 64 entries) when there are at most 16384 streams and the alphabet pads
 * to 8 to 64 entries, so that a small launch spreads each stream's search
 * over several lanes; else 1.  Informational: the output is the same. */
int32_t kvc_decode_lanes(const kvc_desc *desc);
int64_t kvc_cdf_bytes(const kvc_desc *desc);
int64_t kvc_scratch_bytes(const kvc_desc *desc);
int64_t kvc_max_payload_bytes(const kvc_desc *desc);

/*
 * Group quantization, [CG] 2.3 step 1 (and 2.2 for the per-layer bins).
 * For each (layer l, K|V, token) row x of C channels, with MAX = bins/2 - 1:
 *   max1 = max_c |x_c|                       (exact, stored as fp16)
 *   factor = MAX / max1                      (one IEEE fp32 division; 0 if max1 = 0)
 *   sym_c = round_half_even(fp32(x_c * factor) + MAX)   in [0, 2*MAX]
 * every fp32 operation rounded on its own (no fused multiply-add).
 *   kv    [L][2][T][C] fp16 (device, read)
 *   sym   [L][2][T][C] uint8 (device, written)
 *   max1  [L][2][T] fp16 bits (device, written)
 *   cdf   NULL, or [NC][L][2][C][A] uint16 (device, written): when given, the
 *         CDFs of kvc_cdf are produced in the same pass
 * A row holding Inf or NaN sets KVC_DEV_NONFINITE; its outputs are unspecified.
 */
int kvc_quantize(const kvc_desc *desc, const uint16_t *kv, uint8_t *sym, uint16_t *max1,
                 uint16_t *cdf, int32_t *dev_status, void *stream);

/*
 * Several quality levels of one tensor: exactly what kvc_quantize(levels[i],
 * kv, sym[i], max1, cdf[i]) gives for each i, from one pass over kv where the
 * shape allows (the row max is shared; each level has its own bins table,
 * symbols and CDFs).  Each level is then encoded with kvc_encode; chunks of
 * different levels can be sent chunk by chunk (kvc_serialize_chunk), the
 * bandwidth adaptation that chunking serves ([CG] 2.3 step 3, [CG] 4 point 2).
 *   levels     HOST array of n_levels descriptors (1 <= n_levels <= 4) with the same
 *              n_layers, n_channels, n_tokens and chunk_tokens; bins may differ
 *   sym, cdf   HOST arrays of n_levels device pointers (written), laid out as in kvc_quantize
 *   max1       [L][2][T] (device, written once for all levels)
 */
int kvc_quantize_levels(const kvc_desc *levels, int32_t n_levels, const uint16_t *kv,
                        uint8_t *const *sym, uint16_t *max1, uint16_t *const *cdf,
                        int32_t *dev_status, void *stream);

/*
 * Symbol statistics to CDFs, [CG] 2.3 step 2, per 256-token chunk (step 3).
 * For chunk j with N_j tokens, layer, K|V and channel c: n_s = count of
 * symbol s in the chunk's column, C_k = n_0 + .. + n_{k-1}, K = 65536 - A,
 *   cdf_k = k + floor(C_k * K / N_j),  k = 0..A-1     (every frequency >= 1)
 *   sym         [L][2][T][C] uint8 (device, read)
 *   cdf         [NC][L][2][C][A] uint16 (device, written)
 *   dev_status  device int32 (or NULL): a symbol >= A sets KVC_DEV_BAD_SYMBOL,
 *               and the CDFs of its slab are then unspecified (the kernels
 *               stay inside their buffers)
 */
int kvc_cdf(const kvc_desc *desc, const uint8_t *sym, uint16_t *cdf, int32_t *dev_status,
            void *stream);

/*
 * Range coding of every stream and packing, [CG] 2.1 (ac_enc) and 1.2 point 3.
 * Per stream: r = range >> 16; low += r*cdf_s; range = r*f_s; renormalise by
 * bytes while range < 2^24; at the end round low up to a multiple of 2^24;
 * the stream is that number in base 256 without its zero first byte and
 * without trailing zero bytes.  Then stream_len, the slab offsets (exclusive
 * scan) and the payload (streams back to back in stream order) are written.
 *   sym         [L][2][T][C] uint8 (device, read)
 *   cdf         [NC][L][2][C][A] uint16 (device, read)
 *   scratch     device scratch of scratch_bytes >= kvc_scratch_bytes (else KVC_ERR_CAPACITY)
 *   stream_len  [n_streams] uint16 (device, written)
 *   slab_off    [n_slabs + 1] uint64 (device, written; slab_off[n_slabs] = payload size)
 *   payload     payload_cap bytes (device, written); if the payload is larger,
 *               KVC_DEV_PAYLOAD_OVERFLOW is set and only bytes below the cap are written
 * A symbol >= A sets KVC_DEV_BAD_SYMBOL; the streams of its slab are then
 * unspecified (it has no CDF interval to be coded with).
 * Launches (all on `stream`): when layers have fewer bins than A and
 * dev_status is not NULL, the coder is launched once per run of layers whose
 * symbols fit the same power-of-two prefix of the CDF rows, staging only that
 * prefix; a symbol past it (legal in its row) makes a last guard launch code
 * every stream again over whole rows, so the output never depends on it.
 */
int kvc_encode(const kvc_desc *desc, const uint8_t *sym, const uint16_t *cdf, void *scratch,
               int64_t scratch_bytes, uint16_t *stream_len, uint64_t *slab_off, uint8_t *payload,
               int64_t payload_cap, int32_t *dev_status, void *stream);

/*
 * kvc_encode without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops that forbid
 * allocation).  Same arguments, outputs and flags as kvc_encode, minus
 * scratch/scratch_bytes: the workspace is a device array inside the library,
 * KVC_NOALLOC_SCRATCH_BYTES long, one per GPU (held until the process ends;
 * its address is looked up on the first call on each device).  The call
 * allocates nothing.  A shape whose kvc_scratch_bytes exceeds that size
 * returns KVC_ERR_CAPACITY and launches nothing (e.g. one 256-token chunk of
 * 32 layers x 1024 channels fits; 8K tokens do not).  Every call on a GPU
 * uses that GPU's one array: calls that overlap in time on one GPU (other
 * streams, other host threads) race and must be serialised by the caller.
 */
#define KVC_NOALLOC_SCRATCH_BYTES (64u << 20)
int kvc_encode_noalloc(const kvc_desc *desc, const uint8_t *sym, const uint16_t *cdf,
                       uint16_t *stream_len, uint64_t *slab_off, uint8_t *payload, int64_t payload_cap,
                       int32_t *dev_status, void *stream);

/*
 * Parallel decode with fused dequantization, [CG] 2.4 steps 1-2.
 * Per stream: code = first 4 bytes (big-endian), range = 2^32-1; per channel
 * r = range >> 16, s = the largest k with r*cdf_k <= code, code -= r*cdf_s,
 * range = r*f_s, refill bytes while range < 2^24 (bytes past the stream read
 * as 0).  Then y = fp32(fp32(s - MAX) / MAX) * max1, rounded to out_dtype.
 *   payload        payload_bytes bytes (device, read; never read at or past payload_bytes).
 *                  payload_bytes must be a multiple of 4 and at least 16 (the decoder
 *                  reads aligned dwords in 16-byte pieces); it may exceed the packed size.
 *   slab_off       [n_slabs + 1] uint64 (device, read)
 *   stream_len     [n_streams] uint16 (device, read)
 *   cdf            [NC][L][2][C][A] uint16 (device, read)
 *   max1           [L][2][T] fp16 bits (device, read; may be NULL when out is NULL)
 *   sym_out        NULL, or [L][2][T][C] uint8 (device, written): decoded symbols
 *   out            NULL, or [L][2][T][C] of out_dtype (device, written)
 * A stream inconsistent with its CDFs sets KVC_DEV_CORRUPT; C symbols are
 * still written for it.  CDF rows are expected non-decreasing (kvc_quantize,
 * kvc_cdf and kvc_deserialize guarantee it); on a decreasing row the symbol
 * is some k in [0, A).
 * Launches: all on `stream`, except that when layers have fewer bins than A
 * (and dev_status is not NULL) the decode is launched once per run of layers
 * with equal search depth and the runs after the first go on up to three
 * streams the library owns (one set per device, made on first use, default
 * priority), forked from `stream` by an event and joined back into it before
 * a last guard launch on `stream`: all of the call's work is ordered after
 * the work already on `stream`, and later work on `stream` after it (in a
 * captured graph, a fork and a join).  Calls from several host threads take
 * turns on those streams; calls on one device that overlap in time still
 * race on their outputs as usual.
 */
int kvc_decode(const kvc_desc *desc, const uint8_t *payload, int64_t payload_bytes,
               const uint64_t *slab_off, const uint16_t *stream_len, const uint16_t *cdf,
               const uint16_t *max1, uint8_t *sym_out, void *out, int32_t out_dtype,
               int32_t *dev_status, void *stream);

/*
 * Dequantization on its own, [CG] 2.4 step 2, in the page's order:
 *   y = fp32(fp32(sym - MAX) / MAX) * max1, then rounded to out_dtype.
 *   sym   [L][2][T][C] uint8 (device, read)
 *   max1  [L][2][T] fp16 bits (device, read)
 *   out   [L][2][T][C] of out_dtype (device, written)
 */
int kvc_dequantize(const kvc_desc *desc, const uint8_t *sym, const uint16_t *max1, void *out,
                   int32_t out_dtype, void *stream);

/*
 * Byte container: everything kvc_decode needs, in one buffer for storage or
 * the network (the serializer of [CG] 2.1; to_bytes of a KV tensor in [CG]
 * 3.2).  Each CDF row is cut to its own layer's alphabet: entries 1 .. b-2 of
 * the row are stored (b = bins of its layer and K|V); entry 0 is 0 and every
 * entry k >= b-1 is k + 65536 - A, because a quantizer with b bins never
 * emits a symbol above b-2.  Format, version 1 (little-endian, sections at
 * multiples of 16 bytes, padding zero):
 *   header   64 bytes: u32 magic 0x3143564B ("KVC1"), u32 version 1, u32 L,
 *            u32 C, u64 T, u32 Tc, u32 A, u64 payload_bytes, u64 total_bytes,
 *            16 zero bytes
 *   bins     u8 [L][2]
 *   cdf      per slab (chunk, layer, K|V), per channel: entries 1 .. b-2 (u16)
 *   max1     u16 [L][2][T]
 *   lengths  u16 [n_streams]
 *   payload  the streams, the section at least 16 bytes long
 *
 * kvc_container_bytes          total size for a payload of payload_bytes bytes
 * kvc_container_payload_offset offset of the payload section (a multiple of 16)
 */
int64_t kvc_container_bytes(const kvc_desc *desc, int64_t payload_bytes);
int64_t kvc_container_payload_offset(const kvc_desc *desc);

/*
 * Write the container of an encoded KV cache.
 *   cdf, max1, stream_len, slab_off, payload   as kvc_encode left them (device, read);
 *                the payload size is slab_off[n_slabs], read on the device
 *   out          device, 16-byte aligned, out_cap bytes (written); out_cap below
 *                kvc_container_bytes(desc, 0) returns KVC_ERR_CAPACITY
 * A container larger than out_cap sets KVC_DEV_PAYLOAD_OVERFLOW, and nothing is
 * written at or past out_cap; a CDF row that is not of the form above sets
 * KVC_DEV_BAD_CDF (its implied entries are then lost).
 */
int kvc_serialize(const kvc_desc *desc, const uint16_t *cdf, const uint16_t *max1,
                  const uint16_t *stream_len, const uint64_t *slab_off, const uint8_t *payload,
                  uint8_t *out, int64_t out_cap, int32_t *dev_status, void *stream);

/*
 * The container of one chunk, the streaming unit of [CG] 2.3 step 3 (chunks
 * let a sender follow bandwidth swings, [CG] 4 point 2): chunk `chunk` of the
 * encoded tensor `desc` describes, written as a tensor of its own, i.e.
 * exactly what kvc_serialize writes for the descriptor `desc` with n_tokens
 * set to the chunk's token count N_j (its header says T = N_j).  A receiver
 * reads it with kvc_deserialize and kvc_decode under that descriptor and gets
 * the chunk's rows [L][2][N_j][C].  Encoding one tensor at several bins
 * tables (kvc_quantize_levels) and sending each chunk at the level the link
 * allows is the bandwidth adaptation built on it.
 *   cdf, max1, stream_len, slab_off, payload   of the whole tensor, as kvc_encode left them
 *   out          device, 16-byte aligned, out_cap bytes (written); as kvc_serialize
 * The chunk's payload size is read on the device (a difference of two slab
 * offsets); flags as kvc_serialize.
 */
int kvc_serialize_chunk(const kvc_desc *desc, int64_t chunk, const uint16_t *cdf,
                        const uint16_t *max1, const uint16_t *stream_len, const uint64_t *slab_off,
                        const uint8_t *payload, uint8_t *out, int64_t out_cap, int32_t *dev_status,
                        void *stream);

/*
 * Streaming encoder: compute, compress and transmit at the same time ([CG]
 * 4 point 2), chunk by chunk ([CG] 2.3 step 3).  Chunk j is sent at quality
 * level chunk_level[j] (the sender's schedule, e.g. from the link's measured
 * bandwidth): its container is exactly what kvc_serialize_chunk writes for
 * levels[chunk_level[j]], chunk j (so kvc_deserialize + kvc_decode read it).
 * Chunks go in units of at most `chunks_per_unit` consecutive chunks of one
 * level: on compute_stream a unit is encoded (kvc_encode's kernels, on the
 * unit's rows of sym in place) and its chunk containers are written into a
 * staging area, then moved back to back into one half of a device area; on
 * copy_stream the unit before is copied to host_out meanwhile, in one copy of
 * its containers at their exact sizes.  The host thread reads each unit's
 * container sizes once they are written, to issue that copy, so the call
 * returns only when every container is in host_out (both streams
 * synchronised).
 *   levels       HOST array of n_levels descriptors (1..4), as kvc_quantize_levels:
 *                same n_layers, n_channels, n_tokens, chunk_tokens; bins may differ
 *   chunk_level  HOST int32 [NC], each in [0, n_levels)
 *   sym, cdf     HOST arrays of n_levels device pointers: each level's symbols
 *                [L][2][T][C] and CDFs [NC][L][2][C][A_level] (kvc_quantize_levels)
 *   max1         [L][2][T] fp16 bits (device)
 *   chunks_per_unit  1.. , or 0: the larger of about sqrt(2 NC) chunks and enough
 *                chunks for about 2^17 streams (whole-chip encoder launches), at most NC
 *   work         device, 256-byte aligned, work_bytes >= kvc_stream_work_bytes(levels,
 *                n_levels, chunks_per_unit): encoder scratch, one unit's lengths,
 *                offsets and payload, and two staging and two packed halves
 *   host_out     page-locked host memory (hipHostMalloc), host_cap bytes: the
 *                containers of chunks 0, 1, ... back to back (chunk j at the sum of
 *                chunk_bytes[0..j))
 *   chunk_bytes  page-locked host int64 [NC] (written): each container's size
 *   compute_stream, copy_stream  HIP streams (equal priority); the same stream
 *                twice runs every step in order, without overlap
 *   on_chunk     NULL, or called on this thread for each chunk in order once its
 *                container is in host_out: (user, chunk, level, bytes, n_bytes)
 * Returns KVC_ERR_CAPACITY when the containers outgrow host_cap (the chunks
 * copied so far stay valid; no copy passes host_cap), KVC_ERR_HIP on a failed
 * launch or copy.  Device flags as kvc_encode and kvc_serialize_chunk.  The
 * call creates four HIP events for its duration and allocates no memory.
 */
typedef void (*kvc_chunk_fn)(void *user, int64_t chunk, int32_t level, const uint8_t *container,
                             int64_t n_bytes);
int64_t kvc_stream_work_bytes(const kvc_desc *levels, int32_t n_levels, int32_t chunks_per_unit);
int kvc_stream_encode(const kvc_desc *levels, int32_t n_levels, const int32_t *chunk_level,
                      const uint8_t *const *sym, const uint16_t *const *cdf, const uint16_t *max1,
                      int32_t chunks_per_unit, void *work, int64_t work_bytes, uint8_t *host_out,
                      int64_t host_cap, int64_t *chunk_bytes, int32_t *dev_status, void *compute_stream,
                      void *copy_stream, kvc_chunk_fn on_chunk, void *user);

/*
 * Read a container back into the buffers kvc_decode takes.
 *   in           device, 16-byte aligned, in_bytes bytes (read, never past in_bytes)
 *   cdf          [NC][L][2][C][A] uint16 (device, written): the full tables
 *   max1         [L][2][T] (device, written)
 *   stream_len   [n_streams] (device, written)
 *   slab_off     [n_slabs + 1] (device, written): recomputed from the lengths
 * The payload is used in place: kvc_decode(desc, in + kvc_container_payload_offset(desc),
 * in_bytes - that offset, ...).  A header or bins different from the descriptor,
 * or lengths that do not add up to the header's payload size, set
 * KVC_DEV_BAD_CONTAINER.
 */
int kvc_deserialize(const kvc_desc *desc, const uint8_t *in, int64_t in_bytes, uint16_t *cdf,
                    uint16_t *max1, uint16_t *stream_len, uint64_t *slab_off, int32_t *dev_status,
                    void *stream);

/*
 * Token-delta coding with anchors, the step before quantization in the
 * CacheGen write-up ([CG] 1.2 point 1: neighbouring tokens' K/V are close, so
 * differences rather than raw values are coded; [CG] 2.3 step 1 names the
 * anchor-based form).  Anchors are the tokens at chunk-relative positions 0,
 * G, 2G, ... (G = anchor_tokens, 1..65535; every chunk stands alone).
 *   kvc_delta_forward: an anchor row is kept; any other row x becomes
 *     fp16(sat(fp32(x) - fp32(xa_hat))), xa_hat = the codec's reconstruction of its
 *     anchor row (desc's bins: max-abs quantization, then fp16(fp32(q - MAX) /
 *     MAX * max1), as kvc_decode writes it).  The result goes through
 *     kvc_quantize / kvc_encode unchanged.
 *   kvc_delta_inverse: on the tensor kvc_decode wrote (fp16), every
 *     non-anchor row y becomes fp16(sat(fp32(y) + fp32(y_anchor))), in place.
 *   sat() clamps to [-65504, 65504]: a delta between two finite fp16 values can
 *     pass the fp16 range, and is then coded as +-65504 (an error of at most
 *     |delta| - 65504 on that element, counted like any coding error).
 *   kv, delta, y  [L][2][T][C] fp16 (device); kv and delta may be the same
 *                 buffer (else they must not overlap)
 * A row holding Inf or NaN sets KVC_DEV_NONFINITE (kvc_delta_forward); such
 * outputs are unspecified.
 */
int kvc_delta_forward(const kvc_desc *desc, int32_t anchor_tokens, const uint16_t *kv, uint16_t *delta,
                      int32_t *dev_status, void *stream);
int kvc_delta_inverse(const kvc_desc *desc, int32_t anchor_tokens, uint16_t *y, void *stream);

/*
 * The 8-bit comparator: the per-channel INT8 KV quantizer of the page
 * "大模型推理的KV Cache管理：从内存碎片到前缀缓存的优化实战" (KV cache management for LLM
 * inference), section 四, against which the codec's size and error are
 * measured (the CacheGen page's 8-bit baseline, [CG] 1.3).  Per group of
 * `group` contiguous channels of a row (head_dim; it must divide C), in fp32
 * with every operation rounded on its own and round half to even:
 *   scale = (max - min) / 255,  zero_point = clamp(round(-min / scale), 0, 255),
 *   q = clamp(round((x - min) / scale), 0, 255),  y = (q - zero_point) * scale,
 * y written as fp32 (the page's dequantizer returns float32) or rounded to
 * fp16 (out_dtype; where |y| passes 65504 the fp16 value is Inf).
 * A constant group stores q = 0, zero_point = 0 (the printed formula divides 0
 * by 0 there) and decodes to 0.  desc->bins and chunk_tokens are not used
 * (but must be valid).
 *   kv          [L][2][T][C] fp16 (device, read)
 *   q           [L][2][T][C] uint8 (device, written)
 *   scale       [L][2][T][C/group] fp32 (device, written)
 *   zero_point  [L][2][T][C/group] uint8 (device, written)
 *   out         [L][2][T][C] of out_dtype (device, written)
 * Inf or NaN in a group sets KVC_DEV_NONFINITE; that group's outputs are unspecified.
 */
int kvc_int8_quantize(const kvc_desc *desc, int32_t group, const uint16_t *kv, uint8_t *q,
                      float *scale, uint8_t *zero_point, int32_t *dev_status, void *stream);
int kvc_int8_dequantize(const kvc_desc *desc, int32_t group, const uint8_t *q, const float *scale,
                        const uint8_t *zero_point, void *out, int32_t out_dtype, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* KVC_H */
