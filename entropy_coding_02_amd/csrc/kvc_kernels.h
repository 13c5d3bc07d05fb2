// kvc_kernels.h - host-side launchers of the HIP kernels (internal).
#pragma once

#include <hip/hip_runtime.h>

#include "kvc_common.h"

hipError_t launch_quantize_rows(const uint16_t *kv, uint8_t *sym, uint16_t *max1, const KParams &p,
                                int32_t *status, bool vec8, hipStream_t stream);

// Fused quantize + histogram + CDF (one kernel), where the shape allows it.
bool quant_cdf_fused_ok(const KParams &p);
hipError_t launch_quant_cdf(const uint16_t *kv, uint8_t *sym, uint16_t *max1, uint16_t *cdf,
                            const KParams &p, int32_t *status, hipStream_t stream);

// Quality levels (bins tables) of one tensor for the multi-level pass.
#define KVC_MAX_LEVELS 4
struct LevelParams {
    int32_t n;                                       // levels
    int32_t words;                                   // LDS words of all histograms
    int32_t A[KVC_MAX_LEVELS];                       // alphabet of each level
    int32_t hist[KVC_MAX_LEVELS];                    // LDS word offset of each level's histogram
    uint8_t *sym[KVC_MAX_LEVELS];
    uint16_t *cdf[KVC_MAX_LEVELS];
    uint8_t maxq[KVC_MAX_LEVELS][2 * KVC_MAX_LAYERS];  // MAX per (layer, K|V) of each level
};
// The shape qualifies: C % 8 == 0, C <= 1024, every A % 8 == 0 and all
// histograms fit the device's LDS per block.
bool quant_cdf_levels_ok(const KParams &p, const LevelParams &lv);
hipError_t launch_quant_cdf_levels(const uint16_t *kv, uint16_t *max1, const KParams &p,
                                   LevelParams lv, int32_t *status, hipStream_t stream);

hipError_t launch_cdf(const uint8_t *sym, uint16_t *cdf, const KParams &p, int32_t *status,
                      hipStream_t stream);

hipError_t launch_encode(const uint8_t *sym, const uint16_t *cdf, uint8_t *slots,
                         uint64_t *slab_total, uint16_t *stream_len, uint64_t *slab_off,
                         uint8_t *payload, int64_t payload_cap, const KParams &p, int32_t *status,
                         bool vec16, hipStream_t stream);

// Lanes per stream launch_decode uses for this shape (1, 4 or 8).
int decode_lanes_per_stream(const KParams &p);

hipError_t launch_decode(const uint8_t *payload, int64_t payload_bytes, const uint64_t *slab_off,
                         const uint16_t *stream_len, const uint16_t *cdf, const uint16_t *max1,
                         uint8_t *sym_out, void *out, int out_dtype, const KParams &p,
                         int32_t *status, bool vec, hipStream_t stream);

hipError_t launch_dequantize(const uint8_t *sym, const uint16_t *max1, void *out, int out_dtype,
                             const KParams &p, bool vec, hipStream_t stream);

hipError_t launch_zero_u64(uint64_t *dst, hipStream_t stream);

// slab_off [n_slabs + 1] from the stream lengths (exclusive scan of the slab
// sums); with `expect`, a total different from *expect sets KVC_DEV_BAD_CONTAINER.
hipError_t launch_slab_offsets(const uint16_t *stream_len, uint64_t *slab_off, const KParams &p,
                               const uint64_t *expect, int32_t *status, hipStream_t stream);

// Byte container (kvc_container.hip): section offsets, from the descriptor alone.
struct ContainerLayout {
    int64_t bins, cdf, max1, len, pay;  // section offsets
    int64_t chunk_entries;              // compact CDF entries of one chunk
};
ContainerLayout container_layout(const KParams &p);
// total container bytes: the payload section is padded to at least 16 bytes
__host__ __device__ inline int64_t container_total(const ContainerLayout &cl, int64_t payload_bytes)
{
    const int64_t n = payload_bytes < 16 ? 16 : payload_bytes;
    return cl.pay + (n + 15) / 16 * 16;
}
hipError_t launch_serialize(const uint16_t *cdf, const uint16_t *max1, const uint16_t *stream_len,
                            const uint64_t *slab_off, const uint8_t *payload, uint8_t *out,
                            int64_t out_cap, const KParams &p, int32_t *status, hipStream_t stream);
// The total_bytes header field of n containers laid stride bytes apart from
// base (16-byte aligned), into dst[n] (device).
hipError_t launch_container_totals(const uint8_t *base, int64_t stride, int n, uint64_t *dst,
                                   hipStream_t stream);
// n containers stride bytes apart from src (stride a multiple of 16), totals
// in sizes (device), moved back to back into dst (16-byte aligned, at least
// n * stride bytes): container k at the sum of the totals before it.
hipError_t launch_pack_containers(const uint8_t *src, int64_t stride, const uint64_t *sizes, int n,
                                  uint8_t *dst, hipStream_t stream);
// n consecutive chunks j0 .. j0 + n - 1 of one shape (each with p.T tokens):
// the whole tensor's tables (groups of S chunks, table_stride entries apart),
// its max1 rows (max1_T tokens each, chunk j starting at token j * Tc), and
// chunk j0's stream lengths and 2L + 1 slab offsets, chunk j0 + k's following
// k * 2L * p.T lengths and k * 2L offsets further on, all indexing payload.
struct ChunkRun {
    const uint16_t *cdf;
    int32_t S;
    int64_t table_stride;
    const uint16_t *max1;
    int64_t max1_T, Tc, j0;
    const uint16_t *stream_len;
    const uint64_t *off;
    const uint8_t *payload;
    int64_t n;
};
// The containers of a run, container k at out + k * out_stride (each at most
// out_stride bytes); `chunk` describes one chunk as a tensor of its own.
hipError_t launch_serialize_chunks(const ChunkRun &run, uint8_t *out, int64_t out_stride,
                                   const KParams &chunk, int32_t *status, hipStream_t stream);
hipError_t launch_deserialize(const uint8_t *in, int64_t in_bytes, uint16_t *cdf, uint16_t *max1,
                              uint16_t *stream_len, uint64_t *slab_off, const KParams &p,
                              int32_t *status, hipStream_t stream);

// 8-bit comparator quantizer (kvc_int8.hip).
// Token-delta coding (kvc_delta.hip), anchors every G chunk-relative tokens.
hipError_t launch_delta_forward(const uint16_t *kv, uint16_t *out, const KParams &p, int G, bool vec,
                                int32_t *status, hipStream_t stream);
hipError_t launch_delta_inverse(uint16_t *y, const KParams &p, int G, bool vec, hipStream_t stream);

hipError_t launch_int8_quantize(const uint16_t *kv, uint8_t *q, float *scale, uint8_t *zp,
                                int64_t n_rows, int C, int g, bool vec, int32_t *status,
                                hipStream_t stream);
hipError_t launch_int8_dequantize(const uint8_t *q, const float *scale, const uint8_t *zp, void *out,
                                  bool f32, int64_t n_el, int g, hipStream_t stream);
