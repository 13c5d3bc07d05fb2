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

hipError_t launch_cdf(const uint8_t *sym, uint16_t *cdf, const KParams &p, hipStream_t stream);

hipError_t launch_encode(const uint8_t *sym, const uint16_t *cdf, uint8_t *slots,
                         uint64_t *slab_total, uint16_t *stream_len, uint64_t *slab_off,
                         uint8_t *payload, int64_t payload_cap, const KParams &p, int32_t *status,
                         bool vec16, hipStream_t stream);

hipError_t launch_decode(const uint8_t *payload, int64_t payload_bytes, const uint64_t *slab_off,
                         const uint16_t *stream_len, const uint16_t *cdf, const uint16_t *max1,
                         uint8_t *sym_out, void *out, int out_dtype, const KParams &p,
                         int32_t *status, bool vec, hipStream_t stream);

hipError_t launch_dequantize(const uint8_t *sym, const uint16_t *max1, void *out, int out_dtype,
                             const KParams &p, bool vec, hipStream_t stream);

hipError_t launch_zero_u64(uint64_t *dst, hipStream_t stream);
