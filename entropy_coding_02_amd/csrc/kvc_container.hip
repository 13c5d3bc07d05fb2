// kvc_container.hip - the codec's output as one byte buffer, for storage or
// the network (the serializer entry of [CG] 2.1; to_bytes of a KV tensor in
// [CG] 3.2), with each CDF row cut to its own layer's alphabet.
//
// Format, version 1 (little-endian; every section starts at a multiple of 16
// bytes; padding bytes are zero):
//   header   64 bytes: u32 magic 0x3143564B ("KVC1"), u32 version 1, u32 L,
//            u32 C, u64 T, u32 Tc, u32 A, u64 payload_bytes, u64 total_bytes,
//            u32 S (chunks per CDF table), 12 zero bytes
//   bins     u8 [L][2]
//   cdf      per table (group of S chunks, layer, K|V) in that order, per
//            channel: entries 1 .. b-2 of the row as u16 (b = the layer's
//            bins).  Entry 0 is 0 and, since a quantizer with b bins emits
//            symbols up to b-2 only, entry k >= b-1 is k + 65536 - A: both
//            are implied.
//   max1     u16 [L][2][T]
//   lengths  u16 [n_streams]
//   payload  payload_bytes bytes, the section at least 16 bytes long
// The payload section is what kvc_decode reads: whole 16-byte pieces, never
// past the section's end.
#include "kvc_common.h"
#include "kvc_kernels.h"

#include <algorithm>

namespace {

constexpr uint32_t KVC_MAGIC = 0x3143564Bu;

__host__ __device__ inline int64_t r16(int64_t x) { return (x + 15) / 16 * 16; }

// compact CDF entries of the (layer, K|V) pairs before lk, per channel
__device__ inline int64_t lk_prefix(const KParams &p, int lk)
{
    int64_t n = 0;
    for (int i = 0; i < lk; ++i) n += 2 * (int64_t)p.maxq[i];  // bins - 2 = 2 * MAX
    return n;
}

// Header, bins and the padding after them.  One block of 64 threads per
// container; container y of a run (blockIdx.y) takes its offsets off_stride
// further on and is written out_stride bytes further on.
__global__ void k_ser_header(const uint64_t *__restrict__ off0, const uint64_t *__restrict__ off1,
                             uint8_t *__restrict__ out, int64_t out_cap, KParams p,
                             ContainerLayout cl, int32_t *status, int64_t off_stride, int64_t out_stride)
{
    const int64_t y = blockIdx.y;
    if (off0) off0 += y * off_stride;
    off1 += y * off_stride;
    out += y * out_stride;
    const uint64_t pb = *off1 - (off0 ? *off0 : 0u);  // payload bytes
    const int64_t total = container_total(cl, (int64_t)pb);
    const int tid = threadIdx.x;
    if (tid == 0) {
        uint32_t *h = (uint32_t *)out;
        h[0] = KVC_MAGIC;
        h[1] = 1;
        h[2] = (uint32_t)p.L;
        h[3] = (uint32_t)p.C;
        *(uint64_t *)(out + 16) = (uint64_t)p.T;
        h[6] = (uint32_t)p.Tc;
        h[7] = (uint32_t)p.A;
        *(uint64_t *)(out + 32) = pb;
        *(uint64_t *)(out + 40) = (uint64_t)total;
        h[12] = (uint32_t)p.S;
        if (total > out_cap) kvc_flag(status, KVC_DEV_PAYLOAD_OVERFLOW);
    }
    if (tid >= 13 && tid < 16) ((uint32_t *)out)[tid] = 0;
    for (int64_t i = cl.bins + tid; i < cl.cdf; i += blockDim.x) {
        const int64_t lk = i - cl.bins;
        out[i] = lk < 2 * p.L ? (uint8_t)(2 * (p.maxq[lk] + 1)) : 0;
    }
}

// The compact CDF section: one block per table (g, l, kv).  Threads walk the
// table's compact entries (coalesced u16 stores) and check its implied ones.
// Container y of a run (blockIdx.y, chunk j0 + y of a tensor whose table
// groups of S chunks lie table_stride entries apart) is written out_stride
// bytes further on.
__global__ __launch_bounds__(256) void k_ser_cdf(const uint16_t *__restrict__ cdf,
                                                 uint8_t *__restrict__ out, KParams p,
                                                 ContainerLayout cl, int32_t *status, int64_t j0,
                                                 int32_t S, int64_t table_stride, int64_t out_stride)
{
    cdf += (j0 + (int64_t)blockIdx.y) / S * table_stride;
    out += (int64_t)blockIdx.y * out_stride;
    const int64_t slab = blockIdx.x;  // table index g * 2L + lk
    const int64_t twoL = 2 * (int64_t)p.L;
    const int64_t j = slab / twoL;
    const int lk = (int)(slab - j * twoL);
    const int C = p.C, A = p.A, w = 2 * p.maxq[lk];  // w = b - 2 stored entries per row
    const uint32_t K = 65536u - (uint32_t)A;
    const uint16_t *rows = cdf + slab * C * A;
    uint16_t *dst = (uint16_t *)(out + cl.cdf) + j * cl.chunk_entries + (int64_t)C * lk_prefix(p, lk);
    const int64_t n = (int64_t)C * w;
    for (int64_t e = threadIdx.x; e < n; e += blockDim.x) {
        const int64_t c = e / w;
        dst[e] = rows[c * A + 1 + (e - c * w)];
    }
    const int imp = A - w;  // entry 0 and entries w + 1 .. A - 1
    bool bad = false;
    for (int64_t e = threadIdx.x; e < (int64_t)C * imp; e += blockDim.x) {
        const int64_t c = e / imp;
        const int i = (int)(e - c * imp);
        const int k = i == 0 ? 0 : w + i;
        const uint32_t want = k == 0 ? 0u : (uint32_t)k + K;
        bad |= rows[c * A + k] != want;
    }
    if (bad) kvc_flag(status, KVC_DEV_BAD_CDF);
    // zero padding after the last table's rows
    if (slab == (int64_t)p.NG * twoL - 1 && threadIdx.x == 0) {
        const int64_t end = cl.cdf + 2 * (int64_t)p.NG * cl.chunk_entries;
        for (int64_t i = end; i < cl.max1; ++i) out[i] = 0;
    }
}

// Copy n bytes from src to the 4-byte aligned dst, then zero up to
// r16(max(n, min_len)); nothing at or past dst + cap is written.  n is
// n_host, or *n_end - *n_begin when n_end is given (n_begin may be NULL: 0);
// with n_begin the source starts at src + *n_begin.  A 4-byte aligned source
// is copied by dwords, any other byte by byte.  Copy y of a run (blockIdx.y)
// moves src, dst and the offset pointers by y times their strides.
__global__ __launch_bounds__(256) void k_copy_section(const uint8_t *__restrict__ src,
                                                      uint8_t *__restrict__ dst, int64_t n_host,
                                                      const uint64_t *n_begin, const uint64_t *n_end,
                                                      int64_t min_len, int64_t cap, int64_t src_stride,
                                                      int64_t dst_stride, int64_t off_stride)
{
    const int64_t y = blockIdx.y;
    src += y * src_stride;
    dst += y * dst_stride;
    if (n_begin) n_begin += y * off_stride;
    if (n_end) n_end += y * off_stride;
    const int64_t b0 = n_begin ? (int64_t)*n_begin : 0;
    const int64_t n = n_end ? (int64_t)*n_end - b0 : n_host;
    src += b0;
    const bool dw = ((uintptr_t)src & 3) == 0;
    const int64_t end = r16(n > min_len ? n : min_len);
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; 4 * w < end; w += step) {
        const int64_t b = 4 * w;
        uint32_t v;
        if (dw && b + 4 <= n) {
            v = ((const uint32_t *)src)[w];
        } else {
            v = 0;
            for (int i = 0; i < 4; ++i)
                if (b + i < n) v |= (uint32_t)src[b + i] << (8 * i);
        }
        if (b + 4 <= cap) {
            ((uint32_t *)dst)[w] = v;
        } else {
            for (int i = 0; i < 4; ++i)
                if (b + i < cap) dst[b + i] = (uint8_t)(v >> (8 * i));
        }
    }
}

// The max1 rows of chunk j: rows [lk * T + t0, + nj) of every (layer, K|V) lk,
// packed into the section at dst (zero padded to 16 bytes).  Chunk y of a run
// (blockIdx.y) starts t0_stride tokens later and is written dst_stride
// elements further on.
__global__ __launch_bounds__(256) void k_gather_max1(const uint16_t *__restrict__ max1,
                                                     uint16_t *__restrict__ dst, int64_t T,
                                                     int64_t t0, int64_t nj, int64_t n_lk,
                                                     int64_t padded, int64_t t0_stride, int64_t dst_stride)
{
    t0 += (int64_t)blockIdx.y * t0_stride;
    dst += (int64_t)blockIdx.y * dst_stride;
    const int64_t n = n_lk * nj;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < padded / 2; i += step) {
        uint16_t v = 0;
        if (i < n) {
            const int64_t lk = i / nj;
            v = max1[lk * T + t0 + (i - lk * nj)];
        }
        dst[i] = v;
    }
}

// Check the header and bins against the descriptor.  One block of 64 threads.
__global__ void k_deser_check(const uint8_t *__restrict__ in, int64_t in_bytes, KParams p,
                              ContainerLayout cl, int32_t *status)
{
    bool bad = false;
    if (threadIdx.x == 0) {
        const uint32_t *h = (const uint32_t *)in;
        const uint64_t pb = *(const uint64_t *)(in + 32);
        const uint64_t total = *(const uint64_t *)(in + 40);
        bad = h[0] != KVC_MAGIC || h[1] != 1 || h[2] != (uint32_t)p.L || h[3] != (uint32_t)p.C ||
              *(const uint64_t *)(in + 16) != (uint64_t)p.T || h[6] != (uint32_t)p.Tc ||
              h[7] != (uint32_t)p.A || h[12] != (uint32_t)p.S || pb > (uint64_t)in_bytes ||
              total != (uint64_t)container_total(cl, (int64_t)pb) || total > (uint64_t)in_bytes;
    }
    for (int i = threadIdx.x; i < 2 * p.L; i += blockDim.x)
        bad |= in[cl.bins + i] != (uint8_t)(2 * (p.maxq[i] + 1));
    if (bad) kvc_flag(status, KVC_DEV_BAD_CONTAINER);
}

// The full [NG][L][2][C][A] tables from the compact rows: one block per
// table, a thread per table entry (coalesced u16 stores).
__global__ __launch_bounds__(256) void k_deser_cdf(const uint8_t *__restrict__ in,
                                                   uint16_t *__restrict__ cdf, KParams p,
                                                   ContainerLayout cl)
{
    const int64_t slab = blockIdx.x;
    const int64_t twoL = 2 * (int64_t)p.L;
    const int64_t j = slab / twoL;
    const int lk = (int)(slab - j * twoL);
    const int C = p.C, A = p.A, w = 2 * p.maxq[lk];
    const uint32_t K = 65536u - (uint32_t)A;
    const uint16_t *src = (const uint16_t *)(in + cl.cdf) + j * cl.chunk_entries +
                          (int64_t)C * lk_prefix(p, lk);
    uint16_t *rows = cdf + slab * C * A;
    for (int64_t e = threadIdx.x; e < (int64_t)C * A; e += blockDim.x) {
        const int64_t c = e / A;
        const int k = (int)(e - c * A);
        const uint32_t v = k == 0 ? 0u : (k <= w ? (uint32_t)src[c * w + (k - 1)] : (uint32_t)k + K);
        rows[e] = (uint16_t)v;
    }
}

unsigned grid_for(int64_t items, int64_t per_block)
{
    int64_t g = (items + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > 65536) g = 65536;
    return (unsigned)g;
}

// The total_bytes field of n containers laid stride bytes apart, into dst[n].
__global__ void k_container_totals(const uint8_t *__restrict__ base, int64_t stride, int n,
                                   uint64_t *__restrict__ dst)
{
    const int k = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (k < n) dst[k] = *(const uint64_t *)(base + (int64_t)k * stride + 40);
}

// The n containers of a unit, container k at src + k * stride (stride a
// multiple of 16) with its total in sizes[k], moved back to back into dst
// (container k at the sum of the totals before it), so that one copy takes the
// whole unit off the device.  A total is taken rounded up to 16 and at most
// stride, so nothing is read or written past the slots whatever sizes holds
// (the host checks the totals before it copies).  Block (x, k) moves 16-byte
// pieces x, x + gridDim.x, ... of container k.
__global__ void k_pack_containers(const uint8_t *__restrict__ src, int64_t stride,
                                  const uint64_t *__restrict__ sizes, int n, uint8_t *__restrict__ dst)
{
    const int k = (int)blockIdx.y;
    if (k >= n) return;
    auto len_of = [&](int i) -> int64_t {
        const uint64_t v = sizes[i];
        const uint64_t r = v > (uint64_t)stride ? (uint64_t)stride : (v + 15u) & ~(uint64_t)15u;
        return (int64_t)r;
    };
    int64_t off = 0;
    for (int i = 0; i < k; ++i) off += len_of(i);
    const int64_t n16 = len_of(k) / 16;
    const u32x4 *s4 = (const u32x4 *)(src + (int64_t)k * stride);
    u32x4 *d4 = (u32x4 *)(dst + off);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
        d4[i] = s4[i];
}

}  // namespace

ContainerLayout container_layout(const KParams &p)
{
    ContainerLayout cl;
    cl.chunk_entries = 0;
    for (int i = 0; i < 2 * p.L; ++i) cl.chunk_entries += (int64_t)p.C * 2 * p.maxq[i];
    cl.bins = 64;
    cl.cdf = r16(cl.bins + 2 * (int64_t)p.L);
    cl.max1 = r16(cl.cdf + 2 * (int64_t)p.NG * cl.chunk_entries);
    cl.len = r16(cl.max1 + 2 * p.n_rows);
    cl.pay = r16(cl.len + 2 * p.n_streams);
    return cl;
}

hipError_t launch_serialize(const uint16_t *cdf, const uint16_t *max1, const uint16_t *stream_len,
                            const uint64_t *slab_off, const uint8_t *payload, uint8_t *out,
                            int64_t out_cap, const KParams &p, int32_t *status, hipStream_t stream)
{
    const ContainerLayout cl = container_layout(p);
    const int64_t z = 0;
    hipLaunchKernelGGL(k_ser_header, dim3(1), dim3(64), 0, stream, (const uint64_t *)nullptr,
                       slab_off + p.n_slabs, out, out_cap, p, cl, status, z, z);
    const int64_t n_tables = (int64_t)p.NG * 2 * p.L;
    if (n_tables > 0)
        hipLaunchKernelGGL(k_ser_cdf, dim3((unsigned)n_tables), dim3(256), 0, stream, cdf, out, p, cl,
                           status, z, 1, z, z);
    const int64_t rows_b = 2 * p.n_rows, lens_b = 2 * p.n_streams;
    const uint64_t *none = nullptr;
    hipLaunchKernelGGL(k_copy_section, dim3(grid_for(rows_b, 1024)), dim3(256), 0, stream,
                       (const uint8_t *)max1, out + cl.max1, rows_b, none, none, z, cl.len - cl.max1, z, z, z);
    hipLaunchKernelGGL(k_copy_section, dim3(grid_for(lens_b, 1024)), dim3(256), 0, stream,
                       (const uint8_t *)stream_len, out + cl.len, lens_b, none, none, z, cl.pay - cl.len, z, z,
                       z);
    // the payload size is known on the device only: size the grid for the capacity
    hipLaunchKernelGGL(k_copy_section, dim3(grid_for(out_cap - cl.pay, 4096)), dim3(256), 0, stream,
                       payload, out + cl.pay, z, none, slab_off + p.n_slabs, (int64_t)16, out_cap - cl.pay,
                       z, z, z);
    return hipGetLastError();
}

hipError_t launch_serialize_chunks(const ChunkRun &run, uint8_t *out, int64_t out_stride, const KParams &p,
                                   int32_t *status, hipStream_t stream)
{
    // p describes one chunk of the run as a tensor of its own: T = N_j, one
    // chunk, 2L slabs, one table per slab (S = 1)
    if (run.n <= 0) return hipSuccess;
    const ContainerLayout cl = container_layout(p);
    const int64_t twoL = 2 * (int64_t)p.L, out_cap = out_stride;
    const unsigned n = (unsigned)run.n;
    const uint64_t *off0 = run.off, *off1 = run.off + twoL;
    hipLaunchKernelGGL(k_ser_header, dim3(1, n), dim3(64), 0, stream, off0, off1, out, out_cap, p, cl, status,
                       twoL, out_stride);
    if (p.n_slabs > 0)
        hipLaunchKernelGGL(k_ser_cdf, dim3((unsigned)p.n_slabs, n), dim3(256), 0, stream, run.cdf, out, p, cl,
                           status, run.j0, run.S, run.table_stride, out_stride);
    const int64_t nj = p.T, rows_padded = cl.len - cl.max1;
    hipLaunchKernelGGL(k_gather_max1, dim3(grid_for(rows_padded / 2, 1024), n), dim3(256), 0, stream,
                       run.max1, (uint16_t *)(out + cl.max1), run.max1_T, run.j0 * run.Tc, nj, twoL, rows_padded,
                       run.Tc, out_stride / 2);
    const uint64_t *none = nullptr;
    const int64_t lens_b = 2 * p.n_streams, z = 0;
    hipLaunchKernelGGL(k_copy_section, dim3(grid_for(lens_b, 1024), n), dim3(256), 0, stream,
                       (const uint8_t *)run.stream_len, out + cl.len, lens_b, none, none, z, cl.pay - cl.len,
                       lens_b, out_stride, z);
    // a grid-stride copy: enough blocks per chunk to keep the copies wide,
    // not one per 4 KB of the capacity
    const unsigned gp = std::min<unsigned>(grid_for(out_cap - cl.pay, 4096), 256u);
    hipLaunchKernelGGL(k_copy_section, dim3(gp, n), dim3(256), 0, stream, run.payload, out + cl.pay, z, off0,
                       off1, (int64_t)16, out_cap - cl.pay, z, out_stride, twoL);
    return hipGetLastError();
}

hipError_t launch_deserialize(const uint8_t *in, int64_t in_bytes, uint16_t *cdf, uint16_t *max1,
                              uint16_t *stream_len, uint64_t *slab_off, const KParams &p,
                              int32_t *status, hipStream_t stream)
{
    const ContainerLayout cl = container_layout(p);
    hipLaunchKernelGGL(k_deser_check, dim3(1), dim3(64), 0, stream, in, in_bytes, p, cl, status);
    const int64_t n_tables = (int64_t)p.NG * 2 * p.L;
    if (n_tables > 0)
        hipLaunchKernelGGL(k_deser_cdf, dim3((unsigned)n_tables), dim3(256), 0, stream, in, cdf, p, cl);
    const int64_t rows_b = 2 * p.n_rows, lens_b = 2 * p.n_streams;
    if (rows_b > 0) {
        const uint64_t *none = nullptr;
        const int64_t z = 0;
        hipLaunchKernelGGL(k_copy_section, dim3(grid_for(rows_b, 1024)), dim3(256), 0, stream,
                           in + cl.max1, (uint8_t *)max1, rows_b, none, none, z, rows_b, z, z, z);
        hipLaunchKernelGGL(k_copy_section, dim3(grid_for(lens_b, 1024)), dim3(256), 0, stream,
                           in + cl.len, (uint8_t *)stream_len, lens_b, none, none, z, lens_b, z, z, z);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_slab_offsets(stream_len, slab_off, p, (const uint64_t *)(in + 32), status, stream);
}

hipError_t launch_pack_containers(const uint8_t *src, int64_t stride, const uint64_t *sizes, int n,
                                  uint8_t *dst, hipStream_t stream)
{
    if (n > 0)
        hipLaunchKernelGGL(k_pack_containers, dim3(64, (unsigned)n), dim3(256), 0, stream, src, stride, sizes, n,
                           dst);
    return hipGetLastError();
}

hipError_t launch_container_totals(const uint8_t *base, int64_t stride, int n, uint64_t *dst,
                                   hipStream_t stream)
{
    if (n > 0)
        hipLaunchKernelGGL(k_container_totals, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, base,
                           stride, n, dst);
    return hipGetLastError();
}
