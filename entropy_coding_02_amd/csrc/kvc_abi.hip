// kvc_abi.hip - the extern "C" entry points of libkvc.so: argument checks on
// the host, then asynchronous launches on the caller's stream.
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "kvc_common.h"
#include "kvc_kernels.h"

// Encoder workspace of kvc_encode_noalloc: one array per GPU the library runs
// on, held until the process ends, shared by every call on that GPU.  In host
// code its name is only a stand-in; its device address comes from
// hipGetSymbolAddress (per device, kept in noalloc_base below).
static __device__ __align__(256) uint8_t scratch[KVC_NOALLOC_SCRATCH_BYTES];

namespace {

struct Geometry {
    KParams p;
    int64_t slot_area;   // bytes of encoder stream slots
    int64_t scratch;     // total encoder scratch bytes
};

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Validate the descriptor and derive every size; KVC_OK or KVC_ERR_ARG.
int make_geometry(const kvc_desc *d, Geometry &g)
{
    if (!d || !d->bins) return KVC_ERR_ARG;
    if (d->n_layers < 1 || d->n_layers > KVC_MAX_LAYERS) return KVC_ERR_ARG;
    if (d->n_channels < 1 || d->n_channels > 16384) return KVC_ERR_ARG;
    if (d->n_tokens < 0 || d->n_tokens > ((int64_t)1 << 40)) return KVC_ERR_ARG;
    if (d->chunk_tokens < 1 || d->chunk_tokens > 65535 || d->cdf_chunks < 0) return KVC_ERR_ARG;
    memset(&g, 0, sizeof(g));
    KParams &p = g.p;
    int A = 0;
    for (int i = 0; i < 2 * d->n_layers; ++i) {
        int b = d->bins[i];
        if (b < 4 || b > 256 || (b & 1)) return KVC_ERR_ARG;
        p.maxq[i] = (uint8_t)(b / 2 - 1);
        A = b > A ? b : A;
    }
    p.L = d->n_layers;
    p.C = d->n_channels;
    p.A = A;
    p.Tc = d->chunk_tokens;
    p.T = d->n_tokens;
    p.Ts = p.T;
    int64_t NC = (p.T + p.Tc - 1) / p.Tc;
    if (NC > INT32_MAX) return KVC_ERR_ARG;
    p.NC = (int32_t)NC;
    p.S = (int32_t)(d->cdf_chunks <= 1 ? 1 : std::min<int64_t>(d->cdf_chunks, std::max<int64_t>(NC, 1)));
    p.NG = (int32_t)((NC + p.S - 1) / p.S);
    p.j0 = 0;
    if (std::min<int64_t>((int64_t)p.S * p.Tc, p.T) > KVC_MAX_TABLE_TOKENS) return KVC_ERR_ARG;
    p.last_nj = NC ? (int32_t)(p.T - (NC - 1) * p.Tc) : 0;
    p.rn_full = 1.0 / (double)p.Tc;
    p.rn_last = p.last_nj ? 1.0 / (double)p.last_nj : 0.0;
    p.n_rows = 2 * (int64_t)p.L * p.T;
    p.n_streams = p.n_rows;
    p.n_slabs = NC * 2 * p.L;
    p.slot_bytes = round_up(2 * (int64_t)p.C + 16, 16);
    // encoder slots: one per lane of every 256-lane block (slab x ceil(Tc/256))
    g.slot_area = p.n_slabs * ((p.Tc + 255) / 256) * 256 * p.slot_bytes;
    g.scratch = g.slot_area + 8 * p.n_slabs;
    // launch-size limits (1-D grids of 32-bit block counts)
    if (p.n_slabs * ((p.Tc + 255) / 256) >= ((int64_t)1 << 29)) return KVC_ERR_ARG;  // x4 for k_pack
    if (p.n_slabs * ((p.C + 63) / 64) >= ((int64_t)1 << 31)) return KVC_ERR_ARG;
    return KVC_OK;
}

bool aligned(const void *ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

// The tensor as the CDF producers see it: its tables as chunks of S * Tc
// tokens, one table each (the tables are the per-chunk CDFs of that coarser
// chunking; quantization is per row and does not see chunks).
KParams table_params(const KParams &p)
{
    KParams t = p;
    t.Tc = p.S * p.Tc;  // <= KVC_MAX_TABLE_TOKENS when S > 1 (make_geometry)
    if (p.S > 1 && t.Tc > p.T) t.Tc = (int32_t)std::max<int64_t>(p.T, 1);
    t.NC = p.NG;
    t.S = 1;
    t.NG = p.NG;
    t.last_nj = p.NG ? (int32_t)(p.T - (int64_t)(p.NG - 1) * t.Tc) : 0;
    t.rn_full = 1.0 / (double)t.Tc;
    t.rn_last = t.last_nj ? 1.0 / (double)t.last_nj : 0.0;
    t.n_slabs = (int64_t)p.NG * 2 * p.L;
    return t;
}

// Whether the CDF kernels with 16-bit counters (the fused quantize + CDF pass,
// k_cdf_wide) can count a table of these params.
bool short_tables(const KParams &t) { return t.Tc <= 65535; }

// Device address of `scratch` on the current device: looked up with
// hipGetSymbolAddress on the first call on each device (with that device
// current) and kept; NULL if the lookup fails.
constexpr int kMaxDevices = 64;
void *noalloc_base()
{
    static std::mutex mu;
    static void *base[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!base[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        base[dev] = ptr;
    }
    return base[dev];
}

// Device workspace of the streaming encoder for units of up to U chunks
// (sizes are the largest over the levels); every section 256-byte aligned.
struct StreamLayout {
    int32_t U;                                   // chunks per unit
    int64_t len, off, pay, sizes, staging, packed, total;  // section offsets; scratch at 0
    int64_t pay_cap, chunk_cap;                  // unit payload, staging bytes per chunk
};

// Check the level descriptors (as kvc_quantize_levels) and lay out the workspace.
int stream_layout(const kvc_desc *levels, int32_t n_levels, int32_t chunks_per_unit, Geometry *g,
                  StreamLayout &sl)
{
    if (!levels || n_levels < 1 || n_levels > KVC_MAX_LEVELS || chunks_per_unit < 0) return KVC_ERR_ARG;
    for (int l = 0; l < n_levels; ++l) {
        int rc = make_geometry(&levels[l], g[l]);
        if (rc != KVC_OK) return rc;
        if (levels[l].n_layers != levels[0].n_layers || levels[l].n_channels != levels[0].n_channels ||
            levels[l].n_tokens != levels[0].n_tokens || levels[l].chunk_tokens != levels[0].chunk_tokens)
            return KVC_ERR_ARG;
    }
    const KParams &P = g[0].p;
    const int64_t per_chunk = 2 * (int64_t)P.L * P.Tc;  // streams of a full chunk
    // automatic unit: enough chunks for about 2^17 streams (an encoder launch
    // that fills the chip), and about sqrt(2 NC) of them: each unit costs some
    // tens of microseconds of host waiting and idle gaps, while the first
    // unit's encode and the last one's copy are not overlapped
    int64_t U = chunks_per_unit;
    if (!U) {
        const int64_t by_streams = (((int64_t)1 << 17) + per_chunk - 1) / per_chunk;
        int64_t by_count = 1;
        while ((by_count + 1) * (by_count + 1) <= 2 * (int64_t)P.NC) ++by_count;
        U = std::max(by_streams, by_count);
    }
    U = std::max<int64_t>(1, std::min<int64_t>(U, P.NC));
    sl.U = (int32_t)U;
    int64_t scratch = 0, n_streams = 0, n_slabs = 0, chunk_cap = 0;
    for (int l = 0; l < n_levels; ++l) {
        kvc_desc du = levels[l], dc = levels[l];
        du.n_tokens = std::min<int64_t>(U * P.Tc, P.T);
        dc.n_tokens = std::min<int64_t>(P.Tc, P.T);
        Geometry gu, gc;
        int rc = make_geometry(&du, gu);
        if (rc == KVC_OK) rc = make_geometry(&dc, gc);
        if (rc != KVC_OK) return rc;
        scratch = std::max(scratch, gu.scratch);
        n_streams = gu.p.n_streams;
        n_slabs = gu.p.n_slabs;
        const int64_t chunk_pay = gc.p.n_streams * (2 * (int64_t)P.C + 1);
        chunk_cap = std::max(chunk_cap, round_up(container_total(container_layout(gc.p), chunk_pay), 256));
    }
    sl.pay_cap = n_streams * (2 * (int64_t)P.C + 1);
    sl.chunk_cap = chunk_cap;
    sl.len = round_up(scratch, 256);
    sl.off = sl.len + round_up(2 * n_streams, 256);
    sl.pay = sl.off + round_up(8 * (n_slabs + 1), 256);
    sl.sizes = sl.pay + round_up(sl.pay_cap, 256);
    sl.staging = sl.sizes + round_up(8 * U, 256);
    sl.packed = sl.staging + 2 * U * chunk_cap;
    sl.total = sl.packed + 2 * U * chunk_cap;
    return KVC_OK;
}

// Page-locked host memory (a hipHostMalloc allocation).
bool host_pinned(const void *ptr)
{
    hipPointerAttribute_t a;
    const hipError_t e = hipPointerGetAttributes(&a, ptr);
    if (e != hipSuccess) {
        (void)hipGetLastError();  // a pageable pointer is not an error of the caller's streams
        return false;
    }
    return a.type == hipMemoryTypeHost;
}

int launch_status(hipError_t e) { return e == hipSuccess ? KVC_OK : KVC_ERR_HIP; }

}  // namespace

extern "C" {

int kvc_version(void) { return KVC_VERSION; }

const char *kvc_status_string(int status)
{
    switch (status) {
    case KVC_OK: return "ok";
    case KVC_ERR_ARG: return "invalid argument";
    case KVC_ERR_CAPACITY: return "buffer too small";
    case KVC_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
    }
}

int32_t kvc_alphabet(const kvc_desc *desc)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    return rc == KVC_OK ? g.p.A : rc;
}

int64_t kvc_n_chunks(const kvc_desc *desc)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    return rc == KVC_OK ? (int64_t)g.p.NC : rc;
}

int64_t kvc_n_slabs(const kvc_desc *desc)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    return rc == KVC_OK ? g.p.n_slabs : rc;
}

int64_t kvc_n_streams(const kvc_desc *desc)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    return rc == KVC_OK ? g.p.n_streams : rc;
}

int32_t kvc_decode_lanes(const kvc_desc *desc)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    return rc == KVC_OK ? decode_lanes_per_stream(g.p) : rc;
}

int64_t kvc_cdf_bytes(const kvc_desc *desc)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    return rc == KVC_OK ? (int64_t)g.p.NG * 2 * g.p.L * g.p.C * g.p.A * 2 : rc;
}

int64_t kvc_scratch_bytes(const kvc_desc *desc)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    return rc == KVC_OK ? g.scratch : rc;
}

int64_t kvc_max_payload_bytes(const kvc_desc *desc)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    return rc == KVC_OK ? g.p.n_streams * (2 * (int64_t)g.p.C + 1) : rc;
}

int kvc_quantize(const kvc_desc *desc, const uint16_t *kv, uint8_t *sym, uint16_t *max1,
                 uint16_t *cdf, int32_t *dev_status, void *stream)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    if (rc != KVC_OK) return rc;
    if (g.p.n_rows == 0) return KVC_OK;
    if (!kv || !sym || !max1 || !aligned(kv, 4) || !aligned(sym, 4) || !aligned(max1, 2) ||
        (cdf && !aligned(cdf, 4)) || (dev_status && !aligned(dev_status, 4)))
        return KVC_ERR_ARG;
    hipStream_t s = (hipStream_t)stream;
    const bool vec8 = (g.p.C % 8 == 0) && aligned(kv, 16) && aligned(sym, 8);
    const KParams t = table_params(g.p);
    // The fused pass runs one block per table: with fewer tables than the chip
    // has compute units, two passes spread over more blocks finish sooner.
    if (cdf && vec8 && aligned(cdf, 16) && t.n_slabs >= 256 && short_tables(t) && quant_cdf_fused_ok(t))
        return launch_status(launch_quant_cdf(kv, sym, max1, cdf, t, dev_status, s));
    hipError_t e = launch_quantize_rows(kv, sym, max1, g.p, dev_status, vec8, s);
    if (e == hipSuccess && cdf) e = launch_cdf(sym, cdf, t, dev_status, s);
    return launch_status(e);
}

int kvc_quantize_levels(const kvc_desc *levels, int32_t n_levels, const uint16_t *kv,
                        uint8_t *const *sym, uint16_t *max1, uint16_t *const *cdf,
                        int32_t *dev_status, void *stream)
{
    if (!levels || n_levels < 1 || n_levels > KVC_MAX_LEVELS || !sym || !cdf) return KVC_ERR_ARG;
    Geometry g[KVC_MAX_LEVELS];
    for (int l = 0; l < n_levels; ++l) {
        int rc = make_geometry(&levels[l], g[l]);
        if (rc != KVC_OK) return rc;
        if (levels[l].n_layers != levels[0].n_layers || levels[l].n_channels != levels[0].n_channels ||
            levels[l].n_tokens != levels[0].n_tokens ||
            levels[l].chunk_tokens != levels[0].chunk_tokens)
            return KVC_ERR_ARG;
        if (!sym[l] || !cdf[l] || !aligned(sym[l], 4) || !aligned(cdf[l], 4)) return KVC_ERR_ARG;
    }
    const KParams p = table_params(g[0].p);
    if (p.n_rows == 0) return KVC_OK;
    if (!kv || !max1 || !aligned(kv, 4) || !aligned(max1, 2) || (dev_status && !aligned(dev_status, 4)))
        return KVC_ERR_ARG;
    LevelParams lv;
    memset(&lv, 0, sizeof(lv));
    lv.n = n_levels;
    bool fused = p.n_slabs >= 256 && short_tables(p) && aligned(kv, 16);
    for (int l = 0; l < n_levels; ++l) {
        fused = fused && g[l].p.S == g[0].p.S;  // one table geometry for every level
        lv.A[l] = g[l].p.A;
        lv.sym[l] = sym[l];
        lv.cdf[l] = cdf[l];
        memcpy(lv.maxq[l], g[l].p.maxq, sizeof(lv.maxq[l]));
        fused = fused && aligned(sym[l], 8) && aligned(cdf[l], 16);
    }
    if (fused && quant_cdf_levels_ok(p, lv))
        return launch_status(launch_quant_cdf_levels(kv, max1, p, lv, dev_status, (hipStream_t)stream));
    for (int l = 0; l < n_levels; ++l) {  // level by level (max1 written each time, identically)
        int rc = kvc_quantize(&levels[l], kv, sym[l], max1, cdf[l], dev_status, stream);
        if (rc != KVC_OK) return rc;
    }
    return KVC_OK;
}

int kvc_cdf(const kvc_desc *desc, const uint8_t *sym, uint16_t *cdf, int32_t *dev_status,
            void *stream)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    if (rc != KVC_OK) return rc;
    if (g.p.n_rows == 0) return KVC_OK;
    if (!sym || !cdf || !aligned(sym, 4) || !aligned(cdf, 4) || (dev_status && !aligned(dev_status, 4)))
        return KVC_ERR_ARG;
    return launch_status(launch_cdf(sym, cdf, table_params(g.p), dev_status, (hipStream_t)stream));
}

int kvc_encode(const kvc_desc *desc, const uint8_t *sym, const uint16_t *cdf, void *scratch,
               int64_t scratch_bytes, uint16_t *stream_len, uint64_t *slab_off, uint8_t *payload,
               int64_t payload_cap, int32_t *dev_status, void *stream)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    if (rc != KVC_OK) return rc;
    if (!slab_off || !aligned(slab_off, 8) || payload_cap < 0) return KVC_ERR_ARG;
    hipStream_t s = (hipStream_t)stream;
    if (g.p.n_rows == 0) return launch_status(launch_zero_u64(slab_off, s));
    if (!sym || !cdf || !scratch || !stream_len || (!payload && payload_cap > 0) ||
        !aligned(sym, 4) || !aligned(cdf, 4) || !aligned(scratch, 16) || !aligned(stream_len, 2) ||
        !aligned(payload, 4) ||
        (dev_status && !aligned(dev_status, 4)))
        return KVC_ERR_ARG;
    if (scratch_bytes < g.scratch) return KVC_ERR_CAPACITY;
    uint8_t *slots = (uint8_t *)scratch;
    uint64_t *slab_total = (uint64_t *)(slots + g.slot_area);
    const bool vec16 = (g.p.C % 16 == 0) && aligned(sym, 16);
    return launch_status(launch_encode(sym, cdf, slots, slab_total, stream_len, slab_off, payload,
                                       payload_cap, g.p, dev_status, vec16, s));
}

int kvc_encode_noalloc(const kvc_desc *desc, const uint8_t *sym, const uint16_t *cdf,
                       uint16_t *stream_len, uint64_t *slab_off, uint8_t *payload, int64_t payload_cap,
                       int32_t *dev_status, void *stream)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    if (rc != KVC_OK) return rc;
    if (g.scratch > (int64_t)KVC_NOALLOC_SCRATCH_BYTES) return KVC_ERR_CAPACITY;
    void *const base = noalloc_base();
    if (!base) return KVC_ERR_HIP;
    return kvc_encode(desc, sym, cdf, base, (int64_t)KVC_NOALLOC_SCRATCH_BYTES, stream_len, slab_off,
                      payload, payload_cap, dev_status, stream);
}

int kvc_decode(const kvc_desc *desc, const uint8_t *payload, int64_t payload_bytes,
               const uint64_t *slab_off, const uint16_t *stream_len, const uint16_t *cdf,
               const uint16_t *max1, uint8_t *sym_out, void *out, int32_t out_dtype,
               int32_t *dev_status, void *stream)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    if (rc != KVC_OK) return rc;
    if (out && out_dtype != KVC_F16 && out_dtype != KVC_F32) return KVC_ERR_ARG;
    if (g.p.n_rows == 0) return KVC_OK;
    if (!slab_off || !stream_len || !cdf || !payload || payload_bytes < 16 || payload_bytes % 4 != 0 ||
        (!out && !sym_out) || (out && !max1) || !aligned(payload, 4) || !aligned(slab_off, 8) ||
        !aligned(stream_len, 2) || !aligned(cdf, 4) || (dev_status && !aligned(dev_status, 4)))
        return KVC_ERR_ARG;
    const bool vec = (g.p.C % 16 == 0) && (!sym_out || aligned(sym_out, 16)) &&
                     (!out || aligned(out, 16));
    return launch_status(launch_decode(payload, payload_bytes, slab_off, stream_len, cdf, max1,
                                       sym_out, out, out_dtype, g.p, dev_status, vec,
                                       (hipStream_t)stream));
}

int kvc_dequantize(const kvc_desc *desc, const uint8_t *sym, const uint16_t *max1, void *out,
                   int32_t out_dtype, void *stream)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    if (rc != KVC_OK) return rc;
    if (out_dtype != KVC_F16 && out_dtype != KVC_F32) return KVC_ERR_ARG;
    if (g.p.n_rows == 0) return KVC_OK;
    if (!sym || !max1 || !out || !aligned(out, 4)) return KVC_ERR_ARG;
    return launch_status(
        launch_dequantize(sym, max1, out, out_dtype, g.p, false, (hipStream_t)stream));
}

int64_t kvc_container_bytes(const kvc_desc *desc, int64_t payload_bytes)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    if (rc != KVC_OK) return rc;
    if (payload_bytes < 0) return KVC_ERR_ARG;
    return container_total(container_layout(g.p), payload_bytes);
}

int64_t kvc_container_payload_offset(const kvc_desc *desc)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    return rc == KVC_OK ? container_layout(g.p).pay : rc;
}

int kvc_serialize(const kvc_desc *desc, const uint16_t *cdf, const uint16_t *max1,
                  const uint16_t *stream_len, const uint64_t *slab_off, const uint8_t *payload,
                  uint8_t *out, int64_t out_cap, int32_t *dev_status, void *stream)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    if (rc != KVC_OK) return rc;
    const ContainerLayout cl = container_layout(g.p);
    const bool empty = g.p.n_rows == 0;
    if (!out || !aligned(out, 16) || !slab_off || !aligned(slab_off, 8) ||
        (dev_status && !aligned(dev_status, 4)) ||
        (!empty && (!cdf || !max1 || !stream_len || !payload || !aligned(cdf, 4) ||
                    !aligned(max1, 4) || !aligned(stream_len, 4) || !aligned(payload, 4))))
        return KVC_ERR_ARG;
    if (out_cap < container_total(cl, 0)) return KVC_ERR_CAPACITY;
    return launch_status(launch_serialize(cdf, max1, stream_len, slab_off, payload, out, out_cap,
                                          g.p, dev_status, (hipStream_t)stream));
}

int kvc_serialize_chunk(const kvc_desc *desc, int64_t chunk, const uint16_t *cdf,
                        const uint16_t *max1, const uint16_t *stream_len, const uint64_t *slab_off,
                        const uint8_t *payload, uint8_t *out, int64_t out_cap, int32_t *dev_status,
                        void *stream)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    if (rc != KVC_OK) return rc;
    if (chunk < 0 || chunk >= g.p.NC) return KVC_ERR_ARG;
    kvc_desc cd = *desc;  // chunk `chunk` as a tensor of its own
    cd.n_tokens = (chunk == g.p.NC - 1) ? g.p.last_nj : g.p.Tc;
    Geometry gc;
    rc = make_geometry(&cd, gc);
    if (rc != KVC_OK) return rc;
    if (!out || !aligned(out, 16) || !slab_off || !aligned(slab_off, 8) || !cdf || !max1 ||
        !stream_len || !payload || !aligned(cdf, 4) || !aligned(max1, 4) || !aligned(stream_len, 4) ||
        (dev_status && !aligned(dev_status, 4)))
        return KVC_ERR_ARG;
    if (out_cap < container_total(container_layout(gc.p), 0)) return KVC_ERR_CAPACITY;
    const int64_t twoL = 2 * (int64_t)g.p.L;
    const ChunkRun run{cdf, g.p.S, twoL * g.p.C * g.p.A, max1, g.p.T, g.p.Tc, chunk,
                       stream_len + chunk * twoL * g.p.Tc, slab_off + chunk * twoL, payload, 1};
    return launch_status(launch_serialize_chunks(run, out, out_cap, gc.p, dev_status, (hipStream_t)stream));
}

int64_t kvc_stream_work_bytes(const kvc_desc *levels, int32_t n_levels, int32_t chunks_per_unit)
{
    Geometry g[KVC_MAX_LEVELS];
    StreamLayout sl;
    const int rc = stream_layout(levels, n_levels, chunks_per_unit, g, sl);
    return rc == KVC_OK ? sl.total : rc;
}

int kvc_stream_encode(const kvc_desc *levels, int32_t n_levels, const int32_t *chunk_level,
                      const uint8_t *const *sym, const uint16_t *const *cdf, const uint16_t *max1,
                      int32_t chunks_per_unit, void *work, int64_t work_bytes, uint8_t *host_out,
                      int64_t host_cap, int64_t *chunk_bytes, int32_t *dev_status, void *compute_stream,
                      void *copy_stream, kvc_chunk_fn on_chunk, void *user)
{
    Geometry g[KVC_MAX_LEVELS];
    StreamLayout sl;
    int rc = stream_layout(levels, n_levels, chunks_per_unit, g, sl);
    if (rc != KVC_OK) return rc;
    const KParams &P = g[0].p;
    if (P.NC == 0) return KVC_OK;
    if (!chunk_level || !sym || !cdf || !max1 || !aligned(max1, 4) || !work || !aligned(work, 256) ||
        !host_out || host_cap < 0 || !chunk_bytes || !aligned(chunk_bytes, 8) ||
        (dev_status && !aligned(dev_status, 4)))
        return KVC_ERR_ARG;
    for (int l = 0; l < n_levels; ++l)
        if (!sym[l] || !cdf[l] || !aligned(sym[l], 4) || !aligned(cdf[l], 4)) return KVC_ERR_ARG;
    for (int64_t j = 0; j < P.NC; ++j)
        if (chunk_level[j] < 0 || chunk_level[j] >= n_levels) return KVC_ERR_ARG;
    if (!host_pinned(host_out) || !host_pinned(chunk_bytes)) return KVC_ERR_ARG;
    if (work_bytes < sl.total) return KVC_ERR_CAPACITY;

    // units: runs of at most U consecutive chunks of one level
    struct Unit { int64_t ja, jb; int32_t level; };
    std::vector<Unit> units;
    for (int64_t j = 0; j < P.NC;) {
        int64_t jb = j + 1;
        while (jb < P.NC && jb - j < sl.U && chunk_level[jb] == chunk_level[j]) ++jb;
        units.push_back({j, jb, chunk_level[j]});
        j = jb;
    }
    const int64_t n_units = (int64_t)units.size();
    const int64_t twoL = 2 * (int64_t)P.L;
    uint8_t *const wk = (uint8_t *)work;
    uint16_t *const len_u = (uint16_t *)(wk + sl.len);
    uint64_t *const off_u = (uint64_t *)(wk + sl.off);
    uint8_t *const pay_u = wk + sl.pay;
    uint64_t *const sizes_u = (uint64_t *)(wk + sl.sizes);
    const hipStream_t cs = (hipStream_t)compute_stream, xs = (hipStream_t)copy_stream;
    auto staging = [&](int64_t u) { return wk + sl.staging + (u & 1) * sl.U * sl.chunk_cap; };
    auto packed = [&](int64_t u) { return wk + sl.packed + (u & 1) * sl.U * sl.chunk_cap; };

    // serialized[h]: unit containers packed into half h and their sizes in
    // chunk_bytes (compute stream); copied[h]: the copy out of half h done
    // (copy stream)
    hipEvent_t serialized[2] = {}, copied[2] = {};
    for (int h = 0; h < 2 && rc == KVC_OK; ++h)
        if (hipEventCreateWithFlags(&serialized[h], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&copied[h], hipEventDisableTiming) != hipSuccess)
            rc = KVC_ERR_HIP;
    std::vector<int64_t> host_off(P.NC, 0);
    int64_t cursor = 0;

    // Encode unit u and write its containers into staging half u % 2.
    auto enqueue = [&](int64_t u) -> int {
        const Unit &un = units[u];
        const int l = un.level;
        const KParams &pl = g[l].p;
        kvc_desc du = levels[l];
        du.n_tokens = std::min<int64_t>(un.jb * P.Tc, P.T) - un.ja * P.Tc;
        Geometry gu;
        if (make_geometry(&du, gu) != KVC_OK) return KVC_ERR_ARG;
        gu.p.Ts = P.T;     // the unit's rows sit in the whole tensor's row blocks,
        gu.p.S = pl.S;     // and its chunks read the whole tensor's tables
        gu.p.NG = pl.NG;
        gu.p.j0 = un.ja;
        const uint8_t *sym_u = sym[l] + un.ja * P.Tc * P.C;
        const uint16_t *cdf_u = cdf[l];
        uint8_t *slots = wk;
        uint64_t *slab_total = (uint64_t *)(wk + gu.slot_area);
        const bool vec16 = (P.C % 16 == 0) && aligned(sym_u, 16);
        hipError_t e = launch_encode(sym_u, cdf_u, slots, slab_total, len_u, off_u, pay_u, sl.pay_cap, gu.p,
                                     dev_status, vec16, cs);
        uint8_t *const st = staging(u);
        // the unit's full chunks in one set of launches, a shorter last chunk in its own
        const int64_t jfull = std::min<int64_t>(un.jb, P.T / P.Tc);
        for (int64_t ja = un.ja; ja < un.jb && e == hipSuccess;) {
            const int64_t jb = ja < jfull ? jfull : ja + 1, k = ja - un.ja;
            kvc_desc dc = levels[l];
            dc.n_tokens = std::min<int64_t>((ja + 1) * P.Tc, P.T) - ja * P.Tc;
            Geometry gc;
            if (make_geometry(&dc, gc) != KVC_OK) return KVC_ERR_ARG;
            const ChunkRun run{cdf[l], pl.S, twoL * P.C * pl.A, max1, P.T, P.Tc, ja, len_u + k * twoL * P.Tc,
                               off_u + k * twoL, pay_u, jb - ja};
            e = launch_serialize_chunks(run, st + k * sl.chunk_cap, sl.chunk_cap, gc.p, dev_status, cs);
            ja = jb;
        }
        const int n = (int)(un.jb - un.ja);
        if (e == hipSuccess) e = launch_container_totals(st, sl.chunk_cap, n, sizes_u, cs);
        // packed half u % 2 is free once the copy of unit u - 2 is done; the
        // containers then go into it back to back, for one copy per unit
        if (e == hipSuccess && u >= 2) e = hipStreamWaitEvent(cs, copied[u & 1], 0);
        if (e == hipSuccess) e = launch_pack_containers(st, sl.chunk_cap, sizes_u, n, packed(u), cs);
        if (e == hipSuccess)
            e = hipMemcpyAsync(chunk_bytes + un.ja, sizes_u, 8 * (size_t)n, hipMemcpyDeviceToHost, cs);
        if (e == hipSuccess) e = hipEventRecord(serialized[u & 1], cs);
        return launch_status(e);
    };
    // Copy unit u's containers, back to back at their exact sizes, to host_out
    // in one copy (a copy costs several microseconds beyond its bytes).
    auto copy_out = [&](int64_t u) -> int {
        const Unit &un = units[u];
        if (hipEventSynchronize(serialized[u & 1]) != hipSuccess) return KVC_ERR_HIP;
        int64_t total = 0;
        for (int64_t j = un.ja; j < un.jb; ++j) {
            const int64_t n = chunk_bytes[j];
            // not a container this call wrote (a container's total is a multiple of 16)
            if (n <= 0 || n > sl.chunk_cap || n % 16 != 0) return KVC_ERR_HIP;
            if (n > host_cap - cursor - total) return KVC_ERR_CAPACITY;
            host_off[j] = cursor + total;
            total += n;
        }
        if (hipMemcpyAsync(host_out + cursor, packed(u), (size_t)total, hipMemcpyDeviceToHost, xs) != hipSuccess)
            return KVC_ERR_HIP;
        cursor += total;
        return launch_status(hipEventRecord(copied[u & 1], xs));
    };
    // Hand unit u's containers to the caller once their copies are done.
    auto deliver = [&](int64_t u) -> int {
        if (!on_chunk) return KVC_OK;
        if (hipEventSynchronize(copied[u & 1]) != hipSuccess) return KVC_ERR_HIP;
        const Unit &un = units[u];
        for (int64_t j = un.ja; j < un.jb; ++j) on_chunk(user, j, un.level, host_out + host_off[j], chunk_bytes[j]);
        return KVC_OK;
    };
    // Unit u is encoded while unit u - 1 is copied; the callbacks of unit u - 2
    // run after both are queued.
    for (int64_t u = 0; u < n_units && rc == KVC_OK; ++u) {
        rc = enqueue(u);
        if (rc == KVC_OK && u >= 1) rc = copy_out(u - 1);
        if (rc == KVC_OK && u >= 2) rc = deliver(u - 2);
    }
    if (rc == KVC_OK) rc = copy_out(n_units - 1);
    if (rc == KVC_OK && n_units >= 2) rc = deliver(n_units - 2);
    if (rc == KVC_OK) rc = deliver(n_units - 1);
    // drain both streams before the events go (also after an error)
    const hipError_t e1 = hipStreamSynchronize(cs), e2 = hipStreamSynchronize(xs);
    if (rc == KVC_OK && (e1 != hipSuccess || e2 != hipSuccess)) rc = KVC_ERR_HIP;
    for (int h = 0; h < 2; ++h) {
        if (serialized[h]) (void)hipEventDestroy(serialized[h]);
        if (copied[h]) (void)hipEventDestroy(copied[h]);
    }
    return rc;
}

int kvc_deserialize(const kvc_desc *desc, const uint8_t *in, int64_t in_bytes, uint16_t *cdf,
                    uint16_t *max1, uint16_t *stream_len, uint64_t *slab_off, int32_t *dev_status,
                    void *stream)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    if (rc != KVC_OK) return rc;
    const ContainerLayout cl = container_layout(g.p);
    const bool empty = g.p.n_rows == 0;
    if (!in || !aligned(in, 16) || !slab_off || !aligned(slab_off, 8) ||
        (dev_status && !aligned(dev_status, 4)) ||
        (!empty && (!cdf || !max1 || !stream_len || !aligned(cdf, 4) || !aligned(max1, 4) ||
                    !aligned(stream_len, 4))))
        return KVC_ERR_ARG;
    if (in_bytes < container_total(cl, 0)) return KVC_ERR_CAPACITY;
    return launch_status(launch_deserialize(in, in_bytes, cdf, max1, stream_len, slab_off, g.p,
                                            dev_status, (hipStream_t)stream));
}

int kvc_int8_quantize(const kvc_desc *desc, int32_t group, const uint16_t *kv, uint8_t *q,
                      float *scale, uint8_t *zero_point, int32_t *dev_status, void *stream)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    if (rc != KVC_OK) return rc;
    if (group < 1 || g.p.C % group != 0) return KVC_ERR_ARG;
    if (g.p.n_rows == 0) return KVC_OK;
    if (!kv || !q || !scale || !zero_point || !aligned(kv, 4) || !aligned(q, 4) ||
        !aligned(scale, 4) || (dev_status && !aligned(dev_status, 4)))
        return KVC_ERR_ARG;
    const bool vec = aligned(kv, 16) && aligned(q, 8);
    return launch_status(launch_int8_quantize(kv, q, scale, zero_point, g.p.n_rows, g.p.C, group, vec,
                                              dev_status, (hipStream_t)stream));
}

int kvc_int8_dequantize(const kvc_desc *desc, int32_t group, const uint8_t *q, const float *scale,
                        const uint8_t *zero_point, void *out, int32_t out_dtype, void *stream)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    if (rc != KVC_OK) return rc;
    if (group < 1 || g.p.C % group != 0 || (out_dtype != KVC_F16 && out_dtype != KVC_F32)) return KVC_ERR_ARG;
    if (g.p.n_rows == 0) return KVC_OK;
    if (!q || !scale || !zero_point || !out || !aligned(scale, 4) || !aligned(out, 4))
        return KVC_ERR_ARG;
    return launch_status(launch_int8_dequantize(q, scale, zero_point, out, out_dtype == KVC_F32,
                                                g.p.n_rows * g.p.C, group, (hipStream_t)stream));
}

int kvc_delta_forward(const kvc_desc *desc, int32_t anchor_tokens, const uint16_t *kv, uint16_t *delta,
                      int32_t *dev_status, void *stream)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    if (rc != KVC_OK) return rc;
    if (anchor_tokens < 1 || anchor_tokens > 65535) return KVC_ERR_ARG;
    if (g.p.n_rows == 0) return KVC_OK;
    if (!kv || !delta || !aligned(kv, 2) || !aligned(delta, 2) || (dev_status && !aligned(dev_status, 4)))
        return KVC_ERR_ARG;
    const bool vec = g.p.C % 8 == 0 && g.p.C <= 1024 && aligned(kv, 16) && aligned(delta, 16);
    return launch_status(launch_delta_forward(kv, delta, g.p, anchor_tokens, vec, dev_status,
                                              (hipStream_t)stream));
}

int kvc_delta_inverse(const kvc_desc *desc, int32_t anchor_tokens, uint16_t *y, void *stream)
{
    Geometry g;
    int rc = make_geometry(desc, g);
    if (rc != KVC_OK) return rc;
    if (anchor_tokens < 1 || anchor_tokens > 65535) return KVC_ERR_ARG;
    if (g.p.n_rows == 0) return KVC_OK;
    if (!y || !aligned(y, 2)) return KVC_ERR_ARG;
    const bool vec = g.p.C % 8 == 0 && g.p.C <= 1024 && aligned(y, 16);
    return launch_status(launch_delta_inverse(y, g.p, anchor_tokens, vec, (hipStream_t)stream));
}

}  // extern "C"
