// kvc_quantize.hip - group max-abs quantization ([CG] 2.3 step 1), alone or
// fused with the histograms and CDFs of steps 2-3.
//
// One wavefront per (layer, K|V, token) row.  For finite fp16, |x| orders
// like its bit pattern with the sign cleared, so the row max is an integer
// max of (bits & 0x7FFF): exact, and it detects Inf/NaN (>= 0x7C00) for free.
// The quantizer runs in fp32 with one rounding per operation (the library is
// built with -ffp-contract=off): factor = MAX / m by IEEE division,
// p = x * factor, p = p + MAX, q = rint(p) (round half to even).  (The fast
// paths write the product as fma(x, factor, 0), the same single rounding.)
#include "kvc_common.h"
#include "kvc_kernels.h"

namespace {

// Slab of fused-pass block b, numbered so that blocks that run at the same
// time read neighbouring memory: consecutive blocks take consecutive chunks
// of one (layer, K|V), whose rows lie back to back, instead of the 2L slabs
// of one chunk, which lie a whole (layer, K|V) apart (one block per slab).
__device__ inline int64_t slab_in_memory_order(const KParams &p, int64_t b)
{
    return (b % p.NC) * (2 * (int64_t)p.L) + b / p.NC;
}

__device__ __forceinline__ uint32_t quant1f(float x, float factor, float M)
{
    float p = x * factor;
    p = p + M;
    float r = __builtin_rintf(p);
    r = r < 0.0f ? 0.0f : (r > 255.0f ? 255.0f : r);  // only non-finite rows get here
    return (uint32_t)r;
}

__device__ __forceinline__ uint32_t quant1(uint32_t bits, float factor, float M)
{
    float p = kvc_h2f(bits) * factor;
    p = p + M;
    float r = __builtin_rintf(p);
    r = r < 0.0f ? 0.0f : (r > 255.0f ? 255.0f : r);  // only non-finite rows get here
    return (uint32_t)r;
}

// For a finite row (every |x| <= m, so p lies in
// [0, 2 MAX] up to a rounding and |p| < 2^22): p + 1.5 * 2^23 is rounded to
// an integer, ties to even, which is rint(p); its fp32 bits are 0x4B400000 +
// rint(p), the symbol in the low byte.  Rows holding Inf or NaN take the
// clamped quant1 instead (they are flagged; their symbols only stay in range).
// The product is written as fma(x, factor, 0): one rounding of the exact
// product, the same value as x * factor (a zero's sign aside, which the
// + MAX that follows erases), and with x converted from fp16 the compiler
// folds the conversion into one v_fma_mix_f32.
__device__ __forceinline__ uint32_t quant_bits(float x, float factor, float M)
{
    float p = __builtin_fmaf(x, factor, 0.0f);
    p = p + M;
    return __float_as_uint(p + 12582912.0f);
}

// The low bytes of four words, b0 lowest.
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3)
{
    return __builtin_amdgcn_perm(b1, b0, 0x0C0C0400u) | __builtin_amdgcn_perm(b3, b2, 0x04000C0Cu);
}

// Row max of the wave's 64 lanes, uniform: DPP steps within quads, half
// rows and rows, then the row broadcasts; lane 63 ends with the maximum.
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row half mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row bcast 15
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row bcast 31
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// VEC = fp16 elements per lane access: 8 (16-byte loads, C % 8 == 0 and
// 16-byte aligned buffers) or 1 (any C).
template <int VEC>
__global__ __launch_bounds__(256) void k_quantize_rows(const uint16_t *__restrict__ kv,
                                                       uint8_t *__restrict__ sym,
                                                       uint16_t *__restrict__ max1, KParams p,
                                                       int32_t *status)
{
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const int C = p.C;
    for (int64_t row = wave; row < p.n_rows; row += nwaves) {
        const uint16_t *x = kv + row * C;
        uint8_t *q = sym + row * C;
        uint32_t mx = 0;
        // rows of up to 1024 channels stay in registers (two 16-byte pieces per lane)
        constexpr int KREG = VEC == 8 ? 2 : 1;
        u32x4 reg[KREG];
        if constexpr (VEC == 8) {
#pragma unroll
            for (int k = 0; k < KREG; ++k) {
                const int c = (lane + 64 * k) * 8;
                reg[k] = c < C ? *(const u32x4 *)(x + c) : u32x4{0, 0, 0, 0};
            }
            for (int c = (lane + 64 * KREG) * 8; c < C; c += 64 * 8) {
                const u32x4 v = *(const u32x4 *)(x + c);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t a = v[i] & 0x7FFF7FFFu;
                    mx = max(mx, max(a & 0xFFFFu, a >> 16));
                }
            }
#pragma unroll
            for (int k = 0; k < KREG; ++k)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t a = reg[k][i] & 0x7FFF7FFFu;
                    mx = max(mx, max(a & 0xFFFFu, a >> 16));
                }
        } else {
            for (int c = lane; c < C; c += 64) mx = max(mx, (uint32_t)(x[c] & 0x7FFFu));
        }
        mx = (VEC == 8) ? wave_max_dpp(mx) : wave_max_u32(mx);
        const int32_t lk = (int32_t)(row / p.T);
        const float M = (float)p.maxq[lk];
        const float m = kvc_h2f(mx);
        const float factor = (mx != 0) ? M / m : 0.0f;
        if (mx >= 0x7C00u && lane == 0) kvc_flag(status, KVC_DEV_NONFINITE);
        if (lane == 0) max1[row] = (uint16_t)mx;
        if constexpr (VEC == 8) {
            const bool finite = mx < 0x7C00u;
            auto put = [&](int c, const u32x4 &v) {
                uint32_t b[2] = {0, 0};
                if (finite) {
                    uint32_t w[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        w[i] = quant_bits(kvc_h2f((v[i >> 1] >> (16 * (i & 1))) & 0xFFFFu), factor, M);
                    b[0] = pack_low_bytes(w[0], w[1], w[2], w[3]);
                    b[1] = pack_low_bytes(w[4], w[5], w[6], w[7]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t q0 = quant1(v[i] & 0xFFFFu, factor, M);
                        const uint32_t q1 = quant1(v[i] >> 16, factor, M);
                        b[i >> 1] |= (q0 | (q1 << 8)) << ((i & 1) * 16);
                    }
                }
                *(uint2 *)(q + c) = make_uint2(b[0], b[1]);
            };
#pragma unroll
            for (int k = 0; k < KREG; ++k) {
                const int c = (lane + 64 * k) * 8;
                if (c < C) put(c, reg[k]);
            }
            for (int c = (lane + 64 * KREG) * 8; c < C; c += 64 * 8) put(c, *(const u32x4 *)(x + c));
        } else {
            for (int c = lane; c < C; c += 64) q[c] = (uint8_t)quant1(x[c], factor, M);
        }
    }
}

// max over the lane's pieces of |x| as bits (sign cleared), two halves per
// packed 16-bit max.
template <int KREG>
__device__ __forceinline__ uint32_t lane_absmax(const u32x4 (&r)[KREG])
{
    typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
    u16x2 acc = {0, 0};
#pragma unroll
    for (int k = 0; k < KREG; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            acc = __builtin_elementwise_max(acc, __builtin_bit_cast(u16x2, r[k][i] & 0x7FFF7FFFu));
    return max((uint32_t)acc.x, (uint32_t)acc.y);
}

// Histogram layout of the fused passes (C % 8 == 0, C8 = C / 8): the 16-bit
// counter of (symbol s, channel c = 8 pi + i) is half (i & 1) of word
// s * (C / 2) + (i >> 1) * C8 + pi.  At each step the lanes of a wave hold
// consecutive pieces pi of one element slot i, so their atomics go to
// consecutive words (distinct banks) whatever the symbols, and which half a
// counter is does not depend on the data.
__device__ __forceinline__ int hist_word(int s, int i, int pi, int C8)
{
    return s * 4 * C8 + (i >> 1) * C8 + pi;
}

// CDF rows of one slab from its histogram (layout above) at hist: thread j
// takes channel 8 (j % C8) + j / C8, so the lanes of a wave read consecutive
// words.  Rows of A entries (A % 8 == 0) go out as 16-byte stores.
__device__ __forceinline__ void slab_cdf_rows(const uint32_t *hist, uint16_t *cdf, int64_t slab, int C,
                                              int A, double rn)
{
    const int C8 = C / 8;
    const uint32_t K = 65536u - (uint32_t)A;
    for (int j = threadIdx.x; j < C; j += blockDim.x) {
        const int pi = j % C8, i = j / C8;
        const uint32_t *h = hist + hist_word(0, i, pi, C8);
        const int sh = 16 * (i & 1);
        uint32_t *dst = (uint32_t *)(cdf + (slab * C + 8 * pi + i) * A);
        uint32_t Ck = 0;
        for (int k = 0; k < A; k += 8) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = kvc_cdf_entry((uint32_t)(k + 2 * e), Ck, K, rn);
                Ck += (h[(k + 2 * e) * 4 * C8] >> sh) & 0xFFFFu;
                const uint32_t hi = kvc_cdf_entry((uint32_t)(k + 2 * e + 1), Ck, K, rn);
                Ck += (h[(k + 2 * e + 1) * 4 * C8] >> sh) & 0xFFFFu;
                w[e] = lo | (hi << 16);
            }
            *(u32x4 *)(dst + k / 2) = u32x4{w[0], w[1], w[2], w[3]};
        }
    }
}

__device__ __forceinline__ void zero_lds(uint32_t *hist, int words)  // words % 4 == 0
{
    for (int i = 4 * threadIdx.x; i < words; i += 4 * blockDim.x) *(u32x4 *)(hist + i) = u32x4{0, 0, 0, 0};
}

// One element of a finite row: its quantizer bits b (symbol in the low
// byte) counted at the byte offset (b & 0xFFFFFF) * rowb + base, where base
// already takes off the 0x400000 * rowb that the bits' 0x4B40 prefix adds.
__device__ __forceinline__ void count_bits(lds_u8 *h8, uint32_t b, uint32_t rowb, uint32_t base, uint32_t one)
{
    const uint32_t off = (b & 0xFFFFFFu) * rowb + base;
    __hip_atomic_fetch_add((lds_u32 *)(h8 + off), one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Quantization, histograms and CDFs in one pass: one block of 1024 threads
// per slab (chunk, layer, K|V), for C % 8 == 0 and C <= 512 * KREG.  Each
// wave takes whole token rows: the row (8 channels per 16-byte piece, KREG
// pieces per lane) stays in registers for the integer max, the quantizer
// and the symbol stores, and every symbol is counted at once in the LDS
// histogram of 16-bit counters.  After the last row the block turns the
// counts into CDF rows (kvc_cdf_entry).  The input is read once; no pass
// re-reads the symbols.
template <int KREG>
__global__ __launch_bounds__(1024) void k_quant_cdf(const uint16_t *__restrict__ kv,
                                                    uint8_t *__restrict__ sym,
                                                    uint16_t *__restrict__ max1,
                                                    uint16_t *__restrict__ cdf, KParams p,
                                                    int32_t *status)
{
    extern __shared__ uint32_t hist[];
    lds_u8 *const h8 = (lds_u8 *)hist;
    const int64_t slab = slab_in_memory_order(p, blockIdx.x);
    const SlabGeom g = slab_geom(p, slab);
    const int C = p.C, A = p.A, C8 = C / 8;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    zero_lds(hist, (A / 2) * C);
    const float M = (float)p.maxq[g.lk];
    const uint32_t amax = (uint32_t)A - 1u;
    const uint32_t rowb = ((uint32_t)C & 0x7F8u) * 2u;  // bytes from one symbol's counters to the next's
    uint32_t base[KREG][4];
#pragma unroll
    for (int k = 0; k < KREG; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j) base[k][j] = 4u * (uint32_t)hist_word(0, 2 * j, lane + 64 * k, C8) - 0x400000u * rowb;
    __syncthreads();
    // Software pipeline over the wave's rows t = wid, wid + nw, ...: the rows
    // two steps ahead are loaded while the current one is processed (three
    // buffers, in turn, so no registers are copied), so a wave keeps two rows
    // of loads in flight; and a row's symbol stores go out after the next
    // row's data has arrived, so the wait for a load never also waits for
    // stores issued just before it.
    auto load_row = [&](int t, u32x4 *r) {
        const uint16_t *x = kv + (g.row0 + t) * C;
#pragma unroll
        for (int k = 0; k < KREG; ++k) {
            const int pi = lane + 64 * k;
            r[k] = pi < C8 ? *(const u32x4 *)(x + 8 * pi) : u32x4{0, 0, 0, 0};
        }
    };
    u32x4 ba[KREG], bb[KREG], bc[KREG];
    uint32_t qb[KREG][2];  // the previous row's symbols, not yet stored
    int64_t qrow = -1;
    auto store_row = [&]() {
#pragma unroll
        for (int k = 0; k < KREG; ++k) {
            const int pi = lane + 64 * k;
            if (pi < C8) *(uint2 *)(sym + qrow * C + 8 * pi) = make_uint2(qb[k][0], qb[k][1]);
        }
    };
    // row t from cur; the loads of row t + 2 nw into pf
    auto step = [&](int t, const u32x4(&cur)[KREG], u32x4(&pf)[KREG]) {
        const int64_t row = g.row0 + t;
        uint32_t mx = lane_absmax<KREG>(cur);
        if (qrow >= 0) store_row();
        if (t + 2 * nw < g.nj) load_row(t + 2 * nw, pf);
        mx = wave_max_dpp(mx);
        const float m = kvc_h2f(mx);
        const float factor = (mx != 0) ? M / m : 0.0f;
        if (lane == 0) max1[row] = (uint16_t)mx;
        if (mx < 0x7C00u) {
#pragma unroll
            for (int k = 0; k < KREG; ++k) {
                const int pi = lane + 64 * k;
                if (pi >= C8) continue;
                uint32_t b[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    b[i] = quant_bits(kvc_h2f((cur[k][i >> 1] >> (16 * (i & 1))) & 0xFFFFu), factor, M);
                    count_bits(h8, b[i], rowb, base[k][i >> 1], (i & 1) ? 0x10000u : 1u);
                }
                qb[k][0] = pack_low_bytes(b[0], b[1], b[2], b[3]);
                qb[k][1] = pack_low_bytes(b[4], b[5], b[6], b[7]);
            }
        } else {
            if (lane == 0) kvc_flag(status, KVC_DEV_NONFINITE);
#pragma unroll
            for (int k = 0; k < KREG; ++k) {
                const int pi = lane + 64 * k;
                qb[k][0] = qb[k][1] = 0;
                if (pi >= C8) continue;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t q = quant1((cur[k][i >> 1] >> (16 * (i & 1))) & 0xFFFFu, factor, M);
                    qb[k][i >> 2] |= q << (8 * (i & 3));
                    const uint32_t s = q < amax ? q : amax;
                    atomicAdd(&hist[hist_word((int)s, i, pi, C8)], (i & 1) ? 0x10000u : 1u);
                }
            }
        }
        qrow = row;
    };
    if (wid < g.nj) load_row(wid, ba);
    if (wid + nw < g.nj) load_row(wid + nw, bb);
    for (int t = wid; t < g.nj; t += 3 * nw) {
        step(t, ba, bc);
        if (t + nw >= g.nj) break;
        step(t + nw, bb, ba);
        if (t + 2 * nw >= g.nj) break;
        step(t + 2 * nw, bc, bb);
    }
    if (qrow >= 0) store_row();
    __syncthreads();
    slab_cdf_rows(hist, cdf, slab, C, A, g.rn);
}

// Several quality levels (bins tables) of the same tensor in one pass: as
// k_quant_cdf, but each row, read once, is quantized and counted for every
// level (level i: its own MAX per (layer, K|V), symbols, histogram at word
// offset lv.hist[i] of LDS and CDF rows).  The shared row max goes to max1.
template <int KREG>
__global__ __launch_bounds__(1024) void k_quant_cdf_levels(const uint16_t *__restrict__ kv,
                                                           uint16_t *__restrict__ max1, KParams p,
                                                           LevelParams lv, int32_t *status)
{
    extern __shared__ uint32_t hist[];
    const int64_t slab = slab_in_memory_order(p, blockIdx.x);
    const SlabGeom g = slab_geom(p, slab);
    const int C = p.C, C8 = C / 8;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const uint32_t rowb = ((uint32_t)C & 0x7F8u) * 2u;
    zero_lds(hist, lv.words);
    __syncthreads();
    for (int t = wid; t < g.nj; t += nw) {
        const int64_t row = g.row0 + t;
        const uint16_t *x = kv + row * C;
        u32x4 reg[KREG];
#pragma unroll
        for (int k = 0; k < KREG; ++k) {
            const int pi = lane + 64 * k;
            reg[k] = pi < C8 ? *(const u32x4 *)(x + 8 * pi) : u32x4{0, 0, 0, 0};
        }
        const uint32_t mx = wave_max_dpp(lane_absmax<KREG>(reg));
        const float m = kvc_h2f(mx);
        if (lane == 0) max1[row] = (uint16_t)mx;
        if (mx >= 0x7C00u && lane == 0) kvc_flag(status, KVC_DEV_NONFINITE);
        float xf[KREG][8];  // the row's values in fp32, converted once for all levels
#pragma unroll
        for (int k = 0; k < KREG; ++k)
#pragma unroll
            for (int i = 0; i < 8; ++i) xf[k][i] = kvc_h2f((reg[k][i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
#pragma unroll 1
        for (int l = 0; l < lv.n; ++l) {
            const float M = (float)lv.maxq[l][g.lk];
            const float factor = (mx != 0) ? M / m : 0.0f;
            const uint32_t amax = (uint32_t)lv.A[l] - 1u;
            uint32_t *h = hist + lv.hist[l];
            lds_u8 *const h8 = (lds_u8 *)h;
#pragma unroll
            for (int k = 0; k < KREG; ++k) {
                const int pi = lane + 64 * k;
                if (pi >= C8) continue;
                uint32_t q2[2];
                if (mx < 0x7C00u) {
                    uint32_t b[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        b[i] = quant_bits(xf[k][i], factor, M);
                        const uint32_t base = 4u * (uint32_t)hist_word(0, i, pi, C8) - 0x400000u * rowb;
                        count_bits(h8, b[i], rowb, base, (i & 1) ? 0x10000u : 1u);
                    }
                    q2[0] = pack_low_bytes(b[0], b[1], b[2], b[3]);
                    q2[1] = pack_low_bytes(b[4], b[5], b[6], b[7]);
                } else {
                    q2[0] = q2[1] = 0;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const uint32_t q = quant1f(xf[k][i], factor, M);
                        q2[i >> 2] |= q << (8 * (i & 3));
                        const uint32_t s = q < amax ? q : amax;
                        atomicAdd(&h[hist_word((int)s, i, pi, C8)], (i & 1) ? 0x10000u : 1u);
                    }
                }
                *(uint2 *)(lv.sym[l] + row * C + 8 * pi) = make_uint2(q2[0], q2[1]);
            }
        }
    }
    __syncthreads();
#pragma unroll 1
    for (int l = 0; l < lv.n; ++l) slab_cdf_rows(hist + lv.hist[l], lv.cdf[l], slab, C, lv.A[l], g.rn);
}

}  // namespace

// Dynamic LDS of the fused pass, or 0 when the shape does not qualify
// (C % 8, C <= 1024, A % 8, histogram within the device's LDS per block).
static size_t quant_cdf_lds(const KParams &p)
{
    if (p.C % 8 != 0 || p.C > 1024 || p.A % 8 != 0) return 0;
    const size_t bytes = sizeof(uint32_t) * (size_t)(p.A / 2) * (size_t)p.C;
    int dev = 0, lim = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
        return 0;
    return bytes <= (size_t)lim ? bytes : 0;
}

bool quant_cdf_fused_ok(const KParams &p) { return quant_cdf_lds(p) != 0; }

hipError_t launch_quant_cdf(const uint16_t *kv, uint8_t *sym, uint16_t *max1, uint16_t *cdf,
                            const KParams &p, int32_t *status, hipStream_t stream)
{
    if (p.n_slabs == 0) return hipSuccess;
    const size_t lds = quant_cdf_lds(p);
    if (lds == 0) return hipErrorInvalidValue;
    const void *fn = p.C <= 512 ? (const void *)k_quant_cdf<1> : (const void *)k_quant_cdf<2>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    if (p.C <= 512)
        hipLaunchKernelGGL(k_quant_cdf<1>, dim3((unsigned)p.n_slabs), dim3(1024), lds, stream, kv, sym,
                           max1, cdf, p, status);
    else
        hipLaunchKernelGGL(k_quant_cdf<2>, dim3((unsigned)p.n_slabs), dim3(1024), lds, stream, kv, sym,
                           max1, cdf, p, status);
    return hipGetLastError();
}

// LDS bytes of the multi-level pass (setting lv's histogram offsets), or 0
// when the shape does not qualify.
static size_t quant_cdf_levels_lds(const KParams &p, LevelParams &lv)
{
    if (p.C % 8 != 0 || p.C > 1024) return 0;
    lv.words = 0;
    for (int l = 0; l < lv.n; ++l) {
        if (lv.A[l] % 8 != 0) return 0;
        lv.hist[l] = lv.words;
        lv.words += (lv.A[l] / 2) * p.C;
    }
    const size_t lds = sizeof(uint32_t) * (size_t)lv.words;
    int dev = 0, lim = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
        return 0;
    return lds <= (size_t)lim ? lds : 0;
}

bool quant_cdf_levels_ok(const KParams &p, const LevelParams &lv)
{
    LevelParams t = lv;
    return quant_cdf_levels_lds(p, t) != 0;
}

hipError_t launch_quant_cdf_levels(const uint16_t *kv, uint16_t *max1, const KParams &p,
                                   LevelParams lv, int32_t *status, hipStream_t stream)
{
    if (p.n_slabs == 0) return hipSuccess;
    const size_t lds = quant_cdf_levels_lds(p, lv);
    if (lds == 0) return hipErrorInvalidValue;
    const void *fn = p.C <= 512 ? (const void *)k_quant_cdf_levels<1> : (const void *)k_quant_cdf_levels<2>;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    if (p.C <= 512)
        hipLaunchKernelGGL(k_quant_cdf_levels<1>, dim3((unsigned)p.n_slabs), dim3(1024), lds, stream,
                           kv, max1, p, lv, status);
    else
        hipLaunchKernelGGL(k_quant_cdf_levels<2>, dim3((unsigned)p.n_slabs), dim3(1024), lds, stream,
                           kv, max1, p, lv, status);
    return hipGetLastError();
}

hipError_t launch_quantize_rows(const uint16_t *kv, uint8_t *sym, uint16_t *max1, const KParams &p,
                                int32_t *status, bool vec8, hipStream_t stream)
{
    if (p.n_rows == 0) return hipSuccess;
    int64_t blocks = (p.n_rows + 3) / 4;  // one wave per row, 4 waves per block
    const int64_t cap = 256 * 1024;
    if (blocks > cap) blocks = cap;
    if (vec8)
        hipLaunchKernelGGL(k_quantize_rows<8>, dim3((unsigned)blocks), dim3(256), 0, stream, kv, sym,
                           max1, p, status);
    else
        hipLaunchKernelGGL(k_quantize_rows<1>, dim3((unsigned)blocks), dim3(256), 0, stream, kv, sym,
                           max1, p, status);
    return hipGetLastError();
}
