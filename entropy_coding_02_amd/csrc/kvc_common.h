// kvc_common.h - launch geometry and small device helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvc.h"

// Status bit a kvc_encode launch that stages only the first entries of each
// CDF row sets on meeting a symbol past them; the guard launch that follows
// then encodes everything again over whole rows, and k_scan clears the bit,
// so no call leaves it set.
#define KVC_DEV_INTERNAL_REDO (1 << 30)

#define KVC_MAX_LAYERS 256

// Pointers into LDS.  Typed with the LDS address space so the compiler emits
// ds_* instructions (32-bit addresses, own wait counter) rather than flat ones.
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

// Everything a kernel needs to know about the problem, passed by value.
// Slab s = (chunk j, layer l, K|V kv) with lk = 2*l + kv; j = s / (2L).
// CDF table (g, l, kv) serves the slabs of chunks j with floor(j / S) = g.
struct KParams {
    int64_t T;          // tokens
    int64_t Ts;         // token stride of the (layer, K|V) row blocks in kv and sym: T, or the
                        // whole tensor's T when a run of its chunks is encoded as a tensor
    int64_t n_rows;     // 2 * L * T
    int64_t n_slabs;    // NC * 2L
    int64_t n_streams;  // 2 * L * T
    int64_t slot_bytes; // encoder scratch bytes per stream
    int32_t L, C, A, Tc;
    int32_t NC;         // chunks
    int32_t S;          // chunks per CDF table (1: a table per chunk)
    int32_t NG;         // CDF tables per (layer, K|V): ceil(NC / S)
    int64_t j0;         // chunk index of chunk 0 within the tensor whose tables the kernels
                        // read (0; else the first chunk of a run encoded as a tensor)
    int32_t last_nj;    // tokens of the last chunk
    double rn_full;     // 1 / Tc, rounded to double
    double rn_last;     // 1 / last_nj, rounded to double (0 if there are no tokens)
    uint8_t maxq[2 * KVC_MAX_LAYERS];  // MAX = bins/2 - 1 per (l, kv)
};

struct SlabGeom {
    int64_t row0;    // row index of the slab's first token: lk*Ts + j*Tc
    int64_t sid0;    // stream id of the slab's first token
    int64_t tab;     // CDF table of the slab: floor((j + j0) / S) * 2L + lk
    int32_t nj;      // tokens in the slab
    int32_t lk;      // 2*l + kv
    double rn;       // 1 / nj, rounded to double
};

__device__ __forceinline__ SlabGeom slab_geom(const KParams &p, int64_t s)
{
    SlabGeom g;
    int64_t twoL = 2 * (int64_t)p.L;
    int64_t j = s / twoL;
    g.lk = (int32_t)(s - j * twoL);
    g.nj = (j == p.NC - 1) ? p.last_nj : p.Tc;
    g.rn = (j == p.NC - 1) ? p.rn_last : p.rn_full;
    g.row0 = (int64_t)g.lk * p.Ts + j * p.Tc;
    g.sid0 = j * twoL * p.Tc + (int64_t)g.lk * g.nj;
    g.tab = (p.S == 1 ? j + p.j0 : (j + p.j0) / p.S) * twoL + g.lk;
    return g;
}

// CDF entry k of a row whose counts below k sum to Ck, over N tokens, with
// K = 65536 - A:  k + floor(Ck * K / N), rn = 1/N rounded to double.
// Exact for N <= 2^21: x = Ck * K < 2^37 is exact in fp64, and x * rn is x/N
// within a relative 2^-52 (x/N <= K < 2^16: under 2^-36 absolutely).  If x/N
// is an integer m the biased product lands in (m, m + 2^-21); otherwise x/N
// is at least 1/N >= 2^-21 away from both neighbouring integers, and the
// product plus 2^-22 stays strictly between them.  The integer part is the floor.
__device__ __forceinline__ uint32_t kvc_cdf_entry(uint32_t k, uint32_t Ck, uint32_t K, double rn)
{
    const double q = (double)((uint64_t)Ck * K) * rn;
    return k + (uint32_t)(q + 0x1p-22);
}

// Largest number of tokens one CDF table may count (kvc_cdf_entry's bound).
constexpr int64_t KVC_MAX_TABLE_TOKENS = (int64_t)1 << 21;

__device__ __forceinline__ float kvc_h2f(uint32_t bits)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// fp32 to fp16 bits, rounded to nearest even.  The empty asm keeps f a
// rounded fp32 value: otherwise the compiler may fold the product feeding it
// into one mixed-precision FMA that rounds to fp16 once, while every product
// here is defined as rounded to fp32 first and then to fp16.
__device__ __forceinline__ uint32_t kvc_f2h(float f)
{
    __asm__("" : "+v"(f));
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Two floats to a packed fp16 pair (lo in the low half), each rounded to
// nearest even: one v_cvt_pk_f16_f32 on gfx950.
__device__ __forceinline__ uint32_t kvc_f2h2(float lo, float hi)
{
    __asm__("" : "+v"(lo), "+v"(hi));  // as in kvc_f2h
    typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
    typedef float float2_t __attribute__((ext_vector_type(2)));
    const float2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, half2_t));
}

// Nonzero when some byte of w is >= A (4 <= A <= 256), without unpacking the
// bytes: for A <= 128 a byte b is >= A when its top bit is set or its low
// seven bits plus 128 - A carry into bit 7; for A > 128 when its top bit is
// set and its low seven bits plus 256 - A carry into bit 7.  The sums stay
// below 256, so no carry crosses into the next byte.
__host__ __device__ __forceinline__ uint32_t kvc_bytes_ge(uint32_t w, uint32_t A)
{
    if (A >= 256u) return 0u;
    const uint32_t lo = w & 0x7F7F7F7Fu;
    if (A <= 128u) return ((lo + (128u - A) * 0x01010101u) | w) & 0x80808080u;
    return ((lo + (256u - A) * 0x01010101u) & w) & 0x80808080u;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    for (int off = 32; off > 0; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

// The dispatcher hands workgroups to the 8 XCDs (each with its own L2) in
// turn, so block b runs on XCD b % 8.  xcd_block renumbers a grid of nb
// blocks so that consecutive numbers run on one XCD (a bijection of
// [0, nb); the last nb % 8 keep their numbers): blocks of one slab, which
// stage the same CDF rows, then read them through one L2 instead of up to
// eight.  Which XCD runs a block changes nothing but where its reads hit.
__host__ __device__ __forceinline__ int64_t xcd_block(int64_t b, int64_t nb)
{
    const int64_t per = nb >> 3;
    if (b >= (per << 3)) return b;
    return (b & 7) * per + (b >> 3);
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v)
{
    for (int off = 32; off > 0; off >>= 1) v += (uint32_t)__shfl_xor((int)v, off, 64);
    return v;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v)
{
    for (int off = 32; off > 0; off >>= 1) v += (uint64_t)__shfl_xor((unsigned long long)v, off, 64);
    return v;
}

__device__ __forceinline__ void kvc_flag(int32_t *status, int32_t bit)
{
    if (status) atomicOr(status, bit);
}
