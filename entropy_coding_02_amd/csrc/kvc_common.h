// kvc_common.h - launch geometry and small device helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvc.h"

#define KVC_MAX_LAYERS 256

// Pointers into LDS.  Typed with the LDS address space so the compiler emits
// ds_* instructions (32-bit addresses, own wait counter) rather than flat ones.
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// Everything a kernel needs to know about the problem, passed by value.
// Slab s = (chunk j, layer l, K|V kv) with lk = 2*l + kv; j = s / (2L).
struct KParams {
    int64_t T;          // tokens
    int64_t n_rows;     // 2 * L * T
    int64_t n_slabs;    // NC * 2L
    int64_t n_streams;  // 2 * L * T
    int64_t slot_bytes; // encoder scratch bytes per stream
    int32_t L, C, A, Tc;
    int32_t NC;         // chunks
    int32_t last_nj;    // tokens of the last chunk
    uint8_t maxq[2 * KVC_MAX_LAYERS];  // MAX = bins/2 - 1 per (l, kv)
};

struct SlabGeom {
    int64_t row0;    // row index of the slab's first token: lk*T + j*Tc
    int64_t sid0;    // stream id of the slab's first token
    int32_t nj;      // tokens in the slab
    int32_t lk;      // 2*l + kv
};

__device__ __forceinline__ SlabGeom slab_geom(const KParams &p, int64_t s)
{
    SlabGeom g;
    int64_t twoL = 2 * (int64_t)p.L;
    int64_t j = s / twoL;
    g.lk = (int32_t)(s - j * twoL);
    g.nj = (j == p.NC - 1) ? p.last_nj : p.Tc;
    g.row0 = (int64_t)g.lk * p.T + j * p.Tc;
    g.sid0 = j * twoL * p.Tc + (int64_t)g.lk * g.nj;
    return g;
}

__device__ __forceinline__ float kvc_h2f(uint32_t bits)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

__device__ __forceinline__ uint32_t kvc_f2h(float f)
{
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    for (int off = 32; off > 0; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v)
{
    for (int off = 32; off > 0; off >>= 1) v += (uint32_t)__shfl_xor((int)v, off, 64);
    return v;
}

__device__ __forceinline__ void kvc_flag(int32_t *status, int32_t bit)
{
    if (status) atomicOr(status, bit);
}
