// Device helpers shared by the RVQ GEMV kernels (decode on the fly from
// 24-bit code pairs in the tiled record layout; see include/moe.h).
#pragma once

#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    _Float16 a = (_Float16)lo, b = (_Float16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Power-of-two range scaling before a rounding to fp16 (largest finite value
// 65504): for a block whose largest magnitude is amax, e such that
// amax * 2^-e lies in [2^kRangeExp, 2^(kRangeExp + 1)).  The scaled values
// then stay below 2^8, and a sum of 8 of them times codebook entries below
// 16 in magnitude stays below 2^15.  Scaling by 2^-e before the rounding and
// by 2^e after the fp32 sum is exact (ldexp), so only the fp16 rounding
// itself remains, at the same relative size as for unscaled inputs.
constexpr int kRangeExp = 7;
__device__ __forceinline__ int range_exp(float amax) {
    const uint32_t b = __float_as_uint(amax);
    if (!(amax > 0.f) || b >= 0x7F800000u) return 0;   // zero, NaN, inf: no scaling
    const int p = (int)(b >> 23) - 127;                 // floor(log2 amax); -127 for subnormals
    return min(max(p - kRangeExp, -120), 120);
}

// Local item -> (global item, record).
__device__ __forceinline__ const uint8_t *resolve_record(const RecSrc &s, int local, int &item) {
    // uniform across the workgroup: scalar loads of the argument arrays
    // (a vector load of the argument segment is a memory round trip)
    const int t = __builtin_amdgcn_readfirstlane(local / s.n_local);
    const int l = __builtin_amdgcn_readfirstlane(local % s.n_local);
    if (s.table) {
        item = t * s.k + l;
        return (const uint8_t *)s.table[s.idx[item]];
    }
    item = t * s.k + s.rank[l];
    return (const uint8_t *)s.list[l];
}

// Byte address in an LDS codebook of the stage-1 (a) and stage-2 (b) rows of
// group g (0..15) of a 48-byte strip held in 12 dwords d[].
template <int G>
__device__ __forceinline__ void group_addr(const uint32_t (&d)[12], uint32_t &aa, uint32_t &ba) {
    constexpr int bit = 24 * G, i = bit / 32, s = bit % 32;
    uint32_t v;
    if constexpr (s <= 8) v = d[i] >> s;
    else v = __builtin_amdgcn_alignbit(d[i + 1], d[i], s);
    aa = (v << 4) & 0xFFF0u;        // a * 16
    ba = (v >> 8) & 0xFFF0u;        // b * 16
}

// acc[g%4] += sum over the 16 groups of (C[a] + C[b]) . x_group
template <int G>
__device__ __forceinline__ void strip_dot(const uint32_t (&d)[12], const char *cb, const uint32_t *xp,
                                          float (&acc)[4]) {
    if constexpr (G < 16) {
        uint32_t aa, ba;
        group_addr<G>(d, aa, ba);
        const u32x4 ca = *(const u32x4 *)(cb + aa);
        const u32x4 cbv = *(const u32x4 *)(cb + ba);
        const uint32_t x0 = xp[4 * G + 0], x1 = xp[4 * G + 1], x2 = xp[4 * G + 2], x3 = xp[4 * G + 3];
        float a = acc[G & 3];
        a = dot2(ca.x, x0, a);
        a = dot2(ca.y, x1, a);
        a = dot2(ca.z, x2, a);
        a = dot2(ca.w, x3, a);
        a = dot2(cbv.x, x0, a);
        a = dot2(cbv.y, x1, a);
        a = dot2(cbv.z, x2, a);
        a = dot2(cbv.w, x3, a);
        acc[G & 3] = a;
        strip_dot<G + 1>(d, cb, xp, acc);
    }
}

typedef __attribute__((address_space(1))) const u32x4 gu32x4;   // global memory

// Direct global -> LDS copies (global_load_lds_dwordx4): each lane moves 16
// bytes into LDS at the wave-uniform base + 16 * lane, without passing
// through registers, so a workgroup's whole staging is in flight at once.
// Wave v of WAVES moves 1 KB blocks v, v + WAVES, ...  The cache policy is
// kLdsPlain for record data (immutable during a launch) and kLdsCoherent
// (sc1, the policy of an agent-scope load) for data other workgroups of the
// same launch wrote.  The caller waits for vmcnt 0 and synchronises the
// workgroup before reading.
typedef __attribute__((address_space(1))) const void gvoid;
typedef __attribute__((address_space(3))) void lvoid;
constexpr int kLdsPlain = 0, kLdsCoherent = 16;
template <int AUX, int WAVES>
__device__ __forceinline__ void stage_lds_waves(char *dst, const void *src, int nbytes, int wave, int lane) {
    const int nblk = (nbytes + 1023) >> 10;
    for (int b = wave; b < nblk; b += WAVES) {
        const int off = (b << 10) + lane * 16;
        if (off < nbytes)
            __builtin_amdgcn_global_load_lds((gvoid *)((const char *)src + off), (lvoid *)(dst + (b << 10)), 16, 0, AUX);
    }
}

__device__ __forceinline__ void load_strip(const u32x4 *tile_generic, int lane, uint32_t (&d)[12]) {
    gu32x4 *tile = (gu32x4 *)tile_generic;      // codes live in global memory
    const u32x4 w0 = __builtin_nontemporal_load(tile + lane);
    const u32x4 w1 = __builtin_nontemporal_load(tile + 64 + lane);
    const u32x4 w2 = __builtin_nontemporal_load(tile + 128 + lane);
    d[0] = w0.x; d[1] = w0.y; d[2] = w0.z; d[3] = w0.w;
    d[4] = w1.x; d[5] = w1.y; d[6] = w1.z; d[7] = w1.w;
    d[8] = w2.x; d[9] = w2.y; d[10] = w2.z; d[11] = w2.w;
}

}  // namespace
}  // namespace moe
