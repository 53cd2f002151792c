// device_codecs.hpp -- gfx950 device-side number formats and random numbers for the NVFP4 path.
//
// Citation keys: [P1] "Entrenamiento de Modelos de Lenguaje con 4 Bits de Precision";
// [P2] "FP4 All the Way: Formacion totalmente cuantificada de LLM"; [P3] "I ricercatori di
// Nvidia sbloccano il tutorial LLM a 8 bit che corrisponde alle prestazioni a 4 bit".
//
// Every routine here is written for single fp32 operations in IEEE round-to-nearest-even; the
// library is compiled with -ffp-contract=off so no multiply is fused into an add.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// ---- tensor-level scales [P3 Come funziona NVFP4?: multi-level scaling] ----------------------
// The per-tensor level maps the tensor amax A onto 6 * 448 = 2688, the largest product of an
// E2M1 element and an E4M3 scale.  A below 2^-100 (zero included) is treated as zero.
struct TensorScales {
    float k1;      // 448 / A: block amax -> E4M3 target
    float s_enc;   // 2688 / A
    float s_dec;   // A / 2688, the stored decode scale
};

__device__ __forceinline__ TensorScales tensor_scales(float A) {
    TensorScales t;
    if (!(A >= 0x1p-100f)) {
        t.k1 = 448.0f; t.s_enc = 1.0f; t.s_dec = 1.0f;
    } else {
        t.k1 = 448.0f / A;
        t.s_enc = 2688.0f / A;
        t.s_dec = A / 2688.0f;
    }
    return t;
}

// ---- E4M3 (OCP E4M3FN), non-negative operands -----------------------------------------------
// Round to nearest even with saturation at 448 (0x7E); values below 2^-6 use the subnormal
// quantum 2^-9.
__device__ __forceinline__ uint32_t e4m3_encode(float t) {
    if (t >= 448.0f) return 0x7Eu;
    if (t < 0x1p-6f) return (uint32_t)__builtin_rintf(t * 512.0f);
    uint32_t b = __float_as_uint(t);
    b += 0x7FFFFu + ((b >> 20) & 1u);          // round the mantissa to 3 bits, ties to even
    uint32_t r = (b >> 20) - 960u;             // re-bias the exponent from 127 to 7
    return r < 0x7Eu ? r : 0x7Eu;
}

__device__ __forceinline__ float e4m3_decode(uint32_t b) {
    uint32_t e = b >> 3;
    return e == 0 ? (float)(b & 7u) * 0x1p-9f : __uint_as_float((b + 960u) << 20);
}

// Block step: scale byte and the element encode factor s_enc / scale (0 for a zero scale).
__device__ __forceinline__ void block_scale(float amax_b, const TensorScales& ts,
                                            uint32_t& scale_byte, float& enc) {
    float t = amax_b * ts.k1;
    scale_byte = e4m3_encode(t);
    enc = scale_byte == 0 ? 0.0f : ts.s_enc / e4m3_decode(scale_byte);
}

// ---- E2M1 [P1 Caracteristicas: 1 sign, 2 exponent, 1 mantissa bit] --------------------------
// Magnitude index from a grid value held as 2*r in {0,1,2,3,4,6,8,12}: n<=4 -> n, 6->5, 8->6,
// 12->7, i.e. min(n, n/4 + 4).
__device__ __forceinline__ uint32_t e2m1_index_from_twice(uint32_t n) {
    uint32_t q = (n >> 2) + 4u;
    return n < q ? n : q;
}

// Round-to-nearest-even of z2 = 2*z onto the doubled grid {0,1,2,3,4,6,8,12} (saturating),
// returning the 4-bit code of z (sign kept, so -0 and small negatives give 0x8).
// The quantum of the doubled grid is 1 below 4, 2 in [4,8) and 4 in [8,12]; adding and
// removing 2^(E+22) with E = max(exponent(z2), 1) rounds at exactly that quantum.
__device__ __forceinline__ uint32_t e2m1_rne_code2(float z2) {
    uint32_t sign = (__float_as_uint(z2) >> 28) & 8u;
    float a = __builtin_fminf(__builtin_fabsf(z2), 12.0f);
    uint32_t e = __float_as_uint(a) & 0x7F800000u;
    e = e > 0x40000000u ? e : 0x40000000u;
    float C = __uint_as_float(e + (22u << 23));
    float r = (a + C) - C;
    return sign | e2m1_index_from_twice((uint32_t)r);
}

// Stochastic rounding of z2 = 2*z [P2 Describir: stochastic rounding in the backward pass]
// (callers form z2 as z + z from the rounded product z, so the doubling is exact even for
// subnormal z):
// with lo <= |z| < hi the neighbouring grid values, round up iff r16 < 65536 * (|z|-lo)/(hi-lo).
// In the doubled grid the neighbours of a2 = |z2| are lo2 = a2 truncated to its quantum q
// (q = 1 below 4, else the exponent's power / 2), hi2 = lo2 + q, and the comparison
// r16 < (a2 - lo2) * 65536 / q is exact in fp32.  |z| >= 6 saturates without randomness.
__device__ __forceinline__ uint32_t e2m1_sr_code2(float z2, uint32_t r16) {
    uint32_t sign = (__float_as_uint(z2) >> 28) & 8u;
    float a = __builtin_fabsf(z2);
    uint32_t idx;
    if (a >= 12.0f) {
        idx = 7u;
    } else {
        uint32_t ab = __float_as_uint(a);
        // quantum q: 1 for a < 4, else 2^(E-1) for a in [2^E, 2^(E+1))
        float q = a < 4.0f ? 1.0f : __uint_as_float((ab & 0x7F800000u) - (1u << 23));
        float lo = a < 4.0f ? __builtin_floorf(a) : __uint_as_float(ab & 0xFFC00000u);
        float frac = (a - lo) * (65536.0f / q);          // exact: q is a power of two
        float r = ((float)r16 < frac) ? lo + q : lo;
        idx = e2m1_index_from_twice((uint32_t)r);
    }
    return sign | idx;
}

// ---- Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) --------------------------------------
struct u32x4 { uint32_t x, y, z, w; };

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        if (i) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        uint32_t lo0 = 0xD2511F53u * c0, hi0 = __umulhi(0xD2511F53u, c0);
        uint32_t lo1 = 0xCD9E8D57u * c2, hi1 = __umulhi(0xCD9E8D57u, c2);
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    }
    return {c0, c1, c2, c3};
}

// The eight 16-bit uniforms of the SR counter j = idx / 8 (idx a multiple of 8).
__device__ __forceinline__ u32x4 sr_words(uint64_t seed, uint64_t idx8) {
    uint64_t j = idx8 >> 3;
    return philox4x32_10((uint32_t)j, (uint32_t)(j >> 32), 0u, 0u, (uint32_t)seed,
                         (uint32_t)(seed >> 32));
}

// ---- loads ----------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// DPP swap of adjacent lanes (quad_perm [1,0,3,2]).
__device__ __forceinline__ float swap_adjacent(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}

}  // namespace nvfp4
