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

// Publish a workgroup's partial amax m >= 0 into the device-wide maximum *dst (which the caller
// zeroed before the launch).  Non-negative floats order like their bit patterns, so an unsigned
// atomic max applies; a workgroup whose value cannot raise the current maximum skips the atomic,
// so that few of the same-address atomics serialize in L2.  A stale read only costs an atomic.
__device__ __forceinline__ void publish_amax(float* dst, float m) {
    unsigned int* p = reinterpret_cast<unsigned int*>(dst);
    const unsigned int v = __float_as_uint(m);
    if (v > __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
        __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- E4M3 (OCP E4M3FN), non-negative operands -----------------------------------------------
// Round to nearest even with saturation at 448 (0x7E), subnormals (quantum 2^-9) included.
// gfx950's v_cvt_pk_fp8_f32 rounds fp32 to OCP E4M3 to nearest even with E4M3 subnormals; the
// clamp to 448 first supplies the saturation (it would give NaN above 464).  Checked bit for bit
// against a software encoder (the nearest of the 127 values, ties to even) for every fp32 bit
// pattern in [0, 448] and, clamped, up to 2^20.
__device__ __forceinline__ uint32_t e4m3_encode(float t) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(t, 448.0f), 0.0f, 0, false) & 0xFFu;
}

// v_cvt_f32_fp8: exact for every E4M3 byte (all 127 non-negative finite bytes checked).
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
    return __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
}

// Block step: scale byte and the element encode factor s_enc / scale (0 for a zero scale).
// The division is a single correctly rounded fp32 division.
__device__ __forceinline__ void block_scale(float amax_b, const TensorScales& ts,
                                            uint32_t& scale_byte, float& enc) {
    const float t = amax_b * ts.k1;
    scale_byte = e4m3_encode(t);
    const float d = scale_byte == 0 ? 1.0f : e4m3_decode(scale_byte);
    const float e = ts.s_enc / d;
    enc = scale_byte == 0 ? 0.0f : e;
}

// The encode factors of one tensor for every scale byte, enc[b] = fl(s_enc / dec(b)) (0 for
// b = 0; byte 0x7F is never produced), filled once per workgroup so that a block looks up its
// factor instead of dividing: the same single correctly rounded division, done 127 times per
// workgroup instead of once per block.
struct EncTable {
    float v[128];
};

// Every thread of the workgroup must call this (it ends with a barrier).
__device__ __forceinline__ void fill_enc_table(EncTable& t, const TensorScales& ts) {
    for (uint32_t b = threadIdx.x; b < 128; b += blockDim.x) {
        const bool zero = b == 0 || b == 127;
        const float e = ts.s_enc / (zero ? 1.0f : e4m3_decode(b));
        t.v[b] = zero ? 0.0f : e;
    }
    __syncthreads();
}

// block_scale with the factor from the workgroup's table (bit-identical).
__device__ __forceinline__ void block_scale_tab(float amax_b, const TensorScales& ts,
                                                const EncTable& t, uint32_t& scale_byte,
                                                float& enc) {
    scale_byte = e4m3_encode(amax_b * ts.k1);
    enc = t.v[scale_byte];
}

// ---- E2M1 [P1 Caracteristicas: 1 sign, 2 exponent, 1 mantissa bit] --------------------------

// Eight E2M1 codes of z[0..7] rounded to nearest even (ties to the even code, saturating at 6,
// sign kept), packed element 2j -> low nibble of byte j.  gfx950's v_cvt_scalef32_pk_fp4_f32
// with a unit scale performs exactly this rounding for every finite fp32 input.
__device__ __forceinline__ uint32_t e2m1_rne_pack8(const float* z) {
    // each conversion writes one byte of w and keeps the other three, so the four together
    // overwrite all of it: w's starting value is never seen.  Starting from z[0]'s bits lets the
    // first conversion write over z[0]'s register, where an unset start would cost a move.
    uint32_t w = __float_as_uint(z[0]);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, z[0], z[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, z[2], z[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, z[4], z[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, z[6], z[7], 1.0f, 3);
    return w;
}

// Stochastic rounding of one element [P2 Describir: stochastic rounding in the backward pass]:
// with lo <= |z| < hi the neighbouring grid values, round up iff r16 < 65536 (|z|-lo)/(hi-lo);
// |z| >= 6 saturates; sign kept.  Below 8 the E2M1 grid is uniform within three regions: spacing
// h = 1/2 on [0, 2), 1 on [2, 4) and 2 on [4, 8), i.e. h = 2^(k-2) with k the binary exponent of
// |z| (frexp convention) clamped to [1, 3].  With y = |z| / h (exact) and u = r16 / 65536,
// ceil(y - u) = floor(y) + [fract(y) > u], which is the rounded value divided by h.  One fma
// forms y - u: it is exact whenever y >= 1 (y and u lie on a common grid fine enough for 24
// bits), and for y < 1 its single rounding cannot move the value across 0 or below u - 1, so the
// ceiling is unchanged (checked against the definition on 2.2e8 cases, every boundary included).
// The result h * ceil(y - u) lies on the E2M1 grid, or is 8 when |z| >= 6 rounds up, which the
// round-to-nearest encode then saturates to 6.  A ceiling of -0 takes z's sign like any zero.
__device__ __forceinline__ float e2m1_sr_value(float z, uint32_t r16) {
    const float a = __builtin_fabsf(z);
    const int e = __builtin_amdgcn_frexp_expf(a);            // a = m 2^e, m in [0.5, 1)
    const int k = e < 1 ? 1 : (e > 3 ? 3 : e);
    const float y = __builtin_amdgcn_ldexpf(a, 2 - k);
    const float q = __builtin_ceilf(__builtin_fmaf((float)r16, -0x1p-16f, y));
    return __builtin_copysignf(__builtin_amdgcn_ldexpf(q, k - 2), z);
}

// Eight stochastically rounded codes of z[0..7]: element e takes the 16-bit half (e & 1) of
// w[e >> 1] (low half first); packed element 2j -> low nibble of byte j.
__device__ __forceinline__ uint32_t e2m1_sr_pack8(const float* z, const uint32_t* w) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t r16 = (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu);
        v[e] = e2m1_sr_value(z[e], r16);
    }
    return e2m1_rne_pack8(v);    // exact: every v is a grid value (or >= 8, saturated)
}

// ---- Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) --------------------------------------
struct u32x4 { uint32_t x, y, z, w; };

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        if (i) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
        const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
        // three-input xors in one v_bitop3_b32 each (0x96: odd parity of the three inputs)
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32(hi1, c1, k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32(hi0, c3, k1, 0x96);
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
// 16-byte load.  kNT: with the nontemporal hint, for an input read for the last time -- the
// lines are not kept in the caches for later readers (measured on 16384 x 20480 bf16 tensors:
// the dual quantizers 6-8% faster).  A pass whose input is read again next (an amax pass ahead of
// its quantizer) loads normally when the tensor fits the 256 MB last-level cache.
template <bool kNT>
__device__ __forceinline__ uint4 load16(const void* p) {
    if constexpr (kNT) {
        typedef unsigned int u32v4 __attribute__((ext_vector_type(4)));
        const u32v4 v = __builtin_nontemporal_load(reinterpret_cast<const u32v4*>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    } else {
        return *reinterpret_cast<const uint4*>(p);
    }
}

// Tensors of at least this many bytes do not fit the last-level cache: their amax pass streams.
constexpr int64_t kStreamBytes = 256ll << 20;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// DPP swap of adjacent lanes (quad_perm [1,0,3,2]).  Every caller has both lanes of a pair
// active, so no lane reads a disabled one; bound_ctrl lets the compiler fold the move into the
// instruction that consumes it (v_max_f32 with a DPP source).
__device__ __forceinline__ float swap_adjacent(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}

// DPP swap of lane pairs within a quad (quad_perm [2,3,0,1]); the same conditions, for all four
// lanes of a quad.
__device__ __forceinline__ float swap_pairs(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}

}  // namespace nvfp4
