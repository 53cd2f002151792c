// noise.hpp -- the quantization-noise diagnostic shared by the 1D and the Hadamard quantizers
// [P2 "FP4 All the Way: Formacion totalmente cuantificada de LLM", Describir: quantized training
// loses efficiency once the gradient norm falls below about sqrt(3) times the quantization
// noise].  Per tensor: sum x^2 and sum (Q(x) - x)^2, with Q(x) = fl(fl(v * scale) * s_dec) the
// dequantized value and x the tensor that was encoded.
#pragma once

#include "device_codecs.hpp"

namespace nvfp4 {

// Values of eight packed E2M1 codes (element 2j in the low nibble of byte j); with a unit scale
// v_cvt_scalef32_pk_f32_fp4 returns the exact E2M1 values.
__device__ __forceinline__ void e2m1_decode8(uint32_t w, float* v) {
    const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
    v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
}

// One 16-element block's contributions: x holds the encoded values, (lo, hi) their codes and sb
// their scale byte.  The squares are taken of the values times s_enc = 2688 / amax (at most
// 5376 in magnitude, so no fp32 overflow or early underflow) and summed in fp32 over the block;
// blocks are accumulated in fp64.
__device__ __forceinline__ void block_noise(const float* x, uint32_t lo, uint32_t hi,
                                            uint32_t sb, const TensorScales& ts, double& g2,
                                            double& e2) {
    const float sc = e4m3_decode(sb);
    float v[16];
    e2m1_decode8(lo, v);
    e2m1_decode8(hi, v + 8);
    float bg = 0.0f, be = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const float d = (v[e] * sc) * ts.s_dec - x[e];
        const float ys = x[e] * ts.s_enc, ds = d * ts.s_enc;   // |.| <= 5376
        bg += ys * ys;
        be += ds * ds;
    }
    g2 += (double)bg;
    e2 += (double)be;
}

// Workgroup-wide totals of the per-thread sums, divided by s_enc^2, added to sums[0..1] with one
// pair of device atomics per workgroup.  Every thread of the workgroup must call it.
template <int kWgThreads>
__device__ __forceinline__ void publish_noise(double g2, double e2, const TensorScales& ts,
                                              double* sums) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        g2 += __shfl_xor(g2, off);
        e2 += __shfl_xor(e2, off);
    }
    __shared__ double part[2][kWgThreads / 64];
    if ((threadIdx.x & 63) == 0) {
        part[0][threadIdx.x >> 6] = g2;
        part[1][threadIdx.x >> 6] = e2;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double a = 0.0, c = 0.0;
#pragma unroll
        for (int w = 0; w < kWgThreads / 64; ++w) {
            a += part[0][w];
            c += part[1][w];
        }
        const double inv = 1.0 / ((double)ts.s_enc * (double)ts.s_enc);
        atomicAdd(sums, a * inv);
        atomicAdd(sums + 1, c * inv);
    }
}

}  // namespace nvfp4
