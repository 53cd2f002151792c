// gemm_common.hpp -- pieces shared by the NVFP4 and MXFP4 GEMM kernels on gfx950: the XCD-aware
// tile order, an LDS-only workgroup barrier, and the epilogues that write the 32x32 MFMA
// accumulator tiles of a wave's 128 x 64 sub-tile to C.
#pragma once

#include "device_codecs.hpp"

namespace nvfp4 {

typedef float float16v __attribute__((ext_vector_type(16)));

// Workgroup barrier that orders LDS accesses only: outstanding global loads are not waited for.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Map workgroup ids so that the 8 XCDs (round-robin dispatch) each get a contiguous band of
// output tiles, and walk tiles in column groups of kGroupM row-tiles for L2 reuse.
__device__ __forceinline__ void tile_coords(uint32_t bid, uint32_t nbm, uint32_t nbn,
                                            uint32_t& bm, uint32_t& bn) {
    const uint32_t total = nbm * nbn;
    uint32_t id = bid;
    if ((total & 7u) == 0) id = (bid & 7u) * (total >> 3) + (bid >> 3);
    constexpr uint32_t kGroupM = 8;
    const uint32_t per_group = kGroupM * nbn;
    const uint32_t g = id / per_group;
    const uint32_t first_m = g * kGroupM;
    const uint32_t gm = (nbm - first_m) < kGroupM ? (nbm - first_m) : kGroupM;
    const uint32_t in = id - g * per_group;
    bm = first_m + in % gm;
    bn = in / gm;
}

// ---- epilogue --------------------------------------------------------------------------------
// bf16 output, transposed layout (kT): each wave stages its 128 x 64 sub-tile of C (times alpha,
// as bf16, 8 bytes per lane and r/4) in a private 16 KiB LDS region, then writes whole rows with
// 16 bytes per lane, 8 rows of 128 bytes per store instruction (instead of 2 rows of 64 bytes
// with 2 bytes per lane).  In the region a row's 16-byte chunks are permuted by (row / 2) % 8
// so that neither the staging writes nor the row reads conflict on LDS banks.  vec: C and its
// row stride are 16-byte aligned, else the staged values are stored one element at a time.
template <int TM, int TN>
__device__ __forceinline__ void epilogue_bf16(const float16v (&acc)[TM][TN], float alpha,
                                              uint8_t* reg, int lane, int64_t r0, int64_t c0,
                                              int M, int N, uint16_t* C, int64_t ldc, bool vec) {
    static_assert(TM * 32 == 128 && TN * 32 == 64, "wave sub-tile");
    const int lrow = lane & 31, h = lane >> 5;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int row = i * 32 + lrow, c = 4 * j + g, p = c ^ ((row >> 1) & 7);
                const float a0 = acc[i][j][4 * g] * alpha, a1 = acc[i][j][4 * g + 1] * alpha;
                const float a2 = acc[i][j][4 * g + 2] * alpha, a3 = acc[i][j][4 * g + 3] * alpha;
                *reinterpret_cast<uint2*>(reg + row * 128 + p * 16 + h * 8) =
                    make_uint2(f32_to_bf16(a0) | (f32_to_bf16(a1) << 16),
                               f32_to_bf16(a2) | (f32_to_bf16(a3) << 16));
            }
    __syncthreads();
#pragma unroll 4
    for (int pass = 0; pass < 16; ++pass) {
        const int row = pass * 8 + (lane >> 3), c = lane & 7, p = c ^ ((row >> 1) & 7);
        const uint4 v = *reinterpret_cast<const uint4*>(reg + row * 128 + p * 16);
        const int64_t gr = r0 + row, gc = c0 + c * 8;
        if (gr >= M || gc >= N) continue;
        uint16_t* dst = C + gr * ldc + gc;
        if (vec && gc + 8 <= N) {
            *reinterpret_cast<uint4*>(dst) = v;
        } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (gc + e < N) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
    }
}

// fp32 output, column-per-lane layout: for each r the 64 lanes store two rows of 32
// consecutive floats (128 bytes each), which measured faster than staging 32 KiB per wave.
template <int TM, int TN>
__device__ __forceinline__ void epilogue_f32(const float16v (&acc)[TM][TN], float alpha, int lane,
                                             int64_t r0, int64_t c0, int M, int N, float* C,
                                             int64_t ldc) {
    const int lrow = lane & 31, h = lane >> 5;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t col = c0 + j * 32 + lrow;
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = r0 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (row < M) C[row * ldc + col] = acc[i][j][r] * alpha;
            }
        }
}

// C = 0 when the inner dimension is empty (K == 0: every dot product is an empty sum).  Grid-
// stride over the M x N window of C, so any grid size covers it.
template <typename T>
__global__ void __launch_bounds__(256) k_zero_c(T* __restrict__ C, int64_t ldc, int M, int N) {
    const int64_t total = (int64_t)M * N;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256)
        C[(i / N) * ldc + i % N] = T(0);
}

inline void launch_zero_c(void* c, bool bf16, int64_t ldc, int M, int N, hipStream_t st) {
    const int64_t blocks = ((int64_t)M * N + 255) / 256;
    const dim3 grid((unsigned)(blocks < 65536 ? blocks : 65536)), block(256);
    if (bf16)
        hipLaunchKernelGGL(k_zero_c<uint16_t>, grid, block, 0, st, (uint16_t*)c, ldc, M, N);
    else
        hipLaunchKernelGGL(k_zero_c<float>, grid, block, 0, st, (float*)c, ldc, M, N);
}

}  // namespace nvfp4
