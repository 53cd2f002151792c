// gemm_common.hpp -- pieces shared by the NVFP4 and MXFP4 GEMM kernels on gfx950: the XCD-aware
// tile order, an LDS-only workgroup barrier, and the epilogues that write the 32x32 MFMA
// accumulator tiles of a wave's 128 x 64 sub-tile to C.
#pragma once

#include "device_codecs.hpp"
#include "host_util.hpp"

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

// ---- split last round ------------------------------------------------------------------------
constexpr int kGemmTile = 256;      // output tile of both GEMM kernels (BM = BN)

// One wave's accumulators, unscaled, into a dense fp32 256 x 256 partial tile P (row stride 256),
// at the wave's offset (r0, c0) inside the tile.  Both accumulator layouts (see mfma_frags).
template <int TM, int TN, bool kT>
__device__ __forceinline__ void store_partial(const float16v (&acc)[TM][TN], int lane, int r0,
                                              int c0, float* __restrict__ P) {
    const int lrow = lane & 31, h = lane >> 5;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            if constexpr (kT) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int row = r0 + i * 32 + lrow, col = c0 + j * 32 + 8 * g + 4 * h;
                    *reinterpret_cast<float4*>(P + row * kGemmTile + col) =
                        make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                    acc[i][j][4 * g + 3]);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = r0 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                    P[row * kGemmTile + j * 32 + c0 + lrow] = acc[i][j][r];
                }
            }
        }
}

// The tiles split along K: C = alpha * (P_0 + P_1 + ... + P_{splits-1}), the partials added in
// split order (so the result does not depend on which workgroup finished first), alpha = s_dA *
// s_dB (1 when sdA is null: MXFP4 has no tensor scales).  One workgroup of 256 threads per 8 rows
// of a tile, 8 consecutive columns per thread.
template <bool kBF16Out>
__global__ void __launch_bounds__(256)
k_splitk_fixup(const float* __restrict__ ws, uint32_t full, uint32_t splits, int M, int N,
               const float* __restrict__ sdA, const float* __restrict__ sdB, void* __restrict__ C,
               int64_t ldc) {
    constexpr int kRowsPerBlock = 8;
    const uint32_t t_local = blockIdx.x / (kGemmTile / kRowsPerBlock);
    const int row = (blockIdx.x % (kGemmTile / kRowsPerBlock)) * kRowsPerBlock + (threadIdx.x >> 5);
    const int col = (threadIdx.x & 31) * 8;
    const uint32_t nbm = (M + kGemmTile - 1) / kGemmTile, nbn = (N + kGemmTile - 1) / kGemmTile;
    uint32_t bm, bn;
    tile_coords(full + t_local, nbm, nbn, bm, bn);
    const float* p = ws + (size_t)t_local * splits * (kGemmTile * kGemmTile) + row * kGemmTile + col;
    float4 lo = *reinterpret_cast<const float4*>(p), hi = *reinterpret_cast<const float4*>(p + 4);
    for (uint32_t j = 1; j < splits; ++j) {
        const float4 a = *reinterpret_cast<const float4*>(p + (size_t)j * (kGemmTile * kGemmTile));
        const float4 b = *reinterpret_cast<const float4*>(p + (size_t)j * (kGemmTile * kGemmTile) + 4);
        lo.x += a.x; lo.y += a.y; lo.z += a.z; lo.w += a.w;
        hi.x += b.x; hi.y += b.y; hi.z += b.z; hi.w += b.w;
    }
    const float alpha = sdA ? (*sdA) * (*sdB) : 1.0f;
    const float v[8] = {lo.x * alpha, lo.y * alpha, lo.z * alpha, lo.w * alpha,
                        hi.x * alpha, hi.y * alpha, hi.z * alpha, hi.w * alpha};
    const int64_t gr = (int64_t)bm * kGemmTile + row, gc = (int64_t)bn * kGemmTile + col;
    if (gr >= M) return;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if (gc + e >= N) break;
        if constexpr (kBF16Out)
            reinterpret_cast<uint16_t*>(C)[gr * ldc + gc + e] = (uint16_t)f32_to_bf16(v[e]);
        else
            reinterpret_cast<float*>(C)[gr * ldc + gc + e] = v[e];
    }
}

// Split plan: the whole tiles of full rounds of the device's compute units run unsplit; when
// the last round is at most half full its tiles are split along K into `splits` parts (at most
// 8, each at least min_steps K steps of `step` elements), so that the round's units fill the
// device.
struct SplitPlan {
    uint32_t full, tail, splits;
    size_t ws_bytes;
};

constexpr uint32_t kMaxSplits = 8;

inline SplitPlan plan_split(int64_t M, int64_t N, int64_t K, int cus, int step, int min_steps) {
    const uint32_t tiles = (uint32_t)(((M + kGemmTile - 1) / kGemmTile) * ((N + kGemmTile - 1) / kGemmTile));
    SplitPlan p{tiles, 0, 1, 0};
    if (cus <= 0 || K % step != 0) return p;
    const uint32_t tail = tiles % (uint32_t)cus;
    if (tail == 0) return p;
    uint32_t s = (uint32_t)cus / tail;
    s = s < kMaxSplits ? s : kMaxSplits;
    const int64_t nk = K / step;
    while (s > 1 && nk / s < min_steps) --s;
    if (s < 2) return p;
    p.full = tiles - tail;
    p.tail = tail;
    p.splits = s;
    p.ws_bytes = (size_t)tail * s * kGemmTile * kGemmTile * sizeof(float);
    return p;
}

inline int device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}

// The fixup of a split plan's last round (nothing when the plan has no split tiles).
inline void launch_splitk_fixup(const SplitPlan& plan, const float* ws, int M, int N,
                                const float* sdA, const float* sdB, void* c, bool bf16,
                                int64_t ldc, hipStream_t st) {
    if (!plan.tail) return;
    const dim3 grid(plan.tail * (kGemmTile / 8)), block(256);
    if (bf16)
        hipLaunchKernelGGL(k_splitk_fixup<true>, grid, block, 0, st, ws, plan.full, plan.splits, M,
                           N, sdA, sdB, c, ldc);
    else
        hipLaunchKernelGGL(k_splitk_fixup<false>, grid, block, 0, st, ws, plan.full, plan.splits, M,
                           N, sdA, sdB, c, ldc);
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
