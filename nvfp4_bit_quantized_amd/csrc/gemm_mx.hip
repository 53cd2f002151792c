// gemm_mx.hip -- MXFP4 x MXFP4 GEMM on gfx950's block-scaled FP4 MFMA.
//
// The comparison format of [P3] "I ricercatori di Nvidia sbloccano il tutorial LLM a 8 bit che
// corrisponde alle prestazioni a 4 bit", NVFP4 in pratica (MXFP4 needed more training data to
// match NVFP4).  MXFP4 scales are powers of two per 32 elements, which is exactly what
// v_mfma_scale_f32_32x32x64_f8f6f4 applies in hardware, so packed codes go to the matrix core
// without any unpacking:
//   C[m,n] = sum_kb 2^(eA[m,kb] + eB[n,kb]) * sum_{k in kb} vA[m,k] * vB[n,k].
// One MFMA covers K = 64: lane l supplies row l%32 and the 32-element block (l/32) of the
// 64, i.e. 16 bytes of codes plus that block's E8M0 byte.

#include "device_codecs.hpp"
#include "host_util.hpp"

namespace nvfp4 {

typedef int int8v __attribute__((ext_vector_type(8)));
typedef float float16v_mx __attribute__((ext_vector_type(16)));

constexpr int kMxBK = 128;               // K elements per pipeline step (two MFMAs)
constexpr int kMxRowBytes = kMxBK / 2;   // 64 packed bytes per row per step
constexpr int kFmtFp4 = 4;               // f8f6f4 operand format code for E2M1

__device__ __forceinline__ void mx_tile_coords(uint32_t bid, uint32_t nbm, uint32_t nbn,
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

// Stage of ROWS rows: 64 code bytes (four 16-byte chunks) and 4 E8M0 bytes per row.
template <int ROWS, int NT>
struct MxStage {
    static constexpr int kChunks = ROWS * 4;
    static constexpr int kPerThread = (kChunks + NT - 1) / NT;
    uint4 c[kPerThread];
    uint32_t s;

    // K % 128 == 0: rows past the edge clamped to the last row (their results are never stored),
    // k0 past the end clamped to the last step by the caller, so no load is conditional and the
    // compiler's wait counts stay exact.
    __device__ __forceinline__ void load_fast(const uint8_t* codes, const uint8_t* scales,
                                              int64_t rows, int64_t row0, int k0, int K, int tid) {
        static_assert(kChunks % NT == 0 && ROWS <= NT, "fast loader shape");
        const int64_t rb = K / 2, nkb = K / 32;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int ch = tid + i * NT;
            const int r = ch >> 2, q = ch & 3;
            int64_t row = row0 + r;
            row = row < rows - 1 ? row : rows - 1;
            c[i] = *reinterpret_cast<const uint4*>(codes + row * rb + k0 / 2 + q * 16);
        }
        int64_t row = row0 + (tid < ROWS ? tid : 0);
        row = row < rows - 1 ? row : rows - 1;
        s = *reinterpret_cast<const uint32_t*>(scales + row * nkb + k0 / 32);
    }

    __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                         int64_t row0, int k0, int K, int tid) {
        const int64_t rb = K / 2, nkb = K / 32;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int ch = tid + i * NT;
            c[i] = make_uint4(0, 0, 0, 0);
            if (ch < kChunks) {
                const int r = ch >> 2, q = ch & 3;
                const int64_t row = row0 + r;
                const int kk = k0 + q * 32;
                if (row < rows && kk < K) c[i] = *reinterpret_cast<const uint4*>(codes + row * rb + kk / 2);
            }
        }
        s = 0x7F7F7F7Fu;                                          // 2^0 for padding blocks
        if (tid < ROWS) {
            const int64_t row = row0 + tid;
            if (row < rows) {
                const int kb0 = k0 / 32;
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    if (kb0 + b < nkb) s = (s & ~(0xFFu << (8 * b))) | ((uint32_t)scales[row * nkb + kb0 + b] << (8 * b));
            }
        }
    }

    // codes [ROWS][64 B] with the 16-byte chunk index rotated by row % 4, then scales [ROWS].
    __device__ __forceinline__ void store(uint8_t* lc, uint32_t* ls, int tid) const {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int ch = tid + i * NT;
            if (ch < kChunks) {
                const int r = ch >> 2, q = ((ch & 3) + r) & 3;
                *reinterpret_cast<uint4*>(lc + r * kMxRowBytes + q * 16) = c[i];
            }
        }
        if (tid < ROWS) ls[tid] = s;
    }
};

template <int WM, int WN, int TM, int TN, bool kBF16Out, bool kFast>
__global__ void __launch_bounds__(WM * WN * 64)
k_gemm_mxfp4(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
             const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales,
             int M, int N, int K, void* __restrict__ C, int64_t ldc) {
    constexpr int NT = WM * WN * 64, BM = WM * TM * 32, BN = WN * TN * 32;
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * kMxRowBytes];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][BN * kMxRowBytes];
    __shared__ uint32_t lds_sa[2][BM];
    __shared__ uint32_t lds_sb[2][BN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const uint32_t nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
    uint32_t bm, bn;
    mx_tile_coords(blockIdx.x, nbm, nbn, bm, bn);
    const int64_t m0 = (int64_t)bm * BM, n0 = (int64_t)bn * BN;

    float16v_mx acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    MxStage<BM, NT> sa;
    MxStage<BN, NT> sb;
    const int nk = (K + kMxBK - 1) / kMxBK;
    if constexpr (kFast) {
        sa.load_fast(a_codes, a_scales, M, m0, 0, K, tid);
        sb.load_fast(b_codes, b_scales, N, n0, 0, K, tid);
    } else {
        sa.load(a_codes, a_scales, M, m0, 0, K, tid);
        sb.load(b_codes, b_scales, N, n0, 0, K, tid);
    }
    sa.store(lds_a[0], lds_sa[0], tid);
    sb.store(lds_b[0], lds_sb[0], tid);
    __syncthreads();

    const int lrow = lane & 31, h = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if constexpr (kFast) {
            const int kn = (kt + 1 < nk ? kt + 1 : kt) * kMxBK;
            sa.load_fast(a_codes, a_scales, M, m0, kn, K, tid);
            sb.load_fast(b_codes, b_scales, N, n0, kn, K, tid);
        } else if (kt + 1 < nk) {
            sa.load(a_codes, a_scales, M, m0, (kt + 1) * kMxBK, K, tid);
            sb.load(b_codes, b_scales, N, n0, (kt + 1) * kMxBK, K, tid);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int q = 2 * s + h;                      // 32-element block of this lane
            int8v va[TM], vb[TN];
            uint32_t ea[TM], eb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * TM * 32 + i * 32 + lrow;
                const uint4 v = *reinterpret_cast<const uint4*>(&lds_a[cur][r * kMxRowBytes + ((q + r) & 3) * 16]);
                va[i] = int8v{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
                ea[i] = (lds_sa[cur][r] >> (8 * q)) & 0xFFu;
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn * TN * 32 + j * 32 + lrow;
                const uint4 v = *reinterpret_cast<const uint4*>(&lds_b[cur][r * kMxRowBytes + ((q + r) & 3) * 16]);
                vb[j] = int8v{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
                eb[j] = (lds_sb[cur][r] >> (8 * q)) & 0xFFu;
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        va[i], vb[j], acc[i][j], kFmtFp4, kFmtFp4, 0, (int)ea[i], 0, (int)eb[j]);
        }
        if (kFast || kt + 1 < nk) {
            sa.store(lds_a[cur ^ 1], lds_sa[cur ^ 1], tid);
            sb.store(lds_b[cur ^ 1], lds_sb[cur ^ 1], tid);
        }
        if constexpr (kFast) {
            // orders LDS only: the loads were all consumed by the stores above
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
        } else {
            __syncthreads();
        }
    }

#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t col = n0 + wn * TN * 32 + j * 32 + lrow;
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * TM * 32 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (row < M) {
                    const float v = acc[i][j][r];
                    if constexpr (kBF16Out)
                        reinterpret_cast<uint16_t*>(C)[row * ldc + col] = (uint16_t)f32_to_bf16(v);
                    else
                        reinterpret_cast<float*>(C)[row * ldc + col] = v;
                }
            }
        }
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" nvfp4_status mxfp4_gemm(const nvfp4_tensor* a, const nvfp4_tensor* b, void* c,
                                   nvfp4_dtype c_dt, int64_t ldc, void* stream) {
    nvfp4_status s = check_q(a, MXFP4_BLK_1x32, false);
    if (s) return s;
    s = check_q(b, MXFP4_BLK_1x32, false);
    if (s) return s;
    if (a->cols != b->cols) return NVFP4_ERR_SHAPE;
    s = check_output(c, c_dt, a->rows, b->rows, ldc);
    if (s) return s;
    const int64_t M = a->rows, N = b->rows, K = a->cols;
    if (M >= (1ll << 31) || N >= (1ll << 31) || K >= (1ll << 31)) return NVFP4_ERR_SHAPE;
    if (((M + 255) / 256) * ((N + 255) / 256) >= (1ll << 31)) return NVFP4_ERR_SHAPE;   // grid
    if (M == 0 || N == 0) return NVFP4_OK;
    constexpr int WM = 2, WN = 2, TM = 4, TN = 4;
    constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
    const uint32_t nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
    const dim3 grid(nbm * nbn), block(WM * WN * 64);
    hipStream_t st = as_stream(stream);
    const bool fast = K % kMxBK == 0;
#define NVFP4_MX(BF, FAST)                                                                        \
    hipLaunchKernelGGL((k_gemm_mxfp4<WM, WN, TM, TN, BF, FAST>), grid, block, 0, st, a->codes,     \
                       a->scales, b->codes, b->scales, (int)M, (int)N, (int)K, c, ldc)
    if (c_dt == NVFP4_BF16) {
        if (fast) NVFP4_MX(true, true); else NVFP4_MX(true, false);
    } else {
        if (fast) NVFP4_MX(false, true); else NVFP4_MX(false, false);
    }
#undef NVFP4_MX
    return launch_status();
}
