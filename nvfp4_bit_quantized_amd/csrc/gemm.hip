// gemm.hip -- NVFP4 x NVFP4 GEMM with fp32 accumulation on gfx950 MFMA.
//
// [P2] "FP4 All the Way: Formacion totalmente cuantificada de LLM", Describir: weights,
// activations and gradients are all FP4, so the three training GEMMs (fprop, dgrad, wgrad) all
// take two NVFP4 operands.
//
// C[m,n] = s_dA * s_dB * sum_k (vA[m,k] * sA[m,k/16]) * (vB[n,k] * sB[n,k/16])
//
// gfx950's block-scaled FP4 MFMA scales by powers of two per 32 elements, which cannot express
// an E4M3 scale per 16.  Here each product v * s (an E2M1 value times an E4M3 scale) is formed
// exactly in fp16 -- it needs at most 6 significant bits and lies in [2^-10, 2688] -- and fed
// to v_mfma_f32_32x32x16_f16, which accumulates in fp32.  The per-tensor decode scales are
// applied once in the epilogue.
//
// Data flow per workgroup (BM x BN output tile, K in steps of 64):
//   global -> VGPR prefetch of packed codes (32 B per row per step) and scale bytes
//   -> LDS (double buffered, half-swapped rows to spread LDS banks)
//   -> each wave reads 16 B (32 codes) per 32-row MFMA tile and lane, unpacks 8 codes at a time
//      with v_cvt_scalef32_pk_f16_fp4 and multiplies by its block scale (packed fp16)
//   -> MFMA 32x32x16.
// K is permuted inside a step identically for both operands: MFMA k-slot (8h + j) of sub-step
// s reads element 32h + 8s + j of the 64-element step, so a lane's 16 bytes cover two whole
// NVFP4 blocks and one scale serves each sub-step.

#include "device_codecs.hpp"
#include "host_util.hpp"

#include <type_traits>

namespace nvfp4 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;            // K elements per pipeline step
constexpr int kRowBytes = kBK / 2; // packed bytes per row per step

// 8 E2M1 codes (one dword, element 2j in the low nibble of byte j) times a scale -> 8 fp16.
__device__ __forceinline__ half8 unpack8(uint32_t w, half2v s2) {
    half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
    half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
    half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
    half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
    half8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

struct OperandDesc {
    const uint8_t* codes;   // [rows x K/2]
    const uint8_t* scales;  // 1x16: [rows x K/16]; 16x16: [rows/16 x K/16]
    int64_t rows;
    int tiled;              // 1 for 16x16 scales
};

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

template <int WM, int WN, int TM, int TN>
struct GemmCfg {
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = kWaves * 64;
    static constexpr int BM = WM * TM * 32;
    static constexpr int BN = WN * TN * 32;
};

// E4M3 scale byte -> fp16 bits, duplicated into both halves of a dword (exact conversion).
__device__ __forceinline__ uint32_t scale_splat(uint32_t b) {
    const _Float16 h = (_Float16)e4m3_decode(b);
    const uint32_t u = (uint32_t)__builtin_bit_cast(uint16_t, h);
    return u | (u << 16);
}

// LDS image of one operand tile for one K step:
//   codes  [ROWS][32 B]: the two 16-byte halves of a row swapped on rows with bit 2 set, which
//          spreads the 16-byte lane reads of eight consecutive rows over all banks;
//   scales [ROWS][4 dwords]: the four block scales of the step as fp16 pairs (s, s).
template <int ROWS>
struct LdsTile {
    uint8_t codes[ROWS * kRowBytes];
    uint4 scales[ROWS];
};

template <int ROWS, int NT>
__device__ __forceinline__ void store_stage(LdsTile<ROWS>& t, const uint4* c, uint32_t s, int tid) {
    constexpr int kPer = (ROWS * 2 + NT - 1) / NT;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int ch = tid + i * NT;
        if (ch < ROWS * 2) {
            const int r = ch >> 1, h = (ch & 1) ^ ((r >> 2) & 1);
            *reinterpret_cast<uint4*>(t.codes + r * kRowBytes + h * 16) = c[i];
        }
    }
    if (tid < ROWS)
        t.scales[tid] = make_uint4(scale_splat(s & 0xFFu), scale_splat((s >> 8) & 0xFFu),
                                   scale_splat((s >> 16) & 0xFFu), scale_splat(s >> 24));
}

// Global loads of one operand for K % 64 == 0: every thread keeps its own row pointers (rows
// past the end are clamped to the last row; their results are never stored) and advances them
// by one step (32 code bytes, 4 scale bytes) per load, so the loop has no branches and no
// 64-bit multiplies.
template <int ROWS, int NT>
struct FastLoader {
    static constexpr int kPer = (ROWS * 2 + NT - 1) / NT;
    const uint8_t* pc[kPer];
    const uint8_t* ps;
    uint4 c[kPer];
    uint32_t s;

    __device__ __forceinline__ void init(const OperandDesc& op, int64_t row0, int K, int tid) {
        const int64_t last = op.rows - 1;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int ch = (tid + i * NT) % (ROWS * 2);
            int64_t row = row0 + (ch >> 1);
            row = row < last ? row : last;
            pc[i] = op.codes + row * (K / 2) + (ch & 1) * 16;
        }
        int64_t srow = row0 + (tid % ROWS);
        srow = srow < last ? srow : last;
        ps = op.scales + (op.tiled ? srow / 16 : srow) * (K / 16);
    }
    __device__ __forceinline__ void load() {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            c[i] = *reinterpret_cast<const uint4*>(pc[i]);
            pc[i] += kRowBytes;
        }
        s = *reinterpret_cast<const uint32_t*>(ps);
        ps += 4;
    }
};

// Guarded loads for any K % 16 == 0 (zero codes past K and past the last row).
template <int ROWS, int NT>
struct GuardedLoader {
    static constexpr int kPer = (ROWS * 2 + NT - 1) / NT;
    OperandDesc op;
    int64_t row0;
    int K, k0;
    uint4 c[kPer];
    uint32_t s;

    __device__ __forceinline__ void init(const OperandDesc& o, int64_t r0, int k, int) {
        op = o; row0 = r0; K = k; k0 = 0;
    }
    __device__ __forceinline__ void load_at(int tid) {
        const int64_t rb = K / 2;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int ch = tid + i * NT;
            c[i] = make_uint4(0, 0, 0, 0);
            if (ch < ROWS * 2) {
                const int64_t row = row0 + (ch >> 1);
                const int kk = k0 + (ch & 1) * 32;
                if (row < op.rows && kk < K) {
                    const uint8_t* p = op.codes + row * rb + kk / 2;
                    if (kk + 32 <= K) {
                        c[i] = *reinterpret_cast<const uint4*>(p);
                    } else {                                       // K % 32 == 16 tail
                        const uint2 v = *reinterpret_cast<const uint2*>(p);
                        c[i] = make_uint4(v.x, v.y, 0, 0);
                    }
                }
            }
        }
        s = 0;
        if (tid < ROWS) {
            const int64_t row = row0 + tid;
            if (row < op.rows) {
                const int64_t nkb = K / 16;
                const uint8_t* sp = op.tiled ? op.scales + (row / 16) * nkb : op.scales + row * nkb;
                const int kb0 = k0 / 16;
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    if (kb0 + b < nkb) s |= (uint32_t)sp[kb0 + b] << (8 * b);
            }
        }
        k0 += kBK;
    }
};

template <int WM, int WN, int TM, int TN, bool kBF16Out, bool kFast>
__global__ void __launch_bounds__(WM * WN * 64)
k_gemm_nvfp4(OperandDesc A, OperandDesc B, int M, int N, int K, const float* __restrict__ sdA,
             const float* __restrict__ sdB, void* __restrict__ C, int64_t ldc) {
    using Cfg = GemmCfg<WM, WN, TM, TN>;
    constexpr int BM = Cfg::BM, BN = Cfg::BN, NT = Cfg::kThreads;
    __shared__ __attribute__((aligned(16))) LdsTile<BM> lds_a[2];
    __shared__ __attribute__((aligned(16))) LdsTile<BN> lds_b[2];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const uint32_t nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
    uint32_t bm, bn;
    tile_coords(blockIdx.x, nbm, nbn, bm, bn);
    const int64_t m0 = (int64_t)bm * BM, n0 = (int64_t)bn * BN;

    float16v acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    using LA = typename std::conditional<kFast, FastLoader<BM, NT>, GuardedLoader<BM, NT>>::type;
    using LB = typename std::conditional<kFast, FastLoader<BN, NT>, GuardedLoader<BN, NT>>::type;
    LA la;
    LB lb;
    la.init(A, m0, K, tid);
    lb.init(B, n0, K, tid);
    auto load = [&]() {
        if constexpr (kFast) { la.load(); lb.load(); }
        else { la.load_at(tid); lb.load_at(tid); }
    };
    const int nk = (K + kBK - 1) / kBK;
    load();
    store_stage<BM, NT>(lds_a[0], la.c, la.s, tid);
    store_stage<BN, NT>(lds_b[0], lb.c, lb.s, tid);
    __syncthreads();

    const int lrow = lane & 31, h = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load();
        // fragments: 16 bytes (32 codes) and 2 scale pairs per tile and lane
        uint4 fa[TM], fb[TN];
        uint2 xa[TM], xb[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int r = wm * TM * 32 + i * 32 + lrow;
            const int hh = h ^ ((r >> 2) & 1);
            fa[i] = *reinterpret_cast<const uint4*>(&lds_a[cur].codes[r * kRowBytes + hh * 16]);
            xa[i] = reinterpret_cast<const uint2*>(&lds_a[cur].scales[r])[h];
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int r = wn * TN * 32 + j * 32 + lrow;
            const int hh = h ^ ((r >> 2) & 1);
            fb[j] = *reinterpret_cast<const uint4*>(&lds_b[cur].codes[r * kRowBytes + hh * 16]);
            xb[j] = reinterpret_cast<const uint2*>(&lds_b[cur].scales[r])[h];
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            half8 va[TM], vb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const uint32_t w = s == 0 ? fa[i].x : s == 1 ? fa[i].y : s == 2 ? fa[i].z : fa[i].w;
                va[i] = unpack8(w, __builtin_bit_cast(half2v, s < 2 ? xa[i].x : xa[i].y));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const uint32_t w = s == 0 ? fb[j].x : s == 1 ? fb[j].y : s == 2 ? fb[j].z : fb[j].w;
                vb[j] = unpack8(w, __builtin_bit_cast(half2v, s < 2 ? xb[j].x : xb[j].y));
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[i], vb[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            store_stage<BM, NT>(lds_a[cur ^ 1], la.c, la.s, tid);
            store_stage<BN, NT>(lds_b[cur ^ 1], lb.c, lb.s, tid);
        }
        __syncthreads();
    }

    // epilogue: D element r of lane l sits at row 8*(r/4) + 4*(l/32) + r%4, column l%32
    const float alpha = (*sdA) * (*sdB);
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
                    const float v = acc[i][j][r] * alpha;
                    if constexpr (kBF16Out)
                        reinterpret_cast<uint16_t*>(C)[row * ldc + col] = (uint16_t)f32_to_bf16(v);
                    else
                        reinterpret_cast<float*>(C)[row * ldc + col] = v;
                }
            }
        }
}

template <int WM, int WN, int TM, int TN>
static void launch_gemm(const OperandDesc& a, const OperandDesc& b, int M, int N, int K,
                        const float* sdA, const float* sdB, void* c, bool bf16, int64_t ldc,
                        hipStream_t st) {
    using Cfg = GemmCfg<WM, WN, TM, TN>;
    const uint32_t nbm = (M + Cfg::BM - 1) / Cfg::BM, nbn = (N + Cfg::BN - 1) / Cfg::BN;
    const dim3 grid(nbm * nbn), block(Cfg::kThreads);
    const bool fast = K % kBK == 0;
#define NVFP4_GEMM_LAUNCH(BF, FAST)                                                               \
    hipLaunchKernelGGL((k_gemm_nvfp4<WM, WN, TM, TN, BF, FAST>), grid, block, 0, st, a, b, M, N, K, \
                       sdA, sdB, c, ldc)
    if (bf16) {
        if (fast) NVFP4_GEMM_LAUNCH(true, true); else NVFP4_GEMM_LAUNCH(true, false);
    } else {
        if (fast) NVFP4_GEMM_LAUNCH(false, true); else NVFP4_GEMM_LAUNCH(false, false);
    }
#undef NVFP4_GEMM_LAUNCH
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" nvfp4_status nvfp4_gemm(const nvfp4_tensor* a, const nvfp4_tensor* b, void* c,
                                   nvfp4_dtype c_dt, int64_t ldc, void* stream) {
    nvfp4_status s = check_q(a, NVFP4_BLK_1x16, false);
    if (s) return s;
    if (!b) return NVFP4_ERR_NULL;
    if (b->layout != NVFP4_BLK_1x16 && b->layout != NVFP4_BLK_16x16) return NVFP4_ERR_LAYOUT;
    s = check_q(b, b->layout, false);
    if (s) return s;
    if (!a->s_dec || !b->s_dec) return NVFP4_ERR_NULL;
    if (a->cols != b->cols) return NVFP4_ERR_SHAPE;
    s = check_output(c, c_dt, a->rows, b->rows, ldc);
    if (s) return s;
    const int64_t M = a->rows, N = b->rows, K = a->cols;
    if (M >= (1ll << 31) || N >= (1ll << 31) || K >= (1ll << 31)) return NVFP4_ERR_SHAPE;
    if (M == 0 || N == 0) return NVFP4_OK;
    const OperandDesc da{a->codes, a->scales, M, 0};
    const OperandDesc db{b->codes, b->scales, N, b->layout == NVFP4_BLK_16x16 ? 1 : 0};
    launch_gemm<2, 2, 4, 4>(da, db, (int)M, (int)N, (int)K, a->s_dec, b->s_dec, c,
                            c_dt == NVFP4_BF16, ldc, as_stream(stream));
    return launch_status();
}
