// gemm_mx.hip -- MXFP4 x MXFP4 GEMM on gfx950's block-scaled FP4 MFMA.
//
// The comparison format of [P3] "I ricercatori di Nvidia sbloccano il tutorial LLM a 8 bit che
// corrisponde alle prestazioni a 4 bit", NVFP4 in pratica (MXFP4 needed more training data to
// match NVFP4).  MXFP4 scales are powers of two per 32 elements, which is exactly what
// v_mfma_scale_f32_32x32x64_f8f6f4 applies in hardware, so packed codes go to the matrix core
// without any unpacking:
//   C[m,n] = sum_kb 2^(eA[m,kb] + eB[n,kb]) * sum_{k in kb} vA[m,k] * vB[n,k].
// One MFMA covers K = 64: lane l supplies row l%32 and the 32-element block (l/32) of the 64,
// i.e. 16 bytes of codes plus that block's E8M0 byte.
//
// K % 128 == 0: 256 x 256 output tile, 8 waves (2 per SIMD) of 128 x 64.  Since nothing is
// unpacked, operands go from global memory straight into LDS (global_load_lds_dwordx4: each
// lane's 16 bytes land at its slot of a 1 KiB window), with no VGPRs held for the fetch.  The
// last sub-step's MFMAs are deferred past the LDS-only barrier that ends each step, as in the
// NVFP4 kernel, and the epilogues are shared with it.
//   K % 256 == 0 (all the step and FFN-pair shapes): steps of 256 (four MFMA sub-steps) through
//     two 68 KiB stages, one step ahead -- one barrier per 32 MFMAs per wave;
//   otherwise steps of 128 (two sub-steps) through a ring of three 34 KiB stages, two ahead.
// The longer step is what pays: at 128 the waves spent a third of their cycles waiting at the
// per-step barrier and counters with the MFMA pipe 30-37% busy.
// Other K (K % 32 == 0): a plainer kernel with zero-padded guarded loads through registers.

#include "device_codecs.hpp"
#include "gemm_common.hpp"
#include "host_util.hpp"

namespace nvfp4 {

typedef int int8v __attribute__((ext_vector_type(8)));
typedef int int4v __attribute__((ext_vector_type(4)));

constexpr int kMxBK = 128;               // K elements per pipeline step (two MFMAs)
constexpr int kMxRowBytes = kMxBK / 2;   // 64 packed bytes per row per step
constexpr int kFmtFp4 = 4;               // f8f6f4 operand format code for E2M1

// An FP4 MFMA operand: the builtin takes eight dwords (room for FP8); E2M1 uses the first four,
// so the rest is left undefined and the instruction reads a 4-register tuple.
__device__ __forceinline__ int8v fp4_operand(uint4 v) {
    const int4v w = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
    return __builtin_shufflevector(w, w, 0, 1, 2, 3, -1, -1, -1, -1);
}

// ---- K % 128 == 0: direct-to-LDS loads; steps of 128 through a three-stage ring --------------

constexpr int kMxTile = 256;             // BM = BN
constexpr int kMxThreads = 512;          // 8 waves
constexpr int kMxStages = 3;             // LDS ring: the step being multiplied + two in flight
constexpr int kMxDmaPerStep = 5;         // global->LDS loads per wave per step

struct MxOperand {
    const uint8_t* codes;    // [rows x K/2]
    const uint8_t* scales;   // [rows x K/32] E8M0
    int64_t rows;
};

// One step in LDS: per operand 256 rows x four 16-byte chunks (chunk c = K-block c of the step,
// stored at slot c ^ ((r / 4) % 4), so 16 consecutive rows reading one chunk hit 16 distinct
// bank groups) and each row's four E8M0 bytes (byte c = block c).
struct alignas(16) MxStage {
    uint4 a[kMxTile * 4];
    uint4 b[kMxTile * 4];
    uint32_t sa[kMxTile];
    uint32_t sb[kMxTile];
};
static_assert(sizeof(MxStage) == 34816, "stage layout");

__device__ __forceinline__ int mx_swz(int r, int c) { return c ^ ((r >> 2) & 3); }

// global -> LDS without VGPRs: lane l's 16 (or 4) bytes from g land at LDS address lds + 16 l
// (or 4 l); lds is wave-uniform and goes in M0.  Written as asm so that the compiler, which
// cannot tell these writes from the ones in flight for later steps, does not wait for all of
// them before every LDS read; completion is waited for explicitly (wait_vmcnt).  The nop is
// the wait state gfx9 needs between writing M0 and an LDS-DMA load.
__device__ __forceinline__ void lds_dma16(const uint8_t* g, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void lds_dma4(const uint8_t* g, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}

// s_waitcnt vmcnt(n) (gfx9 encoding, expcnt and lgkmcnt left at their maxima): at most n of this
// wave's vector-memory loads still outstanding.  Loads complete in issue order.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// This lane's sources for one step.  Wave w fetches A rows [32w, 32w + 32) and the same B rows
// (two 1 KiB windows each: 16 rows x 64 bytes, lane l -> row l / 4, slot l % 4, which holds
// chunk (l % 4) ^ swizzle), and the scale words of 64 rows: waves 0-3 those of A, 4-7 of B.
// Rows past the matrix are clamped to its last row (never stored); steps past the end are
// clamped to the last step (never read), so every load is in bounds and none is conditional.
struct MxDma {
    const uint8_t *a0, *a1, *b0, *b1, *s;
    int nk;
    __device__ __forceinline__ void init(const MxOperand& A, const MxOperand& B, int64_t m0,
                                         int64_t n0, int K, int wave, int lane) {
        const int64_t rb = K / 2, nkb = K / 32;
        const int rr0 = (2 * wave) * 16 + (lane >> 2), rr1 = rr0 + 16;
        const int c0 = mx_swz(rr0, lane & 3), c1 = mx_swz(rr1, lane & 3);
        const int64_t ma = A.rows - 1, mb = B.rows - 1;
        a0 = A.codes + (m0 + rr0 < ma ? m0 + rr0 : ma) * rb + c0 * 16;
        a1 = A.codes + (m0 + rr1 < ma ? m0 + rr1 : ma) * rb + c1 * 16;
        b0 = B.codes + (n0 + rr0 < mb ? n0 + rr0 : mb) * rb + c0 * 16;
        b1 = B.codes + (n0 + rr1 < mb ? n0 + rr1 : mb) * rb + c1 * 16;
        const bool isb = wave >= 4;
        const int64_t r = (isb ? n0 : m0) + (wave & 3) * 64 + lane, last = isb ? mb : ma;
        s = (isb ? B.scales : A.scales) + (r < last ? r : last) * nkb;
        nk = K / kMxBK;
    }
    // Step `step` into the stage at LDS byte address `stage` (wave-uniform).
    __device__ __forceinline__ void issue(int step, uint32_t stage, int wave) const {
        const int64_t k = step < nk ? step : nk - 1;
        const uint32_t wa = stage + (2 * wave) * 1024;
        lds_dma16(a0 + k * kMxRowBytes, wa);
        lds_dma16(a1 + k * kMxRowBytes, wa + 1024);
        lds_dma16(b0 + k * kMxRowBytes, wa + 16384);
        lds_dma16(b1 + k * kMxRowBytes, wa + 16384 + 1024);
        lds_dma4(s + k * 4, stage + 32768 + wave * 256);
    }
};

// The operands one wave multiplies in one sub-step s (K-block q = 2s + lane / 32 of each row).
template <int TM, int TN>
struct MxFrags {
    uint4 a[TM], b[TN];
    uint32_t ea[TM], eb[TN];
};

template <int TM, int TN>
__device__ __forceinline__ void mx_read_frags(const MxStage& st, MxFrags<TM, TN>& f, int wm, int wn,
                                              int lane, int s) {
    const int lrow = lane & 31, q = 2 * s + (lane >> 5);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int r = wm * TM * 32 + i * 32 + lrow;
        f.a[i] = st.a[r * 4 + mx_swz(r, q)];
        f.ea[i] = (st.sa[r] >> (8 * q)) & 0xFFu;
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int r = wn * TN * 32 + j * 32 + lrow;
        f.b[j] = st.b[r * 4 + mx_swz(r, q)];
        f.eb[j] = (st.sb[r] >> (8 * q)) & 0xFFu;
    }
}

// kT: B is the MFMA's first operand and each accumulator tile is held transposed (the layout
// the staged bf16 epilogue takes); otherwise one output column per lane.  The E8M0 scale of each
// operand is byte SEL of its scale word (the MFMA's op_sel).
template <int TM, int TN, bool kT, int SEL = 0>
__device__ __forceinline__ void mx_mfma(const MxFrags<TM, TN>& f, float16v (&acc)[TM][TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int8v va = fp4_operand(f.a[i]);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int8v vb = fp4_operand(f.b[j]);
            acc[i][j] = kT ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                 vb, va, acc[i][j], kFmtFp4, kFmtFp4, SEL, (int)f.eb[j], SEL, (int)f.ea[i])
                           : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                 va, vb, acc[i][j], kFmtFp4, kFmtFp4, SEL, (int)f.ea[i], SEL, (int)f.eb[j]);
        }
    }
}

template <int WM, int WN, int TM, int TN, bool kBF16Out>
__global__ void __launch_bounds__(kMxThreads)
k_gemm_mxfp4_dma(MxOperand A, MxOperand B, int M, int N, int K, void* __restrict__ C, int64_t ldc) {
    static_assert(WM * WN == kMxThreads / 64 && WM * TM * 32 == kMxTile && WN * TN * 32 == kMxTile,
                  "tile");
    constexpr bool kT = kBF16Out;
    // the stage ring, reused afterwards as the epilogue's staging area (16 KiB per wave)
    constexpr int kRing = kMxStages * (int)sizeof(MxStage), kStaging = (kMxThreads / 64) * 16384;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kRing > kStaging ? kRing : kStaging];
    const MxStage* st = reinterpret_cast<const MxStage*>(lds);
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(lds);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const uint32_t nbm = (M + kMxTile - 1) / kMxTile, nbn = (N + kMxTile - 1) / kMxTile;
    uint32_t bm, bn;
    tile_coords(blockIdx.x, nbm, nbn, bm, bn);
    const int64_t m0 = (int64_t)bm * kMxTile, n0 = (int64_t)bn * kMxTile;

    float16v acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    MxDma dma;
    dma.init(A, B, m0, n0, K, wave, lane);
    const int nk = dma.nk;
    dma.issue(0, lds0, wave);
    dma.issue(1, lds0 + sizeof(MxStage), wave);
    MxFrags<TM, TN> f0, f1;
#pragma unroll
    for (int i = 0; i < TM; ++i) { f1.a[i] = make_uint4(0, 0, 0, 0); f1.ea[i] = 127; }
#pragma unroll
    for (int j = 0; j < TN; ++j) { f1.b[j] = make_uint4(0, 0, 0, 0); f1.eb[j] = 127; }
    wait_vmcnt<kMxDmaPerStep>();                        // step 0 has landed
    lds_barrier();
    mx_read_frags<TM, TN>(st[0], f0, wm, wn, lane, 0);
    // Step kt multiplies stage kt % 3 while steps kt + 1 and kt + 2 are in flight; stage
    // (kt + 2) % 3 held step kt - 1, whose last reads finished before the barrier that ended it.
    int cs = 0;
    for (int kt = 0; kt < nk; ++kt) {
        const int ns = cs == 0 ? 2 : cs - 1;            // (kt + 2) % 3
        dma.issue(kt + 2, lds0 + ns * (uint32_t)sizeof(MxStage), wave);
        mx_mfma<TM, TN, kT>(f1, acc);                   // previous step, sub-step 1
        __builtin_amdgcn_sched_barrier(0);
        mx_read_frags<TM, TN>(st[cs], f1, wm, wn, lane, 1);
        mx_mfma<TM, TN, kT>(f0, acc);                   // sub-step 0
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<kMxDmaPerStep>();                    // step kt + 1 has landed
        lds_barrier();
        cs = cs == 2 ? 0 : cs + 1;
        mx_read_frags<TM, TN>(st[cs], f0, wm, wn, lane, 0);
    }
    mx_mfma<TM, TN, kT>(f1, acc);                       // sub-step 1 of the last step
    wait_vmcnt<0>();                                    // the clamped re-fetches past the end

    const int64_t r0 = m0 + wm * TM * 32, c0 = n0 + wn * TN * 32;
    if constexpr (kBF16Out) {
        const bool vec = (reinterpret_cast<uintptr_t>(C) & 15u) == 0 && (ldc * 2) % 16 == 0;
        __syncthreads();                    // every wave is done with the stage ring
        epilogue_bf16<TM, TN>(acc, 1.0f, lds + wave * 16384, lane, r0, c0, M, N,
                              reinterpret_cast<uint16_t*>(C), ldc, vec);
    } else {
        epilogue_f32<TM, TN>(acc, 1.0f, lane, r0, c0, M, N, reinterpret_cast<float*>(C), ldc);
    }
}

// ---- K % 256 == 0: steps of 256 through two stages ------------------------------------------
constexpr int kD2BK = 256, kD2RowBytes = 128;

// One step in LDS: per operand 256 rows x eight 16-byte chunks (chunk c = K-block c of the step,
// at slot c ^ ((r / 2) % 8): 16 consecutive rows reading one chunk hit 16 distinct bank groups),
// then each row's eight E8M0 bytes as two words (blocks 0-3, 4-7).
struct alignas(16) MxStage2 {
    uint4 a[kMxTile * 8];
    uint4 b[kMxTile * 8];
    uint32_t sa[2][kMxTile];     // a row's scale bytes of blocks 0-3 and 4-7 of the step
    uint32_t sb[2][kMxTile];
};
static_assert(sizeof(MxStage2) == 69632, "stage2");
__device__ __forceinline__ int d2_swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// This lane's sources for one step.  Wave w fetches A rows [32w, 32w + 32) and the same B rows
// as four 1 KiB windows each (8 rows x 128 bytes; lane l -> row l / 8, slot l % 8), and two of
// the sixteen 256-byte scale windows (64 rows' words of A blocks 0-3, A 4-7, B 0-3, B 4-7).  Rows
// past the matrix and steps past K are clamped as in MxDma.  10 loads per wave per step.
struct MxDma2 {
    const uint8_t *a[4], *b[4], *s0, *s1;
    int nk;
    // Sources of steps [kb, kb + nsteps) (the workgroup's K range).
    __device__ __forceinline__ void init(const MxOperand& A, const MxOperand& B, int64_t m0,
                                         int64_t n0, int K, int wave, int lane, int kb, int nsteps) {
        const int64_t rb = K / 2, nkb = K / 32;
        const int64_t ma = A.rows - 1, mb = B.rows - 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rr = (4 * wave + j) * 8 + (lane >> 3);
            const int c = d2_swz(rr, lane & 7);
            a[j] = A.codes + (m0 + rr < ma ? m0 + rr : ma) * rb + (int64_t)kb * kD2RowBytes + c * 16;
            b[j] = B.codes + (n0 + rr < mb ? n0 + rr : mb) * rb + (int64_t)kb * kD2RowBytes + c * 16;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int v = 2 * wave + u;                        // 256-byte window of the scales
            const bool isb = v >= 8;
            const int half = (v >> 2) & 1;
            const int64_t r = (isb ? n0 : m0) + (v & 3) * 64 + lane, last = isb ? mb : ma;
            const uint8_t* p = (isb ? B.scales : A.scales) + (r < last ? r : last) * nkb +
                               (int64_t)kb * 8 + half * 4;
            if (u == 0) s0 = p; else s1 = p;
        }
        nk = nsteps;
    }
    __device__ __forceinline__ void issue(int step, uint32_t stage, int wave) const {
        const int64_t k = step < nk ? step : nk - 1;
#pragma unroll
        for (int j = 0; j < 4; ++j) lds_dma16(a[j] + k * kD2RowBytes, stage + (4 * wave + j) * 1024);
#pragma unroll
        for (int j = 0; j < 4; ++j) lds_dma16(b[j] + k * kD2RowBytes, stage + 32768 + (4 * wave + j) * 1024);
        lds_dma4(s0 + k * 8, stage + 65536 + (2 * wave) * 256);
        lds_dma4(s1 + k * 8, stage + 65536 + (2 * wave + 1) * 256);
    }
};

// The fragments of sub-step s (K-block q = 2s + lane / 32 of each row).  The scales stay in
// registers for the whole step: at s = 0 a lane reads its rows' two scale words (blocks 0-3 and
// 4-7) and keeps the four bytes of its half, blocks h, 2 + h, 4 + h, 6 + h (h = lane / 32), in
// one word (one v_perm), so that sub-step s finds its block in byte s for both halves and the
// MFMA selects it with op_sel = s (no per-sub-step scale read or byte extract).  At s = 1 the
// words are copied from the other fragment set `prev`, which holds sub-step 0 of the same step;
// at s = 2 and 3 the set still holds this step's words from s = 0 or 1.  The main loop takes
// s = 0 in two parts instead (d2_read_frags0, d2_gather_scales, below).
template <int TM, int TN>
__device__ __forceinline__ void d2_read_frags(const MxStage2& st, MxFrags<TM, TN>& f,
                                              const MxFrags<TM, TN>& prev, int wm, int wn,
                                              int lane, int s) {
    const int lrow = lane & 31, q = 2 * s + (lane >> 5);
    const uint32_t sel = (lane >> 5) ? 0x07050301u : 0x06040200u;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int r = wm * TM * 32 + i * 32 + lrow;
        f.a[i] = st.a[r * 8 + d2_swz(r, q)];
        if (s == 0) f.ea[i] = __builtin_amdgcn_perm(st.sa[1][r], st.sa[0][r], sel);
        if (s == 1) f.ea[i] = prev.ea[i];
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int r = wn * TN * 32 + j * 32 + lrow;
        f.b[j] = st.b[r * 8 + d2_swz(r, q)];
        if (s == 0) f.eb[j] = __builtin_amdgcn_perm(st.sb[1][r], st.sb[0][r], sel);
        if (s == 1) f.eb[j] = prev.eb[j];
    }
}

// Sub-step 0 of a step, split in two so that no wave waits on LDS at the top of a step: the
// fragment codes and the rows' raw scale words are read right after the barrier, and the
// gather of a lane's four scale bytes into one word (d2_gather_scales) runs after the previous
// step's deferred MFMAs have been issued, by when the words have arrived.  Same results as
// d2_read_frags at s = 0.
template <int TM, int TN>
struct MxRawScales {
    uint32_t a[TM][2], b[TN][2];
};

template <int TM, int TN>
__device__ __forceinline__ void d2_read_frags0(const MxStage2& st, MxFrags<TM, TN>& f,
                                               MxRawScales<TM, TN>& raw, int wm, int wn, int lane) {
    const int lrow = lane & 31, q = lane >> 5;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int r = wm * TM * 32 + i * 32 + lrow;
        f.a[i] = st.a[r * 8 + d2_swz(r, q)];
        raw.a[i][0] = st.sa[0][r];
        raw.a[i][1] = st.sa[1][r];
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int r = wn * TN * 32 + j * 32 + lrow;
        f.b[j] = st.b[r * 8 + d2_swz(r, q)];
        raw.b[j][0] = st.sb[0][r];
        raw.b[j][1] = st.sb[1][r];
    }
}

template <int TM, int TN>
__device__ __forceinline__ void d2_gather_scales(MxFrags<TM, TN>& f, const MxRawScales<TM, TN>& raw,
                                                 int lane) {
    const uint32_t sel = (lane >> 5) ? 0x07050301u : 0x06040200u;
#pragma unroll
    for (int i = 0; i < TM; ++i) f.ea[i] = __builtin_amdgcn_perm(raw.a[i][1], raw.a[i][0], sel);
#pragma unroll
    for (int j = 0; j < TN; ++j) f.eb[j] = __builtin_amdgcn_perm(raw.b[j][1], raw.b[j][0], sel);
}

// Workgroups [0, full) compute whole tiles; with a split plan, workgroup full + u computes part
// u % splits (steps [j nk / splits, (j + 1) nk / splits)) of tile full + u / splits into the
// fp32 partial tile ws + u * 256 * 256, which k_splitk_fixup adds in part order.
template <int WM, int WN, int TM, int TN, bool kBF16Out>
__global__ void __launch_bounds__(kMxThreads)
k_gemm_mxfp4_d2(MxOperand A, MxOperand B, int M, int N, int K, void* __restrict__ C, int64_t ldc,
                uint32_t full, uint32_t splits, float* __restrict__ ws) {
    constexpr bool kT = kBF16Out;
    constexpr int kRing = 2 * (int)sizeof(MxStage2), kStaging = (kMxThreads / 64) * 16384;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kRing > kStaging ? kRing : kStaging];
    const MxStage2* st = reinterpret_cast<const MxStage2*>(lds);
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(lds);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const uint32_t nbm = (M + kMxTile - 1) / kMxTile, nbn = (N + kMxTile - 1) / kMxTile;
    const int nk_all = K / kD2BK;
    uint32_t tile = blockIdx.x;
    int kb = 0, nsteps = nk_all;
    const bool split = blockIdx.x >= full;           // uniform over the workgroup
    if (split) {
        const uint32_t u = blockIdx.x - full, j = u % splits;
        tile = full + u / splits;
        kb = (int)(((int64_t)j * nk_all) / splits);
        nsteps = (int)(((int64_t)(j + 1) * nk_all) / splits) - kb;
    }
    uint32_t bm, bn;
    tile_coords(tile, nbm, nbn, bm, bn);
    const int64_t m0 = (int64_t)bm * kMxTile, n0 = (int64_t)bn * kMxTile;

    float16v acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    MxDma2 dma;
    dma.init(A, B, m0, n0, K, wave, lane, kb, nsteps);
    const int nk = dma.nk;
    dma.issue(0, lds0, wave);
    MxFrags<TM, TN> f0, f1;
#pragma unroll
    for (int i = 0; i < TM; ++i) { f1.a[i] = make_uint4(0, 0, 0, 0); f1.ea[i] = 0x7F7F7F7Fu; }
#pragma unroll
    for (int j = 0; j < TN; ++j) { f1.b[j] = make_uint4(0, 0, 0, 0); f1.eb[j] = 0x7F7F7F7Fu; }
    MxRawScales<TM, TN> raw;
    wait_vmcnt<0>();
    lds_barrier();
    dma.issue(1, lds0 + sizeof(MxStage2), wave);
    d2_read_frags0<TM, TN>(st[0], f0, raw, wm, wn, lane);
    // Step kt multiplies stage kt % 2 while step kt + 1 lands in the other; after the barrier
    // that ends step kt (all reads of its stage done) step kt + 2 is fetched into it.
    int cs = 0;
    for (int kt = 0; kt < nk; ++kt) {
        const MxStage2& cur = st[cs];
        mx_mfma<TM, TN, kT, 3>(f1, acc);                // previous step, sub-step 3
        __builtin_amdgcn_sched_barrier(0);
        d2_gather_scales<TM, TN>(f0, raw, lane);
        d2_read_frags<TM, TN>(cur, f1, f0, wm, wn, lane, 1);
        mx_mfma<TM, TN, kT, 0>(f0, acc);                // sub-step 0
        __builtin_amdgcn_sched_barrier(0);
        d2_read_frags<TM, TN>(cur, f0, f1, wm, wn, lane, 2);
        mx_mfma<TM, TN, kT, 1>(f1, acc);                // sub-step 1
        __builtin_amdgcn_sched_barrier(0);
        d2_read_frags<TM, TN>(cur, f1, f0, wm, wn, lane, 3);
        mx_mfma<TM, TN, kT, 2>(f0, acc);                // sub-step 2
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<0>();                                // step kt + 1 has landed
        lds_barrier();
        dma.issue(kt + 2, lds0 + cs * (uint32_t)sizeof(MxStage2), wave);
        cs ^= 1;
        d2_read_frags0<TM, TN>(st[cs], f0, raw, wm, wn, lane);
        __builtin_amdgcn_sched_barrier(0);              // issue the reads before the MFMAs
    }
    mx_mfma<TM, TN, kT, 3>(f1, acc);                    // sub-step 3 of the last step
    wait_vmcnt<0>();                                    // the clamped re-fetches past the end

    if (split) {
        store_partial<TM, TN, kT>(acc, lane, wm * TM * 32, wn * TN * 32,
                                  ws + (size_t)(blockIdx.x - full) * (kMxTile * kMxTile));
        return;
    }
    const int64_t r0 = m0 + wm * TM * 32, c0 = n0 + wn * TN * 32;
    if constexpr (kBF16Out) {
        const bool vec = (reinterpret_cast<uintptr_t>(C) & 15u) == 0 && (ldc * 2) % 16 == 0;
        __syncthreads();                    // every wave is done with the stages
        epilogue_bf16<TM, TN>(acc, 1.0f, lds + wave * 16384, lane, r0, c0, M, N,
                              reinterpret_cast<uint16_t*>(C), ldc, vec);
    } else {
        epilogue_f32<TM, TN>(acc, 1.0f, lane, r0, c0, M, N, reinterpret_cast<float*>(C), ldc);
    }
}

// ---- any K % 32 == 0: guarded loads through registers ---------------------------------------

// A stage of ROWS rows: 64 code bytes (four 16-byte chunks) and 4 E8M0 bytes per row.  Blocks
// past K and rows past the matrix load as zero codes with unit scales.
template <int ROWS, int NT>
struct MxRegStage {
    static constexpr int kChunks = ROWS * 4;
    static constexpr int kPerThread = (kChunks + NT - 1) / NT;
    uint4 c[kPerThread];
    uint32_t s;

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
                    if (kb0 + b < nkb)
                        s = (s & ~(0xFFu << (8 * b))) | ((uint32_t)scales[row * nkb + kb0 + b] << (8 * b));
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

template <int WM, int WN, int TM, int TN, bool kBF16Out>
__global__ void __launch_bounds__(WM * WN * 64)
k_gemm_mxfp4_any(const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
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
    tile_coords(blockIdx.x, nbm, nbn, bm, bn);
    const int64_t m0 = (int64_t)bm * BM, n0 = (int64_t)bn * BN;

    float16v acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    MxRegStage<BM, NT> sa;
    MxRegStage<BN, NT> sb;
    const int nk = (K + kMxBK - 1) / kMxBK;
    sa.load(a_codes, a_scales, M, m0, 0, K, tid);
    sb.load(b_codes, b_scales, N, n0, 0, K, tid);
    sa.store(lds_a[0], lds_sa[0], tid);
    sb.store(lds_b[0], lds_sb[0], tid);
    __syncthreads();

    const int lrow = lane & 31, h = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
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
                const uint8_t* p = &lds_a[cur][r * kMxRowBytes + ((q + r) & 3) * 16];
                va[i] = fp4_operand(*reinterpret_cast<const uint4*>(p));
                ea[i] = (lds_sa[cur][r] >> (8 * q)) & 0xFFu;
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn * TN * 32 + j * 32 + lrow;
                const uint8_t* p = &lds_b[cur][r * kMxRowBytes + ((q + r) & 3) * 16];
                vb[j] = fp4_operand(*reinterpret_cast<const uint4*>(p));
                eb[j] = (lds_sb[cur][r] >> (8 * q)) & 0xFFu;
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        va[i], vb[j], acc[i][j], kFmtFp4, kFmtFp4, 0, (int)ea[i], 0, (int)eb[j]);
        }
        if (kt + 1 < nk) {
            sa.store(lds_a[cur ^ 1], lds_sa[cur ^ 1], tid);
            sb.store(lds_b[cur ^ 1], lds_sb[cur ^ 1], tid);
        }
        __syncthreads();
    }
    {
        const int64_t r0 = m0 + wm * TM * 32, c0 = n0 + wn * TN * 32;
        // column-per-lane accumulator layout: element r of tile (i, j) is row
        // r0 + 32 i + 8 (r / 4) + 4 h + r % 4, column c0 + 32 j + lane % 32
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int64_t col = c0 + j * 32 + lrow;
                if (col >= N) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t row = r0 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (row >= M) continue;
                    if constexpr (kBF16Out)
                        reinterpret_cast<uint16_t*>(C)[row * ldc + col] = (uint16_t)f32_to_bf16(acc[i][j][r]);
                    else
                        reinterpret_cast<float*>(C)[row * ldc + col] = acc[i][j][r];
                }
            }
    }
}

constexpr int kMxMinSplitSteps = 4;    // K steps of 256 per split part, at least

static nvfp4_status check_mx_gemm(const nvfp4_tensor* a, const nvfp4_tensor* b, const void* c,
                                  nvfp4_dtype c_dt, int64_t ldc) {
    nvfp4_status s = check_q(a, MXFP4_BLK_1x32, false);
    if (s) return s;
    s = check_q(b, MXFP4_BLK_1x32, false);
    if (s) return s;
    if (a->cols != b->cols) return NVFP4_ERR_SHAPE;
    s = check_output(c, c_dt, a->rows, b->rows, ldc);
    if (s) return s;
    const int64_t M = a->rows, N = b->rows, K = a->cols;
    if (M >= (1ll << 31) || N >= (1ll << 31) || K >= (1ll << 31)) return NVFP4_ERR_SHAPE;
    if (((M + kMxTile - 1) / kMxTile) * ((N + kMxTile - 1) / kMxTile) >= (1ll << 31))
        return NVFP4_ERR_SHAPE;
    return NVFP4_OK;
}

// The plan of a K % 256 == 0 GEMM (the only kernel that splits); whole tiles otherwise.
static SplitPlan mx_plan(int64_t M, int64_t N, int64_t K) {
    if (K % kD2BK != 0) {
        const uint32_t tiles = (uint32_t)(((M + kMxTile - 1) / kMxTile) * ((N + kMxTile - 1) / kMxTile));
        return SplitPlan{tiles, 0, 1, 0};
    }
    return plan_split(M, N, K, device_cus(), kD2BK, kMxMinSplitSteps);
}

static nvfp4_status run_mx_gemm(const nvfp4_tensor* a, const nvfp4_tensor* b, void* c,
                                nvfp4_dtype c_dt, int64_t ldc, const SplitPlan& plan, float* ws,
                                hipStream_t st) {
    const int64_t M = a->rows, N = b->rows, K = a->cols;
    if (M == 0 || N == 0) return NVFP4_OK;
    const bool bf16 = c_dt == NVFP4_BF16;
    if (K == 0) {                                  // no codes to read (they may be null)
        launch_zero_c(c, bf16, ldc, (int)M, (int)N, st);
        return launch_status();
    }
    const uint32_t nbm = (M + kMxTile - 1) / kMxTile, nbn = (N + kMxTile - 1) / kMxTile;
    const dim3 grid(nbm * nbn);
    if (K % kD2BK == 0) {
        const MxOperand da{a->codes, a->scales, M}, db{b->codes, b->scales, N};
        const dim3 g2(plan.full + plan.tail * plan.splits);
        if (bf16)
            hipLaunchKernelGGL((k_gemm_mxfp4_d2<2, 4, 4, 2, true>), g2, dim3(kMxThreads), 0, st,
                               da, db, (int)M, (int)N, (int)K, c, ldc, plan.full, plan.splits, ws);
        else
            hipLaunchKernelGGL((k_gemm_mxfp4_d2<2, 4, 4, 2, false>), g2, dim3(kMxThreads), 0, st,
                               da, db, (int)M, (int)N, (int)K, c, ldc, plan.full, plan.splits, ws);
        launch_splitk_fixup(plan, ws, (int)M, (int)N, nullptr, nullptr, c, bf16, ldc, st);
    } else if (K % kMxBK == 0) {
        const MxOperand da{a->codes, a->scales, M}, db{b->codes, b->scales, N};
        if (bf16)
            hipLaunchKernelGGL((k_gemm_mxfp4_dma<2, 4, 4, 2, true>), grid, dim3(kMxThreads), 0, st,
                               da, db, (int)M, (int)N, (int)K, c, ldc);
        else
            hipLaunchKernelGGL((k_gemm_mxfp4_dma<2, 4, 4, 2, false>), grid, dim3(kMxThreads), 0, st,
                               da, db, (int)M, (int)N, (int)K, c, ldc);
    } else {
        if (bf16)
            hipLaunchKernelGGL((k_gemm_mxfp4_any<2, 2, 4, 4, true>), grid, dim3(256), 0, st,
                               a->codes, a->scales, b->codes, b->scales, (int)M, (int)N, (int)K, c, ldc);
        else
            hipLaunchKernelGGL((k_gemm_mxfp4_any<2, 2, 4, 4, false>), grid, dim3(256), 0, st,
                               a->codes, a->scales, b->codes, b->scales, (int)M, (int)N, (int)K, c, ldc);
    }
    return launch_status();
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" nvfp4_status mxfp4_gemm(const nvfp4_tensor* a, const nvfp4_tensor* b, void* c,
                                   nvfp4_dtype c_dt, int64_t ldc, void* stream) {
    const nvfp4_status s = check_mx_gemm(a, b, c, c_dt, ldc);
    if (s) return s;
    const uint32_t tiles = (uint32_t)(((a->rows + kMxTile - 1) / kMxTile) * ((b->rows + kMxTile - 1) / kMxTile));
    return run_mx_gemm(a, b, c, c_dt, ldc, SplitPlan{tiles, 0, 1, 0}, nullptr, as_stream(stream));
}

extern "C" nvfp4_status mxfp4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, size_t* bytes) {
    if (!bytes) return NVFP4_ERR_NULL;
    if (M < 0 || N < 0 || K < 0 || M >= (1ll << 31) || N >= (1ll << 31) || K >= (1ll << 31))
        return NVFP4_ERR_SHAPE;
    *bytes = (M == 0 || N == 0 || K == 0) ? 0 : mx_plan(M, N, K).ws_bytes;
    return NVFP4_OK;
}

extern "C" nvfp4_status mxfp4_gemm_ws(const nvfp4_tensor* a, const nvfp4_tensor* b, void* c,
                                      nvfp4_dtype c_dt, int64_t ldc, void* workspace,
                                      size_t ws_bytes, void* stream) {
    const nvfp4_status s = check_mx_gemm(a, b, c, c_dt, ldc);
    if (s) return s;
    if (workspace && !aligned16(workspace)) return NVFP4_ERR_ALIGN;
    SplitPlan plan = mx_plan(a->rows, b->rows, a->cols);
    if (plan.tail && (!workspace || ws_bytes < plan.ws_bytes))
        plan = SplitPlan{plan.full + plan.tail, 0, 1, 0};        // too small: whole tiles only
    return run_mx_gemm(a, b, c, c_dt, ldc, plan, static_cast<float*>(workspace), as_stream(stream));
}
