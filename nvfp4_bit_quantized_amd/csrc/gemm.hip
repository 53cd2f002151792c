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
// Workgroup: 8 waves (2 per SIMD), a 256 x 256 output tile, K in steps of 64.
//   global -> VGPR prefetch two steps ahead (one 16-byte code chunk of A and of B and the two
//   matching scale bytes of each per thread and step)
//   -> unpacked once per workgroup by the thread that fetched it: v_cvt_scalef32_pk_f16_fp4,
//      times the block scale (v_pk_mul_f16) -> fp16 tiles [256][64] per operand in LDS, double
//      buffered, with the eight 16-byte chunks of a row permuted against bank conflicts
//   -> each wave reads MFMA-ready fp16 fragments (ds_read_b128) -> v_mfma_f32_32x32x16_f16.
// A step is four sub-steps of 16 K.  The sub-steps form one rolling pipeline: the fragments of
// sub-step s + 1 are read while sub-step s multiplies, a quarter of the next step's unpack/store
// follows each sub-step's MFMAs, and the last sub-step's MFMAs are deferred past the barrier
// that ends the step, where they cover the latency of the first reads of the next step.
// The barrier orders LDS only, so global prefetches stay in flight across it.
// K is permuted inside a step identically for both operands: MFMA k-slot (8h + j) of sub-step
// s reads element 32h + 8s + j of the 64-element step, so a lane's 16 bytes cover two whole
// NVFP4 blocks and one scale serves each sub-step.
// Epilogue: bf16 results are staged per wave in the idle step buffers and leave as 128-byte
// row pieces, 16 bytes per lane; fp32 results are stored directly, one column per lane.

#include "device_codecs.hpp"
#include "gemm_common.hpp"
#include "host_util.hpp"

#include <atomic>


namespace nvfp4 {

constexpr int kMinSplitSteps = 16;   // K steps of 64 per split part, at least

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

constexpr int kBK = 64;             // K elements per pipeline step
constexpr int kRowBytes = kBK / 2;  // packed bytes per row per step
constexpr int kTile = 256;          // BM = BN
constexpr int kThreads = 512;       // 8 waves

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

// ---- LDS step buffer --------------------------------------------------------------------------
// The loading threads turn their code chunk into scaled fp16 right away and store it to LDS,
// so every element is unpacked once per workgroup instead of once per wave that reads it;
// waves then read MFMA-ready fp16 fragments.  LDS per step: [256][64] fp16 per operand, with
// the eight 16-byte chunks of a row permuted by chunk ^ (r & 7) ^ ((r >> 3) & 1) so that 8 or
// 16 consecutive rows reading the same logical chunk hit distinct bank groups.
struct alignas(16) LdsStepU {
    _Float16 a[kTile * kBK];
    _Float16 b[kTile * kBK];
};

// Kept as loaded (no combining of the scale words) so that nothing waits for a fetch before
// the step that stores it.
struct FetchU {
    uint4 a, b;
    uint32_t sa, sb;    // A's and B's two scale bytes for this chunk (low 16 bits)
};

__device__ __forceinline__ int chunk_swz(int r, int q) { return q ^ (r & 7) ^ ((r >> 3) & 1); }

struct FastAddrU {
    const uint8_t *pa, *pb, *psa, *psb;
    // Addresses of step kb (the first step of this workgroup's K range).
    __device__ __forceinline__ void init(const OperandDesc& A, const OperandDesc& B, int64_t m0,
                                         int64_t n0, int K, int t, int kb) {
        const int r = t >> 1, h = t & 1;
        int64_t ra = m0 + r, rb = n0 + r;
        ra = ra < A.rows - 1 ? ra : A.rows - 1;
        rb = rb < B.rows - 1 ? rb : B.rows - 1;
        pa = A.codes + ra * (K / 2) + (int64_t)kb * kRowBytes + h * 16;
        pb = B.codes + rb * (K / 2) + (int64_t)kb * kRowBytes + h * 16;
        psa = A.scales + (A.tiled ? ra / 16 : ra) * (K / 16) + kb * 4 + h * 2;
        psb = B.scales + (B.tiled ? rb / 16 : rb) * (K / 16) + kb * 4 + h * 2;
    }
    // Fetch step kt, then advance to step kt + 1 unless kt is the last step: fetches past the
    // end re-read the last step (the caller never stores them), so no load is conditional.
    __device__ __forceinline__ FetchU fetch(int kt, int nk) {
        FetchU f;
        f.a = *reinterpret_cast<const uint4*>(pa);
        f.b = *reinterpret_cast<const uint4*>(pb);
        f.sa = *reinterpret_cast<const uint16_t*>(psa);
        f.sb = *reinterpret_cast<const uint16_t*>(psb);
        const bool adv = kt + 1 < nk;
        pa += adv ? kRowBytes : 0;
        pb += adv ? kRowBytes : 0;
        psa += adv ? 4 : 0;
        psb += adv ? 4 : 0;
        return f;
    }
};

struct GuardedAddrU {
    OperandDesc A, B;
    int64_t m0, n0;
    int K, t, kstep0;
    __device__ __forceinline__ void init(const OperandDesc& a, const OperandDesc& b, int64_t m,
                                         int64_t n, int k, int tid, int kb) {
        A = a; B = b; m0 = m; n0 = n; K = k; t = tid; kstep0 = kb;
    }
    __device__ __forceinline__ uint4 chunk(const OperandDesc& op, int64_t row, int k0) const {
        const int kk = k0 + (t & 1) * 32;
        if (row >= op.rows || kk >= K) return make_uint4(0, 0, 0, 0);
        const uint8_t* p = op.codes + row * (K / 2) + kk / 2;
        if (kk + 32 <= K) return *reinterpret_cast<const uint4*>(p);
        const uint2 v = *reinterpret_cast<const uint2*>(p);          // K % 32 == 16 tail
        return make_uint4(v.x, v.y, 0, 0);
    }
    __device__ __forceinline__ uint32_t scales2(const OperandDesc& op, int64_t row, int k0) const {
        if (row >= op.rows) return 0;
        const int64_t nkb = K / 16;
        const uint8_t* sp = op.scales + (op.tiled ? row / 16 : row) * nkb;
        const int kb = k0 / 16 + (t & 1) * 2;
        uint32_t v = 0;
        if (kb < nkb) v |= sp[kb];
        if (kb + 1 < nkb) v |= (uint32_t)sp[kb + 1] << 8;
        return v;
    }
    // Steps past K read as zeros.
    __device__ __forceinline__ FetchU fetch(int kt, int) {
        FetchU f;
        const int k0 = (kt + kstep0) * kBK;
        const int64_t ra = m0 + (t >> 1), rb = n0 + (t >> 1);
        f.a = chunk(A, ra, k0);
        f.b = chunk(B, rb, k0);
        f.sa = scales2(A, ra, k0);
        f.sb = scales2(B, rb, k0);
        return f;
    }
};

__device__ __forceinline__ void store_one_u(_Float16* rowp, int r, int h, uint4 c, half2v sc) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const _Float16 s = sc[d >> 1];
        const half8 v = unpack8(w[d], half2v{s, s});
        *reinterpret_cast<half8*>(rowp + 8 * chunk_swz(r, 4 * h + d)) = v;
    }
}

__device__ __forceinline__ void store_step_u(LdsStepU& st, FetchU f, int t) {
    const int r = t >> 1, h = t & 1;
    const half2v sa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.sa, 1.0f, false);
    const half2v sb = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.sb, 1.0f, false);
    store_one_u(&st.a[r * kBK], r, h, f.a, sa);
    store_one_u(&st.b[r * kBK], r, h, f.b, sb);
}

// The fp16 fragments one wave multiplies in one sub-step.
template <int TM, int TN>
struct Frags {
    half8 a[TM], b[TN];
};

template <int TM, int TN>
__device__ __forceinline__ void read_frags(const LdsStepU& st, Frags<TM, TN>& f, int wm, int wn,
                                           int lane, int s) {
    const int lrow = lane & 31, h = lane >> 5;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int r = wm * TM * 32 + i * 32 + lrow;
        f.a[i] = *reinterpret_cast<const half8*>(&st.a[r * kBK + 8 * chunk_swz(r, 4 * h + s)]);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int r = wn * TN * 32 + j * 32 + lrow;
        f.b[j] = *reinterpret_cast<const half8*>(&st.b[r * kBK + 8 * chunk_swz(r, 4 * h + s)]);
    }
}

// Accumulator layouts (the operand order does not change the sums or their speed):
//   kT = false: element r of lane l is C[row 8*(r/4) + 4*(l/32) + r%4][col l%32] of the 32x32
//               tile -- one column per lane;
//   kT = true:  B is the MFMA's first operand and the tile is held transposed, element r of
//               lane l is C[row l%32][col 8*(r/4) + 4*(l/32) + r%4] -- four consecutive columns
//               of one row per r/4.
template <int TM, int TN, bool kT>
__device__ __forceinline__ void mfma_frags(const Frags<TM, TN>& f, float16v (&acc)[TM][TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = kT ? __builtin_amdgcn_mfma_f32_32x32x16_f16(f.b[j], f.a[i], acc[i][j], 0, 0, 0)
                           : __builtin_amdgcn_mfma_f32_32x32x16_f16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// Quarter q of the next step: unpack dword q (8 codes, half an NVFP4 block) of this thread's A
// and B code chunks and store them to the next LDS buffer.
__device__ __forceinline__ void store_quarter(LdsStepU& nxt, const FetchU& f, half2v sa, half2v sb,
                                             int tid, int q) {
    const int r = tid >> 1, h = tid & 1;
    const uint32_t wa = q == 0 ? f.a.x : q == 1 ? f.a.y : q == 2 ? f.a.z : f.a.w;
    const uint32_t wb = q == 0 ? f.b.x : q == 1 ? f.b.y : q == 2 ? f.b.z : f.b.w;
    const _Float16 xa = sa[q >> 1], xb = sb[q >> 1];
    const int p = 8 * chunk_swz(r, 4 * h + q);
    *reinterpret_cast<half8*>(&nxt.a[r * kBK + p]) = unpack8(wa, half2v{xa, xa});
    *reinterpret_cast<half8*>(&nxt.b[r * kBK + p]) = unpack8(wb, half2v{xb, xb});
}

// One K step on `cur`.  On entry f0 holds (or is loading) the step's sub-step-0 fragments and
// f1 the previous step's sub-step-3 fragments, not yet multiplied (zeros before the first
// step).  On exit f1 is loading this step's sub-step-3 fragments, left for the caller to
// multiply after the barrier.  With do_store, the fetched codes `f` of the next step are
// unpacked into `nxt` a quarter at a time between the MFMA groups.
template <int TM, int TN, bool kT>
__device__ __forceinline__ void step_pipe(const LdsStepU& cur, LdsStepU& nxt, const FetchU& f,
                                          bool do_store, float16v (&acc)[TM][TN],
                                          Frags<TM, TN>& f0, Frags<TM, TN>& f1, int wm, int wn,
                                          int lane, int tid) {
    const half2v sa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.sa, 1.0f, false);
    const half2v sb = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.sb, 1.0f, false);
    mfma_frags<TM, TN, kT>(f1, acc);                   // previous step, sub-step 3
    if (do_store) store_quarter(nxt, f, sa, sb, tid, 0);
    __builtin_amdgcn_sched_barrier(0);
    read_frags<TM, TN>(cur, f1, wm, wn, lane, 1);
    mfma_frags<TM, TN, kT>(f0, acc);                   // sub-step 0
    if (do_store) store_quarter(nxt, f, sa, sb, tid, 1);
    __builtin_amdgcn_sched_barrier(0);
    read_frags<TM, TN>(cur, f0, wm, wn, lane, 2);
    mfma_frags<TM, TN, kT>(f1, acc);                   // sub-step 1
    if (do_store) store_quarter(nxt, f, sa, sb, tid, 2);
    __builtin_amdgcn_sched_barrier(0);
    read_frags<TM, TN>(cur, f1, wm, wn, lane, 3);
    mfma_frags<TM, TN, kT>(f0, acc);                   // sub-step 2
    if (do_store) store_quarter(nxt, f, sa, sb, tid, 3);
    __builtin_amdgcn_sched_barrier(0);
}

// Waves are arranged WM x WN over the 256 x 256 tile, each owning TM x TN MFMA tiles of 32x32.
// Workgroups [0, full) each compute one whole output tile.  When the tile count leaves the last
// round of the device partly empty, the remaining tiles are split along K: workgroup full + u
// computes split u % splits (K steps [j nk / splits, (j + 1) nk / splits)) of tile full + u /
// splits and stores its unscaled fp32 sums into the partial tile ws + u * 256 * 256, which
// k_splitk_fixup then adds in split order.
template <int WM, int WN, int TM, int TN, bool kBF16Out, typename Addr>
__global__ void __launch_bounds__(kThreads)
k_gemm_nvfp4(OperandDesc A, OperandDesc B, int M, int N, int K, const float* __restrict__ sdA,
             const float* __restrict__ sdB, void* __restrict__ C, int64_t ldc, uint32_t full,
             uint32_t splits, float* __restrict__ ws) {
    static_assert(WM * WN == kThreads / 64 && WM * TM * 32 == kTile && WN * TN * 32 == kTile, "tile");
    static_assert(sizeof(LdsStepU) * 2 >= (kThreads / 64) * 16384, "epilogue staging");
    constexpr bool kT = kBF16Out;          // accumulator layout suited to each epilogue
    __shared__ LdsStepU st[2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const uint32_t nbm = (M + kTile - 1) / kTile, nbn = (N + kTile - 1) / kTile;
    const int nk_all = (K + kBK - 1) / kBK;
    uint32_t tile = blockIdx.x;
    int kb = 0, nk = nk_all;
    const bool split = blockIdx.x >= full;           // uniform over the workgroup
    if (split) {
        const uint32_t u = blockIdx.x - full, j = u % splits;
        tile = full + u / splits;
        kb = (int)(((int64_t)j * nk_all) / splits);
        nk = (int)(((int64_t)(j + 1) * nk_all) / splits) - kb;
    }
    uint32_t bm, bn;
    tile_coords(tile, nbm, nbn, bm, bn);
    const int64_t m0 = (int64_t)bm * kTile, n0 = (int64_t)bn * kTile;

    float16v acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    Addr addr;
    addr.init(A, B, m0, n0, K, tid, kb);
    FetchU fa = addr.fetch(0, nk);
    store_step_u(st[0], fa, tid);
    FetchU fb = addr.fetch(1, nk);
    Frags<TM, TN> f0, f1;
#pragma unroll
    for (int i = 0; i < TM; ++i) f1.a[i] = half8{};
#pragma unroll
    for (int j = 0; j < TN; ++j) f1.b[j] = half8{};
    lds_barrier();
    read_frags<TM, TN>(st[0], f0, wm, wn, lane, 0);
    // Two steps per trip so that the register sets and LDS buffers have fixed roles:
    // step kt computes st[kt % 2], fetches step kt + 2 and stores step kt + 1.  An odd last
    // step is peeled off after the loop.  The loop body has no branches (fetches past the end
    // are harmless re-reads, their stores go to a buffer nobody reads again), so the compiler's
    // wait counts stay exact and no wave waits for a fetch before the step that stores it.
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        fa = addr.fetch(kt + 2, nk);
        step_pipe<TM, TN, kT>(st[0], st[1], fb, true, acc, f0, f1, wm, wn, lane, tid);
        lds_barrier();
        read_frags<TM, TN>(st[1], f0, wm, wn, lane, 0);
        fb = addr.fetch(kt + 3, nk);
        step_pipe<TM, TN, kT>(st[1], st[0], fa, true, acc, f0, f1, wm, wn, lane, tid);
        lds_barrier();
        read_frags<TM, TN>(st[0], f0, wm, wn, lane, 0);
    }
    if (kt < nk) step_pipe<TM, TN, kT>(st[0], st[1], fb, false, acc, f0, f1, wm, wn, lane, tid);
    mfma_frags<TM, TN, kT>(f1, acc);                   // sub-step 3 of the last step

    if (split) {
        store_partial<TM, TN, kT>(acc, lane, wm * TM * 32, wn * TN * 32,
                                  ws + (size_t)(blockIdx.x - full) * (kTile * kTile));
        return;
    }
    const float alpha = (*sdA) * (*sdB);
    const int64_t r0 = m0 + wm * TM * 32, c0 = n0 + wn * TN * 32;
    if constexpr (kBF16Out) {
        // staged through the (now idle) step buffers, 16 KiB per wave
        const bool vec = (reinterpret_cast<uintptr_t>(C) & 15u) == 0 && (ldc * 2) % 16 == 0;
        __syncthreads();                    // every wave has finished reading the step buffers
        uint8_t* reg = reinterpret_cast<uint8_t*>(&st[0]) + wave * 16384;
        epilogue_bf16<TM, TN>(acc, alpha, reg, lane, r0, c0, M, N, reinterpret_cast<uint16_t*>(C),
                              ldc, vec);
    } else {
        epilogue_f32<TM, TN>(acc, alpha, lane, r0, c0, M, N, reinterpret_cast<float*>(C), ldc);
    }
}

template <int WM, int WN, int TM, int TN>
static void launch_gemm(const OperandDesc& a, const OperandDesc& b, int M, int N, int K,
                        const float* sdA, const float* sdB, void* c, bool bf16, int64_t ldc,
                        const SplitPlan& plan, float* ws, hipStream_t st) {
    const dim3 grid(plan.full + plan.tail * plan.splits), block(kThreads);
    const bool fast = K % kBK == 0;
#define NVFP4_GEMM_LAUNCH(BF, ADDR)                                                               \
    hipLaunchKernelGGL((k_gemm_nvfp4<WM, WN, TM, TN, BF, ADDR>), grid, block, 0, st, a, b, M, N, \
                       K, sdA, sdB, c, ldc, plan.full, plan.splits, ws)
    if (bf16) {
        if (fast) NVFP4_GEMM_LAUNCH(true, FastAddrU); else NVFP4_GEMM_LAUNCH(true, GuardedAddrU);
    } else {
        if (fast) NVFP4_GEMM_LAUNCH(false, FastAddrU); else NVFP4_GEMM_LAUNCH(false, GuardedAddrU);
    }
#undef NVFP4_GEMM_LAUNCH
    launch_splitk_fixup(plan, ws, M, N, sdA, sdB, c, bf16, ldc, st);
}

// Argument checks shared by the GEMM entry points; on success fills the operand descriptors.
static nvfp4_status check_gemm(const nvfp4_tensor* a, const nvfp4_tensor* b, const void* c,
                               nvfp4_dtype c_dt, int64_t ldc) {
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
    if (((M + kTile - 1) / kTile) * ((N + kTile - 1) / kTile) >= (1ll << 31)) return NVFP4_ERR_SHAPE;
    return NVFP4_OK;
}

// plan: the split plan to run (a plan with tail == 0 runs every tile whole); ws: its partials.
static nvfp4_status run_gemm(const nvfp4_tensor* a, const nvfp4_tensor* b, void* c,
                             nvfp4_dtype c_dt, int64_t ldc, const SplitPlan& plan, float* ws,
                             hipStream_t st) {
    const int64_t M = a->rows, N = b->rows, K = a->cols;
    if (M == 0 || N == 0) return NVFP4_OK;
    if (K == 0) {                                  // no codes to read (they may be null)
        launch_zero_c(c, c_dt == NVFP4_BF16, ldc, (int)M, (int)N, st);
        return launch_status();
    }
    const OperandDesc da{a->codes, a->scales, M, 0};
    const OperandDesc db{b->codes, b->scales, N, b->layout == NVFP4_BLK_16x16 ? 1 : 0};
    launch_gemm<2, 4, 4, 2>(da, db, (int)M, (int)N, (int)K, a->s_dec, b->s_dec, c,
                            c_dt == NVFP4_BF16, ldc, plan, ws, st);
    return launch_status();
}

// Scratch of the allocation-free entry point: the split partial tiles, at most 256 of 256 x 256
// fp32 (64 MiB), in one array per device that lives as long as the process.  Host code uses
// only the device address that hipGetSymbolAddress returns for the current device, looked up
// on the first call on that device and kept per device.
constexpr size_t kScratchBytes = (size_t)256 * kTile * kTile * sizeof(float);
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch_ptr[kMaxDevices];

static float* scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return static_cast<float*>(p);
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" nvfp4_status nvfp4_gemm(const nvfp4_tensor* a, const nvfp4_tensor* b, void* c,
                                   nvfp4_dtype c_dt, int64_t ldc, void* stream) {
    const nvfp4_status s = check_gemm(a, b, c, c_dt, ldc);
    if (s) return s;
    const SplitPlan whole{(uint32_t)(((a->rows + kTile - 1) / kTile) * ((b->rows + kTile - 1) / kTile)),
                          0, 1, 0};
    return run_gemm(a, b, c, c_dt, ldc, whole, nullptr, as_stream(stream));
}

extern "C" nvfp4_status nvfp4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, size_t* bytes) {
    if (!bytes) return NVFP4_ERR_NULL;
    if (M < 0 || N < 0 || K < 0 || M >= (1ll << 31) || N >= (1ll << 31) || K >= (1ll << 31))
        return NVFP4_ERR_SHAPE;
    *bytes = (M == 0 || N == 0 || K == 0) ? 0 : plan_split(M, N, K, device_cus(), kBK, kMinSplitSteps).ws_bytes;
    return NVFP4_OK;
}

extern "C" nvfp4_status nvfp4_gemm_ws(const nvfp4_tensor* a, const nvfp4_tensor* b, void* c,
                                      nvfp4_dtype c_dt, int64_t ldc, void* workspace,
                                      size_t ws_bytes, void* stream) {
    const nvfp4_status s = check_gemm(a, b, c, c_dt, ldc);
    if (s) return s;
    if (workspace && !aligned16(workspace)) return NVFP4_ERR_ALIGN;
    SplitPlan plan = plan_split(a->rows, b->rows, a->cols, device_cus(), kBK, kMinSplitSteps);
    if (plan.tail && (!workspace || ws_bytes < plan.ws_bytes))
        plan = SplitPlan{plan.full + plan.tail, 0, 1, 0};        // too small: whole tiles only
    return run_gemm(a, b, c, c_dt, ldc, plan, static_cast<float*>(workspace), as_stream(stream));
}

extern "C" nvfp4_status nvfp4_gemm_ws_noalloc(const nvfp4_tensor* a, const nvfp4_tensor* b, void* c,
                                              nvfp4_dtype c_dt, int64_t ldc, void* stream) {
    const nvfp4_status s = check_gemm(a, b, c, c_dt, ldc);
    if (s) return s;
    const SplitPlan plan = plan_split(a->rows, b->rows, a->cols, device_cus(), kBK, kMinSplitSteps);
    if (plan.ws_bytes > kScratchBytes) return NVFP4_ERR_SCRATCH;
    float* ws = nullptr;
    if (plan.tail && !(ws = scratch_ptr())) return NVFP4_ERR_LAUNCH;
    return run_gemm(a, b, c, c_dt, ldc, plan, ws, as_stream(stream));
}
