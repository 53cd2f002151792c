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
//   global -> VGPR prefetch two steps ahead (one 16-byte code chunk of A and of B and one
//   dword of four scale bytes per thread and step)
//   -> LDS, double buffered: codes [256][32 B] per operand with the two 16-byte halves swapped
//      on rows with bit 2 set (spreads eight consecutive rows over all banks), scales as fp16
//      pairs converted with v_cvt_scalef32_pk_f16_fp8
//   -> each wave reads 16 B (32 codes) per 32-row MFMA tile and lane, unpacks 8 codes at a
//      time with v_cvt_scalef32_pk_f16_fp4 and multiplies them by their block scale (v_pk_mul_f16)
//   -> v_mfma_f32_32x32x16_f16.
// The barrier between steps orders LDS only, so global prefetches stay in flight across it.
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

// Workgroup barrier that orders LDS accesses only: outstanding global loads are not waited for.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
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

// One K step of one workgroup in LDS.
struct alignas(16) LdsStep {
    uint8_t a[kTile * kRowBytes];
    uint8_t b[kTile * kRowBytes];
    uint2 sa[kTile];        // fp16 scale pairs: {s0,s1}, {s2,s3} per row
    uint2 sb[kTile];
};

// What one thread fetches for one K step: A code chunk (thread t: row t/2, half t%2), B code
// chunk (same), and the four scale bytes of row t (t < 256: A) or row t-256 (B).
struct Fetch {
    uint4 a, b;
    uint32_t s;
};

// Global addressing for K % 64 == 0: per-thread pointers (rows past the end clamped to the last
// row, whose results are never stored), advanced by one step per fetch.
struct FastAddr {
    const uint8_t *pa, *pb, *ps;
    __device__ __forceinline__ void init(const OperandDesc& A, const OperandDesc& B, int64_t m0,
                                         int64_t n0, int K, int t) {
        const int r = t >> 1, h = t & 1;
        int64_t ra = m0 + r, rb = n0 + r;
        ra = ra < A.rows - 1 ? ra : A.rows - 1;
        rb = rb < B.rows - 1 ? rb : B.rows - 1;
        pa = A.codes + ra * (K / 2) + h * 16;
        pb = B.codes + rb * (K / 2) + h * 16;
        const OperandDesc& S = t < kTile ? A : B;
        int64_t rs = (t < kTile ? m0 : n0) + (t & (kTile - 1));
        rs = rs < S.rows - 1 ? rs : S.rows - 1;
        ps = S.scales + (S.tiled ? rs / 16 : rs) * (K / 16);
    }
    __device__ __forceinline__ Fetch fetch(int) {
        Fetch f;
        f.a = *reinterpret_cast<const uint4*>(pa);
        f.b = *reinterpret_cast<const uint4*>(pb);
        f.s = *reinterpret_cast<const uint32_t*>(ps);
        pa += kRowBytes;
        pb += kRowBytes;
        ps += 4;
        return f;
    }
};

// Guarded addressing for any K % 16 == 0: zero codes past K and past the last row.
struct GuardedAddr {
    OperandDesc A, B;
    int64_t m0, n0;
    int K, t;
    __device__ __forceinline__ void init(const OperandDesc& a, const OperandDesc& b, int64_t m,
                                         int64_t n, int k, int tid) {
        A = a; B = b; m0 = m; n0 = n; K = k; t = tid;
    }
    __device__ __forceinline__ uint4 chunk(const OperandDesc& op, int64_t row, int k0) const {
        const int kk = k0 + (t & 1) * 32;
        if (row >= op.rows || kk >= K) return make_uint4(0, 0, 0, 0);
        const uint8_t* p = op.codes + row * (K / 2) + kk / 2;
        if (kk + 32 <= K) return *reinterpret_cast<const uint4*>(p);
        const uint2 v = *reinterpret_cast<const uint2*>(p);          // K % 32 == 16 tail
        return make_uint4(v.x, v.y, 0, 0);
    }
    __device__ __forceinline__ Fetch fetch(int kt) {
        Fetch f;
        const int k0 = kt * kBK;
        f.a = chunk(A, m0 + (t >> 1), k0);
        f.b = chunk(B, n0 + (t >> 1), k0);
        const OperandDesc& S = t < kTile ? A : B;
        const int64_t row = (t < kTile ? m0 : n0) + (t & (kTile - 1));
        f.s = 0;
        if (row < S.rows) {
            const int64_t nkb = K / 16;
            const uint8_t* sp = S.scales + (S.tiled ? row / 16 : row) * nkb;
            const int kb0 = k0 / 16;
#pragma unroll
            for (int b = 0; b < 4; ++b)
                if (kb0 + b < nkb) f.s |= (uint32_t)sp[kb0 + b] << (8 * b);
        }
        return f;
    }
};

// Physical 16-byte half of logical half h of row r: swapped when bits 2 and 3 of r differ, so
// that any 8 or 16 consecutive rows read at the same logical half hit distinct bank groups.
__device__ __forceinline__ int half_swz(int r, int h) { return (h ^ (r >> 2) ^ (r >> 3)) & 1; }

__device__ __forceinline__ void store_step(LdsStep& st, Fetch f, int t) {
    const int r = t >> 1, h = half_swz(r, t & 1);
    *reinterpret_cast<uint4*>(&st.a[r * kRowBytes + h * 16]) = f.a;
    *reinterpret_cast<uint4*>(&st.b[r * kRowBytes + h * 16]) = f.b;
    const half2v lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.s, 1.0f, false);
    const half2v hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.s, 1.0f, true);
    const uint2 v = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
    if (t < kTile) st.sa[t] = v; else st.sb[t - kTile] = v;
}

template <int WN, int TM, int TN>
__device__ __forceinline__ void compute_step(const LdsStep& st, float16v (&acc)[TM][TN], int wm,
                                             int wn, int lane) {
    const int lrow = lane & 31, h = lane >> 5;
    uint4 fa[TM], fb[TN];
    half2v xa[TM], xb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int r = wm * TM * 32 + i * 32 + lrow;
        fa[i] = *reinterpret_cast<const uint4*>(&st.a[r * kRowBytes + half_swz(r, h) * 16]);
        xa[i] = __builtin_bit_cast(half2v, reinterpret_cast<const uint32_t*>(&st.sa[r])[h]);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int r = wn * TN * 32 + j * 32 + lrow;
        fb[j] = *reinterpret_cast<const uint4*>(&st.b[r * kRowBytes + half_swz(r, h) * 16]);
        xb[j] = __builtin_bit_cast(half2v, reinterpret_cast<const uint32_t*>(&st.sb[r])[h]);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        // unpack this sub-step's A fragments, then each B fragment right before its MFMAs, so
        // few unpacked operands are live at once
        half8 va[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const uint32_t w = s == 0 ? fa[i].x : s == 1 ? fa[i].y : s == 2 ? fa[i].z : fa[i].w;
            const _Float16 sc = xa[i][s >> 1];
            va[i] = unpack8(w, half2v{sc, sc});
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const uint32_t w = s == 0 ? fb[j].x : s == 1 ? fb[j].y : s == 2 ? fb[j].z : fb[j].w;
            const _Float16 sc = xb[j][s >> 1];
            const half8 vb = unpack8(w, half2v{sc, sc});
#pragma unroll
            for (int i = 0; i < TM; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[i], vb, acc[i][j], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// ---- unpack-once variant -------------------------------------------------------------------
// The loading threads turn their code chunk into scaled fp16 right away and store it to LDS,
// so every element is unpacked once per workgroup instead of once per wave that reads it;
// waves then read MFMA-ready fp16 fragments.  LDS per step: [256][64] fp16 per operand, with
// the eight 16-byte chunks of a row permuted by chunk ^ (r & 7) ^ ((r >> 3) & 1) so that 8 or
// 16 consecutive rows reading the same logical chunk hit distinct bank groups.
struct alignas(16) LdsStepU {
    _Float16 a[kTile * kBK];
    _Float16 b[kTile * kBK];
};

struct FetchU {
    uint4 a, b;
    uint32_t s;     // A's two scale bytes (low half) and B's (high half) for this chunk
};

__device__ __forceinline__ int chunk_swz(int r, int q) { return q ^ (r & 7) ^ ((r >> 3) & 1); }

struct FastAddrU {
    const uint8_t *pa, *pb, *psa, *psb;
    __device__ __forceinline__ void init(const OperandDesc& A, const OperandDesc& B, int64_t m0,
                                         int64_t n0, int K, int t) {
        const int r = t >> 1, h = t & 1;
        int64_t ra = m0 + r, rb = n0 + r;
        ra = ra < A.rows - 1 ? ra : A.rows - 1;
        rb = rb < B.rows - 1 ? rb : B.rows - 1;
        pa = A.codes + ra * (K / 2) + h * 16;
        pb = B.codes + rb * (K / 2) + h * 16;
        psa = A.scales + (A.tiled ? ra / 16 : ra) * (K / 16) + h * 2;
        psb = B.scales + (B.tiled ? rb / 16 : rb) * (K / 16) + h * 2;
    }
    __device__ __forceinline__ FetchU fetch(int) {
        FetchU f;
        f.a = *reinterpret_cast<const uint4*>(pa);
        f.b = *reinterpret_cast<const uint4*>(pb);
        f.s = (uint32_t)*reinterpret_cast<const uint16_t*>(psa) |
              ((uint32_t)*reinterpret_cast<const uint16_t*>(psb) << 16);
        pa += kRowBytes;
        pb += kRowBytes;
        psa += 4;
        psb += 4;
        return f;
    }
};

struct GuardedAddrU {
    OperandDesc A, B;
    int64_t m0, n0;
    int K, t;
    __device__ __forceinline__ void init(const OperandDesc& a, const OperandDesc& b, int64_t m,
                                         int64_t n, int k, int tid) {
        A = a; B = b; m0 = m; n0 = n; K = k; t = tid;
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
    __device__ __forceinline__ FetchU fetch(int kt) {
        FetchU f;
        const int k0 = kt * kBK;
        const int64_t ra = m0 + (t >> 1), rb = n0 + (t >> 1);
        f.a = chunk(A, ra, k0);
        f.b = chunk(B, rb, k0);
        f.s = scales2(A, ra, k0) | (scales2(B, rb, k0) << 16);
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
    const half2v sa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.s, 1.0f, false);
    const half2v sb = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.s, 1.0f, true);
    store_one_u(&st.a[r * kBK], r, h, f.a, sa);
    store_one_u(&st.b[r * kBK], r, h, f.b, sb);
}

template <int TM, int TN>
__device__ __forceinline__ void read_frags_u(const LdsStepU& st, half8 (&va)[TM], half8 (&vb)[TN],
                                             int wm, int wn, int lane, int s) {
    const int lrow = lane & 31, h = lane >> 5;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int r = wm * TM * 32 + i * 32 + lrow;
        va[i] = *reinterpret_cast<const half8*>(&st.a[r * kBK + 8 * chunk_swz(r, 4 * h + s)]);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int r = wn * TN * 32 + j * 32 + lrow;
        vb[j] = *reinterpret_cast<const half8*>(&st.b[r * kBK + 8 * chunk_swz(r, 4 * h + s)]);
    }
}

// One K step: MFMAs on `cur` and, interleaved with them, the unpack/store of the next step's
// fetched codes into `nxt` (a quarter after each sub-step's MFMAs), so that the VALU and LDS
// work overlaps the matrix-core work instead of running between barriers.  Fragments for
// sub-step s + 1 are read while sub-step s computes.
template <int TM, int TN>
__device__ __forceinline__ void step_u(const LdsStepU& cur, LdsStepU& nxt, const FetchU& f,
                                       bool do_store, float16v (&acc)[TM][TN], int wm, int wn,
                                       int lane, int tid) {
    const int r = tid >> 1, h = tid & 1;
    const half2v sa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.s, 1.0f, false);
    const half2v sb = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.s, 1.0f, true);
    const uint32_t wa[4] = {f.a.x, f.a.y, f.a.z, f.a.w}, wb[4] = {f.b.x, f.b.y, f.b.z, f.b.w};
    half8 va[2][TM], vb[2][TN];
    read_frags_u<TM, TN>(cur, va[0], vb[0], wm, wn, lane, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int c = s & 1;
        if (s < 3) read_frags_u<TM, TN>(cur, va[c ^ 1], vb[c ^ 1], wm, wn, lane, s + 1);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[c][i], vb[c][j], acc[i][j], 0, 0, 0);
        if (do_store) {
            const _Float16 xa = sa[s >> 1], xb = sb[s >> 1];
            const int p = 8 * chunk_swz(r, 4 * h + s);
            *reinterpret_cast<half8*>(&nxt.a[r * kBK + p]) = unpack8(wa[s], half2v{xa, xa});
            *reinterpret_cast<half8*>(&nxt.b[r * kBK + p]) = unpack8(wb[s], half2v{xb, xb});
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Pipelines shared by both variants: register prefetch two steps ahead, LDS double buffer.
struct PackedMode {
    using Step = LdsStep;
    template <int WN, int TM, int TN>
    static __device__ __forceinline__ void compute(const Step& st, float16v (&acc)[TM][TN], int wm,
                                                   int wn, int lane) {
        compute_step<WN, TM, TN>(st, acc, wm, wn, lane);
    }
    template <typename F>
    static __device__ __forceinline__ void store(Step& st, F f, int t) { store_step(st, f, t); }
    template <int WN, int TM, int TN, typename F>
    static __device__ __forceinline__ void compute_store(const Step& cur, Step& nxt, const F& f,
                                                         bool do_store, float16v (&acc)[TM][TN],
                                                         int wm, int wn, int lane, int tid) {
        compute_step<WN, TM, TN>(cur, acc, wm, wn, lane);
        if (do_store) store_step(nxt, f, tid);
    }
};

struct UnpackedMode {
    using Step = LdsStepU;
    template <int WN, int TM, int TN>
    static __device__ __forceinline__ void compute(const Step& st, float16v (&acc)[TM][TN], int wm,
                                                   int wn, int lane) {
        FetchU none{};
        step_u<TM, TN>(st, const_cast<Step&>(st), none, false, acc, wm, wn, lane, 0);
    }
    template <typename F>
    static __device__ __forceinline__ void store(Step& st, F f, int t) { store_step_u(st, f, t); }
    template <int WN, int TM, int TN, typename F>
    static __device__ __forceinline__ void compute_store(const Step& cur, Step& nxt, const F& f,
                                                         bool do_store, float16v (&acc)[TM][TN],
                                                         int wm, int wn, int lane, int tid) {
        step_u<TM, TN>(cur, nxt, f, do_store, acc, wm, wn, lane, tid);
    }
};

// Waves are arranged WM x WN over the 256 x 256 tile, each owning TM x TN MFMA tiles of 32x32.
template <int WM, int WN, int TM, int TN, bool kBF16Out, typename Mode, typename Addr>
__global__ void __launch_bounds__(kThreads)
k_gemm_nvfp4(OperandDesc A, OperandDesc B, int M, int N, int K, const float* __restrict__ sdA,
             const float* __restrict__ sdB, void* __restrict__ C, int64_t ldc) {
    static_assert(WM * WN == kThreads / 64 && WM * TM * 32 == kTile && WN * TN * 32 == kTile, "tile");
    __shared__ typename Mode::Step st[2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const uint32_t nbm = (M + kTile - 1) / kTile, nbn = (N + kTile - 1) / kTile;
    uint32_t bm, bn;
    tile_coords(blockIdx.x, nbm, nbn, bm, bn);
    const int64_t m0 = (int64_t)bm * kTile, n0 = (int64_t)bn * kTile;

    float16v acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    Addr addr;
    addr.init(A, B, m0, n0, K, tid);
    const int nk = (K + kBK - 1) / kBK;
    auto f0 = addr.fetch(0), f1 = f0;
    Mode::store(st[0], f0, tid);
    if (nk > 1) f1 = addr.fetch(1);
    lds_barrier();
    // Two steps per trip so that the register sets and LDS buffers have fixed roles:
    // step kt computes st[kt % 2], fetches step kt + 2 and stores step kt + 1.  An odd last
    // step is peeled off after the loop.
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        if (kt + 2 < nk) f0 = addr.fetch(kt + 2);
        Mode::template compute_store<WN, TM, TN>(st[0], st[1], f1, true, acc, wm, wn, lane, tid);
        lds_barrier();
        if (kt + 3 < nk) f1 = addr.fetch(kt + 3);
        Mode::template compute_store<WN, TM, TN>(st[1], st[0], f0, kt + 2 < nk, acc, wm, wn, lane, tid);
        lds_barrier();
    }
    if (kt < nk) Mode::template compute<WN, TM, TN>(st[0], acc, wm, wn, lane);

    // epilogue: D element r of lane l sits at row 8*(r/4) + 4*(l/32) + r%4, column l%32
    const float alpha = (*sdA) * (*sdB);
    const int lrow = lane & 31, h = lane >> 5;
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

template <int WM, int WN, int TM, int TN, bool kUnpackOnce>
static void launch_gemm(const OperandDesc& a, const OperandDesc& b, int M, int N, int K,
                        const float* sdA, const float* sdB, void* c, bool bf16, int64_t ldc,
                        hipStream_t st) {
    const uint32_t nbm = (M + kTile - 1) / kTile, nbn = (N + kTile - 1) / kTile;
    const dim3 grid(nbm * nbn), block(kThreads);
    const bool fast = K % kBK == 0;
    using Mode = typename std::conditional<kUnpackOnce, UnpackedMode, PackedMode>::type;
    using AF = typename std::conditional<kUnpackOnce, FastAddrU, FastAddr>::type;
    using AG = typename std::conditional<kUnpackOnce, GuardedAddrU, GuardedAddr>::type;
#define NVFP4_GEMM_LAUNCH(BF, ADDR)                                                               \
    hipLaunchKernelGGL((k_gemm_nvfp4<WM, WN, TM, TN, BF, Mode, ADDR>), grid, block, 0, st, a, b, M, \
                       N, K, sdA, sdB, c, ldc)
    if (bf16) {
        if (fast) NVFP4_GEMM_LAUNCH(true, AF); else NVFP4_GEMM_LAUNCH(true, AG);
    } else {
        if (fast) NVFP4_GEMM_LAUNCH(false, AF); else NVFP4_GEMM_LAUNCH(false, AG);
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
    launch_gemm<2, 4, 4, 2, true>(da, db, (int)M, (int)N, (int)K, a->s_dec, b->s_dec, c,
                            c_dt == NVFP4_BF16, ldc, as_stream(stream));
    return launch_status();
}
