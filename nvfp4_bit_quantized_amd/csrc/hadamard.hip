// hadamard.hip -- random Hadamard transform + transpose + NVFP4 quantization of the
// weight-gradient operands, and the amax of the transformed tensor, for gfx950.
//
// [P1] "Entrenamiento de Modelos de Lenguaje con 4 Bits de Precision", Metodologia de
// Entrenamiento: the recipe applies random Hadamard transforms.  Here: for every feature f and
// 16-token chunk c of x [T x F], y = (1/4) H16 D x[16c..16c+15, f] with H16 the Sylvester
// Hadamard matrix and D a random +-1 diagonal; y is quantized with 1x16 blocks along tokens and
// written feature-major ([F x T]) so that tokens form the contiguous K of the wgrad GEMM.
//
// Thread mapping: a thread owns 8 consecutive features (one 16-byte bf16 load per token row)
// and one 16-token chunk, so it holds the 16x8 input tile in registers and runs 8 independent
// 16-point fast Walsh-Hadamard transforms.  The quantizers (k_dual_quant, k_mx_quant_t) place
// 32 feature groups side by side in a wave (256 features: 512-byte reads of two token rows per
// load), stage their results in LDS and write whole tile rows.  The quantizer with noise sums
// (k_rht_quant) keeps the direct mapping of 8 feature groups x 8 chunks per wave and stores
// from the threads.
//
// The staged tiling also serves the transposing MXFP4 quantizer of the comparison format (no
// transform; 32-token blocks made of two adjacent chunks held by lanes l and l + 32).

#include "device_codecs.hpp"
#include "host_util.hpp"
#include "noise.hpp"

namespace nvfp4 {

constexpr int kRhtThreads = 256;
constexpr int kFeatPerBlock = 64;                  // 8 feature groups of 8
constexpr int kChunksPerBlock = kRhtThreads / 8;   // 32 chunks = 512 tokens

// 16 token rows x 8 features of one thread, as raw 32-bit words (bf16: 4 per row, fp32: 8).
template <typename T> struct Tile16x8;

template <> struct Tile16x8<uint16_t> {
    uint4 w[16];
    template <bool kNT = true>
    __device__ __forceinline__ void load(const uint16_t* p, int64_t ld) {
#pragma unroll
        for (int i = 0; i < 16; ++i) w[i] = load16<kNT>(p + i * ld);
    }
    __device__ __forceinline__ float get(int i, int f) const {
        const uint32_t v = f < 2 ? w[i].x : f < 4 ? w[i].y : f < 6 ? w[i].z : w[i].w;
        return (f & 1) ? bf16_hi(v) : bf16_lo(v);
    }
    // Row i times d_i (bit i of sign_mask set: d_i = -1), on the packed words: one xor per two
    // elements, bit-identical to negating each unpacked value.
    __device__ __forceinline__ void apply_signs(uint32_t sign_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t s = ((sign_mask >> i) & 1u) ? 0x80008000u : 0u;
            w[i].x ^= s; w[i].y ^= s; w[i].z ^= s; w[i].w ^= s;
        }
    }
    // No instruction: the words are marked as changed, so that values unpacked before this point
    // are not kept live to be reused after it (the tile is smaller packed than unpacked).
    __device__ __forceinline__ void fence() {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            asm volatile("" : "+v"(w[i].x), "+v"(w[i].y), "+v"(w[i].z), "+v"(w[i].w));
    }
};

template <> struct Tile16x8<float> {
    float4 a[16], b[16];
    template <bool kNT = true>
    __device__ __forceinline__ void load(const float* p, int64_t ld) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint4 u = load16<kNT>(p + i * ld), v = load16<kNT>(p + i * ld + 4);
            a[i] = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                               __uint_as_float(u.w));
            b[i] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                               __uint_as_float(v.w));
        }
    }
    __device__ __forceinline__ float get(int i, int f) const {
        const float4& v = f < 4 ? a[i] : b[i];
        const int g = f & 3;
        return g == 0 ? v.x : g == 1 ? v.y : g == 2 ? v.z : v.w;
    }
    __device__ __forceinline__ void apply_signs(uint32_t sign_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t s = ((sign_mask >> i) & 1u) << 31;
            float* e[8] = {&a[i].x, &a[i].y, &a[i].z, &a[i].w, &b[i].x, &b[i].y, &b[i].z, &b[i].w};
#pragma unroll
            for (int k = 0; k < 8; ++k) *e[k] = __uint_as_float(__float_as_uint(*e[k]) ^ s);
        }
    }
    __device__ __forceinline__ void fence() {}
};

// Sign mask: bit j set <=> d_j = -1.  Word 0 of Philox4x32-10(key = sign_seed, counter = 0).
__device__ __forceinline__ uint32_t rht_sign_mask(uint64_t sign_seed) {
    return philox4x32_10(0u, 0u, 0u, 0u, (uint32_t)sign_seed, (uint32_t)(sign_seed >> 32)).x & 0xFFFFu;
}

// For the amax only: |H16 D v| as a butterfly network on the unsigned input.  With v = c (.) u (c
// a vector of signs carried per position, starting at c = d), a butterfly on (i, i + h) gives
// c_i (u_i + s u_{i+h}) and c_i (u_i - s u_{i+h}) with s = c_i c_{i+h}: each butterfly is a pair of
// fmas with a sign factor s, and the carried sign of position i + h becomes c_i.  Since s = +-1
// the fma rounds exactly like the add or subtract and RNE commutes with negation, so |u_i| equals
// |(H16 D v)_i| bit for bit (only the sign of an exact zero can differ, which the amax ignores).
// The quantizer, whose codes keep the sign of zero, uses rht16 below.  The sign factors are the
// same for every thread and kept as integer bit patterns so that they live in scalar registers.
struct RhtPlan {
    uint32_t s[32];     // +-1.0f bit patterns, stage by stage (the amax uses the first 24)
};

__device__ __forceinline__ RhtPlan rht_plan(uint32_t sign_mask) {
    RhtPlan p;
    sign_mask = __builtin_amdgcn_readfirstlane(sign_mask);    // the same in every lane
    uint32_t c[16];     // sign bit of c_i
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = ((sign_mask >> i) & 1u) << 31;
    int k = 0;
#pragma unroll
    for (int hs = 1; hs < 16; hs <<= 1)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if ((i & hs) == 0) {
                p.s[k++] = 0x3F800000u | (c[i] ^ c[i + hs]);
                c[i + hs] = c[i];
            }
    return p;
}

// max_i |(H16 D v)_i| (the 1/4 not applied), v overwritten.  The first three stages run the
// butterfly network above.  In the last stage (pairs i, i + 8) the two results a + s b and
// a - s b (s = +-1) have magnitudes |a| + |b| and ||a| - |b||; rounding is monotonic and
// symmetric, so the larger rounded magnitude is fl(|a| + |b|) bit for bit, and the last stage
// reduces to eight additions of magnitudes.
__device__ __forceinline__ float hd16_absmax(float* v, const RhtPlan& p) {
    int k = 0;
#pragma unroll
    for (int hs = 1; hs < 8; hs <<= 1)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if ((i & hs) == 0) {
                const float a = v[i], b = v[i + hs];
                const float sk = __uint_as_float(p.s[k]);
                v[i] = __builtin_fmaf(sk, b, a);
                v[i + hs] = __builtin_fmaf(-sk, b, a);
                ++k;
            }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, __builtin_fabsf(v[i]) + __builtin_fabsf(v[i + 8]));
    return m;
}

// In place: v <- H16 v, butterflies in the order h = 1, 2, 4, 8.
__device__ __forceinline__ void h16(float* v) {
#pragma unroll
    for (int hs = 1; hs < 16; hs <<= 1)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if ((i & hs) == 0) {
                const float a = v[i], b = v[i + hs];
                v[i] = a + b;
                v[i + hs] = a - b;
            }
}

// In place: v <- (1/4) H16 v, the butterflies then one multiply by 1/4 each.  The random signs D
// are applied before, to the loaded tile (apply_signs), so that the whole is (1/4) H16 D x with D
// applied first.
__device__ __forceinline__ void h16_quarter(float* v) {
    h16(v);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0.25f * v[i];
}

__global__ void k_scalars_rht(const float* src, float* amax_out, float* sdec_out) {
    const float A = *src;
    *amax_out = A;
    *sdec_out = tensor_scales(A).s_dec;
}

struct RhtCoords {
    int64_t f0;      // first feature of the thread
    int64_t c;       // chunk index
    bool valid;
};

__device__ __forceinline__ RhtCoords rht_coords_at(int64_t T, int64_t F, uint32_t bx, uint32_t by) {
    RhtCoords rc;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    rc.f0 = (int64_t)bx * kFeatPerBlock + (lane & 7) * 8;
    rc.c = (int64_t)by * kChunksPerBlock + wave * 8 + (lane >> 3);
    rc.valid = rc.f0 < F && rc.c * 16 < T;
    return rc;
}

// Persistent over (64-feature x 512-token) tiles, at most kRhtAmaxBlocks workgroups, each
// publishing its maximum once (publish_amax).  The factor 1/4 of the transform is applied to the
// maximum instead of to every element: scaling by 1/4 and fp32 rounding are both monotonic, so
// fl(max|t| / 4) = max fl(|t| / 4).
// A workgroup of rht_amax_sub<T> x 256 threads works on that many tiles at a time.  Each thread
// loads the next tile while it transforms the current one (bf16; fp32 tiles take twice the
// registers and are not double-buffered).  Coordinates past the edges are clamped to the last
// valid token chunk / feature group / tile: the duplicates they read leave a maximum unchanged, so
// every load is unconditional.  With kPlain the same pass also takes the amax of x itself (for
// the fused dual-orientation quantizer).
// The amax tiles are 256 features x 8 chunks per 256 threads: a wave reads 512 contiguous bytes
// of each of two token rows per load (instead of 128 bytes of eight), which suits HBM better.
constexpr int kRhtAmaxBlocks = 256;
constexpr int kAmaxFeat = 256, kAmaxChunks = 8;
template <typename T> constexpr int rht_amax_sub() { return 2; }

template <typename T, bool kPlain>
__device__ __forceinline__ void rht_amax_tile(const Tile16x8<T>& t16, const RhtPlan& plan, float& m,
                                              float& mp) {
#pragma unroll
    for (int f = 0; f < 8; ++f) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = t16.get(i, f);
        if constexpr (kPlain) {
#pragma unroll
            for (int i = 0; i < 16; ++i) mp = fmaxf(mp, fabsf(v[i]));
        }
        m = fmaxf(m, hd16_absmax(v, plan));
    }
}

template <typename T, bool kPlain, bool kNT, int kRhtAmaxSub = rht_amax_sub<T>()>
__global__ void __launch_bounds__(kRhtThreads * kRhtAmaxSub)
k_rht_amax(const T* __restrict__ x, int64_t Tn, int64_t F, int64_t ld, uint64_t sign_seed,
           float* amax_out, float* amax_plain_out, uint32_t tiles, FastDiv tiles_per_row) {
    const RhtPlan plan = rht_plan(rht_sign_mask(sign_seed));
    const int lane = threadIdx.x & 63, wave = (threadIdx.x >> 6) % (kRhtThreads / 64);
    const uint32_t sub = threadIdx.x / kRhtThreads;
    const int64_t last_c = Tn / 16 - 1, last_f0 = F - 8;
    auto tile_ptr = [&](uint32_t tile) {
        tile = tile < tiles ? tile : tiles - 1;
        const uint32_t ty = fastdiv(tile, tiles_per_row), tx = tile - ty * tiles_per_row.d;
        int64_t f0 = (int64_t)tx * kAmaxFeat + (lane & 31) * 8;
        int64_t c = (int64_t)ty * kAmaxChunks + wave * 2 + (lane >> 5);
        f0 = f0 < last_f0 ? f0 : last_f0;
        c = c < last_c ? c : last_c;
        return x + c * 16 * ld + f0;
    };
    float m = 0.0f, mp = 0.0f;
    const uint32_t stride = gridDim.x * kRhtAmaxSub;
    uint32_t tile = blockIdx.x * kRhtAmaxSub + sub;
    if constexpr (sizeof(T) == 2) {
        // two register sets with fixed roles; a clamped tile past the end is a harmless duplicate
        Tile16x8<T> ta, tb;
        float mb = 0.0f, mpb = 0.0f;
        ta.template load<kNT>(tile_ptr(tile), ld);
        for (; tile < tiles; tile += 2 * stride) {
            tb.template load<kNT>(tile_ptr(tile + stride), ld);
            __builtin_amdgcn_sched_barrier(0);
            rht_amax_tile<T, kPlain>(ta, plan, m, mp);
            __builtin_amdgcn_sched_barrier(0);
            ta.template load<kNT>(tile_ptr(tile + 2 * stride), ld);
            __builtin_amdgcn_sched_barrier(0);
            rht_amax_tile<T, kPlain>(tb, plan, mb, mpb);
            __builtin_amdgcn_sched_barrier(0);
        }
        m = fmaxf(m, mb);
        mp = fmaxf(mp, mpb);
    } else {
        for (; tile < tiles; tile += stride) {
            Tile16x8<T> cur;
            cur.template load<kNT>(tile_ptr(tile), ld);
            rht_amax_tile<T, kPlain>(cur, plan, m, mp);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        m = fmaxf(m, __shfl_xor(m, off));
        if constexpr (kPlain) mp = fmaxf(mp, __shfl_xor(mp, off));
    }
    m = 0.25f * m;
    constexpr int kWaves = kRhtThreads * kRhtAmaxSub / 64;
    __shared__ float part[2][kWaves];
    if ((threadIdx.x & 63) == 0) {
        part[0][threadIdx.x >> 6] = m;
        part[1][threadIdx.x >> 6] = mp;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = part[0][0], bp = part[1][0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) {
            b = fmaxf(b, part[0][w]);
            bp = fmaxf(bp, part[1][w]);
        }
        publish_amax(amax_out, b);
        if constexpr (kPlain) publish_amax(amax_plain_out, bp);
    }
}

// The transposed copy of one thread's tile (features f0 .. f0 + 7 of the 16 tokens from row0):
// for each feature f, the 16 tokens through (1/4) H16 D, one NVFP4 block of row f0 + f of the
// [F x T] output, handed to emit(f, lo, hi, scale_byte) (codes of tokens 0-7 in lo, 8-15 in hi).
//
// kFold (only while every nonzero encode factor stays >= 2^-124, which a tensor amax A <= 2^120
// ensures): the 1/4 goes into the block's encode factor instead of into each element,
// z = v * fl(enc / 4) for v = H16 D x.  Where v / 4 and enc / 4 are both exact, the two forms
// are the one rounding of v * enc / 4, so z is the same number bit for bit and any rounding
// of it, nearest or stochastic, gives the same code.  enc / 4 is exact above 2^-124.  v / 4 is
// exact for bf16 input: every bf16 value is a multiple of 2^-133 (its smallest subnormal), so
// every butterfly sum is too (below 2^-110 it needs at most 23 bits and is not rounded, above
// it the fp32 spacing is itself a multiple of 2^-133), and v / 4, a multiple of 2^-135, is an
// fp32 number.  For fp32 input v / 4 can round where it is subnormal; then z is below 0.09 in
// both forms (a nonzero block scale needs amax_b * 448 / A >= 2^-10 with A >= 2^-100, and
// enc <= 12 / amax_b), which round to nearest sends to a zero code of v's sign either way, but
// a stochastic rounding of the two could differ.  The block maximum takes the 1/4 after the
// maximum (monotonic, so max fl(|v| / 4) = fl(max |v| / 4)).  One multiply per block replaces
// one per element.
template <typename T, bool kSR, bool kNoise, typename Emit, bool kFold = false>
__device__ __forceinline__ void quant_tile_transposed(const Tile16x8<T>& tile, int64_t f0,
                                                      int64_t row0, int64_t Tn, uint32_t mask,
                                                      const TensorScales& ts, const EncTable& tab,
                                                      uint64_t seed, double& g2, double& e2,
                                                      Emit emit) {
    static_assert(!kFold || (!kNoise && (!kSR || sizeof(T) == 2)),
                  "the folded 1/4 gives the same codes for bf16 input or round to nearest only");
    uint64_t idx = (uint64_t)f0 * (uint64_t)Tn + (uint64_t)row0;    // SR element index
    Tile16x8<T> sgn = tile;
    sgn.apply_signs(__builtin_amdgcn_readfirstlane(mask));     // the same in every lane
#pragma unroll
    for (int f = 0; f < 8; ++f) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = sgn.get(i, f);
        if constexpr (kFold) h16(v); else h16_quarter(v);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
        if constexpr (kFold) m = 0.25f * m;
        uint32_t sb;
        float enc;
        block_scale_tab(m, ts, tab, sb, enc);
        if constexpr (kFold) enc = 0.25f * enc;
        float z[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) z[e] = v[e] * enc;
        uint32_t lo = 0, hi = 0;
        if constexpr (kSR) {
            const u32x4 w0 = sr_words(seed, idx), w1 = sr_words(seed, idx + 8);
            const uint32_t a[4] = {w0.x, w0.y, w0.z, w0.w}, b[4] = {w1.x, w1.y, w1.z, w1.w};
            lo = e2m1_sr_pack8(z, a);
            hi = e2m1_sr_pack8(z + 8, b);
        } else {
            lo = e2m1_rne_pack8(z);
            hi = e2m1_rne_pack8(z + 8);
        }
        emit(f, lo, hi, sb);
        if constexpr (kNoise) block_noise(v, lo, hi, sb, ts, g2, e2);
        idx += (uint64_t)Tn;
    }
}

// The row-wise copy of one thread's tile (features f0 .. f0 + 7 of token rows row0 .. row0 + 15):
// for each row i, its 8 features are one half of a 16-feature NVFP4 block whose other half sits
// in the adjacent lane (lane ^ 1, which holds the same rows and the next or previous 8
// features); the block amax is shared with one DPP lane swap, and emit(i, codes, scale_byte)
// receives the 8 codes (both lanes of a pair get the block's scale byte).  F % 16 == 0, so both
// lanes of a pair are valid or neither is.
template <typename T, bool kSR, typename Emit>
__device__ __forceinline__ void quant_tile_rows(const Tile16x8<T>& tile, int64_t f0, int64_t row0,
                                                int64_t F, const TensorScales& ts,
                                                const EncTable& tab, uint64_t seed, Emit emit) {
    uint64_t idx = (uint64_t)row0 * (uint64_t)F + (uint64_t)f0;          // SR element index
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float y[8];
#pragma unroll
        for (int f = 0; f < 8; ++f) y[f] = tile.get(i, f);
        float m = 0.0f;
#pragma unroll
        for (int f = 0; f < 8; ++f) m = fmaxf(m, fabsf(y[f]));
        // m >= 0: the larger of two non-negative floats is the larger bit pattern
        m = __uint_as_float(max(__float_as_uint(m), __float_as_uint(swap_adjacent(m))));
        uint32_t sb;
        float enc;
        block_scale_tab(m, ts, tab, sb, enc);
        float z[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = y[e] * enc;
        uint32_t packed;
        if constexpr (kSR) {
            const u32x4 w = sr_words(seed, idx);
            const uint32_t words[4] = {w.x, w.y, w.z, w.w};
            packed = e2m1_sr_pack8(z, words);
        } else {
            packed = e2m1_rne_pack8(z);
        }
        emit(i, packed, sb);
        idx += (uint64_t)F;
    }
}

// Stores of the transposed copy straight to the [F x T] output: feature f0 + f's row, 8 code
// bytes and one scale byte for the thread's chunk.
struct GlobalColumnSink {
    uint8_t* cp;          // codes of feature f0, chunk c
    uint8_t* sp;          // scale byte of feature f0, chunk c
    int64_t code_row, scale_row;
    __device__ __forceinline__ void operator()(int f, uint32_t lo, uint32_t hi, uint32_t sb) const {
        *reinterpret_cast<uint2*>(cp + f * code_row) = make_uint2(lo, hi);
        sp[f * scale_row] = (uint8_t)sb;
    }
};

// The Hadamard quantizer with noise sums: the grid is capped in y and each workgroup
// strides over the chunk blocks of its feature block, so that few workgroups publish noise sums
// (same-address fp64 atomics serialize).  Every thread reaches the workgroup reduction.
template <typename T, bool kSR>
__global__ void __launch_bounds__(kRhtThreads)
k_rht_quant(const T* __restrict__ x, int64_t Tn, int64_t F, int64_t ld, uint64_t sign_seed,
            const float* __restrict__ amax_src, uint64_t seed, uint8_t* __restrict__ codes,
            uint8_t* __restrict__ scales, float* amax_out, float* sdec_out, double* sums,
            uint32_t chunk_blocks) {
    const float A = *amax_src;
    const TensorScales ts = tensor_scales(A);
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
        *amax_out = A;
        *sdec_out = ts.s_dec;
    }
    __shared__ EncTable tab;
    fill_enc_table(tab, ts);
    const uint32_t mask = rht_sign_mask(sign_seed);
    double g2 = 0.0, e2 = 0.0;
    for (uint32_t by = blockIdx.y; by < chunk_blocks; by += gridDim.y) {
        const RhtCoords rc = rht_coords_at(Tn, F, blockIdx.x, by);
        if (rc.valid) {
            Tile16x8<T> tile;
            tile.load(x + rc.c * 16 * ld + rc.f0, ld);
            const GlobalColumnSink sink{codes + rc.f0 * (Tn / 2) + rc.c * 8,
                                        scales + rc.f0 * (Tn / 16) + rc.c, Tn / 2, Tn / 16};
            quant_tile_transposed<T, kSR, true>(tile, rc.f0, rc.c * 16, Tn, mask, ts, tab, seed,
                                                g2, e2, sink);
        }
    }
    publish_noise<kRhtThreads>(g2, e2, ts, sums);
}

// Fused dual-orientation quantizer: one read of x gives the row-wise copy [T x F] (as the 1D
// quantizer makes it, element index row * F + col for SR) and the Hadamard-transformed
// transposed copy [F x T] (as k_rht_quant makes it, element index feature * T + token).  With
// kRows false it makes the transposed copy alone (the Hadamard quantizer without noise sums).
//
// A workgroup of 2 kTok threads takes a tile of 256 features x kTok tokens.  Thread (fg, ch) =
// (lane % 32, 2 * wave + lane / 32) owns features 8 fg .. 8 fg + 7 of the 16 tokens of chunk ch,
// so that each load instruction of a wave reads 512 contiguous bytes of two token rows.  Both
// copies are staged in LDS and leave as whole rows of the tile: 128 code bytes and 16 scale
// bytes for each of its kTok token rows, kTok / 2 code bytes and kTok / 16 scale bytes for each
// of its 256 feature rows.  Stored straight from the threads, the transposed copy would leave as
// 8-byte code pieces and single scale bytes of 32 feature rows per store instruction (one memory
// request per piece), and took longer than reading the input.
constexpr int kDualFeat = 256;

template <int kTok, bool kRows>
struct DualStage {
    uint32_t cols[kDualFeat * kTok / 8];     // transposed codes (col_slot)
    uint8_t csc[kDualFeat * (kTok / 16)];    // transposed scale bytes [feature row][chunk]
    uint32_t rows[kRows ? kTok * 32 : 1];    // row-wise codes, 32 words per token row (row_slot)
    uint8_t rsc[kRows ? kTok * 16 : 1];      // row-wise scale bytes [token row][feature block]
};

// LDS word of token row r: rows with bit 4 set trade places with their neighbour, so that the
// two chunks a wave writes (rows r and r + 16) fall in opposite halves of the 64 banks.
__device__ __forceinline__ uint32_t row_slot(uint32_t r) { return (r ^ ((r >> 4) & 1u)) * 32u; }

// LDS word of 8-byte piece q (chunk q) of transposed feature row p, with P = kTok / 8 words per
// row (64 / P rows per pass over the 64 banks) and P / 2 pieces: the row's position within its
// group of 64 / P rows is XORed with bits of p / 8 and its pieces are XOR-permuted by the next
// bits of p / 8, so that the 32 lanes of a half-wave writing one feature of 32 feature groups,
// and the lanes reading whole consecutive rows, each cover all 64 banks.
template <int kTok>
__device__ __forceinline__ uint32_t col_slot(uint32_t p, uint32_t q) {
    constexpr uint32_t P = kTok / 8, R = 64 / P, Q = P / 2;
    const uint32_t g = p >> 3;
    return (p ^ (g & (R - 1))) * P + 2u * (q ^ ((g / R) & (Q - 1)));
}

// Tile of workgroup w of a 1D grid of n tiles, gx of them across the features.  Workgroups are
// dispatched round-robin over the 8 XCDs, each with its own L2, so workgroup w runs on XCD
// w % 8; tile (w % 8) * (n / 8) + w / 8 gives every XCD a contiguous range of tiles, i.e. runs
// of adjacent feature tiles of the same tokens, whose row-wise scale bytes share lines.
// n % 8 != 0: tile w.
__device__ __forceinline__ void dual_tile(uint32_t gx, uint32_t& bx, uint32_t& by) {
    const uint32_t w = blockIdx.x, n = gridDim.x;
    const uint32_t t = (n & 7u) == 0 ? (w & 7u) * (n >> 3) + (w >> 3) : w;
    by = t / gx;
    bx = t - by * gx;
}

// At most 128 VGPRs (4 waves per SIMD) for bf16 input; the fp32 tile holds twice the registers.
template <typename T> constexpr int dual_min_waves() { return sizeof(T) == 2 ? 4 : 2; }

// Tokens per tile, measured on 16384 x 20480 and 16384 x 5120 bf16 tensors: 256 for round to
// nearest (store-bound: fewer, wider row pieces), 128 for stochastic rounding (ALU-bound: more
// workgroups per CU overlap one's stores with another's arithmetic).
template <bool kSR> constexpr int dual_tile_tokens() { return kSR ? 128 : 256; }

// Write-out of a staged tile (every thread of the workgroup calls these after the barrier).
// Transposed codes: 256 feature rows x kTok / 2 bytes, 8 bytes (16 tokens) per lane, whole rows
// of the tile per wave instruction; T % 16 == 0 keeps every piece whole and 8-byte aligned.  A
// thread keeps one piece position q and walks down the feature rows, kThreads / kPieces rows a
// pass, with its destination advanced by a constant instead of recomputed.
template <int kTok>
__device__ __forceinline__ void write_staged_cols(const uint32_t* cols, uint8_t* __restrict__ codes_t,
                                                  int64_t tf, int64_t tt, int64_t F, int64_t Tn) {
    constexpr uint32_t kThreads = 2 * kTok, kPieces = kTok / 16, kStride = kThreads / kPieces;
    static_assert(kThreads % kPieces == 0 && kDualFeat % kStride == 0, "passes");
    const uint32_t q = threadIdx.x % kPieces, p0 = threadIdx.x / kPieces;
    if (tt + q * 16 >= Tn) return;
    uint8_t* dst = codes_t + (tf + p0) * (Tn / 2) + tt / 2 + q * 8;
    const int64_t step = (int64_t)kStride * (Tn / 2);
#pragma unroll
    for (uint32_t i = 0; i < kDualFeat / kStride; ++i) {
        const uint32_t p = p0 + i * kStride;
        if (tf + p < F)
            *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(&cols[col_slot<kTok>(p, q)]);
        dst += step;
    }
}

// Row-wise codes: kTok token rows x 128 bytes (256 features), 16 lanes per token row, 8 bytes
// (16 features) each; F % 16 == 0 keeps every piece whole.  Same walk as write_staged_cols.
template <int kTok>
__device__ __forceinline__ void write_staged_rows(const uint32_t* rows, uint8_t* __restrict__ codes,
                                                  int64_t tf, int64_t tt, int64_t F, int64_t Tn) {
    constexpr uint32_t kThreads = 2 * kTok, kStride = kThreads / 16;
    const uint32_t q = threadIdx.x & 15u, r0 = threadIdx.x >> 4;
    if (tf + q * 16 >= F) return;
    uint8_t* dst = codes + (tt + r0) * (F / 2) + tf / 2 + q * 8;
    const int64_t step = (int64_t)kStride * (F / 2);
#pragma unroll
    for (uint32_t i = 0; i < kTok / kStride; ++i) {
        const uint32_t r = r0 + i * kStride;
        if (tt + r < Tn)
            *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(&rows[row_slot(r) + 2 * q]);
        dst += step;
    }
}

// Scale bytes staged as `rows` rows of `per_row` bytes, going to rows r0 .. of a matrix with
// rows_total rows of row_len bytes, from byte col0 (a multiple of per_row).  4-byte words when
// row_len and per_row are multiples of 4 (then a word is wholly inside or outside the matrix),
// else single bytes.
template <uint32_t kThreads>
__device__ __forceinline__ void write_staged_scales(const uint8_t* stage, uint32_t rows,
                                                    uint32_t per_row, uint8_t* __restrict__ dst,
                                                    int64_t row_len, int64_t r0,
                                                    int64_t rows_total, int64_t col0) {
    if (row_len % 4 == 0 && per_row % 4 == 0) {
        const uint32_t words = per_row / 4;
        for (uint32_t j = threadIdx.x; j < rows * words; j += kThreads) {
            const uint32_t r = j / words, d = j % words;
            if (r0 + r < rows_total && col0 + 4 * d < row_len)
                *reinterpret_cast<uint32_t*>(dst + (r0 + r) * row_len + col0 + 4 * d) =
                    *reinterpret_cast<const uint32_t*>(&stage[r * per_row + 4 * d]);
        }
    } else {
        for (uint32_t j = threadIdx.x; j < rows * per_row; j += kThreads) {
            const uint32_t r = j / per_row, b = j % per_row;
            if (r0 + r < rows_total && col0 + b < row_len)
                dst[(r0 + r) * row_len + col0 + b] = stage[r * per_row + b];
        }
    }
}

template <typename T, bool kSR, bool kRows>
__global__ void __launch_bounds__(2 * dual_tile_tokens<kSR>(), dual_min_waves<T>())
k_dual_quant(const T* __restrict__ x, int64_t Tn, int64_t F, int64_t ld, uint64_t sign_seed,
             const float* __restrict__ amax_src, const float* __restrict__ amax_t_src,
             uint64_t seed, uint64_t seed_t, uint8_t* __restrict__ codes,
             uint8_t* __restrict__ scales, uint8_t* __restrict__ codes_t,
             uint8_t* __restrict__ scales_t, float* amax_out, float* sdec_out, float* amax_t_out,
             float* sdec_t_out) {
    constexpr int kTok = dual_tile_tokens<kSR>();
    constexpr uint32_t kThreads = 2 * kTok, kPieces = kTok / 16;
    const float At = *amax_t_src;
    const TensorScales tst = tensor_scales(At);
    TensorScales ts = tst;
    if constexpr (kRows) ts = tensor_scales(*amax_src);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if constexpr (kRows) {
            *amax_out = *amax_src;
            *sdec_out = ts.s_dec;
        }
        *amax_t_out = At;
        *sdec_t_out = tst.s_dec;
    }
    __shared__ EncTable tab, tab_t;
    __shared__ DualStage<kTok, kRows> stg;
    if constexpr (kRows) fill_enc_table(tab, ts);
    fill_enc_table(tab_t, tst);
    uint32_t bx, by;
    dual_tile((uint32_t)((F + kDualFeat - 1) / kDualFeat), bx, by);
    const int64_t tf = (int64_t)bx * kDualFeat, tt = (int64_t)by * kTok;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t fg = lane & 31u, ch = 2u * (threadIdx.x >> 6) + (lane >> 5);
    const int64_t f0 = tf + fg * 8, row0 = tt + ch * 16;
    if (f0 < F && row0 < Tn) {
        Tile16x8<T> tile;
        tile.load(x + row0 * ld + f0, ld);
        if constexpr (kRows)
            quant_tile_rows<T, kSR>(tile, f0, row0, F, ts, tab, seed,
                                    [&](int i, uint32_t packed, uint32_t sb) {
                                        const uint32_t r = ch * 16 + (uint32_t)i;
                                        stg.rows[row_slot(r) + fg] = packed;
                                        // both lanes of the pair store the same byte
                                        stg.rsc[r * 16 + (fg >> 1)] = (uint8_t)sb;
                                    });
        double g2 = 0.0, e2 = 0.0;             // unused: no noise sums here
        auto to_stage = [&](int f, uint32_t lo, uint32_t hi, uint32_t sb) {
            const uint32_t p = fg * 8 + (uint32_t)f;
            *reinterpret_cast<uint2*>(&stg.cols[col_slot<kTok>(p, ch)]) = make_uint2(lo, hi);
            stg.csc[p * kPieces + ch] = (uint8_t)sb;
        };
        const uint32_t mask = rht_sign_mask(sign_seed);
        // the fold for bf16 input (the fp32 tile leaves no registers for a second code path)
        constexpr bool kFoldable = sizeof(T) == 2;
        if (kFoldable && At <= 0x1p120f)       // the same branch in every lane
            quant_tile_transposed<T, kSR, false, decltype(to_stage), kFoldable>(
                tile, f0, row0, Tn, mask, tst, tab_t, seed_t, g2, e2, to_stage);
        else
            quant_tile_transposed<T, kSR, false>(tile, f0, row0, Tn, mask, tst, tab_t, seed_t, g2,
                                                 e2, to_stage);
    }
    __syncthreads();
    write_staged_cols<kTok>(stg.cols, codes_t, tf, tt, F, Tn);
    write_staged_scales<kThreads>(stg.csc, kDualFeat, kPieces, scales_t, Tn / 16, tf, F, tt / 16);
    if constexpr (kRows) {
        write_staged_rows<kTok>(stg.rows, codes, tf, tt, F, Tn);
        write_staged_scales<kThreads>(stg.rsc, kTok, 16, scales, F / 16, tt, Tn, tf / 16);
    }
}

// Workgroups of the staged quantizer for a T x F input, or -1 if the count reaches 2^31.
static int64_t dual_grid(int64_t T, int64_t F, bool sr) {
    const int64_t tok = sr ? dual_tile_tokens<true>() : dual_tile_tokens<false>();
    const int64_t tiles = ((F + kDualFeat - 1) / kDualFeat) * ((T + tok - 1) / tok);
    return tiles >= (1ll << 31) ? -1 : tiles;
}

// E8M0 exponent of an MXFP4 block with maximum m: floor(log2 m) - 2 clamped to [-127, 127],
// 0 for an all-zero block.
__device__ __forceinline__ int mx_exponent(float m) {
    int e8 = 0;
    if (m > 0.0f) {
        e8 = __builtin_amdgcn_frexp_expf(m) - 1 - 2;   // m = f 2^E, f in [0.5, 1)
        e8 = e8 < -127 ? -127 : (e8 > 127 ? 127 : e8);
    }
    return e8;
}

// The transposed MXFP4 copy of one thread's tile into the LDS stage (kTok-token tiles): for
// each of its 8 features, its 16 tokens are one half of a 32-token block whose other half sits
// in lane l + 32 (the next chunk); codes to cols (col_slot), the scale byte from the even chunk
// to csc.  SR element index feature * T + token.
template <typename T, bool kSR, int kTok = dual_tile_tokens<kSR>()>
__device__ __forceinline__ void mx_tile_transposed(const Tile16x8<T>& tile, int64_t f0, int64_t row0,
                                                   int64_t Tn, uint64_t seed, uint32_t fg,
                                                   uint32_t ch, uint32_t* cols, uint8_t* csc) {
    constexpr uint32_t kBlocks = kTok / 32;
#pragma unroll
    for (int f = 0; f < 8; ++f) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = tile.get(i, f);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
        m = fmaxf(m, __shfl_xor(m, 32));
        const int e8 = mx_exponent(m);
        float z[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) z[e] = __builtin_amdgcn_ldexpf(v[e], -e8);
        uint32_t lo, hi;
        if constexpr (kSR) {
            const uint64_t idx = (uint64_t)(f0 + f) * (uint64_t)Tn + (uint64_t)row0;
            const u32x4 w0 = sr_words(seed, idx), w1 = sr_words(seed, idx + 8);
            const uint32_t a[4] = {w0.x, w0.y, w0.z, w0.w}, b[4] = {w1.x, w1.y, w1.z, w1.w};
            lo = e2m1_sr_pack8(z, a);
            hi = e2m1_sr_pack8(z + 8, b);
        } else {
            lo = e2m1_rne_pack8(z);
            hi = e2m1_rne_pack8(z + 8);
        }
        const uint32_t p = fg * 8 + (uint32_t)f;
        *reinterpret_cast<uint2*>(&cols[col_slot<kTok>(p, ch)]) = make_uint2(lo, hi);
        if ((ch & 1u) == 0) csc[p * kBlocks + ch / 2] = (uint8_t)(e8 + 127);
    }
}

// MXFP4 quantization of x^T [P3 NVFP4 in pratica: MXFP4, 32-element blocks with power-of-two
// scales, is the comparison format], on the staged quantizer's tiles (256 features x kTok
// tokens, 2 kTok threads): the 32 tokens of block b of a feature are chunks 2b and 2b + 1, held
// by lanes l and l + 32 of one wave; the block amax is shared with one lane exchange, E8M0
// exponent floor(log2 amax) - 2 clamped to [-127, 127] (0 for an all-zero block), codes E2M1 of
// x * 2^-exponent (RNE, or SR with element index f * T + t).  Codes and scale bytes are staged
// in LDS and leave as whole tile rows.  T % 32 == 0, so both lanes of a pair are valid or
// neither is.
template <typename T, bool kSR>
__global__ void __launch_bounds__(2 * dual_tile_tokens<kSR>(), dual_min_waves<T>())
k_mx_quant_t(const T* __restrict__ x, int64_t Tn, int64_t F, int64_t ld, uint64_t seed,
             uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    constexpr int kTok = dual_tile_tokens<kSR>();
    constexpr uint32_t kThreads = 2 * kTok, kBlocks = kTok / 32;
    __shared__ uint32_t cols[kDualFeat * kTok / 8];
    __shared__ uint8_t csc[kDualFeat * kBlocks];
    uint32_t bx, by;
    dual_tile((uint32_t)((F + kDualFeat - 1) / kDualFeat), bx, by);
    const int64_t tf = (int64_t)bx * kDualFeat, tt = (int64_t)by * kTok;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t fg = lane & 31u, ch = 2u * (threadIdx.x >> 6) + (lane >> 5);
    const int64_t f0 = tf + fg * 8, row0 = tt + ch * 16;
    if (f0 < F && row0 < Tn) {
        Tile16x8<T> tile;
        tile.load(x + row0 * ld + f0, ld);
        mx_tile_transposed<T, kSR>(tile, f0, row0, Tn, seed, fg, ch, cols, csc);
    }
    __syncthreads();
    write_staged_cols<kTok>(cols, codes, tf, tt, F, Tn);
    write_staged_scales<kThreads>(csc, kDualFeat, kBlocks, scales, Tn / 32, tf, F, tt / 32);
}

// Fused dual-orientation MXFP4 quantizer of the comparison format: one read of x [T x F] gives
// the row-wise copy [T x F] (as mxfp4_quantize_1d makes it: 32-feature blocks, element index
// row * F + col for SR) and the transposed copy [F x T] (as k_mx_quant_t makes it: 32-token
// blocks, element index feature * T + token), on the staged quantizer's tiles.  A 32-feature
// row block is the 8 features of four adjacent lanes (maximum by two DPP exchanges); a 32-token
// block is the two chunks of lanes l and l + 32.  Both copies are staged in LDS and leave as
// whole tile rows.  F % 32 == 0 and T % 32 == 0, so the lanes of a block are valid together.
template <typename T, bool kSR>
__global__ void __launch_bounds__(2 * dual_tile_tokens<kSR>(), dual_min_waves<T>())
k_mx_quant_dual(const T* __restrict__ x, int64_t Tn, int64_t F, int64_t ld, uint64_t seed,
                uint64_t seed_t, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t) {
    constexpr int kTok = dual_tile_tokens<kSR>();
    constexpr uint32_t kThreads = 2 * kTok, kBlocks = kTok / 32;
    __shared__ uint32_t cols[kDualFeat * kTok / 8];
    __shared__ uint8_t csc[kDualFeat * kBlocks];
    __shared__ uint32_t rows[kTok * 32];
    __shared__ uint8_t rsc[kTok * (kDualFeat / 32)];
    uint32_t bx, by;
    dual_tile((uint32_t)((F + kDualFeat - 1) / kDualFeat), bx, by);
    const int64_t tf = (int64_t)bx * kDualFeat, tt = (int64_t)by * kTok;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t fg = lane & 31u, ch = 2u * (threadIdx.x >> 6) + (lane >> 5);
    const int64_t f0 = tf + fg * 8, row0 = tt + ch * 16;
    if (f0 < F && row0 < Tn) {
        Tile16x8<T> tile;
        tile.load(x + row0 * ld + f0, ld);
        // row-wise: token row i, features f0 .. f0 + 7, one quarter of a 32-feature block
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float y[8];
#pragma unroll
            for (int f = 0; f < 8; ++f) y[f] = tile.get(i, f);
            float m = 0.0f;
#pragma unroll
            for (int f = 0; f < 8; ++f) m = fmaxf(m, fabsf(y[f]));
            m = fmaxf(m, swap_adjacent(m));
            m = fmaxf(m, swap_pairs(m));
            const int e8 = mx_exponent(m);
            float z[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) z[e] = __builtin_amdgcn_ldexpf(y[e], -e8);
            uint32_t packed;
            if constexpr (kSR) {
                const u32x4 w = sr_words(seed, (uint64_t)(row0 + i) * (uint64_t)F + (uint64_t)f0);
                const uint32_t words[4] = {w.x, w.y, w.z, w.w};
                packed = e2m1_sr_pack8(z, words);
            } else {
                packed = e2m1_rne_pack8(z);
            }
            const uint32_t r = ch * 16 + (uint32_t)i;
            rows[row_slot(r) + fg] = packed;
            if ((fg & 3u) == 0) rsc[r * (kDualFeat / 32) + fg / 4] = (uint8_t)(e8 + 127);
        }
        tile.fence();
        mx_tile_transposed<T, kSR>(tile, f0, row0, Tn, seed_t, fg, ch, cols, csc);
    }
    __syncthreads();
    write_staged_cols<kTok>(cols, codes_t, tf, tt, F, Tn);
    write_staged_scales<kThreads>(csc, kDualFeat, kBlocks, scales_t, Tn / 32, tf, F, tt / 32);
    write_staged_rows<kTok>(rows, codes, tf, tt, F, Tn);
    write_staged_scales<kThreads>(rsc, kTok, kDualFeat / 32, scales, F / 32, tt, Tn, tf / 32);
}

static dim3 rht_grid(int64_t T, int64_t F) {
    return dim3((unsigned)((F + kFeatPerBlock - 1) / kFeatPerBlock),
                (unsigned)((T / 16 + kChunksPerBlock - 1) / kChunksPerBlock));
}

static nvfp4_status check_rht_input(const void* x, nvfp4_dtype dt, int64_t T, int64_t F, int64_t ld) {
    nvfp4_status s = check_input(x, dt, T, F, ld);
    if (s) return s;
    if (T % 16 != 0 || F % 8 != 0) return NVFP4_ERR_SHAPE;
    // launch limits: quantizer grid (F/64, T/512) with gridDim.y <= 65535, and the amax pass's
    // tile count (F/256 x T/128) in 31 bits
    const int64_t gy = (T / 16 + kChunksPerBlock - 1) / kChunksPerBlock;
    const int64_t amax_tiles = ((F + kAmaxFeat - 1) / kAmaxFeat) * ((T / 16 + kAmaxChunks - 1) / kAmaxChunks);
    if (F >= (1ll << 31) || gy > 65535 || amax_tiles >= (1ll << 31)) return NVFP4_ERR_SHAPE;
    return NVFP4_OK;
}

__global__ void k_fill2_f64(double* p) {
    p[0] = 0.0;
    p[1] = 0.0;
}

__global__ void k_fill2_rht(float* p, float* q) {
    *p = 0.0f;
    if (q) *q = 0.0f;
}

// The amax of the transformed tensor into *dst and, if plain_dst is non-NULL, the amax of x
// itself into *plain_dst, in one pass.
// With `accumulate` false the destinations are zeroed first; otherwise the pass raises them.
static nvfp4_status launch_rht_amax(const void* x, nvfp4_dtype dt, int64_t T, int64_t F, int64_t ld,
                                    uint64_t sign_seed, float* dst, float* plain_dst,
                                    hipStream_t st, bool accumulate = false) {
    if (!accumulate) hipLaunchKernelGGL(k_fill2_rht, dim3(1), dim3(1), 0, st, dst, plain_dst);
    if (T > 0 && F > 0) {
        const uint32_t tx = (uint32_t)((F + kAmaxFeat - 1) / kAmaxFeat);
        const uint32_t tiles = tx * (uint32_t)((T / 16 + kAmaxChunks - 1) / kAmaxChunks);
        const FastDiv tpr = make_fastdiv(tx);
        const int sub = dt == NVFP4_BF16 ? rht_amax_sub<uint16_t>() : rht_amax_sub<float>();
        const uint32_t need = (tiles + sub - 1) / sub;
        const dim3 grid(need < (uint32_t)kRhtAmaxBlocks ? need : (uint32_t)kRhtAmaxBlocks);
        const dim3 block(kRhtThreads * sub);
        const bool stream = T * F * (dt == NVFP4_BF16 ? 2 : 4) >= kStreamBytes;
#define NVFP4_RA(TT, PLAIN, NT)                                                                   \
        hipLaunchKernelGGL((k_rht_amax<TT, PLAIN, NT>), grid, block, 0, st,                       \
                           static_cast<const TT*>(x), T, F, ld, sign_seed, dst, plain_dst, tiles, tpr)
#define NVFP4_RA2(TT, PLAIN)                                                                      \
        do { if (stream) NVFP4_RA(TT, PLAIN, true); else NVFP4_RA(TT, PLAIN, false); } while (0)
        if (dt == NVFP4_BF16) {
            if (plain_dst) NVFP4_RA2(uint16_t, true); else NVFP4_RA2(uint16_t, false);
        } else {
            if (plain_dst) NVFP4_RA2(float, true); else NVFP4_RA2(float, false);
        }
#undef NVFP4_RA2
#undef NVFP4_RA
    }
    return launch_status();
}

static nvfp4_status check_amax_ptr(const float* p) {
    if (!p) return NVFP4_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(p) & 3u) return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" nvfp4_status nvfp4_hadamard_amax(const void* x, nvfp4_dtype dt, int64_t T, int64_t F,
                                            int64_t ld, uint64_t sign_seed, float* amax_out,
                                            void* stream) {
    nvfp4_status s = check_rht_input(x, dt, T, F, ld);
    if (s) return s;
    s = check_amax_ptr(amax_out);
    if (s) return s;
    return launch_rht_amax(x, dt, T, F, ld, sign_seed, amax_out, nullptr, as_stream(stream));
}

extern "C" nvfp4_status nvfp4_hadamard_amax_accumulate(const void* x, nvfp4_dtype dt, int64_t T,
                                                       int64_t F, int64_t ld, uint64_t sign_seed,
                                                       float* amax_inout, void* stream) {
    nvfp4_status s = check_rht_input(x, dt, T, F, ld);
    if (s) return s;
    s = check_amax_ptr(amax_inout);
    if (s) return s;
    return launch_rht_amax(x, dt, T, F, ld, sign_seed, amax_inout, nullptr, as_stream(stream), true);
}

extern "C" nvfp4_status nvfp4_dual_amax(const void* x, nvfp4_dtype dt, int64_t T, int64_t F,
                                        int64_t ld, uint64_t sign_seed, float* amax_out,
                                        float* amax_t_out, void* stream) {
    nvfp4_status s = check_rht_input(x, dt, T, F, ld);
    if (s) return s;
    if ((s = check_amax_ptr(amax_out)) || (s = check_amax_ptr(amax_t_out))) return s;
    if (amax_out == amax_t_out) return NVFP4_ERR_SHAPE;
    return launch_rht_amax(x, dt, T, F, ld, sign_seed, amax_t_out, amax_out, as_stream(stream));
}

extern "C" nvfp4_status nvfp4_dual_amax_accumulate(const void* x, nvfp4_dtype dt, int64_t T,
                                                   int64_t F, int64_t ld, uint64_t sign_seed,
                                                   float* amax_inout, float* amax_t_inout,
                                                   void* stream) {
    nvfp4_status s = check_rht_input(x, dt, T, F, ld);
    if (s) return s;
    if ((s = check_amax_ptr(amax_inout)) || (s = check_amax_ptr(amax_t_inout))) return s;
    if (amax_inout == amax_t_inout) return NVFP4_ERR_SHAPE;
    return launch_rht_amax(x, dt, T, F, ld, sign_seed, amax_t_inout, amax_inout, as_stream(stream),
                           true);
}

constexpr uint32_t kNoiseWorkgroups = 1024;   // target grid size of the quantizer with noise sums

static nvfp4_status hadamard_quantize(const void* x, nvfp4_dtype dt, int64_t ld, uint64_t sign_seed,
                                      const float* amax_in, nvfp4_round rnd, uint64_t seed,
                                      const nvfp4_tensor* out, double* sums, hipStream_t st) {
    nvfp4_status s = check_q(out, NVFP4_BLK_1x16, true);
    if (s) return s;
    const int64_t F = out->rows, T = out->cols;
    s = check_rht_input(x, dt, T, F, ld);
    if (s) return s;
    if (rnd != NVFP4_RNE && rnd != NVFP4_SR) return NVFP4_ERR_DTYPE;
    const float* src = amax_in;
    if (!src) {
        s = launch_rht_amax(x, dt, T, F, ld, sign_seed, out->amax, nullptr, st);
        if (s) return s;
        src = out->amax;
    }
    if (sums) hipLaunchKernelGGL(k_fill2_f64, dim3(1), dim3(1), 0, st, sums);
    if (T == 0 || F == 0) {
        hipLaunchKernelGGL(k_scalars_rht, dim3(1), dim3(1), 0, st, src, out->amax, out->s_dec);
        return launch_status();
    }
    if (!sums) {
        // the staged quantizer without its row-wise copy
        const int64_t tiles = dual_grid(T, F, rnd == NVFP4_SR);
        if (tiles < 0) return NVFP4_ERR_SHAPE;
        const dim3 grid((uint32_t)tiles);
#define NVFP4_RQ(TT, SRV)                                                                         \
        hipLaunchKernelGGL((k_dual_quant<TT, SRV, false>), grid, dim3(2 * dual_tile_tokens<SRV>()), \
                           0, st, static_cast<const TT*>(x), T, F, ld, sign_seed, nullptr, src,   \
                           0, seed, nullptr, nullptr, out->codes, out->scales, nullptr, nullptr,  \
                           out->amax, out->s_dec)
        if (dt == NVFP4_BF16) {
            if (rnd == NVFP4_SR) NVFP4_RQ(uint16_t, true); else NVFP4_RQ(uint16_t, false);
        } else {
            if (rnd == NVFP4_SR) NVFP4_RQ(float, true); else NVFP4_RQ(float, false);
        }
#undef NVFP4_RQ
        return launch_status();
    }
    dim3 grid = rht_grid(T, F);
    const uint32_t chunk_blocks = grid.y;
    const uint32_t cap = (kNoiseWorkgroups + grid.x - 1) / grid.x;
    grid.y = chunk_blocks < cap ? chunk_blocks : cap;
    const dim3 block(kRhtThreads);
#define NVFP4_RQ(TT, SRV)                                                                         \
    hipLaunchKernelGGL((k_rht_quant<TT, SRV>), grid, block, 0, st, static_cast<const TT*>(x), T,  \
                       F, ld, sign_seed, src, seed, out->codes, out->scales, out->amax, out->s_dec, \
                       sums, chunk_blocks)
    if (dt == NVFP4_BF16) {
        if (rnd == NVFP4_SR) NVFP4_RQ(uint16_t, true); else NVFP4_RQ(uint16_t, false);
    } else {
        if (rnd == NVFP4_SR) NVFP4_RQ(float, true); else NVFP4_RQ(float, false);
    }
#undef NVFP4_RQ
    return launch_status();
}

extern "C" nvfp4_status nvfp4_hadamard_quantize(const void* x, nvfp4_dtype dt, int64_t ld,
                                                uint64_t sign_seed, const float* amax_in,
                                                nvfp4_round rnd, uint64_t seed,
                                                const nvfp4_tensor* out, void* stream) {
    return hadamard_quantize(x, dt, ld, sign_seed, amax_in, rnd, seed, out, nullptr,
                             as_stream(stream));
}

extern "C" nvfp4_status nvfp4_hadamard_quantize_noise(const void* x, nvfp4_dtype dt, int64_t ld,
                                                      uint64_t sign_seed, const float* amax_in,
                                                      nvfp4_round rnd, uint64_t seed,
                                                      const nvfp4_tensor* out, double* sums,
                                                      void* stream) {
    if (!sums) return NVFP4_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(sums) & 7u) return NVFP4_ERR_ALIGN;
    return hadamard_quantize(x, dt, ld, sign_seed, amax_in, rnd, seed, out, sums,
                             as_stream(stream));
}

extern "C" nvfp4_status nvfp4_quantize_dual(const void* x, nvfp4_dtype dt, int64_t ld,
                                            uint64_t sign_seed, const float* amax_in,
                                            const float* amax_t_in, nvfp4_round rnd,
                                            uint64_t seed, uint64_t seed_t,
                                            const nvfp4_tensor* out, const nvfp4_tensor* out_t,
                                            void* stream) {
    nvfp4_status s = check_q(out, NVFP4_BLK_1x16, true);
    if (s) return s;
    s = check_q(out_t, NVFP4_BLK_1x16, true);
    if (s) return s;
    const int64_t T = out->rows, F = out->cols;
    if (out_t->rows != F || out_t->cols != T) return NVFP4_ERR_SHAPE;
    s = check_rht_input(x, dt, T, F, ld);
    if (s) return s;
    if (F % 16 != 0) return NVFP4_ERR_SHAPE;
    if (rnd != NVFP4_RNE && rnd != NVFP4_SR) return NVFP4_ERR_DTYPE;
    if (out->amax == out_t->amax || out->s_dec == out_t->s_dec) return NVFP4_ERR_SHAPE;
    hipStream_t st = as_stream(stream);
    const float* src = amax_in;
    const float* src_t = amax_t_in;
    // compute only the maxima the caller did not supply, so a supplied one is never overwritten
    if (!src_t) {
        s = launch_rht_amax(x, dt, T, F, ld, sign_seed, out_t->amax, src ? nullptr : out->amax, st);
        if (s) return s;
        src_t = out_t->amax;
        if (!src) src = out->amax;
    } else if (!src) {
        s = nvfp4_amax(x, dt, T, F, ld, out->amax, stream);
        if (s) return s;
        src = out->amax;
    }
    if (T == 0 || F == 0) {
        hipLaunchKernelGGL(k_scalars_rht, dim3(1), dim3(1), 0, st, src, out->amax, out->s_dec);
        hipLaunchKernelGGL(k_scalars_rht, dim3(1), dim3(1), 0, st, src_t, out_t->amax, out_t->s_dec);
        return launch_status();
    }
    const int64_t tiles = dual_grid(T, F, rnd == NVFP4_SR);
    if (tiles < 0) return NVFP4_ERR_SHAPE;
    const dim3 grid((uint32_t)tiles);         // tiles placed by dual_tile
#define NVFP4_DQ(TT, SRV)                                                                         \
    hipLaunchKernelGGL((k_dual_quant<TT, SRV, true>), grid, dim3(2 * dual_tile_tokens<SRV>()), 0, \
                       st, static_cast<const TT*>(x), T, F, ld, sign_seed, src, src_t, seed,      \
                       seed_t, out->codes, out->scales, out_t->codes, out_t->scales, out->amax,   \
                       out->s_dec, out_t->amax, out_t->s_dec)
    if (dt == NVFP4_BF16) {
        if (rnd == NVFP4_SR) NVFP4_DQ(uint16_t, true); else NVFP4_DQ(uint16_t, false);
    } else {
        if (rnd == NVFP4_SR) NVFP4_DQ(float, true); else NVFP4_DQ(float, false);
    }
#undef NVFP4_DQ
    return launch_status();
}

extern "C" nvfp4_status mxfp4_quantize_1d_t(const void* x, nvfp4_dtype dt, int64_t ld,
                                            nvfp4_round rnd, uint64_t seed,
                                            const nvfp4_tensor* out, void* stream) {
    nvfp4_status s = check_q(out, MXFP4_BLK_1x32, false);
    if (s) return s;
    const int64_t F = out->rows, T = out->cols;
    s = check_rht_input(x, dt, T, F, ld);
    if (s) return s;
    if (T % 32 != 0) return NVFP4_ERR_SHAPE;
    if (rnd != NVFP4_RNE && rnd != NVFP4_SR) return NVFP4_ERR_DTYPE;
    if (T == 0 || F == 0) return NVFP4_OK;
    hipStream_t st = as_stream(stream);
#define NVFP4_MXT(TT, SRV)                                                                        \
    do {                                                                                          \
        const int64_t tiles = dual_grid(T, F, SRV);                                               \
        if (tiles < 0) return NVFP4_ERR_SHAPE;                                                    \
        hipLaunchKernelGGL((k_mx_quant_t<TT, SRV>), dim3((uint32_t)tiles),                        \
                           dim3(2 * dual_tile_tokens<SRV>()), 0, st, static_cast<const TT*>(x),   \
                           T, F, ld, seed, out->codes, out->scales);                              \
    } while (0)
    if (dt == NVFP4_BF16) {
        if (rnd == NVFP4_SR) NVFP4_MXT(uint16_t, true); else NVFP4_MXT(uint16_t, false);
    } else {
        if (rnd == NVFP4_SR) NVFP4_MXT(float, true); else NVFP4_MXT(float, false);
    }
#undef NVFP4_MXT
    return launch_status();
}

extern "C" nvfp4_status mxfp4_quantize_dual(const void* x, nvfp4_dtype dt, int64_t ld,
                                            nvfp4_round rnd, uint64_t seed, uint64_t seed_t,
                                            const nvfp4_tensor* out, const nvfp4_tensor* out_t,
                                            void* stream) {
    nvfp4_status s = check_q(out, MXFP4_BLK_1x32, false);
    if (s) return s;
    s = check_q(out_t, MXFP4_BLK_1x32, false);
    if (s) return s;
    const int64_t T = out->rows, F = out->cols;
    if (out_t->rows != F || out_t->cols != T) return NVFP4_ERR_SHAPE;
    s = check_rht_input(x, dt, T, F, ld);
    if (s) return s;
    if (rnd != NVFP4_RNE && rnd != NVFP4_SR) return NVFP4_ERR_DTYPE;
    if (T == 0 || F == 0) return NVFP4_OK;
    hipStream_t st = as_stream(stream);
#define NVFP4_MXD(TT, SRV)                                                                        \
    do {                                                                                          \
        const int64_t tiles = dual_grid(T, F, SRV);                                               \
        if (tiles < 0) return NVFP4_ERR_SHAPE;                                                    \
        hipLaunchKernelGGL((k_mx_quant_dual<TT, SRV>), dim3((uint32_t)tiles),                     \
                           dim3(2 * dual_tile_tokens<SRV>()), 0, st, static_cast<const TT*>(x),   \
                           T, F, ld, seed, seed_t, out->codes, out->scales, out_t->codes,         \
                           out_t->scales);                                                        \
    } while (0)
    if (dt == NVFP4_BF16) {
        if (rnd == NVFP4_SR) NVFP4_MXD(uint16_t, true); else NVFP4_MXD(uint16_t, false);
    } else {
        if (rnd == NVFP4_SR) NVFP4_MXD(float, true); else NVFP4_MXD(float, false);
    }
#undef NVFP4_MXD
    return launch_status();
}
