// quantize.hip -- per-tensor amax, 1D/2D NVFP4 quantization, dequantization and the MXFP4
// quantizer for gfx950.
//
// Citation keys: [P1] "Entrenamiento de Modelos de Lenguaje con 4 Bits de Precision";
// [P2] "FP4 All the Way: Formacion totalmente cuantificada de LLM"; [P3] "I ricercatori di
// Nvidia sbloccano il tutorial LLM a 8 bit che corrisponde alle prestazioni a 4 bit".
//
// All kernels here are HBM-bound streaming kernels.  The amax, dequantize and MXFP4 kernels
// split rows into "groups" of 8 consecutive elements (one 16-byte bf16 load, one 32-bit store of
// 8 packed codes); the NVFP4 1D quantizer gives each lane a whole 16-element block.  Every
// thread issues all of its loads before any arithmetic, to keep enough bytes in flight.

#include "device_codecs.hpp"
#include "host_util.hpp"
#include "noise.hpp"

namespace nvfp4 {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;     // groups per thread and trip in the amax / dequantize / MX kernels
constexpr int kQUnroll = 2;    // blocks per thread in the NVFP4 1D quantizer (measured: 2 beats 1, 4, 8, 16)
constexpr int kNoiseBlocks = 1024;   // grid cap of the quantizer with the noise sums

// 8 input elements of one group as fp32.
template <typename T> struct Group8;

template <> struct Group8<uint16_t> {   // bf16
    template <bool kNT = true>
    static __device__ __forceinline__ void load(const uint16_t* p, float* y) {
        const uint4 v = load16<kNT>(p);
        y[0] = bf16_lo(v.x); y[1] = bf16_hi(v.x); y[2] = bf16_lo(v.y); y[3] = bf16_hi(v.y);
        y[4] = bf16_lo(v.z); y[5] = bf16_hi(v.z); y[6] = bf16_lo(v.w); y[7] = bf16_hi(v.w);
    }
};

template <> struct Group8<float> {
    template <bool kNT = true>
    static __device__ __forceinline__ void load(const float* p, float* y) {
        const uint4 a = load16<kNT>(p), b = load16<kNT>(p + 4);
        y[0] = __uint_as_float(a.x); y[1] = __uint_as_float(a.y);
        y[2] = __uint_as_float(a.z); y[3] = __uint_as_float(a.w);
        y[4] = __uint_as_float(b.x); y[5] = __uint_as_float(b.y);
        y[6] = __uint_as_float(b.z); y[7] = __uint_as_float(b.w);
    }
};

__global__ void k_fill_f32(float* p, float v) { *p = v; }

// Writes amax/s_dec for an empty tensor (A taken from src, 0 if src is NULL).
__global__ void k_tensor_scalars(const float* src, float* amax_out, float* sdec_out) {
    float A = src ? *src : 0.0f;
    TensorScales ts = tensor_scales(A);
    if (amax_out) *amax_out = A;
    if (sdec_out) *sdec_out = ts.s_dec;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

// ---- per-tensor amax [P3 Come funziona NVFP4?] ------------------------------------------------
// Persistent grid-stride kernel: one 1024-thread workgroup per CU, each thread keeping
// kAmaxUnroll 16-byte loads in flight per trip; each workgroup publishes its maximum once at the
// end (publish_amax).  Few large workgroups: the publishes of more, smaller workgroups to the one
// address cost more than their extra bandwidth gains (measured on MI355X).
constexpr int kAmaxBlocks = 256;
constexpr int kAmaxThreads = 1024;
constexpr int kAmaxUnroll = 8;

template <typename T, bool kNT>
__global__ void __launch_bounds__(kAmaxThreads)
k_amax(const T* __restrict__ x, int64_t ld, uint32_t groups, FastDiv gpr, float* amax_out) {
    float m = 0.0f;
    const uint32_t stride = gridDim.x * kAmaxThreads * kAmaxUnroll;
    for (uint32_t base = blockIdx.x * kAmaxThreads * kAmaxUnroll + threadIdx.x; base < groups;
         base += stride) {
        float y[kAmaxUnroll][8];
#pragma unroll
        for (int u = 0; u < kAmaxUnroll; ++u) {
            uint32_t g = base + u * kAmaxThreads;
            g = g < groups ? g : groups - 1;           // clamped duplicate: max is unchanged
            const uint32_t row = fastdiv(g, gpr);
            const uint32_t cg = g - row * gpr.d;
            Group8<T>::template load<kNT>(x + (int64_t)row * ld + cg * 8, y[u]);
        }
#pragma unroll
        for (int u = 0; u < kAmaxUnroll; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(y[u][e]));
    }
    m = wave_max(m);
    __shared__ float part[kAmaxThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = part[0];
#pragma unroll
        for (int w = 1; w < kAmaxThreads / 64; ++w) b = fmaxf(b, part[w]);
        publish_amax(amax_out, b);
    }
}

static int amax_grid(uint32_t groups) {
    int64_t need = ((int64_t)groups + kAmaxThreads * kAmaxUnroll - 1) / (kAmaxThreads * kAmaxUnroll);
    return (int)(need < 1 ? 1 : (need < kAmaxBlocks ? need : kAmaxBlocks));
}

// ---- 1D quantization [P1 Caracteristicas; P2 Describir] ---------------------------------------
// One lane owns one whole 16-element block: two 16-byte loads (bf16), one 8-byte code store and
// one scale byte.  Each thread handles kQUnroll blocks spaced a workgroup apart, all loads first.
// Blocks past the end load a clamped (valid) block and store nothing.
//
// With kNoise the same pass also accumulates the quantization-noise diagnostic
// [P2 Describir: quantized training loses efficiency once the gradient norm falls below about
// sqrt(3) times the quantization noise]: sums[0] += x^2 and sums[1] += (Q(x) - x)^2, where
// Q(x) = fl(fl(v * scale) * s_dec) is the dequantized value.  The squares are taken of the
// values times s_enc = 2688 / amax (at most 5376 in magnitude, so no fp32 overflow or early
// underflow), each 16-element block is summed in fp32, blocks are accumulated in fp64, and each
// workgroup adds its two totals, divided by s_enc^2, atomically (noise.hpp).

// The work of one k_quant1d thread on kQUnroll blocks starting at block `base` (spaced a
// workgroup apart): all loads first, then per block the scale, the codes and, with kNoise, the
// block's contributions to the two noise sums.
template <typename T, bool kSR, bool kNoise>
__device__ __forceinline__ void quant1d_blocks(const T* __restrict__ x, int64_t ld, uint32_t blocks,
                                               FastDiv bpr, uint32_t cols, const TensorScales& ts,
                                               const EncTable& tab, uint64_t seed,
                                               uint2* __restrict__ codes,
                                               uint8_t* __restrict__ scales, uint32_t base,
                                               double& g2, double& e2) {
    float y[kQUnroll][16];
    uint32_t row[kQUnroll], cb[kQUnroll];
#pragma unroll
    for (int u = 0; u < kQUnroll; ++u) {
        uint32_t b = base + u * kThreads;
        b = b < blocks ? b : blocks - 1;
        row[u] = fastdiv(b, bpr);
        cb[u] = b - row[u] * bpr.d;
        const T* p = x + (int64_t)row[u] * ld + cb[u] * 16;
        Group8<T>::load(p, y[u]);
        Group8<T>::load(p + 8, y[u] + 8);
    }
#pragma unroll
    for (int u = 0; u < kQUnroll; ++u) {
        const uint32_t b = base + u * kThreads;
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(y[u][e]));
        uint32_t sb;
        float enc;
        block_scale_tab(m, ts, tab, sb, enc);
        float z[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) z[e] = y[u][e] * enc;
        uint32_t lo = 0, hi = 0;
        if constexpr (kSR) {
            const uint64_t idx = (uint64_t)row[u] * cols + cb[u] * 16;
            const u32x4 w0 = sr_words(seed, idx), w1 = sr_words(seed, idx + 8);
            const uint32_t wa[4] = {w0.x, w0.y, w0.z, w0.w}, wb[4] = {w1.x, w1.y, w1.z, w1.w};
            lo = e2m1_sr_pack8(z, wa);
            hi = e2m1_sr_pack8(z + 8, wb);
        } else {
            lo = e2m1_rne_pack8(z);
            hi = e2m1_rne_pack8(z + 8);
        }
        if (b < blocks) {
            codes[b] = make_uint2(lo, hi);       // blocks are dense in the code array
            scales[b] = (uint8_t)sb;
            if constexpr (kNoise) block_noise(y[u], lo, hi, sb, ts, g2, e2);
        }
    }
}

template <typename T, bool kSR, bool kNoise>
__global__ void __launch_bounds__(kThreads)
k_quant1d(const T* __restrict__ x, int64_t ld, uint32_t blocks, FastDiv bpr, uint32_t cols,
          const float* __restrict__ amax_src, uint64_t seed, uint2* __restrict__ codes,
          uint8_t* __restrict__ scales, float* amax_out, float* sdec_out, double* sums) {
    const float A = *amax_src;
    const TensorScales ts = tensor_scales(A);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *amax_out = A;
        *sdec_out = ts.s_dec;
    }
    __shared__ EncTable tab;
    fill_enc_table(tab, ts);
    // With kNoise the grid is capped and each workgroup strides over the blocks, so that few
    // workgroups publish sums (same-address fp64 atomics serialize); otherwise the grid covers
    // every block once.
    double g2 = 0.0, e2 = 0.0;
    if constexpr (kNoise) {
        for (uint32_t wbase = blockIdx.x * kThreads * kQUnroll; wbase < blocks;
             wbase += gridDim.x * kThreads * kQUnroll)
            quant1d_blocks<T, kSR, kNoise>(x, ld, blocks, bpr, cols, ts, tab, seed, codes, scales,
                                           wbase + threadIdx.x, g2, e2);
    } else {
        quant1d_blocks<T, kSR, kNoise>(x, ld, blocks, bpr, cols, ts, tab, seed, codes, scales,
                                       blockIdx.x * kThreads * kQUnroll + threadIdx.x, g2, e2);
    }
    if constexpr (kNoise) publish_noise<kThreads>(g2, e2, ts, sums);
}

__global__ void k_fill_f64x2(double* p) {
    p[0] = 0.0;
    p[1] = 0.0;
}

// ---- 2D quantization of weights [P1 Metodologia: two-dimensional block scaling] ---------------
// A workgroup quantizes a 128 x 128 region (8 x 8 tiles of 16 x 16).  Wave v takes rows
// [32v, 32v + 32) of the region; lane l owns the 8 x 8 block at column chunk c = l & 15 and row
// group g = l >> 4 (rows 8g .. 8g + 7 of the wave's 32).  Its eight row loads (16 bytes each for
// bf16) are issued before any arithmetic, and each load instruction of the wave reads four whole
// 256-byte row segments.  A 16 x 16 tile is held by lanes l, l ^ 1, l ^ 16 and l ^ 17, so its
// amax takes two lane exchanges.  The row-wise codes leave as one 4-byte word per block row (16
// lanes write a region row's 64 contiguous bytes).  For the transposed copy each lane transposes
// its 8 x 8 codes in registers (nibble_transpose8) and stages the eight column words in LDS;
// after one barrier 16 consecutive threads write each transposed row's 64 contiguous bytes.
// rows and cols are multiples of 16, so every 8 x 8 block (and tile) is wholly inside or outside
// the matrix; blocks outside load a clamped, valid block and store nothing.
constexpr int kQ2Region = 128;

// In-register transpose of an 8 x 8 matrix of nibbles: on entry nibble j of w[i] is element
// (i, j), on exit nibble i of w[j] is element (i, j).  Three exchange stages: 4 x 4 quadrants
// (16-bit halves), 2 x 2 blocks of bytes, then single nibbles.
__device__ __forceinline__ void nibble_transpose8(uint32_t* w) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t a = w[i], b = w[i + 4];
        w[i] = (a & 0x0000FFFFu) | (b << 16);
        w[i + 4] = (a >> 16) | (b & 0xFFFF0000u);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int i = (q & 1) + 4 * (q >> 1);       // 0, 1, 4, 5
        const uint32_t a = w[i], b = w[i + 2];
        w[i] = (a & 0x00FF00FFu) | ((b & 0x00FF00FFu) << 8);
        w[i + 2] = ((a >> 8) & 0x00FF00FFu) | (b & 0xFF00FF00u);
    }
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
        const uint32_t a = w[i], b = w[i + 1];
        w[i] = (a & 0x0F0F0F0Fu) | ((b & 0x0F0F0F0Fu) << 4);
        w[i + 1] = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
    }
}

template <typename T>
__global__ void __launch_bounds__(kThreads)
k_quant2d(const T* __restrict__ w, int64_t ld, uint32_t rows, uint32_t cols,
          const float* __restrict__ amax_src, uint8_t* __restrict__ codes,
          uint8_t* __restrict__ scales, uint8_t* __restrict__ codes_t,
          uint8_t* __restrict__ scales_t, float* amax_out, float* sdec_out, float* amax_out_t,
          float* sdec_out_t, uint32_t regions_per_row) {
    // [region column][8-row group] code words of the transposed copy; one word of padding per row
    __shared__ uint32_t stage[kQ2Region][kQ2Region / 8 + 1];
    const float A = *amax_src;
    const TensorScales ts = tensor_scales(A);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *amax_out = A;
        *sdec_out = ts.s_dec;
        if (amax_out_t) *amax_out_t = A;
        if (sdec_out_t) *sdec_out_t = ts.s_dec;
    }
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int c = lane & 15, g = lane >> 4;
    const int rg = wv * 4 + g;                                   // 8-row group within the region
    const uint32_t by = blockIdx.x / regions_per_row, bx = blockIdx.x - by * regions_per_row;
    const uint32_t row0 = by * kQ2Region, col0 = bx * kQ2Region;
    const uint32_t r0 = row0 + rg * 8, c0 = col0 + c * 8;
    const bool valid = r0 < rows && c0 < cols;
    const T* src = w + (int64_t)(valid ? r0 : 0) * ld + (valid ? c0 : 0);
    float y[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i) Group8<T>::load(src + i * ld, y[i]);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(y[i][e]));
    m = fmaxf(m, swap_adjacent(m));                  // lane ^ 1: the tile's other column chunk
    m = fmaxf(m, __shfl_xor(m, 16));                 // lane ^ 16: the tile's other row group
    uint32_t sb;
    float enc;
    block_scale(m, ts, sb, enc);
    uint32_t wd[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float z[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = y[i][e] * enc;
        wd[i] = e2m1_rne_pack8(z);
    }
    if (valid) {
        uint8_t* dst = codes + (int64_t)r0 * (cols / 2) + c0 / 2;
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<uint32_t*>(dst + (int64_t)i * (cols / 2)) = wd[i];
        if ((lane & 0x11) == 0) {                    // one lane per tile writes its scale byte(s)
            scales[(int64_t)(r0 / 16) * (cols / 16) + c0 / 16] = (uint8_t)sb;
            if (scales_t) scales_t[(int64_t)(c0 / 16) * (rows / 16) + r0 / 16] = (uint8_t)sb;
        }
    }
    if (!codes_t) return;
    nibble_transpose8(wd);                           // wd[j]: column c0 + j, rows r0 .. r0 + 7
#pragma unroll
    for (int j = 0; j < 8; ++j) stage[c * 8 + j][rg] = wd[j];
    __syncthreads();
    // transposed row (col0 + tc) of [cols x rows]: 16 words for the region's 128 rows
#pragma unroll
    for (int p = 0; p < kQ2Region * 16 / kThreads; ++p) {
        const int idx = p * kThreads + threadIdx.x;
        const int tc = idx >> 4, trg = idx & 15;
        if (col0 + tc < cols && row0 + trg * 8 < rows)
            *reinterpret_cast<uint32_t*>(codes_t + (int64_t)(col0 + tc) * (rows / 2) + row0 / 2 +
                                         trg * 4) = stage[tc][trg];
    }
}

// ---- dequantization -------------------------------------------------------------------------
template <bool kBF16Out>
__global__ void __launch_bounds__(kThreads)
k_dequant(const uint32_t* __restrict__ codes, const uint8_t* __restrict__ scales, int layout,
          const float* __restrict__ sdec_src, uint32_t groups, FastDiv gpr, uint32_t cols,
          void* __restrict__ out, int64_t ld) {
    const float sdec = layout == MXFP4_BLK_1x32 ? 1.0f : *sdec_src;
    const uint32_t base = blockIdx.x * kThreads * kUnroll + threadIdx.x;
    // All loads first (groups past the end load the last group and store nothing).
    uint32_t c[kUnroll], sb[kUnroll], row[kUnroll], cg[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        uint32_t g = base + u * kThreads;
        g = g < groups ? g : groups - 1;
        row[u] = fastdiv(g, gpr);
        cg[u] = g - row[u] * gpr.d;
        c[u] = codes[g];
        const int64_t si = layout == MXFP4_BLK_1x32 ? (int64_t)row[u] * (cols / 32) + cg[u] / 4
                         : layout == NVFP4_BLK_16x16 ? (int64_t)(row[u] / 16) * (cols / 16) + cg[u] / 2
                                                     : (int64_t)row[u] * (cols / 16) + cg[u] / 2;
        sb[u] = scales[si];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        float v[8];
        e2m1_decode8(c[u], v);                       // exact E2M1 values
        if (layout == MXFP4_BLK_1x32) {
            const int e = (int)sb[u] - 127;
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = __builtin_amdgcn_ldexpf(v[i], e);
        } else {
            const float s = e4m3_decode(sb[u]);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = (v[i] * s) * sdec;
        }
        if (base + u * kThreads >= groups) continue;
        if constexpr (kBF16Out) {
            uint4 o;
            o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
            o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
            o.z = f32_to_bf16(v[4]) | (f32_to_bf16(v[5]) << 16);
            o.w = f32_to_bf16(v[6]) | (f32_to_bf16(v[7]) << 16);
            *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + (int64_t)row[u] * ld +
                                      cg[u] * 8) = o;
        } else {
            float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) +
                                                  (int64_t)row[u] * ld + cg[u] * 8);
            o[0] = make_float4(v[0], v[1], v[2], v[3]);
            o[1] = make_float4(v[4], v[5], v[6], v[7]);
        }
    }
}

// ---- MXFP4 quantization (comparison format, [P3 NVFP4 in pratica]) -----------------------------
// Four adjacent lanes hold one 32-element block.  E8M0 exponent = floor(log2 amax_b) - 2.
template <typename T, bool kSR>
__global__ void __launch_bounds__(kThreads)
k_mx_quant(const T* __restrict__ x, int64_t ld, uint32_t groups, FastDiv gpr, uint32_t cols,
           uint64_t seed, uint32_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    const uint32_t base = blockIdx.x * kThreads * kUnroll + threadIdx.x;
    float y[kUnroll][8];
    uint32_t row[kUnroll], cg[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        uint32_t g = base + u * kThreads;
        row[u] = 0; cg[u] = 0;
        if (g < groups) {
            row[u] = fastdiv(g, gpr);
            cg[u] = g - row[u] * gpr.d;
            Group8<T>::load(x + (int64_t)row[u] * ld + cg[u] * 8, y[u]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) y[u][e] = 0.0f;
        }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint32_t g = base + u * kThreads;
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(y[u][e]));
        m = fmaxf(m, swap_adjacent(m));
        m = fmaxf(m, swap_pairs(m));
        int e8 = 0;
        if (m > 0.0f) {
            e8 = __builtin_amdgcn_frexp_expf(m) - 1 - 2;   // m = f 2^E, f in [0.5, 1)
            e8 = e8 < -127 ? -127 : (e8 > 127 ? 127 : e8);
        }
        float z[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = __builtin_amdgcn_ldexpf(y[u][e], -e8);
        uint32_t packed = 0;
        if constexpr (kSR) {
            const uint64_t idx8 = (uint64_t)row[u] * cols + cg[u] * 8;
            const u32x4 w = sr_words(seed, idx8);
            const uint32_t words[4] = {w.x, w.y, w.z, w.w};
            packed = e2m1_sr_pack8(z, words);
        } else {
            packed = e2m1_rne_pack8(z);
        }
        if (g < groups) {
            codes[g] = packed;
            if ((g & 3u) == 0) scales[g >> 2] = (uint8_t)(e8 + 127);
        }
    }
}

// ---- format sweep: quantize-dequantize with a chosen block size and scale format -------------
// [P2 Describir: block size, scale format and rounding are the FP4 design choices explored.]
// One lane per block of B (8, 16 or 32) elements.  kE8M0 = false: E4M3 block scale under the
// per-tensor fp32 scale (the NVFP4 steps); true: E8M0 scale 2^(floor(log2 amax_b) - 2), no
// tensor scale (the MXFP4 steps).  Writes the dequantized fp32 values and, when sums is
// non-NULL, adds sum x^2 and sum (y - x)^2 (fp64, one atomic pair per workgroup).
template <typename T, int B, bool kE8M0, bool kSR>
__global__ void __launch_bounds__(kThreads)
k_qdq(const T* __restrict__ x, int64_t ld, uint32_t blocks, FastDiv bpr, uint32_t cols,
      const float* __restrict__ amax_src, uint64_t seed, float* __restrict__ y, int64_t ldy,
      double* sums) {
    const uint32_t b = blockIdx.x * kThreads + threadIdx.x;
    TensorScales ts{448.0f, 1.0f, 1.0f};
    if constexpr (!kE8M0) ts = tensor_scales(*amax_src);
    double g2 = 0.0, e2 = 0.0;
    if (b < blocks) {
        const uint32_t row = fastdiv(b, bpr), cb = b - row * bpr.d;
        const T* p = x + (int64_t)row * ld + cb * B;
        float v[B];
#pragma unroll
        for (int g = 0; g < B / 8; ++g) Group8<T>::load(p + 8 * g, v + 8 * g);
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < B; ++e) m = fmaxf(m, fabsf(v[e]));
        uint32_t sb = 0;
        float enc = 0.0f;
        int e8 = 0;
        if constexpr (kE8M0) {
            if (m > 0.0f) {
                e8 = __builtin_amdgcn_frexp_expf(m) - 1 - 2;
                e8 = e8 < -127 ? -127 : (e8 > 127 ? 127 : e8);
            }
        } else {
            block_scale(m, ts, sb, enc);
        }
        const float sc = kE8M0 ? 1.0f : e4m3_decode(sb);
        float* out = y + (int64_t)row * ldy + cb * B;
#pragma unroll
        for (int g = 0; g < B / 8; ++g) {
            float z[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                z[e] = kE8M0 ? __builtin_amdgcn_ldexpf(v[8 * g + e], -e8) : v[8 * g + e] * enc;
            uint32_t packed;
            if constexpr (kSR) {
                const u32x4 w = sr_words(seed, (uint64_t)row * cols + cb * B + 8 * g);
                const uint32_t words[4] = {w.x, w.y, w.z, w.w};
                packed = e2m1_sr_pack8(z, words);
            } else {
                packed = e2m1_rne_pack8(z);
            }
            float q[8];
            e2m1_decode8(packed, q);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                q[e] = kE8M0 ? __builtin_amdgcn_ldexpf(q[e], e8) : (q[e] * sc) * ts.s_dec;
            reinterpret_cast<float4*>(out + 8 * g)[0] = make_float4(q[0], q[1], q[2], q[3]);
            reinterpret_cast<float4*>(out + 8 * g)[1] = make_float4(q[4], q[5], q[6], q[7]);
            if (sums) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const double xv = v[8 * g + e], d = (double)q[e] - xv;
                    g2 += xv * xv;
                    e2 += d * d;
                }
            }
        }
    }
    if (sums) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            g2 += __shfl_xor(g2, off);
            e2 += __shfl_xor(e2, off);
        }
        __shared__ double part[2][kThreads / 64];
        if ((threadIdx.x & 63) == 0) {
            part[0][threadIdx.x >> 6] = g2;
            part[1][threadIdx.x >> 6] = e2;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            double a = 0.0, c = 0.0;
#pragma unroll
            for (int w = 0; w < kThreads / 64; ++w) {
                a += part[0][w];
                c += part[1][w];
            }
            atomicAdd(sums, a);
            atomicAdd(sums + 1, c);
        }
    }
}

static int stream_grid(uint32_t groups, int unroll = kUnroll) {
    int64_t n = ((int64_t)groups + kThreads * unroll - 1) / (kThreads * unroll);
    return (int)(n < 1 ? 1 : n);
}

// Launch the amax pass for a dense [rows x cols] input: it raises *dst to the tensor's amax;
// with `accumulate` false *dst is zeroed first.
static nvfp4_status launch_amax(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols,
                                int64_t ld, float* dst, hipStream_t st, bool accumulate = false) {
    if (!accumulate) hipLaunchKernelGGL(k_fill_f32, dim3(1), dim3(1), 0, st, dst, 0.0f);
    const int64_t g64 = rows * (cols / 8);
    if (g64 > 0) {
        const uint32_t groups = (uint32_t)g64;
        const FastDiv gpr = make_fastdiv((uint32_t)(cols / 8));
        const dim3 grid(amax_grid(groups));
        const bool stream = rows * cols * (dt == NVFP4_BF16 ? 2 : 4) >= kStreamBytes;
#define NVFP4_AMAX(TT, NT)                                                                        \
    hipLaunchKernelGGL((k_amax<TT, NT>), grid, dim3(kAmaxThreads), 0, st,                         \
                       static_cast<const TT*>(x), ld, groups, gpr, dst)
        if (dt == NVFP4_BF16) {
            if (stream) NVFP4_AMAX(uint16_t, true); else NVFP4_AMAX(uint16_t, false);
        } else {
            if (stream) NVFP4_AMAX(float, true); else NVFP4_AMAX(float, false);
        }
#undef NVFP4_AMAX
    }
    return launch_status();
}

static bool too_big(int64_t rows, int64_t cols) {
    return rows * (cols / 8) >= (int64_t(1) << 31);
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" const char* nvfp4_status_string(nvfp4_status s) {
    switch (s) {
        case NVFP4_OK: return "ok";
        case NVFP4_ERR_NULL: return "a required pointer is NULL";
        case NVFP4_ERR_SHAPE: return "invalid or mismatched shape";
        case NVFP4_ERR_DTYPE: return "unknown dtype or rounding mode";
        case NVFP4_ERR_ALIGN: return "pointer or row stride not 16-byte aligned";
        case NVFP4_ERR_LAYOUT: return "tensor layout not allowed for this call";
        case NVFP4_ERR_LAUNCH: return "kernel launch failed";
        case NVFP4_ERR_SCRATCH: return "the call needs more than the library's fixed scratch buffer";
    }
    return "unknown status";
}

static nvfp4_status amax_entry(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols,
                               int64_t ld, float* amax_out, void* stream, bool accumulate) {
    nvfp4_status s = check_input(x, dt, rows, cols, ld);
    if (s) return s;
    if (!amax_out) return NVFP4_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(amax_out) & 3u) return NVFP4_ERR_ALIGN;
    if (cols % 8 != 0) return NVFP4_ERR_SHAPE;
    if (too_big(rows, cols)) return NVFP4_ERR_SHAPE;
    return launch_amax(x, dt, rows, cols, ld, amax_out, as_stream(stream), accumulate);
}

extern "C" nvfp4_status nvfp4_amax(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols,
                                   int64_t ld, float* amax_out, void* stream) {
    return amax_entry(x, dt, rows, cols, ld, amax_out, stream, false);
}

extern "C" nvfp4_status nvfp4_amax_accumulate(const void* x, nvfp4_dtype dt, int64_t rows,
                                              int64_t cols, int64_t ld, float* amax_inout,
                                              void* stream) {
    return amax_entry(x, dt, rows, cols, ld, amax_inout, stream, true);
}

static nvfp4_status quantize_1d(const void* x, nvfp4_dtype dt, int64_t ld, const float* amax_in,
                                nvfp4_round rnd, uint64_t seed, const nvfp4_tensor* out,
                                double* sums, hipStream_t st) {
    nvfp4_status s = check_q(out, NVFP4_BLK_1x16, true);
    if (s) return s;
    s = check_input(x, dt, out->rows, out->cols, ld);
    if (s) return s;
    if (rnd != NVFP4_RNE && rnd != NVFP4_SR) return NVFP4_ERR_DTYPE;
    if (too_big(out->rows, out->cols)) return NVFP4_ERR_SHAPE;
    const float* src = amax_in;
    if (!src) {
        s = launch_amax(x, dt, out->rows, out->cols, ld, out->amax, st);
        if (s) return s;
        src = out->amax;
    }
    if (sums) hipLaunchKernelGGL(k_fill_f64x2, dim3(1), dim3(1), 0, st, sums);
    const uint32_t blocks = (uint32_t)(out->rows * (out->cols / 16));
    if (blocks == 0) {
        hipLaunchKernelGGL(k_tensor_scalars, dim3(1), dim3(1), 0, st, src, out->amax, out->s_dec);
        return launch_status();
    }
    const FastDiv bpr = make_fastdiv((uint32_t)(out->cols / 16));
    const int full = stream_grid(blocks, kQUnroll);
    const dim3 grid(sums && full > kNoiseBlocks ? kNoiseBlocks : full), block(kThreads);
    uint2* codes = reinterpret_cast<uint2*>(out->codes);
    const uint32_t cols = (uint32_t)out->cols;
#define NVFP4_Q1(T, SRV, NZ)                                                                     \
    hipLaunchKernelGGL((k_quant1d<T, SRV, NZ>), grid, block, 0, st, static_cast<const T*>(x), ld, \
                       blocks, bpr, cols, src, seed, codes, out->scales, out->amax, out->s_dec,   \
                       sums)
#define NVFP4_Q1R(T, NZ)                                                                          \
    if (rnd == NVFP4_SR) NVFP4_Q1(T, true, NZ); else NVFP4_Q1(T, false, NZ)
    if (dt == NVFP4_BF16) {
        if (sums) NVFP4_Q1R(uint16_t, true); else NVFP4_Q1R(uint16_t, false);
    } else {
        if (sums) NVFP4_Q1R(float, true); else NVFP4_Q1R(float, false);
    }
#undef NVFP4_Q1R
#undef NVFP4_Q1
    return launch_status();
}

extern "C" nvfp4_status nvfp4_quantize_1d(const void* x, nvfp4_dtype dt, int64_t ld,
                                          const float* amax_in, nvfp4_round rnd, uint64_t seed,
                                          const nvfp4_tensor* out, void* stream) {
    return quantize_1d(x, dt, ld, amax_in, rnd, seed, out, nullptr, as_stream(stream));
}

extern "C" nvfp4_status nvfp4_quantize_1d_noise(const void* x, nvfp4_dtype dt, int64_t ld,
                                                const float* amax_in, nvfp4_round rnd,
                                                uint64_t seed, const nvfp4_tensor* out,
                                                double* sums, void* stream) {
    if (!sums) return NVFP4_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(sums) & 7u) return NVFP4_ERR_ALIGN;
    return quantize_1d(x, dt, ld, amax_in, rnd, seed, out, sums, as_stream(stream));
}

extern "C" nvfp4_status nvfp4_quantize_2d(const void* w, nvfp4_dtype dt, int64_t ld,
                                          const float* amax_in, const nvfp4_tensor* out,
                                          const nvfp4_tensor* out_t, void* stream) {
    nvfp4_status s = check_q(out, NVFP4_BLK_16x16, true);
    if (s) return s;
    if (out_t) {
        s = check_q(out_t, NVFP4_BLK_16x16, false);
        if (s) return s;
        if (out_t->rows != out->cols || out_t->cols != out->rows) return NVFP4_ERR_SHAPE;
    }
    s = check_input(w, dt, out->rows, out->cols, ld);
    if (s) return s;
    if (too_big(out->rows, out->cols)) return NVFP4_ERR_SHAPE;
    hipStream_t st = as_stream(stream);
    const float* src = amax_in;
    if (!src) {
        s = launch_amax(w, dt, out->rows, out->cols, ld, out->amax, st);
        if (s) return s;
        src = out->amax;
    }
    float* amax_t = out_t ? out_t->amax : nullptr;
    float* sdec_t = out_t ? out_t->s_dec : nullptr;
    if (out->rows == 0 || out->cols == 0) {
        hipLaunchKernelGGL(k_tensor_scalars, dim3(1), dim3(1), 0, st, src, out->amax, out->s_dec);
        if (out_t) hipLaunchKernelGGL(k_tensor_scalars, dim3(1), dim3(1), 0, st, src, amax_t, sdec_t);
        return launch_status();
    }
    const uint32_t rows = (uint32_t)out->rows, cols = (uint32_t)out->cols;
    const uint32_t rpr = (cols + kQ2Region - 1) / kQ2Region;
    const dim3 grid(rpr * ((rows + kQ2Region - 1) / kQ2Region)), block(kThreads);
    uint8_t* ct = out_t ? out_t->codes : nullptr;
    uint8_t* sct = out_t ? out_t->scales : nullptr;
    if (dt == NVFP4_BF16)
        hipLaunchKernelGGL(k_quant2d<uint16_t>, grid, block, 0, st, static_cast<const uint16_t*>(w),
                           ld, rows, cols, src, out->codes, out->scales, ct, sct, out->amax,
                           out->s_dec, amax_t, sdec_t, rpr);
    else
        hipLaunchKernelGGL(k_quant2d<float>, grid, block, 0, st, static_cast<const float*>(w), ld,
                           rows, cols, src, out->codes, out->scales, ct, sct, out->amax,
                           out->s_dec, amax_t, sdec_t, rpr);
    return launch_status();
}

extern "C" nvfp4_status nvfp4_dequantize(const nvfp4_tensor* q, void* y, nvfp4_dtype dt,
                                         int64_t ld, void* stream) {
    if (!q) return NVFP4_ERR_NULL;
    nvfp4_status s = check_q(q, q->layout, q->layout != MXFP4_BLK_1x32);
    if (s) return s;
    if (q->layout != NVFP4_BLK_1x16 && q->layout != NVFP4_BLK_16x16 && q->layout != MXFP4_BLK_1x32)
        return NVFP4_ERR_LAYOUT;
    s = check_input(y, dt, q->rows, q->cols, ld);
    if (s) return s;
    if (too_big(q->rows, q->cols)) return NVFP4_ERR_SHAPE;
    const uint32_t groups = (uint32_t)(q->rows * (q->cols / 8));
    if (groups == 0) return NVFP4_OK;
    const FastDiv gpr = make_fastdiv((uint32_t)(q->cols / 8));
    const dim3 grid(stream_grid(groups)), block(kThreads);
    hipStream_t st = as_stream(stream);
    const uint32_t* codes = reinterpret_cast<const uint32_t*>(q->codes);
    if (dt == NVFP4_BF16)
        hipLaunchKernelGGL(k_dequant<true>, grid, block, 0, st, codes, q->scales, (int)q->layout,
                           q->s_dec, groups, gpr, (uint32_t)q->cols, y, ld);
    else
        hipLaunchKernelGGL(k_dequant<false>, grid, block, 0, st, codes, q->scales, (int)q->layout,
                           q->s_dec, groups, gpr, (uint32_t)q->cols, y, ld);
    return launch_status();
}

extern "C" nvfp4_status mxfp4_quantize_1d(const void* x, nvfp4_dtype dt, int64_t ld, nvfp4_round rnd,
                                          uint64_t seed, const nvfp4_tensor* out, void* stream) {
    nvfp4_status s = check_q(out, MXFP4_BLK_1x32, false);
    if (s) return s;
    s = check_input(x, dt, out->rows, out->cols, ld);
    if (s) return s;
    if (rnd != NVFP4_RNE && rnd != NVFP4_SR) return NVFP4_ERR_DTYPE;
    if (too_big(out->rows, out->cols)) return NVFP4_ERR_SHAPE;
    const uint32_t groups = (uint32_t)(out->rows * (out->cols / 8));
    if (groups == 0) return NVFP4_OK;
    const FastDiv gpr = make_fastdiv((uint32_t)(out->cols / 8));
    const dim3 grid(stream_grid(groups)), block(kThreads);
    hipStream_t st = as_stream(stream);
    uint32_t* codes = reinterpret_cast<uint32_t*>(out->codes);
    const uint32_t cols = (uint32_t)out->cols;
#define NVFP4_MXQ(T, SRV)                                                                        \
    hipLaunchKernelGGL((k_mx_quant<T, SRV>), grid, block, 0, st, static_cast<const T*>(x), ld,    \
                       groups, gpr, cols, seed, codes, out->scales)
    if (dt == NVFP4_BF16) {
        if (rnd == NVFP4_SR) NVFP4_MXQ(uint16_t, true); else NVFP4_MXQ(uint16_t, false);
    } else {
        if (rnd == NVFP4_SR) NVFP4_MXQ(float, true); else NVFP4_MXQ(float, false);
    }
#undef NVFP4_MXQ
    return launch_status();
}

extern "C" nvfp4_status nvfp4_qdq(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols,
                                  int64_t ld, int32_t block, int32_t scale_fmt,
                                  const float* amax_in, nvfp4_round rnd, uint64_t seed, float* y,
                                  int64_t ldy, float* amax_out, double* sums, void* stream) {
    nvfp4_status s = check_input(x, dt, rows, cols, ld);
    if (s) return s;
    if (block != 8 && block != 16 && block != 32) return NVFP4_ERR_SHAPE;
    if (scale_fmt != 0 && scale_fmt != 1) return NVFP4_ERR_DTYPE;
    if (rnd != NVFP4_RNE && rnd != NVFP4_SR) return NVFP4_ERR_DTYPE;
    if (cols % block != 0 || too_big(rows, cols)) return NVFP4_ERR_SHAPE;
    s = check_input(y, NVFP4_F32, rows, cols, ldy);
    if (s) return s;
    if (scale_fmt == 0 && !amax_in && !amax_out) return NVFP4_ERR_NULL;
    if (amax_out && (reinterpret_cast<uintptr_t>(amax_out) & 3u)) return NVFP4_ERR_ALIGN;
    if (sums && (reinterpret_cast<uintptr_t>(sums) & 7u)) return NVFP4_ERR_ALIGN;
    hipStream_t st = as_stream(stream);
    const float* src = amax_in;
    if (scale_fmt == 0 && !src) {
        s = launch_amax(x, dt, rows, cols, ld, amax_out, st);
        if (s) return s;
        src = amax_out;
    } else if (amax_out) {
        hipLaunchKernelGGL(k_tensor_scalars, dim3(1), dim3(1), 0, st,
                           scale_fmt == 0 ? src : nullptr, amax_out, nullptr);
    }
    if (sums) hipLaunchKernelGGL(k_fill_f64x2, dim3(1), dim3(1), 0, st, sums);
    const uint32_t blocks = (uint32_t)(rows * (cols / block));
    if (blocks == 0) return launch_status();
    const FastDiv bpr = make_fastdiv((uint32_t)(cols / block));
    const dim3 grid((blocks + kThreads - 1) / kThreads), blk(kThreads);
#define NVFP4_QDQ(TT, BB, E8, SRV)                                                                \
    hipLaunchKernelGGL((k_qdq<TT, BB, E8, SRV>), grid, blk, 0, st, static_cast<const TT*>(x), ld, \
                       blocks, bpr, (uint32_t)cols, src, seed, y, ldy, sums)
#define NVFP4_QDQ_R(TT, BB, E8)                                                                   \
    if (rnd == NVFP4_SR) NVFP4_QDQ(TT, BB, E8, true); else NVFP4_QDQ(TT, BB, E8, false)
#define NVFP4_QDQ_F(TT, BB)                                                                       \
    if (scale_fmt == 1) NVFP4_QDQ_R(TT, BB, true); else NVFP4_QDQ_R(TT, BB, false)
#define NVFP4_QDQ_B(TT)                                                                           \
    if (block == 8) NVFP4_QDQ_F(TT, 8); else if (block == 16) NVFP4_QDQ_F(TT, 16);               \
    else NVFP4_QDQ_F(TT, 32)
    if (dt == NVFP4_BF16) { NVFP4_QDQ_B(uint16_t); } else { NVFP4_QDQ_B(float); }
#undef NVFP4_QDQ_B
#undef NVFP4_QDQ_F
#undef NVFP4_QDQ_R
#undef NVFP4_QDQ
    return launch_status();
}
