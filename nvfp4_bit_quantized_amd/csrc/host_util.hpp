// host_util.hpp -- argument validation and launch helpers shared by the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nvfp4.h"

namespace nvfp4 {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t dtype_size(nvfp4_dtype dt) { return dt == NVFP4_F32 ? 4 : 2; }

inline bool dtype_ok(nvfp4_dtype dt) { return dt == NVFP4_F32 || dt == NVFP4_BF16; }

// A dense input matrix: rows >= 0, ld >= cols, 16-byte aligned rows.
inline nvfp4_status check_input(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols,
                                int64_t ld) {
    if (!dtype_ok(dt)) return NVFP4_ERR_DTYPE;
    if (rows < 0 || cols < 0 || ld < cols) return NVFP4_ERR_SHAPE;
    if (rows > 0 && cols > 0 && !x) return NVFP4_ERR_NULL;
    if (x && (!aligned16(x) || (ld * (int64_t)dtype_size(dt)) % 16 != 0)) return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

// A GEMM output [rows x cols] with row stride ld: element-aligned (results are stored one
// element at a time), ld >= cols.
inline nvfp4_status check_output(const void* c, nvfp4_dtype dt, int64_t rows, int64_t cols,
                                 int64_t ld) {
    if (!dtype_ok(dt)) return NVFP4_ERR_DTYPE;
    if (rows < 0 || cols < 0 || ld < cols) return NVFP4_ERR_SHAPE;
    if (rows > 0 && cols > 0 && !c) return NVFP4_ERR_NULL;
    if (c && (reinterpret_cast<uintptr_t>(c) % dtype_size(dt)) != 0) return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

// An NVFP4/MXFP4 tensor descriptor with the given layout.
inline nvfp4_status check_q(const nvfp4_tensor* q, int32_t layout, bool need_scalars) {
    if (!q) return NVFP4_ERR_NULL;
    if (q->layout != layout || q->reserved != 0) return NVFP4_ERR_LAYOUT;
    if (q->rows < 0 || q->cols < 0) return NVFP4_ERR_SHAPE;
    int64_t kb = layout == MXFP4_BLK_1x32 ? 32 : 16;
    if (q->cols % kb != 0) return NVFP4_ERR_SHAPE;
    if (layout == NVFP4_BLK_16x16 && q->rows % 16 != 0) return NVFP4_ERR_SHAPE;
    bool empty = q->rows == 0 || q->cols == 0;
    if (!empty && (!q->codes || !q->scales)) return NVFP4_ERR_NULL;
    if (need_scalars && (!q->amax || !q->s_dec)) return NVFP4_ERR_NULL;
    if ((q->codes && !aligned16(q->codes)) || (q->scales && !aligned16(q->scales)))
        return NVFP4_ERR_ALIGN;
    if ((q->amax && (reinterpret_cast<uintptr_t>(q->amax) & 3u)) ||
        (q->s_dec && (reinterpret_cast<uintptr_t>(q->s_dec) & 3u)))
        return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

inline nvfp4_status launch_status() {
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_LAUNCH;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Division n / d for 32-bit n by a fixed divisor, as a multiply-high and a shift (Granlund and
// Montgomery's round-up method); exact for every n < 2^31.
struct FastDiv {
    uint32_t d, mul, shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f{d, 0, 0};
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    f.shift = s;
    f.mul = (uint32_t)((((1ull << 32) * ((1ull << s) - d)) / d) + 1);
    return f;
}

__device__ __forceinline__ uint32_t fastdiv(uint32_t n, const FastDiv& f) {
    uint32_t t = __umulhi(n, f.mul);
    return (t + n) >> f.shift;
}

}  // namespace nvfp4
