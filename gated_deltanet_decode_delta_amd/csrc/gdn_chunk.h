// gdn_chunk.h -- device helpers of the 16-token chunked sequence kernels at
// D = 128 (gdn_seq_split.hip, gdn_seq_group.hip): the fp32 matrix-core product,
// the in-row suffix product step and raw buffer loads/stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {
namespace chunk {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kC = 16;            // tokens per chunk
// LDS row strides (floats).  A 16-byte read by lanes (g, li) of row li,
// columns 4g .. 4g + 3 is served without bank conflicts on gfx950 when 32
// lanes fall into distinct 16-byte slots of a 512-byte window, i.e. when the
// row stride in 16-byte units is 2 mod 4: 24 floats for the 16x16 chunk
// matrices (20 cost four extra cycles per read).  The k / q rows keep 132:
// 136 frees their 16-byte reads but puts two-way conflicts on the update's
// 4-byte reads of a column (token 4g + s, column li), which 132 serves
// conflict-free, and measured slower.
constexpr int kKS = kD + 4;       // a chunk's k / q rows
constexpr int kTS = kC + 8;       // the 16x16 chunk matrices

// One 16x16x4 fp32 matrix-core product: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; the accumulator holds D[4 (l / 16) + r][l % 16] in its
// register r.
__device__ __forceinline__ f32x4 mfma(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// The value of the lane N places higher in the same 16-lane DPP row, or 1 past
// the end of the row (a step of an in-row suffix product).
template <int N>
__device__ __forceinline__ float dpp_from_above(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(x), 0x100 + N,
                                                      0xF, 0xF, false));
}

// The value of the lane N places lower in the same 16-lane DPP row, or 1 before
// its start (a step of an in-row prefix product).
template <int N>
__device__ __forceinline__ float dpp_from_below(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(x), 0x110 + N,
                                                      0xF, 0xF, false));
}

// Raw buffer descriptors.  A descriptor covers nbytes from p (stride 0); the
// hardware range check on the lane offset (offset + instruction offset) makes
// a load at or past nbytes return 0 and drops a store there.  The kernels move
// each descriptor's base to the chunk's first row, so that the lane offsets
// stay fixed over the loop and the rows past T need no predicate.  Callers keep
// every extent below 2^31 bytes.
__device__ inline __amdgpu_buffer_rsrc_t buf_rsrc(const float *p, int64_t nbytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p), (short)0,
                                             nbytes > 0 ? (int)nbytes : 0, 0x00020000);
}
__device__ inline f32x4 buf_load4(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ inline float buf_load1(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ inline void buf_store1(__amdgpu_buffer_rsrc_t r, int off, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), r, off, 0, 0);
}

}  // namespace chunk
}  // namespace gdn
