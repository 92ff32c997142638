// gdn_device.h -- device helpers shared by the gfx950 kernels of libgdn.
//
// Wave64 cross-lane sums use DPP (data-parallel primitives): a lane reads a
// register of another lane of its 16-lane DPP row as an operand, without going
// through LDS.  The 32-lane warp shuffles of the CUDA kernels on the pages are
// replaced by these in-row patterns:
//   quad_perm [1,0,3,2]  = lane ^ 1
//   quad_perm [2,3,0,1]  = lane ^ 2
//   row_half_mirror      = lane ^ 7 within each 8-lane half-row
//   row_mirror           = lane ^ 15 within the 16-lane row
// After ^1 and ^2 every lane of a quad holds the quad's sum, so the two mirrors
// pair each quad with the other quad of its half-row, then each half-row with
// the other half.  Every lane of the group ends with the same bits (addition
// is commutative), and the order is fixed, so results are deterministic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kDppXor1 = 0xB1;        // quad_perm(1,0,3,2)
constexpr int kDppXor2 = 0x4E;        // quad_perm(2,3,0,1)
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

template <int CTRL>
__device__ __forceinline__ float dpp_get(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over an aligned group of N consecutive lanes (N in 1, 2, 4, 8, 16); every
// lane of the group receives the total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group width");
    if constexpr (N >= 2) x += dpp_get<kDppXor1>(x);
    if constexpr (N >= 4) x += dpp_get<kDppXor2>(x);
    if constexpr (N >= 8) x += dpp_get<kDppHalfMirror>(x);
    if constexpr (N >= 16) x += dpp_get<kDppMirror>(x);
    return x;
}

// Sum over an aligned group of N consecutive lanes for any power of two N <= 64
// (used off the per-token path).  Beyond 16 lanes it exchanges through
// ds_bpermute (hardware lane crossbar).
template <int N>
__device__ __forceinline__ float group_sum_wide(float x) {
    if constexpr (N <= 16) {
        return group_sum<N>(x);
    } else {
        x = group_sum<16>(x);
#pragma unroll
        for (int off = 16; off < N; off <<= 1) x += __shfl_xor(x, off, 64);
        return x;
    }
}

// Maximum over each aligned group of 32 lanes of a wave64 (ds_bpermute).
__device__ __forceinline__ float group_max32(float x) {
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 32));
    return x;
}

// fp32 -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// silu(z) = z sigmoid(z), with the IEEE division and a full-precision exp.
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

}  // namespace gdn
