// gdn_convert.hip -- fp32 <-> binary16 state pool converters.
//
// metrale "layers/ops/ssm_gdn_a.rs", `ssm_h_state_f32_to_f16` /
// `ssm_h_state_f16_to_f32`: grid-stride element-wise conversion of a whole state
// pool, round to nearest even on narrowing, src and dst distinct.  Here each
// thread moves 8 elements per iteration (two float4 <-> one 16-byte binary16
// vector) so every access is a 16-byte load or store; a scalar loop covers the
// n % 8 tail.  The narrowing uses the hardware fp32 -> binary16 conversion,
// which rounds to nearest even with binary16 subnormals kept (the default
// floating-point mode of a HIP kernel).
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kCvtThreads = 256;

__global__ void __launch_bounds__(kCvtThreads) f32_to_f16_kernel(const float *__restrict__ src,
                                                                uint16_t *__restrict__ dst,
                                                                int64_t n) {
    const int64_t nvec = n / 8;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t first = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const f32x4 *s4 = reinterpret_cast<const f32x4 *>(src);
    half8 *d8 = reinterpret_cast<half8 *>(dst);
    for (int64_t i = first; i < nvec; i += stride) {
        const f32x4 a = __builtin_nontemporal_load(s4 + 2 * i);
        const f32x4 b = __builtin_nontemporal_load(s4 + 2 * i + 1);
        half8 hv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            hv[e] = (_Float16)a[e];
            hv[4 + e] = (_Float16)b[e];
        }
        __builtin_nontemporal_store(hv, d8 + i);
    }
    for (int64_t i = nvec * 8 + first; i < n; i += stride) {
        const _Float16 hv = (_Float16)src[i];
        dst[i] = __builtin_bit_cast(uint16_t, hv);
    }
}

__global__ void __launch_bounds__(kCvtThreads) f16_to_f32_kernel(const uint16_t *__restrict__ src,
                                                                float *__restrict__ dst,
                                                                int64_t n) {
    const int64_t nvec = n / 8;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t first = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const half8 *s8 = reinterpret_cast<const half8 *>(src);
    f32x4 *d4 = reinterpret_cast<f32x4 *>(dst);
    for (int64_t i = first; i < nvec; i += stride) {
        const half8 hv = __builtin_nontemporal_load(s8 + i);
        f32x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[e] = (float)hv[e];
            b[e] = (float)hv[4 + e];
        }
        __builtin_nontemporal_store(a, d4 + 2 * i);
        __builtin_nontemporal_store(b, d4 + 2 * i + 1);
    }
    for (int64_t i = nvec * 8 + first; i < n; i += stride)
        dst[i] = (float)__builtin_bit_cast(_Float16, src[i]);
}

static unsigned cvt_grid(int64_t n) {
    // enough waves to fill 256 CUs several times over; the loops are grid-stride
    int64_t blocks = (n / 8 + kCvtThreads - 1) / kCvtThreads;
    if (blocks < 1) blocks = 1;
    if (blocks > 4096) blocks = 4096;
    return (unsigned)blocks;
}

hipError_t launch_f32_to_f16(const float *src, uint16_t *dst, int64_t n, hipStream_t stream) {
    return launch(f32_to_f16_kernel, dim3(cvt_grid(n)), dim3(kCvtThreads), 0, stream, src, dst, n);
}

hipError_t launch_f16_to_f32(const uint16_t *src, float *dst, int64_t n, hipStream_t stream) {
    return launch(f16_to_f32_kernel, dim3(cvt_grid(n)), dim3(kCvtThreads), 0, stream, src, dst, n);
}

}  // namespace gdn
