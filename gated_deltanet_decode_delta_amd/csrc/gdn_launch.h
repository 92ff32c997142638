// gdn_launch.h -- internal interface between the C ABI (gdn_api.hip) and the
// kernel translation units.  Not installed; the public contract is gdn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Everything a decode or sequence launch needs; strides in elements.
struct StepArgs {
    void *state;             // fp32 or binary16 pool
    int64_t pitch;           // elements of the state type per sequence slot
    const float *q;
    const float *k;
    int64_t qk_stride;
    const float *v;
    int64_t v_stride;
    const float *alpha;
    const float *beta;
    int64_t ab_stride;
    const float *z;          // NULL: raw output
    int64_t z_stride;
    const float *gn;
    float eps;
    float scale;             // 1 / sqrt(Dk)
    void *out;               // kOutNormQ8: fp32 y, may be NULL
    int64_t out_stride;
    int8_t *codes;           // kOutNormQ8: int8 codes of y, rows codes_stride apart
    int64_t codes_stride;
    float *scales;           // kOutNormQ8: one scale per 32 values, rows scales_stride apart
    int64_t scales_stride;
    int32_t batch;
    int32_t seq_len;         // 1 for decode
    int32_t nk;
    int32_t nv;
};

// The layer's input stage fused in front of the decode: conv ring, weights,
// raw gate inputs and per-head gate parameters (strides in elements).
struct FrontArgs {
    float *ring;             // [B] slots of taps rows of C = (2 NK + NV) D channels
    int64_t ring_stride;
    const float *x;          // this token's projection rows, channels q | k | v
    int64_t x_stride;
    const float *w;          // [taps][C]
    int32_t taps;
    const float *br;         // write-strength logits, rows g_stride apart
    const float *ar;         // decay inputs, same rows
    int64_t g_stride;
    const float *dt;         // [NV] decay bias
    const float *rate;       // [NV] decay exponent (negative)
    float l2_eps;
};

constexpr int kMaxTaps = 8;

// Launches `kernel` and returns the status of that launch alone.  A failed HIP
// call stays recorded in its thread until hipGetLastError reads it, so reading
// that after a <<<>>> launch would report an earlier failure of the caller's
// as the library's own.
template <typename T>
struct Same {
    using type = T;
};
template <typename... P>
inline hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                         typename Same<P>::type... args) {
    void *argv[] = {static_cast<void *>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, lds, stream);
}

enum OutMode { kOutRawF32 = 0, kOutNormF32 = 1, kOutNormBF16 = 2, kOutNormQ8 = 3 };

hipError_t launch_decode(const StepArgs &a, int dim, bool f16_state, OutMode mode,
                         hipStream_t stream);
hipError_t launch_seq(const StepArgs &a, int dim, OutMode mode, hipStream_t stream);
hipError_t launch_verify(const StepArgs &a, int dim, float *inter, int64_t inter_pitch, bool norm,
                         hipStream_t stream);
// ring_out NULL: the ring is updated in place (one workgroup per key head);
// otherwise the new ring goes to ring_out (one workgroup per value head)
hipError_t launch_fused(const StepArgs &a, const FrontArgs &f, float *ring_out, int dim, bool norm,
                        hipStream_t stream);
size_t fused_lds_bytes(int dim, int heads_per_key_head);
hipError_t launch_seq_mfma(const StepArgs &a, OutMode mode, hipStream_t stream);   // dim 128
// dim 128 without a workspace: one workgroup per (sequence, key head, quarter)
// forming its chunk quantities itself; seq_group_fits says whether the shape
// suits it (at most three value heads per key head, 32-bit lane offsets)
bool seq_group_fits(const StepArgs &a);
hipError_t launch_seq_group(const StepArgs &a, OutMode mode, hipStream_t stream);
// Floats of one workspace record of the split sequence path: one per (sequence,
// value head, 16-token chunk) -- T and G (16x16 each, row-major), beta, P and D.
constexpr int kSeqRec = 576;
// dim 128: chunk pre-pass into ws, then the state pass (four workgroups per
// head) writing raw o; with a.z set, then the gated norm over the output rows
hipError_t launch_seq_split(const StepArgs &a, float *ws, hipStream_t stream);
// the gated norm over T-token output rows in place (a.out raw o, a.z, a.gn; dim 128)
hipError_t launch_norm_rows(const StepArgs &a, hipStream_t stream);
hipError_t launch_f32_to_f16(const float *src, uint16_t *dst, int64_t n, hipStream_t stream);
hipError_t launch_f16_to_f32(const uint16_t *src, float *dst, int64_t n, hipStream_t stream);

}  // namespace gdn
