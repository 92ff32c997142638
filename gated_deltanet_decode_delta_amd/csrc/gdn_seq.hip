// gdn_seq.hip -- T-token gated delta rule recurrence with the state on chip.
//
// metrale "layers/ops/ssm_gdn_a.rs", `gdn_prefill_regresident`: the recurrence
// runs token by token inside one launch with the head state held in registers,
// so each state slot is read once at the start and written once at the end,
// whatever the sequence length.
//
// This token loop serves every head dim except D = 128, which launch_seq sends
// to the chunked matrix-core kernel of gdn_seq_mfma.hip.
//
// Mapping (gfx950).  Rows of a head's state are independent given the head's
// per-token k, q, alpha and beta, so without the fused norm a head is split
// over RB workgroups of D/RB rows each (RB = 4 for D >= 64).  With the norm a
// workgroup owns the whole head.  Row i is held by L = 8 lanes, each
// keeping D/8 of its columns in VGPRs; S_i.k and S_i.q are in-row DPP
// all-reductions, so no barrier is needed per token.  The lanes of a row own
// 16-byte column pieces interleaved across the row, so each per-token LDS read
// of k or q is 128 contiguous bytes (broadcast to every row, no bank conflict).
//
// Deferred decay.  Within a chunk of TC tokens the state is kept as
// S_t = P_t * R_t with P_t the running product of alpha over the chunk.  Then
//     coef_t = beta_t (v_t - P_t (R k_t)),   o_t = (P_t (R q_t) + coef_t (k_t.q_t)) / sqrt(D),
//     R <- R + (coef_t / P_t) k_t^T,
// one FMA per state element instead of a multiply and an FMA, and R is folded
// back (S = P_last R) once per chunk.  If a chunk's running product leaves
// [2^-40, 2^40] (strong forgetting, alpha near 0) or is not finite, that chunk
// takes the direct update S <- alpha S + coef k^T instead, so any alpha works.
//
// Per-token inputs are staged through LDS in chunks of TC tokens.  At the start
// of a chunk every thread issues its global loads for the NEXT chunk into
// registers, hiding their latency behind the current chunk; the chunk's
// outputs collect in LDS.  At the chunk end (one barrier) the outputs are
// written as coalesced float4 rows -- with the gated RMS norm of logicaffeine
// "codegen_cuda/gdn.rs" `gdn_gate_norm` when z is given -- then the prefetched
// inputs are stored, k.q is reduced per token and the chunk's decay products are
// scanned with DPP (second barrier).  Staging and epilogue share one thread <->
// 16-byte piece mapping, so a thread overwrites only the z piece it consumed.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <int D, bool NORM>
struct SeqTile {
    static constexpr int L = (NORM && D >= 256) ? 4 : (D / 4 < 8 ? D / 4 : 8);  // lanes per row
    static constexpr int C = D / L;                        // state columns per lane
    static constexpr int NCH = C / 4;                      // float4 pieces per lane and row
    static constexpr int RB = (!NORM && D >= 64) ? 4 : 1;  // workgroups per head
    static constexpr int ROWS = D / RB;                    // rows per workgroup
    static constexpr int NT = ROWS * L < 64 ? 64 : ROWS * L;
    static constexpr int TC = D > 128 ? 8 : 16;            // tokens per staged chunk
    static constexpr int TPT = D / 4;                      // 16-byte pieces per token row of k/q/z
    static constexpr int JKQ = (TC * TPT + NT - 1) / NT;   // k/q/z pieces per thread
    static constexpr int VPT = ROWS / 4 < 1 ? 1 : ROWS / 4;// 16-byte pieces per token of v and o
    static constexpr int JV = (TC * VPT + NT - 1) / NT;    // v/o pieces per thread
    static constexpr bool KEEP_K = NCH <= 8;               // k pieces stay in VGPRs for the update
    static constexpr int WPE = NT >= 1024 ? 4 : 3;         // waves per SIMD the compiler may assume
    static_assert(C % 4 == 0, "float4 pieces");
    static_assert(NT % TPT == 0, "a token's pieces sit in consecutive lanes");
    static_assert(TC <= 16, "one DPP row scans the chunk's decays");
    static_assert(ROWS % 4 == 0 || ROWS < 4, "v/o rows in 16-byte pieces");
};

constexpr float kScaleLo = 0x1p-40f;
constexpr float kScaleHi = 0x1p40f;

// inclusive product over the lanes of a 16-lane DPP row (a lane with no
// left neighbour at distance d sees 1.0 through the DPP "old" operand)
__device__ __forceinline__ float row_prefix_product(float x) {
    x *= __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(x), 0x111, 0xF, 0xF, false));
    x *= __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(x), 0x112, 0xF, 0xF, false));
    x *= __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(x), 0x114, 0xF, 0xF, false));
    x *= __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(x), 0x118, 0xF, 0xF, false));
    return x;
}

template <int D, bool NORM>
__global__ void __launch_bounds__((SeqTile<D, NORM>::NT)) __attribute__((amdgpu_waves_per_eu(1, SeqTile<D, NORM>::WPE)))
seq_kernel(StepArgs a) {
    using TL = SeqTile<D, NORM>;
    constexpr int L = TL::L, NCH = TL::NCH, C = TL::C, TC = TL::TC, TPT = TL::TPT;
    constexpr int NT = TL::NT, RB = TL::RB, ROWS = TL::ROWS, VPT = TL::VPT;
    constexpr int JKQ = TL::JKQ, JV = TL::JV;
    constexpr bool KEEP_K = TL::KEEP_K;

    __shared__ float4 k_s[TC * TPT], q_s[TC * TPT];
    __shared__ float4 z_s[NORM ? TC * TPT : 1];
    __shared__ float4 v_s[TC * VPT], o_s[TC * VPT];
    __shared__ float4 par_s[TC];      // beta, P, 1/P, k.q
    __shared__ float fold_s;          // S = fold * R at the chunk end; 0 marks a direct-update chunk

    const int wg = blockIdx.x;
    const int head = wg / RB;
    const int rb = wg - head * RB;
    const int b = head / a.nv;
    const int h = head - b * a.nv;
    const int g = h % a.nk;  // tiled key-head pairing
    const int T = a.seq_len;
    const int tid = threadIdx.x;
    const int r = tid / L;            // row within the workgroup
    const int p = tid % L;            // lane within the row
    const bool row_active = r < ROWS;
    const int row = rb * ROWS + r;    // row of the head's state
    const int64_t row_base = (int64_t)b * T;

    float *slot = static_cast<float *>(a.state) + (int64_t)b * a.pitch + (int64_t)h * (D * D);

    float s[C];
    if (row_active) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const float4 x = *reinterpret_cast<const float4 *>(slot + (int64_t)row * D + (i * L + p) * 4);
            s[4 * i + 0] = x.x; s[4 * i + 1] = x.y; s[4 * i + 2] = x.z; s[4 * i + 3] = x.w;
        }
    }
    float4 gn4[NORM ? JKQ : 1];
    if constexpr (NORM) {
#pragma unroll
        for (int j = 0; j < JKQ; ++j)
            gn4[j] = *reinterpret_cast<const float4 *>(a.gn + ((tid + j * NT) % TPT) * 4);
    }

    // prefetch registers for one chunk
    float4 pk[JKQ], pq[JKQ], pz[NORM ? JKQ : 1], pv[JV];
    float pal = 1.0f, pbe = 0.0f;
    auto prefetch = [&](int t0) {
        const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int j = 0; j < JKQ; ++j) {
            const int idx = tid + j * NT;
            const int tt = idx / TPT, col = (idx % TPT) * 4;
            pk[j] = pq[j] = zero;
            if constexpr (NORM) pz[j] = zero;
            if (idx < TC * TPT && t0 + tt < T) {
                const int64_t rr = row_base + t0 + tt;
                pk[j] = *reinterpret_cast<const float4 *>(a.k + rr * a.qk_stride + (int64_t)g * D + col);
                pq[j] = *reinterpret_cast<const float4 *>(a.q + rr * a.qk_stride + (int64_t)g * D + col);
                if constexpr (NORM)
                    pz[j] = *reinterpret_cast<const float4 *>(a.z + rr * a.z_stride + (int64_t)h * D + col);
            }
        }
#pragma unroll
        for (int j = 0; j < JV; ++j) {
            const int idx = tid + j * NT;
            const int tt = idx / VPT, col = (idx % VPT) * 4;
            pv[j] = zero;
            if (idx < TC * VPT && t0 + tt < T) {
                const int64_t rr = row_base + t0 + tt;
                const float *src = a.v + rr * a.v_stride + (int64_t)h * D + rb * ROWS + col;
                if constexpr (ROWS >= 4) pv[j] = *reinterpret_cast<const float4 *>(src);
                else pv[j].x = src[0];
            }
        }
        pal = 1.0f;
        pbe = 0.0f;
        if (tid < TC && t0 + tid < T) {
            const int64_t rr = row_base + t0 + tid;
            pal = a.alpha[rr * a.ab_stride + h];
            pbe = a.beta[rr * a.ab_stride + h];
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int j = 0; j < JKQ; ++j) {
            const int idx = tid + j * NT;
            if (idx < TC * TPT) {   // uniform over each token's TPT consecutive lanes
                k_s[idx] = pk[j];
                q_s[idx] = pq[j];
                if constexpr (NORM) z_s[idx] = pz[j];
                float kq = pk[j].x * pq[j].x;
                kq = fmaf(pk[j].y, pq[j].y, kq);
                kq = fmaf(pk[j].z, pq[j].z, kq);
                kq = fmaf(pk[j].w, pq[j].w, kq);
                kq = group_sum_wide<TPT>(kq);
                if (idx % TPT == 0) par_s[idx / TPT].w = kq;
            }
        }
#pragma unroll
        for (int j = 0; j < JV; ++j) {
            const int idx = tid + j * NT;
            if (idx < TC * VPT) v_s[idx] = pv[j];
        }
        if (tid < 16) {   // the chunk's decay products, lanes 0..TC-1 of wave 0
            const float P = row_prefix_product(pal);
            float lo = P, hi = P;
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) {
                lo = fminf(lo, __shfl_xor(lo, off, 16));
                hi = fmaxf(hi, __shfl_xor(hi, off, 16));
            }
            const float last = __shfl(P, TC - 1, 16);
            const bool direct = !(lo >= kScaleLo && hi <= kScaleHi);   // also catches NaN
            if (tid < TC) {
                par_s[tid].x = pbe;
                par_s[tid].y = direct ? pal : P;
                par_s[tid].z = direct ? 1.0f : 1.0f / P;
            }
            if (tid == 0) fold_s = direct ? 0.0f : last;
        }
    };

    prefetch(0);
    stage();
    // Drain every outstanding load (the state rows included) before the chunk
    // loop: otherwise the compiler keeps conservative vmcnt waits inside the
    // token loop, which would also wait for the next chunk's prefetch.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int t0 = 0; t0 < T; t0 += TC) {
        const bool has_next = t0 + TC < T;
        if (has_next) prefetch(t0 + TC);
        const int nt = T - t0 < TC ? T - t0 : TC;
        const float fold = fold_s;
        const bool direct = fold == 0.0f;

        if (row_active) {
            for (int tt = 0; tt < nt; ++tt) {
                const float4 par = par_s[tt];
                float4 kv[KEEP_K ? NCH : 1];
                float pu = 0.f, pw = 0.f;
#pragma unroll
                for (int i = 0; i < NCH; ++i) {
                    const float4 k4 = k_s[tt * TPT + i * L + p];
                    if constexpr (KEEP_K) kv[i] = k4;
                    const float4 q4 = q_s[tt * TPT + i * L + p];
                    pu = fmaf(s[4 * i + 0], k4.x, pu);
                    pu = fmaf(s[4 * i + 1], k4.y, pu);
                    pu = fmaf(s[4 * i + 2], k4.z, pu);
                    pu = fmaf(s[4 * i + 3], k4.w, pu);
                    pw = fmaf(s[4 * i + 0], q4.x, pw);
                    pw = fmaf(s[4 * i + 1], q4.y, pw);
                    pw = fmaf(s[4 * i + 2], q4.z, pw);
                    pw = fmaf(s[4 * i + 3], q4.w, pw);
                    if constexpr (!KEEP_K) {
                        if (i % 4 == 3) __builtin_amdgcn_sched_barrier(0);
                    }
                }
                const float u = group_sum<L>(pu);
                const float w = group_sum<L>(pw);
                const float vr = reinterpret_cast<const float *>(v_s)[tt * (VPT * 4) + r];
                const float coef = par.x * (vr - par.y * u);
                const float o = (par.y * w + coef * par.w) * a.scale;
                const float dk = coef * par.z;
                // A direct-update chunk decays the state first (uniform branch);
                // the k-update below is then shared, in place, by both cases.
                if (direct) {
#pragma unroll
                    for (int i = 0; i < C; ++i) s[i] *= par.y;
                }
#pragma unroll
                for (int i = 0; i < NCH; ++i) {
                    const float4 k4 = KEEP_K ? kv[KEEP_K ? i : 0] : k_s[tt * TPT + i * L + p];
                    s[4 * i + 0] = fmaf(dk, k4.x, s[4 * i + 0]);
                    s[4 * i + 1] = fmaf(dk, k4.y, s[4 * i + 1]);
                    s[4 * i + 2] = fmaf(dk, k4.z, s[4 * i + 2]);
                    s[4 * i + 3] = fmaf(dk, k4.w, s[4 * i + 3]);
                }
                // every lane of the row holds the same o, so all of them store it
                reinterpret_cast<float *>(o_s)[tt * (VPT * 4) + r] = o;
            }
            if (!direct) {
#pragma unroll
                for (int i = 0; i < C; ++i) s[i] *= fold;
            }
        }
        __syncthreads();   // o_s complete; staged inputs of this chunk consumed

        if constexpr (NORM) {
            // ROWS == D: token tt's outputs are pieces tt*TPT .. +TPT-1, held by
            // TPT consecutive lanes, the same pieces as the token's z
#pragma unroll
            for (int j = 0; j < JKQ; ++j) {
                const int idx = tid + j * NT;
                const int tt = idx / TPT;
                if (idx < TC * TPT && tt < nt) {
                    float4 o4 = o_s[idx];
                    float ss = o4.x * o4.x;
                    ss = fmaf(o4.y, o4.y, ss);
                    ss = fmaf(o4.z, o4.z, ss);
                    ss = fmaf(o4.w, o4.w, ss);
                    ss = group_sum_wide<TPT>(ss);
                    const float rr = sqrtf(ss * (1.0f / D) + a.eps);
                    const float4 z4 = z_s[idx];
                    o4.x = (gn4[j].x * o4.x / rr) * silu(z4.x);
                    o4.y = (gn4[j].y * o4.y / rr) * silu(z4.y);
                    o4.z = (gn4[j].z * o4.z / rr) * silu(z4.z);
                    o4.w = (gn4[j].w * o4.w / rr) * silu(z4.w);
                    const int64_t orow = row_base + t0 + tt;
                    *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + orow * a.out_stride +
                                                (int64_t)h * D + (idx % TPT) * 4) = o4;
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < JV; ++j) {
                const int idx = tid + j * NT;
                const int tt = idx / VPT;
                if (idx < TC * VPT && tt < nt) {
                    const int64_t orow = row_base + t0 + tt;
                    float *dst = static_cast<float *>(a.out) + orow * a.out_stride + (int64_t)h * D +
                                 rb * ROWS + (idx % VPT) * 4;
                    if constexpr (ROWS >= 4) *reinterpret_cast<float4 *>(dst) = o_s[idx];
                    else dst[0] = o_s[idx].x;
                }
            }
        }
        if (has_next) stage();
        __syncthreads();   // next chunk staged; o_s free again
    }

    if (row_active) {
#pragma unroll
        for (int i = 0; i < NCH; ++i)
            *reinterpret_cast<float4 *>(slot + (int64_t)row * D + (i * L + p) * 4) =
                make_float4(s[4 * i + 0], s[4 * i + 1], s[4 * i + 2], s[4 * i + 3]);
    }
}

// LDS bytes a workgroup declares statically (the arrays of seq_kernel)
template <int D, bool NORM>
constexpr int seq_static_lds() {
    using TL = SeqTile<D, NORM>;
    return 16 * (2 * TL::TC * TL::TPT + (NORM ? TL::TC * TL::TPT : 1) + 2 * TL::TC * TL::VPT + TL::TC) + 16;
}

template <int D, bool NORM>
static hipError_t go(const StepArgs &a, hipStream_t stream) {
    using TL = SeqTile<D, NORM>;
    const unsigned grid = (unsigned)((int64_t)a.batch * a.nv * TL::RB);
    // At most three workgroups per CU: with four, the dispatcher fills some
    // CUs with four and leaves others short, and the busiest CU sets the time.
    // Reserving LDS beyond a quarter of the CU's 160 KiB caps residency at three.
    constexpr int kCapBytes = 160 * 1024 / 4 + 1024;
    constexpr int kDyn = seq_static_lds<D, NORM>() < kCapBytes ? kCapBytes - seq_static_lds<D, NORM>() : 0;
    return launch(seq_kernel<D, NORM>, dim3(grid), dim3(TL::NT), kDyn, stream, a);
}

template <bool NORM>
static hipError_t by_dim(const StepArgs &a, int dim, hipStream_t stream) {
    switch (dim) {
        case 4: return go<4, NORM>(a, stream);
        case 8: return go<8, NORM>(a, stream);
        case 16: return go<16, NORM>(a, stream);
        case 32: return go<32, NORM>(a, stream);
        case 64: return go<64, NORM>(a, stream);
        case 128: return go<128, NORM>(a, stream);
        case 256: return go<256, NORM>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_seq(const StepArgs &a, int dim, OutMode mode, hipStream_t stream) {
    // D = 128 (every head shape of the Qwen3.5/3.8 family) runs chunked on the
    // matrix cores, a workgroup per key-head quarter where the shape allows it,
    // else a workgroup per head; the other head dims use the register-resident
    // token loop
    if (dim == 128) return seq_group_fits(a) ? launch_seq_group(a, mode, stream)
                                             : launch_seq_mfma(a, mode, stream);
    if (mode == kOutRawF32) return by_dim<false>(a, dim, stream);
    if (mode == kOutNormF32) return by_dim<true>(a, dim, stream);
    return hipErrorInvalidValue;
}

}  // namespace gdn
