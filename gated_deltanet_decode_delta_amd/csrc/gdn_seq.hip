// gdn_seq.hip -- T-token gated delta rule recurrence with the state on chip.
//
// metrale "layers/ops/ssm_gdn_a.rs", `gdn_prefill_regresident`: the recurrence
// runs token by token inside one launch with the head state held in registers,
// so each state slot is read once at the start and written once at the end,
// whatever the sequence length.
//
// Mapping (gfx950): one workgroup per (sequence b, value head h).  Row i of the
// D x D state is held by LPR = 4 consecutive lanes (a DPP quad), each keeping
// D/4 of its columns in VGPRs (32 at D = 128, 512 threads).  The quad's two
// per-row partial sums (S_i.k and S_i.q) are combined with two DPP adds, so a
// token needs no barrier: every quad derives coef_i and o_i itself and updates
// its own columns.  Columns are interleaved by 16 bytes between the four lanes
// of a quad so that the per-token LDS reads of k and q (the same for every row)
// are 64 contiguous bytes per instruction: broadcast, no bank conflicts.
//
// The per-token inputs are staged through LDS in chunks of TC tokens: at the
// start of a chunk every thread issues its global loads for the NEXT chunk into
// registers (one 16-byte piece of k, q, v and z each), so their latency hides
// behind the current chunk's arithmetic; the chunk's raw outputs collect in
// LDS.  At the chunk end (one barrier) the same threads write the outputs as
// coalesced float4 rows -- applying the gated RMS norm of logicaffeine
// "codegen_cuda/gdn.rs" `gdn_gate_norm` per token when z is given -- then store
// the prefetched inputs into the staging arrays and compute k.q for each staged
// token (second barrier).  Staging and epilogue use one thread <-> one 16-byte
// piece mapping, so a thread overwrites only the z piece it has just consumed.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

template <int D>
struct SeqTile {
    static constexpr int LPR = D >= 16 ? 4 : D / 4;        // lanes per state row
    static constexpr int CS = D / LPR;                     // state columns per lane
    static constexpr int NCH = CS / 4;                     // float4 pieces per lane
    static constexpr int NT = D * LPR < 64 ? 64 : D * LPR; // threads
    static constexpr int TC = D > 128 ? 8 : 16;            // tokens per staged chunk
    static constexpr int TPT = D / 4;                      // float4 pieces per token row
    static constexpr int STAGE = TC * TPT;                 // pieces per array per chunk
    static_assert(STAGE <= NT, "one staging piece per thread");
    static_assert(CS % 4 == 0, "float4 pieces");
};

template <int D, bool NORM>
__global__ void __launch_bounds__((SeqTile<D>::NT)) seq_kernel(StepArgs a) {
    using TL = SeqTile<D>;
    constexpr int LPR = TL::LPR, NCH = TL::NCH, CS = TL::CS, TC = TL::TC, TPT = TL::TPT;
    constexpr int STAGE = TL::STAGE;

    __shared__ float4 k_s[STAGE], q_s[STAGE], v_s[STAGE], o_s[STAGE];
    __shared__ float4 z_s[NORM ? STAGE : 1];
    __shared__ float kq_s[TC], al_s[TC], be_s[TC];

    const int wg = blockIdx.x;
    const int b = wg / a.nv;
    const int h = wg - b * a.nv;
    const int g = h % a.nk;  // tiled key-head pairing
    const int T = a.seq_len;
    const int tid = threadIdx.x;
    const int r = tid / LPR;         // state row of this lane
    const int p = tid % LPR;         // position in the row's quad
    const bool row_active = r < D;
    const int64_t row_base = (int64_t)b * T;   // input/output row of token 0

    // staging/epilogue piece of this thread
    const bool stager = tid < STAGE;
    const int st_tok = tid / TPT;
    const int st_col = (tid % TPT) * 4;

    float *slot = static_cast<float *>(a.state) + (int64_t)b * a.pitch + (int64_t)h * (D * D);

    // state row r, columns (i*LPR + p)*4 .. +3 for i < NCH
    float s[CS];
    if (row_active) {
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const float4 x = *reinterpret_cast<const float4 *>(slot + (int64_t)r * D + (i * LPR + p) * 4);
            s[4 * i + 0] = x.x; s[4 * i + 1] = x.y; s[4 * i + 2] = x.z; s[4 * i + 3] = x.w;
        }
    }
    float4 gn4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (NORM) {
        if (stager) gn4 = *reinterpret_cast<const float4 *>(a.gn + st_col);
    }

    // prefetch registers for one chunk
    float4 pk, pq, pv, pz;
    float pal = 0.f, pbe = 0.f;
    auto prefetch = [&](int t0) {
        const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
        pk = pq = pv = pz = zero;
        const int t = t0 + st_tok;
        if (stager && t < T) {
            const int64_t row = row_base + t;
            pk = *reinterpret_cast<const float4 *>(a.k + row * a.qk_stride + (int64_t)g * D + st_col);
            pq = *reinterpret_cast<const float4 *>(a.q + row * a.qk_stride + (int64_t)g * D + st_col);
            pv = *reinterpret_cast<const float4 *>(a.v + row * a.v_stride + (int64_t)h * D + st_col);
            if constexpr (NORM)
                pz = *reinterpret_cast<const float4 *>(a.z + row * a.z_stride + (int64_t)h * D + st_col);
        }
        if (tid < TC && t0 + tid < T) {
            const int64_t row = row_base + t0 + tid;
            pal = a.alpha[row * a.ab_stride + h];
            pbe = a.beta[row * a.ab_stride + h];
        }
    };
    auto stage = [&]() {
        if (stager) {
            k_s[tid] = pk;
            q_s[tid] = pq;
            v_s[tid] = pv;
            if constexpr (NORM) z_s[tid] = pz;
            float kq = pk.x * pq.x;
            kq = fmaf(pk.y, pq.y, kq);
            kq = fmaf(pk.z, pq.z, kq);
            kq = fmaf(pk.w, pq.w, kq);
            kq = group_sum_wide<TPT>(kq);
            if (tid % TPT == 0) kq_s[st_tok] = kq;
        }
        if (tid < TC) {
            al_s[tid] = pal;
            be_s[tid] = pbe;
        }
    };

    prefetch(0);
    stage();
    __syncthreads();

    for (int t0 = 0; t0 < T; t0 += TC) {
        const bool has_next = t0 + TC < T;
        if (has_next) prefetch(t0 + TC);
        const int nt = T - t0 < TC ? T - t0 : TC;

        if (row_active) {
            for (int tt = 0; tt < nt; ++tt) {
                // keep this token's k pieces in VGPRs for the update when they fit
                // (D <= 128); at D = 256 re-read them from LDS instead of spilling
                constexpr bool kKeepK = NCH <= 8;
                float4 kv[kKeepK ? NCH : 1];
                float pu = 0.f, pw = 0.f;
#pragma unroll
                for (int i = 0; i < NCH; ++i) {
                    const float4 k4 = k_s[tt * TPT + i * LPR + p];
                    if constexpr (kKeepK) kv[i] = k4;
                    const float4 qv = q_s[tt * TPT + i * LPR + p];
                    pu = fmaf(s[4 * i + 0], k4.x, pu);
                    pu = fmaf(s[4 * i + 1], k4.y, pu);
                    pu = fmaf(s[4 * i + 2], k4.z, pu);
                    pu = fmaf(s[4 * i + 3], k4.w, pu);
                    pw = fmaf(s[4 * i + 0], qv.x, pw);
                    pw = fmaf(s[4 * i + 1], qv.y, pw);
                    pw = fmaf(s[4 * i + 2], qv.z, pw);
                    pw = fmaf(s[4 * i + 3], qv.w, pw);
                    // at D = 256 keep the scheduler from hoisting every LDS read
                    // ahead of the FMAs (that would need more than 128 VGPRs)
                    if constexpr (!kKeepK) {
                        if (i % 4 == 3) __builtin_amdgcn_sched_barrier(0);
                    }
                }
                const float u = group_sum<LPR>(pu);
                const float w = group_sum<LPR>(pw);
                const float al = al_s[tt], be = be_s[tt], kq = kq_s[tt];
                const float vr = reinterpret_cast<const float *>(v_s)[tt * D + r];
                const float coef = be * (vr - al * u);
                const float o = (al * w + coef * kq) * a.scale;
#pragma unroll
                for (int i = 0; i < NCH; ++i) {
                    float4 k4;
                    if constexpr (kKeepK) k4 = kv[i];
                    else k4 = k_s[tt * TPT + i * LPR + p];
                    s[4 * i + 0] = al * s[4 * i + 0] + coef * k4.x;
                    s[4 * i + 1] = al * s[4 * i + 1] + coef * k4.y;
                    s[4 * i + 2] = al * s[4 * i + 2] + coef * k4.z;
                    s[4 * i + 3] = al * s[4 * i + 3] + coef * k4.w;
                }
                if (p == 0) reinterpret_cast<float *>(o_s)[tt * D + r] = o;
            }
        }
        __syncthreads();   // o_s complete; staged inputs of this chunk consumed

        if (stager && st_tok < nt) {
            const int64_t row = row_base + t0 + st_tok;
            float4 o4 = o_s[tid];
            if constexpr (NORM) {
                float ss = o4.x * o4.x;
                ss = fmaf(o4.y, o4.y, ss);
                ss = fmaf(o4.z, o4.z, ss);
                ss = fmaf(o4.w, o4.w, ss);
                ss = group_sum_wide<TPT>(ss);
                const float rr = sqrtf(ss * (1.0f / D) + a.eps);
                const float4 z4 = z_s[tid];
                o4.x = (gn4.x * o4.x / rr) * silu(z4.x);
                o4.y = (gn4.y * o4.y / rr) * silu(z4.y);
                o4.z = (gn4.z * o4.z / rr) * silu(z4.z);
                o4.w = (gn4.w * o4.w / rr) * silu(z4.w);
            }
            *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + row * a.out_stride +
                                        (int64_t)h * D + st_col) = o4;
        }
        if (has_next) stage();
        __syncthreads();   // next chunk staged; o_s free again
    }

    if (row_active) {
#pragma unroll
        for (int i = 0; i < NCH; ++i)
            *reinterpret_cast<float4 *>(slot + (int64_t)r * D + (i * LPR + p) * 4) =
                make_float4(s[4 * i + 0], s[4 * i + 1], s[4 * i + 2], s[4 * i + 3]);
    }
}

template <int D, bool NORM>
static hipError_t go(const StepArgs &a, hipStream_t stream) {
    const unsigned grid = (unsigned)((int64_t)a.batch * a.nv);
    hipLaunchKernelGGL((seq_kernel<D, NORM>), dim3(grid), dim3(SeqTile<D>::NT), 0, stream, a);
    return hipGetLastError();
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
    if (mode == kOutRawF32) return by_dim<false>(a, dim, stream);
    if (mode == kOutNormF32) return by_dim<true>(a, dim, stream);
    return hipErrorInvalidValue;
}

}  // namespace gdn
