// gdn_seq_mfma.hip -- the T-token recurrence at D = 128 on the fp32 matrix cores.
//
// Same operation as the register-resident token loop of gdn_seq.hip (metrale
// "layers/ops/ssm_gdn_a.rs", `gdn_prefill_regresident`; the update of
// logicaffeine "codegen_cuda/gdn.rs", `gdn_step`), evaluated C = 16 tokens at a
// time so that the state contractions become 16x16x4 fp32 MFMA products.
// Within a chunk, with M[t][s] = alpha_{s+1} ... alpha_t (M[t][t] = 1),
// P_t = alpha_0 ... alpha_t and S0 the state at the chunk start, unrolling
// S_t = alpha_t S_{t-1} + c_t k_t^T gives
//     c_t + sum_{s<t} beta_t M[t][s] (k_s.k_t) c_s = beta_t (v_t - P_t S0 k_t)
//     o_t = P_t S0 q_t + sum_{s<=t} M[t][s] (k_s.q_t) c_s
//     S_end = P_15 S0 + sum_s M[15][s] c_s k_s^T
// so per chunk: U = S0 K^T and W = S0 Q^T (MFMA), the 16x16 unit lower
// triangular system (I + A) (its inverse T by forward substitution on the
// vector ALU), C = R T^T with R = beta (V - P U) (MFMA), O = P W + C G^T (MFMA)
// and S <- P_15 S + (C diag(M[15][.])) K (MFMA).  The range products M are
// formed directly (no division by a running product), so any alpha >= 0 works,
// including alpha = 0.  Rounding differs from the token loop by reordering
// only; both are checked against the same fp64 oracle.
//
// Mapping.  One workgroup of eight waves per (sequence, value head), two per
// SIMD; wave w owns state rows [16w, 16w+16).  (On gfx950 one SIMD does not
// run matrix-core and vector-ALU instructions at the same time, even from
// different waves, so the second wave hides latency rather than adding
// throughput.)  The state lives in the MFMA accumulator layout transposed:
// register r of tile m of lane l holds S[16w + l%16][16m + 4(l/16) + r].  That
// is exactly the B-operand layout of the product K S^T with the contraction
// index j ordered (m, r, l/16), so the state never moves between the U/W
// products and the update.  k and q of a chunk are staged in LDS (read once per
// 16-row tile instead of once per lane).  The chunk-level quantities run ahead
// of the state work: during chunk c, chunk c+2 is staged and its k.k / k.q tiles
// and range products formed, and the triangular inverse of chunk c+1 is
// solved, so the first half of every chunk is the U / W products alone, equal
// on every SIMD; two workgroup barriers per chunk.  v goes from global memory
// straight to the lanes that use it.  The kernel writes the raw o; with z the
// gated norm follows as a second pass over the output rows.
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kC = 16;           // tokens per chunk
constexpr int kWaves = 8;        // wave w owns state rows [16w, 16w + 16)
constexpr int kThreads = 64 * kWaves;
constexpr int kKS = kD + 4;      // row stride (floats) of k_s / q_s
constexpr int kTS = kC + 4;      // row stride of the 16x16 matrices in LDS
constexpr int kPieces = kC * kD / 4 / kThreads;   // 16-byte pieces of a chunk's k (or q) per thread
constexpr int kPartWaves = 3;    // waves 1..3 form the chunk's k.k / k.q (16-column slices 3,3,2)
constexpr int kSolveWave = 0;    // forms A and solves for T, while waves 1..3 form the k.k / k.q
constexpr int kBufs = 3;         // chunks c, c+1 and c+2 are staged during chunk c
static_assert(kPieces * kThreads * 4 == kC * kD, "staging covers the chunk exactly");

__device__ __forceinline__ f32x4 mfma(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// The value of the lane N places higher in the same 16-lane DPP row (row_shl),
// or 1 past the end of the row.
template <int N>
__device__ __forceinline__ float dpp_from_above(float x) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8, "row shift");
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(x), 0x100 + N,
                                                      0xF, 0xF, false));
}

}  // namespace

__global__ void __launch_bounds__(kThreads) seq_mfma_kernel(StepArgs a) {
    // Chunk data: buffer c % 3 holds chunk c's k, q, alpha, beta, P and D
    // (chunks c, c+1, c+2 are live during chunk c); the k.k / k.q partials, M,
    // M^T and T of chunk c sit in buffer c & 1 (written one or two chunks
    // ahead, read during chunk c - 1 or c).
    __shared__ __align__(16) float k_s[kBufs][kC * kKS], q_s[kBufs][kC * kKS];
    __shared__ f32x4 part_s[2][kPartWaves][2][64];       // partial k.k and k.q tiles
    __shared__ __align__(16) float a_s[kC * kTS], t_s[2][kC * kTS];  // A and T = (I + A)^{-1}
    __shared__ __align__(16) float m_s[2][kC * kTS], mt_s[2][kC * kTS]; // M[t][s] and its transpose
    __shared__ __align__(16) float al_s[kBufs][kC], be_s[kBufs][kC], p_s[kBufs][kC], d_s[kBufs][kC];

    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, g = l >> 4, li = l & 15;
    const int head = blockIdx.x;
    const int b = head / a.nv;
    const int h = head - b * a.nv;
    const int kh = h % a.nk;  // tiled key-head pairing
    const int T = a.seq_len;
    const int64_t row_base = (int64_t)b * T;
    float *slot = static_cast<float *>(a.state) + (int64_t)b * a.pitch + (int64_t)h * (kD * kD);
    const int64_t vcol = (int64_t)h * kD + 16 * w + li;   // this lane's v / z / output column

    // Stored state: the true state is gam * S, with S[m][r] holding
    // S[row 16w + li][col 16m + 4g + r].  Keeping the chunk decays in the scalar
    // gam leaves S to the matrix cores alone.
    const int row = 16 * w + li;
    f32x4 S[8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
        S[m] = *reinterpret_cast<const f32x4 *>(slot + (int64_t)row * kD + 16 * m + 4 * g);
    float gam = 1.0f;

    // prefetch registers for one chunk: 16-byte pieces f = tid + 256u of the
    // chunk's k and q ([16][128]); v (and z) of the lane's own (t, i) entries
    float4 pk[kPieces], pq[kPieces];
    float pv[4];
    float pal = 1.0f, pbe = 0.0f;
    // element offsets of this lane's prefetch rows at t0 = 0: k/q piece u is
    // token f >> 5, columns (f & 31) * 4 .. +3 (f = tid + 512u); v is the lane's
    // column of tokens 4g .. 4g + 3
    int64_t kq_off[kPieces];
#pragma unroll
    for (int u = 0; u < kPieces; ++u) {
        const int f = tid + kThreads * u;
        kq_off[u] = (row_base + (f >> 5)) * a.qk_stride + (int64_t)kh * kD + (f & 31) * 4;
    }
    const int64_t v_off = (row_base + 4 * g) * a.v_stride + vcol;
    auto prefetch = [&](int t0) {
        if (t0 + kC <= T) {   // a whole chunk: uniform row offsets, nothing to clamp
            const int64_t dqk = (int64_t)t0 * a.qk_stride;
#pragma unroll
            for (int u = 0; u < kPieces; ++u) {
                pk[u] = *reinterpret_cast<const float4 *>(a.k + kq_off[u] + dqk);
                pq[u] = *reinterpret_cast<const float4 *>(a.q + kq_off[u] + dqk);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pv[r] = a.v[v_off + (int64_t)(t0 + r) * a.v_stride];
            }
            {   // every lane loads (token tid % 16): no divergent branch among the loads
                const int64_t rr = row_base + t0 + (tid & (kC - 1));
                pal = a.alpha[rr * a.ab_stride + h];
                pbe = a.beta[rr * a.ab_stride + h];
            }
            return;
        }
        // Padding tokens (past T): alpha 1, beta 0 and zero k/q/v leave the
        // state and every real token unchanged.  Their loads read row T-1
        // (always valid) and are zeroed by a select, so no load is predicated.
        const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < kPieces; ++u) {
            const int f = tid + kThreads * u;     // < kC * kD / 4
            const int t = f >> 5, col = (f & 31) * 4;
            const bool ok = t0 + t < T;
            const int64_t rr = row_base + (ok ? t0 + t : T - 1);
            const int64_t off = rr * a.qk_stride + (int64_t)kh * kD + col;
            const float4 kx = *reinterpret_cast<const float4 *>(a.k + off);
            const float4 qx = *reinterpret_cast<const float4 *>(a.q + off);
            pk[u] = ok ? kx : zero;
            pq[u] = ok ? qx : zero;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 4 * g + r;
            const bool ok = t0 + t < T;
            const int64_t rr = row_base + (ok ? t0 + t : T - 1);
            const float vx = a.v[rr * a.v_stride + vcol];
            pv[r] = ok ? vx : 0.f;
        }
        pal = 1.0f;
        pbe = 0.0f;
        if (tid < kC && t0 + tid < T) {
            const int64_t rr = row_base + t0 + tid;
            pal = a.alpha[rr * a.ab_stride + h];
            pbe = a.beta[rr * a.ab_stride + h];
        }
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int u = 0; u < kPieces; ++u) {
            const int f = tid + kThreads * u;
            const int t = f >> 5, col = (f & 31) * 4;
            *reinterpret_cast<float4 *>(&k_s[buf][t * kKS + col]) = pk[u];
            *reinterpret_cast<float4 *>(&q_s[buf][t * kKS + col]) = pq[u];
        }
        if (tid < kC) {
            al_s[buf][tid] = pal;
            be_s[buf][tid] = pbe;
        }
    };

    // Waves 4..7, one thread per (t, s) with s the lane's place in its 16-lane
    // DPP row: the range products M[t][s] = alpha_{s+1} ... alpha_t of the
    // staged chunk (0 above the diagonal), its transpose, the last row D[s] =
    // M[15][s] and the prefix products P_t = alpha_0 M[t][0].  With x_s =
    // alpha_{s+1} for s < t (else 1), M[t][s] is the suffix product x_s ...
    // x_15 along the row: four DPP row shifts.  No division, so any alpha >= 0
    // (zero included) is exact to fp32 rounding.
    float unit[kC];   // column li of the identity (the solve's right-hand side)
#pragma unroll
    for (int t = 0; t < kC; ++t) unit[t] = t == li ? 1.0f : 0.0f;

    auto range_products = [&](int b3, int par) {
        if (w >= kWaves - 4) {
            const int e = tid - (kWaves - 4) * 64;   // 0 .. 255
            const int t = e >> 4, s = e & 15;
            float m = al_s[b3][s < t ? s + 1 : 0];   // index kept inside the row
        m = s < t ? m : 1.0f;
            m *= dpp_from_above<1>(m);
            m *= dpp_from_above<2>(m);
            m *= dpp_from_above<4>(m);
            m *= dpp_from_above<8>(m);
            const float v = t >= s ? m : 0.0f;
            m_s[par][t * kTS + s] = v;
            mt_s[par][s * kTS + t] = v;
            if (t == kC - 1) d_s[b3][s] = v;
            if (s == 0) p_s[b3][t] = al_s[b3][0] * v;
        }
    };

    // waves 1..3 (SIMDs 1..3) form a part each of the chunk's k.k and k.q
    // products (16-column slices 3p .. 3p + 2 of the 8); the parts are summed
    // when read.  Waves 4..7 form the range products meanwhile.
    auto tiles = [&](int b3, int par) {
        if (w >= 1 && w <= kPartWaves) {
            const int pw = w - 1;
            f32x4 KK = f32x4{0.f, 0.f, 0.f, 0.f}, KQ = KK;
#pragma unroll
            for (int mm = 0; mm < 3; ++mm) {
                const int m = 3 * pw + mm;
                if (m < kD / 16) {
                    const f32x4 ka = *reinterpret_cast<const f32x4 *>(&k_s[b3][li * kKS + 16 * m + 4 * g]);
                    const f32x4 qa = *reinterpret_cast<const f32x4 *>(&q_s[b3][li * kKS + 16 * m + 4 * g]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        KK = mfma(ka[r], ka[r], KK);   // k_t . k_s
                        KQ = mfma(ka[r], qa[r], KQ);   // k_t . q_s
                    }
                }
            }
            part_s[par][pw][0][l] = KK;
            part_s[par][pw][1][l] = KQ;
        }
    };
    auto partials = [&](int b3, int par) {
        range_products(b3, par);
        tiles(b3, par);
    };

    // Wave 0: A[a][b] = beta_a M[a][b] (k_a.k_b) for b < a, then T = (I + A)^{-1}
    // column by column (lane column li, forward substitution with the identity
    // column as right-hand side: the entries above li come out exactly 0 and
    // x[li] exactly 1).  Lane (g, li) owns A[4g + r][li]; k.k is symmetric, so
    // no value moves between lanes before the LDS round trip.  A is stored
    // transposed (a_s row s = column s of A), and the substitution is column
    // oriented: once x[s] is final it is taken out of every later x[t], so the
    // dependent chain is one FMA per step.
    auto solve = [&](int b3, int par) {
        if (w == kSolveWave) {
            const f32x4 bet = *reinterpret_cast<const f32x4 *>(&be_s[b3][4 * g]);
            const f32x4 mA = *reinterpret_cast<const f32x4 *>(&mt_s[par][li * kTS + 4 * g]);  // M[4g+r][li]
            f32x4 acol;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int ai = 4 * g + r;
                float kk = 0.f;
#pragma unroll
                for (int v2 = 0; v2 < kPartWaves; ++v2) kk += part_s[par][v2][0][l][r];
                acol[r] = li < ai ? bet[r] * mA[r] * kk : 0.0f;
            }
            *reinterpret_cast<f32x4 *>(&a_s[li * kTS + 4 * g]) = acol;   // A[4g+r][li]
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
            float x[kC];
#pragma unroll
            for (int t = 0; t < kC; ++t) x[t] = unit[t];
#pragma unroll
            for (int s2 = 0; s2 < kC - 1; ++s2) {
#pragma unroll
                for (int t4 = (s2 + 1) / 4; t4 < kC / 4; ++t4) {
                    const f32x4 av = *reinterpret_cast<const f32x4 *>(&a_s[s2 * kTS + 4 * t4]);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * t4 + e > s2) x[4 * t4 + e] = fmaf(-av[e], x[s2], x[4 * t4 + e]);
                }
            }
            if (g == 0) {
#pragma unroll
                for (int t = 0; t < kC; ++t) t_s[par][t * kTS + li] = x[t];
            }
        }
    };

    float vcur[4], vn1[4], vn2[4];
    auto take = [&](float *vd) {
#pragma unroll
        for (int r = 0; r < 4; ++r) vd[r] = pv[r];
    };
    // Prologue: chunk 0 staged and prepared, chunk 1 staged and prepared, T of
    // chunk 0 solved, chunk 2's loads in flight.
    prefetch(0);
    stage(0);
    take(vcur);
    // drain every load (the state included) so that no conservative vmcnt wait
    // lands inside the chunk loop, where it would also wait for the prefetch
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kC < T) prefetch(kC);
    partials(0, 0);
    if (kC < T) {
        stage(1);
        take(vn1);
    }
    __syncthreads();
    if (2 * kC < T) prefetch(2 * kC);
    solve(0, 0);
    if (kC < T) partials(1, 1);
    __syncthreads();

    // Per chunk c (chunk buffer b3 = c % 3, pair buffer par = c & 1), two barriers:
    //   U, W on the matrix cores (every wave alike); chunk c+2 staged
    //   -- barrier: chunk c+2 visible --
    //   chunk c+2's range products (waves 4..7, first, so that the two waves of
    //   a SIMD are not both in the dependent C' -> O chain at once); C', O,
    //   outputs, state update; prefetch of chunk c+3; chunk c+2's k.k, k.q
    //   partials (waves 1..3); A and T of chunk c+1 (wave 0)
    //   -- barrier: chunk c+2 prepared, T(c+1) visible, every read of chunk c done --
    float *outp = static_cast<float *>(a.out);
    for (int t0 = 0, b3 = 0, par = 0; t0 < T; t0 += kC, b3 = b3 == kBufs - 1 ? 0 : b3 + 1, par ^= 1) {
        const int b3n1 = b3 == kBufs - 1 ? 0 : b3 + 1;     // buffer of chunk c+1
        const int b3n2 = b3n1 == kBufs - 1 ? 0 : b3n1 + 1; // buffer of chunk c+2
        const int nt = T - t0 < kC ? T - t0 : kC;
        // G[b][a] = M[b][a] (q_b.k_a) for a <= b, lane (g, li) holding a = 4g + r,
        // b = li (the MFMA A-operand layout of O += G C'); k_a.q_b is the tile
        // entry of the k.q product, so no value moves between lanes.
        const f32x4 mG = *reinterpret_cast<const f32x4 *>(&m_s[par][li * kTS + 4 * g]);    // M[li][4g+r]
        f32x4 Ga;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float kq = 0.f;
#pragma unroll
            for (int v2 = 0; v2 < kPartWaves; ++v2) kq += part_s[par][v2][1][l][r];
            Ga[r] = mG[r] * kq;   // M[li][a] is 0 above the diagonal
        }

        // U^T = K S^T and W^T = Q S^T on the matrix cores (four independent
        // accumulation chains keep back-to-back MFMAs free of dependencies)
        f32x4 Ua = f32x4{0.f, 0.f, 0.f, 0.f}, Ub = Ua, Wa = Ua, Wb = Ua;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const f32x4 ka = *reinterpret_cast<const f32x4 *>(&k_s[b3][li * kKS + 16 * m + 4 * g]);
            const f32x4 qa = *reinterpret_cast<const f32x4 *>(&q_s[b3][li * kKS + 16 * m + 4 * g]);
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
                Ua = mfma(ka[r], S[m][r], Ua);
                Wa = mfma(qa[r], S[m][r], Wa);
                Ub = mfma(ka[r + 1], S[m][r + 1], Ub);
                Wb = mfma(qa[r + 1], S[m][r + 1], Wb);
            }
        }
        const f32x4 U = Ua + Ub, W = Wa + Wb;
        if (t0 + 2 * kC < T) {
            stage(b3n2);
            take(vn2);
        }
        __syncthreads();   // chunk c+2 staged
        if (t0 + 2 * kC < T) range_products(b3n2, par);   // waves 4..7, ahead of their state work

        const f32x4 bet = *reinterpret_cast<const f32x4 *>(&be_s[b3][4 * g]);
        const f32x4 Ta = *reinterpret_cast<const f32x4 *>(&t_s[par][li * kTS + 4 * g]);
        const f32x4 Pt = *reinterpret_cast<const f32x4 *>(&p_s[b3][4 * g]);
        const f32x4 Dt = *reinterpret_cast<const f32x4 *>(&d_s[b3][4 * g]);
        const float Plast = p_s[b3][kC - 1];

        // R = beta (v - P gam U);  C' = T R;  O = P gam W + G C'
        f32x4 R, Cp, O;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float pg = Pt[r] * gam;
            R[r] = bet[r] * (vcur[r] - pg * U[r]);
            O[r] = pg * W[r];
        }
        {
            f32x4 c0 = f32x4{0.f, 0.f, 0.f, 0.f}, c1 = c0;
            c0 = mfma(Ta[0], R[0], c0);
            c1 = mfma(Ta[1], R[1], c1);
            c0 = mfma(Ta[2], R[2], c0);
            c1 = mfma(Ta[3], R[3], c1);
            Cp = c0 + c1;
            f32x4 o1 = f32x4{0.f, 0.f, 0.f, 0.f};
            O = mfma(Ga[0], Cp[0], O);
            o1 = mfma(Ga[1], Cp[1], o1);
            O = mfma(Ga[2], Cp[2], O);
            o1 = mfma(Ga[3], Cp[3], o1);
            O += o1;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 4 * g + r;
            // a whole chunk stores without per-token branches
            if (nt == kC || t < nt) outp[(row_base + t0 + t) * a.out_stride + vcol] = O[r] * a.scale;
        }

        // true state: gam S -> P_15 gam S + K^T (C' diag(M[15][.]))^T.  Keep the
        // decay in gam (S += K^T (C' M[15][.] / gam')^T) while gam' stays in
        // [2^-60, 2^60]; otherwise fold it into S first (strong forgetting).
        float gnew = gam * Plast;
        float cscale;
        if (gnew >= 0x1p-60f && gnew <= 0x1p60f) {
            cscale = 1.0f / gnew;
        } else {
            const float f = gnew;
#pragma unroll
            for (int m = 0; m < 8; ++m) S[m] *= f;
            gnew = 1.0f;
            cscale = 1.0f;
        }
        gam = gnew;
#pragma unroll
        for (int r = 0; r < 4; ++r) Cp[r] *= Dt[r] * cscale;
        // k of token 4g + s4, column 16m + li: the A operand of the update
        const float *kc = &k_s[b3][4 * g * kKS + li];
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
            for (int m = 0; m < 8; ++m) S[m] = mfma(kc[s4 * kKS + 16 * m], Cp[s4], S[m]);

        // chunk c+3's loads go out after this chunk's output stores: the wait for
        // them (at the next staging) then never waits on a store issued later
        if (t0 + 3 * kC < T) prefetch(t0 + 3 * kC);
        if (t0 + 2 * kC < T) tiles(b3n2, par);   // chunk c+2 uses pair buffer par too
        if (t0 + kC < T) solve(b3n1, par ^ 1);
        __syncthreads();   // chunk c+2 prepared; T(c+1) visible; every read of chunk c done
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            vcur[r] = vn1[r];
            vn1[r] = vn2[r];
        }
    }

#pragma unroll
    for (int m = 0; m < 8; ++m)
        *reinterpret_cast<f32x4 *>(slot + (int64_t)row * kD + 16 * m + 4 * g) = S[m] * gam;
}

hipError_t launch_seq_mfma(const StepArgs &a, OutMode mode, hipStream_t stream) {
    const unsigned grid = (unsigned)((int64_t)a.batch * a.nv);
    if (mode != kOutRawF32 && mode != kOutNormF32) return hipErrorInvalidValue;
    // with z the output rows get the gated norm in a second pass: fusing it here
    // (a workgroup-wide sum per token) took 1.56 ms against 1.42 ms for the pair
    const hipError_t e = launch(seq_mfma_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
    if (e != hipSuccess || mode == kOutRawF32) return e;
    return launch_norm_rows(a, stream);
}

}  // namespace gdn
