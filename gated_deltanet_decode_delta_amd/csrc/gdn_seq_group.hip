// gdn_seq_group.hip -- the T-token recurrence at D = 128 without a workspace:
// every workgroup forms the chunk quantities it needs itself, for all value
// heads of one key head, and holds one quarter (or, on small grids, one
// eighth) of their state rows.
//
// Same chunked algebra as gdn_seq_mfma.hip and gdn_seq_split.hip (16 tokens per
// chunk; metrale "layers/ops/ssm_gdn_a.rs" `gdn_prefill_regresident` for the
// operation, the update of logicaffeine "codegen_cuda/gdn.rs" `gdn_step`): with
// M[t][s] = alpha_{s+1} ... alpha_t, P_t = alpha_0 ... alpha_t and S0 the state
// at the chunk start,
//     C' = T R,  R = beta (V - P S0 K^T),  T = (I + A)^{-1},
//          A[t][s] = beta_t M[t][s] (k_s.k_t)  (s < t)
//     O  = P S0 Q^T + C' G^T,  G[t][s] = M[t][s] (k_s.q_t)  (s <= t)
//     S_end = P_15 S0 + C' diag(M[15][.]) K.
//
// Mapping.  With the tiled pairing the value heads of key head g are g, g + NK,
// ..., g + (R - 1) NK (R = NV / NK, at most 3), and they all read the same k
// and q.  One workgroup takes (sequence, key head, quarter): rows 32 quarter ..
// +31 of each of those R heads, four waves per head laid out as in the
// workspace path's state pass (wave (strip, half) owns 16 rows x 64 key
// columns, four 16x16 accumulator tiles), 4 R waves in all.  The chunk's k
// and q are staged once for the R heads, and its k.k / k.q tiles are formed
// once for them, so forming T and G in the workgroup costs 64 extra
// matrix-core products per chunk per workgroup (on 12 R-independent product
// streams of 52) and one triangular solve for the R heads side by side (lane
// group g solves head g).  At the real shape (B = 4, NK = 16, R = 3) that is
// 256 workgroups of 12 waves, one per CU, three waves per SIMD, against 192
// workgroups of eight waves for the kernel that gives each head one workgroup.
// Grids of at most 32 key-head groups (B = 1, 2 at NK = 16) would leave CUs
// idle; at R = 3 they run in eighths: rows 16 eighth .. +15, one strip, two
// waves per head, twice the workgroups.
//
// One workgroup barrier per chunk.  The two halves of a strip exchange their
// partial products over their 64 columns (half 0 hands over its U and W parts,
// half 1 its U part) and then both form C' = T R, so nothing else has to pass
// between them within the chunk; the exchange buffers alternate by chunk parity
// and alpha, beta, P and D are kept four chunks deep, so a wave that runs ahead
// into the next chunk never overwrites what a slower one still reads.  The
// chunk-level work runs ahead of the state work.  During chunk c:
//   before the barrier: U / W products (every wave); chunk c + 2 staged
//     (k, q, alpha, beta); then A, T and G of chunk c (wave 0, after its own
//     products);
//   after it: the strip chains (R, C'; O and its stores in half 1); the loads
//     of chunk c + 3's k, q, alpha, beta and chunk c + 1's v; the state
//     update; chunk c + 2's k.k / k.q partial tiles (waves 1..3) and range
//     products M, P, D (one wave per SIMD).
#include "gdn_chunk.h"
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

using namespace chunk;

namespace {

constexpr int kBufs = 3;        // k and q in LDS: chunks c, c + 1, c + 2
// per-head stride of the 16 x 16 chunk matrices in LDS: four words past a
// multiple of the bank window, so lane groups that address different heads in
// one instruction (the solve's stores of T) fall into different banks
constexpr int kHS = kC * kTS + 4;

}  // namespace

// SL is the number of row slices a head's 128 rows are split into: 4
// (quarters, two strips of 16 rows per head, four waves) or, at R = 3 only, 8
// (eighths, one strip, two waves per head) for grids too small to fill the chip.
template <int R, int SL>
__global__ void __launch_bounds__(64 * R * (SL == 4 ? 4 : 2)) seq_group_kernel(StepArgs a, int nc) {
    static_assert(SL == 4 || (SL == 8 && R == 3), "eighths only at three value heads per key head");
    constexpr int NSTRIP = SL == 4 ? 2 : 1;    // strips of 16 rows per head in a workgroup
    constexpr int WPH = 2 * NSTRIP;            // waves per head
    constexpr int NT = 64 * R * WPH;
    constexpr int KQP = (512 + NT - 1) / NT;   // 16-byte pieces of a chunk's k (and of q) per thread
    constexpr int kParts = SL == 4 ? 3 : 2;     // partial k.k / k.q tiles
    __shared__ __align__(16) float kq_s[kBufs][2][kC * kKS];   // [chunk % 3][k, q] rows of a chunk
    __shared__ __align__(16) float ab_s[4][2][R][kC];          // [chunk % 4][alpha, beta][head]
    __shared__ __align__(16) float pd_s[4][2][R][kC];          // [chunk % 4][P, D][head]
    __shared__ f32x4 part_s[2][kParts][2][64];                 // [chunk & 1][part][k.k, k.q]
    __shared__ __align__(16) float m_s[2][R][kHS];             // [chunk & 1] M[t][s]
    __shared__ __align__(16) float t_s[2][R][kHS];             // [chunk & 1] T row-major
    __shared__ __align__(16) float g_s[2][R][kHS];             // [chunk & 1] G / sqrt(D) row-major
    __shared__ __align__(16) float a_s[R][kHS];                // a_s[s][t] = A[t][s] of the chunk solved
    // [chunk & 1][strip][U from half 0, W from half 0, U from half 1]: the
    // partial products over each half's 64 columns that the strip exchanges
    __shared__ f32x4 x_s[2][NSTRIP * R][3][64];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, g = l >> 4, li = l & 15;
    const int m = w / WPH;                   // value head m of the key head
    const int half = w & 1, strip = (w >> 1) % NSTRIP;

    // Block -> (sequence, key head, slice): the SL slices of a key head get
    // indices equal modulo 8, so they run on one XCD and share its L2 for the
    // key head's k and q rows.
    const int ngroups = a.batch * a.nk;
    const int full = ngroups / 8 * 8;
    int grp, slice;
    {
        const int bid = blockIdx.x;
        if (bid < full * SL) {
            const int r = bid % (8 * SL);
            grp = bid / (8 * SL) * 8 + (r & 7);
            slice = r >> 3;
        } else {
            const int r = bid - full * SL, rem = ngroups - full;
            grp = full + r % rem;
            slice = r / rem;
        }
    }
    const int b = grp / a.nk;
    const int kh = grp - b * a.nk;
    const int h = kh + m * a.nk;             // tiled pairing
    const int T = a.seq_len;
    const int64_t row_base = (int64_t)b * T;
    const int row = (kD / SL) * slice + 16 * strip + li;     // state row (value index) of head h
    float *srow = static_cast<float *>(a.state) + (int64_t)b * a.pitch + (int64_t)h * (kD * kD) +
                  (int64_t)row * kD + 64 * half + 4 * g;

    // The true state is gam * S; S[t4][r] = S[row][64 half + 16 t4 + 4 g + r].
    f32x4 S[4];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) S[t4] = *reinterpret_cast<const f32x4 *>(srow + 16 * t4);
    float gam = 1.0f;

    // k and q of a chunk: pieces f = tid + NT u - kqb in [0, 512), token f >> 5,
    // columns (f % 32) * 4, through descriptors based at the chunk's first row
    // (rows past T read 0); alpha and beta of head e >> 4, token e % 16 for
    // e = tid - (NT - 16 R) >= 0 (alpha 1, beta 0 past T: such tokens change
    // nothing).  The highest threads do it, so that wave 0 goes from its
    // products to the solve with no staging in between.
    constexpr int kqb = KQP * NT - 512;
    const int abe = tid - (NT - 16 * R);
    const int64_t kq0 = row_base * a.qk_stride + (int64_t)kh * kD;
    int kq_off[KQP];
#pragma unroll
    for (int u = 0; u < KQP; ++u) {
        const int f = tid + NT * u - kqb;
        kq_off[u] = (int)((((f & 511) >> 5) * a.qk_stride + (f & 31) * 4) * 4);
    }
    f32x4 pk[KQP], pq[KQP];
    float pal = 1.0f, pbe = 0.0f;
    const bool ab_thread = abe >= 0;
    const int64_t ab_col = kh + (int64_t)(abe >> 4) * a.nk;
    auto prefetch = [&](int c) {
        const int t0 = c * kC;
        const int64_t off = kq0 + (int64_t)t0 * a.qk_stride;   // uniform
        const int64_t nb = (int64_t)(T - t0) * a.qk_stride * 4;
        const __amdgpu_buffer_rsrc_t rk = buf_rsrc(a.k + off, nb), rq = buf_rsrc(a.q + off, nb);
#pragma unroll
        for (int u = 0; u < KQP; ++u) {
            if (tid + NT * u >= kqb) {
                pk[u] = buf_load4(rk, kq_off[u]);
                pq[u] = buf_load4(rq, kq_off[u]);
            }
        }
        pal = 1.0f;
        pbe = 0.0f;
        if (ab_thread && t0 + (abe & 15) < T) {
            const int64_t rr = (row_base + t0 + (abe & 15)) * a.ab_stride + ab_col;
            pal = a.alpha[rr];
            pbe = a.beta[rr];
        }
    };
    auto stage = [&](int c) {
        const int b3 = c % kBufs;
#pragma unroll
        for (int u = 0; u < KQP; ++u) {
            const int f = tid + NT * u - kqb;
            if (f >= 0) {
                *reinterpret_cast<f32x4 *>(&kq_s[b3][0][(f >> 5) * kKS + (f & 31) * 4]) = pk[u];
                *reinterpret_cast<f32x4 *>(&kq_s[b3][1][(f >> 5) * kKS + (f & 31) * 4]) = pq[u];
            }
        }
        if (ab_thread) {
            ab_s[c & 3][0][abe >> 4][abe & 15] = pal;
            ab_s[c & 3][1][abe >> 4][abe & 15] = pbe;
        }
    };

    // The chunk-level work is spread so that each SIMD ends up with about the
    // same matrix-core and vector-ALU time: the half-1 waves (SIMDs 1, 3) carry
    // four more products each than the half-0 waves (SIMDs 0, 2), and wave 0
    // (SIMD 0) the solve.  The waves doing it raise their priority meanwhile:
    // the chunk's barrier waits for the last of them (0.968 -> 0.962 ms).
    //
    // Range products, by the four waves of one head slot (waves 4..7, or 0..3
    // when R = 1, one per SIMD): wave rw takes rows t = 4 rw + g of every head,
    // lane li the column s.  With x_s = alpha_{s+1} for s < t (else 1), M[t][s]
    // is the suffix product x_s ... x_15 along the 16-lane row (no division, so
    // any alpha >= 0 is exact to fp32 rounding).  Also P_t = alpha_0 M[t][0]
    // and D[s] = M[15][s].  Lane s reads alpha_s (one LDS round trip for all
    // heads) and takes alpha_{s+1} from the lane above.  In eighths, waves 1
    // and 5 (both on SIMD 1) take rows 0..7 and 8..15, two passes each.
    constexpr int kRangeW0 = R > 1 ? 4 : 0;
    constexpr int kRangePasses = SL == 4 ? 1 : 2;
    auto range_products = [&](int c) {
        const bool mine = SL == 4 ? (w >= kRangeW0 && w < kRangeW0 + 4) : (w == 1 || w == 5);
        if (mine) {
            __builtin_amdgcn_s_setprio(2);
            const int b4 = c & 3, par = c & 1;
            const int q0 = SL == 4 ? w - kRangeW0 : (w == 1 ? 0 : 2);   // first row quad
            const int s = li;
            float al[R];
#pragma unroll
            for (int hm = 0; hm < R; ++hm) al[hm] = ab_s[b4][0][hm][s];
#pragma unroll
            for (int pass = 0; pass < kRangePasses; ++pass)
#pragma unroll
            for (int hm = 0; hm < R; ++hm) {
                const int t = 4 * (q0 + pass) + g;
                const float up = dpp_from_above<1>(al[hm]);
                float x = s < t ? up : 1.0f;
                x *= dpp_from_above<1>(x);
                x *= dpp_from_above<2>(x);
                x *= dpp_from_above<4>(x);
                x *= dpp_from_above<8>(x);
                const float v = t >= s ? x : 0.0f;
                m_s[par][hm][t * kTS + s] = v;
                if (t == kC - 1) pd_s[b4][1][hm][s] = v;
                if (s == 0) pd_s[b4][0][hm][t] = al[hm] * v;
            }
            __builtin_amdgcn_s_setprio(0);
        }
    };

    // k.k and k.q tiles in parts over the 16-column slices, two slices (four
    // 16-byte operand rows, requested together) at a time.  In quarters three
    // parts: wave 2 (SIMD 2) slices 0..3, wave 1 (SIMD 1) slices 4, 5, wave 3
    // (SIMD 3) slices 6, 7.  In eighths two: wave 2 slices 0..3, wave 3 slices
    // 4..7 (SIMDs 2 and 3 hold one state wave each there).  Lane (g, li),
    // register r holds k_{4g+r}.k_{li} and k_{4g+r}.q_{li}; the parts are
    // summed where they are used.
    auto tiles = [&](int c) {
        if (SL == 4 ? (w >= 1 && w <= 3) : (w == 2 || w == 3)) {
            __builtin_amdgcn_s_setprio(2);
            const int b3 = c % kBufs, par = c & 1;
            const float *kr = &kq_s[b3][0][li * kKS + 4 * g];
            const float *qr = &kq_s[b3][1][li * kKS + 4 * g];
            f32x4 KK = f32x4{0.f, 0.f, 0.f, 0.f}, KQ = KK;
            auto two_slices = [&](int s0) {
                f32x4 ka[2], qa[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    ka[i] = *reinterpret_cast<const f32x4 *>(kr + 16 * (s0 + i));
                    qa[i] = *reinterpret_cast<const f32x4 *>(qr + 16 * (s0 + i));
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        KK = mfma(ka[i][r], ka[i][r], KK);
                        KQ = mfma(ka[i][r], qa[i][r], KQ);
                    }
            };
            const int s0 = SL == 4 ? (w == 2 ? 0 : w == 1 ? 4 : 6) : (w == 2 ? 0 : 4);
            two_slices(s0);
            if (SL == 8 || w == 2) two_slices(s0 + 2);
            const int part = SL == 4 ? w - 1 : w - 2;
            part_s[par][part][0][l] = KK;
            part_s[par][part][1][l] = KQ;
            __builtin_amdgcn_s_setprio(0);
        }
    };

    // Wave 0: A, T and G of chunk c for the R heads.  Lane (g, li) owns
    // A[4g + r][li] = beta_{4g+r} M[4g+r][li] (k_{4g+r}.k_{li}) below the
    // diagonal and G[li][4g + r] = M[li][4g+r] (k_{4g+r}.q_{li}) / sqrt(D); k.k is
    // symmetric, so no value moves between lanes before LDS.  Then lane group g
    // solves head g: T = (I + A)^{-1} column li by column-oriented forward
    // substitution with the identity column as right-hand side (the entries
    // above li come out exactly 0 and T[li][li] exactly 1).  Every LDS value
    // the first part needs is requested at once; the entries of A on and above
    // the diagonal, which the solve never reads, are masked by a multiply (a
    // select let the compiler move loads behind a branch and wait on each).
    auto solve = [&](int c) {
        if (w == 0) {
            __builtin_amdgcn_s_setprio(2);
            const int b4 = c & 3, par = c & 1;
            f32x4 KKp[kParts], KQp[kParts], bet[R], mG[R], mA[R];
#pragma unroll
            for (int v2 = 0; v2 < kParts; ++v2) {
                KKp[v2] = part_s[par][v2][0][l];
                KQp[v2] = part_s[par][v2][1][l];
            }
#pragma unroll
            for (int hm = 0; hm < R; ++hm) {
                bet[hm] = *reinterpret_cast<const f32x4 *>(&ab_s[b4][1][hm][4 * g]);
                mG[hm] = *reinterpret_cast<const f32x4 *>(&m_s[par][hm][li * kTS + 4 * g]);   // M[li][4g+r]
#pragma unroll
                for (int r = 0; r < 4; ++r) mA[hm][r] = m_s[par][hm][(4 * g + r) * kTS + li];   // M[4g+r][li]
            }
            f32x4 KK = KKp[0], KQ = KQp[0];
#pragma unroll
            for (int v2 = 1; v2 < kParts; ++v2) {
                KK += KKp[v2];
                KQ += KQp[v2];
            }
            const f32x4 KQs = KQ * a.scale;
            f32x4 below;
#pragma unroll
            for (int r = 0; r < 4; ++r) below[r] = li < 4 * g + r ? 1.0f : 0.0f;
#pragma unroll
            for (int hm = 0; hm < R; ++hm) {
                *reinterpret_cast<f32x4 *>(&a_s[hm][li * kTS + 4 * g]) = bet[hm] * mA[hm] * KK * below;
                *reinterpret_cast<f32x4 *>(&g_s[par][hm][li * kTS + 4 * g]) = mG[hm] * KQs;
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
            const int hs = g < R ? g : R - 1;   // lane groups past R repeat the last head, unwritten
            // the identity column is formed here, not hoisted out of the chunk
            // loop (16 registers held across it)
            float one = 1.0f;
            asm volatile("" : "+v"(one));
            float x[kC];
#pragma unroll
            for (int t = 0; t < kC; ++t) x[t] = t == li ? one : 0.0f;
#pragma unroll
            for (int s2 = 0; s2 < kC - 1; ++s2) {
#pragma unroll
                for (int t4 = (s2 + 1) / 4; t4 < kC / 4; ++t4) {
                    const f32x4 av = *reinterpret_cast<const f32x4 *>(&a_s[hs][s2 * kTS + 4 * t4]);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * t4 + e > s2) x[4 * t4 + e] = fmaf(-av[e], x[s2], x[4 * t4 + e]);
                }
            }
            if (g < R) {
#pragma unroll
                for (int t = 0; t < kC; ++t) t_s[par][g][t * kTS + li] = x[t];
            }
            __builtin_amdgcn_s_setprio(0);
        }
    };

    // v of the lane's row for tokens 4g .. 4g+3 (rows past T read 0)
    const int64_t v0 = row_base * a.v_stride + (int64_t)h * kD;
    const int v_off = (int)((4 * g * a.v_stride + row) * 4);
    const int v_step = (int)(a.v_stride * 4);
    float vv[4];
    auto load_v = [&](int c) {
        const int t0 = c * kC;
        const __amdgpu_buffer_rsrc_t rv =
            buf_rsrc(a.v + v0 + (int64_t)t0 * a.v_stride, (int64_t)(T - t0) * a.v_stride * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) vv[r] = buf_load1(rv, v_off + r * v_step);
    };

    // Prologue: chunks 0 and 1 staged, their range products and tiles formed;
    // chunk 2's loads and chunk 0's v in flight.
    prefetch(0);
    __builtin_amdgcn_s_waitcnt(0);
    stage(0);
    if (nc > 1) {
        prefetch(1);
        __builtin_amdgcn_s_waitcnt(0);
        stage(1);
    }
    __syncthreads();
    range_products(0);
    tiles(0);
    if (nc > 1) {
        range_products(1);
        tiles(1);
    }
    if (nc > 2) prefetch(2);
    load_v(0);
    // drain every load (the state included) so that no conservative vmcnt wait
    // lands inside the chunk loop
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    const float *o0 = static_cast<const float *>(a.out) + row_base * a.out_stride + (int64_t)h * kD;
    const int o_off = (int)((4 * g * a.out_stride + row) * 4);
    const int o_step = (int)(a.out_stride * 4);
    for (int c = 0; c < nc; ++c) {
        const int b3 = c % kBufs, par = c & 1;
        const int t0 = c * kC;
        // partial U^T = K S^T and W^T = Q S^T over this wave's 64 columns: Mp is
        // U in half 0 and W in half 1, Xp the other one
        f32x4 Mp = f32x4{0.f, 0.f, 0.f, 0.f}, Xp = Mp;
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            const int col = 64 * half + 16 * t4 + 4 * g;
            const f32x4 ma = *reinterpret_cast<const f32x4 *>(&kq_s[b3][half][li * kKS + col]);
            const f32x4 xa = *reinterpret_cast<const f32x4 *>(&kq_s[b3][half ^ 1][li * kKS + col]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                Mp = mfma(ma[r], S[t4][r], Mp);
                Xp = mfma(xa[r], S[t4][r], Xp);
            }
        }
        const int si = NSTRIP * m + strip;
        if (half == 0) {
            x_s[par][si][0][l] = Mp;
            x_s[par][si][1][l] = Xp;
        } else {
            x_s[par][si][2][l] = Xp;
        }
        if (c + 2 < nc) stage(c + 2);
        solve(c);          // wave 0, after its own products
        // beta, P and D of head m at 4g.. (published by the previous barrier),
        // read before this one so that their latency is spent waiting at it
        const int b4 = c & 3;
        const f32x4 Br = *reinterpret_cast<const f32x4 *>(&ab_s[b4][1][m][4 * g]);
        const f32x4 Pr = *reinterpret_cast<const f32x4 *>(&pd_s[b4][0][m][4 * g]);
        const f32x4 Dr = *reinterpret_cast<const f32x4 *>(&pd_s[b4][1][m][4 * g]);
        const float p15 = pd_s[b4][0][m][kC - 1];
        // The one barrier of the chunk: partials visible; chunk c + 2 staged; T
        // and G of chunk c visible.  Every buffer written before it is read
        // after it and not written again before the next chunk's barrier
        // (partials by chunk parity, alpha / beta / P / D four chunks deep).
        __syncthreads();

        // The strip chain's LDS operands are requested first, in one batch with
        // no branch on the half (LDS answers a wave's requests in order, so the
        // chain's first wait covers only them): T[li][4g..] and G[li][4g..] /
        // sqrt(D) of head m, the other half's U part (slot 2 for half 0, slot 0
        // for half 1) and half 0's W part (used by half 1).  Then the update's
        // k operands (token 4g + s4, column 64 half + 16 t4 + li), whose latency
        // passes under the chain.
        const f32x4 Tr = *reinterpret_cast<const f32x4 *>(&t_s[par][m][li * kTS + 4 * g]);
        const f32x4 Uo = x_s[par][si][2 - 2 * half][l];
        const f32x4 Gr = *reinterpret_cast<const f32x4 *>(&g_s[par][m][li * kTS + 4 * g]);
        const f32x4 Wo = x_s[par][si][1][l];
        float kcv[16];
        {
            const float *kc = &kq_s[b3][0][4 * g * kKS + 64 * half + li];
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
                for (int t4 = 0; t4 < 4; ++t4) kcv[4 * s4 + t4] = kc[s4 * kKS + 16 * t4];
        }
        // gam S -> P_15 gam S + K^T (C' diag(D))^T: the decay is kept in gam
        // while it stays in [2^-60, 2^60] and folded into S otherwise.
        // 1 / gam' is the hardware reciprocal: the scale of one chunk's
        // contribution is off by an ulp or so, far inside the tolerance.
        const float gc = gam;
        float gnew = gc * p15;
        float cscale;
        if (__builtin_expect(gnew >= 0x1p-60f && gnew <= 0x1p60f, 1)) {
            cscale = __builtin_amdgcn_rcpf(gnew);
        } else {
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) S[t4] *= gnew;
            gnew = 1.0f;
            cscale = 1.0f;
        }
        gam = gnew;
        const f32x4 Ds = Dr * cscale;
        // Both halves of a strip form R = beta (v - P gam U) and C' = T R (so
        // no second barrier passes C' between them); half 1 also forms
        // O = P gam W + G C' and stores the four tokens.  Both update their
        // own columns with C'.
        __builtin_amdgcn_s_setprio(2);   // the strip's dependent chain ahead of other waves' products
        const f32x4 U = (half == 0 ? Mp : Xp) + Uo;
        f32x4 Rv;
#pragma unroll
        for (int r = 0; r < 4; ++r) Rv[r] = Br[r] * (vv[r] - Pr[r] * gc * U[r]);
        f32x4 X = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) X = mfma(Tr[r], Rv[r], X);
        if (half == 1) {
            const f32x4 W = Mp + Wo;
            const float gs = gc * a.scale;
            f32x4 O;   // G carries the 1 / sqrt(D) of the output
#pragma unroll
            for (int r = 0; r < 4; ++r) O[r] = Pr[r] * gs * W[r];
#pragma unroll
            for (int r = 0; r < 4; ++r) O = mfma(Gr[r], X[r], O);
            const __amdgpu_buffer_rsrc_t ro =
                buf_rsrc(o0 + (int64_t)t0 * a.out_stride, (int64_t)(T - t0) * a.out_stride * 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) buf_store1(ro, o_off + r * o_step, O[r]);
        }
        __builtin_amdgcn_s_setprio(0);
        // The loads for later chunks go out here, after this chunk's stores and
        // before the update: chunk c + 3's k, q, alpha, beta, then chunk c + 1's
        // v (rows past T read 0, so it needs no bound).  The vector memory
        // counter retires in order, and these are the last memory operations
        // of the chunk: the staging of chunk c + 3 waits with the four v loads
        // still in flight, and the next chain's wait for v has nothing younger
        // to wait for.  Issued after the update, every wave waited on them at
        // the next chain, most of a memory latency for the late ones (0.936 ->
        // 0.914 ms).
        if (c + 3 < nc) prefetch(c + 3);
        load_v(c + 1);

        X *= Ds;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4) S[t4] = mfma(kcv[4 * s4 + t4], X[s4], S[t4]);

        if (c + 2 < nc) {
            tiles(c + 2);
            range_products(c + 2);
        }
    }

#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) *reinterpret_cast<f32x4 *>(srow + 16 * t4) = S[t4] * gam;
}

bool seq_group_fits(const StepArgs &a) {
    // at most three value heads per key head: with four the workgroup has 1024
    // threads, which caps a wave at 128 VGPRs, and the loop spills (2.15 ms
    // against 1.22 ms for one workgroup per head at B = 4, T = 4096, NV = 64).
    // The grid and the 32-bit lane offsets of the buffer loads and stores,
    // which reach the last row of a whole chunk (padding rows included), must
    // fit.
    const int r = a.nv / a.nk;
    int64_t widest = a.qk_stride > a.v_stride ? a.qk_stride : a.v_stride;
    widest = widest > a.out_stride ? widest : a.out_stride;
    const int64_t rows = a.seq_len > kC ? a.seq_len : kC;
    return r >= 1 && r <= 3 && (int64_t)a.batch * a.nk * 4 <= INT32_MAX &&
           ((int64_t)a.batch * a.seq_len * a.nv + 15) / 16 <= INT32_MAX &&
           rows * widest * 4 + 1024 <= INT32_MAX;
}

hipError_t launch_seq_group(const StepArgs &a, OutMode mode, hipStream_t stream) {
    if (mode != kOutRawF32 && mode != kOutNormF32) return hipErrorInvalidValue;
    const int nc = (a.seq_len + kC - 1) / kC;
    const int r = a.nv / a.nk;
    const int64_t ngroups = (int64_t)a.batch * a.nk;
    // Eighths when a grid of them still runs in one pass over the compute
    // units (B * NK <= 32 on 256 CUs): twice the workgroups of quarters there.
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 0;
    const bool eighths = r == 3 && ngroups * 8 <= cus;
    const unsigned grid = (unsigned)(ngroups * (eighths ? 8 : 4));
    hipError_t e;
    switch (r) {
        case 1: e = launch(seq_group_kernel<1, 4>, dim3(grid), dim3(256), 0, stream, a, nc); break;
        case 2: e = launch(seq_group_kernel<2, 4>, dim3(grid), dim3(512), 0, stream, a, nc); break;
        case 3:
            e = eighths ? launch(seq_group_kernel<3, 8>, dim3(grid), dim3(384), 0, stream, a, nc)
                        : launch(seq_group_kernel<3, 4>, dim3(grid), dim3(768), 0, stream, a, nc);
            break;
        default: return hipErrorInvalidValue;
    }
    // with z the output rows get the gated norm in a second pass (four or
    // eight workgroups hold a head's rows between them)
    if (e != hipSuccess || mode == kOutRawF32) return e;
    return launch_norm_rows(a, stream);
}

}  // namespace gdn
