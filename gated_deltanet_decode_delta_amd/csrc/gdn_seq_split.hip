// gdn_seq_split.hip -- the T-token recurrence at D = 128, raw output, with the
// state-independent chunk quantities formed once ahead and each head split over
// four workgroups.
//
// Same chunked algebra as gdn_seq_mfma.hip (16 tokens per chunk; metrale
// "layers/ops/ssm_gdn_a.rs" `gdn_prefill_regresident` for the operation, the
// update of logicaffeine "codegen_cuda/gdn.rs" `gdn_step`): with M[t][s] =
// alpha_{s+1} ... alpha_t, P_t = alpha_0 ... alpha_t and S0 the state at the
// chunk start,
//     C' = T R,  R = beta (V - P S0 K^T),  T = (I + A)^{-1},
//          A[t][s] = beta_t M[t][s] (k_s.k_t)  (s < t)
//     O  = P S0 Q^T + C' G^T,  G[t][s] = M[t][s] (k_s.q_t)  (s <= t)
//     S_end = P_15 S0 + C' diag(M[15][.]) K.
// T, G, beta, P and D = M[15][.] depend on the inputs only.  A pre-pass
// (`prep_kernel`) forms them for every (sequence, value head, chunk) into a
// workspace: the k.k and k.q tiles once per key head instead of once per value
// head, and the triangular inverse by forward substitution off the state
// kernel's SIMDs.
//
// The state pass (`split_kernel`): one workgroup of four waves per quarter of a
// head (32 state rows).  Wave (strip, half) owns rows 16 strip .. +15 of the
// quarter and key columns 64 half .. +63: four 16x16 accumulator tiles.  The
// two halves of a strip form partial U = S0 K^T and W = S0 Q^T over their
// columns and exchange them through LDS; half 0 then forms C', half 1 O from
// it, and both update their own columns.  192 heads make 768 workgroups, three
// per CU and three waves per SIMD on all 256 CUs, each wave issuing 52
// matrix-core products per chunk (a workgroup per head puts two 104-product
// waves on each SIMD of 192 CUs).  Waves of different workgroups share a SIMD,
// so one workgroup's barrier and chain latency are covered by the others'
// products.
#include "gdn_chunk.h"
#include "gdn_device.h"
#include "gdn_launch.h"

namespace gdn {

using namespace chunk;

// ---------------------------------------------------------------------------
// Pre-pass: one wave per (sequence b, key head kh, chunk c).  Tokens past T
// get alpha 1, beta 0 and zero k, q, so they change nothing.  k and q go
// straight from global memory into the matrix-core operand layout (lane (g, li)
// holds row li, columns 16m + 4g .. +3), and the alpha, beta loads of up to 16
// value heads are issued together, ahead of the work on them.  Four value
// heads at a time share the wave: each forms its M, A, G, beta, P and D in
// turn, then lane group g solves head g, so one substitution serves four heads
// and only A passes through LDS (M[li][4g..] for G comes from a prefix product
// along the lane row).  Four waves per SIMD (100 VGPRs, no spill; five spill):
// the pre-pass is bound by its own traffic, so more waves in flight help.
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4))) prep_kernel(StepArgs a, float *ws,
                                                                                           int nc) {
    constexpr int kHG = 16;   // value heads whose alpha, beta are staged at once
    // per head of four: a_s[s][t] = A[t][s], heads four words apart in the banks
    __shared__ __align__(16) float a_s[4][kC * kTS + 4];
    __shared__ __align__(16) float al_s[kHG][kC];
    __shared__ __align__(16) float be_s[kHG][kC];

    const int l = threadIdx.x, g = l >> 4, li = l & 15;
    const int item = blockIdx.x;
    const int c = item % nc;
    const int bk = item / nc;
    const int kh = bk % a.nk;
    const int b = bk / a.nk;
    const int T = a.seq_len;
    const int t0 = c * kC;
    const int64_t row_base = (int64_t)b * T;
    const int rep = a.nv / a.nk;

    const bool rok = t0 + li < T;
    const int64_t roff = (row_base + (rok ? t0 + li : T - 1)) * a.qk_stride + (int64_t)kh * kD + 4 * g;
    f32x4 kr[kD / 16], qr[kD / 16];
#pragma unroll
    for (int m = 0; m < kD / 16; ++m) {
        kr[m] = *reinterpret_cast<const f32x4 *>(a.k + roff + 16 * m);
        qr[m] = *reinterpret_cast<const f32x4 *>(a.q + roff + 16 * m);
    }
    // alpha, beta of value heads m0 .. m0 + 15: entry e = l + 64 j is head e / 16, token e % 16
    float ar[4], br[4];
    auto load_ab = [&](int m0) {
        const int ng = rep - m0 < kHG ? rep - m0 : kHG;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = l + 64 * j, m = e >> 4, t = e & 15;
            if (m < ng) {
                const bool ok = t0 + t < T;
                const int64_t rr = (row_base + (ok ? t0 + t : T - 1)) * a.ab_stride + kh + (int64_t)(m0 + m) * a.nk;
                const float ax = a.alpha[rr], bx = a.beta[rr];
                ar[j] = ok ? ax : 1.0f;
                br[j] = ok ? bx : 0.0f;
            }
        }
    };
    auto store_ab = [&](int m0) {
        const int ng = rep - m0 < kHG ? rep - m0 : kHG;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = l + 64 * j, m = e >> 4, t = e & 15;
            if (m < ng) {
                al_s[m][t] = ar[j];
                be_s[m][t] = br[j];
            }
        }
    };
    load_ab(0);
    if (!rok) {
#pragma unroll
        for (int m = 0; m < kD / 16; ++m) {
            kr[m] = f32x4{0.f, 0.f, 0.f, 0.f};
            qr[m] = kr[m];
        }
    }
    // lane (g, li), register r: KK[r] = k_{4g+r}.k_{li}, KQ[r] = k_{4g+r}.q_{li}
    f32x4 K0 = f32x4{0.f, 0.f, 0.f, 0.f}, K1 = K0, Q0 = K0, Q1 = K0;
#pragma unroll
    for (int m = 0; m < kD / 16; ++m) {
        K0 = mfma(kr[m][0], kr[m][0], K0);
        Q0 = mfma(kr[m][0], qr[m][0], Q0);
        K1 = mfma(kr[m][1], kr[m][1], K1);
        Q1 = mfma(kr[m][1], qr[m][1], Q1);
        K0 = mfma(kr[m][2], kr[m][2], K0);
        Q0 = mfma(kr[m][2], qr[m][2], Q0);
        K1 = mfma(kr[m][3], kr[m][3], K1);
        Q1 = mfma(kr[m][3], qr[m][3], Q1);
    }
    const f32x4 KK = K0 + K1, KQ = Q0 + Q1;

    for (int m0 = 0; m0 < rep; m0 += kHG) {
        __syncthreads();   // the previous group's reads of al_s, be_s are done
        store_ab(m0);
        if (m0 + kHG < rep) load_ab(m0 + kHG);
        __syncthreads();
        const int ng = rep - m0 < kHG ? rep - m0 : kHG;
        // value heads mg .. mg + 3 of the group side by side: lane group g
        // solves head mg + g
        for (int mg = 0; mg < ng; mg += 4) {
            const int nh = ng - mg < 4 ? ng - mg : 4;
#pragma unroll
            for (int hm = 0; hm < 4; ++hm) {
                if (hm >= nh) break;
                const int mm = mg + hm;
                const int h = kh + (m0 + mm) * a.nk;   // tiled pairing: value heads kh, kh + NK, ...
                float *rec = ws + (((int64_t)b * a.nv + h) * nc + c) * kSeqRec;
                // M[4g + r][li] by suffix products along the DPP row (no division)
                f32x4 Mv, acol;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 4 * g + r;
                    float x = al_s[mm][li < t ? li + 1 : 0];   // index kept to written entries
                    x = li < t ? x : 1.0f;
                    x *= dpp_from_above<1>(x);
                    x *= dpp_from_above<2>(x);
                    x *= dpp_from_above<4>(x);
                    x *= dpp_from_above<8>(x);
                    Mv[r] = t >= li ? x : 0.0f;
                    acol[r] = li < t ? be_s[mm][t] * Mv[r] * KK[r] : 0.0f;
                }
                *reinterpret_cast<f32x4 *>(&a_s[hm][li * kTS + 4 * g]) = acol;   // a_s[s][t] = A[t][s]
                // M[li][4g + r] for G: a prefix product along the row gives
                // alpha_{4g+4} ... alpha_li, and the three below it follow by
                // one multiply each (1 on the diagonal, 0 above it)
                float y = li >= 4 * g + 4 ? al_s[mm][li] : 1.0f;
                y *= dpp_from_below<1>(y);
                y *= dpp_from_below<2>(y);
                y *= dpp_from_below<4>(y);
                y *= dpp_from_below<8>(y);
                const f32x4 up = *reinterpret_cast<const f32x4 *>(&al_s[mm][4 * g]);   // alpha_{4g} .. alpha_{4g+3}
                f32x4 Mg;
                Mg[3] = li >= 4 * g + 3 ? y : 0.0f;
                Mg[2] = li > 4 * g + 2 ? up[3] * Mg[3] : (li == 4 * g + 2 ? 1.0f : 0.0f);
                Mg[1] = li > 4 * g + 1 ? up[2] * Mg[2] : (li == 4 * g + 1 ? 1.0f : 0.0f);
                Mg[0] = li > 4 * g ? up[1] * Mg[1] : (li == 4 * g ? 1.0f : 0.0f);
                // workspace record: G / sqrt(D) row-major, beta, P, D (T below)
                *reinterpret_cast<f32x4 *>(rec + 256 + li * kC + 4 * g) = Mg * KQ * a.scale;
                if (g == 0) rec[512 + li] = be_s[mm][li];
                if (li == 0) *reinterpret_cast<f32x4 *>(rec + 528 + 4 * g) = al_s[mm][0] * Mv;   // P_t = alpha_0 M[t][0]
                if (g == 3) rec[544 + li] = Mv[3];                                             // D[s] = M[15][s]
            }
            __syncthreads();
            // T = (I + A)^{-1} of head mg + g, column li per lane: column-oriented
            // forward substitution, rows of the transposed A read four at a
            // time; the column goes to the record's T (row-major) directly
            if (g < nh) {
                float x[kC];
#pragma unroll
                for (int t = 0; t < kC; ++t) x[t] = t == li ? 1.0f : 0.0f;
#pragma unroll
                for (int s2 = 0; s2 < kC - 1; ++s2) {
#pragma unroll
                    for (int t4 = (s2 + 1) / 4; t4 < kC / 4; ++t4) {
                        const f32x4 av = *reinterpret_cast<const f32x4 *>(&a_s[g][s2 * kTS + 4 * t4]);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (4 * t4 + e > s2) x[4 * t4 + e] = fmaf(-av[e], x[s2], x[4 * t4 + e]);
                    }
                }
                const int h = kh + (m0 + mg + g) * a.nk;
                float *rec = ws + (((int64_t)b * a.nv + h) * nc + c) * kSeqRec;
#pragma unroll
                for (int t = 0; t < kC; ++t) rec[t * kC + li] = x[t];
            }
            __syncthreads();   // a_s free for the next heads
        }
    }
}

// ---------------------------------------------------------------------------
// State pass.  Block b_id -> (head, quarter): the four quarters of a head get
// indices equal modulo 8, so they run on one XCD and share its L2 for the
// head's workspace records and k, q rows.
__global__ void __launch_bounds__(256) split_kernel(StepArgs a, const float *ws, int nc) {
    __shared__ __align__(16) float kq_s[2][2][kC * kKS];   // [buffer][k, q] of a chunk
    __shared__ f32x4 x_s[4][64];      // each wave's partial that its partner needs
    __shared__ f32x4 c_s[2][64];      // C' of each strip

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l = tid & 63, g = l >> 4, li = l & 15;
    const int half = w & 1, strip = w >> 1;

    const int nheads = a.batch * a.nv;
    const int full = nheads / 8 * 8;
    int head, quarter;
    {
        const int bid = blockIdx.x;
        if (bid < full * 4) {
            const int r = bid & 31;
            head = (bid >> 5) * 8 + (r & 7);
            quarter = r >> 3;
        } else {
            const int r = bid - full * 4, rem = nheads - full;
            head = full + r % rem;
            quarter = r / rem;
        }
    }
    const int b = head / a.nv;
    const int h = head - b * a.nv;
    const int kh = h % a.nk;
    const int T = a.seq_len;
    const int64_t row_base = (int64_t)b * T;
    const int row = 32 * quarter + 16 * strip + li;          // state row (value index)
    float *srow = static_cast<float *>(a.state) + (int64_t)b * a.pitch + (int64_t)h * (kD * kD) +
                  (int64_t)row * kD + 64 * half + 4 * g;
    const float *wsh = ws + (int64_t)head * nc * kSeqRec;

    // The true state is gam * S; S[m][r] = S[row][64 half + 16 m + 4 g + r].
    f32x4 S[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) S[m] = *reinterpret_cast<const f32x4 *>(srow + 16 * m);
    float gam = 1.0f;

    // k and q of a chunk: pieces f = tid + 256 u (u = 0, 1), token f >> 5 =
    // tid / 32 + 8 u, columns (tid % 32) * 4, read through descriptors based at
    // the chunk's first row.  Rows past T (the tail chunk and the chunks after
    // it) read 0 (the pre-pass gives those tokens beta 0 and alpha 1, so their
    // k, q and v only meet zero coefficients).
    const int tl = tid >> 5;
    const int64_t kq0 = row_base * a.qk_stride + (int64_t)kh * kD;
    int kq_off[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) kq_off[u] = (int)(((tl + 8 * u) * a.qk_stride + (tid & 31) * 4) * 4);
    f32x4 pk[2], pq[2];   // vector-typed so they stay in registers
    auto prefetch_kq = [&](int c) {
        const int t0 = c * kC;
        const int64_t off = kq0 + (int64_t)t0 * a.qk_stride;   // uniform
        const int64_t nb = (int64_t)(T - t0) * a.qk_stride * 4;
        const __amdgpu_buffer_rsrc_t rk = buf_rsrc(a.k + off, nb), rq = buf_rsrc(a.q + off, nb);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            pk[u] = buf_load4(rk, kq_off[u]);
            pq[u] = buf_load4(rq, kq_off[u]);
        }
    };
    auto stage = [&](int c) {
        const int bb = c & 1;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int f = tid + 256 * u;
            *reinterpret_cast<f32x4 *>(&kq_s[bb][0][(f >> 5) * kKS + (f & 31) * 4]) = pk[u];
            *reinterpret_cast<f32x4 *>(&kq_s[bb][1][(f >> 5) * kKS + (f & 31) * 4]) = pq[u];
        }
    };
    // per-chunk data of the lane: v of its row for tokens 4g .. 4g+3, and the
    // workspace record (T[li][4g..], G[li][4g..], beta, P, D at 4g..)
    const int64_t v0 = row_base * a.v_stride + (int64_t)h * kD;
    const int v_off = (int)((4 * g * a.v_stride + row) * 4);
    const int v_step = (int)(a.v_stride * 4);
    const int lrec = li * kC + 4 * g;
    float vv[4];
    f32x4 Tr, Gr, Br, Pr, Dr;
    // Only half 0 uses v (rows past T read 0).  Both halves load the whole
    // record: loading T in one half and G in the other made the compiler keep
    // the pair in scratch.
    auto load_chunk = [&](int c) {
        const int t0 = c * kC;
        const float *rec = wsh + (int64_t)(c < nc ? c : nc - 1) * kSeqRec;   // uniform
        const __amdgpu_buffer_rsrc_t rv =
            buf_rsrc(a.v + v0 + (int64_t)t0 * a.v_stride, (int64_t)(T - t0) * a.v_stride * 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            vv[r] = 0.0f;
            if (half == 0) vv[r] = buf_load1(rv, v_off + r * v_step);
        }
        Tr = *reinterpret_cast<const f32x4 *>(rec + lrec);
        Gr = *reinterpret_cast<const f32x4 *>(rec + 256 + lrec);
        Br = *reinterpret_cast<const f32x4 *>(rec + 512 + 4 * g);
        Pr = *reinterpret_cast<const f32x4 *>(rec + 528 + 4 * g);
        Dr = *reinterpret_cast<const f32x4 *>(rec + 544 + 4 * g);
    };

    // Prologue: chunk 0 staged; chunk 1's k, q and chunk 0's v and record in flight.
    prefetch_kq(0);
    stage(0);
    // drain every load (the state included) so that no conservative vmcnt wait
    // lands inside the chunk loop
    __builtin_amdgcn_s_waitcnt(0);
    prefetch_kq(1);
    load_chunk(0);
    __syncthreads();

    // o of the lane's row for tokens 4g .. 4g+3 (stores past T are dropped)
    const float *o0 = static_cast<const float *>(a.out) + row_base * a.out_stride + (int64_t)h * kD;
    const int o_off = (int)((4 * g * a.out_stride + row) * 4);
    const int o_step = (int)(a.out_stride * 4);
    for (int c = 0; c < nc; ++c) {
        const int bb = c & 1;
        const int t0 = c * kC;
        // the update's k operands (token 4g + s4, column 64 half + 16 m + li),
        // requested now so that their LDS latency is long past at the update
        float kcv[16];
        {
            const float *kc = &kq_s[bb][0][4 * g * kKS + 64 * half + li];
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
                for (int m = 0; m < 4; ++m) kcv[4 * s4 + m] = kc[s4 * kKS + 16 * m];
        }
        // partial U^T = K S^T and W^T = Q S^T over this wave's 64 columns,
        // one accumulator each (a product accumulating into its own
        // destination issues back to back).  Mp is the one the wave goes on
        // with (U in half 0, W in half 1), Xp the one its partner needs: the
        // operand rows are picked by half, so no select of results is needed.
        f32x4 Mp = f32x4{0.f, 0.f, 0.f, 0.f}, Xp = Mp;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int col = 64 * half + 16 * m + 4 * g;
            const f32x4 ma = *reinterpret_cast<const f32x4 *>(&kq_s[bb][half][li * kKS + col]);
            const f32x4 xa = *reinterpret_cast<const f32x4 *>(&kq_s[bb][half ^ 1][li * kKS + col]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                Mp = mfma(ma[r], S[m][r], Mp);
                Xp = mfma(xa[r], S[m][r], Xp);
            }
        }
        x_s[w][l] = Xp;
        __syncthreads();   // partials visible; every wave is past chunk c - 1
        // chunk c + 1 into the buffer chunk c - 1 used (rows past the end are
        // staged too, into a buffer no one reads); visible after the next barrier
        stage(c + 1);
        // gam S -> P_15 gam S + K^T (C' diag(D))^T: the decay is kept in gam
        // while it stays in [2^-60, 2^60] and folded into S otherwise.  Done
        // here, ahead of the chain (which uses gc, gam at the chunk start), so
        // that nothing after half 1's stores waits on a load.  P_15 is lane
        // 48's last P.  1 / gam' comes from the hardware reciprocal: the scale
        // of one chunk's contribution is off by an ulp or so, far inside the
        // tolerance, and both halves compute the same value.
        const float gc = gam;
        // The element goes through an opaque copy first: hipcc (clang 22,
        // ROCm 7.2) lowers a lane read of element 3 of a four-float vector as
        // a read of element 0's register.
        float p15 = Pr[3];
        asm volatile("" : "+v"(p15));
        float gnew = gc * __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                        __builtin_bit_cast(int, p15), 48));
        float cscale;
        if (__builtin_expect(gnew >= 0x1p-60f && gnew <= 0x1p60f, 1)) {
            cscale = __builtin_amdgcn_rcpf(gnew);
        } else {
#pragma unroll
            for (int m = 0; m < 4; ++m) S[m] *= gnew;
            gnew = 1.0f;
            cscale = 1.0f;
        }
        gam = gnew;
        f32x4 Ds = Dr * cscale;
        asm volatile("" : "+v"(Ds));   // formed here, before half 1's stores
        // The strip's chain is split between its halves: half 0 forms
        // R = beta (v - P gam U) and C' = T R and passes C' on through LDS;
        // half 1 forms O = P gam W + G C' and stores the four tokens.  Both
        // update their own columns with C'.
        // X: C' in half 0; in half 1 the first term of O, then C' once read.
        // One variable for both halves keeps the branch joins free of copies.
        f32x4 X;
        __builtin_amdgcn_s_setprio(2);   // the strip's dependent chain ahead of other waves' products
        if (half == 0) {
            const f32x4 U = Mp + x_s[w ^ 1][l];
            f32x4 R;
#pragma unroll
            for (int r = 0; r < 4; ++r) R[r] = Br[r] * (vv[r] - Pr[r] * gc * U[r]);
            X = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < 4; ++r) X = mfma(Tr[r], R[r], X);
            c_s[strip][l] = X;
            __builtin_amdgcn_s_setprio(0);
        } else {
            const f32x4 W = Mp + x_s[w ^ 1][l];
            const float gs = gc * a.scale;
#pragma unroll
            for (int r = 0; r < 4; ++r) X[r] = Pr[r] * gs * W[r];
        }
        __syncthreads();   // C' visible; chunk c + 1 staged; every read of chunk c - 1's buffers done
        if (half == 1) {
            const f32x4 Cp = c_s[strip][l];
            f32x4 O = X;   // G carries the 1 / sqrt(D) of the output
#pragma unroll
            for (int r = 0; r < 4; ++r) O = mfma(Gr[r], Cp[r], O);
            const __amdgpu_buffer_rsrc_t ro =
                buf_rsrc(o0 + (int64_t)t0 * a.out_stride, (int64_t)(T - t0) * a.out_stride * 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) buf_store1(ro, o_off + r * o_step, O[r]);
            X = Cp;
            __builtin_amdgcn_s_setprio(0);
        }

        X *= Ds;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
            for (int m = 0; m < 4; ++m) S[m] = mfma(kcv[4 * s4 + m], X[s4], S[m]);

        // loads for the next chunks go out after this chunk's stores
        prefetch_kq(c + 2);
        load_chunk(c + 1);
    }

#pragma unroll
    for (int m = 0; m < 4; ++m) *reinterpret_cast<f32x4 *>(srow + 16 * m) = S[m] * gam;
}

// ---------------------------------------------------------------------------
// Gated RMS norm over the output rows, in place (the state pass writes raw o;
// four workgroups per head cannot form a head's sum of o^2 between them).
// logicaffeine "codegen_cuda/gdn.rs" `gdn_gate_norm`: r = sqrt(mean_i o_i^2 + eps),
// y_i = gn_i o_i / r * z_i sigmoid(z_i).  Sixteen lanes per (row, head), eight
// values each; the sum is a DPP reduction within the sixteen.
__global__ void __launch_bounds__(256) norm_rows_kernel(StepArgs a, int64_t items) {
    const int64_t item = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);   // (row, head)
    if (item >= items) return;   // whole sixteen-lane groups leave together
    const int j = threadIdx.x & 15;
    const int64_t row = item / a.nv;
    const int h = (int)(item - row * a.nv);
    float *o = static_cast<float *>(a.out) + row * a.out_stride + (int64_t)h * kD + 8 * j;
    const float *z = a.z + row * a.z_stride + (int64_t)h * kD + 8 * j;
    const f32x4 o0 = *reinterpret_cast<const f32x4 *>(o), o1 = *reinterpret_cast<const f32x4 *>(o + 4);
    const f32x4 z0 = *reinterpret_cast<const f32x4 *>(z), z1 = *reinterpret_cast<const f32x4 *>(z + 4);
    // the norm weight needs only 4-byte alignment: scalar loads (it stays in cache)
    const float *gp = a.gn + 8 * j;
    const f32x4 g0 = f32x4{gp[0], gp[1], gp[2], gp[3]}, g1 = f32x4{gp[4], gp[5], gp[6], gp[7]};
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += o0[e] * o0[e] + o1[e] * o1[e];
    ss = group_sum<16>(ss);
    const float r = sqrtf(ss * (1.0f / kD) + a.eps);
    f32x4 y0, y1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        y0[e] = (g0[e] * o0[e] / r) * silu(z0[e]);
        y1[e] = (g1[e] * o1[e] / r) * silu(z1[e]);
    }
    *reinterpret_cast<f32x4 *>(o) = y0;
    *reinterpret_cast<f32x4 *>(o + 4) = y1;
}

hipError_t launch_seq_split(const StepArgs &a, float *ws, hipStream_t stream) {
    const int nc = (a.seq_len + kC - 1) / kC;
    const int64_t items = (int64_t)a.batch * a.nk * nc;
    hipError_t e = launch(prep_kernel, dim3((unsigned)items), dim3(64), 0, stream, a, ws, nc);
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)((int64_t)a.batch * a.nv * 4);
    e = launch(split_kernel, dim3(grid), dim3(256), 0, stream, a, (const float *)ws, nc);
    if (e != hipSuccess || a.z == nullptr) return e;
    return launch_norm_rows(a, stream);
}

hipError_t launch_norm_rows(const StepArgs &a, hipStream_t stream) {
    const int64_t rows = (int64_t)a.batch * a.seq_len * a.nv;   // (row, head) pairs
    return launch(norm_rows_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, a, rows);
}

}  // namespace gdn
