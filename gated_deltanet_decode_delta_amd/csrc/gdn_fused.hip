// gdn_fused.hip -- the decode step with the layer's input stage fused in front:
// depthwise causal conv over a ring of the last `taps` projection rows, silu,
// per-head L2 normalisation of q and k, and the two gates, then the gated delta
// rule step and (optionally) the gated RMS norm of every value head.
// Sources: logicaffeine "codegen_cuda/gdn.rs", kernels `gk_conv_silu_l2` (ring
// shift, append, reduce, silu; L2 of the leading 2 NK head blocks with eps inside
// the root) and `gk_gdn_gates` (beta = sigmoid(br), decay = (1 + e^(ar+dt))^rate);
// metrale "layers/ops/ssm_gdn_a.rs", `gdn_decode_f32_conv_norm` (all of it in
// one decode launch, one block per key head owning its value heads' conv rows).
//
// Mapping.  One workgroup per (sequence b, key head g).  With the tiled pairing
// h = g + m NK (m < R = NV / NK), that workgroup is the only one that reads or
// writes the ring channels of q_g, k_g and v_h of its R value heads, so the
// in-place ring shift needs no synchronisation between workgroups.  The input
// stage runs once per key head (not once per value head), leaves its (2 + R) D
// features in LDS, and the R state tiles then stream through registers one
// after the other in the decode mapping of gdn_tile.h (load once, update, store
// once).  The extra bytes per head-step are the ring rows of its channels and
// the conv weights, a few KiB against the 128 KiB tile.
#include <type_traits>

#include "gdn_launch.h"
#include "gdn_tile.h"

namespace gdn {

size_t fused_lds_bytes(int dim, int r) {
    return sizeof(float) * ((size_t)(2 + r) * dim + 2 * (size_t)r + 2);
}

template <int D, bool NORM>
__global__ void __launch_bounds__((DecodeTile<D, float>::NT))
fused_kernel(StepArgs a, FrontArgs f) {
    using TL = DecodeTile<D, float>;
    using V = typename VecT<float, TL::VEC>::type;
    constexpr int LPR = TL::LPR, NCH = TL::NCH, C = TL::C, RPL = TL::RPL, VEC = TL::VEC;
    constexpr int NT = TL::NT;

    extern __shared__ __align__(16) float lds[];
    const int R = a.nv / a.nk;
    float *feat = lds;                 // [(2 + R) D]: q_g, k_g, then v of the R value heads
    float *gal = lds + (2 + R) * D;    // [R] decay
    float *gbe = gal + R;              // [R] write strength
    float *den = gbe + R;              // [2] L2 denominators of q_g and k_g
    __shared__ float part[2][TL::NT / 64];   // per-wave sums of o^2, by head parity

    const int wg = blockIdx.x;
    const int b = wg / a.nk;
    const int g = wg - b * a.nk;
    const int tid = threadIdx.x;
    const int64_t CH = (int64_t)(2 * a.nk + a.nv) * D;
    const int taps = f.taps;

    // tile mapping; the first value head's tile is requested before the input
    // stage so that its HBM latency overlaps the conv and the L2 norms
    const int p = tid % LPR;
    const int grp = tid / LPR;
    const bool active = grp < TL::NGA;
    const int row0 = grp * RPL;
    float s[RPL][C];
    // the tiles' vectors through buffer descriptors with the decode's cache policy
    auto tile_off = [&](int r, int c) { return ((row0 + r) * D + (c * LPR + p) * VEC) * (int)sizeof(float); };
    auto load_tile = [&](int m) {
        const float *slot = static_cast<const float *>(a.state) + (int64_t)b * a.pitch +
                            (int64_t)(g + m * a.nk) * (D * D);
        const __amdgpu_buffer_rsrc_t srs = tile_rsrc(slot, D * D * (int)sizeof(float));
#pragma unroll
        for (int r = 0; r < RPL; ++r)
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const V x = load_tile_vec<V>(srs, tile_off(r, c));
#pragma unroll
                for (int e = 0; e < VEC; ++e) s[r][c * VEC + e] = x[e];
            }
    };
    if (active) load_tile(0);

    // ---- conv ring: shift, append, reduce, silu -- this workgroup's channels
    {
        float *ring = f.ring + (int64_t)b * f.ring_stride;
        const float *x = f.x + (int64_t)b * f.x_stride;
        const int nvec = (2 + R) * (D / 4);
        for (int j4 = tid; j4 < nvec; j4 += NT) {
            const int j = 4 * j4;
            int64_t c;                                  // channel in the projection row
            if (j < D) {
                c = (int64_t)g * D + j;
            } else if (j < 2 * D) {
                c = (int64_t)(a.nk + g) * D + (j - D);
            } else {
                const int m = (j - 2 * D) / D;
                c = (int64_t)(2 * a.nk + g + m * a.nk) * D + (j - (2 + m) * D);
            }
            const float4 xv = *reinterpret_cast<const float4 *>(x + c);
            float4 hist[kMaxTaps - 1];                  // old rows 1 .. taps-1
#pragma unroll
            for (int t = 0; t < kMaxTaps - 1; ++t)
                if (t < taps - 1) hist[t] = *reinterpret_cast<const float4 *>(ring + (t + 1) * CH + c);
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int t = 0; t < kMaxTaps - 1; ++t)
                if (t < taps - 1) {
                    const float4 wv = *reinterpret_cast<const float4 *>(f.w + t * CH + c);
                    acc.x = fmaf(hist[t].x, wv.x, acc.x);
                    acc.y = fmaf(hist[t].y, wv.y, acc.y);
                    acc.z = fmaf(hist[t].z, wv.z, acc.z);
                    acc.w = fmaf(hist[t].w, wv.w, acc.w);
                }
            const float4 wl = *reinterpret_cast<const float4 *>(f.w + (int64_t)(taps - 1) * CH + c);
            acc.x = fmaf(xv.x, wl.x, acc.x);
            acc.y = fmaf(xv.y, wl.y, acc.y);
            acc.z = fmaf(xv.z, wl.z, acc.z);
            acc.w = fmaf(xv.w, wl.w, acc.w);
#pragma unroll
            for (int t = 0; t < kMaxTaps - 1; ++t)
                if (t < taps - 1) *reinterpret_cast<float4 *>(ring + t * CH + c) = hist[t];
            *reinterpret_cast<float4 *>(ring + (int64_t)(taps - 1) * CH + c) = xv;
            feat[j + 0] = silu(acc.x);
            feat[j + 1] = silu(acc.y);
            feat[j + 2] = silu(acc.z);
            feat[j + 3] = silu(acc.w);
        }
        // ---- gates of the R value heads
        for (int m = tid; m < R; m += NT) {
            const int h = g + m * a.nk;
            const int64_t e = (int64_t)b * f.g_stride + h;
            gbe[m] = 1.0f / (1.0f + expf(-f.br[e]));
            gal[m] = powf(1.0f + expf(f.ar[e] + f.dt[h]), f.rate[h]);
        }
    }
    __syncthreads();
    // ---- L2 of q_g and k_g: x / sqrt(sum x^2 + eps)
    if (tid < 64) {
        float sq = 0.f, sk = 0.f;
        for (int i = tid; i < D; i += 64) {
            sq = fmaf(feat[i], feat[i], sq);
            sk = fmaf(feat[D + i], feat[D + i], sk);
        }
        sq = group_sum_wide<64>(sq);
        sk = group_sum_wide<64>(sk);
        if (tid == 0) {
            den[0] = sqrtf(sq + f.l2_eps);
            den[1] = sqrtf(sk + f.l2_eps);
        }
    }
    __syncthreads();
    for (int i = tid; i < 2 * D; i += NT) feat[i] = feat[i] / den[i >= D ? 1 : 0];
    __syncthreads();

    // ---- the R value heads, one state tile at a time
    float kk[C], qq[C];
    float kq = 0.f;
    if (active) {
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int e4 = 0; e4 < VEC; e4 += 4) {
                const int col = (c * LPR + p) * VEC + e4;
                const float4 q4 = *reinterpret_cast<const float4 *>(feat + col);
                const float4 k4 = *reinterpret_cast<const float4 *>(feat + D + col);
                kk[c * VEC + e4 + 0] = k4.x; kk[c * VEC + e4 + 1] = k4.y;
                kk[c * VEC + e4 + 2] = k4.z; kk[c * VEC + e4 + 3] = k4.w;
                qq[c * VEC + e4 + 0] = q4.x; qq[c * VEC + e4 + 1] = q4.y;
                qq[c * VEC + e4 + 2] = q4.z; qq[c * VEC + e4 + 3] = q4.w;
            }
#pragma unroll
        for (int i = 0; i < C; ++i) kq = fmaf(kk[i], qq[i], kq);
        kq = group_sum<LPR>(kq);
    }
    const float gr = (NORM && active && p < RPL) ? a.gn[row0 + p] : 0.0f;

    for (int m = 0; m < R; ++m) {
        const int h = g + m * a.nk;
        float *slot = static_cast<float *>(a.state) + (int64_t)b * a.pitch + (int64_t)h * (D * D);
        float o_mine = 0.f, sumsq = 0.f, zr = 0.f;
        if (active) {
            if (m > 0) load_tile(m);
            if constexpr (NORM) {
                if (p < RPL) zr = a.z[(int64_t)b * a.z_stride + (int64_t)h * D + row0 + p];
            }
            const float alpha = gal[m];
            const float beta = gbe[m];
            const float *vh = feat + (2 + m) * D;
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
                float pu = 0.f, pw = 0.f;
#pragma unroll
                for (int i = 0; i < C; ++i) {
                    pu = fmaf(s[r][i], kk[i], pu);
                    pw = fmaf(s[r][i], qq[i], pw);
                }
                const float u = group_sum<LPR>(pu);
                const float w = group_sum<LPR>(pw);
                const float coef = beta * (vh[row0 + r] - alpha * u);
                const float o = (alpha * w + coef * kq) * a.scale;
                sumsq = fmaf(o, o, sumsq);
                if (r == p) o_mine = o;
                V x;
                const __amdgpu_buffer_rsrc_t srs = tile_rsrc(slot, D * D * (int)sizeof(float));
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) x[e] = alpha * s[r][c * VEC + e] + coef * kk[c * VEC + e];
                    store_tile_vec<V>(srs, tile_off(r, c), x);
                }
            }
        }
        float *outp = static_cast<float *>(a.out);
        const int64_t orow = (int64_t)b * a.out_stride + (int64_t)h * D + row0 + p;
        if constexpr (!NORM) {
            if (active && p < RPL) outp[orow] = o_mine;
        } else {
            // one barrier per head; the partials alternate between two buffers so
            // that head m + 2 never overwrites what a slow thread still reads
            const float wsum = wave_groups_sum<LPR>(active ? sumsq : 0.f);
            if ((tid & 63) == 0) part[m & 1][tid >> 6] = wsum;
            __syncthreads();
            if (active && p < RPL) {
                float tot = 0.f;
#pragma unroll
                for (int i = 0; i < TL::NT / 64; ++i) tot += part[m & 1][i];
                const float r = sqrtf(tot * (1.0f / D) + a.eps);
                outp[orow] = (gr * o_mine / r) * silu(zr);
            }
        }
    }
}

// The same step when the new ring goes to a second buffer (ring_out): the old
// ring is then read-only, so one workgroup per (sequence, value head) can run
// the input stage of its own key head redundantly (q_g and k_g from L2) next to
// its own v channels, exactly like the plain decode's one tile per workgroup.
// Only the workgroup of the key head's first value head (h < NK) writes the new
// q_g / k_g ring rows; every workgroup writes its own v rows.  For taps <= 4
// the input stage's loads are issued first and the tile's right after them,
// so the conv and the L2 norms run while the tile is in flight.
template <int D, bool NORM>
__global__ void __launch_bounds__((DecodeTile<D, float>::NT))
fused_split_kernel(StepArgs a, FrontArgs f, float *ring_out) {
    using TL = DecodeTile<D, float>;
    using V = typename VecT<float, TL::VEC>::type;
    constexpr int LPR = TL::LPR, NCH = TL::NCH, C = TL::C, RPL = TL::RPL, VEC = TL::VEC;
    constexpr int NT = TL::NT;
    static_assert(3 * D / 4 <= NT, "one four-channel vector per thread");
    constexpr int kShort = 4;

    __shared__ __align__(16) float feat[3 * D];   // q_g, k_g, v_h
    __shared__ float gates[2], den[2];
    __shared__ float part[TL::NT / 64];      // per-wave sums of o^2

    const int wg = blockIdx.x;
    const int b = wg / a.nv;
    const int h = wg - b * a.nv;
    const int g = h % a.nk;
    const int tid = threadIdx.x;
    const int64_t CH = (int64_t)(2 * a.nk + a.nv) * D;
    const int taps = f.taps;

    const int p = tid % LPR;
    const int grp = tid / LPR;
    const bool active = grp < TL::NGA;
    const int row0 = grp * RPL;
    float *slot = static_cast<float *>(a.state) + (int64_t)b * a.pitch + (int64_t)h * (D * D);
    // the tile's vectors through a buffer descriptor with the decode's cache policy
    const __amdgpu_buffer_rsrc_t srs = tile_rsrc(slot, D * D * (int)sizeof(float));
    auto tile_off = [&](int r, int c) { return ((row0 + r) * D + (c * LPR + p) * VEC) * (int)sizeof(float); };
    float s[RPL][C];
    auto load_tile = [&]() {
#pragma unroll
        for (int r = 0; r < RPL; ++r)
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const V x = load_tile_vec<V>(srs, tile_off(r, c));
#pragma unroll
                for (int e = 0; e < VEC; ++e) s[r][c * VEC + e] = x[e];
            }
    };

    // ---- input stage: thread tid < 3D/4 owns four channels
    const float *ring = f.ring + (int64_t)b * f.ring_stride;
    float *rout = ring_out + (int64_t)b * f.ring_stride;
    const bool mine = tid < 3 * D / 4;
    const int j = 4 * tid;
    const int64_t c = j < D ? (int64_t)g * D + j
                    : j < 2 * D ? (int64_t)(a.nk + g) * D + (j - D)
                                : (int64_t)(2 * a.nk + h) * D + (j - 2 * D);
    const bool writes = j >= 2 * D || h < a.nk;    // the new ring rows this workgroup stores
    auto conv = [&](auto maxt, bool prefetch) {
        constexpr int MAXT = decltype(maxt)::value;
        float4 xv, hist[MAXT - 1], w[MAXT];
        if (mine) {
            xv = *reinterpret_cast<const float4 *>(f.x + (int64_t)b * f.x_stride + c);
#pragma unroll
            for (int t = 0; t < MAXT - 1; ++t)
                if (t < taps - 1) hist[t] = *reinterpret_cast<const float4 *>(ring + (t + 1) * CH + c);
#pragma unroll
            for (int t = 0; t < MAXT; ++t)
                if (t < taps) w[t] = *reinterpret_cast<const float4 *>(f.w + t * CH + c);
        }
        if (prefetch && active) load_tile();
        if (mine) {
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int t = 0; t < MAXT; ++t)
                if (t < taps) {
                    const float4 hv = t < taps - 1 ? hist[t < MAXT - 1 ? t : 0] : xv;
                    acc.x = fmaf(hv.x, w[t].x, acc.x);
                    acc.y = fmaf(hv.y, w[t].y, acc.y);
                    acc.z = fmaf(hv.z, w[t].z, acc.z);
                    acc.w = fmaf(hv.w, w[t].w, acc.w);
                }
            if (writes) {
#pragma unroll
                for (int t = 0; t < MAXT - 1; ++t)
                    if (t < taps - 1) *reinterpret_cast<float4 *>(rout + t * CH + c) = hist[t];
                *reinterpret_cast<float4 *>(rout + (int64_t)(taps - 1) * CH + c) = xv;
            }
            feat[j + 0] = silu(acc.x);
            feat[j + 1] = silu(acc.y);
            feat[j + 2] = silu(acc.z);
            feat[j + 3] = silu(acc.w);
        }
    };
    if (taps <= kShort) {
        conv(std::integral_constant<int, kShort>{}, true);
    } else {
        conv(std::integral_constant<int, kMaxTaps>{}, false);
        if (active) load_tile();
    }
    if (tid == 0) {
        const int64_t e = (int64_t)b * f.g_stride + h;
        gates[0] = powf(1.0f + expf(f.ar[e] + f.dt[h]), f.rate[h]);
        gates[1] = 1.0f / (1.0f + expf(-f.br[e]));
    }
    __syncthreads();
    if (tid < 64) {   // L2 of q_g and k_g: x / sqrt(sum x^2 + eps)
        float sq = 0.f, sk = 0.f;
        for (int i = tid; i < D; i += 64) {
            sq = fmaf(feat[i], feat[i], sq);
            sk = fmaf(feat[D + i], feat[D + i], sk);
        }
        sq = group_sum_wide<64>(sq);
        sk = group_sum_wide<64>(sk);
        if (tid == 0) {
            den[0] = sqrtf(sq + f.l2_eps);
            den[1] = sqrtf(sk + f.l2_eps);
        }
    }
    __syncthreads();

    // ---- the step on this value head's tile
    float o_mine = 0.f, sumsq = 0.f, zr = 0.f, gr = 0.f;
    if (active) {
        const float dq = den[0], dk = den[1];
        float kk[C], qq[C];
#pragma unroll
        for (int cc = 0; cc < NCH; ++cc)
#pragma unroll
            for (int e4 = 0; e4 < VEC; e4 += 4) {
                const int col = (cc * LPR + p) * VEC + e4;
                const float4 q4 = *reinterpret_cast<const float4 *>(feat + col);
                const float4 k4 = *reinterpret_cast<const float4 *>(feat + D + col);
                kk[cc * VEC + e4 + 0] = k4.x / dk; kk[cc * VEC + e4 + 1] = k4.y / dk;
                kk[cc * VEC + e4 + 2] = k4.z / dk; kk[cc * VEC + e4 + 3] = k4.w / dk;
                qq[cc * VEC + e4 + 0] = q4.x / dq; qq[cc * VEC + e4 + 1] = q4.y / dq;
                qq[cc * VEC + e4 + 2] = q4.z / dq; qq[cc * VEC + e4 + 3] = q4.w / dq;
            }
        if constexpr (NORM) {
            if (p < RPL) {
                zr = a.z[(int64_t)b * a.z_stride + (int64_t)h * D + row0 + p];
                gr = a.gn[row0 + p];
            }
        }
        float kq = 0.f;
#pragma unroll
        for (int i = 0; i < C; ++i) kq = fmaf(kk[i], qq[i], kq);
        kq = group_sum<LPR>(kq);
        const float alpha = gates[0], beta = gates[1];
        const float *vh = feat + 2 * D;
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            float pu = 0.f, pw = 0.f;
#pragma unroll
            for (int i = 0; i < C; ++i) {
                pu = fmaf(s[r][i], kk[i], pu);
                pw = fmaf(s[r][i], qq[i], pw);
            }
            const float u = group_sum<LPR>(pu);
            const float w = group_sum<LPR>(pw);
            const float coef = beta * (vh[row0 + r] - alpha * u);
            const float o = (alpha * w + coef * kq) * a.scale;
            sumsq = fmaf(o, o, sumsq);
            if (r == p) o_mine = o;
            V x;
#pragma unroll
            for (int cc = 0; cc < NCH; ++cc) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) x[e] = alpha * s[r][cc * VEC + e] + coef * kk[cc * VEC + e];
                store_tile_vec<V>(srs, tile_off(r, cc), x);
            }
        }
    }
    float *outp = static_cast<float *>(a.out);
    const int64_t orow = (int64_t)b * a.out_stride + (int64_t)h * D + row0 + p;
    if constexpr (!NORM) {
        if (active && p < RPL) outp[orow] = o_mine;
    } else {
        const float wsum = wave_groups_sum<LPR>(active ? sumsq : 0.f);
        if ((tid & 63) == 0) part[tid >> 6] = wsum;
        __syncthreads();
        if (active && p < RPL) {
            float tot = 0.f;
#pragma unroll
            for (int i = 0; i < TL::NT / 64; ++i) tot += part[i];
            const float r = sqrtf(tot * (1.0f / D) + a.eps);
            outp[orow] = (gr * o_mine / r) * silu(zr);
        }
    }
}

template <int D, bool NORM>
static hipError_t go_fused(const StepArgs &a, const FrontArgs &f, float *ring_out, hipStream_t stream) {
    if (ring_out) {
        const unsigned grid = (unsigned)((int64_t)a.batch * a.nv);
        return launch(fused_split_kernel<D, NORM>, dim3(grid), dim3(DecodeTile<D, float>::NT), 0,
                      stream, a, f, ring_out);
    }
    const unsigned grid = (unsigned)((int64_t)a.batch * a.nk);
    const size_t lds = fused_lds_bytes(D, a.nv / a.nk);
    return launch(fused_kernel<D, NORM>, dim3(grid), dim3(DecodeTile<D, float>::NT), lds, stream, a, f);
}

template <bool NORM>
static hipError_t fused_by_dim(const StepArgs &a, const FrontArgs &f, float *ro, int dim, hipStream_t st) {
    switch (dim) {
        case 4: return go_fused<4, NORM>(a, f, ro, st);
        case 8: return go_fused<8, NORM>(a, f, ro, st);
        case 16: return go_fused<16, NORM>(a, f, ro, st);
        case 32: return go_fused<32, NORM>(a, f, ro, st);
        case 64: return go_fused<64, NORM>(a, f, ro, st);
        case 128: return go_fused<128, NORM>(a, f, ro, st);
        case 256: return go_fused<256, NORM>(a, f, ro, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fused(const StepArgs &a, const FrontArgs &f, float *ring_out, int dim, bool norm,
                        hipStream_t stream) {
    return norm ? fused_by_dim<true>(a, f, ring_out, dim, stream)
                : fused_by_dim<false>(a, f, ring_out, dim, stream);
}

}  // namespace gdn
