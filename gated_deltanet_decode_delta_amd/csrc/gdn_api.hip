// gdn_api.hip -- the extern "C" entry points of libgdn.so (contract: gdn.h).
//
// Every call validates its arguments on the host first -- shapes, strides,
// alignment and address-range overlap -- and returns before any HIP call if
// one is wrong, so a rejected call leaves every buffer untouched.  Only then is
// the kernel launched on the caller's stream.  No allocation, no
// synchronisation, no printing.
#include <algorithm>
#include <math.h>
#include <mutex>
#include <stdint.h>

#include "../../include/gdn.h"
#include "gdn_launch.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

struct Span {
    __int128 lo = 0, hi = 0;  // byte range [lo, hi); empty when lo == hi
};

constexpr __int128 kMaxBytes = (__int128)1 << 62;

// Bytes touched by `rows` rows of `width` elements, `stride` elements apart.
bool make_span(const void *p, int64_t rows, int64_t stride, int64_t width, int64_t elem, Span *out) {
    if (rows <= 0 || width <= 0) { *out = Span{}; return true; }
    const __int128 n = (__int128)(rows - 1) * stride + width;
    const __int128 bytes = n * elem;
    if (bytes > kMaxBytes) return false;
    out->lo = (__int128)(uintptr_t)p;
    out->hi = out->lo + bytes;
    return true;
}

bool overlap(const Span &a, const Span &b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void *p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

bool supported_dim(int32_t d) {
    return d == 4 || d == 8 || d == 16 || d == 32 || d == 64 || d == 128 || d == 256;
}

struct Call {
    const void *state;
    int64_t pitch;
    int state_elem;     // 4 or 2 bytes
    const float *q, *k;
    int64_t qk_stride;
    const float *v;
    int64_t v_stride;
    const float *alpha, *beta;
    int64_t ab_stride;
    const float *z;     // may be NULL when the raw output is asked for
    int64_t z_stride;
    const float *gn;
    float eps;
    bool norm;
    const void *out;
    int out_elem;
    int64_t out_stride;
    int32_t batch, seq_len, nk, nv, dk, dv;
    bool out_optional = false;  // out may be NULL (then it is neither checked nor written)
};

// Byte ranges of every array of a validated call.
struct Spans {
    Span st, q, k, v, al, be, z, gn, out;
};

gdn_status validate(const Call &c, bool *empty, Spans *spans_out = nullptr) {
    *empty = false;
    if (c.batch < 0 || c.seq_len < 0) return GDN_ERR_SHAPE;
    if (c.nk <= 0 || c.nv <= 0 || c.nv % c.nk != 0) return GDN_ERR_SHAPE;
    if (c.dk <= 0 || c.dv <= 0) return GDN_ERR_SHAPE;
    if (c.dk != c.dv || !supported_dim(c.dk)) return GDN_ERR_UNSUPPORTED;
    if ((int64_t)c.batch * c.nv > INT32_MAX) return GDN_ERR_SHAPE;
    if (c.norm && (!isfinite(c.eps) || c.eps < 0.0f)) return GDN_ERR_ARG;
    if (c.batch == 0 || c.seq_len == 0) { *empty = true; return GDN_OK; }

    if (!c.state || !c.q || !c.k || !c.v || !c.alpha || !c.beta) return GDN_ERR_NULL;
    if (!c.out && !c.out_optional) return GDN_ERR_NULL;
    const bool has_out = c.out != nullptr;
    if (c.norm && (!c.z || !c.gn)) return GDN_ERR_NULL;

    const int64_t D = c.dk;
    const int64_t rows = (int64_t)c.batch * c.seq_len;
    const int64_t slot = (int64_t)c.nv * D * D;
    const int64_t vw = (int64_t)c.nv * D;
    const int64_t qkw = (int64_t)c.nk * D;
    // strides: large enough for their row (only meaningful with more than one row)
    if (c.batch > 1 && c.pitch < slot) return GDN_ERR_STRIDE;
    if (rows > 1 && (c.qk_stride < qkw || c.v_stride < vw || c.ab_stride < c.nv ||
                     (has_out && c.out_stride < vw) || (c.norm && c.z_stride < vw)))
        return GDN_ERR_STRIDE;
    // alignment of the vector-accessed arrays
    const int64_t state_vec = 16 / c.state_elem;
    if (!aligned(c.state, 16) || (c.batch > 1 && c.pitch % state_vec != 0)) return GDN_ERR_STRIDE;
    if (!aligned(c.q, 16) || !aligned(c.k, 16) || !aligned(c.v, 16) || !aligned(c.out, 16))
        return GDN_ERR_STRIDE;
    if (rows > 1 && (c.qk_stride % 4 || c.v_stride % 4 || (has_out && c.out_stride % 4)))
        return GDN_ERR_STRIDE;
    if (c.norm && (!aligned(c.z, 16) || (rows > 1 && c.z_stride % 4))) return GDN_ERR_STRIDE;
    if (!aligned(c.alpha, 4) || !aligned(c.beta, 4) || (c.norm && !aligned(c.gn, 4)))
        return GDN_ERR_STRIDE;

    // address ranges
    Spans sp;
    Span &st = sp.st, &q = sp.q, &k = sp.k, &v = sp.v, &al = sp.al, &be = sp.be, &z = sp.z,
         &gn = sp.gn, &out = sp.out;
    bool ok = make_span(c.state, c.batch, c.pitch, slot, c.state_elem, &st) &&
              make_span(c.q, rows, c.qk_stride, qkw, 4, &q) &&
              make_span(c.k, rows, c.qk_stride, qkw, 4, &k) &&
              make_span(c.v, rows, c.v_stride, vw, 4, &v) &&
              make_span(c.alpha, rows, c.ab_stride, c.nv, 4, &al) &&
              make_span(c.beta, rows, c.ab_stride, c.nv, 4, &be) &&
              make_span(c.out, has_out ? rows : 0, c.out_stride, vw, c.out_elem, &out);
    if (c.norm) ok = ok && make_span(c.z, rows, c.z_stride, vw, 4, &z) && make_span(c.gn, 1, D, D, 4, &gn);
    if (!ok) return GDN_ERR_STRIDE;
    const Span *inputs[] = {&q, &k, &v, &al, &be, &z, &gn};
    for (const Span *in : inputs)
        if (overlap(st, *in) || overlap(out, *in)) return GDN_ERR_ALIAS;
    if (overlap(st, out)) return GDN_ERR_ALIAS;
    if (spans_out) *spans_out = sp;
    return GDN_OK;
}

// A further output array of a validated call: `rows` rows of `width` elements,
// `stride` apart; non-NULL, rows wide enough, base aligned to `align` bytes, and
// overlapping no other array of the call.
gdn_status check_extra_out(const Spans &sp, const void *p, int64_t rows, int64_t stride,
                           int64_t width, int64_t elem, uintptr_t align, Span *span) {
    if (!p) return GDN_ERR_NULL;
    if (rows > 1 && stride < width) return GDN_ERR_STRIDE;
    if (!aligned(p, align)) return GDN_ERR_STRIDE;
    if (!make_span(p, rows, stride, width, elem, span)) return GDN_ERR_STRIDE;
    const Span *all[] = {&sp.st, &sp.q, &sp.k, &sp.v, &sp.al, &sp.be, &sp.z, &sp.gn, &sp.out};
    for (const Span *x : all)
        if (overlap(*span, *x)) return GDN_ERR_ALIAS;
    return GDN_OK;
}

// A call with a single row never steps to a second one, so validate() leaves
// its strides unchecked; the kernels still size buffer ranges from them.  Here
// each such stride is raised to at least its row width (row 0 is unchanged),
// so every kernel sees strides that hold their rows.
int64_t row_stride(const Call &c, int64_t stride, int64_t width) {
    const bool single = (int64_t)c.batch * c.seq_len <= 1;
    return single && stride < width ? width : stride;
}

gdn::StepArgs to_args(const Call &c, void *state, void *out) {
    const int64_t vw = (int64_t)c.nv * c.dv;
    gdn::StepArgs a;
    a.state = state;
    a.pitch = c.batch <= 1 && c.pitch < (int64_t)c.nv * c.dk * c.dv ? (int64_t)c.nv * c.dk * c.dv
                                                                    : c.pitch;
    a.q = c.q;
    a.k = c.k;
    a.qk_stride = row_stride(c, c.qk_stride, (int64_t)c.nk * c.dk);
    a.v = c.v;
    a.v_stride = row_stride(c, c.v_stride, vw);
    a.alpha = c.alpha;
    a.beta = c.beta;
    a.ab_stride = row_stride(c, c.ab_stride, c.nv);
    a.z = c.z;
    a.z_stride = row_stride(c, c.z_stride, vw);
    a.gn = c.gn;
    a.eps = c.eps;
    a.scale = (float)(1.0 / sqrt((double)c.dk));
    a.out = out;
    a.out_stride = row_stride(c, c.out_stride, vw);
    a.codes = nullptr;
    a.codes_stride = 0;
    a.scales = nullptr;
    a.scales_stride = 0;
    a.batch = c.batch;
    a.seq_len = c.seq_len;
    a.nk = c.nk;
    a.nv = c.nv;
    return a;
}

gdn_status finish(hipError_t e) {
    if (e == hipSuccess) return GDN_OK;
    g_last_hip_error = (int32_t)e;
    return GDN_ERR_HIP;
}

}  // namespace

extern "C" {

gdn_status gdn_decode(float *state, int64_t state_seq_stride, const float *q, const float *k,
                      int64_t qk_stride, const float *v, int64_t v_stride, const float *alpha,
                      const float *beta, int64_t ab_stride, float *out, int64_t out_stride,
                      int32_t batch, int32_t num_k_heads, int32_t num_v_heads, int32_t k_dim,
                      int32_t v_dim, void *stream) {
    Call c{state, state_seq_stride, 4, q, k, qk_stride, v, v_stride, alpha, beta, ab_stride,
           nullptr, 0, nullptr, 0.0f, false, out, 4, out_stride,
           batch, 1, num_k_heads, num_v_heads, k_dim, v_dim};
    bool empty;
    gdn_status s = validate(c, &empty);
    if (s != GDN_OK || empty) return s;
    return finish(gdn::launch_decode(to_args(c, state, out), k_dim, false, gdn::kOutRawF32,
                                     (hipStream_t)stream));
}

gdn_status gdn_decode_norm(float *state, int64_t state_seq_stride, const float *q, const float *k,
                           int64_t qk_stride, const float *v, int64_t v_stride, const float *alpha,
                           const float *beta, int64_t ab_stride, const float *z, int64_t z_stride,
                           const float *norm_weight, float eps, void *out, int32_t out_dtype,
                           int64_t out_stride, int32_t batch, int32_t num_k_heads,
                           int32_t num_v_heads, int32_t k_dim, int32_t v_dim, void *stream) {
    if (out_dtype != GDN_F32 && out_dtype != GDN_BF16) return GDN_ERR_DTYPE;
    Call c{state, state_seq_stride, 4, q, k, qk_stride, v, v_stride, alpha, beta, ab_stride,
           z, z_stride, norm_weight, eps, true, out, out_dtype == GDN_F32 ? 4 : 2, out_stride,
           batch, 1, num_k_heads, num_v_heads, k_dim, v_dim};
    bool empty;
    gdn_status s = validate(c, &empty);
    if (s != GDN_OK || empty) return s;
    return finish(gdn::launch_decode(to_args(c, state, out), k_dim, false,
                                     out_dtype == GDN_F32 ? gdn::kOutNormF32 : gdn::kOutNormBF16,
                                     (hipStream_t)stream));
}

gdn_status gdn_decode_norm_q(float *state, int64_t state_seq_stride, const float *q,
                             const float *k, int64_t qk_stride, const float *v, int64_t v_stride,
                             const float *alpha, const float *beta, int64_t ab_stride,
                             const float *z, int64_t z_stride, const float *norm_weight, float eps,
                             float *out, int64_t out_stride, int8_t *codes, int64_t codes_stride,
                             float *scales, int64_t scales_stride, int32_t batch,
                             int32_t num_k_heads, int32_t num_v_heads, int32_t k_dim,
                             int32_t v_dim, void *stream) {
    Call c{state, state_seq_stride, 4, q, k, qk_stride, v, v_stride, alpha, beta, ab_stride,
           z, z_stride, norm_weight, eps, true, out, 4, out_stride,
           batch, 1, num_k_heads, num_v_heads, k_dim, v_dim};
    c.out_optional = true;
    bool empty;
    Spans sp;
    gdn_status s = validate(c, &empty, &sp);
    if (s != GDN_OK) return s;
    if (v_dim % 32 != 0) return GDN_ERR_UNSUPPORTED;
    if (empty) return GDN_OK;
    const int64_t vw = (int64_t)num_v_heads * v_dim;
    Span cs, ss;
    s = check_extra_out(sp, codes, batch, codes_stride, vw, 1, 1, &cs);
    if (s != GDN_OK) return s;
    s = check_extra_out(sp, scales, batch, scales_stride, vw / 32, 4, 4, &ss);
    if (s != GDN_OK) return s;
    if (overlap(cs, ss)) return GDN_ERR_ALIAS;
    gdn::StepArgs a = to_args(c, state, out);
    a.codes = codes;
    a.codes_stride = codes_stride;
    a.scales = scales;
    a.scales_stride = scales_stride;
    return finish(gdn::launch_decode(a, k_dim, false, gdn::kOutNormQ8, (hipStream_t)stream));
}

gdn_status gdn_decode_f16state(uint16_t *state, int64_t state_seq_stride, const float *q,
                               const float *k, int64_t qk_stride, const float *v, int64_t v_stride,
                               const float *alpha, const float *beta, int64_t ab_stride,
                               const float *z, int64_t z_stride, const float *norm_weight,
                               float eps, void *out, int32_t out_dtype, int64_t out_stride,
                               int32_t batch, int32_t num_k_heads, int32_t num_v_heads,
                               int32_t k_dim, int32_t v_dim, void *stream) {
    const bool norm = z != nullptr;
    if (out_dtype != GDN_F32 && out_dtype != GDN_BF16) return GDN_ERR_DTYPE;
    if (!norm && out_dtype != GDN_F32) return GDN_ERR_DTYPE;
    Call c{state, state_seq_stride, 2, q, k, qk_stride, v, v_stride, alpha, beta, ab_stride,
           z, z_stride, norm_weight, eps, norm, out, out_dtype == GDN_F32 ? 4 : 2, out_stride,
           batch, 1, num_k_heads, num_v_heads, k_dim, v_dim};
    bool empty;
    gdn_status s = validate(c, &empty);
    if (s != GDN_OK || empty) return s;
    const gdn::OutMode mode = !norm ? gdn::kOutRawF32
                                    : (out_dtype == GDN_F32 ? gdn::kOutNormF32 : gdn::kOutNormBF16);
    return finish(gdn::launch_decode(to_args(c, state, out), k_dim, true, mode, (hipStream_t)stream));
}

gdn_status gdn_recurrence_seq(float *state, int64_t state_seq_stride, const float *q,
                              const float *k, int64_t qk_stride, const float *v, int64_t v_stride,
                              const float *alpha, const float *beta, int64_t ab_stride,
                              const float *z, int64_t z_stride, const float *norm_weight,
                              float eps, float *out, int64_t out_stride, int32_t batch,
                              int32_t seq_len, int32_t num_k_heads, int32_t num_v_heads,
                              int32_t k_dim, int32_t v_dim, void *stream) {
    const bool norm = z != nullptr;
    Call c{state, state_seq_stride, 4, q, k, qk_stride, v, v_stride, alpha, beta, ab_stride,
           z, z_stride, norm_weight, eps, norm, out, 4, out_stride,
           batch, seq_len, num_k_heads, num_v_heads, k_dim, v_dim};
    bool empty;
    gdn_status s = validate(c, &empty);
    if (s != GDN_OK || empty) return s;
    return finish(gdn::launch_seq(to_args(c, state, out), k_dim,
                                  norm ? gdn::kOutNormF32 : gdn::kOutRawF32, (hipStream_t)stream));
}

int64_t gdn_seq_workspace_bytes(int32_t batch, int32_t seq_len, int32_t num_v_heads,
                                int32_t k_dim, int32_t v_dim) {
    if (batch < 0 || seq_len < 0 || num_v_heads < 0) return -1;
    if (k_dim != 128 || v_dim != 128) return 0;
    const __int128 chunks = ((__int128)seq_len + 15) / 16;
    const __int128 bytes = (__int128)batch * num_v_heads * chunks * gdn::kSeqRec * 4;
    if (bytes > kMaxBytes) return -1;
    return (int64_t)bytes;
}

}  // extern "C"

namespace {

// Whether a validated sequence call takes the workspace path (D = 128, split
// state pass).  That path launches one pre-pass workgroup per (sequence, key
// head, chunk), four state-pass workgroups per value head and one norm
// workgroup per 16 (row, head) pairs, and the state pass reads q, k, v and
// writes o through buffer descriptors with 32-bit offsets.  Those offsets reach
// the last row of a whole 16-token chunk, padding rows past the end included,
// so they must fit 32 bits over max(T, 16) rows.  A shape whose grids would not
// fit 32 bits, whose rows of one sequence (at least 16 of them) span 2^31 bytes
// or more in q, k, v or o, or another head dim, runs the kernels without a
// workspace.
bool seq_split_path(const gdn::StepArgs &a, int32_t k_dim) {
    const int64_t widest = std::max(a.qk_stride, std::max(a.v_stride, a.out_stride));
    return !(k_dim != 128 || (int64_t)a.batch * a.nk * ((a.seq_len + 15) / 16) > INT32_MAX ||
             (int64_t)a.batch * a.nv * 4 > INT32_MAX ||
             ((int64_t)a.batch * a.seq_len * a.nv + 15) / 16 > INT32_MAX ||
             (int64_t)std::max(a.seq_len, 16) * widest * 4 + 1024 > INT32_MAX);
}

}  // namespace

// Scratch memory of gdn_recurrence_seq_noalloc: the workspace records of the
// split sequence path in the library's own device memory, so that the call
// allocates nothing.  Each GPU the library runs on holds its own copy, loaded
// with the code object and kept until the process ends.  Host code never uses
// this name as an address: the device address comes from hipGetSymbolAddress,
// once per device (scratch_address below).
static __device__ __align__(256) float scratch[GDN_SEQ_NOALLOC_MAX_BYTES / 4];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, resolved on the
// first call there (with that device current) and kept per device.
hipError_t scratch_address(float **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<float *>(g_scratch_ptr[dev]);
    return hipSuccess;
}

}  // namespace

extern "C" {

gdn_status gdn_recurrence_seq_ws(float *state, int64_t state_seq_stride, const float *q,
                                 const float *k, int64_t qk_stride, const float *v,
                                 int64_t v_stride, const float *alpha, const float *beta,
                                 int64_t ab_stride, const float *z, int64_t z_stride,
                                 const float *norm_weight, float eps, float *out,
                                 int64_t out_stride, int32_t batch, int32_t seq_len,
                                 int32_t num_k_heads, int32_t num_v_heads, int32_t k_dim,
                                 int32_t v_dim, void *workspace, int64_t workspace_bytes,
                                 void *stream) {
    const bool norm = z != nullptr;
    Call c{state, state_seq_stride, 4, q, k, qk_stride, v, v_stride, alpha, beta, ab_stride,
           z, z_stride, norm_weight, eps, norm, out, 4, out_stride,
           batch, seq_len, num_k_heads, num_v_heads, k_dim, v_dim};
    bool empty;
    Spans sp;
    gdn_status s = validate(c, &empty, &sp);
    if (s != GDN_OK || empty) return s;
    gdn::StepArgs a = to_args(c, state, out);
    if (!seq_split_path(a, k_dim))
        return finish(gdn::launch_seq(a, k_dim, norm ? gdn::kOutNormF32 : gdn::kOutRawF32,
                                      (hipStream_t)stream));
    const int64_t need = gdn_seq_workspace_bytes(batch, seq_len, num_v_heads, k_dim, v_dim);
    if (need < 0) return GDN_ERR_SHAPE;
    if (!workspace) return GDN_ERR_NULL;
    if (workspace_bytes < need) return GDN_ERR_ARG;
    Span ws;
    s = check_extra_out(sp, workspace, 1, need / 4, need / 4, 4, 16, &ws);
    if (s != GDN_OK) return s;
    return finish(gdn::launch_seq_split(a, static_cast<float *>(workspace), (hipStream_t)stream));
}

gdn_status gdn_recurrence_seq_noalloc(float *state, int64_t state_seq_stride, const float *q,
                                      const float *k, int64_t qk_stride, const float *v,
                                      int64_t v_stride, const float *alpha, const float *beta,
                                      int64_t ab_stride, const float *z, int64_t z_stride,
                                      const float *norm_weight, float eps, float *out,
                                      int64_t out_stride, int32_t batch, int32_t seq_len,
                                      int32_t num_k_heads, int32_t num_v_heads, int32_t k_dim,
                                      int32_t v_dim, void *stream) {
    const bool norm = z != nullptr;
    Call c{state, state_seq_stride, 4, q, k, qk_stride, v, v_stride, alpha, beta, ab_stride,
           z, z_stride, norm_weight, eps, norm, out, 4, out_stride,
           batch, seq_len, num_k_heads, num_v_heads, k_dim, v_dim};
    bool empty;
    gdn_status s = validate(c, &empty);
    if (s != GDN_OK || empty) return s;
    gdn::StepArgs a = to_args(c, state, out);
    if (!seq_split_path(a, k_dim))
        return finish(gdn::launch_seq(a, k_dim, norm ? gdn::kOutNormF32 : gdn::kOutRawF32,
                                      (hipStream_t)stream));
    const int64_t need = gdn_seq_workspace_bytes(batch, seq_len, num_v_heads, k_dim, v_dim);
    if (need < 0) return GDN_ERR_SHAPE;
    if (need > (int64_t)GDN_SEQ_NOALLOC_MAX_BYTES) return GDN_ERR_SCRATCH;
    // the scratch address is the current device's: a stream of another device
    // would run the kernels there with this device's address
    if (stream != nullptr) {
        int cur = 0;
        hipDevice_t sdev = 0;
        if (hipGetDevice(&cur) == hipSuccess && hipStreamGetDevice((hipStream_t)stream, &sdev) == hipSuccess &&
            sdev != cur)
            return GDN_ERR_ARG;
    }
    // every record the state pass reads is written by the pre-pass of the same
    // call first, so nothing in the scratch has to start at zero
    float *ws = nullptr;
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return finish(e);
    return finish(gdn::launch_seq_split(a, ws, (hipStream_t)stream));
}

gdn_status gdn_decode_verify(float *state, int64_t state_seq_stride, float *inter_state,
                             int64_t inter_pitch, const float *q, const float *k, int64_t qk_stride,
                             const float *v, int64_t v_stride, const float *alpha, const float *beta,
                             int64_t ab_stride, const float *z, int64_t z_stride,
                             const float *norm_weight, float eps, float *out, int64_t out_stride,
                             int32_t batch, int32_t num_tokens, int32_t num_k_heads,
                             int32_t num_v_heads, int32_t k_dim, int32_t v_dim, void *stream) {
    const bool norm = z != nullptr;
    if (num_tokens < 1 || num_tokens > GDN_VERIFY_MAX_TOKENS) return GDN_ERR_SHAPE;
    Call c{state, state_seq_stride, 4, q, k, qk_stride, v, v_stride, alpha, beta, ab_stride,
           z, z_stride, norm_weight, eps, norm, out, 4, out_stride,
           batch, num_tokens, num_k_heads, num_v_heads, k_dim, v_dim};
    bool empty;
    Spans sp;
    gdn_status s = validate(c, &empty, &sp);
    if (s != GDN_OK || empty) return s;
    if (num_tokens > 1) {
        const int64_t slot = (int64_t)num_v_heads * k_dim * v_dim;
        const int64_t slots = (int64_t)batch * (num_tokens - 1);
        Span in;
        s = check_extra_out(sp, inter_state, slots, inter_pitch, slot, 4, 16, &in);
        if (s != GDN_OK) return s;
        if (slots > 1 && inter_pitch % 4 != 0) return GDN_ERR_STRIDE;
    }
    return finish(gdn::launch_verify(to_args(c, state, out), k_dim, inter_state, inter_pitch, norm,
                                     (hipStream_t)stream));
}

gdn_status gdn_decode_fused(float *state, int64_t state_seq_stride, float *conv_state,
                            int64_t conv_seq_stride, float *conv_state_out, const float *x,
                            int64_t x_stride,
                            const float *conv_weight, int32_t taps, const float *br,
                            const float *ar, int64_t gate_stride, const float *dt_bias,
                            const float *decay_rate, float l2_eps, const float *z,
                            int64_t z_stride, const float *norm_weight, float eps, float *out,
                            int64_t out_stride, int32_t batch, int32_t num_k_heads,
                            int32_t num_v_heads, int32_t k_dim, int32_t v_dim, void *stream) {
    const bool norm = z != nullptr;
    if (batch < 0 || num_k_heads <= 0 || num_v_heads <= 0 || num_v_heads % num_k_heads != 0 ||
        k_dim <= 0 || v_dim <= 0 || taps < 1 || taps > gdn::kMaxTaps)
        return GDN_ERR_SHAPE;
    if (k_dim != v_dim || !supported_dim(k_dim)) return GDN_ERR_UNSUPPORTED;
    // the two-buffer launch has batch * num_v_heads workgroups (the larger grid)
    if ((int64_t)batch * num_v_heads > INT32_MAX) return GDN_ERR_SHAPE;
    if (!isfinite(l2_eps) || l2_eps < 0.0f) return GDN_ERR_ARG;
    if (norm && (!isfinite(eps) || eps < 0.0f)) return GDN_ERR_ARG;
    const int32_t D = k_dim;
    const bool in_place = conv_state_out == nullptr;
    if (in_place && gdn::fused_lds_bytes(D, num_v_heads / num_k_heads) > 64 * 1024)
        return GDN_ERR_UNSUPPORTED;
    if (batch == 0) return GDN_OK;

    if (!state || !conv_state || !x || !conv_weight || !br || !ar || !dt_bias || !decay_rate || !out)
        return GDN_ERR_NULL;
    if (norm && !norm_weight) return GDN_ERR_NULL;
    const int64_t slot = (int64_t)num_v_heads * D * D;
    const int64_t ch = (int64_t)(2 * num_k_heads + num_v_heads) * D;
    const int64_t ring = taps * ch;
    const int64_t vw = (int64_t)num_v_heads * D;
    const bool many = batch > 1;
    if (many && (state_seq_stride < slot || conv_seq_stride < ring || x_stride < ch ||
                 gate_stride < num_v_heads || out_stride < vw || (norm && z_stride < vw)))
        return GDN_ERR_STRIDE;
    if (!aligned(state, 16) || !aligned(conv_state, 16) || !aligned(conv_state_out, 16) ||
        !aligned(x, 16) ||
        !aligned(conv_weight, 16) || !aligned(out, 16) || (norm && !aligned(z, 16)))
        return GDN_ERR_STRIDE;
    if (many && (state_seq_stride % 4 || conv_seq_stride % 4 || x_stride % 4 || out_stride % 4 ||
                 (norm && z_stride % 4)))
        return GDN_ERR_STRIDE;
    if (!aligned(br, 4) || !aligned(ar, 4) || !aligned(dt_bias, 4) || !aligned(decay_rate, 4) ||
        (norm && !aligned(norm_weight, 4)))
        return GDN_ERR_STRIDE;

    Span st, rg, ro, xs, w, b_, a_, dt, rt, z_, gn, o;
    bool ok = make_span(state, batch, state_seq_stride, slot, 4, &st) &&
              make_span(conv_state_out, in_place ? 0 : batch, conv_seq_stride, ring, 4, &ro) &&
              make_span(conv_state, batch, conv_seq_stride, ring, 4, &rg) &&
              make_span(x, batch, x_stride, ch, 4, &xs) &&
              make_span(conv_weight, 1, ring, ring, 4, &w) &&
              make_span(br, batch, gate_stride, num_v_heads, 4, &b_) &&
              make_span(ar, batch, gate_stride, num_v_heads, 4, &a_) &&
              make_span(dt_bias, 1, num_v_heads, num_v_heads, 4, &dt) &&
              make_span(decay_rate, 1, num_v_heads, num_v_heads, 4, &rt) &&
              make_span(out, batch, out_stride, vw, 4, &o);
    if (norm) ok = ok && make_span(z, batch, z_stride, vw, 4, &z_) && make_span(norm_weight, 1, D, D, 4, &gn);
    if (!ok) return GDN_ERR_STRIDE;
    const Span *written[] = {&st, &rg, &ro, &o};   // rg is only read when ro is given
    const Span *all[] = {&st, &rg, &ro, &o, &xs, &w, &b_, &a_, &dt, &rt, &z_, &gn};
    for (const Span *wr : written)
        for (const Span *x2 : all)
            if (wr != x2 && overlap(*wr, *x2)) return GDN_ERR_ALIAS;

    gdn::StepArgs a{};
    a.state = state;
    a.pitch = state_seq_stride;
    a.z = z;
    a.z_stride = z_stride;
    a.gn = norm_weight;
    a.eps = eps;
    a.scale = (float)(1.0 / sqrt((double)D));
    a.out = out;
    a.out_stride = out_stride;
    a.batch = batch;
    a.seq_len = 1;
    a.nk = num_k_heads;
    a.nv = num_v_heads;
    gdn::FrontArgs f;
    f.ring = conv_state;
    f.ring_stride = conv_seq_stride;
    f.x = x;
    f.x_stride = x_stride;
    f.w = conv_weight;
    f.taps = taps;
    f.br = br;
    f.ar = ar;
    f.g_stride = gate_stride;
    f.dt = dt_bias;
    f.rate = decay_rate;
    f.l2_eps = l2_eps;
    return finish(gdn::launch_fused(a, f, conv_state_out, D, norm, (hipStream_t)stream));
}

static gdn_status check_convert(const void *src, const void *dst, int64_t n, int src_elem,
                                 int dst_elem, bool *empty) {
    *empty = false;
    if (n < 0) return GDN_ERR_SHAPE;
    if (n == 0) { *empty = true; return GDN_OK; }
    if (!src || !dst) return GDN_ERR_NULL;
    if (!aligned(src, 16) || !aligned(dst, 16)) return GDN_ERR_STRIDE;
    Span a, b;
    if (!make_span(src, 1, n, n, src_elem, &a) || !make_span(dst, 1, n, n, dst_elem, &b))
        return GDN_ERR_STRIDE;
    if (overlap(a, b)) return GDN_ERR_ALIAS;
    return GDN_OK;
}

gdn_status gdn_state_f32_to_f16(const float *src, uint16_t *dst, int64_t n, void *stream) {
    bool empty;
    gdn_status s = check_convert(src, dst, n, 4, 2, &empty);
    if (s != GDN_OK || empty) return s;
    return finish(gdn::launch_f32_to_f16(src, dst, n, (hipStream_t)stream));
}

gdn_status gdn_state_f16_to_f32(const uint16_t *src, float *dst, int64_t n, void *stream) {
    bool empty;
    gdn_status s = check_convert(src, dst, n, 2, 4, &empty);
    if (s != GDN_OK || empty) return s;
    return finish(gdn::launch_f16_to_f32(src, dst, n, (hipStream_t)stream));
}

const char *gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_NULL: return "GDN_ERR_NULL: a required pointer is NULL";
        case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: invalid batch, length or head counts";
        case GDN_ERR_STRIDE: return "GDN_ERR_STRIDE: stride/pitch too small or misaligned";
        case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: head dims must be equal powers of two in [4, 256]";
        case GDN_ERR_ALIAS: return "GDN_ERR_ALIAS: state/output overlaps another buffer";
        case GDN_ERR_DTYPE: return "GDN_ERR_DTYPE: unsupported output dtype";
        case GDN_ERR_HIP: return "GDN_ERR_HIP: kernel launch failed";
        case GDN_ERR_ARG: return "GDN_ERR_ARG: invalid scalar argument or stream";
        case GDN_ERR_SCRATCH:
            return "GDN_ERR_SCRATCH: the call needs more than the library's static scratch "
                   "(GDN_SEQ_NOALLOC_MAX_BYTES per GPU)";
    }
    return "unknown gdn_status";
}

int32_t gdn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
