/*
 * gdn.h -- C ABI of libgdn.so: the gated delta rule (Gated DeltaNet) state
 * recurrence on AMD Instinct MI355X (gfx950).
 *
 * The operation (logicaffeine "codegen_cuda/gdn.rs", kernel `gdn_step`): for
 * sequence b and value head h, with key head g = h mod NK (tiled pairing, the
 * `ggml_repeat` broadcast, NOT h / (NV/NK)), the head's Dv x Dk state S is
 * advanced by one token as
 *
 *     u = S k_g,  w = S q_g,  coef_i = beta (v_i - alpha u_i)
 *     o_i = (alpha w_i + coef_i (k_g . q_g)) / sqrt(Dk)          (= (S' q_g)_i / sqrt(Dk))
 *     S  <- alpha S + coef k_g^T                                 (= alpha S (I - beta k k^T) + beta v k^T)
 *
 * and optionally followed by the gated RMS norm of the same page's kernel
 * `gdn_gate_norm`: y_i = gn_i o_i / sqrt(mean_j o_j^2 + eps) * z_i sigmoid(z_i)
 * (norm, then weight, then gate).  alpha is a linear decay multiplier and beta
 * the write strength, one scalar each per (token, value head).
 *
 * The entry points mirror the launchers of metrale "layers/ops/ssm_gdn_a.rs"
 * (`gdn_decode`, `gdn_decode_f32_strided_norm`, `gdn_decode_f16_strided_norm`,
 * `gdn_prefill_regresident`, `ssm_h_state_f32_to_f16`, `ssm_h_state_f16_to_f32`):
 * device pointers, element strides per sequence row, a state slot pitch, a
 * stream, and an error code instead of a panic.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers   Every array pointer is a DEVICE pointer (hipMalloc / torch CUDA
 *            tensors).  The caller owns all memory; the library allocates no
 *            device memory, keeps no state except a thread-local last HIP error,
 *            and never synchronises.  Calls are asynchronous on `stream`
 *            (a hipStream_t; NULL = the null stream).
 * Strides    All strides and pitches count ELEMENTS of the array's own type,
 *            never bytes.  Sequence b's q/k row starts at q + b*qk_stride
 *            (key head g at + g*Dk); v, z and out rows at + b*stride (value
 *            head h at + h*Dv); alpha/beta at + b*ab_stride + h.  The state slot
 *            of sequence b starts at state + b*state_seq_stride; value head h's
 *            tile at + h*Dv*Dk, row-major with row i = value index and column
 *            j = key index (key index contiguous).  A pitch larger than
 *            NV*Dv*Dk leaves a pad that is never read or written.
 * Alignment  state, q, k, v, z and out base pointers must be 16-byte aligned,
 *            and their row strides / pitch a multiple of 4 elements (of 8 for a
 *            binary16 state pitch).  alpha, beta and norm_weight need only
 *            natural (4-byte) alignment.  Anything else returns GDN_ERR_STRIDE:
 *            there is no slow fallback path.
 * Shapes     k_dim == v_dim, a power of two in [4, 256]; num_v_heads a
 *            multiple of num_k_heads; batch (and seq_len) >= 0.  A zero batch
 *            or seq_len is a valid no-op (nothing is read, written or launched).
 * Aliasing   Read-only inputs may alias each other (e.g. q|k|v inside one packed
 *            projection row).  The state and the output must not overlap any
 *            input or each other: GDN_ERR_ALIAS (checked on address ranges).
 * Errors     Validation happens before any HIP call; on failure no buffer is
 *            touched and nothing is launched.  A failed launch returns
 *            GDN_ERR_HIP and gdn_last_hip_error() gives the hipError_t.
 *            Nothing prints, aborts or throws across the ABI.
 * Results    Bitwise deterministic run to run: fixed reduction orders, no
 *            atomics.  Non-finite inputs propagate; finite inputs in the ranges
 *            the recurrence is used with never produce NaN or Inf.
 * Threads    The functions are re-entrant; concurrent calls on distinct
 *            streams are safe when their output/state ranges are disjoint.
 */
#ifndef GDN_H
#define GDN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,        /* a required pointer is NULL                                   */
    GDN_ERR_SHAPE = 2,       /* negative batch/seq_len, non-positive heads, NV % NK != 0,
                                batch * num_v_heads above INT32_MAX (one launch's grid)       */
    GDN_ERR_STRIDE = 3,      /* stride/pitch too small for its row, or misaligned pointer     */
    GDN_ERR_UNSUPPORTED = 4, /* k_dim != v_dim, or not a power of two in [4, 256]             */
    GDN_ERR_ALIAS = 5,       /* state/out overlaps an input or each other; converter in-place */
    GDN_ERR_DTYPE = 6,       /* out_dtype is not GDN_F32 / GDN_BF16 (or not allowed here)     */
    GDN_ERR_HIP = 7,         /* the kernel launch failed; see gdn_last_hip_error()            */
    GDN_ERR_ARG = 8,         /* a scalar argument is invalid (eps negative or not finite), or
                                a stream of another device (gdn_recurrence_seq_noalloc)        */
    GDN_ERR_SCRATCH = 9      /* gdn_recurrence_seq_noalloc: the shape needs more scratch than
                                GDN_SEQ_NOALLOC_MAX_BYTES                                      */
} gdn_status;

enum { GDN_F32 = 0, GDN_BF16 = 1 };

/*
 * gdn_decode -- one token for every (sequence, value head) pair: the state is
 * advanced in place and the raw output o is written as fp32.
 * Source: logicaffeine codegen_cuda/gdn.rs, kernel `gdn_step`; metrale
 * ssm_gdn_a.rs, launchers `gdn_decode` and `gdn_decode_f32_strided`.
 *   state  fp32 [batch][state_seq_stride], slot layout as above (read+write)
 *   q, k   fp32 rows of >= num_k_heads*k_dim, qk_stride apart (read)
 *   v      fp32 rows of >= num_v_heads*v_dim, v_stride apart (read)
 *   alpha, beta  fp32 rows of >= num_v_heads, ab_stride apart (read)
 *   out    fp32 rows of num_v_heads*v_dim, out_stride apart (write)
 */
gdn_status gdn_decode(float *state, int64_t state_seq_stride,
                      const float *q, const float *k, int64_t qk_stride,
                      const float *v, int64_t v_stride,
                      const float *alpha, const float *beta, int64_t ab_stride,
                      float *out, int64_t out_stride,
                      int32_t batch, int32_t num_k_heads, int32_t num_v_heads,
                      int32_t k_dim, int32_t v_dim, void *stream);

/*
 * gdn_decode_norm -- gdn_decode with the gated RMS norm fused into the same
 * kernel: out receives y (fp32 or bf16 rounded to nearest-even) and no raw o is
 * written anywhere.  Source: logicaffeine codegen_cuda/gdn.rs, kernel
 * `gdn_gate_norm`; metrale ssm_gdn_a.rs, launchers `gdn_decode_f32_norm` and
 * `gdn_decode_f32_strided_norm`.
 *   z            fp32 rows of >= num_v_heads*v_dim, z_stride apart (read)
 *   norm_weight  fp32 [v_dim], shared by all heads (read)
 *   eps          >= 0, inside the square root (the model uses 1e-6)
 *   out          out_dtype (GDN_F32 or GDN_BF16) rows, out_stride apart (write)
 */
gdn_status gdn_decode_norm(float *state, int64_t state_seq_stride,
                           const float *q, const float *k, int64_t qk_stride,
                           const float *v, int64_t v_stride,
                           const float *alpha, const float *beta, int64_t ab_stride,
                           const float *z, int64_t z_stride, const float *norm_weight, float eps,
                           void *out, int32_t out_dtype, int64_t out_stride,
                           int32_t batch, int32_t num_k_heads, int32_t num_v_heads,
                           int32_t k_dim, int32_t v_dim, void *stream);

/*
 * gdn_decode_norm_q -- gdn_decode_norm with the int8 activation quantisation of
 * the output fused into the epilogue, for an int8 projection that follows.
 * Source: logicaffeine codegen_cuda/gdn.rs, kernel `gdn_gate_norm_q`: in groups
 * of 32 consecutive values of a head's y, scale = max|y| / 127 (1 when the group
 * is all zero) and code = y / scale rounded to nearest, ties to even; both
 * divisions are correctly rounded fp32 operations on the fp32 y.
 *   out     fp32 y rows as in gdn_decode_norm, or NULL to skip writing y
 *   codes   int8 rows of num_v_heads*v_dim, codes_stride apart (write; any alignment)
 *   scales  fp32 rows of num_v_heads*v_dim/32, scales_stride apart (write);
 *           scale e of row b covers codes[b][32e .. 32e+31]
 * v_dim must be a multiple of 32 (32, 64, 128 or 256), else GDN_ERR_UNSUPPORTED.
 * codes and scales must not overlap each other or any other array (GDN_ERR_ALIAS).
 */
gdn_status gdn_decode_norm_q(float *state, int64_t state_seq_stride,
                             const float *q, const float *k, int64_t qk_stride,
                             const float *v, int64_t v_stride,
                             const float *alpha, const float *beta, int64_t ab_stride,
                             const float *z, int64_t z_stride, const float *norm_weight, float eps,
                             float *out, int64_t out_stride,
                             int8_t *codes, int64_t codes_stride,
                             float *scales, int64_t scales_stride,
                             int32_t batch, int32_t num_k_heads, int32_t num_v_heads,
                             int32_t k_dim, int32_t v_dim, void *stream);

/*
 * gdn_decode_f16state -- the IEEE binary16 state twin of gdn_decode_norm.
 * The state is read as binary16, all arithmetic is fp32, and the updated state
 * is rounded to nearest-even binary16 on store (subnormals kept).
 * state_seq_stride is the slot pitch in HALVES, set by the caller's pool layout
 * (it may exceed NV * Dv * Dk).  z == NULL selects the raw output o, which then
 * must be GDN_F32; otherwise norm_weight is required and out is y as in
 * gdn_decode_norm.  Source: metrale ssm_gdn_a.rs, launcher
 * `gdn_decode_f16_strided_norm`.
 */
gdn_status gdn_decode_f16state(uint16_t *state, int64_t state_seq_stride,
                               const float *q, const float *k, int64_t qk_stride,
                               const float *v, int64_t v_stride,
                               const float *alpha, const float *beta, int64_t ab_stride,
                               const float *z, int64_t z_stride, const float *norm_weight,
                               float eps, void *out, int32_t out_dtype, int64_t out_stride,
                               int32_t batch, int32_t num_k_heads, int32_t num_v_heads,
                               int32_t k_dim, int32_t v_dim, void *stream);

/*
 * gdn_recurrence_seq -- seq_len tokens of every (sequence, value head), the
 * state held on chip across tokens: each slot is read once at the start and
 * written once at the end.  Token t of sequence b uses input row
 * r = b*seq_len + t of q, k, v, z, alpha, beta and writes output row r.
 * z == NULL gives the raw o; otherwise the fused gated norm y (norm_weight
 * required).  Output is fp32.  Source: metrale ssm_gdn_a.rs, launcher
 * `gdn_prefill_regresident` (token-sequential recurrence with the state in
 * registers), generalised to any supported head dim.
 */
gdn_status gdn_recurrence_seq(float *state, int64_t state_seq_stride,
                              const float *q, const float *k, int64_t qk_stride,
                              const float *v, int64_t v_stride,
                              const float *alpha, const float *beta, int64_t ab_stride,
                              const float *z, int64_t z_stride, const float *norm_weight,
                              float eps, float *out, int64_t out_stride,
                              int32_t batch, int32_t seq_len, int32_t num_k_heads,
                              int32_t num_v_heads, int32_t k_dim, int32_t v_dim, void *stream);

/*
 * gdn_recurrence_seq_ws -- gdn_recurrence_seq with a caller-provided device
 * workspace.  Same operation, arguments, layouts and results (within the fp32
 * tolerance; the summation order differs).  For k_dim == v_dim == 128 it runs
 * in two launches: a pre-pass forms, for every (sequence, value head, 16-token
 * chunk), the input-only quantities of the chunked form of the recurrence (the
 * inverse of the chunk's unit lower triangular system, the decayed k.q matrix,
 * beta and the decay products) into the workspace, and the state pass then
 * splits each head over four workgroups and writes the raw o.  With z, a third
 * launch applies the gated norm to the output rows in place.  Any other head
 * dim, a shape whose launch grids would exceed 2^31 workgroups, or one where
 * seq_len rows of q, k, v or out span 2^31 bytes or more (seq_len * stride *
 * 4), ignores the workspace (it may be NULL) and runs as gdn_recurrence_seq.  Source: metrale ssm_gdn_a.rs, launcher
 * `gdn_prefill_regresident` (the operation); the chunked form is exact algebra
 * on logicaffeine gdn.rs `gdn_step`.
 *   workspace        device memory of at least gdn_seq_workspace_bytes(...)
 *                    bytes, 16-byte aligned, overlapping no other argument
 *                    (GDN_ERR_NULL, GDN_ERR_ARG if smaller, GDN_ERR_STRIDE if
 *                    misaligned, GDN_ERR_ALIAS).  Owned by the caller; its
 *                    contents are scratch, written and read within the call
 *                    (calls that share a workspace must be ordered on one
 *                    stream).
 *   workspace_bytes  its size in bytes.
 */
gdn_status gdn_recurrence_seq_ws(float *state, int64_t state_seq_stride,
                                 const float *q, const float *k, int64_t qk_stride,
                                 const float *v, int64_t v_stride,
                                 const float *alpha, const float *beta, int64_t ab_stride,
                                 const float *z, int64_t z_stride, const float *norm_weight,
                                 float eps, float *out, int64_t out_stride,
                                 int32_t batch, int32_t seq_len, int32_t num_k_heads,
                                 int32_t num_v_heads, int32_t k_dim, int32_t v_dim,
                                 void *workspace, int64_t workspace_bytes, void *stream);

/*
 * gdn_seq_workspace_bytes -- bytes of workspace gdn_recurrence_seq_ws uses for
 * this shape: batch * num_v_heads * ceil(seq_len / 16) * 2304 when
 * k_dim == v_dim == 128, else 0 (no workspace used).  -1 for a negative or
 * overflowing shape.  Host-only; touches no device.
 */
int64_t gdn_seq_workspace_bytes(int32_t batch, int32_t seq_len, int32_t num_v_heads,
                                int32_t k_dim, int32_t v_dim);

/* Size of the static scratch array behind gdn_recurrence_seq_noalloc, per GPU. */
#define GDN_SEQ_NOALLOC_MAX_BYTES (64ll << 20)

/*
 * gdn_recurrence_seq_noalloc -- for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  gdn_recurrence_seq_ws with the workspace taken from a static
 * array inside the library instead of from the caller: same arguments as
 * gdn_recurrence_seq, same kernels, results bit for bit equal to
 * gdn_recurrence_seq_ws on the same inputs.  The call itself allocates nothing
 * (no hipMalloc, no hipFree, no allocating library routine).
 *   limit      the shape may need at most GDN_SEQ_NOALLOC_MAX_BYTES (64 MiB) of
 *              workspace, gdn_seq_workspace_bytes(batch, seq_len, num_v_heads,
 *              128, 128) -- e.g. batch * num_v_heads * ceil(seq_len / 16) <=
 *              29127 records: one sequence of 48 heads up to 9696 tokens.  A
 *              larger shape returns GDN_ERR_SCRATCH before anything is
 *              launched.  Shapes that run without a workspace (another head
 *              dim, very wide strides; see gdn_recurrence_seq_ws) need none.
 *   set-up     The library holds one copy of the array per GPU for the life of
 *              the process.  The first call on a device (with that device
 *              current, as for any call: `stream` must belong to the current
 *              device, and a stream of another device returns GDN_ERR_ARG)
 *              resolves its address there with hipGetSymbolAddress; make that
 *              first call outside graph capture.
 *   sharing    Every call on one GPU uses that GPU's one array, and the array
 *              keeps the last call's contents.  Calls that may overlap on one
 *              GPU (two streams, two host threads) race on it and give wrong
 *              results; order them on one stream.  Nothing in the array needs
 *              to start at zero: each call writes every record it reads.
 * Errors as gdn_recurrence_seq, plus GDN_ERR_SCRATCH, and GDN_ERR_ARG for a
 * stream of another device.
 */
gdn_status gdn_recurrence_seq_noalloc(float *state, int64_t state_seq_stride,
                                      const float *q, const float *k, int64_t qk_stride,
                                      const float *v, int64_t v_stride,
                                      const float *alpha, const float *beta, int64_t ab_stride,
                                      const float *z, int64_t z_stride, const float *norm_weight,
                                      float eps, float *out, int64_t out_stride,
                                      int32_t batch, int32_t seq_len, int32_t num_k_heads,
                                      int32_t num_v_heads, int32_t k_dim, int32_t v_dim,
                                      void *stream);

/*
 * gdn_decode_verify -- num_tokens (1..GDN_VERIFY_MAX_TOKENS) consecutive tokens
 * per sequence in one launch, keeping the state after every token but the last
 * for rollback: when a speculative (draft) token is rejected, the state after
 * the last accepted token is already in inter_state.  Source: metrale
 * ssm_gdn_a.rs, launcher `gdn_decode_chunk2` (two tokens, the intermediate
 * state written for draft rejection), generalised to up to 8 tokens.
 *   Token t of sequence b uses input row r = b*num_tokens + t of q, k, v, z,
 *   alpha, beta and writes output row r (raw o when z is NULL, else y as in
 *   gdn_decode_norm; fp32).
 *   state        fp32 pool as in gdn_decode: read once, final state written once.
 *   inter_state  fp32, batch*(num_tokens-1) slots of inter_pitch elements; slot
 *                b*(num_tokens-1) + t holds the state after token t, head h at
 *                + h*Dv*Dk (same tile layout).  May be NULL when num_tokens == 1.
 *                Must not overlap any other buffer (GDN_ERR_ALIAS).
 */
#define GDN_VERIFY_MAX_TOKENS 8
gdn_status gdn_decode_verify(float *state, int64_t state_seq_stride,
                             float *inter_state, int64_t inter_pitch,
                             const float *q, const float *k, int64_t qk_stride,
                             const float *v, int64_t v_stride,
                             const float *alpha, const float *beta, int64_t ab_stride,
                             const float *z, int64_t z_stride, const float *norm_weight, float eps,
                             float *out, int64_t out_stride,
                             int32_t batch, int32_t num_tokens, int32_t num_k_heads,
                             int32_t num_v_heads, int32_t k_dim, int32_t v_dim, void *stream);

/*
 * gdn_decode_fused -- one token with the layer's input stage fused in front of
 * the step: the projection row x (channels q | k | v, before the conv) goes
 * through the depthwise causal conv over the sequence's ring of the last `taps`
 * rows and silu; every q and k head block is divided by sqrt(sum of its squares
 * + l2_eps); beta = sigmoid(br) and alpha = (1 + exp(ar + dt_bias))^decay_rate
 * per value head; then the step (and, with z, the gated RMS norm) of
 * gdn_decode / gdn_decode_norm.  Sources: logicaffeine codegen_cuda/gdn.rs,
 * kernels `gk_conv_silu_l2` and `gk_gdn_gates`; metrale ssm_gdn_a.rs, launcher
 * `gdn_decode_f32_conv_norm`.
 *   C = (2*num_k_heads + num_v_heads) * D channels (D = k_dim = v_dim).
 *   conv_state   fp32, per sequence taps rows of C channels, row 0 the oldest;
 *                slot b at conv_state + b*conv_seq_stride, row t at + t*C.
 *                The new ring is the old one shifted up by one row with x
 *                appended as row taps-1.
 *   conv_state_out  NULL: the new ring replaces the old one in place (one
 *                workgroup per key head owns its channels; the features of
 *                its NV/NK value heads must fit 64 KiB of LDS, else
 *                GDN_ERR_UNSUPPORTED).  Otherwise a second buffer of the same
 *                layout and stride that receives the new ring while conv_state
 *                is only read (one workgroup per value head; faster); callers
 *                alternate the two buffers from token to token.
 *   x            fp32 rows of >= C, x_stride apart (read)
 *   conv_weight  fp32 [taps][C] (read); taps in [1, 8]
 *   br, ar       fp32 rows of >= num_v_heads, gate_stride apart (read)
 *   dt_bias, decay_rate  fp32 [num_v_heads] (read); decay_rate is the negative
 *                exponent itself (no further exp is applied)
 *   l2_eps       >= 0, inside the square root of the q/k normalisation
 *   z            NULL: raw o is written; else the gated norm as gdn_decode_norm
 *   out          fp32 rows of num_v_heads*v_dim, out_stride apart (write)
 * state, conv_state, conv_state_out and out must not overlap each other or any
 * input (GDN_ERR_ALIAS).  conv_state(_out), x and conv_weight need 16-byte
 * alignment and (for batch > 1) strides that are multiples of 4.
 */
gdn_status gdn_decode_fused(float *state, int64_t state_seq_stride,
                            float *conv_state, int64_t conv_seq_stride, float *conv_state_out,
                            const float *x, int64_t x_stride,
                            const float *conv_weight, int32_t taps,
                            const float *br, const float *ar, int64_t gate_stride,
                            const float *dt_bias, const float *decay_rate, float l2_eps,
                            const float *z, int64_t z_stride, const float *norm_weight, float eps,
                            float *out, int64_t out_stride,
                            int32_t batch, int32_t num_k_heads, int32_t num_v_heads,
                            int32_t k_dim, int32_t v_dim, void *stream);

/*
 * State pool converters: n elements, fp32 -> binary16 with round to
 * nearest-even (subnormals kept, overflow to infinity, NaN stays NaN), and
 * binary16 -> fp32 (exact).  src and dst must not overlap (an in-place
 * narrowing would race): GDN_ERR_ALIAS.  Both 16-byte aligned.  n == 0 is a
 * no-op.  Source: metrale ssm_gdn_a.rs, `ssm_h_state_f32_to_f16` and
 * `ssm_h_state_f16_to_f32`.
 */
gdn_status gdn_state_f32_to_f16(const float *src, uint16_t *dst, int64_t n, void *stream);
gdn_status gdn_state_f16_to_f32(const uint16_t *src, float *dst, int64_t n, void *stream);

/* Static, human-readable name of a status code. */
const char *gdn_status_string(gdn_status s);

/* The hipError_t of the calling thread's last GDN_ERR_HIP (0 if none yet). */
int32_t gdn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
