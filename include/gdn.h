/*
 * gdn.h -- C ABI of libgdn, the Gated DeltaNet mixer hot path for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation ("Qwen3.8 27B" model card, Gated DeltaNet bullet): the fused
 * q|k|v projection goes through a depthwise causal conv of width 4 and silu;
 * q and k are L2-normalised per head; each value head keeps a [dv, dk] f32
 * state S that the gated delta rule decays by
 *     alpha_t = exp(-exp(A_log) * softplus(a_t + dt_bias))
 * and writes at rate beta_t = sigmoid(b_t):
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t (q_scale * q_t);
 * the head outputs are RMS-normalised (scale 1 + w, f32) and gated by
 * silu(z).  16 q/k heads serve 48 value heads: value head h reads q/k head
 * h / (Hv / Hk).  Per the card's state paragraph, prefill runs one batch
 * and decode_rows advances persistent rows whose sequence lengths differ;
 * each row holds its conv history and recurrent state in f32.
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE pointers, row-major, owned by the caller.
 *    The library never allocates device memory, frees, synchronises, logs
 *    or aborts, with two exceptions: the first gdn_linear or
 *    gdn_linear_tune call on a device that goes to hipBLASLt creates the
 *    handle kept for that device, and gdn_linear_tune synchronises (see
 *    there).
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *    the default stream) and the call returns at once.  Device faults, if
 *    any, surface at the caller's next synchronisation.
 *  - All arguments are validated on the host first.  On any error nothing
 *    is enqueued and a nonzero gdn_status is returned; gdn_status_str()
 *    names it.  Calls are stateless and thread-safe.
 *  - dtype arguments take a gdn_dtype value: GDN_F32 or GDN_BF16 (bf16
 *    stored as its 16-bit pattern).  Arithmetic is f32 (MFMA for the chunked
 *    prefill: bf16 operands, f32 accumulation).
 *  - Alignment: f32 state and conv-history pointers 16 bytes; q/k/v/o/x/y/z
 *    16 bytes with row strides that keep every head 16-byte aligned.
 *  - Head widths: only dk = dv = 128 is implemented (GDN_ERR_UNSUPPORTED
 *    otherwise); Hv must be a multiple of Hk.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 2

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_NULL = 1,        /* a required pointer is NULL */
  GDN_ERR_SHAPE = 2,       /* a size or stride is out of range */
  GDN_ERR_DTYPE = 3,       /* unknown or unsupported dtype combination */
  GDN_ERR_ALIGN = 4,       /* a pointer or stride breaks the alignment rules */
  GDN_ERR_UNSUPPORTED = 5, /* valid but not implemented (e.g. head width != 128) */
  GDN_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required */
  GDN_ERR_LAUNCH = 7,      /* the HIP runtime refused the launch */
  GDN_ERR_SCRATCH = 8      /* larger than the no-allocation entry point's fixed scratch */
} gdn_status;

typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Prefill algorithm.  AUTO picks CHUNKED for bf16 q/k/v and SEQUENTIAL for
 * f32 q/k/v.  SEQUENTIAL runs the recurrence token by token in f32 (any
 * dtype; f32 inputs keep f32 accuracy).  CHUNKED uses the chunk-of-64 WY/UT
 * form on bf16 MFMA with f32 accumulation and an f32 state carried between
 * chunks; it accepts bf16 q/k/v only (its bf16 operands cannot give f32
 * inputs their f32 accuracy): CHUNKED with f32 q/k/v returns
 * GDN_ERR_UNSUPPORTED. */
typedef enum gdn_algo { GDN_ALGO_AUTO = 0, GDN_ALGO_SEQUENTIAL = 1, GDN_ALGO_CHUNKED = 2 } gdn_algo;

/* Head counts and widths: 16, 48, 128, 128 for the model's layer. */
typedef struct gdn_dims {
  int32_t n_qk_heads; /* Hk */
  int32_t n_v_heads;  /* Hv, a multiple of Hk */
  int32_t head_k_dim; /* dk (128) */
  int32_t head_v_dim; /* dv (128) */
} gdn_dims;

/* Static string naming a status code (never NULL). */
const char* gdn_status_str(int status);

/* GDN_ABI_VERSION of the loaded library. */
int gdn_abi_version(void);

/*
 * gdn_conv_silu -- depthwise causal conv + silu, optional per-head L2.
 * ("Qwen3.8 27B" card, Gated DeltaNet bullet; llm-arch-viz module tree:
 * conv1d 10240x1x4 without bias.)
 *   x           [B, T, C] in dtype x_dt, token (b, t) at (b*T + t)*x_tok_stride
 *               elements (x_tok_stride >= C, a multiple of 8; C for a
 *               contiguous x, wider for the q|k|v columns of a buffer that
 *               also holds z, as one in_proj_qkvz product writes them).
 *   y           [B, T, C] contiguous in dtype y_dt (f32 output keeps the
 *               normalised q/k unrounded for the recurrence); y must not
 *               overlap x.
 *   w           [C, W] f32; w[c][W-1] multiplies the current token,
 *               w[c][0] the input W-1 tokens back (cross-correlation).
 *   conv_state  [B, W-1, C] f32, in/out: the last W-1 inputs before this
 *               call on entry, the last W-1 inputs of [history; x] on exit.
 *               NULL means a zero history and nothing is written.
 *   y[b,t,c] = silu(sum_i w[c][i] * xhat[b, t+i, c]) with xhat = [history; x];
 *   then for c < l2_channels, each group of head_dim channels of y is divided
 *   by sqrt(sum of squares + l2_eps).
 * Constraints: W == 4; C % 8 == 0; l2_channels % head_dim == 0 and
 * l2_channels <= C; head_dim == 128 when l2_channels > 0; T == 0 is a no-op.
 */
int gdn_conv_silu(const void* x, int64_t x_tok_stride, int32_t x_dt, void* y, int32_t y_dt,
                  const float* w, float* conv_state, int32_t B, int32_t T, int32_t C, int32_t W,
                  int32_t l2_channels, int32_t head_dim, float l2_eps, void* stream);

/*
 * Bytes of device workspace gdn_prefill needs for these sizes and algorithm
 * (0 for the sequential algorithm, and for f32 q/k/v, which never run
 * chunked).  The caller allocates it; its contents need no initialisation
 * and are scratch after the call.
 */
size_t gdn_prefill_workspace_bytes(int32_t B, int32_t T, gdn_dims dims, int32_t qkv_dt,
                                   int32_t algo);

/*
 * gdn_prefill -- the gated delta rule over T tokens of B sequences, with the
 * state carried in and out (the card's prefill; a long prompt is continued
 * from where the previous call stopped when state_in holds that call's
 * state_out, as the code-generation page's prefill chunks start at a given
 * position).
 *   q, k   [B, T, Hk, dk] in qkv_dt; element (b,t,h,i) at
 *          b*T*tok_stride + t*tok_stride + h*dk + i (strides in elements),
 *          so q, k and v may be views into the conv output (stride 10240).
 *   v      [B, T, Hv, dv] in qkv_dt, same addressing with v_tok_stride.
 *   a, b   [B, T, Hv] contiguous in gate_dt (the gate pre-activations).
 *   A_log, dt_bias  [Hv] f32.
 *   state_in   [B, Hv, dv, dk] f32 (S row-major, dk fastest); NULL = zeros.
 *   state_out  [B, Hv, dv, dk] f32; NULL = not written; may equal state_in.
 *   o      [B, T, Hv, dv] contiguous in dtype o_dt; o_t uses the state
 *          after token t's update.
 *   q_scale multiplies q (1.0 for the model's layer).
 *   algo   a gdn_algo value.
 *   workspace  device scratch of at least gdn_prefill_workspace_bytes(...)
 *          bytes (may be NULL when that is 0), 256-byte aligned.
 * With T == 0 only the state passes through (state_out = state_in, or
 * zeros); the token pointers may then be NULL.
 * Errors: GDN_ERR_WORKSPACE if the workspace is too small;
 * GDN_ERR_UNSUPPORTED for algo CHUNKED with f32 q/k/v.
 */
int gdn_prefill(const void* q, int64_t q_tok_stride, const void* k, int64_t k_tok_stride,
                const void* v, int64_t v_tok_stride, int32_t qkv_dt, const void* a,
                const void* b, int32_t gate_dt, const float* A_log, const float* dt_bias,
                const float* state_in, float* state_out, void* o, int32_t o_dt, int32_t B,
                int32_t T, gdn_dims dims, float q_scale, int32_t algo, void* workspace,
                size_t workspace_bytes, void* stream);

/*
 * gdn_decode_rows -- one new token for each of R persistent rows whose
 * lengths differ, the state updated in place (the card's decode_rows;
 * "Qwen3.8 27B" model card, state paragraph).
 *   q, k   [R, Hk, dk] in qkv_dt, row r at r*row_stride (elements).
 *   v      [R, Hv, dv] in qkv_dt, row r at r*v_row_stride.
 *   a, b   [R, Hv] contiguous in gate_dt.
 *   A_log, dt_bias  [Hv] f32.
 *   state  [R, Hv, dv, dk] f32, row r's state at index r; read and written.
 *   lengths [R] int32 tokens already consumed by each row, or NULL (all rows
 *          active).  The rule uses no positions, so lengths only mark idle
 *          rows: lengths[r] < 0 leaves row r's state untouched and writes
 *          zeros to its output.
 *   o      [R, Hv, dv] contiguous in qkv_dt.
 * The conv step for decode is gdn_conv_silu with B = R, T = 1.
 */
int gdn_decode_rows(const void* q, int64_t q_row_stride, const void* k, int64_t k_row_stride,
                    const void* v, int64_t v_row_stride, int32_t qkv_dt, const void* a,
                    const void* b, int32_t gate_dt, const float* A_log, const float* dt_bias,
                    float* state, const int32_t* lengths, void* o, int32_t R, gdn_dims dims,
                    float q_scale, void* stream);

/*
 * gdn_decode_rows_multi -- K new tokens for each of R persistent rows (a
 * draft of K tokens to verify, the shape of the blog's multi-token
 * prediction and speculative decoding, over the card's decode_rows rows of
 * differing lengths).  Each row's state is read once, advanced through its K tokens
 * in order and written once; K tokens equal K successive gdn_decode_rows
 * calls, bit for bit.
 *   q, k   token t of row r at r*row_stride + t*tok_stride (elements), each
 *          [Hk, dk]; v likewise [Hv, dv].
 *   a, b   [R, K, Hv] contiguous in gate_dt; A_log, dt_bias [Hv] f32.
 *   state  [R, Hv, dv, dk] f32, read and written in place (the state after
 *          all K tokens).
 *   snapshots  [R, K, Hv, dv, dk] f32 or NULL: snapshots[r][t] receives row
 *          r's state after its token t, so a verifier that accepts n tokens
 *          continues from snapshots[r][n-1].  Must not overlap state.
 *   lengths [R] int32 or NULL, as in gdn_decode_rows: < 0 marks an idle row
 *          (state and snapshots untouched, outputs zero).
 *   o      [R, K, Hv, dv] contiguous in qkv_dt.
 * K == 0 or R == 0 is a no-op.
 */
int gdn_decode_rows_multi(const void* q, int64_t q_row_stride, int64_t q_tok_stride,
                          const void* k, int64_t k_row_stride, int64_t k_tok_stride,
                          const void* v, int64_t v_row_stride, int64_t v_tok_stride,
                          int32_t qkv_dt, const void* a, const void* b, int32_t gate_dt,
                          const float* A_log, const float* dt_bias, float* state,
                          float* snapshots, const int32_t* lengths, void* o, int32_t R,
                          int32_t K, gdn_dims dims, float q_scale, void* stream);

/*
 * gdn_gated_rmsnorm -- y = x / sqrt(mean(x^2) + eps) * (1 + w) * silu(z) per
 * row of D ("Qwen3.8 27B" card, Gated DeltaNet and Norms bullets;
 * llm-arch-viz: RMSNormGated of width 128, eps 1e-06).
 *   x, y     [N, H, D] contiguous in dtype `dt`; y may equal x.
 *   z        [N, H, D] in dtype `dt`, token n at n*z_tok_stride elements
 *            (z_tok_stride >= H*D, a multiple of 8; H*D when contiguous).
 *   w        [D] f32, shared by all heads.
 * Constraints: D == 128.
 */
int gdn_gated_rmsnorm(const void* x, const void* z, int64_t z_tok_stride, void* y, int32_t dt,
                      const float* w, int32_t N, int32_t H, int32_t D, float eps, void* stream);

/*
 * Bytes of device workspace gdn_prefill_slots needs for R rows of at most
 * max_len new tokens (0 if R or max_len is 0).
 */
size_t gdn_prefill_slots_workspace_bytes(int32_t R, int32_t max_len, gdn_dims dims);

/*
 * gdn_prefill_slots -- ragged prefill of persistent rows, each row
 * continuing from its own state with its own number of new tokens ("Qwen3.8
 * 27B" model card, state paragraph: rows stay in place between calls, each
 * with its own length, conv history and f32 recurrent state).  The rule
 * uses no positions, so a row's length so far only lives in its state.
 * Chunks of 64 start at each row's first new token.
 *   q, k   [total_tokens, Hk, dk] in qkv_dt, token t at t*tok_stride
 *          (elements); v [total_tokens, Hv, dv] likewise: the rows' new
 *          tokens packed one row after another.
 *   a, b   [total_tokens, Hv] contiguous in gate_dt; A_log, dt_bias [Hv] f32.
 *   cu_seqlens  [R + 1] int32, DEVICE: row r's tokens are
 *          [cu_seqlens[r], cu_seqlens[r+1]) of the packed axis, with
 *          cu_seqlens[0] = 0, non-decreasing, cu_seqlens[R] = total_tokens
 *          and no row longer than max_len.  The kernels clamp the offsets
 *          into [0, total_tokens] and a row to max_len tokens, so bad
 *          offsets give wrong rows, never accesses outside the arrays.
 *   state  [R, Hv, dv, dk] f32, row r's state at index r, read and written
 *          in place; a row with no new tokens keeps its state.
 *   o      [total_tokens, Hv, dv] contiguous in o_dt.
 *   max_len  the longest row (host value; sizes the launch and workspace).
 *   workspace  at least gdn_prefill_slots_workspace_bytes(R, max_len, dims)
 *          bytes, 256-byte aligned.
 * bf16 q/k/v run the chunked algorithm (bf16 MFMA); f32 q/k/v run token by
 * token in f32 (the workspace may then be NULL).  R == 0, max_len == 0 or
 * total_tokens == 0 is a no-op.
 */
int gdn_prefill_slots(const void* q, int64_t q_tok_stride, const void* k, int64_t k_tok_stride,
                      const void* v, int64_t v_tok_stride, int32_t qkv_dt, const void* a,
                      const void* b, int32_t gate_dt, const float* A_log, const float* dt_bias,
                      const int32_t* cu_seqlens, float* state, void* o, int32_t o_dt, int32_t R,
                      int32_t max_len, int32_t total_tokens, gdn_dims dims, float q_scale,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace gdn_mixer_prefill needs (0 if B or T is 0 or the
 * dims are invalid), enough for either dtype.  The caller allocates it; no
 * initialisation is needed.
 */
size_t gdn_mixer_prefill_workspace_bytes(int32_t B, int32_t T, gdn_dims dims);

/*
 * gdn_mixer_prefill -- the whole mixer between the projections for T tokens
 * of B sequences, in the order the "Qwen3.8 27B" model card's Gated DeltaNet
 * bullet gives: depthwise causal conv (width 4) + silu over the q|k|v
 * channels, L2 of each q and k head, the gated delta rule with the state
 * carried in and out, and the per-head RMSNorm (scale 1 + w) gated by
 * silu(z).  bf16 inputs: the same result as gdn_conv_silu (f32 output) ->
 * gdn_prefill (chunked) -> gdn_gated_rmsnorm, without the f32 round trip of
 * v: the conv writes q|k in f32 and v in bf16 to the workspace (the chunked
 * prefill rounds v to bf16 anyway).  f32 inputs: conv (f32 output) ->
 * sequential f32 recurrence -> norm, f32 throughout.
 *   qkv    [B, T, C] in dt, C = 2*Hk*dk + Hv*dv, channels [q heads | k heads |
 *          v heads]; token (b, t) at (b*T + t)*qkv_tok_stride elements.
 *   z      [B, T, Hv*dv] in dt (the output gate); token (b, t) at
 *          (b*T + t)*z_tok_stride.  The strides (>= C and >= Hv*dv, multiples
 *          of 8) let qkv and z be the two column ranges of one [B, T, C +
 *          Hv*dv] buffer, the output of in_proj_qkv and in_proj_z stored as
 *          one weight and run as one gdn_linear.
 *   conv_w [C, 4] f32 (w[c][3] multiplies the current token);
 *   conv_state [B, 3, C] f32 in/out as in gdn_conv_silu, or NULL (zero
 *          history, not written).
 *   a, b   [B, T, Hv] contiguous in gate_dt; A_log, dt_bias [Hv] f32.
 *   norm_w [dv] f32 (the scale is 1 + norm_w), shared by all heads.
 *   state_in / state_out  [B, Hv, dv, dk] f32 as in gdn_prefill.
 *   y      [B, T, Hv*dv] contiguous in dt; must not overlap qkv, z or the
 *          workspace (each over the extent its stride spans).
 *   l2_eps (1e-6) inside the q/k L2 norm; norm_eps (1e-6) of the RMSNorm.
 *   workspace  at least gdn_mixer_prefill_workspace_bytes(B, T, dims) bytes,
 *          256-byte aligned; scratch after the call.
 * With T == 0 the conv history is left as it is and the state passes
 * through.  Errors as for the three calls it replaces; GDN_ERR_SHAPE if y
 * overlaps qkv, z or the workspace.
 */
int gdn_mixer_prefill(const void* qkv, int64_t qkv_tok_stride, const void* z,
                      int64_t z_tok_stride, int32_t dt, const float* conv_w,
                      float* conv_state, const void* a, const void* b, int32_t gate_dt,
                      const float* A_log, const float* dt_bias, const float* norm_w,
                      const float* state_in, float* state_out, void* y, int32_t B, int32_t T,
                      gdn_dims dims, float q_scale, float l2_eps, float norm_eps,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace gdn_gate_proj needs for M tokens (0 when none
 * is needed or the sizes are invalid).  The caller allocates it; no
 * initialisation is needed.
 */
size_t gdn_gate_proj_workspace_bytes(int32_t M, int32_t K, int32_t H);

/*
 * gdn_gate_proj -- the two gate projections of the mixer, with f32 weights.
 * ("Qwen/Qwen3.8-27B" architecture viewer, module tree: in_proj_a and
 * in_proj_b, 5120 -> 48 each; the "qwen38" code-generation page, extra
 * kernels: these two small projections keep f32 weights.)
 *   a[m][h] = sum_k x[m][k] W_a[h][k],   b[m][h] = sum_k x[m][k] W_b[h][k]
 *   x         [M, K] bf16 with row stride x_ld (elements); the hidden state.
 *   W_a, W_b  [H, K] f32, contiguous (the Linear layout, output-major).
 *   a, b      [M, H] f32 with row stride ab_ld; they feed the gates of
 *             gdn_prefill / gdn_decode_rows (gate dtype GDN_F32) directly.
 *   workspace at least gdn_gate_proj_workspace_bytes(M, K, H) bytes,
 *             256-byte aligned (NULL when that is 0); scratch after the call.
 * The weights are used unrounded: each is split exactly into three bf16
 * parts on the fly, and every product is exact in f32.  K is cut into
 * ranges whose f32 partial sums are added in a fixed order (results do not
 * vary from run to run).
 * Constraints: x_dt == GDN_BF16 and H <= 64 (GDN_ERR_UNSUPPORTED
 * otherwise); K > 0 and K % 32 == 0; H > 0 and H % 16 == 0; x_ld >= K,
 * x_ld % 8 == 0; ab_ld >= H; x, W_a, W_b 16-byte aligned; a and b must not
 * overlap x or the workspace.  M == 0 is a no-op.
 */
int gdn_gate_proj(const void* x, int64_t x_ld, int32_t x_dt, const float* W_a,
                  const float* W_b, float* a, float* b, int64_t ab_ld, int32_t M, int32_t K,
                  int32_t H, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace recommended for gdn_linear (32 MiB).  Smaller
 * workspaces (including none) are accepted; they limit the algorithms
 * hipBLASLt may choose.
 */
size_t gdn_linear_workspace_bytes(void);

/*
 * gdn_linear -- a bf16 linear layer, y = x W^T: the mixer's in_proj_qkv
 * (5120 -> 10240), in_proj_z (5120 -> 6144) and out_proj (6144 -> 5120)
 * ("Qwen/Qwen3.8-27B" architecture viewer, module tree).
 *   x  [M, K] bf16, row stride x_ld (elements).
 *   W  [N, K] bf16, row stride w_ld (the Linear layout, output-major).
 *   y  [M, N] in y_dt (GDN_BF16 or GDN_F32), row stride y_ld; must not
 *      overlap x or W.
 *   y[m][n] = sum_k x[m][k] W[n][k], f32 accumulation, one rounding to y_dt.
 * Two engines serve it.  Shapes the library's own MFMA GEMM suits run there
 * (gdn_linear_kernel says which form): its tiled form when the shape fills
 * the GPU (K a multiple of 64, N a multiple of 160, 192, 256 or 320, and at
 * least one full round of 256-row by that-width tiles over the GPU's CUs),
 * or its few-row form for M <= 64 (K and N multiples of 64, enough 64-row
 * weight blocks times equal K ranges for about three quarters of the CUs;
 * more than one K range puts ranges * M * N f32 partial sums in the
 * workspace and adds them in a fixed order): no allocation, no handle,
 * nothing but the product enqueued, results independent of the workspace's
 * contents.  Every other shape runs on hipBLASLt
 * (whichever libhipblaslt.so.1 the process loaded first serves the call; a
 * loaded library of another major version than the header this library was
 * built with gives GDN_ERR_UNSUPPORTED).  The first call on a device that
 * goes to hipBLASLt creates its handle and keeps it (hipBLASLt may allocate
 * then; make that call before any graph capture).  A shape's hipBLASLt plan
 * (descriptors and the heuristic's first algorithm that fits the workspace)
 * is made on the host by its first call, with nothing enqueued or awaited
 * beyond the product, and kept for the 64 most recent shapes; a shape timed
 * by gdn_linear_tune keeps the engine and plan that won.  Calls from several
 * threads are serialised by a lock while they enqueue.
 *   workspace  scratch for hipBLASLt and for the few-row form's partial
 *              sums, 256-byte aligned, workspace_bytes long
 *              (gdn_linear_workspace_bytes() recommended), or NULL with 0;
 *              must not overlap x, W or y (GDN_ERR_SHAPE).
 * Constraints: M >= 0 (0 is a no-op), N > 0, K > 0; x_ld >= K, w_ld >= K,
 * y_ld >= N, each a multiple of 8; x, W, y 16-byte aligned.
 * GDN_ERR_UNSUPPORTED if the shape goes to hipBLASLt and it has no
 * algorithm for it within the workspace; GDN_ERR_LAUNCH if the product
 * fails to enqueue.
 */
int gdn_linear(const void* x, int64_t x_ld, const void* W, int64_t w_ld, void* y, int64_t y_ld,
               int32_t y_dt, int32_t M, int32_t N, int32_t K, void* workspace,
               size_t workspace_bytes, void* stream);

/*
 * gdn_linear_tune -- gdn_linear that also times the shape's algorithms: up
 * to eight of hipBLASLt's candidates that fit the workspace, and the
 * library's GEMM when gdn_linear_kernel names one of its forms, run on this call's
 * own buffers and stream (one warm-up and three timed runs each; each writes
 * y, and the call's product is written last), the fastest is kept as the
 * shape's plan for later gdn_linear calls, and the call synchronises the
 * stream.  For callers with a fixed set of shapes (a model's projections at
 * a set batch), once per shape, before any graph capture.  Arguments,
 * result and errors as gdn_linear.
 */
int gdn_linear_tune(const void* x, int64_t x_ld, const void* W, int64_t w_ld, void* y,
                    int64_t y_ld, int32_t y_dt, int32_t M, int32_t N, int32_t K, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * gdn_linear_kernel -- which engine an untimed gdn_linear call of this shape,
 * with a workspace of workspace_bytes, uses on the current device: the block
 * width in outputs of the library's MFMA GEMM (160, 192, 256 or 320 for its
 * tiled form, 64 for its few-row form), 0 for hipBLASLt, or a negative
 * gdn_status if the arguments are invalid or the device cannot be queried.
 * Host only; enqueues nothing.  (A shape timed by gdn_linear_tune uses the
 * engine that won, which this does not report.)
 */
int gdn_linear_kernel(int32_t M, int32_t N, int32_t K, int64_t x_ld, int64_t w_ld,
                      size_t workspace_bytes);

/* Size of the fixed device scratch of gdn_prefill_noalloc: 64 MiB, enough
 * for the chunked prefill of B*T <= 1152 tokens at 16 q/k and 48 value heads
 * (gdn_prefill_workspace_bytes gives the need of other sizes). */
#define GDN_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * gdn_prefill_noalloc -- gdn_prefill without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  The chunked
 * algorithm's scratch is a fixed device array inside the library
 * (GDN_NOALLOC_SCRATCH_BYTES; every GPU the library runs on holds its own
 * copy until the process ends); the call allocates nothing and does not
 * synchronise.  Its first call on a device looks up the array's device
 * address.  All calls on one GPU share the array, so calls that overlap on a
 * GPU (other streams or threads) race: serialise them.  Arguments, results
 * and errors as gdn_prefill; GDN_ERR_SCRATCH if
 * gdn_prefill_workspace_bytes(B, T, dims, qkv_dt, algo) exceeds
 * GDN_NOALLOC_SCRATCH_BYTES (nothing is enqueued).
 */
int gdn_prefill_noalloc(const void* q, int64_t q_tok_stride, const void* k, int64_t k_tok_stride,
                        const void* v, int64_t v_tok_stride, int32_t qkv_dt, const void* a,
                        const void* b, int32_t gate_dt, const float* A_log, const float* dt_bias,
                        const float* state_in, float* state_out, void* o, int32_t o_dt,
                        int32_t B, int32_t T, gdn_dims dims, float q_scale, int32_t algo,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
