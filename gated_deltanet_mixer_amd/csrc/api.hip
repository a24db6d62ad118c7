// The C ABI (include/gdn.h): host-side validation, then one or two launches on
// the caller's stream.  Nothing here allocates or synchronises (gdn_linear's
// first call on a device that goes to hipBLASLt creates its handle, and
// gdn_linear_tune times on the stream; both in proj.hip).
#include <hip/hip_runtime.h>

#include "../../include/gdn.h"
#include "launch.hpp"

namespace {

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }
size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const char* x = static_cast<const char*>(a);
  const char* y = static_cast<const char*>(b);
  return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

// The whole mixer's workspace: the conv output (q|k in f32, v in bf16), then
// the chunked prefill's workspace.
struct MixerWs {
  size_t qk_bytes, v_bytes, chunk_bytes;
  size_t total() const { return qk_bytes + v_bytes + chunk_bytes; }
};
MixerWs mixer_ws(int32_t B, int32_t T, const gdn_dims& d) {
  MixerWs w;
  w.qk_bytes = round256((size_t)B * T * 2 * d.n_qk_heads * d.head_k_dim * 4);
  w.v_bytes = round256((size_t)B * T * d.n_v_heads * d.head_v_dim * 2);
  w.chunk_bytes = gdn::prefill_chunked_workspace_bytes(B, T, d.n_qk_heads, d.n_v_heads);
  return w;
}
bool dtype_ok(int32_t d) { return d == GDN_F32 || d == GDN_BF16; }

// The chunked algorithm runs on bf16 MFMA and serves bf16 q/k/v only: f32
// inputs go to the sequential f32 kernel (AUTO), and an explicit CHUNKED
// request with f32 q/k/v is refused.
bool uses_chunked(int32_t algo, int32_t qkv_dt) {
  return qkv_dt == GDN_BF16 && (algo == GDN_ALGO_CHUNKED || algo == GDN_ALGO_AUTO);
}
size_t dsize(int32_t d) { return d == GDN_BF16 ? 2 : 4; }

int launch_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH; }

// The conv runs one workgroup per (batch, token block, channel block),
// numbered in 32 bits.
bool conv_grid_ok(int64_t B, int64_t T, int64_t C) {
  const int64_t chans = gdn::CONV_THREADS * 8;
  return B * ((T + gdn::CONV_TB - 1) / gdn::CONV_TB) * ((C + chans - 1) / chans) + 8 < INT32_MAX;
}

// Shared checks of the recurrence inputs.
int check_dims(const gdn_dims& d) {
  if (d.n_qk_heads <= 0 || d.n_v_heads <= 0 || d.head_k_dim <= 0 || d.head_v_dim <= 0)
    return GDN_ERR_SHAPE;
  if (d.n_v_heads % d.n_qk_heads != 0) return GDN_ERR_SHAPE;
  if (d.head_k_dim != 128 || d.head_v_dim != 128) return GDN_ERR_UNSUPPORTED;
  return GDN_OK;
}

}  // namespace

extern "C" {

const char* gdn_status_str(int status) {
  switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_NULL: return "GDN_ERR_NULL: a required pointer is NULL";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: a size or stride is out of range";
    case GDN_ERR_DTYPE: return "GDN_ERR_DTYPE: unsupported dtype";
    case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN: pointer or stride misaligned";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: valid but not implemented";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
    case GDN_ERR_LAUNCH: return "GDN_ERR_LAUNCH: kernel launch failed";
    case GDN_ERR_SCRATCH:
      return "GDN_ERR_SCRATCH: larger than the no-allocation entry point's fixed scratch";
    default: return "unknown gdn_status";
  }
}

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

int gdn_conv_silu(const void* x, int64_t x_tok_stride, int32_t x_dt, void* y, int32_t y_dt,
                  const float* w, float* conv_state, int32_t B, int32_t T, int32_t C, int32_t W,
                  int32_t l2_channels, int32_t head_dim, float l2_eps, void* stream) {
  if (!x || !y || !w) return GDN_ERR_NULL;
  if (!dtype_ok(x_dt) || !dtype_ok(y_dt)) return GDN_ERR_DTYPE;
  if (B < 0 || T < 0 || C <= 0 || W < 1 || l2_channels < 0 || l2_channels > C)
    return GDN_ERR_SHAPE;
  if (W != 4) return GDN_ERR_UNSUPPORTED;
  if (C % 8 != 0 || x_tok_stride < C) return GDN_ERR_SHAPE;
  if (x_tok_stride % 8 != 0) return GDN_ERR_ALIGN;
  if (l2_channels > 0) {
    if (head_dim <= 0 || l2_channels % head_dim != 0) return GDN_ERR_SHAPE;
    if (head_dim != 128) return GDN_ERR_UNSUPPORTED;
  }
  if (!conv_grid_ok(B, T, C)) return GDN_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(w, 16) ||
      (conv_state && !aligned(conv_state, 16)))
    return GDN_ERR_ALIGN;
  if (B == 0 || T == 0) return GDN_OK;
  const size_t xbytes = ((size_t)((int64_t)B * T - 1) * x_tok_stride + C) * dsize(x_dt);
  const size_t ybytes = (size_t)B * T * C * dsize(y_dt);
  if (overlaps(y, ybytes, x, xbytes)) return GDN_ERR_SHAPE;  // y overlaps x
  return launch_status(gdn::launch_conv_silu(x, x_tok_stride, x_dt, y, y_dt, w, conv_state, B,
                                             T, C, l2_channels, l2_eps,
                                             static_cast<hipStream_t>(stream)));
}

size_t gdn_prefill_workspace_bytes(int32_t B, int32_t T, gdn_dims dims, int32_t qkv_dt,
                                   int32_t algo) {
  if (B <= 0 || T <= 0 || check_dims(dims) != GDN_OK) return 0;
  if (!uses_chunked(algo, qkv_dt)) return 0;
  return gdn::prefill_chunked_workspace_bytes(B, T, dims.n_qk_heads, dims.n_v_heads);
}

int gdn_prefill(const void* q, int64_t q_tok_stride, const void* k, int64_t k_tok_stride,
                const void* v, int64_t v_tok_stride, int32_t qkv_dt, const void* a,
                const void* b, int32_t gate_dt, const float* A_log, const float* dt_bias,
                const float* state_in, float* state_out, void* o, int32_t o_dt, int32_t B,
                int32_t T, gdn_dims dims, float q_scale, int32_t algo, void* workspace,
                size_t workspace_bytes, void* stream) {
  if (!A_log || !dt_bias) return GDN_ERR_NULL;
  if (T != 0 && (!q || !k || !v || !a || !b || !o)) return GDN_ERR_NULL;  // T == 0 reads none
  if (!dtype_ok(qkv_dt) || !dtype_ok(gate_dt) || !dtype_ok(o_dt)) return GDN_ERR_DTYPE;
  if (algo != GDN_ALGO_AUTO && algo != GDN_ALGO_SEQUENTIAL && algo != GDN_ALGO_CHUNKED)
    return GDN_ERR_SHAPE;
  int st = check_dims(dims);
  if (st != GDN_OK) return st;
  const int Hk = dims.n_qk_heads, Hv = dims.n_v_heads;
  if (B < 0 || T < 0) return GDN_ERR_SHAPE;
  if (q_tok_stride < (int64_t)Hk * 128 || k_tok_stride < (int64_t)Hk * 128 ||
      v_tok_stride < (int64_t)Hv * 128)
    return GDN_ERR_SHAPE;
  if ((int64_t)B * Hv * 8 > INT32_MAX || (int64_t)B * T > INT32_MAX) return GDN_ERR_SHAPE;
  if (q_tok_stride % 8 || k_tok_stride % 8 || v_tok_stride % 8) return GDN_ERR_ALIGN;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(a, dsize(gate_dt)) || !aligned(b, dsize(gate_dt)) || !aligned(A_log, 4) ||
      !aligned(dt_bias, 4) || (state_in && !aligned(state_in, 16)) ||
      (state_out && !aligned(state_out, 16)))
    return GDN_ERR_ALIGN;
  if (algo == GDN_ALGO_CHUNKED && qkv_dt != GDN_BF16) return GDN_ERR_UNSUPPORTED;
  const bool chunked = uses_chunked(algo, qkv_dt);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B == 0) return GDN_OK;
  if (chunked && T > 0) {
    const size_t need = gdn::prefill_chunked_workspace_bytes(B, T, Hk, Hv);
    if (workspace_bytes < need || (need > 0 && !workspace)) return GDN_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return GDN_ERR_ALIGN;
    return launch_status(gdn::launch_prefill_chunked(
        q, q_tok_stride, k, k_tok_stride, v, v_tok_stride, qkv_dt, qkv_dt, a, b, gate_dt, A_log,
        dt_bias, state_in, state_out, o, o_dt, B, T, nullptr, 0, Hk, Hv, q_scale, workspace, s));
  }
  // Sequential algorithm (also the T == 0 state pass-through).
  return launch_status(gdn::launch_prefill_sequential(
      q, q_tok_stride, k, k_tok_stride, v, v_tok_stride, qkv_dt, a, b, gate_dt, A_log, dt_bias,
      state_in, state_out, o, o_dt, B, T, nullptr, 0, Hk, Hv, q_scale, s));
}

int gdn_decode_rows(const void* q, int64_t q_row_stride, const void* k, int64_t k_row_stride,
                    const void* v, int64_t v_row_stride, int32_t qkv_dt, const void* a,
                    const void* b, int32_t gate_dt, const float* A_log, const float* dt_bias,
                    float* state, const int32_t* lengths, void* o, int32_t R, gdn_dims dims,
                    float q_scale, void* stream) {
  if (!q || !k || !v || !a || !b || !A_log || !dt_bias || !state || !o) return GDN_ERR_NULL;
  if (!dtype_ok(qkv_dt) || !dtype_ok(gate_dt)) return GDN_ERR_DTYPE;
  int st = check_dims(dims);
  if (st != GDN_OK) return st;
  const int Hk = dims.n_qk_heads, Hv = dims.n_v_heads;
  if (R < 0) return GDN_ERR_SHAPE;
  if (q_row_stride < (int64_t)Hk * 128 || k_row_stride < (int64_t)Hk * 128 ||
      v_row_stride < (int64_t)Hv * 128)
    return GDN_ERR_SHAPE;
  if ((int64_t)R * Hv * 8 > INT32_MAX) return GDN_ERR_SHAPE;  // eight workgroups per (row, head)
  if (q_row_stride % 8 || k_row_stride % 8 || v_row_stride % 8) return GDN_ERR_ALIGN;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(state, 16) || !aligned(a, dsize(gate_dt)) || !aligned(b, dsize(gate_dt)) ||
      !aligned(A_log, 4) || !aligned(dt_bias, 4) || (lengths && !aligned(lengths, 4)))
    return GDN_ERR_ALIGN;
  if (R == 0) return GDN_OK;
  return launch_status(gdn::launch_decode_rows(q, q_row_stride, k, k_row_stride, v, v_row_stride,
                                               qkv_dt, a, b, gate_dt, A_log, dt_bias, state,
                                               lengths, o, R, Hk, Hv, q_scale,
                                               static_cast<hipStream_t>(stream)));
}

int gdn_decode_rows_multi(const void* q, int64_t q_row_stride, int64_t q_tok_stride,
                          const void* k, int64_t k_row_stride, int64_t k_tok_stride,
                          const void* v, int64_t v_row_stride, int64_t v_tok_stride,
                          int32_t qkv_dt, const void* a, const void* b, int32_t gate_dt,
                          const float* A_log, const float* dt_bias, float* state,
                          float* snapshots, const int32_t* lengths, void* o, int32_t R,
                          int32_t K, gdn_dims dims, float q_scale, void* stream) {
  if (!q || !k || !v || !a || !b || !A_log || !dt_bias || !state || !o) return GDN_ERR_NULL;
  if (!dtype_ok(qkv_dt) || !dtype_ok(gate_dt)) return GDN_ERR_DTYPE;
  int st = check_dims(dims);
  if (st != GDN_OK) return st;
  const int Hk = dims.n_qk_heads, Hv = dims.n_v_heads;
  if (R < 0 || K < 0) return GDN_ERR_SHAPE;
  if (q_tok_stride < (int64_t)Hk * 128 || k_tok_stride < (int64_t)Hk * 128 ||
      v_tok_stride < (int64_t)Hv * 128 || q_row_stride < 0 || k_row_stride < 0 ||
      v_row_stride < 0)
    return GDN_ERR_SHAPE;
  if ((int64_t)R * Hv * 4 > INT32_MAX || (int64_t)R * K * Hv > INT32_MAX) return GDN_ERR_SHAPE;
  if (q_row_stride % 8 || k_row_stride % 8 || v_row_stride % 8 || q_tok_stride % 8 ||
      k_tok_stride % 8 || v_tok_stride % 8)
    return GDN_ERR_ALIGN;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(state, 16) || (snapshots && !aligned(snapshots, 16)) ||
      !aligned(a, dsize(gate_dt)) || !aligned(b, dsize(gate_dt)) || !aligned(A_log, 4) ||
      !aligned(dt_bias, 4) || (lengths && !aligned(lengths, 4)))
    return GDN_ERR_ALIGN;
  const size_t sbytes = (size_t)R * Hv * 128 * 128 * 4;
  if (snapshots && overlaps(snapshots, sbytes * K, state, sbytes)) return GDN_ERR_SHAPE;
  if (R == 0 || K == 0) return GDN_OK;
  return launch_status(gdn::launch_decode_rows_multi(
      q, q_row_stride, q_tok_stride, k, k_row_stride, k_tok_stride, v, v_row_stride,
      v_tok_stride, qkv_dt, a, b, gate_dt, A_log, dt_bias, state, snapshots, lengths, o, R, K, Hk,
      Hv, q_scale, static_cast<hipStream_t>(stream)));
}

int gdn_gated_rmsnorm(const void* x, const void* z, int64_t z_tok_stride, void* y, int32_t dt,
                      const float* w, int32_t N, int32_t H, int32_t D, float eps, void* stream) {
  if (!x || !z || !y || !w) return GDN_ERR_NULL;
  if (!dtype_ok(dt)) return GDN_ERR_DTYPE;
  if (N < 0 || H < 0 || D <= 0) return GDN_ERR_SHAPE;
  if (D != 128) return GDN_ERR_UNSUPPORTED;
  if (z_tok_stride < (int64_t)H * D) return GDN_ERR_SHAPE;
  if (z_tok_stride % 8 != 0) return GDN_ERR_ALIGN;
  const int64_t rows = (int64_t)N * H;
  if ((rows + 63) / 64 > INT32_MAX) return GDN_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(z, 16) || !aligned(y, 16) || !aligned(w, 16))
    return GDN_ERR_ALIGN;
  if (rows == 0) return GDN_OK;
  return launch_status(gdn::launch_gated_rmsnorm(x, z, z_tok_stride, y, dt, w, N, H, eps,
                                                 static_cast<hipStream_t>(stream)));
}

size_t gdn_prefill_slots_workspace_bytes(int32_t R, int32_t max_len, gdn_dims dims) {
  if (R <= 0 || max_len <= 0 || check_dims(dims) != GDN_OK) return 0;
  return gdn::prefill_chunked_workspace_bytes(R, max_len, dims.n_qk_heads, dims.n_v_heads);
}

int gdn_prefill_slots(const void* q, int64_t q_tok_stride, const void* k, int64_t k_tok_stride,
                      const void* v, int64_t v_tok_stride, int32_t qkv_dt, const void* a,
                      const void* b, int32_t gate_dt, const float* A_log, const float* dt_bias,
                      const int32_t* cu_seqlens, float* state, void* o, int32_t o_dt, int32_t R,
                      int32_t max_len, int32_t total_tokens, gdn_dims dims, float q_scale,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!A_log || !dt_bias || !cu_seqlens || !state) return GDN_ERR_NULL;
  if (total_tokens != 0 && (!q || !k || !v || !a || !b || !o)) return GDN_ERR_NULL;
  if (!dtype_ok(qkv_dt) || !dtype_ok(gate_dt) || !dtype_ok(o_dt)) return GDN_ERR_DTYPE;
  int st = check_dims(dims);
  if (st != GDN_OK) return st;
  const int Hk = dims.n_qk_heads, Hv = dims.n_v_heads;
  if (R < 0 || max_len < 0 || total_tokens < 0) return GDN_ERR_SHAPE;
  if (q_tok_stride < (int64_t)Hk * 128 || k_tok_stride < (int64_t)Hk * 128 ||
      v_tok_stride < (int64_t)Hv * 128)
    return GDN_ERR_SHAPE;
  if ((int64_t)R * Hv * 8 > INT32_MAX || (int64_t)R * ((max_len + 63) / 64) * Hv > INT32_MAX)
    return GDN_ERR_SHAPE;
  if (q_tok_stride % 8 || k_tok_stride % 8 || v_tok_stride % 8) return GDN_ERR_ALIGN;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(a, dsize(gate_dt)) || !aligned(b, dsize(gate_dt)) || !aligned(A_log, 4) ||
      !aligned(dt_bias, 4) || !aligned(cu_seqlens, 4) || !aligned(state, 16))
    return GDN_ERR_ALIGN;
  if (R == 0 || max_len == 0 || total_tokens == 0) return GDN_OK;  // every row is empty
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (qkv_dt == GDN_F32)  // f32 inputs: token by token in f32, in place
    return launch_status(gdn::launch_prefill_sequential(
        q, q_tok_stride, k, k_tok_stride, v, v_tok_stride, qkv_dt, a, b, gate_dt, A_log, dt_bias,
        state, state, o, o_dt, R, max_len, cu_seqlens, total_tokens, Hk, Hv, q_scale, s));
  const size_t need = gdn::prefill_chunked_workspace_bytes(R, max_len, Hk, Hv);
  if (workspace_bytes < need || !workspace) return GDN_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return GDN_ERR_ALIGN;
  return launch_status(gdn::launch_prefill_chunked(
      q, q_tok_stride, k, k_tok_stride, v, v_tok_stride, qkv_dt, qkv_dt, a, b, gate_dt, A_log,
      dt_bias, state, state, o, o_dt, R, max_len, cu_seqlens, total_tokens, Hk, Hv, q_scale,
      workspace, s));
}

size_t gdn_mixer_prefill_workspace_bytes(int32_t B, int32_t T, gdn_dims dims) {
  if (B <= 0 || T <= 0 || check_dims(dims) != GDN_OK) return 0;
  return mixer_ws(B, T, dims).total();
}

int gdn_mixer_prefill(const void* qkv, int64_t qkv_tok_stride, const void* z,
                      int64_t z_tok_stride, int32_t dt, const float* conv_w,
                      float* conv_state, const void* a, const void* b, int32_t gate_dt,
                      const float* A_log, const float* dt_bias, const float* norm_w,
                      const float* state_in, float* state_out, void* y, int32_t B, int32_t T,
                      gdn_dims dims, float q_scale, float l2_eps, float norm_eps,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!conv_w || !A_log || !dt_bias || !norm_w) return GDN_ERR_NULL;
  if (T != 0 && (!qkv || !z || !a || !b || !y)) return GDN_ERR_NULL;
  if (!dtype_ok(dt) || !dtype_ok(gate_dt)) return GDN_ERR_DTYPE;
  int st = check_dims(dims);
  if (st != GDN_OK) return st;
  const int Hk = dims.n_qk_heads, Hv = dims.n_v_heads;
  const int L2C = 2 * Hk * 128, C = L2C + Hv * 128;
  if (B < 0 || T < 0) return GDN_ERR_SHAPE;
  if ((int64_t)B * Hv * 8 > INT32_MAX || (int64_t)B * T > INT32_MAX) return GDN_ERR_SHAPE;
  if (!conv_grid_ok(B, T, C)) return GDN_ERR_SHAPE;
  if (T != 0 && (qkv_tok_stride < C || z_tok_stride < (int64_t)Hv * 128)) return GDN_ERR_SHAPE;
  if (qkv_tok_stride % 8 != 0 || z_tok_stride % 8 != 0) return GDN_ERR_ALIGN;
  if (!aligned(qkv, 16) || !aligned(z, 16) || !aligned(y, 16) || !aligned(conv_w, 16) ||
      (conv_state && !aligned(conv_state, 16)) || !aligned(a, dsize(gate_dt)) ||
      !aligned(b, dsize(gate_dt)) || !aligned(A_log, 4) || !aligned(dt_bias, 4) ||
      !aligned(norm_w, 16) || (state_in && !aligned(state_in, 16)) ||
      (state_out && !aligned(state_out, 16)))
    return GDN_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B == 0) return GDN_OK;
  if (T == 0)  // no tokens: conv history unchanged, the state passes through
    return launch_status(gdn::launch_prefill_sequential(
        nullptr, Hk * 128, nullptr, Hk * 128, nullptr, Hv * 128, dt, nullptr, nullptr, gate_dt,
        A_log, dt_bias, state_in, state_out, nullptr, dt, B, 0, nullptr, 0, Hk, Hv, q_scale,
        s));
  const MixerWs w = mixer_ws(B, T, dims);
  if (workspace_bytes < w.total() || !workspace) return GDN_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return GDN_ERR_ALIGN;
  const size_t ybytes = (size_t)B * T * Hv * 128 * dsize(dt);
  const size_t tokens = (size_t)B * T;
  const size_t zbytes = ((tokens - 1) * z_tok_stride + Hv * 128) * dsize(dt);
  const size_t qkvbytes = ((tokens - 1) * qkv_tok_stride + C) * dsize(dt);
  if (overlaps(y, ybytes, workspace, w.total()) || overlaps(y, ybytes, z, zbytes) ||
      overlaps(y, ybytes, qkv, qkvbytes))
    return GDN_ERR_SHAPE;
  if (dt == GDN_F32) {
    // f32 inputs keep f32 accuracy: the conv writes [B, T, C] f32 to the
    // workspace (B*T*C*4 bytes, less than the chunked layout's total), the
    // recurrence runs token by token in f32 on views of it, and the norm
    // runs in place on y.
    float* yc = static_cast<float*>(workspace);
    hipError_t e = gdn::launch_conv_silu(qkv, qkv_tok_stride, dt, yc, GDN_F32, conv_w,
                                         conv_state, B, T, C, L2C, l2_eps, s);
    if (e != hipSuccess) return GDN_ERR_LAUNCH;
    e = gdn::launch_prefill_sequential(yc, C, yc + Hk * 128, C, yc + L2C, C, GDN_F32, a, b,
                                       gate_dt, A_log, dt_bias, state_in, state_out, y, dt, B, T,
                                       nullptr, 0, Hk, Hv, q_scale, s);
    if (e != hipSuccess) return GDN_ERR_LAUNCH;
    return launch_status(gdn::launch_gated_rmsnorm(y, z, z_tok_stride, y, dt, norm_w,
                                                   (int64_t)B * T, Hv, norm_eps, s));
  }
  char* ws = static_cast<char*>(workspace);
  float* yqk = reinterpret_cast<float*>(ws);
  uint16_t* yv = reinterpret_cast<uint16_t*>(ws + w.qk_bytes);
  void* chunk_ws = ws + w.qk_bytes + w.v_bytes;
  hipError_t e = gdn::launch_conv_silu_split(qkv, qkv_tok_stride, dt, yqk, yv, conv_w,
                                             conv_state, B, T, C, L2C, l2_eps, s);
  if (e != hipSuccess) return GDN_ERR_LAUNCH;
  e = gdn::launch_prefill_chunked(yqk, L2C, yqk + Hk * 128, L2C, yv, Hv * 128, GDN_F32, GDN_BF16,
                                  a, b, gate_dt, A_log, dt_bias, state_in, state_out, y, dt, B, T,
                                  nullptr, 0, Hk, Hv, q_scale, chunk_ws, s);
  if (e != hipSuccess) return GDN_ERR_LAUNCH;
  return launch_status(gdn::launch_gated_rmsnorm(y, z, z_tok_stride, y, dt, norm_w,
                                                 (int64_t)B * T, Hv, norm_eps, s));
}

size_t gdn_gate_proj_workspace_bytes(int32_t M, int32_t K, int32_t H) {
  if (M <= 0 || K <= 0 || K % 32 != 0 || H <= 0 || H % 16 != 0 || H > 64) return 0;
  return round256(gdn::gate_proj_workspace_bytes(M, K, H));
}

int gdn_gate_proj(const void* x, int64_t x_ld, int32_t x_dt, const float* W_a,
                  const float* W_b, float* a, float* b, int64_t ab_ld, int32_t M, int32_t K,
                  int32_t H, void* workspace, size_t workspace_bytes, void* stream) {
  if (M < 0 || K <= 0 || H <= 0) return GDN_ERR_SHAPE;
  if (!dtype_ok(x_dt)) return GDN_ERR_DTYPE;
  if (x_dt != GDN_BF16 || H > 64) return GDN_ERR_UNSUPPORTED;
  if (K % 32 != 0 || H % 16 != 0 || x_ld < K || ab_ld < H) return GDN_ERR_SHAPE;
  if (M == 0) return GDN_OK;
  if (!x || !W_a || !W_b || !a || !b) return GDN_ERR_NULL;
  if ((int64_t)M * (2 * H / 4) / 256 + 1 > INT32_MAX) return GDN_ERR_SHAPE;
  if (x_ld % 8 != 0 || !aligned(x, 16) || !aligned(W_a, 16) || !aligned(W_b, 16))
    return GDN_ERR_ALIGN;
  const size_t need = gdn::gate_proj_workspace_bytes(M, K, H);
  if (workspace_bytes < need || (need > 0 && !workspace)) return GDN_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 256)) return GDN_ERR_ALIGN;
  const size_t xbytes = ((size_t)(M - 1) * x_ld + K) * 2;
  const size_t abytes = ((size_t)(M - 1) * ab_ld + H) * 4;
  if (overlaps(a, abytes, x, xbytes) || overlaps(b, abytes, x, xbytes)) return GDN_ERR_SHAPE;
  if (need > 0 && (overlaps(a, abytes, workspace, need) || overlaps(b, abytes, workspace, need)))
    return GDN_ERR_SHAPE;
  return launch_status(gdn::launch_gate_proj(static_cast<const uint16_t*>(x), x_ld, W_a, W_b, a,
                                             b, ab_ld, M, K, H, workspace,
                                             static_cast<hipStream_t>(stream)));
}

size_t gdn_linear_workspace_bytes(void) { return (size_t)32 << 20; }

static int linear_call(const void* x, int64_t x_ld, const void* W, int64_t w_ld, void* y,
                       int64_t y_ld, int32_t y_dt, int32_t M, int32_t N, int32_t K,
                       void* workspace, size_t workspace_bytes, bool tune, void* stream) {
  if (M < 0 || N <= 0 || K <= 0) return GDN_ERR_SHAPE;
  if (!dtype_ok(y_dt)) return GDN_ERR_DTYPE;
  if (x_ld < K || w_ld < K || y_ld < N) return GDN_ERR_SHAPE;
  if (M == 0) return GDN_OK;
  if (!x || !W || !y) return GDN_ERR_NULL;
  if (workspace_bytes > 0 && !workspace) return GDN_ERR_WORKSPACE;
  if (x_ld % 8 || w_ld % 8 || y_ld % 8) return GDN_ERR_ALIGN;
  if (!aligned(x, 16) || !aligned(W, 16) || !aligned(y, 16)) return GDN_ERR_ALIGN;
  if (workspace && !aligned(workspace, 256)) return GDN_ERR_ALIGN;
  const size_t xbytes = ((size_t)(M - 1) * x_ld + K) * 2;
  const size_t wbytes = ((size_t)(N - 1) * w_ld + K) * 2;
  const size_t ybytes = ((size_t)(M - 1) * y_ld + N) * dsize(y_dt);
  if (overlaps(y, ybytes, x, xbytes) || overlaps(y, ybytes, W, wbytes)) return GDN_ERR_SHAPE;
  if (workspace_bytes > 0 &&
      (overlaps(workspace, workspace_bytes, x, xbytes) ||
       overlaps(workspace, workspace_bytes, W, wbytes) ||
       overlaps(workspace, workspace_bytes, y, ybytes)))
    return GDN_ERR_SHAPE;
  switch (gdn::launch_linear(static_cast<const uint16_t*>(x), x_ld,
                             static_cast<const uint16_t*>(W), w_ld, y, y_ld, y_dt, M, N, K,
                             workspace, workspace_bytes, tune, static_cast<hipStream_t>(stream))) {
    case gdn::LinearStatus::kOk: return GDN_OK;
    case gdn::LinearStatus::kNoAlgorithm:
    case gdn::LinearStatus::kBadLibrary: return GDN_ERR_UNSUPPORTED;
    default: return GDN_ERR_LAUNCH;
  }
}

int gdn_linear(const void* x, int64_t x_ld, const void* W, int64_t w_ld, void* y, int64_t y_ld,
               int32_t y_dt, int32_t M, int32_t N, int32_t K, void* workspace,
               size_t workspace_bytes, void* stream) {
  return linear_call(x, x_ld, W, w_ld, y, y_ld, y_dt, M, N, K, workspace, workspace_bytes, false,
                     stream);
}

int gdn_linear_tune(const void* x, int64_t x_ld, const void* W, int64_t w_ld, void* y,
                    int64_t y_ld, int32_t y_dt, int32_t M, int32_t N, int32_t K, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return linear_call(x, x_ld, W, w_ld, y, y_ld, y_dt, M, N, K, workspace, workspace_bytes, true,
                     stream);
}

int gdn_linear_kernel(int32_t M, int32_t N, int32_t K, int64_t x_ld, int64_t w_ld,
                      size_t workspace_bytes) {
  if (M < 0 || N <= 0 || K <= 0 || x_ld < K || w_ld < K) return -GDN_ERR_SHAPE;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return -GDN_ERR_LAUNCH;
  const int width = gdn::gemm_bf16_width(M, N, K, x_ld, w_ld, cus);
  if (width) return width * 32;
  return gdn::gemm_fewrow_splits(M, N, K, x_ld, w_ld, cus, workspace_bytes) ? 64 : 0;
}

}  // extern "C"
