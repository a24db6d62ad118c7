// Internal launchers, one per kernel family.  Arguments are already validated
// by the C ABI layer (api.hip); dtype codes: 0 = f32, 1 = bf16.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Conv workgroup shape: CONV_TB tokens (measured best of 8, 16, 32, 64) by
// CONV_THREADS threads of 8 channels each.
constexpr int CONV_TB = 8;
constexpr int CONV_THREADS = 256;

// x's token (b, t) starts at (b*T + t) * x_ts elements; y is [B, T, C].
hipError_t launch_conv_silu(const void* x, int64_t x_ts, int x_dt, void* y, int y_dt,
                            const float* w, float* conv_state, int B, int T, int C,
                            int l2_channels, float l2_eps, hipStream_t stream);

// The same conv with two outputs: channels below l2_channels in f32 to yqk
// [B, T, l2_channels], the others in bf16 to yv [B, T, C - l2_channels].
hipError_t launch_conv_silu_split(const void* x, int64_t x_ts, int x_dt, float* yqk,
                                  uint16_t* yv, const float* w, float* conv_state, int B, int T,
                                  int C, int l2_channels, float l2_eps, hipStream_t stream);

// x, y [N, H, 128] contiguous; z's token n starts at n * z_ts elements.
hipError_t launch_gated_rmsnorm(const void* x, const void* z, int64_t z_ts, void* y, int dt,
                                const float* w, int64_t N, int H, float eps, hipStream_t stream);

hipError_t launch_decode_rows(const void* q, int64_t q_rs, const void* k, int64_t k_rs,
                              const void* v, int64_t v_rs, int qkv_dt, const void* a,
                              const void* b, int gate_dt, const float* A_log,
                              const float* dt_bias, float* state, const int32_t* lengths, void* o,
                              int R, int Hk, int Hv, float q_scale, hipStream_t stream);

// K tokens per row; snapshots (may be NULL) [R, K, Hv, 128, 128].
hipError_t launch_decode_rows_multi(const void* q, int64_t q_rs, int64_t q_ts, const void* k,
                                    int64_t k_rs, int64_t k_ts, const void* v, int64_t v_rs,
                                    int64_t v_ts, int qkv_dt, const void* a, const void* b,
                                    int gate_dt, const float* A_log, const float* dt_bias,
                                    float* state, float* snapshots, const int32_t* lengths,
                                    void* o, int R, int K, int Hk, int Hv, float q_scale,
                                    hipStream_t stream);

// Token-by-token f32 prefill.  With cu NULL the B rows are T tokens each at
// stride T; with cu (device, [B + 1] offsets into a packed axis of `total`
// tokens) row b is tokens [cu[b], cu[b+1]), at most T of them.  state_in may
// equal state_out.
hipError_t launch_prefill_sequential(const void* q, int64_t q_ts, const void* k, int64_t k_ts,
                                     const void* v, int64_t v_ts, int qkv_dt, const void* a,
                                     const void* b, int gate_dt, const float* A_log,
                                     const float* dt_bias, const float* state_in,
                                     float* state_out, void* o, int o_dt, int B, int T,
                                     const int32_t* cu, int total, int Hk, int Hv, float q_scale,
                                     hipStream_t stream);

// Chunked (WY/UT form) prefill on bf16 MFMA.  q and k share qk_dt; v has
// its own dtype (f32 q/k with bf16 v is the whole mixer's layout).  With cu
// NULL the B rows are T tokens each at stride T; with cu (device, [B + 1]
// offsets into a packed axis of `total` tokens) row b is tokens
// [cu[b], cu[b+1]), at most T of them.
size_t prefill_chunked_workspace_bytes(int B, int T, int Hk, int Hv);

hipError_t launch_prefill_chunked(const void* q, int64_t q_ts, const void* k, int64_t k_ts,
                                  const void* v, int64_t v_ts, int qk_dt, int v_dt, const void* a,
                                  const void* b, int gate_dt, const float* A_log,
                                  const float* dt_bias, const float* state_in, float* state_out,
                                  void* o, int o_dt, int B, int T, const int32_t* cu, int total,
                                  int Hk, int Hv, float q_scale, void* workspace,
                                  hipStream_t stream);

// Gate projections with f32 weights: a[m][h] = sum_k x[m][k] Wa[h][k], b
// likewise; x bf16 [M][x_ld], Wa and Wb f32 [H][K], a and b f32 [M][ab_ld].
// K % 32 == 0, H % 16 == 0, H <= 64.  The workspace (256-byte aligned) holds
// the partial sums over K ranges; gate_proj_workspace_bytes gives its size.
size_t gate_proj_workspace_bytes(int M, int K, int H);
hipError_t launch_gate_proj(const uint16_t* x, int64_t x_ld, const float* Wa, const float* Wb,
                            float* a, float* b, int64_t ab_ld, int M, int K, int H, void* workspace,
                            hipStream_t stream);

// The library's bf16 GEMM y[M][N] = x[M][K] W[N][K]^T (gemm.hip): the block
// width code (5, 6, 8 or 10: 160, 192, 256 or 320 outputs) that suits the
// shape on a GPU of `cus` CUs, or 0 when the shape should go to hipBLASLt.
int gemm_bf16_width(int M, int N, int K, int64_t x_ld, int64_t w_ld, int cus);
hipError_t launch_gemm_bf16(const uint16_t* x, int64_t x_ld, const uint16_t* W, int64_t w_ld,
                            void* y, int64_t y_ld, int y_dt, int M, int N, int K, int width,
                            hipStream_t stream);
// Its few-row form for M <= 64: the number of equal K ranges (1 = straight to
// y; more need splits * M * N * 4 bytes of workspace for the partial sums)
// that suits the shape, or 0 when the shape should go elsewhere.
int gemm_fewrow_splits(int M, int N, int K, int64_t x_ld, int64_t w_ld, int cus,
                       size_t ws_bytes);
hipError_t launch_gemm_fewrow(const uint16_t* x, int64_t x_ld, const uint16_t* W, int64_t w_ld,
                              void* y, int64_t y_ld, int y_dt, int M, int N, int K, int splits,
                              void* workspace, hipStream_t stream);

// bf16 linear layer y[M][N] = x[M][K] W[N][K]^T, f32 accumulation, y in bf16
// (y_dt 1) or f32 (y_dt 0): the library's tiled GEMM when gemm_bf16_width
// picks a width, else its few-row form when gemm_fewrow_splits allows it,
// else hipBLASLt.  `tune` times hipBLASLt's candidates and the library's
// kernel for the shape (synchronises) and keeps the fastest for later calls
// of the same shape.
enum class LinearStatus { kOk, kNoAlgorithm, kBadLibrary, kLaunchFailed };
LinearStatus launch_linear(const uint16_t* x, int64_t x_ld, const uint16_t* W, int64_t w_ld,
                           void* y, int64_t y_ld, int y_dt, int M, int N, int K, void* workspace,
                           size_t workspace_bytes, bool tune, hipStream_t stream);

}  // namespace gdn
