// Gated RMSNorm per (token, head): y = x / sqrt(mean(x^2) + eps) * (1 + w) * silu(z)
// ("Qwen3.8 27B" model card: head outputs RMS-normalised and gated by silu(z);
// "Norms": scale 1 + w, computed in f32; llm-arch-viz: RMSNormGated of width
// 128 shared by all heads, eps 1e-06).
//
// Mapping: a 128-wide head row is 16 lanes x 8 elements (16-byte bf16 loads);
// the mean of squares is a DPP row reduction.  Each 16-lane group handles
// NORM_ROWS rows with all loads issued first.  HBM-bound: read x and z once,
// write y once.  y may equal x (the whole mixer normalises its output in
// place), so x and y are not declared restrict: each lane reads its elements
// of a row before it writes them, and no lane touches another lane's.  x and
// y are [N, H, 128] contiguous; z's token n starts at n * z_ts (a view into
// a wider buffer, such as one in_proj_qkvz product's output, is read in
// place).
#include "common.hpp"
#include "launch.hpp"

namespace gdn {

constexpr int NORM_THREADS = 256;
constexpr int NORM_ROWS = 4;  // rows per 16-lane group
constexpr int NORM_ROWS_PER_WG = NORM_THREADS / 16 * NORM_ROWS;

template <typename T>
__global__ __launch_bounds__(NORM_THREADS) void gated_rmsnorm_kernel(
    const T* x, const T* __restrict__ z, int64_t z_ts, int H, T* y,
    const float* __restrict__ w, int64_t rows, float eps) {
  const int lane16 = threadIdx.x & 15;
  const int grp = threadIdx.x >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * NORM_ROWS_PER_WG + grp * NORM_ROWS;
  float wp[8];
  load8(w + lane16 * 8, wp);
#pragma unroll
  for (int i = 0; i < 8; ++i) wp[i] += 1.0f;

  float xv[NORM_ROWS][8], zv[NORM_ROWS][8];
#pragma unroll
  for (int r = 0; r < NORM_ROWS; ++r) {
    if (row0 + r < rows) {
      load8(x + (row0 + r) * 128 + lane16 * 8, xv[r]);
      const int64_t n = (row0 + r) / H;
      load8(z + n * z_ts + (row0 + r - n * H) * 128 + lane16 * 8, zv[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < NORM_ROWS; ++r) {
    if (row0 + r < rows) {  // uniform over the 16-lane group
      float ss = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(xv[r][i], xv[r][i], ss);
      ss = sum16(ss);
      const float inv = rsqrtf(ss * (1.0f / 128.0f) + eps);
      float out[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = xv[r][i] * inv * wp[i] * silu_f(zv[r][i]);
      store8(y + (row0 + r) * 128 + lane16 * 8, out);
    }
  }
}

hipError_t launch_gated_rmsnorm(const void* x, const void* z, int64_t z_ts, void* y, int dt,
                                const float* w, int64_t N, int H, float eps, hipStream_t stream) {
  const int64_t rows = N * H;
  const int64_t nwg = (rows + NORM_ROWS_PER_WG - 1) / NORM_ROWS_PER_WG;
  if (dt == 1) {
    hipLaunchKernelGGL(gated_rmsnorm_kernel<uint16_t>, dim3((unsigned)nwg), dim3(NORM_THREADS), 0,
                       stream, (const uint16_t*)x, (const uint16_t*)z, z_ts, H, (uint16_t*)y, w,
                       rows, eps);
  } else {
    hipLaunchKernelGGL(gated_rmsnorm_kernel<float>, dim3((unsigned)nwg), dim3(NORM_THREADS), 0,
                       stream, (const float*)x, (const float*)z, z_ts, H, (float*)y, w, rows,
                       eps);
  }
  return hipGetLastError();
}

}  // namespace gdn
