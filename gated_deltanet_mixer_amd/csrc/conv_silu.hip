// Depthwise causal conv (width 4) + silu over the q|k|v channels, with the L2
// normalisation of each q and k head fused in, and the per-row conv history
// read and rewritten in f32 ("Qwen3.8 27B" model card, Gated DeltaNet bullet
// and state paragraph; llm-arch-viz module tree: conv1d 10240x1x4, no bias).
//
// y[b,t,c] = silu(sum_i w[c,i] * xhat[b,t+i,c]),  xhat = [hist (3 rows); x],
// then for c < l2_channels each head_dim group of y is divided by
// sqrt(sum of squares + l2_eps).  hist_out = the last 3 rows of xhat.
//
// Input: token (b, t) of x starts at (b*T + t) * x_ts (a view into a wider
// buffer, such as the [T, 16384] output of one in_proj_qkvz product, is
// read in place).  Output: channels below l2_channels go to ya (row stride
// ya_stride), the others to yb at channel c - l2_channels (row stride
// yb_stride), each in its own dtype.  The plain call points both at one
// [B, T, C] buffer; the whole mixer keeps q|k in f32 and v in bf16 (the
// chunked prefill rounds v to bf16 anyway, so the bf16 copy changes no
// result).
//
// Mapping: one thread owns 8 consecutive channels (one 16-byte bf16 load per
// token) and walks CONV_TB consecutive tokens, keeping the previous 3 inputs
// in registers, so every input element is read once (plus a 3-token halo per
// block, served from L2: the block before it ran on the same XCD).  A
// 128-channel head is 16 lanes, so the L2 sum is a DPP row reduction.  HBM-bound: one read of x and one write of y.
#include "common.hpp"
#include "launch.hpp"

namespace gdn {


// A row piece of 8 inputs as loaded (packed bf16 or two float4), unpacked
// only when used, which keeps the loads in flight cheap in registers.
template <typename TX> struct Raw8;
template <> struct Raw8<uint16_t> {
  u16x8 v;
  __device__ void load(const uint16_t* p) { v = *reinterpret_cast<const u16x8*>(p); }
  __device__ float operator[](int i) const { return bf2f(v[i]); }
};
template <> struct Raw8<float> {
  float4 a, b;
  __device__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ float operator[](int i) const {
    const float r[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    return r[i];
  }
};

// Streaming (non-temporal) stores of 8 outputs: the whole mixer's conv output
// is read once by the prep, and keeping it out of the last-level cache leaves
// that to the prep's workspace, which the chain reads next.
__device__ __forceinline__ void store8_stream(float* p, const float* in) {
  __builtin_nontemporal_store(f32x4{in[0], in[1], in[2], in[3]}, reinterpret_cast<f32x4*>(p));
  __builtin_nontemporal_store(f32x4{in[4], in[5], in[6], in[7]}, reinterpret_cast<f32x4*>(p + 4));
}
__device__ __forceinline__ void store8_stream(uint16_t* p, const float* in) {
  u16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = f2bf(in[i]);
  __builtin_nontemporal_store(v, reinterpret_cast<u16x8*>(p));
}

template <typename TX, typename TYA, typename TYB, bool kStream>
__global__ __launch_bounds__(CONV_THREADS) void conv_silu_kernel(
    const TX* __restrict__ x, int64_t x_ts, TYA* __restrict__ ya, int64_t ya_stride,
    TYB* __restrict__ yb, int64_t yb_stride, const float* __restrict__ w, float* conv_state,
    int nb, int Tlen, int C, int l2_channels, float l2_eps) {
  // Workgroups whose ids agree mod 8 share an XCD; each XCD takes a
  // contiguous run of (batch, token block, channel block) so a block's 3-row
  // halo was read into the same L2 by its neighbour.
  const int nx = (C + CONV_THREADS * 8 - 1) / (CONV_THREADS * 8);
  const int ny = (Tlen + CONV_TB - 1) / CONV_TB;
  const int total = nx * ny * nb;  // < 2^31 (checked on the host)
  const int per = (total + 7) / 8;
  const int lin = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lin >= total) return;
  const int bx = lin % nx, by = (lin / nx) % ny;
  const int b = lin / (nx * ny);
  const int t0 = by * CONV_TB;
  const int t1 = min(Tlen, t0 + CONV_TB);
  const int c0 = (bx * CONV_THREADS + threadIdx.x) * 8;
  if (c0 >= C) return;  // C % 8 == 0; a 16-lane head group is all in or all out

  // Row bases are uniform; the thread's channel offset is added last, so the
  // loads and stores take a scalar base and one per-thread offset.
  const TX* xrows = x + (int64_t)b * Tlen * x_ts;
  const TX* xb = xrows + (uint32_t)c0;
  const bool l2 = c0 < l2_channels;  // uniform over a 16-lane head group
  TYA* yarows = ya + (int64_t)b * Tlen * ya_stride;
  TYB* ybrows = yb + (int64_t)b * Tlen * yb_stride;
  const uint32_t ca = (uint32_t)c0, cb = (uint32_t)(c0 - l2_channels);

  float wt[4][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 wv = *reinterpret_cast<const float4*>(w + (int64_t)(c0 + i) * 4);
    wt[0][i] = wv.x; wt[1][i] = wv.y; wt[2][i] = wv.z; wt[3][i] = wv.w;
  }

  // h[j] = xhat row (t0 + j) = input at token t0 - 3 + j.
  float h[3][8];
  if (t0 == 0) {
    float* cs = conv_state ? conv_state + (int64_t)b * 3 * C + c0 : nullptr;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      if (cs) load8(cs + (int64_t)j * C, h[j]);
      else {
#pragma unroll
        for (int i = 0; i < 8; ++i) h[j][i] = 0.0f;
      }
    }
    // The first token block owns the history update, so an in/out buffer is
    // read before it is written and by the same thread.
    if (cs) {
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int r = Tlen + j;  // xhat row
        float nv[8];
        if (r < 3) {
#pragma unroll
          for (int i = 0; i < 8; ++i) nv[i] = h[r][i];
        } else {
          load8(xb + (int64_t)(r - 3) * x_ts, nv);
        }
        store8(cs + (int64_t)j * C, nv);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 3; ++j) load8(xb + (int64_t)(t0 - 3 + j) * x_ts, h[j]);
  }

  constexpr int U = 8;  // loads in flight per thread
  for (int t = t0; t < t1; t += U) {
    Raw8<TX> xs[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (t + u < t1) xs[u].load(xrows + (int64_t)(t + u) * x_ts + ca);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t + u < t1) {
        float yv[8];
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float acc = wt[0][i] * h[0][i];
          acc = fmaf(wt[1][i], h[1][i], acc);
          acc = fmaf(wt[2][i], h[2][i], acc);
          acc = fmaf(wt[3][i], xs[u][i], acc);
          yv[i] = silu_f(acc);
          ss = fmaf(yv[i], yv[i], ss);
        }
        if (l2) {
          ss = sum16(ss);
          const float r = rsqrtf(ss + l2_eps);
#pragma unroll
          for (int i = 0; i < 8; ++i) yv[i] *= r;
        }
        if constexpr (kStream) {
          if (l2) store8_stream(yarows + (int64_t)(t + u) * ya_stride + ca, yv);
          else store8_stream(ybrows + (int64_t)(t + u) * yb_stride + cb, yv);
        } else {
          if (l2) store8(yarows + (int64_t)(t + u) * ya_stride + ca, yv);
          else store8(ybrows + (int64_t)(t + u) * yb_stride + cb, yv);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          h[0][i] = h[1][i];
          h[1][i] = h[2][i];
          h[2][i] = xs[u][i];
        }
      }
    }
  }
}

template <typename TX, typename TYA, typename TYB, bool kStream = false>
static void launch_conv_t(const void* x, int64_t x_ts, void* ya, int64_t ya_stride, void* yb,
                          int64_t yb_stride, const float* w, float* conv_state, int B, int T,
                          int C, int l2_channels, float l2_eps, hipStream_t stream) {
  const int64_t total = (int64_t)((C + CONV_THREADS * 8 - 1) / (CONV_THREADS * 8)) *
                        ((T + CONV_TB - 1) / CONV_TB) * B;
  dim3 grid((unsigned)(((total + 7) / 8) * 8));
  hipLaunchKernelGGL((conv_silu_kernel<TX, TYA, TYB, kStream>), grid, dim3(CONV_THREADS), 0, stream,
                     (const TX*)x, x_ts, (TYA*)ya, ya_stride, (TYB*)yb, yb_stride, w,
                     conv_state, B, T, C, l2_channels, l2_eps);
}

hipError_t launch_conv_silu(const void* x, int64_t x_ts, int x_dt, void* y, int y_dt,
                            const float* w, float* conv_state, int B, int T, int C,
                            int l2_channels, float l2_eps, hipStream_t stream) {
  // One [B, T, C] output: the second part starts l2_channels into each row.
  const size_t ds = y_dt == 1 ? 2 : 4;
  void* yb = static_cast<char*>(y) + (size_t)l2_channels * ds;
  if (x_dt == 1 && y_dt == 1)
    launch_conv_t<uint16_t, uint16_t, uint16_t>(x, x_ts, y, C, yb, C, w, conv_state, B, T, C,
                                                l2_channels, l2_eps, stream);
  else if (x_dt == 1)
    launch_conv_t<uint16_t, float, float>(x, x_ts, y, C, yb, C, w, conv_state, B, T, C,
                                          l2_channels, l2_eps, stream);
  else if (y_dt == 1)
    launch_conv_t<float, uint16_t, uint16_t>(x, x_ts, y, C, yb, C, w, conv_state, B, T, C,
                                             l2_channels, l2_eps, stream);
  else
    launch_conv_t<float, float, float>(x, x_ts, y, C, yb, C, w, conv_state, B, T, C,
                                       l2_channels, l2_eps, stream);
  return hipGetLastError();
}

hipError_t launch_conv_silu_split(const void* x, int64_t x_ts, int x_dt, float* yqk,
                                  uint16_t* yv, const float* w, float* conv_state, int B, int T,
                                  int C, int l2_channels, float l2_eps, hipStream_t stream) {
  if (x_dt == 1)
    launch_conv_t<uint16_t, float, uint16_t, true>(x, x_ts, yqk, l2_channels, yv,
                                                   C - l2_channels, w, conv_state, B, T, C,
                                                   l2_channels, l2_eps, stream);
  else
    launch_conv_t<float, float, uint16_t, true>(x, x_ts, yqk, l2_channels, yv, C - l2_channels,
                                                w, conv_state, B, T, C, l2_channels, l2_eps,
                                                stream);
  return hipGetLastError();
}

}  // namespace gdn
