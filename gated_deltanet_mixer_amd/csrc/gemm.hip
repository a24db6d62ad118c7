// bf16 linear layers y = x W^T on MFMA, for the projections on either side of
// the mixer ("Qwen/Qwen3.8-27B" architecture viewer, module tree: in_proj_qkv
// 5120->10240, in_proj_z 5120->6144, out_proj 6144->5120; a Linear layer
// stores W as [out][in], so both operands are contiguous along k).
//
// y[M][N] = sum_k x[M][k] W[N][k] with f32 accumulation of exact bf16
// products (v_mfma_f32_16x16x32_bf16), one rounding to y's dtype.
//
// A workgroup computes a block of 256 x rows by BN = 32 NA W rows (NA = 5,
// 6, 8 or 10: 160 to 320 outputs); eight waves, two per SIMD, each own 64 x
// rows by 16 NA W rows (NA x 4 accumulator tiles of 16 x 16).  k advances in
// stages of 64 through two LDS buffers: the next stage's rows go from global
// memory straight into LDS (buffer loads with the LDS bit, 1 KB per wave
// instruction) while the current one is multiplied.  Rows are 128 bytes in
// LDS, their eight 16-byte chunks stored at chunk ^ (row & 7), so that each
// fragment read (16 rows, one chunk each) touches every bank once.  A stage's
// two 32-wide halves are read into registers before the first half's MFMAs
// (both halves for NA <= 8; one half at a time for NA = 10, whose 160
// accumulators leave room for one).  x rows at or past M lie outside the x
// buffer resource's range and load as zeros; their outputs are not stored.
//
// The width is picked per shape so that the tiles fill whole rounds of the
// GPU's CUs: the three prefill shapes at 4096 tokens take 512, 512 and 256
// tiles (in_proj_qkv and out_proj at 320 wide, in_proj_z at 192).  Measured
// against the hipBLASLt plan (tuned) in the same process at 4096 tokens:
// in_proj_qkv 325 vs 366 us, in_proj_z 232 vs 234 us, out_proj 202 vs 210 us.
//
// A few-row form for M <= 64 (a decode step's rows) follows the tiled one:
// a weight stream split over K where the weight blocks alone are too few.
#include <hip/hip_runtime.h>

#include "chunk_common.hpp"
#include "launch.hpp"

namespace gdn {

namespace {

using chunk::mfma16;

constexpr int GM_ROWS = 256;   // x rows per block
constexpr int GK = 64;         // k per stage
constexpr int G_THREADS = 512;

template <typename TY>
__device__ __forceinline__ void store4(TY* p, const f32x4& v);
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, const f32x4& v) {
  u16x4 o;
  o[0] = f2bf(v[0]);
  o[1] = f2bf(v[1]);
  o[2] = f2bf(v[2]);
  o[3] = f2bf(v[3]);
  *reinterpret_cast<u16x4*>(p) = o;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, const f32x4& v) {
  *reinterpret_cast<f32x4*>(p) = v;
}

template <int NA, typename TY>
__global__ __launch_bounds__(G_THREADS) void gemm_bf16_kernel(
    const uint16_t* __restrict__ x, int64_t x_ld, const uint16_t* __restrict__ W, int64_t w_ld,
    TY* __restrict__ y, int64_t y_ld, int M, int K, int tiles_m, int tiles_n) {
  constexpr int BN = 32 * NA;
  // One array: buffer b holds W's rows at b*LB and x's rows at b*LB + BN*GK.
  // (With an array per operand the compiler cannot tell the loads into one
  // buffer from the reads of the other and waits for every load in flight.)
  constexpr int LB = (BN + GM_ROWS) * GK;
  __shared__ __attribute__((aligned(16))) uint16_t Ls[2 * LB];

  // Tiles are dealt to the 8 XCDs in contiguous runs (ids that agree mod 8
  // share an XCD); within a run, groups of 4 x-row blocks walk W's blocks,
  // so an XCD's L2 serves each W block to 4 tiles and each x block to many.
  const int ntiles = tiles_m * tiles_n;
  const int per = (ntiles + 7) / 8;
  const int t = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (t >= ntiles) return;
  constexpr int GROUP = 4;
  const int gsize = GROUP * tiles_n;
  const int g = t / gsize, first_m = g * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (t % gsize) % gsz;
  const int tn = (t % gsize) / gsz;
  const int m0 = __builtin_amdgcn_readfirstlane(tm * GM_ROWS);
  const int n0 = __builtin_amdgcn_readfirstlane(tn * BN);

  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wn = w & 1, wm = w >> 1;

  // Loads: a wave instruction fills 8 rows (1 KB); lane l writes row l / 8,
  // slot l % 8, which holds logical chunk (l % 8) ^ (l / 8).  W's BN / 8
  // instructions are dealt NA / 2 to a wave when that is whole, else in turn;
  // wave w fills x rows 32 w .. 32 w + 31.
  typedef __attribute__((address_space(3))) void lds_t;
  const int lrow = lane >> 3, lch = (lane & 7) ^ lrow;
  const int xrows = min(M - m0, GM_ROWS);
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + (int64_t)n0 * w_ld), (short)0,
      __builtin_amdgcn_readfirstlane((int)(BN * 2 * (int)w_ld)), 0x00020000);
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(x + (int64_t)m0 * x_ld), (short)0,
      __builtin_amdgcn_readfirstlane((int)(xrows * 2 * (int)x_ld)), 0x00020000);
  constexpr int WQ = BN / 8;
  constexpr bool kWhole = WQ % 8 == 0;
  const uint32_t wo = (uint32_t)(((kWhole ? w * (WQ / 8) * 8 : 0) + lrow) * w_ld * 2 + lch * 16);
  const uint32_t xo = (uint32_t)((w * 32 + lrow) * x_ld * 2 + lch * 16);
  auto load_stage = [&](int buf, int k0) {
#pragma unroll
    for (int j = 0; j < (WQ + 7) / 8; ++j) {
      const int q = kWhole ? w * (WQ / 8) + j : w + 8 * j;
      if (kWhole || q < WQ)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wres, (lds_t*)&Ls[buf * LB + q * 8 * GK], 16, wo,
            (uint32_t)(k0 * 2 + (kWhole ? j : q) * 16 * w_ld), 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xres, (lds_t*)&Ls[buf * LB + BN * GK + (w * 32 + 8 * j) * GK], 16, xo,
          (uint32_t)(k0 * 2 + j * 16 * x_ld), 0, 0);
  };

  // Fragment i of half s: row base + 16 i + li, logical chunk 4 s + lg, which
  // sits at (4 s + lg) ^ (li & 7).  A operand: W rows (outputs n), B operand:
  // x rows (tokens m), so a lane's four results are four consecutive n.
  const int sw = li & 7;
  const int arow = (wn * 16 * NA + li) * GK, brow = BN * GK + (wm * 64 + li) * GK;

  f32x4 acc[NA][4];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = K / GK;
  load_stage(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): stage 0 is in LDS
  chunk::lds_barrier();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) load_stage(buf ^ 1, (kt + 1) * GK);
    const uint16_t* L = &Ls[buf * LB];
    if constexpr (NA <= 8) {
      bf16x8 fa[2][NA], fb[2][4];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int pc = ((4 * s + lg) ^ sw) * 8;
#pragma unroll
        for (int i = 0; i < NA; ++i) fa[s][i] = chunk::ld_frag(L + arow + i * 16 * GK + pc);
#pragma unroll
        for (int i = 0; i < 4; ++i) fb[s][i] = chunk::ld_frag(L + brow + i * 16 * GK + pc);
        if (s == 0) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the first half is in
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[a][b] = mfma16(fa[s][a], fb[s][b], acc[a][b]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 fa[NA], fb[4];
        const int pc = ((4 * s + lg) ^ sw) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) fb[i] = chunk::ld_frag(L + brow + i * 16 * GK + pc);
#pragma unroll
        for (int i = 0; i < NA; ++i) fa[i] = chunk::ld_frag(L + arow + i * 16 * GK + pc);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[a][b] = mfma16(fa[a], fb[b], acc[a][b]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next stage is in LDS
    chunk::lds_barrier();                // and every wave is done with this one
  }

  // acc[a][b][r] = y[m0 + 64 wm + 16 b + li][n0 + 16 NA wn + 16 a + 4 lg + r]
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int m = m0 + wm * 64 + 16 * b + li;
    if (m < M) {
#pragma unroll
      for (int a = 0; a < NA; ++a)
        store4<TY>(y + (int64_t)m * y_ld + n0 + wn * 16 * NA + 16 * a + 4 * lg, acc[a][b]);
    }
  }
}

// Relative cost of a 32-column slice of a tile at each width (measured per
// 32 columns at K = 5120: 320 and 256 wide alike, 192 wide 18% and 160 wide
// 25% dearer).
float width_cost(int na) { return na == 6 ? 1.18f : na == 5 ? 1.25f : 1.0f; }

template <int NA>
hipError_t launch_width(const uint16_t* x, int64_t x_ld, const uint16_t* W, int64_t w_ld, void* y,
                        int64_t y_ld, int y_dt, int M, int N, int K, hipStream_t stream) {
  const int tiles_m = (M + GM_ROWS - 1) / GM_ROWS, tiles_n = N / (32 * NA);
  const int nt = tiles_m * tiles_n;
  const dim3 grid((unsigned)((nt + 7) / 8 * 8));
  if (y_dt == 1)
    hipLaunchKernelGGL((gemm_bf16_kernel<NA, uint16_t>), grid, dim3(G_THREADS), 0, stream, x, x_ld,
                       W, w_ld, static_cast<uint16_t*>(y), y_ld, M, K, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<NA, float>), grid, dim3(G_THREADS), 0, stream, x, x_ld, W,
                       w_ld, static_cast<float*>(y), y_ld, M, K, tiles_m, tiles_n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Few-row form, for M <= 64 (a decode step's projections): a weight stream.
// A workgroup takes 64 W rows by all (up to 64) x rows over one of `splits`
// equal K ranges; eight waves, wave w owning W rows 16 (w & 3) .. + 15 by x
// rows 32 (w >> 2) .. + 31.  k advances in stages of 64 through a ring of
// FR_NS LDS buffers filled straight from global memory FR_NS - 1 stages ahead
// (8 KB of W rows and 8 KB of x rows per stage; rows and chunks laid out as
// in the tiled form).  With one K range the result goes to y; otherwise each
// range writes f32 partial sums to the workspace and a second kernel adds
// them in range order, so results do not depend on timing.  Measured at 64
// rows against the tuned hipBLASLt plan: in_proj_qkvz (16384 x 5120, one
// range, 256 workgroups) 38.6 vs 44.2 us, out_proj (5120 x 6144, three
// ranges, 240 workgroups) 17.0 vs 21.0 us.
constexpr int FR_ROWS = 64;  // x rows
constexpr int FR_BN = 64;    // W rows per workgroup
constexpr int FR_NS = 4;     // LDS stages in the ring

template <typename TY>
__global__ __launch_bounds__(G_THREADS) void gemm_fewrow_kernel(
    const uint16_t* __restrict__ x, int64_t x_ld, const uint16_t* __restrict__ W, int64_t w_ld,
    TY* __restrict__ y, int64_t y_ld, float* __restrict__ part, int M, int N, int KS,
    int tiles_n, int splits) {
  constexpr int LB = (FR_BN + FR_ROWS) * GK;       // elements per stage
  constexpr int NPW = (FR_BN + FR_ROWS) / 8 / 8;   // 1 KB loads per wave per stage
  static_assert((FR_NS - 2) * NPW < 16, "one vmcnt field");
  __shared__ __attribute__((aligned(16))) uint16_t Ls[FR_NS * LB];
  const int id = blockIdx.x;
  if (id >= tiles_n * splits) return;
  const int tn = id % tiles_n, sp = id / tiles_n;
  const int n0 = __builtin_amdgcn_readfirstlane(tn * FR_BN);
  const int k0 = __builtin_amdgcn_readfirstlane(sp * KS);
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), wn = w & 3, wm = w >> 2;
  typedef __attribute__((address_space(3))) void lds_t;
  const int lrow = lane >> 3, lch = (lane & 7) ^ lrow;
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + (int64_t)n0 * w_ld + k0), (short)0,
      __builtin_amdgcn_readfirstlane((int)(FR_BN * 2 * (int)w_ld)), 0x00020000);
  // x rows at or past M lie outside the range and load as zeros.
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(x + k0), (short)0, __builtin_amdgcn_readfirstlane((int)(M * 2 * (int)x_ld)),
      0x00020000);
  // Load q (8 rows) of a stage: q < FR_BN / 8 are W rows, the rest x rows.
  auto load_stage = [&](int buf, int kt) {
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
      const int q = w * NPW + j;
      lds_t* dst = (lds_t*)&Ls[buf * LB + q * 8 * GK];
      if (q < FR_BN / 8)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wres, dst, 16, (uint32_t)((q * 8 + lrow) * w_ld * 2 + lch * 16), kt * GK * 2, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xres, dst, 16, (uint32_t)(((q - FR_BN / 8) * 8 + lrow) * x_ld * 2 + lch * 16),
            kt * GK * 2, 0, 0);
    }
  };
  const int sw = li & 7;
  const int arow = (wn * 16 + li) * GK, brow = FR_BN * GK + (wm * 32 + li) * GK;
  f32x4 acc[2];
  acc[0] = acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int KT = KS / GK;
#pragma unroll
  for (int s = 0; s < FR_NS - 1; ++s)
    if (s < KT) load_stage(s, s);
  for (int kt = 0; kt < KT; ++kt) {
    // Stage kt is in LDS once at most the loads of the FR_NS - 2 later
    // stages are in flight (all of them near the end).
    if (kt + FR_NS - 2 <= KT - 1)
      __builtin_amdgcn_s_waitcnt(0x0F70 | ((FR_NS - 2) * NPW));
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    chunk::lds_barrier();  // every wave's loads of stage kt are in; stage kt - 1 is done
    if (kt + FR_NS - 1 < KT) load_stage((kt + FR_NS - 1) % FR_NS, kt + FR_NS - 1);
    const uint16_t* L = &Ls[(kt % FR_NS) * LB];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int pc = ((4 * s + lg) ^ sw) * 8;
      const bf16x8 fa = chunk::ld_frag(L + arow + pc);
      const bf16x8 fb0 = chunk::ld_frag(L + brow + pc);
      const bf16x8 fb1 = chunk::ld_frag(L + brow + 16 * GK + pc);
      acc[0] = mfma16(fa, fb0, acc[0]);
      acc[1] = mfma16(fa, fb1, acc[1]);
    }
  }
  // acc[b][r] = y[32 wm + 16 b + li][n0 + 16 wn + 4 lg + r]
  const int n = n0 + wn * 16 + 4 * lg;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int m = wm * 32 + 16 * b + li;
    if (m < M) {
      if (splits == 1)
        store4<TY>(y + (int64_t)m * y_ld + n, acc[b]);
      else
        store4<float>(part + ((int64_t)sp * M + m) * N + n, acc[b]);
    }
  }
}

// y[m][n] = the K ranges' partial sums of (m, n) added in range order.
template <typename TY>
__global__ __launch_bounds__(256) void gemm_split_sum_kernel(const float* __restrict__ part,
                                                             int splits, int M, int N,
                                                             TY* __restrict__ y, int64_t y_ld) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= (int64_t)M * N) return;
  const int m = (int)(i / N), n = (int)(i % N);
  f32x4 s = *reinterpret_cast<const f32x4*>(part + i);
  for (int p = 1; p < splits; ++p) s += *reinterpret_cast<const f32x4*>(part + (int64_t)p * M * N + i);
  store4<TY>(y + (int64_t)m * y_ld + n, s);
}

template <typename TY>
hipError_t launch_fewrow_t(const uint16_t* x, int64_t x_ld, const uint16_t* W, int64_t w_ld,
                           void* y, int64_t y_ld, int M, int N, int K, int splits, void* ws,
                           hipStream_t stream) {
  const int tiles_n = N / FR_BN;
  hipLaunchKernelGGL((gemm_fewrow_kernel<TY>), dim3((unsigned)(tiles_n * splits)),
                     dim3(G_THREADS), 0, stream, x, x_ld, W, w_ld, static_cast<TY*>(y), y_ld,
                     static_cast<float*>(ws), M, N, K / splits, tiles_n, splits);
  if (splits > 1) {
    const int64_t quads = (int64_t)M * N / 4;
    hipLaunchKernelGGL((gemm_split_sum_kernel<TY>), dim3((unsigned)((quads + 255) / 256)),
                       dim3(256), 0, stream, static_cast<const float*>(ws), splits, M, N,
                       static_cast<TY*>(y), y_ld);
  }
  return hipGetLastError();
}

}  // namespace

int gemm_fewrow_splits(int M, int N, int K, int64_t x_ld, int64_t w_ld, int cus,
                       size_t ws_bytes) {
  if (M < 1 || M > FR_ROWS || N <= 0 || K <= 0 || K % GK || N % FR_BN || cus <= 0) return 0;
  if (x_ld > (1 << 21) || w_ld > (1 << 21)) return 0;  // 32-bit row offsets
  const int64_t tiles = N / FR_BN;
  if (tiles > (1 << 24)) return 0;
  // The fewest equal K ranges (whole stages, at least four a range, partial
  // sums within the workspace) that give about three quarters of a round of
  // the CUs; none: the shape goes elsewhere.
  for (int s : {1, 2, 3, 4, 5, 6, 8, 10, 12, 16}) {
    if (K % (GK * s)) continue;
    if (K / s < 4 * GK) break;
    if (s > 1 && (size_t)s * M * N * 4 > ws_bytes) break;
    if (tiles * s * 4 >= (int64_t)cus * 3) return s;
  }
  return 0;
}

hipError_t launch_gemm_fewrow(const uint16_t* x, int64_t x_ld, const uint16_t* W, int64_t w_ld,
                              void* y, int64_t y_ld, int y_dt, int M, int N, int K, int splits,
                              void* workspace, hipStream_t stream) {
  if (splits < 1 || K % (GK * splits) || N % FR_BN || M < 1 || M > FR_ROWS ||
      (splits > 1 && !workspace))
    return hipErrorInvalidValue;
  return y_dt == 1 ? launch_fewrow_t<uint16_t>(x, x_ld, W, w_ld, y, y_ld, M, N, K, splits,
                                               workspace, stream)
                   : launch_fewrow_t<float>(x, x_ld, W, w_ld, y, y_ld, M, N, K, splits,
                                            workspace, stream);
}

int gemm_bf16_width(int M, int N, int K, int64_t x_ld, int64_t w_ld, int cus) {
  // Shape limits of the kernel: k in whole stages, N in whole blocks, each
  // operand's block rows addressable by a 32-bit buffer range.
  if (M <= 0 || N <= 0 || K <= 0 || K % GK || cus <= 0) return 0;
  if (x_ld > (1 << 21) || w_ld > (1 << 21) || M > (1 << 30)) return 0;  // 32-bit row indices
  const int64_t tiles_m = (M + GM_ROWS - 1) / GM_ROWS;
  int best = 0;
  float best_cost = 0.0f;
  for (int na : {10, 8, 6, 5}) {
    if (N % (32 * na)) continue;
    const int64_t tiles = tiles_m * (N / (32 * na));
    if (tiles > (1 << 28)) continue;
    const int64_t rounds = (tiles + cus - 1) / cus;
    // Worth it only with at least one full round of the CUs, the last round
    // at least three quarters full on average.
    if (tiles < cus || tiles * 4 < rounds * cus * 3) continue;
    const float cost = (float)rounds * na * width_cost(na);
    if (best == 0 || cost < best_cost) {
      best = na;
      best_cost = cost;
    }
  }
  return best;
}

hipError_t launch_gemm_bf16(const uint16_t* x, int64_t x_ld, const uint16_t* W, int64_t w_ld,
                            void* y, int64_t y_ld, int y_dt, int M, int N, int K, int na,
                            hipStream_t stream) {
  switch (na) {
    case 5: return launch_width<5>(x, x_ld, W, w_ld, y, y_ld, y_dt, M, N, K, stream);
    case 6: return launch_width<6>(x, x_ld, W, w_ld, y, y_ld, y_dt, M, N, K, stream);
    case 8: return launch_width<8>(x, x_ld, W, w_ld, y, y_ld, y_dt, M, N, K, stream);
    case 10: return launch_width<10>(x, x_ld, W, w_ld, y, y_ld, y_dt, M, N, K, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
