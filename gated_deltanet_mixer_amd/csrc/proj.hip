// The projections on either side of the mixer ("Qwen/Qwen3.8-27B" architecture
// viewer, module tree: in_proj_qkv 5120->10240, in_proj_z 5120->6144,
// in_proj_a / in_proj_b 5120->48, out_proj 6144->5120; each maps x to x W^T
// with W stored [out][in]).
//
// * The two 48-wide gate projections keep their weights in f32 (the "qwen38"
//   code-generation page, extra kernels: rounding that [d, 48] matrix would
//   put the gates at risk for a negligible saving).  gate_proj_kernel runs them
//   on bf16 MFMA without rounding a weight: each f32 weight w is cut by
//   truncation into three bf16 parts, hi + lo + lo2 == w exactly (each part
//   holds 8 of w's 24 significant bits), and a bf16 activation times a bf16
//   part is exact in f32, so three MFMAs per k-step give the f32-weight
//   product with f32 accumulation.
// * in_proj_qkv, in_proj_z and out_proj are plain bf16 GEMMs with f32
//   accumulation.  Shapes that fill the GPU with the library's own tiled GEMM
//   (gemm.hip) run there, shapes of at most 64 rows (a decode step) on its
//   few-row form when that has enough weight blocks; the others go to
//   hipBLASLt.  One hipBLASLt handle
//   per device is created on its first use and kept until the process ends;
//   the plans of recent shapes (descriptors and the heuristic's first
//   candidate that fits the workspace, or the fastest of the library's GEMM
//   and several candidates when the caller asks for timing) are cached
//   beside it.  The library links libhipblaslt.so.1 by soname: in a process
//   that already holds a copy of that library (PyTorch ships one), that copy
//   serves these calls.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <algorithm>
#include <deque>
#include <map>
#include <mutex>
#include <tuple>

#include "chunk_common.hpp"
#include "launch.hpp"

namespace gdn {

using chunk::mfma16;

// ---------------------------------------------------------------------------
// Gate projections, split over K.  Pass 1: workgroup = 16*MT tokens x all 2H
// outputs x one of KS contiguous ranges of 32-wide k-steps; wave w owns output
// tile w (16 outputs of [a | b]) and multiplies every token of the workgroup
// (MT 16-row MFMA tiles), so each x value is fetched from memory once per
// workgroup (the waves share it in L1) and each weight once per token tile.
// The partial sums go to the workspace, [KS][M][2H] f32; pass 2 adds the KS
// partials of each output in order 0..KS-1 (results do not depend on timing).
// With KS == 1, pass 1 writes a and b directly.

// Bits [31:16] of a and of b packed as two bf16 (a in the low half).
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
  return (b & 0xffff0000u) | (a >> 16);
}

// Eight f32 weights as three bf16 operands whose sum is exact.
__device__ __forceinline__ void split3(const float4& w0, const float4& w1, bf16x8& hi, bf16x8& lo,
                                       bf16x8& lo2) {
  const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  uint32_t u0[8], u1[8], u2[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    u0[i] = __float_as_uint(w[i]);
    const float r1 = w[i] - __uint_as_float(u0[i] & 0xffff0000u);
    u1[i] = __float_as_uint(r1);
    const float r2 = r1 - __uint_as_float(u1[i] & 0xffff0000u);
    u2[i] = __float_as_uint(r2);
  }
  uint32_t h[4], l[4], m[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack_hi16(u0[2 * i], u0[2 * i + 1]);
    l[i] = pack_hi16(u1[2 * i], u1[2 * i + 1]);
    m[i] = pack_hi16(u2[2 * i], u2[2 * i + 1]);
  }
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
  lo = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
  lo2 = __builtin_bit_cast(bf16x8, u32x4{m[0], m[1], m[2], m[3]});
}

// One k-step's operands: eight weights of this lane's output and eight x
// values of each of its MT token rows.
template <int MT>
struct GateStep {
  float4 w0, w1;
  bf16x8 xf[MT];
};

constexpr int kGateMaxTiles = 8;  // 2H / 16 <= 8 output tiles (H <= 64)

// Number of K ranges for M tokens: about one workgroup per CU (256; 512, 768
// and 1024 measured slower at 4096 tokens), at least four k-steps per range.
int gate_splits(int M, int K) {
  const int tok = M >= 1024 ? 64 : 16;
  const int mtiles = (M + tok - 1) / tok;
  const int nsteps = K / 32;
  const int want = (256 + mtiles - 1) / mtiles;
  return std::max(1, std::min(want, nsteps / 4));
}

template <int MT>
__global__ __launch_bounds__(64 * kGateMaxTiles) void gate_part_kernel(
    const uint16_t* __restrict__ x, int64_t x_ld, const float* __restrict__ Wa,
    const float* __restrict__ Wb, float* __restrict__ part, float* __restrict__ a,
    float* __restrict__ b, int64_t ab_ld, int M, int K, int H) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
  const int tok0 = blockIdx.x * 16 * MT;
  const int o = w * 16 + li;  // this lane's output column of [a | b]
  const float* wrow = (o < H ? Wa + (int64_t)o * K : Wb + (int64_t)(o - H) * K) + lg * 8;
  // Rows past M read row M-1 (in bounds); their results are not stored.
  const uint16_t* xr[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
    xr[i] = x + (int64_t)min(tok0 + 16 * i + li, M - 1) * x_ld + lg * 8;

  // This workgroup's k-steps [sb, se) of the K/32.  Four operand sets in
  // rotation, named statically by unrolling four steps per trip: a set is
  // reloaded for four steps later as soon as its step is multiplied, so no
  // register is copied while its load is in flight.  Loads are unconditional
  // (clamped to the last k-step), so the compiler's count of loads in flight
  // stays exact; so is every multiply (a branch around one made the compiler
  // drain all loads at the top of each trip).
  const int nsteps = K >> 5, ks = blockIdx.y, KS = gridDim.y;
  const int sb = (int)((int64_t)ks * nsteps / KS), se = (int)((int64_t)(ks + 1) * nsteps / KS);
  const int last = se - 1;
  auto load = [&](int st, GateStep<MT>& g) __attribute__((always_inline)) {
    const int k = min(st, last) * 32;
    g.w0 = *reinterpret_cast<const float4*>(wrow + k);
    g.w1 = *reinterpret_cast<const float4*>(wrow + k + 4);
#pragma unroll
    for (int i = 0; i < MT; ++i) g.xf[i] = *reinterpret_cast<const bf16x8*>(xr[i] + k);
  };
  f32x4 acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  GateStep<MT> g[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) load(sb + u, g[u]);
  // The scheduling barriers keep each reload where it is written: left free,
  // the scheduler sinks the loads next to their use and the prefetch is lost.
  __builtin_amdgcn_sched_barrier(0);
  for (int j = sb; j < se; j += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // A step past se multiplies zero weights (a select, not a branch).
      const bool live = j + u < se;
      const float4 z4 = {0.f, 0.f, 0.f, 0.f};
      bf16x8 hi, lo, lo2;
      split3(live ? g[u].w0 : z4, live ? g[u].w1 : z4, hi, lo, lo2);
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        acc[i] = mfma16(g[u].xf[i], hi, acc[i]);
        acc[i] = mfma16(g[u].xf[i], lo, acc[i]);
        acc[i] = mfma16(g[u].xf[i], lo2, acc[i]);
      }
      load(j + u + 4, g[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // D[4 lg + r][li] of token tile i: token tok0 + 16 i + 4 lg + r, output o.
  const int NO = 2 * H;
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = tok0 + 16 * i + 4 * lg + r;
      if (t >= M) continue;
      if (part)
        part[((int64_t)ks * M + t) * NO + o] = acc[i][r];
      else
        (o < H ? a + o : b + (o - H))[(int64_t)t * ab_ld] = acc[i][r];
    }
  }
}

// The same product for many tokens (64 per workgroup), with the token tile
// staged through LDS: per 64-wide k-stage the workgroup reads the 64 x rows
// with eight adjacent lanes per 128-byte piece (the MFMA order, lane = row,
// reads them at about half that rate, and six waves each fetched them
// through L1), writes them to a double-buffered LDS tile, and the waves read
// their fragments from there.  x pieces and each wave's weights are loaded
// four stages ahead in registers; one barrier per stage.  The buffer written
// at stage s was last read at stage s - 2, before the barrier of stage s - 1.
constexpr int GL_KC = 64;  // k per stage (two 32-wide k-steps)
constexpr int GL_XP = 72;  // LDS pitch (bf16): 144-byte rows, conflict-free b128 reads

struct GateLdsStage {
  float4 w[4];         // this lane's 8 weights of each of the stage's two k-steps
  uint32_t x0[4], x1[4];  // x pieces tid and tid + 384 (the latter for tid < 128)
};

__global__ __launch_bounds__(64 * kGateMaxTiles) void gate_part_lds_kernel(
    const uint16_t* __restrict__ x, int64_t x_ld, const float* __restrict__ Wa,
    const float* __restrict__ Wb, float* __restrict__ part, float* __restrict__ a,
    float* __restrict__ b, int64_t ab_ld, int M, int K, int H) {
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][64 * GL_XP];
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int w = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const int tok0 = blockIdx.x * 64;
  const int o = w * 16 + li;  // this lane's output column of [a | b]
  const float* wrow = (o < H ? Wa + (int64_t)o * K : Wb + (int64_t)(o - H) * K) + lg * 8;
  // x pieces (row p / 8, 16-byte column p % 8 of a stage): tid, and tid +
  // nthr while that is below 512 (the launch gives at least 256 threads, so
  // the two cover all 512).  Rows past M read row M-1.
  const int p0 = tid, p1 = tid + nthr;
  const bool two = p1 < 512;
  const int xr0 = p0 >> 3, xr1 = min(p1, 511) >> 3, xc0 = (p0 & 7) * 8, xc1 = (p1 & 7) * 8;
  const uint16_t* xp0 = x + (int64_t)min(tok0 + xr0, M - 1) * x_ld + xc0;
  const uint16_t* xp1 = x + (int64_t)min(tok0 + xr1, M - 1) * x_ld + xc1;

  const int nst = K / GL_KC, ks = blockIdx.y, KS = gridDim.y;
  const int sb = (int)((int64_t)ks * nst / KS), se = (int)((int64_t)(ks + 1) * nst / KS);
  const int last = se - 1;
  auto load = [&](int st, GateLdsStage& g) __attribute__((always_inline)) {
    const int k = min(st, last) * GL_KC;
    g.w[0] = *reinterpret_cast<const float4*>(wrow + k);
    g.w[1] = *reinterpret_cast<const float4*>(wrow + k + 4);
    g.w[2] = *reinterpret_cast<const float4*>(wrow + k + 32);
    g.w[3] = *reinterpret_cast<const float4*>(wrow + k + 36);
    const uint4 v0 = *reinterpret_cast<const uint4*>(xp0 + k);
    const uint4 v1 = *reinterpret_cast<const uint4*>(xp1 + k);
    g.x0[0] = v0.x; g.x0[1] = v0.y; g.x0[2] = v0.z; g.x0[3] = v0.w;
    g.x1[0] = v1.x; g.x1[1] = v1.y; g.x1[2] = v1.z; g.x1[3] = v1.w;
  };
  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  GateLdsStage g[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) load(sb + u, g[u]);
  __builtin_amdgcn_sched_barrier(0);
  for (int j = sb; j < se; j += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = j + u, bb = s & 1;
      // A stage past se multiplies zero weights (a select, not a branch).
      const bool live = s < se;
      *reinterpret_cast<uint4*>(&Xs[bb][xr0 * GL_XP + xc0]) =
          uint4{g[u].x0[0], g[u].x0[1], g[u].x0[2], g[u].x0[3]};
      if (two)
        *reinterpret_cast<uint4*>(&Xs[bb][xr1 * GL_XP + xc1]) =
            uint4{g[u].x1[0], g[u].x1[1], g[u].x1[2], g[u].x1[3]};
      const float4 z4 = {0.f, 0.f, 0.f, 0.f};
      bf16x8 hi[2], lo[2], lo2[2];
      split3(live ? g[u].w[0] : z4, live ? g[u].w[1] : z4, hi[0], lo[0], lo2[0]);
      split3(live ? g[u].w[2] : z4, live ? g[u].w[3] : z4, hi[1], lo[1], lo2[1]);
      load(s + 4, g[u]);
      __builtin_amdgcn_sched_barrier(0);
      chunk::lds_barrier();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 xf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          xf[i] = chunk::ld_frag(&Xs[bb][(16 * i + li) * GL_XP + kk * 32 + lg * 8]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[i] = mfma16(xf[i], hi[kk], acc[i]);
          acc[i] = mfma16(xf[i], lo[kk], acc[i]);
          acc[i] = mfma16(xf[i], lo2[kk], acc[i]);
        }
      }
    }
  }
  // D[4 lg + r][li] of token tile i: token tok0 + 16 i + 4 lg + r, output o.
  const int NO = 2 * H;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = tok0 + 16 * i + 4 * lg + r;
      if (t >= M) continue;
      if (part)
        part[((int64_t)ks * M + t) * NO + o] = acc[i][r];
      else
        (o < H ? a + o : b + (o - H))[(int64_t)t * ab_ld] = acc[i][r];
    }
  }
}

// Pass 2: one thread per four consecutive outputs of one token.
__global__ __launch_bounds__(256) void gate_sum_kernel(const float* __restrict__ part,
                                                       float* __restrict__ a,
                                                       float* __restrict__ b, int64_t ab_ld,
                                                       int M, int H, int KS) {
  const int NO = 2 * H, per_tok = NO / 4;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)M * per_tok) return;
  const int t = (int)(id / per_tok), o = (int)(id % per_tok) * 4;
  const int64_t stride = (int64_t)M * NO;
  const float* p = part + (int64_t)t * NO + o;
  // Up to 20 partials are loaded before any is added (a load-add chain waits
  // out the memory latency once per partial; at 64 tokens, 40 ranges, 20 a
  // batch took the pass from 5.8-6.3 to 4.2-4.8 us against 8); the adds still
  // run in order.
  constexpr int kBatch = 20;
  float4 s = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < KS; k0 += kBatch) {
    float4 v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (k0 + j < KS) v[j] = *reinterpret_cast<const float4*>(p + (int64_t)(k0 + j) * stride);
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (k0 + j < KS) {
        s.x += v[j].x; s.y += v[j].y; s.z += v[j].z; s.w += v[j].w;
      }
    }
  }
  // H % 16 == 0, so the four outputs lie all in a or all in b.
  float* dst = (o < H ? a + o : b + (o - H)) + (int64_t)t * ab_ld;
  dst[0] = s.x; dst[1] = s.y; dst[2] = s.z; dst[3] = s.w;
}

size_t gate_proj_workspace_bytes(int M, int K, int H) {
  const int KS = gate_splits(M, K);
  return KS > 1 ? (size_t)KS * M * 2 * H * sizeof(float) : 0;
}

hipError_t launch_gate_proj(const uint16_t* x, int64_t x_ld, const float* Wa, const float* Wb,
                            float* a, float* b, int64_t ab_ld, int M, int K, int H, void* workspace,
                            hipStream_t stream) {
  const int KS = gate_splits(M, K), NT = 2 * H / 16;
  float* part = KS > 1 ? static_cast<float*>(workspace) : nullptr;
  if (M >= 1024 && K % GL_KC == 0 && NT >= 4) {  // >= 256 threads: two x pieces each cover 512
    hipLaunchKernelGGL(gate_part_lds_kernel, dim3((M + 63) / 64, KS), dim3(64 * NT), 0, stream,
                       x, x_ld, Wa, Wb, part, a, b, ab_ld, M, K, H);
  } else if (M >= 1024) {
    hipLaunchKernelGGL(gate_part_kernel<4>, dim3((M + 63) / 64, KS), dim3(64 * NT), 0, stream, x,
                       x_ld, Wa, Wb, part, a, b, ab_ld, M, K, H);
  } else {
    hipLaunchKernelGGL(gate_part_kernel<1>, dim3((M + 15) / 16, KS), dim3(64 * NT), 0, stream, x,
                       x_ld, Wa, Wb, part, a, b, ab_ld, M, K, H);
  }
  if (KS > 1) {
    const int64_t threads = (int64_t)M * (2 * H / 4);
    hipLaunchKernelGGL(gate_sum_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       stream, part, a, b, ab_ld, M, H, KS);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bf16 linear layers on hipBLASLt.  Row-major y[M][N] = x[M][K] W[N][K]^T is
// the column-major product D (N x M) = op(A) B with A = W viewed as a K x N
// column-major matrix (op = transpose) and B = x viewed as K x M.

namespace {

struct LtPlan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t A = nullptr, B = nullptr, D = nullptr;
  hipblasLtMatmulAlgo_t algo;
  bool ok = false;     // hipBLASLt has an algorithm for the shape
  bool tuned = false;  // made by a timed call
  float ms = 0.0f;     // the chosen algorithm's time for three runs (timed plans)
  int own = 0;         // nonzero: the library's tiled GEMM at this width won the timing
  int few = 0;         // nonzero: its few-row form with this many K ranges won
};

using PlanKey = std::tuple<int, int, int, int, int64_t, int64_t, int64_t, int, size_t>;

// Plans made without timing are kept for the kMaxPlans most recent shapes
// (a ragged caller brings a new M on almost every call); timed plans stay.
constexpr size_t kMaxPlans = 64;

std::mutex g_lt_mu;
std::map<int, hipblasLtHandle_t> g_lt_handle;
std::map<int, int> g_cus;  // CUs per device
std::map<PlanKey, LtPlan> g_lt_plans;
std::deque<PlanKey> g_lt_untimed;  // keys of untimed plans, oldest first

void destroy_plan(LtPlan& p) {
  if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
  if (p.A) hipblasLtMatrixLayoutDestroy(p.A);
  if (p.B) hipblasLtMatrixLayoutDestroy(p.B);
  if (p.D) hipblasLtMatrixLayoutDestroy(p.D);
  p = LtPlan{};
}

// Builds the plan for one shape; false if hipBLASLt has no algorithm for it.
// Without `tune` it takes the heuristic's first candidate that fits the
// workspace: host work only, nothing enqueued or awaited.  With `tune`, up to
// kTune of the fitting candidates are timed on the caller's own buffers and
// stream (one warm-up and three timed runs each, all writing y, which the
// call then writes again) and the fastest is kept; that synchronises.
bool make_plan(hipblasLtHandle_t h, LtPlan& p, bool tune, const void* x, int64_t x_ld,
               const void* W, int64_t w_ld, void* y, int64_t y_ld, int y_dt, int M, int N, int K,
               void* workspace, size_t ws_bytes, hipStream_t stream) {
  const hipblasOperation_t opA = HIPBLAS_OP_T, opB = HIPBLAS_OP_N;
  const hipDataType dty = y_dt == 1 ? HIP_R_16BF : HIP_R_32F;
  if (hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS)
    return false;
  hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opA, sizeof(opA));
  hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opB, sizeof(opB));
  if (hipblasLtMatrixLayoutCreate(&p.A, HIP_R_16BF, K, N, w_ld) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&p.B, HIP_R_16BF, K, M, x_ld) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&p.D, dty, N, M, y_ld) != HIPBLAS_STATUS_SUCCESS)
    return false;
  hipblasLtMatmulPreference_t pref;
  if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) return false;
  const uint64_t cap = ws_bytes;
  hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &cap,
                                        sizeof(cap));
  // Several candidates, best first: some hipBLASLt builds rank first an
  // algorithm that needs more workspace than the cap allows.
  constexpr int kCand = 16, kTune = 8;
  hipblasLtMatmulHeuristicResult_t res[kCand];
  int n = 0;
  const hipblasStatus_t st =
      hipblasLtMatmulAlgoGetHeuristic(h, p.desc, p.A, p.B, p.D, p.D, pref, kCand, res, &n);
  hipblasLtMatmulPreferenceDestroy(pref);
  if (st != HIPBLAS_STATUS_SUCCESS) return false;
  int fit[kCand], nfit = 0;
  for (int i = 0; i < n && i < kCand; ++i)
    if (res[i].state == HIPBLAS_STATUS_SUCCESS && res[i].workspaceSize <= ws_bytes)
      fit[nfit++] = i;
  if (nfit == 0) return false;
  p.algo = res[fit[0]].algo;
  if (!tune) return true;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return true;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return true;
  }
  const float alpha = 1.0f, beta = 0.0f;
  float best = 0.0f;
  for (int c = 0; c < nfit && c < kTune; ++c) {
    const hipblasLtMatmulAlgo_t* al = &res[fit[c]].algo;
    auto run = [&]() {
      return hipblasLtMatmul(h, p.desc, &alpha, W, p.A, x, p.B, &beta, y, p.D, y, p.D, al,
                             workspace, ws_bytes, stream) == HIPBLAS_STATUS_SUCCESS;
    };
    if (!run()) continue;
    bool ok = hipEventRecord(e0, stream) == hipSuccess;
    for (int r = 0; r < 3 && ok; ++r) ok = run();
    ok = ok && hipEventRecord(e1, stream) == hipSuccess && hipEventSynchronize(e1) == hipSuccess;
    float ms = 0.0f;
    if (!ok || hipEventElapsedTime(&ms, e0, e1) != hipSuccess) continue;
    if (best == 0.0f || ms < best) {
      best = ms;
      p.algo = *al;
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  p.ms = best;
  return true;
}

// Times one of the library's GEMM launches (`run`) the way make_plan times a
// candidate (one warm-up and three timed runs on the caller's buffers and
// stream); 0 if it could not be timed.
template <typename Run>
float time_runs(Run run, hipStream_t stream) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return 0.0f;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return 0.0f;
  }
  float ms = 0.0f;
  bool ok = run() && hipEventRecord(e0, stream) == hipSuccess;
  for (int r = 0; r < 3 && ok; ++r) ok = run();
  ok = ok && hipEventRecord(e1, stream) == hipSuccess && hipEventSynchronize(e1) == hipSuccess;
  if (!ok || hipEventElapsedTime(&ms, e0, e1) != hipSuccess) ms = 0.0f;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return ms;
}

}  // namespace

LinearStatus launch_linear(const uint16_t* x, int64_t x_ld, const uint16_t* W, int64_t w_ld,
                           void* y, int64_t y_ld, int y_dt, int M, int N, int K, void* workspace,
                           size_t workspace_bytes, bool tune, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LinearStatus::kLaunchFailed;
  std::lock_guard<std::mutex> lock(g_lt_mu);
  auto cit = g_cus.find(dev);
  if (cit == g_cus.end()) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 0;
    cit = g_cus.emplace(dev, cus).first;
  }
  const int width = gemm_bf16_width(M, N, K, x_ld, w_ld, cit->second);
  const int splits =
      width ? 0
            : gemm_fewrow_splits(M, N, K, x_ld, w_ld, cit->second, workspace ? workspace_bytes : 0);
  auto own = [&](int wd) {
    return launch_gemm_bf16(x, x_ld, W, w_ld, y, y_ld, y_dt, M, N, K, wd, stream) == hipSuccess
               ? LinearStatus::kOk
               : LinearStatus::kLaunchFailed;
  };
  auto few = [&](int sp) {
    return launch_gemm_fewrow(x, x_ld, W, w_ld, y, y_ld, y_dt, M, N, K, sp, workspace,
                              stream) == hipSuccess
               ? LinearStatus::kOk
               : LinearStatus::kLaunchFailed;
  };
  const PlanKey key{dev, M, N, K, x_ld, w_ld, y_ld, y_dt, workspace_bytes};
  auto pit = g_lt_plans.find(key);
  // A timed plan decides; without one, a shape the library's GEMM suits
  // (tiled, or its few-row form) runs there.
  if (!tune && pit != g_lt_plans.end() && pit->second.tuned) {
    if (pit->second.own) return own(pit->second.own);
    if (pit->second.few) return few(pit->second.few);
  }
  if (!tune && (pit == g_lt_plans.end() || !pit->second.tuned)) {
    if (width) return own(width);
    if (splits) return few(splits);
  }

  auto hit = g_lt_handle.find(dev);
  if (hit == g_lt_handle.end()) {
    hipblasLtHandle_t h = nullptr;
    if (hipblasLtCreate(&h) != HIPBLAS_STATUS_SUCCESS)
      return width ? own(width) : splits ? few(splits) : LinearStatus::kLaunchFailed;
    // The descriptors and results passed here follow this header's major
    // version (the soname's); a loaded library of another major is refused.
    int ver = 0;
    if (hipblasLtGetVersion(h, &ver) != HIPBLAS_STATUS_SUCCESS ||
        ver / 100000 != HIPBLASLT_VERSION_MAJOR) {
      hipblasLtDestroy(h);
      return width ? own(width) : splits ? few(splits) : LinearStatus::kBadLibrary;
    }
    hit = g_lt_handle.emplace(dev, h).first;
  }
  if (pit != g_lt_plans.end() && tune && !pit->second.tuned) {
    g_lt_untimed.erase(std::find(g_lt_untimed.begin(), g_lt_untimed.end(), key));
    destroy_plan(pit->second);
    g_lt_plans.erase(pit);
    pit = g_lt_plans.end();
  }
  if (pit == g_lt_plans.end()) {
    if (!tune && g_lt_untimed.size() >= kMaxPlans) {
      auto old = g_lt_plans.find(g_lt_untimed.front());
      destroy_plan(old->second);
      g_lt_plans.erase(old);
      g_lt_untimed.pop_front();
    }
    LtPlan p;
    p.ok = make_plan(hit->second, p, tune, x, x_ld, W, w_ld, y, y_ld, y_dt, M, N, K, workspace,
                     workspace_bytes, stream);
    p.tuned = tune;
    if (tune && (width || splits)) {
      // The library's kernel wins when it is faster, or when hipBLASLt has
      // nothing for the shape.
      const float ms = width ? time_runs([&]() { return own(width) == LinearStatus::kOk; }, stream)
                             : time_runs([&]() { return few(splits) == LinearStatus::kOk; },
                                         stream);
      if (!p.ok || (ms > 0.0f && (p.ms == 0.0f || ms < p.ms))) {
        p.own = width;
        p.few = splits;
      }
    }
    pit = g_lt_plans.emplace(key, p).first;
    if (!tune) g_lt_untimed.push_back(key);
  }
  const LtPlan& p = pit->second;
  if (p.own) return own(p.own);
  if (p.few) return few(p.few);
  if (!p.ok) return LinearStatus::kNoAlgorithm;
  const float alpha = 1.0f, beta = 0.0f;
  const hipblasStatus_t st =
      hipblasLtMatmul(hit->second, p.desc, &alpha, W, p.A, x, p.B, &beta, y, p.D, y, p.D, &p.algo,
                      workspace, workspace_bytes, stream);
  return st == HIPBLAS_STATUS_SUCCESS ? LinearStatus::kOk : LinearStatus::kLaunchFailed;
}

}  // namespace gdn
