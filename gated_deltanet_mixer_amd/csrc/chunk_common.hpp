// Shared pieces of the chunked prefill kernels (gfx950): tile constants, MFMA
// wrappers, LDS-only barrier, operand loads and the fragment orders that the
// prep and fused kernels write and the chain reads.
//
// MFMA operand layouts (checked on the device): v_mfma_f32_16x16x32_bf16 --
// lane l holds A[l%16][8(l/16)..+7], B[8(l/16)..+7][l%16]; the 16x16x16 form
// holds A[l%16][4(l/16)..+3], B[4(l/16)..+3][l%16]; both give D[4(l/16)+r][l%16],
// r = 0..3, which is also the 16x16x16 B layout, so its results chain.
#pragma once
#include "common.hpp"

namespace gdn {
namespace chunk {

constexpr int CK = 64;   // chunk length
constexpr int DH = 128;  // head width
constexpr int XP = 72;   // pitch (bf16) of [*, 64] LDS tiles: 144-byte rows, 16-byte aligned
constexpr int FP = 68;   // pitch (f32) of [64, 64] f32 LDS tiles: 272-byte rows
constexpr int RP = DH + 8;  // pitch (bf16) of [*, 128] LDS tiles: 272-byte rows

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16k16(const s16x4& a, const s16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Workgroup barrier for LDS data only: waits for this wave's LDS operations,
// not for its global loads and stores, so prefetched loads stay in flight.
// The memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ bf16x8 ld_frag(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ s16x4 ld_frag4(const uint16_t* p) {
  return *reinterpret_cast<const s16x4*>(p);
}

__device__ __forceinline__ bf16x8 zero_frag() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
  return z;
}

// Element access goes through a whole-vector bit cast: a bit cast of one
// element of a __bf16 vector does not select that element here.
__device__ __forceinline__ u16x8 frag_bits(const bf16x8& f) {
  return __builtin_bit_cast(u16x8, f);
}

// Eight consecutive q/k/v values as a bf16 operand (hi) and, for f32 input,
// the bf16 rounding of the remainder (lo), so that hi + lo carries ~16 bits.
__device__ __forceinline__ void load_row8(const uint16_t* p, bf16x8& hi, bf16x8& lo) {
  hi = ld_frag(p);
  lo = zero_frag();
}
__device__ __forceinline__ void load_row8(const float* p, bf16x8& hi, bf16x8& lo) {
  float x[8];
  load8(p, x);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h = (__bf16)x[i];
    hi[i] = h;
    lo[i] = (__bf16)(x[i] - (float)h);
  }
}

__device__ __forceinline__ s16x4 to_s16x4(float a, float b, float c, float d) {
  s16x4 r;
  r[0] = (short)f2bf(a); r[1] = (short)f2bf(b); r[2] = (short)f2bf(c); r[3] = (short)f2bf(d);
  return r;
}

template <typename TO>
__device__ __forceinline__ void st4(TO* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void st4<uint16_t>(uint16_t* p, float a, float b, float c, float d) {
  u16x4 v;
  v[0] = f2bf(a); v[1] = f2bf(b); v[2] = f2bf(c); v[3] = f2bf(d);
  *reinterpret_cast<u16x4*>(p) = v;
}

// Four values as two bf16 parts, hi = bf16(x) and lo = bf16(x - hi), stored
// at hi_p and lo_p (hi + lo carries ~16 significant bits).
__device__ __forceinline__ void st4_split(uint16_t* hi_p, uint16_t* lo_p, float a, float b,
                                          float c, float d) {
  u16x4 h, l;
  const float v[4] = {a, b, c, d};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = f2bf(v[i]);
    l[i] = f2bf(v[i] - bf2f(h[i]));
  }
  *reinterpret_cast<u16x4*>(hi_p) = h;
  *reinterpret_cast<u16x4*>(lo_p) = l;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_scan(float x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// The chain kernel's operands, per chunk, in the order its lanes load them:
// "fragment-major", so that each of its 16-byte-per-lane loads reads 1 KB of
// contiguous memory.  Lane l = li + 16 lg of chain wave w holds, for step kk,
//   Wf[w][kk][l][j]  = W[16w + li][32kk + 8lg + j]            (t, dk)
//   Qf[w][kk][l][j]  = Q[16w + li][32kk + 8lg + j]            (t, dk), bf16
//   Pf[w][kk][l][j]  = P[16w + li][32kk + 8lg + j]            (t, s), kk < 2
//   Ktf[w][i][kk][l][j] = K[32kk + 8lg + j][32w + 16i + li]   (s, dk), kk < 2
//   Utf[sl][w][vb][l][r] = Ut[16w + 4lg + r][32sl + dvp(vb, li)] (t, dv), r < 4
// with dvp(vb, m) = 8(m/4) + 4vb + m%4: the chain multiplies the dv rows of a
// 32-column slice in that order, so that each lane of its output tile ends up
// with 8 consecutive dv of one token.
// Position of dv within a 32-column slice under the chain's row order.
__device__ __forceinline__ int dvp(int vb, int m) { return 8 * (m >> 2) + 4 * vb + (m & 3); }

// Offset of element (t, c) of a 64 x (32 m) tile in the Wf/Qf/Pf order, for a
// 4-wide run of c starting at a multiple of 4 (what one MFMA result lane holds
// after the operand swap): m = number of 32-wide k steps.
__device__ __forceinline__ int frag_off(int t, int col, int m) {
  const int w = t >> 4, li = t & 15, kk = col >> 5, lg = (col >> 3) & 3, j = col & 7;
  return ((w * m + kk) * 64 + li + 16 * lg) * 8 + j;
}

}  // namespace chunk
}  // namespace gdn
