// The gated delta rule evaluated token by token in f32, for decode_rows and
// for the sequential prefill ("Qwen3.8 27B" model card, Gated DeltaNet bullet
// and state paragraph; the update S_t = a_t S_{t-1}(I - b_t k_t k_t^T) +
// b_t v_t k_t^T, o_t = S_t q_t).
//
// Row i of S (value channel i) evolves on its own given k, q, v_i and the
// gates:  u_i = S_i . k,  d_i = b (v_i - a u_i),  S_i <- a S_i + d_i k,
// o_i = S_i . q = a (S_i . q)_old + d_i (k . q).
// Every kernel gives each row to 16 lanes, 8 f32 per lane, so its dot
// products are DPP row sums.
#include "common.hpp"
#include "launch.hpp"

namespace gdn {

__device__ __forceinline__ float dot8(const float* a, const float* b) {
  float s = a[0] * b[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) s = fmaf(a[i], b[i], s);
  return s;
}

// ---------------------------------------------------------------------------
// decode_rows: one new token per fixed row, state [R, Hv, 128, 128] updated in
// place.  HBM-bound: 64 KiB read and 64 KiB written per (row, head).
// DEC_PARTS workgroups per (row, value head), each with 16 value rows: wave w
// owns rows 16 part + 4w + g (g = lane / 16), loaded before any arithmetic.
// Lane l of a 16-lane group holds elements 4l..4l+3 and 64+4l..64+4l+3 of its
// row, so each 16-byte load or store instruction covers 256 contiguous bytes
// of four rows.  Against one workgroup per (row, head) with 8 contiguous
// elements per lane this runs at 5.5 TB/s instead of 4.8 TB/s: the finer grid
// leaves no tail of half-empty rounds.  Two parts of 64 rows ran 76.7 us at
// 64 rows, four of 32 rows 72.6-73.4 us, eight of 16 rows 69.8-71.1 us (rocprof).
// (Non-temporal stores measured no faster.)  The multi-token kernel keeps
// four parts of 32 rows (two rows a lane): with eight it went 225 -> 275 us.
constexpr int DEC_THREADS = 256;
constexpr int DEC_PARTS = 8;
constexpr int DEC_IT = 128 / DEC_PARTS / 16;  // rows per 16-lane group
constexpr int MULTI_PARTS = 4;
constexpr int MULTI_IT = 128 / MULTI_PARTS / 16;

// The 8 elements lane l16 of a 16-lane group holds of a 128-wide row.
__device__ __forceinline__ void load_row_halves(const float* row, int l16, float* out) {
  const float4 a = *reinterpret_cast<const float4*>(row + 4 * l16);
  const float4 b = *reinterpret_cast<const float4*>(row + 64 + 4 * l16);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}
template <typename T>
__device__ __forceinline__ void load_row_halves(const T* row, int l16, float* out) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[j] = load1(row + 4 * l16 + j);
    out[4 + j] = load1(row + 64 + 4 * l16 + j);
  }
}
// State rows (and snapshots) are written once per call and not read again
// before other layers' traffic evicts them: non-temporal stores.  The
// multi-token kernel, which writes a snapshot per token, ran 9-14% faster
// with them (decode_rows alone no differently).
__device__ __forceinline__ void store_row_halves(float* row, int l16, const float* in) {
  __builtin_nontemporal_store(f32x4{in[0], in[1], in[2], in[3]},
                              reinterpret_cast<f32x4*>(row + 4 * l16));
  __builtin_nontemporal_store(f32x4{in[4], in[5], in[6], in[7]},
                              reinterpret_cast<f32x4*>(row + 64 + 4 * l16));
}

template <typename T, typename G>
__global__ __launch_bounds__(DEC_THREADS) void decode_rows_kernel(
    const T* __restrict__ q, int64_t q_rs, const T* __restrict__ k, int64_t k_rs,
    const T* __restrict__ v, int64_t v_rs, const G* __restrict__ a, const G* __restrict__ b,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias, float* __restrict__ state,
    const int32_t* __restrict__ lengths, T* __restrict__ o, int Hk, int Hv, float q_scale) {
  const int part = blockIdx.x % DEC_PARTS;
  const int rh = blockIdx.x / DEC_PARTS;
  const int r = rh / Hv;
  const int h = rh - r * Hv;
  const int kh = h / (Hv / Hk);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, grp = lane >> 4, l16 = lane & 15;
  const int row0 = part * (128 / DEC_PARTS) + wave * 4 * DEC_IT + grp;  // + 4 it
  T* ob = o + ((int64_t)r * Hv + h) * 128;
  if (lengths && lengths[r] < 0) {  // idle row: state untouched, output zero
    if (tid < 128 / DEC_PARTS) store1(ob + part * (128 / DEC_PARTS) + tid, 0.0f);
    return;
  }
  float* Sb = state + ((int64_t)r * Hv + h) * (128 * 128);
  float s[DEC_IT][8];
#pragma unroll
  for (int it = 0; it < DEC_IT; ++it) load_row_halves(Sb + (row0 + 4 * it) * 128, l16, s[it]);

  float kv[8], qv[8];
  load_row_halves(k + r * k_rs + kh * 128, l16, kv);
  load_row_halves(q + r * q_rs + kh * 128, l16, qv);
#pragma unroll
  for (int i = 0; i < 8; ++i) qv[i] *= q_scale;
  float vr[DEC_IT];
#pragma unroll
  for (int it = 0; it < DEC_IT; ++it) vr[it] = load1(v + r * v_rs + h * 128 + row0 + 4 * it);
  const float al = expf(gate_log_alpha(load1(a + (int64_t)r * Hv + h), A_log[h], dt_bias[h]));
  const float be = gate_beta(load1(b + (int64_t)r * Hv + h));
  const float kq = sum16(dot8(kv, qv));

#pragma unroll
  for (int it = 0; it < DEC_IT; ++it) {
    const int row = row0 + 4 * it;
    const float su = sum16(dot8(s[it], kv));
    const float sq = sum16(dot8(s[it], qv));
    const float d = be * (vr[it] - al * su);
    float sn[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sn[i] = fmaf(al, s[it][i], d * kv[i]);
    store_row_halves(Sb + row * 128, l16, sn);
    if (l16 == 0) store1(ob + row, fmaf(al, sq, d * kq));
  }
}

// ---------------------------------------------------------------------------
// decode_rows over K tokens per row (a draft of K tokens to verify): the same
// mapping, the state held in registers across the K tokens, so it is read and
// written once; optionally the state after each token is written to
// snapshots[r][t] (the states a verifier rolls back to).  Each token's
// arithmetic is that of decode_rows_kernel, in the same order, so K tokens
// here equal K successive decode_rows calls bit for bit.
template <typename T, typename G>
__global__ __launch_bounds__(DEC_THREADS) void decode_rows_multi_kernel(
    const T* __restrict__ q, int64_t q_rs, int64_t q_ts, const T* __restrict__ k, int64_t k_rs,
    int64_t k_ts, const T* __restrict__ v, int64_t v_rs, int64_t v_ts, const G* __restrict__ a,
    const G* __restrict__ b, const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    float* __restrict__ state, float* __restrict__ snapshots, const int32_t* __restrict__ lengths,
    T* __restrict__ o, int K, int Hk, int Hv, float q_scale) {
  const int part = blockIdx.x % MULTI_PARTS;
  const int rh = blockIdx.x / MULTI_PARTS;
  const int r = rh / Hv;
  const int h = rh - r * Hv;
  const int kh = h / (Hv / Hk);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, grp = lane >> 4, l16 = lane & 15;
  const int row0 = part * (128 / MULTI_PARTS) + wave * 4 * MULTI_IT + grp;  // + 4 it
  if (lengths && lengths[r] < 0) {  // idle row: state and snapshots untouched, output zero
    for (int t = 0; t < K; ++t)
      if (tid < 128 / MULTI_PARTS)
        store1(o + (((int64_t)r * K + t) * Hv + h) * 128 + part * (128 / MULTI_PARTS) + tid, 0.0f);
    return;
  }
  float* Sb = state + ((int64_t)r * Hv + h) * (128 * 128);
  float s[MULTI_IT][8];
#pragma unroll
  for (int it = 0; it < MULTI_IT; ++it) load_row_halves(Sb + (row0 + 4 * it) * 128, l16, s[it]);
  const float Al = A_log[h], Db = dt_bias[h];

  for (int t = 0; t < K; ++t) {
    float kv[8], qv[8];
    load_row_halves(k + r * k_rs + t * k_ts + kh * 128, l16, kv);
    load_row_halves(q + r * q_rs + t * q_ts + kh * 128, l16, qv);
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] *= q_scale;
    float vr[MULTI_IT];
#pragma unroll
    for (int it = 0; it < MULTI_IT; ++it)
      vr[it] = load1(v + r * v_rs + t * v_ts + h * 128 + row0 + 4 * it);
    const int64_t gi = ((int64_t)r * K + t) * Hv + h;
    const float al = expf(gate_log_alpha(load1(a + gi), Al, Db));
    const float be = gate_beta(load1(b + gi));
    const float kq = sum16(dot8(kv, qv));
    T* ob = o + gi * 128;
    float* snap = snapshots ? snapshots + (((int64_t)r * K + t) * Hv + h) * (128 * 128) : nullptr;
#pragma unroll
    for (int it = 0; it < MULTI_IT; ++it) {
      const int row = row0 + 4 * it;
      const float su = sum16(dot8(s[it], kv));
      const float sq = sum16(dot8(s[it], qv));
      const float d = be * (vr[it] - al * su);
#pragma unroll
      for (int i = 0; i < 8; ++i) s[it][i] = fmaf(al, s[it][i], d * kv[i]);
      if (snap) store_row_halves(snap + row * 128, l16, s[it]);
      if (l16 == 0) store1(ob + row, fmaf(al, sq, d * kq));
    }
  }
#pragma unroll
  for (int it = 0; it < MULTI_IT; ++it) store_row_halves(Sb + (row0 + 4 * it) * 128, l16, s[it]);
}

// ---------------------------------------------------------------------------
// Sequential prefill: state rows live in registers for the whole sequence.
// One workgroup per (batch, value head, block of 16 value rows); tokens are
// staged SEQ_TT at a time in LDS (k, q as f32, this block's v, the gates),
// then each 16-lane group runs the recurrence for its row.
constexpr int SEQ_THREADS = 256;
constexpr int SEQ_TT = 32;

template <typename T, typename G, typename TO>
__global__ __launch_bounds__(SEQ_THREADS) void recurrent_prefill_kernel(
    const T* __restrict__ q, int64_t q_ts, const T* __restrict__ k, int64_t k_ts,
    const T* __restrict__ v, int64_t v_ts, const G* __restrict__ a, const G* __restrict__ b,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    const float* state_in, float* state_out, TO* __restrict__ o, int Tlen,
    const int32_t* __restrict__ cu, int total, int Hk, int Hv, float q_scale) {
  __shared__ float ks[SEQ_TT][128];
  __shared__ float qs[SEQ_TT][128];
  __shared__ float vs[SEQ_TT][16];
  __shared__ float als[SEQ_TT], bes[SEQ_TT];

  const int blk = blockIdx.x & 7;
  const int bh = blockIdx.x >> 3;
  const int h = bh % Hv;
  const int bb = bh / Hv;
  const int kh = h / (Hv / Hk);
  const int tid = threadIdx.x, grp = tid >> 4, l16 = tid & 15;
  const int row = blk * 16 + grp;
  const float Al = A_log[h], Db = dt_bias[h];

  const int64_t sbase = ((int64_t)bb * Hv + h) * (128 * 128) + (int64_t)row * 128 + l16 * 8;
  float s[8];
  if (state_in) load8(state_in + sbase, s);
  else {
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = 0.0f;
  }

  // Row bb's tokens: Tlen at stride Tlen, or with cu (device [B + 1] offsets
  // into a packed axis of `total` tokens) [cu[bb], cu[bb+1]), at most Tlen of
  // them; offsets are clamped into [0, total].
  int64_t tbase = (int64_t)bb * Tlen;
  int tlen = Tlen;
  if (cu != nullptr) {
    const int s0 = max(0, min(cu[bb], total));
    const int e0 = max(s0, min(cu[bb + 1], total));
    tbase = s0;
    tlen = min(e0 - s0, Tlen);
  }
  const T* qb = q + tbase * q_ts + kh * 128;
  const T* kb = k + tbase * k_ts + kh * 128;
  const T* vb = v + tbase * v_ts + h * 128 + blk * 16;
  const G* ab = a + tbase * Hv + h;
  const G* bbp = b + tbase * Hv + h;
  TO* obp = o + (tbase * Hv + h) * 128 + row;

  for (int t0 = 0; t0 < tlen; t0 += SEQ_TT) {
    const int n = min(SEQ_TT, tlen - t0);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int tt = grp + 16 * half;
      if (tt < n) {
        float tmp[8];
        load8(kb + (int64_t)(t0 + tt) * k_ts + l16 * 8, tmp);
        *reinterpret_cast<float4*>(&ks[tt][l16 * 8]) = make_float4(tmp[0], tmp[1], tmp[2], tmp[3]);
        *reinterpret_cast<float4*>(&ks[tt][l16 * 8 + 4]) = make_float4(tmp[4], tmp[5], tmp[6], tmp[7]);
        load8(qb + (int64_t)(t0 + tt) * q_ts + l16 * 8, tmp);
#pragma unroll
        for (int i = 0; i < 8; ++i) tmp[i] *= q_scale;
        *reinterpret_cast<float4*>(&qs[tt][l16 * 8]) = make_float4(tmp[0], tmp[1], tmp[2], tmp[3]);
        *reinterpret_cast<float4*>(&qs[tt][l16 * 8 + 4]) = make_float4(tmp[4], tmp[5], tmp[6], tmp[7]);
      }
    }
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int idx = tid + rep * SEQ_THREADS;
      const int tt = idx >> 4, j = idx & 15;
      if (tt < n) vs[tt][j] = load1(vb + (int64_t)(t0 + tt) * v_ts + j);
    }
    if (tid < n) {
      als[tid] = expf(gate_log_alpha(load1(ab + (int64_t)(t0 + tid) * Hv), Al, Db));
      bes[tid] = gate_beta(load1(bbp + (int64_t)(t0 + tid) * Hv));
    }
    __syncthreads();
    for (int tt = 0; tt < n; ++tt) {
      float kv[8], qv[8];
      const float4 k0 = *reinterpret_cast<const float4*>(&ks[tt][l16 * 8]);
      const float4 k1 = *reinterpret_cast<const float4*>(&ks[tt][l16 * 8 + 4]);
      const float4 q0 = *reinterpret_cast<const float4*>(&qs[tt][l16 * 8]);
      const float4 q1 = *reinterpret_cast<const float4*>(&qs[tt][l16 * 8 + 4]);
      kv[0] = k0.x; kv[1] = k0.y; kv[2] = k0.z; kv[3] = k0.w;
      kv[4] = k1.x; kv[5] = k1.y; kv[6] = k1.z; kv[7] = k1.w;
      qv[0] = q0.x; qv[1] = q0.y; qv[2] = q0.z; qv[3] = q0.w;
      qv[4] = q1.x; qv[5] = q1.y; qv[6] = q1.z; qv[7] = q1.w;
      const float al = als[tt], be = bes[tt];
      const float su = sum16(dot8(s, kv));
      const float sq = sum16(dot8(s, qv));
      const float kq = sum16(dot8(kv, qv));
      const float d = be * (vs[tt][grp] - al * su);
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] = fmaf(al, s[i], d * kv[i]);
      if (l16 == 0) store1(obp + (int64_t)(t0 + tt) * Hv * 128, fmaf(al, sq, d * kq));
    }
    __syncthreads();
  }
  if (state_out) store8(state_out + sbase, s);
}

template <typename T, typename G>
static void launch_decode_t(const void* q, int64_t q_rs, const void* k, int64_t k_rs,
                            const void* v, int64_t v_rs, const void* a, const void* b,
                            const float* A_log, const float* dt_bias, float* state,
                            const int32_t* lengths, void* o, int R, int Hk, int Hv, float q_scale,
                            hipStream_t stream) {
  hipLaunchKernelGGL((decode_rows_kernel<T, G>), dim3(R * Hv * DEC_PARTS), dim3(DEC_THREADS), 0,
                     stream,
                     (const T*)q, q_rs, (const T*)k, k_rs, (const T*)v, v_rs, (const G*)a,
                     (const G*)b, A_log, dt_bias, state, lengths, (T*)o, Hk, Hv, q_scale);
}

hipError_t launch_decode_rows(const void* q, int64_t q_rs, const void* k, int64_t k_rs,
                              const void* v, int64_t v_rs, int qkv_dt, const void* a,
                              const void* b, int gate_dt, const float* A_log,
                              const float* dt_bias, float* state, const int32_t* lengths, void* o,
                              int R, int Hk, int Hv, float q_scale, hipStream_t stream) {
  if (qkv_dt == 1 && gate_dt == 1)
    launch_decode_t<uint16_t, uint16_t>(q, q_rs, k, k_rs, v, v_rs, a, b, A_log, dt_bias, state,
                                        lengths, o, R, Hk, Hv, q_scale, stream);
  else if (qkv_dt == 1)
    launch_decode_t<uint16_t, float>(q, q_rs, k, k_rs, v, v_rs, a, b, A_log, dt_bias, state,
                                     lengths, o, R, Hk, Hv, q_scale, stream);
  else if (gate_dt == 1)
    launch_decode_t<float, uint16_t>(q, q_rs, k, k_rs, v, v_rs, a, b, A_log, dt_bias, state,
                                     lengths, o, R, Hk, Hv, q_scale, stream);
  else
    launch_decode_t<float, float>(q, q_rs, k, k_rs, v, v_rs, a, b, A_log, dt_bias, state,
                                  lengths, o, R, Hk, Hv, q_scale, stream);
  return hipGetLastError();
}

template <typename T, typename G>
static void launch_decode_multi_t(const void* q, int64_t q_rs, int64_t q_ts, const void* k,
                                  int64_t k_rs, int64_t k_ts, const void* v, int64_t v_rs,
                                  int64_t v_ts, const void* a, const void* b, const float* A_log,
                                  const float* dt_bias, float* state, float* snapshots,
                                  const int32_t* lengths, void* o, int R, int K, int Hk, int Hv,
                                  float q_scale, hipStream_t stream) {
  hipLaunchKernelGGL((decode_rows_multi_kernel<T, G>), dim3(R * Hv * MULTI_PARTS), dim3(DEC_THREADS),
                     0, stream,
                     (const T*)q, q_rs, q_ts, (const T*)k, k_rs, k_ts, (const T*)v, v_rs, v_ts,
                     (const G*)a, (const G*)b, A_log, dt_bias, state, snapshots, lengths, (T*)o, K,
                     Hk, Hv, q_scale);
}

hipError_t launch_decode_rows_multi(const void* q, int64_t q_rs, int64_t q_ts, const void* k,
                                    int64_t k_rs, int64_t k_ts, const void* v, int64_t v_rs,
                                    int64_t v_ts, int qkv_dt, const void* a, const void* b,
                                    int gate_dt, const float* A_log, const float* dt_bias,
                                    float* state, float* snapshots, const int32_t* lengths,
                                    void* o, int R, int K, int Hk, int Hv, float q_scale,
                                    hipStream_t stream) {
  if (qkv_dt == 1 && gate_dt == 1)
    launch_decode_multi_t<uint16_t, uint16_t>(q, q_rs, q_ts, k, k_rs, k_ts, v, v_rs, v_ts, a, b,
                                              A_log, dt_bias, state, snapshots, lengths, o, R, K,
                                              Hk, Hv, q_scale, stream);
  else if (qkv_dt == 1)
    launch_decode_multi_t<uint16_t, float>(q, q_rs, q_ts, k, k_rs, k_ts, v, v_rs, v_ts, a, b,
                                           A_log, dt_bias, state, snapshots, lengths, o, R, K, Hk,
                                           Hv, q_scale, stream);
  else if (gate_dt == 1)
    launch_decode_multi_t<float, uint16_t>(q, q_rs, q_ts, k, k_rs, k_ts, v, v_rs, v_ts, a, b,
                                           A_log, dt_bias, state, snapshots, lengths, o, R, K, Hk,
                                           Hv, q_scale, stream);
  else
    launch_decode_multi_t<float, float>(q, q_rs, q_ts, k, k_rs, k_ts, v, v_rs, v_ts, a, b, A_log,
                                        dt_bias, state, snapshots, lengths, o, R, K, Hk, Hv,
                                        q_scale, stream);
  return hipGetLastError();
}

template <typename T, typename G, typename TO>
static void launch_seq_t(const void* q, int64_t q_ts, const void* k, int64_t k_ts, const void* v,
                         int64_t v_ts, const void* a, const void* b, const float* A_log,
                         const float* dt_bias, const float* state_in, float* state_out, void* o,
                         int B, int Tlen, const int32_t* cu, int total, int Hk, int Hv,
                         float q_scale, hipStream_t stream) {
  hipLaunchKernelGGL((recurrent_prefill_kernel<T, G, TO>), dim3(B * Hv * 8), dim3(SEQ_THREADS), 0,
                     stream, (const T*)q, q_ts, (const T*)k, k_ts, (const T*)v, v_ts, (const G*)a,
                     (const G*)b, A_log, dt_bias, state_in, state_out, (TO*)o, Tlen, cu, total,
                     Hk, Hv, q_scale);
}

template <typename T, typename G>
static void launch_seq_o(int o_dt, const void* q, int64_t q_ts, const void* k, int64_t k_ts,
                         const void* v, int64_t v_ts, const void* a, const void* b,
                         const float* A_log, const float* dt_bias, const float* state_in,
                         float* state_out, void* o, int B, int Tlen, const int32_t* cu, int total,
                         int Hk, int Hv, float q_scale, hipStream_t stream) {
  if (o_dt == 1)
    launch_seq_t<T, G, uint16_t>(q, q_ts, k, k_ts, v, v_ts, a, b, A_log, dt_bias, state_in,
                                 state_out, o, B, Tlen, cu, total, Hk, Hv, q_scale, stream);
  else
    launch_seq_t<T, G, float>(q, q_ts, k, k_ts, v, v_ts, a, b, A_log, dt_bias, state_in,
                              state_out, o, B, Tlen, cu, total, Hk, Hv, q_scale, stream);
}

hipError_t launch_prefill_sequential(const void* q, int64_t q_ts, const void* k, int64_t k_ts,
                                     const void* v, int64_t v_ts, int qkv_dt, const void* a,
                                     const void* b, int gate_dt, const float* A_log,
                                     const float* dt_bias, const float* state_in,
                                     float* state_out, void* o, int o_dt, int B, int T,
                                     const int32_t* cu, int total, int Hk, int Hv, float q_scale,
                                     hipStream_t stream) {
  if (qkv_dt == 1 && gate_dt == 1)
    launch_seq_o<uint16_t, uint16_t>(o_dt, q, q_ts, k, k_ts, v, v_ts, a, b, A_log, dt_bias,
                                     state_in, state_out, o, B, T, cu, total, Hk, Hv, q_scale, stream);
  else if (qkv_dt == 1)
    launch_seq_o<uint16_t, float>(o_dt, q, q_ts, k, k_ts, v, v_ts, a, b, A_log, dt_bias, state_in,
                                  state_out, o, B, T, cu, total, Hk, Hv, q_scale, stream);
  else if (gate_dt == 1)
    launch_seq_o<float, uint16_t>(o_dt, q, q_ts, k, k_ts, v, v_ts, a, b, A_log, dt_bias, state_in,
                                  state_out, o, B, T, cu, total, Hk, Hv, q_scale, stream);
  else
    launch_seq_o<float, float>(o_dt, q, q_ts, k, k_ts, v, v_ts, a, b, A_log, dt_bias, state_in,
                               state_out, o, B, T, cu, total, Hk, Hv, q_scale, stream);
  return hipGetLastError();
}

}  // namespace gdn
