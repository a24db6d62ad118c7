// Chunked prefill of the gated delta rule on bf16 MFMA (gfx950).  The rule
// ("Qwen3.8 27B" model card, Gated DeltaNet bullet):
//   S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,  o_t = S_t q_t.
//
// Chunk form (exact in exact arithmetic).  For a chunk of n <= 64 tokens with
// G_t = sum_{s<=t} log a_s, gamma_t = e^{G_t}, H = S^T [dk, dv]:
//   A_tj = b_t e^{G_t - G_j} (k_t . k_j)  (j < t),   T = (I + A)^{-1}
//   W  = T diag(b gamma) K,   Ut = T diag(b) V
//   U  = Ut - W H
//   O  = diag(gamma) Q H + (M o Q K^T) U,   M_tj = e^{G_t - G_j} (j <= t)
//   H' = gamma_last H + K^T diag(e^{G_last - G_s}) U
// Only non-positive exponents are ever taken.  Padding rows of a short last
// chunk carry g = 0, b = 0 and zero k/q/v, which leaves every formula exact.
//
// Two kernels:
//  * chunk_prep: four waves per (batch, value head, chunk), fully parallel.
//    Gates and their prefix sum; K K^T and Q K^T on MFMA; T by blocks: the
//    four 16x16 diagonal blocks by forward substitution in f32, the six
//    off-diagonal blocks by three levels of 16x16x16 MFMA products; then W
//    and Ut on MFMA.  The chunk's K and Q rows are loaded coalesced and
//    staged in LDS (f32 rows in two halves of 64 dims), where each wave
//    reads its operand fragments.  Writes W, Ut^T, P = q_scale M o QK^T, the
//    decay factors e^{G_t} and e^{G_last - G_t} (f32) and (once per q/k
//    head) K^T and Q to the workspace, each in the order the chain's lanes
//    load it.  With f32 q/k, K K^T and Q K^T are formed from a two-term bf16
//    split of both operands: k_s . k_t and q . k are small next to the
//    vectors' norms (unit vectors in 128 dimensions), so they need more than
//    bf16 operand precision.  A flagged chunk (below) also forms T again
//    from split operands.
//  * chunk_chain: one workgroup per (batch, value head, slice of dv: 32
//    columns, or 64 when the batch has more 32-column slices than CUs),
//    sequential over chunks.  The f32 state slice lives in MFMA
//    accumulator registers of four state waves; four output waves form O.
//    Each wave loads its own operands two chunks ahead straight into
//    registers; the bf16 copy of the state and U^T are exchanged in LDS.
//    The dv columns of H are independent, which is what allows the slicing.
#include <type_traits>

#include "chunk_common.hpp"
#include "launch.hpp"

namespace gdn {

using namespace chunk;

namespace {

// Ut and P of a chunk-head flagged by the prep also get a second bf16 part
// (lo = bf16(x - hi), so hi + lo carries ~16 significant bits).  The chain
// sums U and P over a chunk's tokens; when a chunk's keys are nearly parallel
// and its write rates high, those sums cancel (U_t ~ v_t - v_{t-1}) and a
// one-part bf16 rounding of each term costs ~2% of the result.  The flag
// (F) marks such chunks: any |T_ts|, s < t, of T = (I + A)^{-1} above
// kSplitThreshold.  Unflagged chunks leave the lo parts unwritten and unread.
struct WsLayout {
  uint16_t* W;    // [B*Hv*NC][8192]  Wf
  uint16_t* Ut;   // [B*Hv*NC][8192]  Utf, hi part
  uint16_t* UtL;  // [B*Hv*NC][8192]  Utf, lo part
  uint16_t* P;    // [B*Hv*NC][4096]  Pf, hi part
  uint16_t* PL;   // [B*Hv*NC][4096]  Pf, lo part
  float* G;       // [B*Hv*NC][128]: e^{G_t} (t < 64), then e^{G_last - G_t} (t < 64)
  uint16_t* Kt;   // [B*Hk*NC][8192]  Ktf
  uint16_t* Qb;   // [B*Hk*NC][8192]  Qf
  int32_t* F;     // [B*Hv*NC]: 1 if the chunk-head uses the two-part Ut and P
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(void* base, int B, int T, int Hk, int Hv) {
  const size_t NC = (size_t)(T + CK - 1) / CK;
  const size_t nch = (size_t)B * Hv * NC, nck = (size_t)B * Hk * NC;
  char* p = static_cast<char*>(base);
  WsLayout L;
  L.W = reinterpret_cast<uint16_t*>(p);   p += align256(nch * CK * DH * 2);
  L.Ut = reinterpret_cast<uint16_t*>(p);  p += align256(nch * DH * CK * 2);
  L.UtL = reinterpret_cast<uint16_t*>(p); p += align256(nch * DH * CK * 2);
  L.P = reinterpret_cast<uint16_t*>(p);   p += align256(nch * CK * CK * 2);
  L.PL = reinterpret_cast<uint16_t*>(p);  p += align256(nch * CK * CK * 2);
  L.G = reinterpret_cast<float*>(p);     p += align256(nch * 2 * CK * 4);
  L.Kt = reinterpret_cast<uint16_t*>(p); p += align256(nck * DH * CK * 2);
  L.Qb = reinterpret_cast<uint16_t*>(p); p += align256(nck * CK * DH * 2);
  L.F = reinterpret_cast<int32_t*>(p);   p += align256(nch * 4);
  return L;
}

}  // namespace

size_t prefill_chunked_workspace_bytes(int B, int T, int Hk, int Hv) {
  const size_t NC = (size_t)(T + CK - 1) / CK;
  const size_t nch = (size_t)B * Hv * NC, nck = (size_t)B * Hk * NC;
  return align256(nch * CK * DH * 2) + 2 * align256(nch * DH * CK * 2) +
         2 * align256(nch * CK * CK * 2) + align256(nch * 2 * CK * 4) +
         align256(nck * DH * CK * 2) + align256(nck * CK * DH * 2) + align256(nch * 4);
}

// Token span of row bb: rows of T tokens at stride T, or, with cu (device
// [rows + 1] offsets into a packed token axis of `total` tokens), row bb's
// tokens [cu[bb], cu[bb+1]), at most T of them (T is then the longest row).
// The offsets are clamped into [0, total], so bad offsets cannot reach
// outside the token arrays.
__device__ __forceinline__ void row_span(const int32_t* cu, int total, int bb, int T,
                                         int64_t& base, int& len) {
  if (cu == nullptr) {
    base = (int64_t)bb * T;
    len = T;
    return;
  }
  const int s = max(0, min(cu[bb], total));
  const int e = max(s, min(cu[bb + 1], total));
  base = s;
  len = min(e - s, T);
}

// Value head (and slice) of the r-th workgroup of a round: workgroups whose
// ids agree mod 8 run on one XCD, and the XCD's k-th unit (of `per` units per
// head, grp heads per q/k group) belongs to group (k / (grp per)) * 8 + xcd,
// so a group's heads and slices share an XCD and its L2, and groups are dealt
// round-robin over the XCDs.  Needs a whole number of groups per XCD round;
// otherwise the plain order (heads round-robin).  Returns head * per + slice.
__device__ __forceinline__ int xcd_head(int r, int ngroups, int grp, int per) {
  if ((ngroups & 7) != 0) return r;
  const int x = r & 7, k = r >> 3;
  const int g = (k / (grp * per)) * 8 + x, rest = k % (grp * per);
  return (g * grp + rest / per) * per + rest % per;
}

// ---------------------------------------------------------------------------
// Phase 1: per (batch, value head, chunk), four waves.  Wave w owns token
// block w (16 tokens) of every tile loop; the serial parts of the inverse run
// on wave 0 while the others wait at LDS-only barriers.
constexpr int PREP_THREADS = 256;
// Floor of a token's log-decay in the chunk form (see the gate computation).
// e^{-128} is below the smallest f32 subnormal, and a chunk's prefix sums stay
// within 64 * 128, where f32 differences keep ~1e-3 absolute accuracy.
constexpr float kLogAlphaFloor = 128.0f;
// A chunk-head whose T = (I + A)^{-1} has an off-diagonal entry above this in
// magnitude keeps Ut and P in two bf16 parts.  Measured against the f64
// definition on CPU emulations of the chunk arithmetic over a grid of key
// correlations, write rates and decays: with every |T_ts| below 0.4 the
// one-part form stays within 1e-2; the 1e-2..3e-2 errors start near 0.45
// (nearly parallel keys, write rates near 1, slow decay).  Random unit keys
// give 0.1-0.3; the keys of the whole mixer (conv + silu + L2) 0.25-0.47.
constexpr float kSplitThreshold = 0.4f;

template <typename TI, typename TV, typename G_T>
__global__ __launch_bounds__(PREP_THREADS, 3) void chunk_prep_kernel(
    const TI* __restrict__ q, int64_t q_ts, const TI* __restrict__ k, int64_t k_ts,
    const TV* __restrict__ v, int64_t v_ts, const G_T* __restrict__ a,
    const G_T* __restrict__ b, const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    WsLayout ws, int T, const int32_t* __restrict__ cu, int total, int Hk, int Hv, int NC,
    float q_scale) {
  constexpr bool kSplit = sizeof(TI) == 4;  // f32 q/k: two-term K K^T and Q K^T
  // Region R: first A (f32 [64][FP]), then K^T, then V^T (bf16 [128][XP]).
  // T (f32 [64][FP]) follows R and lives from the inverse to the end.  With
  // bf16 q/k the block first holds the chunk's K and Q rows as loaded
  // ([64][RP] each), until every wave has its operand fragments.
  constexpr int kRegion = DH * XP;  // halves; A (CK * FP * 2 halves) fits in it
  static_assert(CK * FP * 2 <= kRegion, "A fits in region R");
  constexpr int kTotal = kRegion + CK * FP * 2;
  constexpr int kStage = 2 * CK * RP;
  __shared__ __attribute__((aligned(16))) uint16_t L[kTotal > kStage ? kTotal : kStage];
  __shared__ __attribute__((aligned(16))) float Gs[CK], Bs[CK], BGs[CK];  // G, b, b e^G
  __shared__ float Tmax;  // max |T_ts|, s < t (the two-part flag)
  float* Af = reinterpret_cast<float*>(L);            // A, f32, row-major [64][FP]
  float* Tf = reinterpret_cast<float*>(L + kRegion);  // T, f32, row-major [64][FP]
  uint16_t* XT = L;

  // Chunk-major order: the workgroups of one chunk index run together, so the
  // chain, which reads chunk 0 first, finds every head's data equally recent
  // in the last-level cache.  Ids that agree mod 8 share an XCD; the q/k
  // groups (the value heads that read one q/k head) are dealt round-robin
  // over the XCDs with all of a group's value heads on the same one, so they
  // share its L2 for K and Q, and the rows of a ragged batch spread evenly.
  const int nbh = gridDim.x / NC;
  const int c = blockIdx.x / nbh;
  const int bh = xcd_head(blockIdx.x % nbh, nbh / (Hv / Hk), Hv / Hk, 1);
  const int h = bh % Hv, bb = bh / Hv;
  const int grp = Hv / Hk, kh = h / grp;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;
  int64_t tbase;
  int tlen;
  row_span(cu, total, bb, T, tbase, tlen);
  const int t0 = c * CK;  // within the row
  if (t0 >= tlen) return;  // a shorter row of a ragged batch
  const int n = min(CK, tlen - t0);
  const int64_t chunk = (int64_t)bh * NC + c;

  const TI* kbase = k + (tbase + t0) * k_ts + kh * DH;
  const TI* qbase = q + (tbase + t0) * q_ts + kh * DH;
  const TV* vbase = v + (tbase + t0) * v_ts + h * DH;

  // The chunk's K and Q rows and wave 0's gate inputs are loaded first (V
  // later, below).  Wave w's K K^T and Q K^T tiles (t block, s block; see the
  // calls below) need four 16-row operand blocks:
  //   w 0: K0 K1 Q0 Q1    w 1: K1 K3 Q3 -    w 2: K0 K1 K2 Q2    w 3: K0 K2 K3 Q3
  // (nibble s of the wave's table: bit 3 used, bit 2 Q, bits 0-1 block), read
  // from the rows staged in LDS.
  float a_raw = 0.0f, b_raw = 0.0f;
  if (w == 0 && lane < n) {
    const int64_t gi = (tbase + t0 + lane) * Hv + h;
    a_raw = load1(a + gi);
    b_raw = load1(b + gi);
  }
  const unsigned slots = w == 0 ? 0xDC98u : w == 1 ? 0x0FB9u : w == 2 ? 0xEA98u : 0xFBA8u;
  bf16x8 f[4][4], fl[4][4], vf[4];
  // The chunk's 64 K rows and 64 Q rows are loaded with 16 adjacent lanes
  // per 256-byte row, staged in LDS, and each wave reads its fragments from
  // there.  Loaded straight into fragments instead (the MFMA operand order,
  // lane = row), the rows arrive at about half the rate, and the waves'
  // operand blocks overlap (15 block loads for 8 blocks): prep 68 -> 56 us
  // for bf16, 101 -> 75 us for f32 at B=1 T=4096.
  constexpr bool kStaged = !kSplit;
  typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
  u32x4s stg[8];
  // f32 q/k go through the same block in two halves of 64 dims (a [64][68]
  // f32 tile each for K and Q), both halves' loads issued here.
  constexpr bool kStagedF = kSplit;
  constexpr int RPF = 68;  // f32 pitch of a staged half: 272-byte rows
  u32x4s stgf[2][8];
  if (kStagedF) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int u = (j & 3) * PREP_THREADS + tid;  // 16-byte unit of a [64][64] f32 half
        const int t = u >> 4, col = hh * 64 + (u & 15) * 4;
        const TI* src = (j < 4 ? kbase + (int64_t)t * k_ts : qbase + (int64_t)t * q_ts) + col;
        if (t < n) stgf[hh][j] = *reinterpret_cast<const u32x4s*>(src);
        else stgf[hh][j] = u32x4s{0u, 0u, 0u, 0u};
      }
  }
  if (kStaged) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int u = (j & 3) * PREP_THREADS + tid;  // 16-byte unit of a [64][128] tile
      const int t = u >> 4, col = (u & 15) * 8;
      const TI* src = (j < 4 ? kbase + (int64_t)t * k_ts : qbase + (int64_t)t * q_ts) + col;
      if (t < n) stg[j] = *reinterpret_cast<const u32x4s*>(src);
      else stg[j] = u32x4s{0u, 0u, 0u, 0u};
    }
  }
  // V block w, loaded once the K K^T / Q K^T tiles are done (it is first
  // used for Ut, after the inverse).  In flight from entry, its words would
  // sit beside the K/Q operand blocks: with f32 input that pushes the kernel
  // past the 168 registers that let three workgroups share a SIMD, and with
  // bf16 it costs 17 registers (123 against 106) for no gain.
  auto load_v = [&]() {
    const int t = w * 16 + li;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 unused;
      if (t < n) load_row8(vbase + (int64_t)t * v_ts + kk * 32 + lg * 8, vf[kk], unused);
      else vf[kk] = zero_frag();
    }
  };

  // Gates for token `lane` (wave 0); padding tokens get g = 0, b = 0.
  // g is floored at -kLogAlphaFloor: alpha = 0 (a = +inf, or an overflowing
  // softplus) would give g = -inf and NaN differences G_t - G_s.  Every decay
  // factor that spans such a token is then e^{<= -128}, which is 0 in f32, as
  // alpha itself is; a NaN g stays NaN.
  if (w == 0) {
    float g = 0.0f, be = 0.0f;
    if (lane < n) {
      g = gate_log_alpha(a_raw, A_log[h], dt_bias[h]);
      if (g < -kLogAlphaFloor) g = -kLogAlphaFloor;
      be = gate_beta(b_raw);
    }
    const float Gl = wave_scan(g, lane);
    Gs[lane] = Gl;
    Bs[lane] = be;
    BGs[lane] = be * __expf(Gl);
    // The chain's decay factors, computed once here rather than in its
    // sequential steps: e^{G_t}, and e^{G_last - G_t} (G_last = G_63, since
    // padding tokens add g = 0).
    ws.G[chunk * 2 * CK + lane] = __expf(Gl);
    ws.G[chunk * 2 * CK + CK + lane] = __expf(__shfl(Gl, CK - 1) - Gl);
  }
  if (kStaged) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int u = (j & 3) * PREP_THREADS + tid;
      *reinterpret_cast<u32x4s*>(&L[(j >> 2) * CK * RP + (u >> 4) * RP + (u & 15) * 8]) = stg[j];
    }
  }
  lds_barrier();
  if (kStaged) {
    // Wave w's operand blocks (slot code: bit 3 used, bit 2 Q, bits 0-1 block).
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const int code = (slots >> (4 * sl)) & 15;
      const uint16_t* base = L + ((code >> 2) & 1) * CK * RP + ((code & 3) * 16 + li) * RP + lg * 8;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (code & 8) f[sl][kk] = ld_frag(base + kk * 32);
        else f[sl][kk] = zero_frag();
        fl[sl][kk] = zero_frag();
      }
    }
    lds_barrier();  // the block is rewritten by the K K^T tiles below
  }
  if (kStagedF) {
    float* Lf = reinterpret_cast<float*>(L);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (hh == 1) lds_barrier();  // every wave has read the first half
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int u = (j & 3) * PREP_THREADS + tid;
        *reinterpret_cast<u32x4s*>(&Lf[(j >> 2) * CK * RPF + (u >> 4) * RPF + (u & 15) * 4]) =
            stgf[hh][j];
      }
      lds_barrier();
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const int code = (slots >> (4 * sl)) & 15;
        const float* base =
            Lf + ((code >> 2) & 1) * CK * RPF + ((code & 3) * 16 + li) * RPF + lg * 8;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int kk = hh * 2 + k2;
          if (code & 8) {
            load_row8(base + k2 * 32, f[sl][kk], fl[sl][kk]);
          } else {
            f[sl][kk] = zero_frag();
            fl[sl][kk] = zero_frag();
          }
        }
      }
    }
    lds_barrier();  // the block is rewritten by the K K^T tiles below
  }

  // K K^T tile (tb, sb) from slots (st, ss) -> A: D[t][s], lane (li = s, lg)
  // holds t = 16 tb + 4 lg + r; the diagonal blocks in f32, the others bf16.
  auto kkt = [&](int st, int ss, int tb, int sb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kSplit) {
        acc = mfma16(f[st][kk], fl[ss][kk], acc);
        acc = mfma16(fl[st][kk], f[ss][kk], acc);
      }
      acc = mfma16(f[st][kk], f[ss][kk], acc);
    }
    const int s = sb * 16 + li;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = tb * 16 + lg * 4 + r;
      Af[t * FP + s] = (s < t) ? Bs[t] * __expf(Gs[t] - Gs[s]) * acc[r] : 0.0f;
    }
  };
  // (Q K^T)^T tile [s block sb][t block tb] from Q slot qs and K slot ks:
  // C[s][t] = K_s . Q_t -> P in the chain's fragment order.
  // The lo parts of this lane's P values wait in registers (slot = call
  // number) until the inverse tells whether the chunk needs them.
  u16x4 plo[4];
  int poff[4];
  auto qkt = [&](int qs, int ks, int tb, int sb, int slot) {
    f32x4 pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      pq = mfma16(f[ks][kk], f[qs][kk], pq);
      if (kSplit) {
        pq = mfma16(f[ks][kk], fl[qs][kk], pq);
        pq = mfma16(fl[ks][kk], f[qs][kk], pq);
      }
    }
    const int tq = tb * 16 + li;
    float pv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int sq = sb * 16 + lg * 4 + r;
      pv[r] = (sq <= tq) ? q_scale * __expf(Gs[tq] - Gs[sq]) * pq[r] : 0.0f;
    }
    const int off = frag_off(tq, sb * 16 + lg * 4, 2);
    u16x4 h;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      h[r] = f2bf(pv[r]);
      plo[slot][r] = f2bf(pv[r] - bf2f(h[r]));
    }
    *reinterpret_cast<u16x4*>(ws.P + chunk * (CK * CK) + off) = h;
    poff[slot] = off;
  };
  // Zero tile of P above the diagonal at (tb, tb + 1): the chain reads (0,1)
  // and (2,3) of them (P is used in 32-column steps).
  auto pzero = [&](int tb, int slot) {
    const int off = frag_off(tb * 16 + li, (tb + 1) * 16 + lg * 4, 2);
    const u16x4 z = {0, 0, 0, 0};
    *reinterpret_cast<u16x4*>(ws.P + chunk * (CK * CK) + off) = z;
    plo[slot] = z;
    poff[slot] = off;
  };
  if (w == 0) {
    kkt(0, 0, 0, 0); kkt(1, 0, 1, 0);
    qkt(2, 0, 0, 0, 0); qkt(3, 0, 1, 0, 1); qkt(3, 1, 1, 1, 2);
    pzero(0, 3);
  } else if (w == 1) {
    kkt(0, 0, 1, 1); kkt(1, 0, 3, 1);
    qkt(2, 0, 3, 1, 0); qkt(2, 1, 3, 3, 1);
  } else if (w == 2) {
    kkt(2, 2, 2, 2); kkt(2, 0, 2, 0); kkt(2, 1, 2, 1);
    qkt(3, 0, 2, 0, 0); qkt(3, 1, 2, 1, 1); qkt(3, 2, 2, 2, 2);
    pzero(2, 3);
  } else {
    kkt(2, 2, 3, 3); kkt(2, 0, 3, 0); kkt(2, 1, 3, 2);
    qkt(3, 0, 3, 0, 0); qkt(3, 1, 3, 2, 1);
  }
  load_v();
  lds_barrier();

  // T = (I + A)^{-1} in f32.  Diagonal blocks (wave 0): lane (block lg,
  // column li), forward substitution over the block's 16 rows.  Waves 1-3
  // zero the six blocks above the diagonal.
  float tmax = 0.0f;  // wave 0: max |T_ts|, s < t
  if (w == 0) {
    float x[16];
    const float* Ab = Af + lg * 16 * FP + lg * 16;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float acc = (t == li) ? 1.0f : 0.0f;
#pragma unroll
      for (int s4 = 0; s4 < t; s4 += 4) {
        const float4 a4 = *reinterpret_cast<const float4*>(Ab + t * FP + s4);
        acc = fmaf(-a4.x, x[s4], acc);
        if (s4 + 1 < t) acc = fmaf(-a4.y, x[s4 + 1], acc);
        if (s4 + 2 < t) acc = fmaf(-a4.z, x[s4 + 2], acc);
        if (s4 + 3 < t) acc = fmaf(-a4.w, x[s4 + 3], acc);
      }
      x[t] = acc;
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      Tf[(lg * 16 + t) * FP + lg * 16 + li] = x[t];
      if (t > li) tmax = fmaxf(tmax, fabsf(x[t]));
    }
  } else {
    const int idx = (w - 1) * 64 + lane;  // 0..191: 6 blocks x 16 rows x 2 halves
    const int blk = idx >> 5, row = (idx & 31) >> 1, half = idx & 1;
    const int bi = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
    const int bj = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
    float* dst = &Tf[(bi * 16 + row) * FP + bj * 16 + half * 8];
    *reinterpret_cast<float4*>(dst) = make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  lds_barrier();

  // T, off-diagonal blocks (wave 0): T_ij = -T_ii sum_{j<=m<i} A_im T_mj,
  // level by level on 16x16x16 MFMA; a result (D layout) is the B layout of
  // the next product, so the levels chain in registers.  First with bf16
  // operands; the largest |T_ts| (s < t) of that T decides whether the chunk
  // is a two-part one, and a two-part chunk's blocks are then formed again
  // with both f32 operands split into bf16 hi + lo parts (hi*hi + hi*lo +
  // lo*hi: ~16-bit operands, f32 accumulation).
  if (w == 0) {
    struct Frag { s16x4 hi, lo; };
    auto make = [](float a, float b, float c, float d, auto two) {
      Frag f;
      f.hi = to_s16x4(a, b, c, d);
      if (decltype(two)::value)
        f.lo = to_s16x4(a - bf2f((uint16_t)f.hi[0]), b - bf2f((uint16_t)f.hi[1]),
                        c - bf2f((uint16_t)f.hi[2]), d - bf2f((uint16_t)f.hi[3]));
      return f;
    };
    // A operand: rows of block (i, j) of an f32 LDS matrix, 4 columns per lane.
    auto a_op = [&](const float* M, int i, int j, auto two) {
      const float4 v = *reinterpret_cast<const float4*>(&M[(i * 16 + li) * FP + j * 16 + lg * 4]);
      return make(v.x, v.y, v.z, v.w, two);
    };
    // B operand: 4 rows of one column of block (j, j) of T.
    auto b_diag = [&](int j, auto two) {
      const float* c = &Tf[(j * 16 + lg * 4) * FP + j * 16 + li];
      return make(c[0], c[FP], c[2 * FP], c[3 * FP], two);
    };
    auto b_reg = [&](const f32x4& v, auto two) { return make(v[0], v[1], v[2], v[3], two); };
    auto mul = [&](const Frag& a, const Frag& b, f32x4 acc, auto two) {
      if (decltype(two)::value) {
        acc = mfma16k16(a.lo, b.hi, acc);
        acc = mfma16k16(a.hi, b.lo, acc);
      }
      return mfma16k16(a.hi, b.hi, acc);
    };
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    auto blocks = [&](auto two) {
      // T_ij = -T_ii X, stored to LDS; returned for the next levels.
      auto finish = [&](int i, int j, const f32x4& X) {
        const f32x4 y = mul(a_op(Tf, i, i, two), b_reg(X, two), z, two);
        f32x4 t;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          t[r] = -y[r];
          Tf[(i * 16 + lg * 4 + r) * FP + j * 16 + li] = t[r];
          tmax = fmaxf(tmax, fabsf(t[r]));
        }
        return t;
      };
      const Frag t00 = b_diag(0, two), t11 = b_diag(1, two), t22 = b_diag(2, two);
      const f32x4 t10 = finish(1, 0, mul(a_op(Af, 1, 0, two), t00, z, two));
      const f32x4 t21 = finish(2, 1, mul(a_op(Af, 2, 1, two), t11, z, two));
      finish(3, 2, mul(a_op(Af, 3, 2, two), t22, z, two));
      const f32x4 t20 = finish(
          2, 0, mul(a_op(Af, 2, 1, two), b_reg(t10, two), mul(a_op(Af, 2, 0, two), t00, z, two), two));
      finish(3, 1,
             mul(a_op(Af, 3, 2, two), b_reg(t21, two), mul(a_op(Af, 3, 1, two), t11, z, two), two));
      finish(3, 0,
             mul(a_op(Af, 3, 2, two), b_reg(t20, two),
                 mul(a_op(Af, 3, 1, two), b_reg(t10, two), mul(a_op(Af, 3, 0, two), t00, z, two),
                     two),
                 two));
    };
    blocks(std::false_type{});
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off));
    if (tmax > kSplitThreshold) blocks(std::true_type{});  // wave-uniform
    if (lane == 0) Tmax = tmax;
  }
  lds_barrier();
  const bool split = Tmax > kSplitThreshold;
  if (tid == 0) ws.F[chunk] = split ? 1 : 0;
  if (split) {
    const int nslots = (w == 0 || w == 2) ? 4 : 2;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
      if (sl < nslots)
        *reinterpret_cast<u16x4*>(ws.PL + chunk * (CK * CK) + poff[sl]) = plo[sl];
  }

  // K^T of token block w into LDS (the A blocks are no longer needed); K
  // block w is in slot 0 for waves 0 and 1 and in slot 2 for waves 2 and 3.
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const u16x8 bits = frag_bits(w < 2 ? f[0][kk] : f[2][kk]);
#pragma unroll
    for (int i = 0; i < 8; ++i) XT[(kk * 32 + lg * 8 + i) * XP + w * 16 + li] = bits[i];
  }
  // bf16 Q for the chain (Qf: the fragments as held here), once per q/k head:
  // Q blocks 0 and 1 from wave 0's slots 2 and 3, Q block w from slot 3 of
  // waves 2 and 3.
  if (h % grp == 0) {
    uint16_t* dst = ws.Qb + (((int64_t)bb * Hk + kh) * NC + c) * (CK * DH);
    if (w == 0) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        *reinterpret_cast<u16x8*>(dst + ((0 * 4 + kk) * 64 + lane) * 8) = frag_bits(f[2][kk]);
        *reinterpret_cast<u16x8*>(dst + ((1 * 4 + kk) * 64 + lane) * 8) = frag_bits(f[3][kk]);
      }
    } else if (w >= 2) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        *reinterpret_cast<u16x8*>(dst + ((w * 4 + kk) * 64 + lane) * 8) = frag_bits(f[3][kk]);
    }
  }
  lds_barrier();

  // K^T to the workspace once per q/k head (the first value head of the group).
  if (h % grp == 0) {
    uint16_t* dst = ws.Kt + (((int64_t)bb * Hk + kh) * NC + c) * (DH * CK);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // 16-byte piece idx = ((cw * 2 + ci) * 2 + kk) * 64 + cl of Ktf.
      const int idx = i * PREP_THREADS + tid;
      const int cl = idx & 63, kk = (idx >> 6) & 1, ci = (idx >> 7) & 1, cw = idx >> 8;
      const int dk = 32 * cw + 16 * ci + (cl & 15), s = 32 * kk + 8 * (cl >> 4);
      *reinterpret_cast<u16x8*>(dst + idx * 8) = *reinterpret_cast<const u16x8*>(&XT[dk * XP + s]);
    }
  }

  // Rows of T scaled by a per-column factor (b gamma for W, b for Ut), as an
  // MFMA operand in two bf16 parts (hi + lo), read from LDS when needed.
  auto trow = [&](int tb, int kk, const float* colscale, bf16x8& hi, bf16x8& lo, bool two) {
    const float* row = &Tf[(tb * 16 + li) * FP + kk * 32 + lg * 8];
    const float4 r0 = *reinterpret_cast<const float4*>(row);
    const float4 r1 = *reinterpret_cast<const float4*>(row + 4);
    const float4 s0 = *reinterpret_cast<const float4*>(&colscale[kk * 32 + lg * 8]);
    const float4 s1 = *reinterpret_cast<const float4*>(&colscale[kk * 32 + lg * 8 + 4]);
    const float v[8] = {r0.x * s0.x, r0.y * s0.y, r0.z * s0.z, r0.w * s0.w,
                        r1.x * s1.x, r1.y * s1.y, r1.z * s1.z, r1.w * s1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) hi[i] = (__bf16)v[i];
    if (two) {
#pragma unroll
      for (int i = 0; i < 8; ++i) lo[i] = (__bf16)(v[i] - (float)hi[i]);
    }
  };

  // W^T tiles [dk block][t block] = K^T (T diag(b gamma))^T, stored as Wf;
  // wave w takes dk blocks 2w and 2w+1.  T is lower triangular, so t blocks 0
  // and 1 need only s < 32.  K is exact in bf16; T diag(b gamma) takes two
  // parts.
  {
    bf16x8 kt[2][2];
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        kt[d][kk] = ld_frag(&XT[((2 * w + d) * 16 + li) * XP + kk * 32 + lg * 8]);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      bf16x8 tg0, tg0l, tg1, tg1l;
      trow(tb, 0, BGs, tg0, tg0l, split);
      if (tb >= 2) trow(tb, 1, BGs, tg1, tg1l, split);
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (split) {
          acc = mfma16(kt[d][0], tg0l, acc);
          if (tb >= 2) acc = mfma16(kt[d][1], tg1l, acc);
        }
        acc = mfma16(kt[d][0], tg0, acc);
        if (tb >= 2) acc = mfma16(kt[d][1], tg1, acc);
        const int t = tb * 16 + li, dk = (2 * w + d) * 16 + lg * 4;
        st4<uint16_t>(ws.W + chunk * (CK * DH) + frag_off(t, dk, 4), acc[0], acc[1], acc[2],
                      acc[3]);
      }
    }
  }
  lds_barrier();

  // V^T of token block w into LDS.
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const u16x8 bits = frag_bits(vf[kk]);
#pragma unroll
    for (int i = 0; i < 8; ++i) XT[(kk * 32 + lg * 8 + i) * XP + w * 16 + li] = bits[i];
  }
  lds_barrier();

  // Ut tiles [t block][dv block] = (T diag(b)) V, stored as Utf; wave w takes
  // dv blocks 2w and 2w+1.
  bf16x8 vt[2][2];
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      vt[d][kk] = ld_frag(&XT[((2 * w + d) * 16 + li) * XP + kk * 32 + lg * 8]);
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    bf16x8 tb0, tb0l, tb1, tb1l;
    trow(tb, 0, Bs, tb0, tb0l, split);
    if (tb >= 2) trow(tb, 1, Bs, tb1, tb1l, split);
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const int vb = 2 * w + d;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (split) {
        acc = mfma16(tb0l, vt[d][0], acc);
        if (tb >= 2) acc = mfma16(tb1l, vt[d][1], acc);
      }
      acc = mfma16(tb0, vt[d][0], acc);
      if (tb >= 2) acc = mfma16(tb1, vt[d][1], acc);
      // Utf[sl = vb / 2][w = tb][cvb][cli + 16 lg][0..3] with dvp(cvb, cli) = the
      // column within the slice, 16 (vb % 2) + li.
      const int col = 16 * (vb & 1) + li;
      const int cvb = (col >> 2) & 1, cli = 4 * (col >> 3) + (col & 3);
      const int64_t off =
          chunk * (CK * DH) + ((vb >> 1) * 4 + tb) * 512 + cvb * 256 + (cli + 16 * lg) * 4;
      if (split) st4_split(ws.Ut + off, ws.UtL + off, acc[0], acc[1], acc[2], acc[3]);
      else st4<uint16_t>(ws.Ut + off, acc[0], acc[1], acc[2], acc[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// Phase 2: per (batch, value head, slice of NV value columns), sequential
// over chunks; eight waves in two roles.  State waves 0-3 carry the
// recurrence: wave w owns token rows [16w, 16w+16) of U and key rows
// [32w, 32w+32) of the f32 state slice H.  Output waves 4-7 produce O for
// token rows [16(w-4), 16(w-4)+16).  Every operand a wave multiplies with is
// its own (rows of W, K^T and Ut, or of Q and P, and the gate sums), so those
// go from global memory straight into registers, two chunks ahead, in MFMA
// operand order.  The bf16 copy of H and U^T are exchanged in LDS behind two
// barriers per chunk:
//   state:  U = Ut - W H -> LDS | barrier | H update -> LDS | barrier
//   output: (Q H)^T          | barrier | O = .. + P U    | barrier
constexpr int CH_THREADS = 512;

// Column u / 2 * 32 + dvp(u % 2, m) of a slice: the 32-column pieces of a
// slice each keep the dvp row order.
__device__ __forceinline__ int dvp2(int u, int m) { return 32 * (u >> 1) + dvp(u & 1, m); }

template <int NV>
struct StateRegs {
  bf16x8 w[4];        // W[16w + li][32kk + 8lg ..]
  bf16x8 kt[2][2];    // K^T[32w + 16i + li][32kk + 8lg ..]
  u16x4 ut[NV / 16];  // Ut[16w + 4lg ..][dv0 + dvp2(u, li)], hi part
  f32x4 sc;           // e^{G_last - G_t}, t = 16w + 4lg ..
  float gl;           // e^{G_last}
  int split;          // the chunk's two-part flag (read with flag_set)
};

struct OutRegs {
  bf16x8 q[4];   // Q[16w + li][32kk + 8lg ..]
  bf16x8 p[2];   // P[16w + li][32kk + 8lg ..], hi part
  float gt;      // e^{G_t}, t = 16w + li
  int split;     // the chunk's two-part flag (read with flag_set)
};

// The chunk's two-part flag, loaded with the chunk's other operands and
// read (made wave-uniform) in the chunk's own step.
__device__ __forceinline__ int chunk_flag(const WsLayout& ws, int64_t chunk) {
  return ws.F[chunk];
}
__device__ __forceinline__ bool flag_set(int raw) {
  return __builtin_amdgcn_readfirstlane(raw) != 0;
}

__device__ __forceinline__ bf16x8 gld_frag(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

template <int NV>
__device__ __forceinline__ void state_fetch(StateRegs<NV>& R, const WsLayout& ws, int bb, int bh,
                                            int kh, int c, int Hk, int NC, int sl, int w,
                                            int lane) {
  const int64_t chunk = (int64_t)bh * NC + c;
  const int64_t kchunk = ((int64_t)bb * Hk + kh) * NC + c;
  const uint16_t* wp = ws.W + chunk * (CK * DH) + (w * 4 * 64 + lane) * 8;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) R.w[kk] = gld_frag(wp + kk * 512);
  const uint16_t* kp = ws.Kt + kchunk * (DH * CK) + (w * 4 * 64 + lane) * 8;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) R.kt[i][kk] = gld_frag(kp + (i * 2 + kk) * 512);
  // Ut is stored per 32-column piece (the prep's Utf[piece][w][vb]).
#pragma unroll
  for (int u = 0; u < NV / 16; ++u) {
    const int64_t off = chunk * (CK * DH) + ((sl * (NV / 32) + (u >> 1)) * 4 + w) * 512 +
                        (u & 1) * 256 + lane * 4;
    R.ut[u] = *reinterpret_cast<const u16x4*>(ws.Ut + off);
  }
  const float* gp = ws.G + chunk * 2 * CK;
  R.sc = *reinterpret_cast<const f32x4*>(gp + CK + 16 * w + 4 * (lane >> 4));
  R.gl = gp[CK - 1];
  R.split = chunk_flag(ws, chunk);
}

// The lo part of Ut for a two-part chunk, loaded in the chunk's own step and
// used at once: a load for a later step, issued only for some chunks, would
// leave the compiler's count of loads in flight inexact for every chunk.
template <int NV>
__device__ __forceinline__ void state_fetch_lo(u16x4* utl, const WsLayout& ws, int bh, int c,
                                               int NC, int sl, int w, int lane) {
  const int64_t chunk = (int64_t)bh * NC + c;
#pragma unroll
  for (int u = 0; u < NV / 16; ++u) {
    const int64_t off = chunk * (CK * DH) + ((sl * (NV / 32) + (u >> 1)) * 4 + w) * 512 +
                        (u & 1) * 256 + lane * 4;
    utl[u] = *reinterpret_cast<const u16x4*>(ws.UtL + off);
  }
}

// Q comes from the prep's fragment-order bf16 copy: reading the input rows
// (16 rows a 64-byte piece each per load, rows a token stride apart) costs
// the chain more than the copy costs the prep.
__device__ __forceinline__ void out_fetch(OutRegs& R, const WsLayout& ws, int bb, int bh, int kh,
                                          int c, int Hk, int NC, int w, int lane) {
  const int64_t chunk = (int64_t)bh * NC + c;
  const int li = lane & 15;
  const int64_t kchunk = ((int64_t)bb * Hk + kh) * NC + c;
  const uint16_t* qp = ws.Qb + kchunk * (CK * DH) + (w * 4 * 64 + lane) * 8;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) R.q[kk] = gld_frag(qp + kk * 512);
  // P is causal: token blocks 0 and 1 use only its first 32 columns.
  const int64_t po = chunk * (CK * CK) + (w * 2 * 64 + lane) * 8;
  R.p[0] = gld_frag(ws.P + po);
  // Loaded unconditionally (waves 0 and 1 reload the first tile and ignore
  // it), so the compiler's count of loads in flight stays exact.
  R.p[1] = gld_frag(ws.P + po + (w >= 2 ? 512 : 0));
  R.gt = ws.G[chunk * 2 * CK + 16 * w + li];
  R.split = chunk_flag(ws, chunk);
}

// The lo part of P for a two-part chunk, loaded in the chunk's own step (as
// state_fetch_lo).
__device__ __forceinline__ void out_fetch_lo(bf16x8* pl, const WsLayout& ws, int bh, int c,
                                             int NC, int w, int lane) {
  const int64_t po = ((int64_t)bh * NC + c) * (CK * CK) + (w * 2 * 64 + lane) * 8;
  pl[0] = gld_frag(ws.PL + po);
  pl[1] = gld_frag(ws.PL + po + (w >= 2 ? 512 : 0));
}

// NV = 32 or 64 value columns per slice.  Each wave loads its operands
// kDepth chunks ahead (kDepth + 1 register sets in rotation): two for both
// widths, which fit in the 256 VGPRs a wave has with one workgroup per CU.
template <int NV>
constexpr int chain_depth() { return 2; }

// One row's chain (state and output waves), as the kernel below sets it up.
template <int NV, typename TO>
__device__ __forceinline__ void chain_run(const WsLayout& ws, const float* state_in,
                                          float* state_out, TO* __restrict__ o, int Hk, int Hv,
                                          int NC, float q_scale, int bb, int bh, int h, int kh,
                                          int sl, int64_t tbase, int tlen, uint16_t* Sb,
                                          uint16_t* Utl, uint16_t* UtlL, uint16_t* Usl,
                                          uint16_t* UslL) {
  constexpr int NVB = NV / 16;  // 16-column blocks per slice
  constexpr int kDepth = chain_depth<NV>();
  const int dv0 = sl * NV;
  const int ncr = (tlen + CK - 1) / CK;  // this row's chunks (NC is the workspace stride)
  // Chunk index for a fetch ahead: past the row's last chunk the loads repeat
  // it (an empty row loads chunk 0 and uses nothing).
  auto ahead = [&](int cc) { return max(0, min(cc, ncr - 1)); };
  const int tid = threadIdx.x, lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);
  const bool state_wave = tid < 256;

  if (state_wave) {
    StateRegs<NV> RA, RB, RC;
    state_fetch<NV>(RA, ws, bb, bh, kh, 0, Hk, NC, sl, w, lane);
    if (kDepth == 2) state_fetch<NV>(RB, ws, bb, bh, kh, ahead(1), Hk, NC, sl, w, lane);

    f32x4 H[2][NVB];  // H[dk = 16(2w+i) + 4lg + r][dv = dv0 + 16vb + li]
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        const int dk = (2 * w + i) * 16 + lg * 4, dv = dv0 + vb * 16 + li;
        if (state_in) {
          const float4 s4 =
              *reinterpret_cast<const float4*>(state_in + ((int64_t)bh * DH + dv) * DH + dk);
          H[i][vb] = f32x4{s4.x, s4.y, s4.z, s4.w};
        } else {
          H[i][vb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        st4<uint16_t>(&Sb[(vb * 16 + li) * RP + dk], H[i][vb][0], H[i][vb][1], H[i][vb][2],
                      H[i][vb][3]);
      }
    }
    lds_barrier();

    // Chunk c + 2 is loaded at step c; past the last chunk the loads repeat it
    // (unconditional loads keep the compiler's count of loads in flight exact).
    auto step = [&](const StateRegs<NV>& R, StateRegs<NV>& next, int c) {
      // Scheduling fence: no work of one chunk step moves into another.
      __builtin_amdgcn_sched_barrier(0);
      const int cn = ahead(c + kDepth);
      state_fetch<NV>(next, ws, bb, bh, kh, cn, Hk, NC, sl, w, lane);
      // (1) U = Ut - W H against the bf16 state copy, dv rows in dvp order.
      f32x4 accU[NVB];
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) accU[vb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb)
          accU[vb] = mfma16(R.w[kk], ld_frag(&Sb[dvp2(vb, li) * RP + kk * 32 + lg * 8]), accU[vb]);
      // (2) U^T to LDS, plain and scaled by e^{G_last - G_s}.  A two-part
      // chunk also adds Ut's lo part (loaded here, in its own step) and
      // writes the lo parts of both copies.
      const float sc[4] = {R.sc[0], R.sc[1], R.sc[2], R.sc[3]};
      float u[NVB][4];
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
        for (int r = 0; r < 4; ++r) u[vb][r] = bf2f(R.ut[vb][r]) - accU[vb][r];
      const bool two = flag_set(R.split);
      if (two) {
        u16x4 utl[NVB];
        state_fetch_lo<NV>(utl, ws, bh, c, NC, sl, w, lane);
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) {
          const int off = dvp2(vb, li) * XP + w * 16 + lg * 4;
#pragma unroll
          for (int r = 0; r < 4; ++r) u[vb][r] += bf2f(utl[vb][r]);
          st4_split(&Utl[off], &UtlL[off], u[vb][0], u[vb][1], u[vb][2], u[vb][3]);
          st4_split(&Usl[off], &UslL[off], u[vb][0] * sc[0], u[vb][1] * sc[1], u[vb][2] * sc[2],
                    u[vb][3] * sc[3]);
        }
      } else {
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) {
          const int off = dvp2(vb, li) * XP + w * 16 + lg * 4;
          st4<uint16_t>(&Utl[off], u[vb][0], u[vb][1], u[vb][2], u[vb][3]);
          st4<uint16_t>(&Usl[off], u[vb][0] * sc[0], u[vb][1] * sc[1], u[vb][2] * sc[2],
                        u[vb][3] * sc[3]);
        }
      }
      lds_barrier();
      // (3) H <- gamma_last H + K^T diag(e^{G_last - G_s}) U (for a two-part
      // chunk also + K^T of U's lo part), then its bf16 copy for the next
      // chunk (every wave finished reading the old copy before the barrier
      // above).
      const float gl = R.gl;
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        const bf16x8 u0 = ld_frag(&Usl[(vb * 16 + li) * XP + lg * 8]);
        const bf16x8 u1 = ld_frag(&Usl[(vb * 16 + li) * XP + 32 + lg * 8]);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          f32x4 hcur = H[i][vb];
#pragma unroll
          for (int r = 0; r < 4; ++r) hcur[r] *= gl;
          hcur = mfma16(R.kt[i][0], u0, hcur);
          hcur = mfma16(R.kt[i][1], u1, hcur);
          H[i][vb] = hcur;
        }
      }
      if (two) {
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) {
          const bf16x8 u0l = ld_frag(&UslL[(vb * 16 + li) * XP + lg * 8]);
          const bf16x8 u1l = ld_frag(&UslL[(vb * 16 + li) * XP + 32 + lg * 8]);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            H[i][vb] = mfma16(R.kt[i][0], u0l, H[i][vb]);
            H[i][vb] = mfma16(R.kt[i][1], u1l, H[i][vb]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb)
          st4<uint16_t>(&Sb[(vb * 16 + li) * RP + (2 * w + i) * 16 + lg * 4], H[i][vb][0],
                        H[i][vb][1], H[i][vb][2], H[i][vb][3]);
      lds_barrier();
    };
    int c = 0;
    if constexpr (kDepth == 2) {
      for (; c + 3 <= ncr; c += 3) {
        step(RA, RC, c);
        step(RB, RA, c + 1);
        step(RC, RB, c + 2);
      }
      if (c < ncr) step(RA, RC, c);
      if (c + 1 < ncr) step(RB, RA, c + 1);
    } else {
      for (; c + 2 <= ncr; c += 2) {
        step(RA, RB, c);
        step(RB, RA, c + 1);
      }
      if (c < ncr) step(RA, RB, c);
    }

    if (state_out) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) {
          const int dk = (2 * w + i) * 16 + lg * 4, dv = dv0 + vb * 16 + li;
          *reinterpret_cast<float4*>(state_out + ((int64_t)bh * DH + dv) * DH + dk) =
              make_float4(H[i][vb][0], H[i][vb][1], H[i][vb][2], H[i][vb][3]);
        }
      }
    }
  } else {
    const int tr = w * 16 + li;
    OutRegs RA, RB, RC;
    out_fetch(RA, ws, bb, bh, kh, 0, Hk, NC, w, lane);
    if (kDepth == 2) out_fetch(RB, ws, bb, bh, kh, ahead(1), Hk, NC, w, lane);
    lds_barrier();
    // `full` (std::true_type) marks a chunk of CK tokens, whose store needs no
    // row check.
    auto step = [&](const OutRegs& R, OutRegs& next, int c, auto full) {
      __builtin_amdgcn_sched_barrier(0);
      // (Q H)^T against the same state copy as this chunk's U.
      f32x4 accQ[NVB];
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) accQ[vb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb)
          accQ[vb] = mfma16(ld_frag(&Sb[dvp2(vb, li) * RP + kk * 32 + lg * 8]), R.q[kk], accQ[vb]);
      // The loads of chunk c + 2 go out after (Q H)^T: issued at the start of
      // the step they queue behind the state waves' loads, and (Q H)^T gates
      // the first barrier.
      __builtin_amdgcn_sched_barrier(0);
      const int cn = ahead(c + kDepth);
      out_fetch(next, ws, bb, bh, kh, cn, Hk, NC, w, lane);
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      // O^T = q_scale gamma_t (Q H)^T + U^T P^T; P is causal, so token blocks
      // 0 and 1 need only s < 32.  Lane (li, lg) ends with dv 8lg..8lg+7 of
      // token 16w + li (dvp order), one 8-wide store.  A two-part chunk adds
      // the lo-part products (loaded here, in its own step): (Uh + Ul)(Ph + Pl)
      // without Ul Pl.
      const float gq = q_scale * R.gt;
      f32x4 acc[NVB];
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        const int ro = dvp2(vb, li) * XP + lg * 8;
        acc[vb] = mfma16(ld_frag(&Utl[ro]), R.p[0], f32x4{0.f, 0.f, 0.f, 0.f});
        if (w >= 2) acc[vb] = mfma16(ld_frag(&Utl[ro + 32]), R.p[1], acc[vb]);
      }
      if (flag_set(R.split)) {
        bf16x8 pl[2];
        out_fetch_lo(pl, ws, bh, c, NC, w, lane);
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) {
          const int ro = dvp2(vb, li) * XP + lg * 8;
          acc[vb] = mfma16(ld_frag(&UtlL[ro]), R.p[0], acc[vb]);
          acc[vb] = mfma16(ld_frag(&Utl[ro]), pl[0], acc[vb]);
          if (w >= 2) {
            acc[vb] = mfma16(ld_frag(&UtlL[ro + 32]), R.p[1], acc[vb]);
            acc[vb] = mfma16(ld_frag(&Utl[ro + 32]), pl[1], acc[vb]);
          }
        }
      }
      float ov[4 * NVB];
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
        for (int r = 0; r < 4; ++r) ov[4 * vb + r] = fmaf(gq, accQ[vb][r], acc[vb][r]);
      const int t0 = c * CK;
      if (decltype(full)::value || tr < min(CK, tlen - t0)) {
#pragma unroll
        for (int j = 0; j < NV / 32; ++j)
          store8(o + ((tbase + t0 + tr) * Hv + h) * DH + dv0 + 32 * j + 8 * lg, ov + 8 * j);
      }
      lds_barrier();
    };
    int c = 0;
    const int nfull = tlen / CK;
    if constexpr (kDepth == 2) {
      for (; c + 3 <= nfull; c += 3) {
        step(RA, RC, c, std::true_type{});
        step(RB, RA, c + 1, std::true_type{});
        step(RC, RB, c + 2, std::true_type{});
      }
      if (c < ncr) step(RA, RC, c, std::false_type{});
      if (c + 1 < ncr) step(RB, RA, c + 1, std::false_type{});
      if (c + 2 < ncr) step(RC, RB, c + 2, std::false_type{});
    } else {
      for (; c + 2 <= nfull; c += 2) {
        step(RA, RB, c, std::true_type{});
        step(RB, RA, c + 1, std::true_type{});
      }
      if (c < ncr) step(RA, RB, c, std::false_type{});
      if (c + 1 < ncr) step(RB, RA, c + 1, std::false_type{});
    }
  }
}

template <int NV, typename TO>
__global__ __launch_bounds__(CH_THREADS, 2) void chunk_chain_kernel(
    WsLayout ws, const float* state_in,
    float* state_out, TO* __restrict__ o, int B, int T, const int32_t* __restrict__ cu,
    int total, int Hk, int Hv, int NC, float q_scale) {
  constexpr int NSL = DH / NV;  // slices per head
  static_assert(NV == 32 || NV == 64, "slices are one or two 32-column pieces");
  // U^T goes through LDS as bf16, for two-part chunks with a second bf16
  // part (lo): the state update and the output sum U over a chunk's tokens,
  // sums that cancel when keys are nearly parallel.
  __shared__ __attribute__((aligned(16))) uint16_t Sb[NV * RP];    // S slice [dv][dk], bf16
  __shared__ __attribute__((aligned(16))) uint16_t Utl[NV * XP];   // U^T [dv][s], hi
  __shared__ __attribute__((aligned(16))) uint16_t UtlL[NV * XP];  // U^T [dv][s], lo
  __shared__ __attribute__((aligned(16))) uint16_t Usl[NV * XP];   // U^T e^{G_last - G_s}, hi
  __shared__ __attribute__((aligned(16))) uint16_t UslL[NV * XP];  // U^T e^{G_last - G_s}, lo

  // The NSL slices of a head, and the heads of a q/k group, run on one XCD
  // and share its L2 for W, P, K^T, G and Q; groups are dealt round-robin
  // over the XCDs (rows of a ragged batch spread evenly).
  const int id = blockIdx.x;
  int hs, sl;
  if (((B * Hk) & 7) == 0) {
    const int u = xcd_head(id, B * Hk, Hv / Hk, NSL);
    hs = u / NSL;
    sl = u % NSL;
  } else {
    hs = (id >> 3) / NSL * 8 + (id & 7);
    sl = (id >> 3) % NSL;
  }
  if (hs >= B * Hv) return;
  const int bh = hs, bb = bh / Hv, h = bh % Hv, kh = h / (Hv / Hk);
  int64_t tbase;
  int tlen;
  row_span(cu, total, bb, T, tbase, tlen);
  chain_run<NV, TO>(ws, state_in, state_out, o, Hk, Hv, NC, q_scale, bb, bh, h, kh, sl, tbase,
                    tlen, Sb, Utl, UtlL, Usl, UslL);
}

namespace {

template <typename TI, typename TV, typename TG>
void launch_prep(const void* q, int64_t q_ts, const void* k, int64_t k_ts, const void* v,
                 int64_t v_ts, const void* a, const void* b, const float* A_log,
                 const float* dt_bias, const WsLayout& ws, int B, int T, const int32_t* cu,
                 int total, int Hk, int Hv, int NC, float q_scale, hipStream_t stream) {
  hipLaunchKernelGGL((chunk_prep_kernel<TI, TV, TG>), dim3((unsigned)((int64_t)B * Hv * NC)),
                     dim3(PREP_THREADS),
                     0, stream, (const TI*)q, q_ts, (const TI*)k, k_ts, (const TV*)v, v_ts,
                     (const TG*)a, (const TG*)b, A_log, dt_bias, ws, T, cu, total, Hk, Hv, NC,
                     q_scale);
}

template <typename TI, typename TV>
void launch_prep_g(int gate_dt, const void* q, int64_t q_ts, const void* k, int64_t k_ts,
                   const void* v, int64_t v_ts, const void* a, const void* b, const float* A_log,
                   const float* dt_bias, const WsLayout& ws, int B, int T, const int32_t* cu,
                   int total, int Hk, int Hv, int NC, float q_scale, hipStream_t stream) {
  if (gate_dt == 1)
    launch_prep<TI, TV, uint16_t>(q, q_ts, k, k_ts, v, v_ts, a, b, A_log, dt_bias, ws, B, T, cu,
                                  total, Hk, Hv, NC, q_scale, stream);
  else
    launch_prep<TI, TV, float>(q, q_ts, k, k_ts, v, v_ts, a, b, A_log, dt_bias, ws, B, T, cu,
                               total, Hk, Hv, NC, q_scale, stream);
}

// Up to this many 32-column (head, slice) units, one per CU (256 CUs), the
// chain runs 32-column slices; beyond it 64-column slices, still one
// workgroup per CU.  At B = 2 (384 narrow units) the wide form takes the
// chain from 183 to 134 us: a wide workgroup's step costs about as much as
// two narrow ones (the head's W, K^T, Q and P are pulled once for twice the
// columns), and 192 wide units run in one round on the 256 CUs where 384
// narrow ones need two.
constexpr int kChainNarrow = 256;

template <typename TO>
void launch_chain(const WsLayout& ws, const float* state_in, float* state_out,
                  void* o, int B, int T, const int32_t* cu, int total, int Hk, int Hv, int NC,
                  float q_scale, hipStream_t stream) {
  const int64_t units = ((int64_t)B * Hv + 7) / 8 * 8 * (DH / 32);  // whole XCD rounds of heads
  const int64_t per_xcd = units / 8;
  if (units <= kChainNarrow)
    hipLaunchKernelGGL((chunk_chain_kernel<32, TO>), dim3((unsigned)(per_xcd * 8)),
                       dim3(CH_THREADS), 0, stream, ws, state_in, state_out, (TO*)o, B, T, cu,
                       total, Hk, Hv, NC, q_scale);
  else
    hipLaunchKernelGGL((chunk_chain_kernel<64, TO>), dim3((unsigned)(per_xcd * 8 / 2)),
                       dim3(CH_THREADS), 0, stream, ws, state_in, state_out, (TO*)o, B, T, cu,
                       total, Hk, Hv, NC, q_scale);
}

}  // namespace

hipError_t launch_prefill_chunked(const void* q, int64_t q_ts, const void* k, int64_t k_ts,
                                  const void* v, int64_t v_ts, int qk_dt, int v_dt, const void* a,
                                  const void* b, int gate_dt, const float* A_log,
                                  const float* dt_bias, const float* state_in, float* state_out,
                                  void* o, int o_dt, int B, int T, const int32_t* cu, int total,
                                  int Hk, int Hv, float q_scale, void* workspace,
                                  hipStream_t stream) {
  const int NC = (T + CK - 1) / CK;
  const WsLayout ws = ws_layout(workspace, B, T, Hk, Hv);
  if (qk_dt == 1 && v_dt == 1)
    launch_prep_g<uint16_t, uint16_t>(gate_dt, q, q_ts, k, k_ts, v, v_ts, a, b, A_log, dt_bias,
                                      ws, B, T, cu, total, Hk, Hv, NC, q_scale, stream);
  else if (qk_dt == 0 && v_dt == 1)
    launch_prep_g<float, uint16_t>(gate_dt, q, q_ts, k, k_ts, v, v_ts, a, b, A_log, dt_bias, ws,
                                   B, T, cu, total, Hk, Hv, NC, q_scale, stream);
  else
    return hipErrorInvalidValue;  // other combinations are not instantiated
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (o_dt == 1)
    launch_chain<uint16_t>(ws, state_in, state_out, o, B, T, cu, total, Hk, Hv, NC, q_scale,
                           stream);
  else
    launch_chain<float>(ws, state_in, state_out, o, B, T, cu, total, Hk, Hv, NC, q_scale, stream);
  return hipGetLastError();
}

}  // namespace gdn
