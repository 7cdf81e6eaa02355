// chunk_bwd.hip -- reverse mode of the chunked gated delta rule: gradients of
// q, k, v, the gate (g or its logit), beta and h0 for an upstream gradient of
// o and of the final state, over 16-token tiles in fp32 arithmetic.
//
// The pages ("Deep Dive: The Next Generation of Ultra-Long Context Sparse MoE
// LLMs", sec. 3.2; "Core Technologies Behind Ultra-Long-Context Sparse MoE
// Large Models", sec. 2.1 and 2.3) describe the tiled forward pass and frame
// the bounded decay around BF16 training; they print no backward pass.  The
// one here is the adjoint of the tiled forward form, derived by hand.  Inside
// a tile that starts from state H (d_k x d_v), with G the in-tile running sum
// of g, gamma = exp(G), E[t][i] = exp(G_t - G_i) (i <= t), ec_i = exp(G_C - G_i):
//   A = strict-lower(beta_t E KK^T),  T = (I + A)^-1,  P = lower(E Q K^T)
//   Y = diag(beta) (V - diag(gamma) K H),  U = T Y
//   O = diag(gamma) Q H + P U,  H' = gamma_C H + (diag(ec) K)^T U
// and, for upstream dO and dH' (the gradient of the tile's end state):
//   dU = diag(ec) K dH' + P^T dO,  dY = T^T dU,  dV = diag(beta) dY
//   dH = gamma_C dH' + Q^T diag(gamma) dO - K^T diag(beta gamma) dY
//   dQ = diag(gamma) dO H^T + (dP o E) K,          dP = lower(dO U^T)
//   dK = -diag(beta gamma) dY H^T + diag(ec) U dH'^T + (dP o E)^T Q + M K + M^T K
//        with dA = -strict-lower(dY U^T) and M = dA o beta_t E
//   dbeta_t = dY_t . (V_t - gamma_t (K H)_t) + sum_i dA[t][i] E[t][i] KK[t][i]
//   dG (per in-tile running sum) collects the gamma, E, ec and gamma_C terms,
//   and dg is its reverse running sum within the tile.
// A tail tile is padded with q = k = v = do = 0, g = 0, beta = 0: each padded
// token is an identity step and its gradients are dropped.
//
// Four kernels:
//   bwd_prep_kernel     per tile: G, beta, T, P and E*KK^T into a record;
//   bwd_hstates_mfma_kernel  per (sequence, head, 16 columns of d_v), serial
//                       over tiles on the fp32 MFMA: the state at every tile
//                       start;
//   bwd_dh_mfma_kernel  same split, serial backwards: dH' at every tile end,
//                       and dh0;
//   bwd_grad_kernel     per tile, all of d_v (one 16-column slice per wave at a
//                       time): dq, dk, dv, dbeta, dg.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "la_bwd.h"
#include "la_device.h"
#include "la_launch.h"

namespace la {
namespace {

// ----------------------- states at every tile start, on the matrix cores
// One workgroup per sequence, head and 16 columns of d_v, serial over tiles,
// the products on the fp32 MFMA: wave 0 ("chain") keeps the fp32 state slice H (d_k x 16) in
// registers, in accumulator order (lane (n, grp) register i of tile t holds
// H[16t + 4grp + i][n]); per tile it stores H, then
//   R = K H,  Y = diag(beta) (V - diag(gamma) R),  U = T Y,
//   H' = gamma_C H + K^T diag(ec) U.
// Waves 1..NP ("loaders") stage tiles in LDS -- K as A fragments and as K^T
// fragments, T, the slice of V, gamma, ec, beta, gamma_C -- double-buffered by
// epochs of NP tiles, their global loads issued two epochs ahead.
template <int DK>
struct HsRec {
  static constexpr int NS = DK / 32, NT = DK / 16;
  static constexpr int KF = 0;                     // K: NS x 64 lanes x 8 f32
  static constexpr int KT = KF + NS * 64 * 8 * 4;  // K^T: NT x 64 x 4
  static constexpr int TI = KT + NT * 64 * 4 * 4;  // T: 16 x 16 row-major
  static constexpr int VF = TI + 256 * 4;          // V slice: 64 x 4
  static constexpr int GM = VF + 64 * 4 * 4;       // gamma[16]
  static constexpr int EC = GM + 64;               // ec[16]
  static constexpr int BT = EC + 64;               // beta[16]
  static constexpr int GC = BT + 64;               // gamma_C (x4)
  static constexpr int BYTES = GC + 16;
  static_assert(BYTES % 16 == 0, "alignment");
};

// A 32-deep fragment's 8 elements as fp32 (lo = j 0..3, hi = j 4..7).
__device__ inline Elt<float>::F32 frag_f32(const Elt<float>::F32& x) { return x; }
__device__ inline Elt<float>::F32 frag_f32(const Elt<__bf16>::F32& x) {
  Elt<float>::F32 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r.lo[j] = (float)x.v[j];
    r.hi[j] = (float)x.v[4 + j];
  }
  return r;
}

template <typename E, int DK>
struct HsRaw {
  typename Elt<E>::F32 kf[DK / 32];
  f32x4 ti;
  E vv[4];
  float g, bt, gC;
};

template <typename E, int DK, int NP>
__global__ __launch_bounds__(64 * (NP + 1)) void bwd_hstates_mfma_kernel(BwdArgs a) {
  using R = HsRec<DK>;
  using X = Elt<float>;
  using F16 = X::F16;
  using F32 = X::F32;
  constexpr int NS = R::NS, NT = R::NT;
  __shared__ __attribute__((aligned(16))) char smem[2 * NP * R::BYTES];
  const int NV = a.Dv / 16;
  const int sl = (int)(blockIdx.x % NV);
  const int64_t bh = blockIdx.x / NV;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int v0 = 16 * sl;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, grp = lane >> 4;
  const BSeq sq = bwd_seq(a, b, h);
  const int NC = sq.NC;
  const int NE = (NC + NP - 1) / NP;
  auto rec_of = [&](int c) -> char* { return smem + (((c / NP) & 1) * NP + c % NP) * R::BYTES; };

  if (wave == 0) {
    f32x4 Hacc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Hacc[t][i] = a.h0 ? a.h0[(bh * DK + 16 * t + 4 * grp + i) * a.Dv + v0 + n] : 0.f;
    }
    __syncthreads();  // epoch 0 staged
    for (int ep = 0; ep < NE; ++ep) {
      for (int j = 0; j < NP; ++j) {
        const int c = ep * NP + j;
        if (c >= NC) break;
        const char* rec = rec_of(c);
        // the state at the tile start, in fragment order (see BRec)
        f32x4* hsp = reinterpret_cast<f32x4*>(a.hs + (sq.rbase + c) * (int64_t)DK * a.Dv +
                                              (int64_t)(v0 / 16) * DK * 16);
#pragma unroll
        for (int t = 0; t < NT; ++t) hsp[t * 64 + lane] = Hacc[t];
        f32x4 Rk = zero4();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const F32 kf = reinterpret_cast<const F32*>(rec + R::KF)[s * 64 + lane];
          Rk = X::mma32(kf, X::from_acc2(Hacc[2 * s], Hacc[2 * s + 1]), Rk);
        }
        const f32x4 vf = reinterpret_cast<const f32x4*>(rec + R::VF)[lane];
        const f32x4 gm = reinterpret_cast<const f32x4*>(rec + R::GM)[grp];
        const f32x4 ec = reinterpret_cast<const f32x4*>(rec + R::EC)[grp];
        const f32x4 bt = reinterpret_cast<const f32x4*>(rec + R::BT)[grp];
        const float gC = *reinterpret_cast<const float*>(rec + R::GC);
        f32x4 Y;
#pragma unroll
        for (int i = 0; i < 4; ++i) Y[i] = bt[i] * (vf[i] - gm[i] * Rk[i]);
        const F16 ti = *reinterpret_cast<const F16*>(rec + R::TI + (n * 16 + 4 * grp) * 4);
        const f32x4 U = X::mma16(ti, X::from_acc(Y), zero4());
        f32x4 Up;
#pragma unroll
        for (int i = 0; i < 4; ++i) Up[i] = ec[i] * U[i];
        const F16 ub = X::from_acc(Up);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const F16 kt = reinterpret_cast<const F16*>(rec + R::KT)[t * 64 + lane];
          Hacc[t] = Hacc[t] * gC;
          Hacc[t] = X::mma16(kt, ub, Hacc[t]);
        }
      }
      __syncthreads();  // this epoch consumed, the next one staged
    }
    return;
  }

  // ---------------------------------------------------------------- loaders
  const int p = wave - 1;
  const E* kp = static_cast<const E*>(a.k);
  const E* vp = static_cast<const E*>(a.v);
  auto rowk = [&](int t) -> int64_t { return (sq.tok0 + t) * a.H + h; };
  auto load = [&](HsRaw<E, DK>& r, int c) {
    if (NC == 0) return;          // an empty sequence loads nothing
    c = min(c, NC - 1);
    const int t = min(c * kT + n, sq.T - 1);
    const int64_t base = rowk(t) * DK;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c0 = 32 * s + 4 * grp, c1 = c0 + 16;
      if constexpr (sizeof(E) == 2) {
        const bf16x4 k0 = *reinterpret_cast<const bf16x4*>(kp + base + c0);
        const bf16x4 k1 = *reinterpret_cast<const bf16x4*>(kp + base + c1);
        r.kf[s].v = bf16x8{k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
      } else {
        r.kf[s].lo = *reinterpret_cast<const f32x4*>(kp + base + c0);
        r.kf[s].hi = *reinterpret_cast<const f32x4*>(kp + base + c1);
      }
    }
    const float* rec = a.rec + (sq.rbase + c) * BRec::FLOATS;
    r.ti = reinterpret_cast<const f32x4*>(rec + BRec::TINV)[lane];
    r.g = rec[BRec::G + n];
    r.bt = rec[BRec::BETA + n];
    r.gC = rec[BRec::G + kT - 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) r.vv[i] = vp[rowk(min(c * kT + 4 * grp + i, sq.T - 1)) * a.Dv + v0 + n];
  };
  auto store = [&](const HsRaw<E, DK>& r, int c) {
    if (c >= NC) return;
    char* rec = rec_of(c);
    const bool ok = c * kT + n < sq.T;        // token row n of this tile exists
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      F32 k32 = frag_f32(r.kf[s]);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        k32.lo[jj] = ok ? k32.lo[jj] : 0.f;
        k32.hi[jj] = ok ? k32.hi[jj] : 0.f;
      }
      reinterpret_cast<F32*>(rec + R::KF)[s * 64 + lane] = k32;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int ch = 32 * s + (jj < 4 ? 4 * grp + jj : 16 + 4 * grp + jj - 4);
        const float kv = jj < 4 ? k32.lo[jj] : k32.hi[jj - 4];
        // K^T in the chain's A-fragment order: tile ch / 16, lane (ch % 16, n / 4), register n % 4
        reinterpret_cast<float*>(rec + R::KT)[((ch >> 4) * 64 + (n >> 2) * 16 + (ch & 15)) * 4 +
                                              (n & 3)] = kv;
      }
    }
    reinterpret_cast<f32x4*>(rec + R::TI)[lane] = r.ti;
    f32x4 vf;
#pragma unroll
    for (int i = 0; i < 4; ++i) vf[i] = (c * kT + 4 * grp + i < sq.T) ? Elt<E>::to_f(r.vv[i]) : 0.f;
    reinterpret_cast<f32x4*>(rec + R::VF)[lane] = vf;
    if (grp == 0) {
      reinterpret_cast<float*>(rec + R::GM)[n] = __expf(r.g);
      reinterpret_cast<float*>(rec + R::EC)[n] = __expf(r.gC - r.g);
      reinterpret_cast<float*>(rec + R::BT)[n] = r.bt;
      if (n == 0) *reinterpret_cast<float*>(rec + R::GC) = __expf(r.gC);
    }
  };
  HsRaw<E, DK> ra, rb;
  load(ra, p);
  store(ra, p);                 // epoch 0
  load(ra, NP + p);             // epoch 1, staged during epoch 0
  __syncthreads();
  for (int ep = 0; ep < NE; ep += 2) {
    load(rb, (ep + 2) * NP + p);
    store(ra, (ep + 1) * NP + p);
    __syncthreads();
    if (ep + 1 < NE) {
      load(ra, (ep + 3) * NP + p);
      store(rb, (ep + 2) * NP + p);
      __syncthreads();
    }
  }
}

// --------------- gradients of every tile's end state, on the matrix cores
// One workgroup per sequence, head and 16 columns of d_v, tiles from last to
// first, the products on the fp32 MFMA: wave 0 keeps D = dL/dH' of the current tile (d_k x 16) in
// registers in accumulator order; per tile it stores D, then
//   dU = diag(ec) K D + P^T dO,  dY = T^T dU,
//   D' = gamma_C D + Q^T diag(gamma) dO - K^T diag(beta gamma) dY,
// and after the first tile writes dh0.  SPW chain waves per workgroup (one
// per 16-column slice) share what the loader waves stage: K (A fragments and
// K^T fragments), Q^T fragments, P^T, T^T, the slice of dO and the per-token
// factors, double-buffered by epochs in processing order (m = 0 is the last
// tile).
template <int DK, int SPW>
struct HdRec {
  static constexpr int NS = DK / 32, NT = DK / 16;
  static constexpr int KF = 0;                     // K: NS x 64 lanes x 8 f32
  static constexpr int KT = KF + NS * 64 * 8 * 4;  // K^T: NT x 64 x 4
  static constexpr int QT = KT + NT * 64 * 4 * 4;  // Q^T: NT x 64 x 4
  static constexpr int PT = QT + NT * 64 * 4 * 4;  // P^T: 16 x 16 row-major
  static constexpr int TT = PT + 256 * 4;          // T^T: 16 x 16 row-major
  static constexpr int DO = TT + 256 * 4;          // dO slices: SPW x 64 x 4
  static constexpr int GM = DO + SPW * 64 * 4 * 4; // gamma[16]
  static constexpr int EC = GM + 64;               // ec[16]
  static constexpr int BT = EC + 64;               // beta[16]
  static constexpr int GC = BT + 64;               // gamma_C (x4)
  static constexpr int BYTES = GC + 16;
  static_assert(BYTES % 16 == 0, "alignment");
};

template <typename E, int DK, int SPW>
struct HdRaw {
  typename Elt<E>::F32 kf[DK / 32];
  typename Elt<E>::F32 qf[DK / 32];
  f32x4 pm, tm;
  E dd[SPW][4];
  float g, bt, gC;
};

template <typename E, int DK, int NP, int SPW>
__global__ __launch_bounds__(64 * (NP + SPW)) void bwd_dh_mfma_kernel(BwdArgs a) {
  using R = HdRec<DK, SPW>;
  using X = Elt<float>;
  using F16 = X::F16;
  using F32 = X::F32;
  constexpr int NS = R::NS, NT = R::NT;
  __shared__ __attribute__((aligned(16))) char smem[2 * NP * R::BYTES];
  // SPW column slices of 16 per workgroup, one chain wave each
  const int NW = a.Dv / (16 * SPW);
  const int sl = (int)(blockIdx.x % NW);
  const int64_t bh = blockIdx.x / NW;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, grp = lane >> 4;
  const BSeq sq = bwd_seq(a, b, h);
  const int NC = sq.NC;
  const int NE = (NC + NP - 1) / NP;
  // records by processing index m (tile NC - 1 - m)
  auto rec_of = [&](int m) -> char* { return smem + (((m / NP) & 1) * NP + m % NP) * R::BYTES; };

  if (wave < SPW) {
    const int v0 = 16 * (SPW * sl + wave);
    f32x4 D[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        D[t][i] = a.dhT ? a.dhT[(bh * DK + 16 * t + 4 * grp + i) * a.Dv + v0 + n] : 0.f;
    }
    __syncthreads();  // epoch 0 staged
    for (int ep = 0; ep < NE; ++ep) {
      for (int j = 0; j < NP; ++j) {
        const int m = ep * NP + j;
        if (m >= NC) break;
        const int c = NC - 1 - m;
        const char* rec = rec_of(m);
        f32x4* dsp = reinterpret_cast<f32x4*>(a.dhs + (sq.rbase + c) * (int64_t)DK * a.Dv +
                                              (int64_t)(v0 / 16) * DK * 16);
#pragma unroll
        for (int t = 0; t < NT; ++t) dsp[t * 64 + lane] = D[t];
        f32x4 KD = zero4();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const F32 kf = reinterpret_cast<const F32*>(rec + R::KF)[s * 64 + lane];
          KD = X::mma32(kf, X::from_acc2(D[2 * s], D[2 * s + 1]), KD);
        }
        const f32x4 dO = reinterpret_cast<const f32x4*>(rec + R::DO)[wave * 64 + lane];
        const f32x4 gm = reinterpret_cast<const f32x4*>(rec + R::GM)[grp];
        const f32x4 ec = reinterpret_cast<const f32x4*>(rec + R::EC)[grp];
        const f32x4 bt = reinterpret_cast<const f32x4*>(rec + R::BT)[grp];
        const float gC = *reinterpret_cast<const float*>(rec + R::GC);
        f32x4 eKD;
#pragma unroll
        for (int i = 0; i < 4; ++i) eKD[i] = ec[i] * KD[i];
        const F16 pt = *reinterpret_cast<const F16*>(rec + R::PT + (n * 16 + 4 * grp) * 4);
        const F16 tt = *reinterpret_cast<const F16*>(rec + R::TT + (n * 16 + 4 * grp) * 4);
        const f32x4 dU = X::mma16(pt, X::from_acc(dO), eKD);
        const f32x4 dY = X::mma16(tt, X::from_acc(dU), zero4());
        f32x4 nZ, Og;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          nZ[i] = -(bt[i] * gm[i] * dY[i]);
          Og[i] = gm[i] * dO[i];
        }
        const F16 zb = X::from_acc(nZ), ob = X::from_acc(Og);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const F16 qt = reinterpret_cast<const F16*>(rec + R::QT)[t * 64 + lane];
          const F16 kt = reinterpret_cast<const F16*>(rec + R::KT)[t * 64 + lane];
          D[t] = D[t] * gC;
          D[t] = X::mma16(qt, ob, D[t]);
          D[t] = X::mma16(kt, zb, D[t]);
        }
      }
      __syncthreads();  // this epoch consumed, the next one staged
    }
    if (a.dh0) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a.dh0[(bh * DK + 16 * t + 4 * grp + i) * a.Dv + v0 + n] = D[t][i];
      }
    }
    return;
  }

  // ---------------------------------------------------------------- loaders
  const int p = wave - SPW;
  const E* kp = static_cast<const E*>(a.k);
  const E* qp = static_cast<const E*>(a.q);
  const E* dp = static_cast<const E*>(a.dout);
  const int v0 = 16 * SPW * sl;
  auto rowk = [&](int t) -> int64_t { return (sq.tok0 + t) * a.H + h; };
  auto load = [&](HdRaw<E, DK, SPW>& r, int m) {
    if (NC == 0) return;          // an empty sequence loads nothing
    const int c = NC - 1 - min(m, NC - 1);
    const int t = min(c * kT + n, sq.T - 1);
    const int64_t base = rowk(t) * DK;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c0 = 32 * s + 4 * grp, c1 = c0 + 16;
      if constexpr (sizeof(E) == 2) {
        const bf16x4 k0 = *reinterpret_cast<const bf16x4*>(kp + base + c0);
        const bf16x4 k1 = *reinterpret_cast<const bf16x4*>(kp + base + c1);
        const bf16x4 q0 = *reinterpret_cast<const bf16x4*>(qp + base + c0);
        const bf16x4 q1 = *reinterpret_cast<const bf16x4*>(qp + base + c1);
        r.kf[s].v = bf16x8{k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
        r.qf[s].v = bf16x8{q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
      } else {
        r.kf[s].lo = *reinterpret_cast<const f32x4*>(kp + base + c0);
        r.kf[s].hi = *reinterpret_cast<const f32x4*>(kp + base + c1);
        r.qf[s].lo = *reinterpret_cast<const f32x4*>(qp + base + c0);
        r.qf[s].hi = *reinterpret_cast<const f32x4*>(qp + base + c1);
      }
    }
    const float* rec = a.rec + (sq.rbase + c) * BRec::FLOATS;
    r.pm = reinterpret_cast<const f32x4*>(rec + BRec::P)[lane];
    r.tm = reinterpret_cast<const f32x4*>(rec + BRec::TINV)[lane];
    r.g = rec[BRec::G + n];
    r.bt = rec[BRec::BETA + n];
    r.gC = rec[BRec::G + kT - 1];
#pragma unroll
    for (int w = 0; w < SPW; ++w) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        r.dd[w][i] = dp[rowk(min(c * kT + 4 * grp + i, sq.T - 1)) * a.Dv + v0 + 16 * w + n];
    }
  };
  auto store = [&](const HdRaw<E, DK, SPW>& r, int m) {
    if (m >= NC) return;
    const int c = NC - 1 - m;
    char* rec = rec_of(m);
    const bool ok = c * kT + n < sq.T;        // token row n of this tile exists
    float* kt = reinterpret_cast<float*>(rec + R::KT);
    float* qt = reinterpret_cast<float*>(rec + R::QT);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      F32 k32 = frag_f32(r.kf[s]), q32 = frag_f32(r.qf[s]);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        k32.lo[jj] = ok ? k32.lo[jj] : 0.f;
        k32.hi[jj] = ok ? k32.hi[jj] : 0.f;
        q32.lo[jj] = ok ? q32.lo[jj] : 0.f;
        q32.hi[jj] = ok ? q32.hi[jj] : 0.f;
      }
      reinterpret_cast<F32*>(rec + R::KF)[s * 64 + lane] = k32;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int ch = 32 * s + (jj < 4 ? 4 * grp + jj : 16 + 4 * grp + jj - 4);
        // transposed A fragments: tile ch / 16, lane (ch % 16, n / 4), register n % 4
        const int at = ((ch >> 4) * 64 + (n >> 2) * 16 + (ch & 15)) * 4 + (n & 3);
        kt[at] = jj < 4 ? k32.lo[jj] : k32.hi[jj - 4];
        qt[at] = jj < 4 ? q32.lo[jj] : q32.hi[jj - 4];
      }
    }
    // P and T arrive row-major (lane l holds row l / 4, columns 4 (l % 4) ..);
    // store them transposed
    float* pt = reinterpret_cast<float*>(rec + R::PT);
    float* tt = reinterpret_cast<float*>(rec + R::TT);
    const int row = lane >> 2, col = 4 * (lane & 3);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pt[(col + i) * 16 + row] = r.pm[i];
      tt[(col + i) * 16 + row] = r.tm[i];
    }
#pragma unroll
    for (int w = 0; w < SPW; ++w) {
      f32x4 dd;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dd[i] = (c * kT + 4 * grp + i < sq.T) ? Elt<E>::to_f(r.dd[w][i]) : 0.f;
      reinterpret_cast<f32x4*>(rec + R::DO)[w * 64 + lane] = dd;
    }
    if (grp == 0) {
      reinterpret_cast<float*>(rec + R::GM)[n] = __expf(r.g);
      reinterpret_cast<float*>(rec + R::EC)[n] = __expf(r.gC - r.g);
      reinterpret_cast<float*>(rec + R::BT)[n] = r.bt;
      if (n == 0) *reinterpret_cast<float*>(rec + R::GC) = __expf(r.gC);
    }
  };
  HdRaw<E, DK, SPW> ra, rb;
  load(ra, p);
  store(ra, p);                 // epoch 0
  load(ra, NP + p);             // epoch 1, staged during epoch 0
  __syncthreads();
  for (int ep = 0; ep < NE; ep += 2) {
    load(rb, (ep + 2) * NP + p);
    store(ra, (ep + 1) * NP + p);
    __syncthreads();
    if (ep + 1 < NE) {
      load(ra, (ep + 3) * NP + p);
      store(rb, (ep + 2) * NP + p);
      __syncthreads();
    }
  }
}

// --------------------------------------------------- per-tile gradients
__device__ inline float sum16(float x) {
  x += __shfl_xor(x, 1, 16);
  x += __shfl_xor(x, 2, 16);
  x += __shfl_xor(x, 4, 16);
  x += __shfl_xor(x, 8, 16);
  return x;
}

// Column slices need no workgroup barriers: wave w takes the 16-column slices
// w, w + 4, ... of d_v end to end.  Per slice, straight from the
// fragment-order states in registers:
//   K H, Q H, K dH' (fp32 MFMA over d_k),  Y, U = T Y, dU = diag(ec) K dH' +
//   P^T dO, dY = T^T dU (MFMA), dv, and the wave's partial sums of dP = dO U^T,
//   dA = -dY U^T, dq += diag(gamma) dO H^T, dk += -diag(beta gamma) dY H^T +
//   diag(ec) U dH'^T and of the per-token row terms.
// The contractions over the slice's columns need row fragments of dO, dY, U
// and of each 16-row block of H and dH': 16 x 16 transposes through a
// wave-private LDS tile.  One cross-wave reduction per tile, then the in-tile
// terms and the gate / beta gradients.  Two workgroups share a compute unit
// (registers and LDS are sized for that): one's loads and barriers overlap the
// other's matrix products.
template <typename E, int DK>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_grad_kernel(BwdArgs a) {
  constexpr int KP = DK + 4;
  constexpr int NT = DK / 16;          // 16-row blocks of d_k
  constexpr int RT = DK / 64;          // of them, owned by each wave at the end
  constexpr int TP = 20;               // transposition tile pitch (floats)
  using X = Elt<float>;
  using F16 = X::F16;
  __shared__ __attribute__((aligned(16))) float sK[kT][KP];
  __shared__ __attribute__((aligned(16))) float sQ[kT][KP];
  __shared__ float sTi[kT][kT + 1], sP[kT][kT + 1];
  __shared__ float sG[kT], sB[kT], sGam[kT], sEc[kT];
  // per-wave transposition tiles (four per wave) during the slices; the
  // cross-wave reduction of the dq / dk partials afterwards
  constexpr int TR_BYTES = 4 * 4 * kT * TP * 4, RED_BYTES = 4 * NT * 64 * 16;
  __shared__ __attribute__((aligned(16))) char sU8[TR_BYTES > RED_BYTES ? TR_BYTES : RED_BYTES];
  __shared__ __attribute__((aligned(16))) f32x4 sRedS[4][2][64];   // dP, dA partials
  __shared__ float sRow[4][3][kT];                                    // row sums B, G, W
  __shared__ float sPE[kT][kT + 1], sM[kT][kT + 1], sPP[kT][kT + 1], sAA[kT][kT + 1];
  __shared__ float sRowB[kT], sRowG[kT], sRowW[kT], sRowAK[kT];
  __shared__ float sHdH[4];
  const int tid = threadIdx.x;
  const int64_t tile = blockIdx.x;
  int b, h, c;
  if (!bwd_tile(a, tile, b, h, c)) return;   // an unused slot: the whole block
  const BSeq sq = bwd_seq(a, b, h);
  const int t = tid >> 4, j = tid & 15;        // (token, column) / (token, token) view
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, n = tid & 15, grp = (tid >> 4) & 3;
  const float* rec = a.rec + tile * BRec::FLOATS;
  const E* vp = static_cast<const E*>(a.v);
  const E* dop = static_cast<const E*>(a.dout);
  const float* Hb = a.hs + tile * (int64_t)DK * a.Dv;
  const float* Db = a.dhs + tile * (int64_t)DK * a.Dv;
  const int NV = a.Dv / 16;
  // the slice in hand: H and dH' fragments (accumulator order), v and dO of
  // tokens 4 grp + i, column 16 jb + n; the first is requested before the
  // tile is staged.
  f32x4 Hf[NT], Df[NT], vv, dd;
  auto fetch_hd = [&](int jb, int r) {
    Hf[r] = reinterpret_cast<const f32x4*>(Hb + (int64_t)jb * DK * 16)[r * 64 + lane];
    Df[r] = reinterpret_cast<const f32x4*>(Db + (int64_t)jb * DK * 16)[r * 64 + lane];
  };
  auto fetch_vd = [&](int jb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tk = c * kT + 4 * grp + i;
      const int64_t ro = ((sq.tok0 + tk) * a.H + h) * a.Dv + 16 * jb + n;
      vv[i] = tk < sq.T ? ld1(vp + ro) : 0.f;
      dd[i] = tk < sq.T ? ld1(dop + ro) : 0.f;
    }
  };
  if (w < NV) {
#pragma unroll
    for (int r = 0; r < NT; ++r) fetch_hd(w, r);
    fetch_vd(w);
  }
  load_tile<E, DK, KP>(sK, static_cast<const E*>(a.k), sq, c, h, a);
  load_tile<E, DK, KP>(sQ, static_cast<const E*>(a.q), sq, c, h, a);
  sTi[t][j] = rec[BRec::TINV + tid];
  sP[t][j] = rec[BRec::P + tid];
  const float ekk = rec[BRec::EKK + tid];
  float gamC;
  load_scalars(rec, sG, sB, sGam, sEc, gamC);
  __syncthreads();

  const int tkn = c * kT + n;                          // token of row fragments
  const int64_t ron = (sq.tok0 + tkn) * a.H + h;
  float (*tr)[TP] = reinterpret_cast<float (*)[TP]>(sU8 + w * 4 * kT * TP * 4);
  // X in accumulator order -> row fragment (lane (n, grp) register jj =
  // X[n][4 grp + jj]) through 16 x 16 tiles, up to four per LDS round trip
  auto transpose = [&](float (*tl)[TP], const f32x4& x) -> f32x4 {
#pragma unroll
    for (int i = 0; i < 4; ++i) tl[4 * grp + i][n] = x[i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const f32x4 r = *reinterpret_cast<const f32x4*>(&tl[n][4 * grp]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return r;
  };
  auto transpose_n = [&](auto& x, auto& y) {
    constexpr int M = sizeof(x) / sizeof(x[0]);
    static_assert(M <= 4, "four tiles per wave");
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) tr[m * kT + 4 * grp + i][n] = x[m][i];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int m = 0; m < M; ++m) y[m] = *reinterpret_cast<const f32x4*>(&tr[m * kT + n][4 * grp]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  f32x4 dQp[NT], dKp[NT];
#pragma unroll
  for (int r = 0; r < NT; ++r) dQp[r] = dKp[r] = zero4();
  f32x4 pB = zero4(), pG = zero4(), pW = zero4(), dPp = zero4(), dAp = zero4();
  float hdh = 0.f;
  for (int jb = w; jb < NV; jb += 4) {
    if (jb != w) {
#pragma unroll
      for (int r = 0; r < NT; ++r) fetch_hd(jb, r);
      fetch_vd(jb);
    }
    f32x4 KH = zero4(), QH = zero4(), KdH = zero4();
#pragma unroll
    for (int r = 0; r < NT; ++r) {
      const F16 kf{*reinterpret_cast<const f32x4*>(&sK[n][16 * r + 4 * grp])};
      const F16 qf{*reinterpret_cast<const f32x4*>(&sQ[n][16 * r + 4 * grp])};
      KH = X::mma16(kf, F16{Hf[r]}, KH);
      QH = X::mma16(qf, F16{Hf[r]}, QH);
      KdH = X::mma16(kf, F16{Df[r]}, KdH);
#pragma unroll
      for (int i = 0; i < 4; ++i) hdh += Hf[r][i] * Df[r][i];
    }
    // this lane's tokens in accumulator order (4 grp + i) and in row order (n),
    // and T, P^T, T^T as A fragments, re-read from LDS per slice (registers
    // are what limits the waves per SIMD here)
    f32x4 gm4, bt4, ec4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gm4[i] = sGam[4 * grp + i];
      bt4[i] = sB[4 * grp + i];
      ec4[i] = sEc[4 * grp + i];
    }
    const float gmn = sGam[n], btn = sB[n], ecn = sEc[n];
    F16 Tf, PTf, TTf;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      Tf.v[jj] = sTi[n][4 * grp + jj];
      PTf.v[jj] = sP[4 * grp + jj][n];
      TTf.v[jj] = sTi[4 * grp + jj][n];
    }
    f32x4 vres, Y, eKD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      vres[i] = vv[i] - gm4[i] * KH[i];
      Y[i] = bt4[i] * vres[i];
      eKD[i] = ec4[i] * KdH[i];
    }
    const f32x4 U = X::mma16(Tf, F16{Y}, zero4());
    const f32x4 dU = X::mma16(PTf, F16{dd}, eKD);
    const f32x4 dY = X::mma16(TTf, F16{dU}, zero4());
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pB[i] += dY[i] * vres[i];
      pG[i] += gm4[i] * QH[i] * dd[i] - bt4[i] * gm4[i] * dY[i] * KH[i];
      pW[i] += eKD[i] * U[i];
    }
    f32x4 acc3[3] = {U, dd, dY}, row3[3];
    transpose_n(acc3, row3);
    const f32x4 Ur = row3[0], DOr = row3[1], DYr = row3[2];
    // dv = diag(beta) dY, a row fragment: token n, columns 16 jb + 4 grp + 0..3
    if (tkn < sq.T)
      *reinterpret_cast<f32x4*>(a.dv + ron * a.Dv + 16 * jb + 4 * grp) = btn * DYr;
    dPp = X::mma16(F16{DOr}, F16{Ur}, dPp);
    dAp = X::mma16(F16{DYr}, F16{Ur}, dAp);
    f32x4 aO, aY, aU;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      aO[jj] = gmn * DOr[jj];
      aY[jj] = -btn * gmn * DYr[jj];
      aU[jj] = ecn * Ur[jj];
    }
#pragma unroll
    for (int r = 0; r < NT; r += 2) {
      f32x4 acc4[4] = {Hf[r], Df[r], Hf[r + 1], Df[r + 1]}, row4[4];
      transpose_n(acc4, row4);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        dQp[r + e] = X::mma16(F16{aO}, F16{row4[2 * e]}, dQp[r + e]);
        dKp[r + e] = X::mma16(F16{aY}, F16{row4[2 * e]}, dKp[r + e]);
        dKp[r + e] = X::mma16(F16{aU}, F16{row4[2 * e + 1]}, dKp[r + e]);
      }
    }
  }

  // ---- cross-wave reduction
  // row sums over the 16 columns of a lane row, then over the waves
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      pB[i] += __shfl_xor(pB[i], m, 16);
      pG[i] += __shfl_xor(pG[i], m, 16);
      pW[i] += __shfl_xor(pW[i], m, 16);
    }
  }
  for (int m = 1; m < 64; m <<= 1) hdh += __shfl_xor(hdh, m, 64);
  __syncthreads();                       // every wave is done with its tiles
  f32x4* red = reinterpret_cast<f32x4*>(sU8);
#pragma unroll
  for (int r = 0; r < NT; ++r) red[(w * NT + r) * 64 + lane] = dQp[r];
  sRedS[w][0][lane] = dPp;
  sRedS[w][1][lane] = dAp;
  if (n == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sRow[w][0][4 * grp + i] = pB[i];
      sRow[w][1][4 * grp + i] = pG[i];
      sRow[w][2][4 * grp + i] = pW[i];
    }
  }
  if (lane == 0) sHdH[w] = hdh;
  __syncthreads();
  f32x4 dQa[RT], dKa[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    dQa[r] = zero4();
    for (int v = 0; v < 4; ++v) dQa[r] += red[(v * NT + RT * w + r) * 64 + lane];
  }
  // dP, dA at (token t, token i = j): accumulator lane 16 (t / 4) + j, register t % 4
  float dPacc = 0.f, dAacc = 0.f;
  for (int v = 0; v < 4; ++v) {
    dPacc += sRedS[v][0][16 * (t >> 2) + j][t & 3];
    dAacc -= sRedS[v][1][16 * (t >> 2) + j][t & 3];
  }
  __syncthreads();                       // the dq partials are read
#pragma unroll
  for (int r = 0; r < NT; ++r) red[(w * NT + r) * 64 + lane] = dKp[r];
  {
    const int i = j;
    const float e = i <= t ? __expf(sG[t] - sG[i]) : 0.f;
    const float dP = i <= t ? dPacc : 0.f;
    const float dA = i < t ? dAacc : 0.f;
    sPE[t][i] = dP * e;
    sM[t][i] = dA * sB[t] * e;
    sPP[t][i] = dP * sP[t][i];
    sAA[t][i] = dA * sB[t] * ekk;
    const float rak = sum16(dA * ekk);
    if (j == 0) {
      sRowB[t] = sRow[0][0][t] + sRow[1][0][t] + sRow[2][0][t] + sRow[3][0][t];
      sRowG[t] = sRow[0][1][t] + sRow[1][1][t] + sRow[2][1][t] + sRow[3][1][t];
      sRowW[t] = sRow[0][2][t] + sRow[1][2][t] + sRow[2][2][t] + sRow[3][2][t];
      sRowAK[t] = rak;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    dKa[r] = zero4();
    for (int v = 0; v < 4; ++v) dKa[r] += red[(v * NT + RT * w + r) * 64 + lane];
  }
  // in-tile terms: dQ += (dP o E) K, dK += (dP o E)^T Q + (M + M^T) K
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int i = 4 * kk + grp;
    const float aPE = sPE[n][i], aPEt = sPE[i][n], aMM = sM[n][i] + sM[i][n];
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int col = 16 * (RT * w + r) + n;
      const float bK = sK[i][col], bQ = sQ[i][col];
      dQa[r] = __builtin_amdgcn_mfma_f32_16x16x4f32(aPE, bK, dQa[r], 0, 0, 0);
      dKa[r] = __builtin_amdgcn_mfma_f32_16x16x4f32(aPEt, bQ, dKa[r], 0, 0, 0);
      dKa[r] = __builtin_amdgcn_mfma_f32_16x16x4f32(aMM, bK, dKa[r], 0, 0, 0);
    }
  }
  // dq, dk rows as 16-byte pieces: transposed through a tile in this wave's
  // share of sRedS, whose dP / dA partials were read before the last barrier
  {
    float (*tq)[TP] = reinterpret_cast<float (*)[TP]>(&sRedS[w][0][0]);
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const f32x4 q4 = transpose(tq, dQa[r]);
      const f32x4 k4 = transpose(tq, dKa[r]);
      if (tkn < sq.T) {
        *reinterpret_cast<f32x4*>(a.dq + ron * DK + 16 * (RT * w + r) + 4 * grp) = q4;
        *reinterpret_cast<f32x4*>(a.dk + ron * DK + 16 * (RT * w + r) + 4 * grp) = k4;
      }
    }
  }
  {
    // dg_u = sum_{t >= u} dG_t, with dG_t the gradient of the in-tile running
    // sum G_t.  The E-terms of P and A enter dG_t with + for the row and - for
    // the column, so their sum over t >= u keeps exactly the entries with row
    // >= u and column < u; the ec-terms keep the tokens before u; gamma_C
    // enters every u.  Summed in this form nothing large cancels.  Lane (u, i)
    // takes W_i (i < u) or G_i (i >= u) and column i of PP + AA over the rows
    // t >= u when i < u; a 16-lane sum then gives dg_u - gamma_C <H, dH'>.
    const int u = tid >> 4, i = tid & 15;
    float x = i < u ? sRowW[i] : sRowG[i];
#pragma unroll
    for (int t2 = 0; t2 < kT; ++t2) {
      const float y = sPP[t2][i] + sAA[t2][i];
      x += (t2 >= u && i < u) ? y : 0.f;
    }
    x = sum16(x);
    const int tk = c * kT + u;
    if (i == 0 && tk < sq.T) {
      const float dg = gamC * (sHdH[0] + sHdH[1] + sHdH[2] + sHdH[3]) + x;
      const int64_t idx = (sq.tok0 + tk) * a.H + h;
      float out = dg;
      if (a.gate_logit) {
        const float s = sigmoid_f(a.gate[idx]);
        out = -a.G * s * (1.f - s) * dg;
      }
      a.dgate[idx] = out;
      a.dbeta[idx] = sRowB[u] + sRowAK[u];
    }
  }
}

template <typename E, int DK>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
  // batched: every tile of every sequence; packed: every slot (unused ones
  // return at once)
  const int64_t tiles = a.cu ? (int64_t)a.H * a.nslot : (int64_t)a.B * a.H * a.NT;
  const int64_t slices = (int64_t)a.B * a.H * (a.Dv / 16);
  hipLaunchKernelGGL((bwd_prep_kernel<E, DK>), dim3((unsigned)tiles), dim3(kBwdThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_hstates_mfma_kernel<E, DK, 2>), dim3((unsigned)slices), dim3(64 * 3), 0,
                     st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // two column slices per workgroup when the slice count is even: the staged
  // tile then serves two chain waves, and half as many workgroups (at one per
  // compute unit, for the LDS they take) fit in one round
  if ((a.Dv / 16) % 2 == 0)
    hipLaunchKernelGGL((bwd_dh_mfma_kernel<E, DK, 2, 2>), dim3((unsigned)(slices / 2)),
                       dim3(64 * 4), 0, st, a);
  else
    hipLaunchKernelGGL((bwd_dh_mfma_kernel<E, DK, 2, 1>), dim3((unsigned)slices), dim3(64 * 3), 0,
                       st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_grad_kernel<E, DK>), dim3((unsigned)tiles), dim3(kBwdThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

long long chunk_bwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int fp32) {
  if (chunk_bwd_bf16_path(Dk, Dv, fp32)) return chunk_bwd_bf16_workspace_bytes(B, T, H, Dk, Dv);
  const long long nt = (T + kT - 1) / kT;
  const long long tiles = (long long)B * H * nt;
  return tiles * (BRec::FLOATS * 4LL + 2LL * Dk * Dv * 4LL);
}

hipError_t launch_chunk_bwd(const void* q, const void* k, const void* v, const void* dout,
                            const float* gate, int gate_logit, float G, const float* beta,
                            const float* h0, const float* dhT, float* dq, float* dk, float* dv,
                            float* dgate, float* dbeta, float* dh0, int B, int T, int H, int Dk,
                            int Dv, int fp32, void* ws, hipStream_t st) {
  return launch_chunk_bwd_varlen(q, k, v, dout, gate, gate_logit, G, beta, h0, dhT, dq, dk, dv,
                                 dgate, dbeta, dh0, nullptr, B, T, H, Dk, Dv, fp32, ws, st);
}

long long chunk_bwd_varlen_workspace_bytes(int T, int nseq, int H, int Dk, int Dv, int fp32) {
  if (chunk_bwd_bf16_path(Dk, Dv, fp32))
    return chunk_bwd_bf16_varlen_workspace_bytes(T, nseq, H, Dk, Dv);
  const long long tiles = (long long)H * (T / kT + nseq + 1);
  return tiles * (BRec::FLOATS * 4LL + 2LL * Dk * Dv * 4LL);
}

hipError_t launch_chunk_bwd_varlen(const void* q, const void* k, const void* v, const void* dout,
                                   const float* gate, int gate_logit, float G, const float* beta,
                                   const float* h0, const float* dhT, float* dq, float* dk,
                                   float* dv, float* dgate, float* dbeta, float* dh0,
                                   const int* cu, int B, int T, int H, int Dk, int Dv, int fp32,
                                   void* ws, hipStream_t st) {
  if (chunk_bwd_bf16_path(Dk, Dv, fp32))
    return launch_chunk_bwd_bf16(q, k, v, dout, gate, gate_logit, G, beta, h0, dhT, dq, dk, dv,
                                 dgate, dbeta, dh0, cu, B, T, H, Dk, Dv, ws, st);
  const int NT = (T + kT - 1) / kT;
  const int nslot = cu ? T / kT + B + 1 : 0;
  const int64_t tiles = cu ? (int64_t)H * nslot : (int64_t)B * H * NT;
  char* w = static_cast<char*>(ws);
  BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.dout = dout;
  a.gate = gate; a.beta = beta; a.h0 = h0; a.dhT = dhT;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dgate = dgate; a.dbeta = dbeta; a.dh0 = dh0;
  a.rec = reinterpret_cast<float*>(w);
  a.hs = reinterpret_cast<float*>(w + tiles * BRec::FLOATS * 4);
  a.dhs = a.hs + tiles * (int64_t)Dk * Dv;
  a.gate_logit = gate_logit; a.G = G;
  a.B = B; a.T = T; a.H = H; a.Dv = Dv; a.NT = NT;
  a.cu = cu; a.nslot = nslot;
  if (fp32) return Dk == 128 ? launch_bwd_t<float, 128>(a, st) : launch_bwd_t<float, 64>(a, st);
  return Dk == 128 ? launch_bwd_t<__bf16, 128>(a, st) : launch_bwd_t<__bf16, 64>(a, st);
}

}  // namespace la
