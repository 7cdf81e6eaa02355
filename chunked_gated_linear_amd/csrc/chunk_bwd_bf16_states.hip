// chunk_bwd_bf16_states.hip -- the two serial chains of the bf16 reverse pass
// (see chunk_bwd_bf16.hip for the algebra and the checkpoint layout): the
// forward chain keeps the state H at every kHS-th tile start and the gradient
// chain the state gradient D at every group end, both as packed bf16 hi / lo
// words; one launch runs both kinds of block.  Compiled on its own (with
// LLVM's default machine scheduler) so that its files' scheduler choices stay
// apart.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "la_bwd.h"
#include "la_bwd_bf16.h"
#include "la_device.h"

namespace la {
namespace {

// ------------------------------------ states at every kHS-th tile
// Record of one staged tile (bytes).
template <int DK, int SPW>
struct H2Rec {
  static constexpr int KR = 0;                       // K rows
  static constexpr int TF = Rows<DK>::BYTES;         // [T hi | T lo] A fragments
  static constexpr int VF = TF + 1024;               // V rows of the slices (Slab)
  static constexpr int GM = VF + Slab<SPW>::BYTES;   // gamma[16]
  static constexpr int EC = GM + 64;                 // ec[16]
  static constexpr int BT = EC + 64;                 // beta[16]
  static constexpr int GC = BT + 64;                 // gamma_C
  static constexpr int BYTES = GC + 16;
  static_assert(BYTES % 16 == 0, "alignment");
};

template <int DK, int SPW>
struct H2Raw {
  uint4 kr[DK / 32];     // K row pieces: lane (n, grp), piece x = columns 32 x + 8 grp .. + 7 of row n
  f32x4 ti;
  uint4 vr[Slab<SPW>::NPC];
  float g, bt, gC;
};


template <int DK, int NP, int SPW>
__device__ inline void hstates_body(const BwdArgs& a, int64_t blk, char* smem) {
  using R = H2Rec<DK, SPW>;
  using RW = Rows<DK>;
  constexpr int NS = DK / 32, NT = DK / 16;
  const int NW = a.Dv / (16 * SPW);
  const int sl = (int)(blk % NW);
  const int64_t bh = blk / NW;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, grp = lane >> 4;
  const BSeq sq = bwd_seq(a, b, h);
  const int NC = sq.NC;
  const int NE = (NC + NP - 1) / NP;
  auto rec_of = [&](int c) -> char* { return smem + (((c / NP) & 1) * NP + c % NP) * R::BYTES; };

  if (wave < SPW) {
    const int v0 = 16 * (SPW * sl + wave);
    f32x4 Hacc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Hacc[t][i] = a.h0 ? a.h0[(bh * DK + 16 * t + 4 * grp + i) * a.Dv + v0 + n] : 0.f;
    }
    bf16x8 Hh[NS], Hl[NS];
    split_state<NS>(Hacc, Hh, Hl);
    unsigned* const hw =
        a.hw + grp_base(a, b, h) * kHPG * DK * a.Dv + (int64_t)(v0 / 16) * DK * 16;
    __syncthreads();  // epoch 0 staged
    for (int ep = 0; ep < NE; ++ep) {
      for (int j = 0; j < NP; ++j) {
        const int c = ep * NP + j;
        if (c >= NC) break;
        const char* rec = rec_of(c);
        if (c % kHS == 0) {
          uint4* dst = reinterpret_cast<uint4*>(hw + (int64_t)(c / kHS) * DK * a.Dv);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const bf16x8 hh = Hh[t >> 1], hl = Hl[t >> 1];
            dst[t * 64 + lane] = (t & 1) ? pack_words(second4(hh), second4(hl))
                                         : pack_words(first4(hh), first4(hl));
          }
        }
        // R = K H
        f32x4 Rk = zero4();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const bf16x8 ka = RW::afrag(rec + R::KR, s, n, grp);
          Rk = mma32b(ka, Hl[s], Rk);
          Rk = mma32b(ka, Hh[s], Rk);
        }
        const f32x4 vf = to_f4(Slab<SPW>::get(rec + R::VF, wave, n, grp));
        const f32x4 gm = *reinterpret_cast<const f32x4*>(rec + R::GM + 16 * grp);
        const f32x4 ec = *reinterpret_cast<const f32x4*>(rec + R::EC + 16 * grp);
        const f32x4 bt = *reinterpret_cast<const f32x4*>(rec + R::BT + 16 * grp);
        const float gC = *reinterpret_cast<const float*>(rec + R::GC);
        const bf16x8 tf = *reinterpret_cast<const bf16x8*>(rec + R::TF + 16 * lane);
        f32x4 Y;
#pragma unroll
        for (int i = 0; i < 4; ++i) Y[i] = bt[i] * (vf[i] - gm[i] * Rk[i]);
        const Sp4 sy = split4(Y);
        f32x4 U = mma32b(tf, cat8(sy.h, sy.h), zero4());
        U = mma32b_lo(tf, sy.l, U);
        f32x4 Up;
#pragma unroll
        for (int i = 0; i < 4; ++i) Up[i] = ec[i] * U[i];
        const Sp4 su = split4(Up);
        const bf16x8 ub = cat8(su.h, su.l);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const bf16x4 kt = RW::tfrag(rec + R::KR, t, n, grp);
          Hacc[t] = Hacc[t] * gC;
          Hacc[t] = mma32b(cat8(kt, kt), ub, Hacc[t]);
        }
        split_state<NS>(Hacc, Hh, Hl);
      }
      __syncthreads();  // this epoch consumed, the next one staged
    }
    if (a.hTo) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a.hTo[(bh * DK + 16 * t + 4 * grp + i) * a.Dv + v0 + n] = Hacc[t][i];
      }
    }
    return;
  }

  // ---------------------------------------------------------------- loaders
  // 2 NP loader waves: wave p stages tile p % NP of every epoch of parity
  // p / NP, loading it two epochs ahead
  const int p = (wave - SPW) % NP, q = (wave - SPW) / NP;
  const __bf16* kp = static_cast<const __bf16*>(a.k);
  const __bf16* vp = static_cast<const __bf16*>(a.v);
  const int v0 = 16 * SPW * sl;
  // Loads past the sequence end read its last token and are zeroed when
  // staged: no loaded value is touched before then, so that staging one
  // epoch does not wait for the next epoch's loads (vector loads complete in
  // order).  Addresses are a uniform base per tile (token 16 c, head h) plus
  // a 32-bit lane offset; K row pieces as lane (n, grp), piece x: columns
  // 32 x + 8 grp .. + 7 of row n.
  const int tsk = a.H * DK, tsv = a.H * a.Dv;     // token strides, elements
  auto load = [&](H2Raw<DK, SPW>& r, int c) {
    if (NC == 0) return;          // an empty sequence loads nothing
    c = min(c, NC - 1);
    const __bf16* k0 = kp + ((sq.tok0 + 16 * c) * a.H + h) * DK;
    const int koff = min(n, sq.T - 1 - 16 * c) * tsk + 8 * grp;
#pragma unroll
    for (int x = 0; x < DK / 32; ++x) r.kr[x] = *reinterpret_cast<const uint4*>(k0 + koff + 32 * x);
    const float* rec = a.rec + (sq.rbase + c) * BRec::FLOATS;
    r.ti = reinterpret_cast<const f32x4*>(rec + BRec::TINV)[lane];
    r.g = rec[BRec::G + n];
    r.bt = rec[BRec::BETA + n];
    r.gC = rec[BRec::G + kT - 1];
    Slab<SPW>::load(r.vr, vp + ((sq.tok0 + 16 * c) * a.H + h) * a.Dv + v0, tsv, sq.T - 1 - 16 * c, lane);
  };
  // CHK: the tile reaches past the sequence end, and loads there are zeroed
  auto stage = [&](const H2Raw<DK, SPW>& r, int c, auto chk) {
    constexpr bool CHK = decltype(chk)::value;
    char* rec = rec_of(c);
    const bool rok = !CHK || 16 * c + n < sq.T;
#pragma unroll
    for (int x = 0; x < DK / 32; ++x)
      *reinterpret_cast<uint4*>(rec + R::KR + n * RW::PITCH + 16 * (4 * x + grp)) = zero_if(rok, r.kr[x]);
    // T arrives row-major: lane l holds T[l / 4][4 (l % 4) + e]
#pragma unroll
    for (int e = 0; e < 4; ++e) put_op(rec + R::TF, lane >> 2, 4 * (lane & 3) + e, r.ti[e], false);
    Slab<SPW>::template stage<CHK>(rec + R::VF, r.vr, sq.T - 16 * c, lane);
    if (grp == 0) {
      reinterpret_cast<float*>(rec + R::GM)[n] = __expf(r.g);
      reinterpret_cast<float*>(rec + R::EC)[n] = __expf(r.gC - r.g);
      reinterpret_cast<float*>(rec + R::BT)[n] = r.bt;
      if (n == 0) *reinterpret_cast<float*>(rec + R::GC) = __expf(r.gC);
    }
  };
  auto store = [&](const H2Raw<DK, SPW>& r, int c) {
    if (c >= NC) return;
    if (16 * c + 16 <= sq.T) stage(r, c, std::false_type{});
    else stage(r, c, std::true_type{});
  };
  H2Raw<DK, SPW> r;
  load(r, q * NP + p);
  if (q == 0) {
    store(r, p);                // epoch 0
    load(r, 2 * NP + p);
  }
  __syncthreads();
  for (int ep = 0; ep < NE; ++ep) {
    // the chain runs epoch ep; epoch ep + 1 is staged by the loaders of its parity
    if (((ep + 1) & 1) == q) {
      store(r, (ep + 1) * NP + p);
      load(r, (ep + 3) * NP + p);
    }
    __syncthreads();
  }
}

// ------------------------------------ state gradients at every group end
// The gradient chain steps over pairs of tiles (c, c - 1), c odd, from the
// last tile down.  With D the gradient at the end of tile c,
//   D_mid   = gC_c D + Q_c^T diag(gamma_c) dO_c - K_c^T diag(beta_c gamma_c) dY_c,
//   K_{c-1} D_mid = gC_c K_{c-1} D + M1 dO_c + M2 dY_c,
//     M1 = K_{c-1} Q_c^T diag(gamma_c),  M2 = -K_{c-1} K_c^T diag(beta_c gamma_c),
//   D_start = gC_{c-1} D_mid + Q_{c-1}^T diag(gamma_{c-1}) dO_{c-1}
//             - K_{c-1}^T diag(beta_{c-1} gamma_{c-1}) dY_{c-1},
// so that the products with the state (K_c D, K_{c-1} D) and its split happen
// once per pair; the 16 x 16 operators M1 and M2 depend on the inputs only
// (each chain wave forms them from the staged rows, on the matrix cores,
// beside its K D products).  An odd tile count puts an empty tile NC in front
// (no rows, unit decay: the identity step).
template <int DK, int SPW>
struct D2Rec {
  static constexpr int KR = 0;                       // K rows
  static constexpr int QR = Rows<DK>::BYTES;         // Q rows
  static constexpr int PT = 2 * Rows<DK>::BYTES;     // [P^T hi | P^T lo] A fragments
  static constexpr int TT = PT + 1024;               // [T^T hi | T^T lo]
  static constexpr int DO = TT + 1024;               // dO rows of the slices (Slab)
  static constexpr int GM = DO + Slab<SPW>::BYTES;   // gamma[16]
  static constexpr int EC = GM + 64;                 // ec[16]
  static constexpr int BT = EC + 64;                 // beta[16]
  static constexpr int GC = BT + 64;                 // gamma_C
  static constexpr int BYTES = GC + 16;
  static_assert(BYTES % 16 == 0, "alignment");
};

// Row pieces of a tile as the loaders hold them: lane (n, grp), piece x, has
// columns 32 x + 8 grp .. + 7 of row n.
template <int DK, int SPW>
struct D2Raw {
  uint4 kr[DK / 32], qr[DK / 32];
  f32x4 pm, tm;
  uint4 dr[Slab<SPW>::NPC];
  float g, bt, gC;
};


template <int DK, int NP, int SPW>
__device__ inline void dh_body(const BwdArgs& a, int64_t blk, char* smem) {
  static_assert(NP % 2 == 0, "the gradient chain stages whole pairs of tiles");
  using R = D2Rec<DK, SPW>;
  using RW = Rows<DK>;
  constexpr int NS = DK / 32, NT = DK / 16;
  const int NW = a.Dv / (16 * SPW);
  const int sl = (int)(blk % NW);
  const int64_t bh = blk / NW;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  // roles rotated against the forward-state blocks (chain waves last), so that
  // the chain waves of the two kinds of block sharing a compute unit tend to
  // sit on different SIMDs
  const int wave = (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) + SPW) % (2 * NP + SPW);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, grp = lane >> 4;
  const BSeq sq = bwd_seq(a, b, h);
  const int NC = sq.NC;
  const int NCe = NC + (NC & 1);              // with the empty front tile when NC is odd
  const int NE = (NCe + NP - 1) / NP;
  // records by processing index m (tile NCe - 1 - m)
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
    bf16x8 Dh[NS], Dl[NS];
    split_state<NS>(D, Dh, Dl);
    unsigned* const dw = a.dw + grp_base(a, b, h) * DK * a.Dv + (int64_t)(v0 / 16) * DK * 16;
    __syncthreads();  // epoch 0 staged
    for (int ep = 0; ep < NE; ++ep) {
      for (int j = 0; j < NP; j += 2) {
        const int m = ep * NP + j;
        if (m >= NCe) break;
        const int c = NCe - 1 - m;          // the pair's later tile; c - 1 the earlier
        const char* ra = rec_of(m);
        const char* rb = rec_of(m + 1);
        // every group end is the end of some pair's later tile
        if (c % kGS == kGS - 1 || c >= NC - 1) {
          uint4* dst = reinterpret_cast<uint4*>(dw + (int64_t)(min(c, NC - 1) / kGS) * DK * a.Dv);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const bf16x8 dh = Dh[t >> 1], dl = Dl[t >> 1];
            dst[t * 64 + lane] = (t & 1) ? pack_words(second4(dh), second4(dl))
                                         : pack_words(first4(dh), first4(dl));
          }
        }
        // K_c D and K_{c-1} D; beside them Q_c K_{c-1}^T and K_c K_{c-1}^T,
        // whose accumulators hold, at lane (n, grp) register i, (K_{c-1}
        // Q_c^T)[n][4 grp + i] and (K_{c-1} K_c^T)[n][4 grp + i]: the lane's
        // parts of the split A fragments of M1 and M2 once scaled
        f32x4 KA = zero4(), KB = zero4(), A1 = zero4(), A2 = zero4();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const bf16x8 ka = RW::afrag(ra + R::KR, s, n, grp);
          const bf16x8 kb = RW::afrag(rb + R::KR, s, n, grp);
          const bf16x8 qa = RW::afrag(ra + R::QR, s, n, grp);
          KA = mma32b(ka, Dl[s], KA);
          KB = mma32b(kb, Dl[s], KB);
          A1 = mma32b(qa, kb, A1);
          KA = mma32b(ka, Dh[s], KA);
          KB = mma32b(kb, Dh[s], KB);
          A2 = mma32b(ka, kb, A2);
        }
        const float gCa = *reinterpret_cast<const float*>(ra + R::GC);
        const float gCb = *reinterpret_cast<const float*>(rb + R::GC);
        const float gP = gCa * gCb;
#pragma unroll
        for (int t = 0; t < NT; ++t) D[t] = D[t] * gP;
        // the later tile: dU = P^T dO + diag(ec) K D, dY = T^T dU
        const bf16x4 doa = Slab<SPW>::get(ra + R::DO, wave, n, grp);
        const f32x4 gma = *reinterpret_cast<const f32x4*>(ra + R::GM + 16 * grp);
        const f32x4 eca = *reinterpret_cast<const f32x4*>(ra + R::EC + 16 * grp);
        const f32x4 bta = *reinterpret_cast<const f32x4*>(ra + R::BT + 16 * grp);
        const bf16x8 pta = *reinterpret_cast<const bf16x8*>(ra + R::PT + 16 * lane);
        const bf16x8 tta = *reinterpret_cast<const bf16x8*>(ra + R::TT + 16 * lane);
        f32x4 eKA;
#pragma unroll
        for (int i = 0; i < 4; ++i) eKA[i] = eca[i] * KA[i];
        const f32x4 dUa = mma32b(pta, cat8(doa, doa), eKA);
        const Sp4 sua = split4(dUa);
        f32x4 dYa = mma32b(tta, cat8(sua.h, sua.h), zero4());
        dYa = mma32b_lo(tta, sua.l, dYa);
        const Sp4 sya = split4(dYa);
        // the later tile's terms of D_start, scaled by the earlier tile's gamma_C
        const f32x4 dOa = to_f4(doa);
        f32x4 Oa, Za;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float gg = gCb * gma[i];
          Oa[i] = gg * dOa[i];
          Za[i] = -(bta[i] * gg * dYa[i]);
        }
        const Sp4 soa = split4(Oa), sza = split4(Za);
        const bf16x8 ozha = cat8(soa.h, sza.h), ozla = cat8(soa.l, sza.l);
        // K_{c-1} D_mid = gC_c K_{c-1} D + M1 dO_c + M2 dY_c
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          A1[i] *= gma[i];
          A2[i] *= -(bta[i] * gma[i]);
        }
        const Sp4 s1 = split4(A1), s2 = split4(A2);
        const bf16x8 m1 = cat8(s1.h, s1.l), m2 = cat8(s2.h, s2.l);
        KB = KB * gCa;
        KB = mma32b(m1, cat8(doa, doa), KB);
        KB = mma32b(m2, cat8(sya.h, sya.h), KB);
        KB = mma32b_lo(m2, sya.l, KB);
        // D += [Q^T | K^T] [Og ; Z], the 32-deep contraction taking the 16
        // tokens of each; the later tile's update is spread over the earlier
        // tile's serial steps (NT / 4 row blocks of D at a time)
        auto a_terms = [&](int t0) {
#pragma unroll
          for (int t = t0; t < t0 + NT / 4; ++t) {
            const bf16x8 qk = cat8(RW::tfrag(ra + R::QR, t, n, grp), RW::tfrag(ra + R::KR, t, n, grp));
            D[t] = mma32b(qk, ozha, D[t]);
            D[t] = mma32b(qk, ozla, D[t]);
          }
        };
        a_terms(0);
        // the earlier tile
        const bf16x4 dob = Slab<SPW>::get(rb + R::DO, wave, n, grp);
        const f32x4 gmb = *reinterpret_cast<const f32x4*>(rb + R::GM + 16 * grp);
        const f32x4 ecb = *reinterpret_cast<const f32x4*>(rb + R::EC + 16 * grp);
        const f32x4 btb = *reinterpret_cast<const f32x4*>(rb + R::BT + 16 * grp);
        const bf16x8 ptb = *reinterpret_cast<const bf16x8*>(rb + R::PT + 16 * lane);
        const bf16x8 ttb = *reinterpret_cast<const bf16x8*>(rb + R::TT + 16 * lane);
        f32x4 eKB;
#pragma unroll
        for (int i = 0; i < 4; ++i) eKB[i] = ecb[i] * KB[i];
        const f32x4 dUb = mma32b(ptb, cat8(dob, dob), eKB);
        a_terms(NT / 4);
        const Sp4 sub = split4(dUb);
        f32x4 dYb = mma32b(ttb, cat8(sub.h, sub.h), zero4());
        dYb = mma32b_lo(ttb, sub.l, dYb);
        a_terms(NT / 2);
        const f32x4 dOb = to_f4(dob);
        f32x4 Ob, Zb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Ob[i] = gmb[i] * dOb[i];
          Zb[i] = -(btb[i] * gmb[i] * dYb[i]);
        }
        const Sp4 sob = split4(Ob), szb = split4(Zb);
        const bf16x8 ozhb = cat8(sob.h, szb.h), ozlb = cat8(sob.l, szb.l);
        a_terms(3 * NT / 4);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const bf16x8 qk = cat8(RW::tfrag(rb + R::QR, t, n, grp), RW::tfrag(rb + R::KR, t, n, grp));
          D[t] = mma32b(qk, ozhb, D[t]);
          D[t] = mma32b(qk, ozlb, D[t]);
        }
        split_state<NS>(D, Dh, Dl);
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
  // 2 NP loader waves: wave p stages tile p % NP of every epoch of parity
  // p / NP, loading it two epochs ahead
  const int p = (wave - SPW) % NP, q = (wave - SPW) / NP;
  const __bf16* kp = static_cast<const __bf16*>(a.k);
  const __bf16* qp = static_cast<const __bf16*>(a.q);
  const __bf16* dp = static_cast<const __bf16*>(a.dout);
  const int v0 = 16 * SPW * sl;
  // Loads past the sequence end read its last token (NC > 0, so there is one)
  // and are zeroed when staged: no loaded value is touched before then, so
  // that staging one epoch does not wait for the next epoch's loads (vector
  // loads complete in order).  Addresses are a uniform base per tile (token
  // 16 c, head h) plus a 32-bit lane offset.
  const int tsk = a.H * DK, tsv = a.H * a.Dv;     // token strides, elements
  auto tile_base = [&](const __bf16* src, int c, int width) {
    return src + ((sq.tok0 + 16 * c) * a.H + h) * width;
  };
  auto rows = [&](const __bf16* src, int c, uint4* out) {
    const __bf16* b0 = tile_base(src, c, DK);
    const int off = min(n, sq.T - 1 - 16 * c) * tsk + 8 * grp;
#pragma unroll
    for (int x = 0; x < DK / 32; ++x) out[x] = *reinterpret_cast<const uint4*>(b0 + off + 32 * x);
  };
  auto load = [&](D2Raw<DK, SPW>& r, int m) {
    if (NC == 0) return;          // an empty sequence loads nothing
    const int c = NCe - 1 - min(m, NCe - 1);
    rows(kp, c, r.kr);
    rows(qp, c, r.qr);
    // the empty front tile (c == NC) reads tile NC - 1's record, replaced by
    // zeros when staged
    const float* rec = a.rec + (sq.rbase + min(c, NC - 1)) * BRec::FLOATS;
    r.pm = reinterpret_cast<const f32x4*>(rec + BRec::P)[lane];
    r.tm = reinterpret_cast<const f32x4*>(rec + BRec::TINV)[lane];
    r.g = rec[BRec::G + n];
    r.bt = rec[BRec::BETA + n];
    r.gC = rec[BRec::G + kT - 1];
    Slab<SPW>::load(r.dr, tile_base(dp, c, a.Dv) + v0, tsv, sq.T - 1 - 16 * c, lane);
  };
  // CHK: the tile reaches past the sequence end, and loads there are zeroed
  auto stage = [&](const D2Raw<DK, SPW>& r, int m, auto chk) {
    constexpr bool CHK = decltype(chk)::value;
    char* rec = rec_of(m);
    const int c = NCe - 1 - m;
    const bool rok = !CHK || 16 * c + n < sq.T;
#pragma unroll
    for (int x = 0; x < DK / 32; ++x) {
      *reinterpret_cast<uint4*>(rec + R::KR + n * RW::PITCH + 16 * (4 * x + grp)) = zero_if(rok, r.kr[x]);
      *reinterpret_cast<uint4*>(rec + R::QR + n * RW::PITCH + 16 * (4 * x + grp)) = zero_if(rok, r.qr[x]);
    }
    // the empty front tile: no rows, P = T = 0, unit decay, beta = 0
    const bool real = !CHK || c < NC;
    // P and T arrive row-major (lane l holds row l / 4, columns 4 (l % 4) + e)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      put_op(rec + R::PT, lane >> 2, 4 * (lane & 3) + e, real ? r.pm[e] : 0.f, true);
      put_op(rec + R::TT, lane >> 2, 4 * (lane & 3) + e, real ? r.tm[e] : 0.f, true);
    }
    Slab<SPW>::template stage<CHK>(rec + R::DO, r.dr, sq.T - 16 * c, lane);
    if (grp == 0) {
      const float g = real ? r.g : 0.f, gC = real ? r.gC : 0.f;
      reinterpret_cast<float*>(rec + R::GM)[n] = __expf(g);
      reinterpret_cast<float*>(rec + R::EC)[n] = __expf(gC - g);
      reinterpret_cast<float*>(rec + R::BT)[n] = real ? r.bt : 0.f;
      if (n == 0) *reinterpret_cast<float*>(rec + R::GC) = __expf(gC);
    }
  };
  auto store = [&](const D2Raw<DK, SPW>& r, int m) {
    if (m >= NCe) return;
    // only the tiles at the sequence end need zeroing (a uniform test)
    if (16 * (NCe - 1 - m) + 16 <= sq.T) stage(r, m, std::false_type{});
    else stage(r, m, std::true_type{});
  };
  D2Raw<DK, SPW> r;
  load(r, q * NP + p);
  if (q == 0) {
    store(r, p);                // epoch 0
    load(r, 2 * NP + p);
  }
  __syncthreads();
  for (int ep = 0; ep < NE; ++ep) {
    // the chain runs epoch ep; epoch ep + 1 is staged by the loaders of its parity
    if (((ep + 1) & 1) == q) {
      store(r, (ep + 1) * NP + p);
      load(r, (ep + 3) * NP + p);
    }
    __syncthreads();
  }
}

// The forward states and the state gradients do not depend on each other: one
// launch runs both, blocks [0, nblk) the first and [nblk, 2 nblk) the second,
// so that the two serial chains share the compute units.  Each block has SPW
// chain waves (one per 16-column slice) and 2 NP loader waves.
template <int DK, int NP, int SPW>
__global__ __launch_bounds__(64 * (2 * NP + SPW)) void bwd2_states_kernel(BwdArgs a, int nblk) {
  constexpr int HB = 2 * NP * H2Rec<DK, SPW>::BYTES, DB = 2 * NP * D2Rec<DK, SPW>::BYTES;
  __shared__ __attribute__((aligned(16))) char smem[HB > DB ? HB : DB];
  if ((int)blockIdx.x < nblk) hstates_body<DK, NP, SPW>(a, blockIdx.x, smem);
  else dh_body<DK, NP, SPW>(a, blockIdx.x - nblk, smem);
}

}  // namespace

hipError_t launch_bwd_bf16_states(const void* args, size_t args_bytes, int Dk, int spw, unsigned grid,
                                  int nblk, hipStream_t st) {
  if (args_bytes != sizeof(BwdArgs) || (Dk != 64 && Dk != 128)) return hipErrorInvalidValue;
  BwdArgs a;
  std::memcpy(&a, args, sizeof a);
  const bool big = Dk == 128;
  if (spw == 4) {
    if (big) hipLaunchKernelGGL((bwd2_states_kernel<128, 2, 4>), dim3(grid), dim3(64 * 8), 0, st, a, nblk);
    else hipLaunchKernelGGL((bwd2_states_kernel<64, 2, 4>), dim3(grid), dim3(64 * 8), 0, st, a, nblk);
  } else if (spw == 2) {
    if (big) hipLaunchKernelGGL((bwd2_states_kernel<128, 2, 2>), dim3(grid), dim3(64 * 6), 0, st, a, nblk);
    else hipLaunchKernelGGL((bwd2_states_kernel<64, 2, 2>), dim3(grid), dim3(64 * 6), 0, st, a, nblk);
  } else if (spw == 1) {
    if (big) hipLaunchKernelGGL((bwd2_states_kernel<128, 2, 1>), dim3(grid), dim3(64 * 5), 0, st, a, nblk);
    else hipLaunchKernelGGL((bwd2_states_kernel<64, 2, 1>), dim3(grid), dim3(64 * 5), 0, st, a, nblk);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace la
