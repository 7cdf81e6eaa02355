// chunk_bwd_bf16.hip -- the reverse pass for bf16 q, k, v and dout on the bf16
// matrix cores, with the forward states kept only at every kHS-th tile and the
// state gradients at every kGS-th.
//
// Same algebra as chunk_bwd.hip (the adjoint of the tiled forward form; the
// pages -- "Deep Dive: The Next Generation of Ultra-Long Context Sparse MoE
// LLMs", sec. 3.2, and "Core Technologies Behind Ultra-Long-Context Sparse MoE
// Large Models", sec. 2.1 and 2.3 -- give the tiled forward pass and frame the
// bounded decay around BF16 training, and print no backward pass).  What
// differs is where the work runs and what goes through memory:
//
//  * Products.  q, k, v and dout are bf16, so they enter the bf16 MFMA
//    exactly.  Every float32 operand X (the state H, its gradient D, T, P, Y,
//    U, dU, dY and their scaled forms) is split into bf16 parts X = X_hi +
//    X_lo + e with |e| <= 2^-16 |X|, and a product of two split operands keeps
//    the three terms hi.hi + lo.hi + hi.lo; a product with an exact bf16
//    operand keeps both parts.  A 16-deep contraction runs as 32-deep MFMAs:
//    [X, X] . [Y_hi ; Y_lo] with one split operand, [X_hi | X_lo] . [Y_hi ;
//    Y_hi] then [X_hi | X_lo] . [Y_lo ; 0] with two.
//    Accumulation is float32 throughout and the state and state gradient are
//    carried in float32.
//  * Checkpoints.  The state chain stores H only at the start of every kHS-th
//    tile and the gradient chain stores D = dL/dH' only at the end of every
//    group of kGS tiles, each as packed (hi, lo) bf16 words (4 bytes per
//    element, the float32 size).  The gradient kernel takes one group per
//    workgroup and walks its tiles backwards: it rebuilds H at the start of
//    tile j by stepping the forward recurrence j % kHS times from the nearest
//    stored state, and carries D backwards tile by tile,
//        D_{j-1} = gamma_C D_j + Q^T diag(gamma) dO - K^T diag(beta gamma) dY,
//    from the group's stored end.  With kHS = 2 and kGS = 4: 3/8 of the state
//    traffic of storing both at every tile, for 0.5 extra forward steps per
//    tile.
//
// Three launches:
//   bwd_prep_wave_kernel  the per-tile record of la_bwd.h, one wave per tile;
//   bwd2_states_kernel    (chunk_bwd_bf16_states.hip) two kinds of block in
//                         one launch, per (sequence, head, SPW slices of 16
//                         columns of d_v): the forward chain, serial over
//                         tiles (H at every kHS-th tile), and the gradient
//                         chain, serial backwards over pairs of tiles (D at
//                         every group end, and dh0); the two do not depend on
//                         each other;
//   bwd2_grad_kernel      per group of kGS tiles, all of d_v (one 16-column
//                         slice per wave): dq, dk, dv, dbeta, dg.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "la_bwd.h"
#include "la_bwd_bf16.h"
#include "la_device.h"
#include "la_launch.h"

namespace la {
namespace {

// ------------------------------------------------------------- tile prep
// The per-tile record (in-tile running sum G of the log-decay, beta, T =
// (I + A)^{-1}, P = E o Q K^T, E o K K^T) with one wave per tile: K K^T and
// Q K^T on the bf16 MFMA (the bf16 rows enter exactly; float32 sums), G summed
// in token order, and T by forward substitution, one column per lane.
template <int DK>
__global__ __launch_bounds__(256) void bwd_prep_wave_kernel(BwdArgs a, int64_t ntiles) {
  constexpr int NS = DK / 32;
  __shared__ float sA[4][kT][kT + 1];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, n = lane & 15, grp = lane >> 4;
  const int64_t tile = (int64_t)blockIdx.x * 4 + w;
  int b, h, c;
  if (tile >= ntiles || !bwd_tile(a, tile, b, h, c)) return;   // the whole wave
  const BSeq sq = bwd_seq(a, b, h);
  // lane (n, grp): token n of the tile; elements 32 s + 8 grp .. + 7 of its
  // k and q rows (one 32-deep fragment per s, the same for both operands)
  const int tok = c * kT + n;
  const bool in = tok < sq.T;
  const int64_t row = (sq.tok0 + tok) * a.H + h;
  bf16x8 kf[NS], qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    kf[s] = bf16x8{};
    qf[s] = bf16x8{};
    if (in) {
      kf[s] = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.k) + row * DK + 32 * s + 8 * grp);
      qf[s] = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(a.q) + row * DK + 32 * s + 8 * grp);
    }
  }
  const float gx = in ? gate_at(a, row) : 0.f;
  const float bx = in ? a.beta[row] : 0.f;
  // K K^T and Q K^T: lane (n, grp) register r holds entry (4 grp + r, n)
  f32x4 kk = zero4(), qk = zero4();
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    kk = mma32b(kf[s], kf[s], kk);
    qk = mma32b(qf[s], kf[s], qk);
  }
  // G in token order (each lane: its column n and its rows 4 grp + r), beta of the rows
  float Gc = 0.f, acc = 0.f;
  f32x4 Gr = zero4(), Br = zero4();
#pragma unroll
  for (int t = 0; t < kT; ++t) {
    acc += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gx), t));
    const float bt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bx), t));
    Gc = t == n ? acc : Gc;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      Gr[r] = t == 4 * grp + r ? acc : Gr[r];
      Br[r] = t == 4 * grp + r ? bt : Br[r];
    }
  }
  float* const rec = a.rec + tile * BRec::FLOATS;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 4 * grp + r;
    const float e = n <= t ? __expf(Gr[r] - Gc) : 0.f;
    const float ekk = n < t ? e * kk[r] : 0.f;
    rec[BRec::EKK + kT * t + n] = ekk;
    rec[BRec::P + kT * t + n] = e * qk[r];
    sA[w][t][n] = Br[r] * ekk;
  }
  wave_fence();
  // (I + A) T = I: lane j < 16 takes column j, row by row
  if (lane < kT) {
    float tc[kT];
#pragma unroll
    for (int r = 0; r < kT; ++r) {
      float sacc = r == lane ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < r; ++m) sacc -= sA[w][r][m] * tc[m];
      tc[r] = sacc;
      rec[BRec::TINV + kT * r + lane] = sacc;
    }
    rec[BRec::G + lane] = Gc;
    rec[BRec::BETA + lane] = bx;
  }
}

// --------------------------------------------------- per-group gradients
// LDS of the gradient kernel (bytes).
template <int DK>
struct G2Lds {
  static constexpr int NT = DK / 16;
  static constexpr int ROWS = Rows<DK>::BYTES;
  static constexpr int KR = 0;                         // K rows of the group's tiles
  static constexpr int QR = KR + kGS * ROWS;           // Q rows
  static constexpr int TF = QR + kGS * ROWS;           // [T hi | T lo] A fragments, 1 KB per tile
  static constexpr int TT = TF + kGS * 1024;           // [T^T hi | T^T lo]
  static constexpr int PT = TT + kGS * 1024;           // [P^T hi | P^T lo]
  static constexpr int PM = PT + kGS * 1024;           // P float32, 16 x 17 per tile
  static constexpr int EK = PM + kGS * 1088;           // E o K K^T float32, 16 x 16 per tile
  static constexpr int SC = EK + kGS * 1024;           // per tile G, beta, gamma, ec, dg/dg' [16] each
  static constexpr int XR = SC + kGS * 512;            // transposition tiles / reduction
  static constexpr int XT = 4 * NT / 2 > 9 ? 4 * NT / 2 : 9;   // transposition tiles per wave
  static constexpr int XW = XT * 512;                  // transposition bytes per wave
  static constexpr int XBYTES = 8 * XW > 8 * NT * 1024 ? 8 * XW : 8 * NT * 1024;
  static constexpr int RS = XR + XBYTES;               // dP, dA partials: 8 waves x 2 x 1 KB
  static constexpr int RW = RS + 8 * 2 * 1024;         // row sums: 8 waves x 3 x 16 floats
  static constexpr int TL = RW + 8 * 3 * 64;           // PE, M, PP, AA: 4 x 16 x 17 floats
  static constexpr int TR = TL + 4 * 1088;             // row B, G, W, AK [16] each
  static constexpr int HD = TR + 256;                  // <H, dH'> per wave
  static constexpr int BYTES = HD + 32;
};

template <int DK>
__global__ __launch_bounds__(512) void bwd2_grad_kernel(BwdArgs a) {
  using L = G2Lds<DK>;
  using RW = Rows<DK>;
  constexpr int NS = DK / 32, NT = DK / 16;
  __shared__ __attribute__((aligned(16))) char sm[L::BYTES];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, n = lane & 15, grp = lane >> 4;
  int b, h, g;
  if (!bwd2_group(a, blockIdx.x, b, h, g)) return;   // a slot no group uses: the whole block
  const BSeq sq = bwd_seq(a, b, h);
  const int c0 = kGS * g;
  const int GSn = min(kGS, sq.NC - c0);
  const int64_t gi = grp_base(a, b, h) + g;
  const int NV = a.Dv / 16;
  const bool act = w < NV;            // waves beyond the slices only join the reductions
  const int v0 = 16 * w;
  const __bf16* vp = static_cast<const __bf16*>(a.v);
  const __bf16* dop = static_cast<const __bf16*>(a.dout);

  // ---- this wave's slice of the group's checkpoints (the states at tiles 0
  // and kHS and the end-state gradient dH', packed words), requested before
  // the staging loads; the start state of the next tile is requested at the
  // end of each tile (an L2 hit)
  const int64_t ckoff = gi * DK * a.Dv + (int64_t)w * DK * 16;
  // start state stored at tile kHS * (j / kHS) of the group
  auto hp = [&](int j) {
    return reinterpret_cast<const uint4*>(a.hw + (gi * kHPG + j / kHS) * DK * a.Dv +
                                          (int64_t)w * DK * 16);
  };
  uint4 hw8[NT], dw8[NT];
  // v and dO of the group's tiles in this wave's slice, read as rows (lane
  // (n, grp): token n, columns 4 grp .. 4 grp + 3; zeros past the sequence end)
  uint2 vrow[kGS], orow[kGS];
  if (act) {
    const uint4* const dp = reinterpret_cast<const uint4*>(a.dw + ckoff);
    const uint4* const h0p = hp(GSn - 1);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      hw8[t] = h0p[t * 64 + lane];
      dw8[t] = dp[t * 64 + lane];
    }
#pragma unroll
    for (int m = 0; m < kGS; ++m) {
      const int tok = 16 * (c0 + m) + n;
      const int64_t e = ((sq.tok0 + tok) * a.H + h) * a.Dv + v0 + 4 * grp;
      vrow[m] = tok < sq.T ? *reinterpret_cast<const uint2*>(vp + e) : uint2{0u, 0u};
      orow[m] = tok < sq.T ? *reinterpret_cast<const uint2*>(dop + e) : uint2{0u, 0u};
    }
  }

  // ---- stage the group's k and q rows (zeros past the sequence end) and
  // tile operators; every global load is issued before the first LDS write
  {
    constexpr int PER_ROW = 2 * DK / 16;                 // 16-byte pieces of a row
    constexpr int PER_T = 16 * PER_ROW;                  // pieces of a tile's rows
    constexpr int NLD = (2 * kGS * PER_T + 511) / 512;   // k and q pieces per thread
    constexpr int NRC = (kGS * 256 + 511) / 512;         // operator elements per thread
    uint4 u[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int x = tid + 512 * i;
      const int qk = x / (kGS * PER_T), rem = x % (kGS * PER_T);
      const int j = rem / PER_T, r = (rem % PER_T) / PER_ROW, p = rem % PER_ROW;
      const int tok = 16 * (c0 + j) + r;
      u[i] = uint4{0u, 0u, 0u, 0u};
      if (qk < 2 && j < GSn && tok < sq.T) {
        const __bf16* src = static_cast<const __bf16*>(qk ? a.q : a.k);
        u[i] = *reinterpret_cast<const uint4*>(src + ((sq.tok0 + tok) * a.H + h) * DK + 8 * p);
      }
    }
    float tv[NRC], pv[NRC], ev[NRC];
#pragma unroll
    for (int i = 0; i < NRC; ++i) {
      const int x = tid + 512 * i;
      if (x < GSn * 256) {
        const float* rec = a.rec + (sq.rbase + c0 + (x >> 8)) * BRec::FLOATS;
        tv[i] = rec[BRec::TINV + (x & 255)];
        pv[i] = rec[BRec::P + (x & 255)];
        ev[i] = rec[BRec::EKK + (x & 255)];
      }
    }
    const bool small = tid < GSn * 16;
    const int sj = tid >> 4, st = tid & 15, stok = 16 * (c0 + sj) + st;
    float gv = 0.f, gC = 0.f, btv = 0.f, xg = 0.f;
    if (small) {
      const float* rec = a.rec + (sq.rbase + c0 + sj) * BRec::FLOATS;
      gv = rec[BRec::G + st];
      gC = rec[BRec::G + kT - 1];
      btv = rec[BRec::BETA + st];
      if (a.gate_logit && stok < sq.T) xg = a.gate[(sq.tok0 + stok) * a.H + h];
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int x = tid + 512 * i;
      const int qk = x / (kGS * PER_T), rem = x % (kGS * PER_T);
      const int j = rem / PER_T, r = (rem % PER_T) / PER_ROW, p = rem % PER_ROW;
      if (qk < 2)
        *reinterpret_cast<uint4*>(sm + (qk ? L::QR : L::KR) + j * L::ROWS + r * RW::PITCH + 16 * p) = u[i];
    }
#pragma unroll
    for (int i = 0; i < NRC; ++i) {
      const int x = tid + 512 * i;
      if (x < GSn * 256) {
        const int j = x >> 8, e = x & 255, t = e >> 4, ii = e & 15;
        put_op(sm + L::TF + j * 1024, t, ii, tv[i], false);
        put_op(sm + L::TT + j * 1024, t, ii, tv[i], true);
        put_op(sm + L::PT + j * 1024, t, ii, pv[i], true);
        reinterpret_cast<float*>(sm + L::PM + j * 1088)[t * 17 + ii] = pv[i];
        reinterpret_cast<float*>(sm + L::EK + j * 1024)[e] = ev[i];
      }
    }
    if (small) {
      float* sc = reinterpret_cast<float*>(sm + L::SC + sj * 512);
      sc[st] = gv;
      sc[16 + st] = btv;
      sc[32 + st] = __expf(gv);
      sc[48 + st] = __expf(gC - gv);
      // dL/dx = dg/dx * dL/dg in logit mode (g = -G sigmoid(x)), 1 in log mode
      float dgx = 1.f;
      if (a.gate_logit && stok < sq.T) {
        const float sg = sigmoid_f(xg);
        dgx = -a.G * sg * (1.f - sg);
      }
      sc[64 + st] = dgx;
    }
  }
  // dH' of the tile in hand, as split fragments (carried backwards tile by
  // tile; each step rounds it to hi + lo, as the stored checkpoints are)
  bf16x8 Dh[NS], Dl[NS];
  char* const xr = sm + L::XR + w * L::XW;         // this wave's transposition tiles
  // v and dO in accumulator layout (lane (n, grp) holds rows 4 grp .. 4 grp + 3
  // of column n): the row reads above, transposed through the wave's tiles
  bf16x4 vg[kGS], og[kGS];
  if (act) {
    words_state<NS>(dw8, 1, Dh, Dl);
#pragma unroll
    for (int m = 0; m < kGS; ++m) {
      tr_put(xr + m * 512, lane, __builtin_bit_cast(bf16x4, vrow[m]));
      tr_put(xr + (kGS + m) * 512, lane, __builtin_bit_cast(bf16x4, orow[m]));
    }
    wave_fence();
#pragma unroll
    for (int m = 0; m < kGS; ++m) {
      vg[m] = tr_get(xr + m * 512, n, grp);
      og[m] = tr_get(xr + (kGS + m) * 512, n, grp);
    }
  }
  static_assert(2 * kGS <= L::XT, "v and dO tiles fit the wave's transposition area");
  __syncthreads();

  f32x4* const red = reinterpret_cast<f32x4*>(sm + L::XR);
  f32x4* const rs = reinterpret_cast<f32x4*>(sm + L::RS);
  float* const rw = reinterpret_cast<float*>(sm + L::RW);
  float (*const sPE)[17] = reinterpret_cast<float (*)[17]>(sm + L::TL);
  float (*const sM)[17] = reinterpret_cast<float (*)[17]>(sm + L::TL + 1088);
  float (*const sPP)[17] = reinterpret_cast<float (*)[17]>(sm + L::TL + 2 * 1088);
  float (*const sAA)[17] = reinterpret_cast<float (*)[17]>(sm + L::TL + 3 * 1088);
  float* const sRowB = reinterpret_cast<float*>(sm + L::TR);
  float* const sRowG = sRowB + 16;
  float* const sRowW = sRowB + 32;
  float* const sRowAK = sRowB + 48;
  float* const sHdH = reinterpret_cast<float*>(sm + L::HD);

  for (int j = GSn - 1; j >= 0; --j) {
    // The per-thread indices are re-derived every tile from an opaque copy of
    // the lane, so that no hoisted per-thread address stays live across the
    // loop (such addresses spill, and each reload waits for all memory
    // operations in flight).
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const int lane = lane_o, n = lane_o & 15, grp = lane_o >> 4, tid = 64 * w + lane_o;
    // v or dO of tile m of the group (m wave-uniform: selects, no indexing)
    auto pick = [](const bf16x4* x, int m) {
      static_assert(kGS == 4, "four tiles per group");
      return m == 0 ? x[0] : m == 1 ? x[1] : m == 2 ? x[2] : x[3];
    };
    const int c = c0 + j;
    const char* kr = sm + L::KR + j * L::ROWS;
    const char* qr = sm + L::QR + j * L::ROWS;
    const float* sc = reinterpret_cast<const float*>(sm + L::SC + j * 512);
    const float gamC = __expf(sc[kT - 1]);
    f32x4 pB = zero4(), pG = zero4(), pW = zero4(), dPp = zero4(), dAp = zero4();
    float hdh = 0.f;
    bf16x8 ozh, ozl;             // [gamma dO ; -beta gamma dY], hi and lo parts, for the step to j - 1
    bf16x8 dO8, ayuh, ayul;      // row fragments: [dO, dO], [aY | aU] hi and lo parts
    bf16x8 Hh[NS], Hl[NS];       // H at the start of tile j, split
    if (act) {
      // H at the start of tile j: j % kHS forward steps from the state stored
      // at tile kHS * (j / kHS)
      const bf16x4 dob = pick(og, j);
      const int jb = j - j % kHS;
      f32x4 Hacc[NT];
      words_state<NS>(hw8, 1, Hh, Hl);
      if (j > jb) {
#pragma unroll
        for (int t = 0; t < NT; ++t) Hacc[t] = words_f4(hw8[t]);
      }
      for (int m = jb; m < j; ++m) {
        const char* km = sm + L::KR + m * L::ROWS;
        const float* scm = reinterpret_cast<const float*>(sm + L::SC + m * 512);
        // K H as two independent chains (hi and lo parts of H), every k
        // fragment read first
        bf16x8 ka[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) ka[s] = RW::afrag(km, s, n, grp);
        f32x4 Rl = zero4(), Rh = zero4();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          Rl = mma32b(ka[s], Hl[s], Rl);
          Rh = mma32b(ka[s], Hh[s], Rh);
        }
        const f32x4 Rk = Rh + Rl;
        const f32x4 vf = to_f4(pick(vg, m));
        const f32x4 gm = *reinterpret_cast<const f32x4*>(scm + 32 + 4 * grp);
        const f32x4 ec = *reinterpret_cast<const f32x4*>(scm + 48 + 4 * grp);
        const f32x4 bt = *reinterpret_cast<const f32x4*>(scm + 16 + 4 * grp);
        const float gCm = __expf(scm[kT - 1]);
        const bf16x8 tf = *reinterpret_cast<const bf16x8*>(sm + L::TF + m * 1024 + 16 * lane);
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
          const bf16x4 kt = RW::tfrag(km, t, n, grp);
          Hacc[t] = Hacc[t] * gCm;
          Hacc[t] = mma32b(cat8(kt, kt), ub, Hacc[t]);
        }
        split_state<NS>(Hacc, Hh, Hl);
      }

      // K H, Q H, K dH' and H^T dH' (its trace is <H, dH'>)
      f32x4 KH = zero4(), QH = zero4(), KdH = zero4(), HtD = zero4();
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 ka = RW::afrag(kr, s, n, grp);
        const bf16x8 qa = RW::afrag(qr, s, n, grp);
        KH = mma32b(ka, Hl[s], KH);
        KH = mma32b(ka, Hh[s], KH);
        QH = mma32b(qa, Hl[s], QH);
        QH = mma32b(qa, Hh[s], QH);
        KdH = mma32b(ka, Dl[s], KdH);
        KdH = mma32b(ka, Dh[s], KdH);
        HtD = mma32b(Hl[s], Dh[s], HtD);
        HtD = mma32b(Hh[s], Dl[s], HtD);
        HtD = mma32b(Hh[s], Dh[s], HtD);
      }
      hdh = (n >> 2) == grp ? HtD[n & 3] : 0.f;
      const f32x4 gm4 = *reinterpret_cast<const f32x4*>(sc + 32 + 4 * grp);
      const f32x4 bt4 = *reinterpret_cast<const f32x4*>(sc + 16 + 4 * grp);
      const f32x4 ec4 = *reinterpret_cast<const f32x4*>(sc + 48 + 4 * grp);
      const f32x4 vf = to_f4(pick(vg, j)), dd = to_f4(dob);
      const bf16x8 tf = *reinterpret_cast<const bf16x8*>(sm + L::TF + j * 1024 + 16 * lane);
      const bf16x8 tt = *reinterpret_cast<const bf16x8*>(sm + L::TT + j * 1024 + 16 * lane);
      const bf16x8 pt = *reinterpret_cast<const bf16x8*>(sm + L::PT + j * 1024 + 16 * lane);
      f32x4 vres, Y, eKD;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vres[i] = vf[i] - gm4[i] * KH[i];
        Y[i] = bt4[i] * vres[i];
        eKD[i] = ec4[i] * KdH[i];
      }
      const Sp4 sy = split4(Y);
      f32x4 U = mma32b(tf, cat8(sy.h, sy.h), zero4());
      U = mma32b_lo(tf, sy.l, U);
      const f32x4 dU = mma32b(pt, cat8(dob, dob), eKD);
      const Sp4 sdu = split4(dU);
      f32x4 dY = mma32b(tt, cat8(sdu.h, sdu.h), zero4());
      dY = mma32b_lo(tt, sdu.l, dY);
      f32x4 aY, aU;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pB[i] = dY[i] * vres[i];
        pG[i] = gm4[i] * QH[i] * dd[i] - bt4[i] * gm4[i] * dY[i] * KH[i];
        pW[i] = eKD[i] * U[i];
        aY[i] = -(bt4[i] * gm4[i] * dY[i]);
        aU[i] = ec4[i] * U[i];
      }
      // dv = diag(beta) dY: row 4 grp + i, columns v0 .. v0 + 15
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 16 * c + 4 * grp + i;
        if (tok < sq.T) a.dv[((sq.tok0 + tok) * a.H + h) * a.Dv + v0 + n] = bt4[i] * dY[i];
      }
      // row fragments of dO, U, dY, aY, aU
      const Sp4 su = split4(U), sdy = split4(dY), say = split4(aY), sau = split4(aU);
      {
        f32x4 Og;
#pragma unroll
        for (int i = 0; i < 4; ++i) Og[i] = gm4[i] * dd[i];
        const Sp4 so = split4(Og);
        ozh = cat8(so.h, say.h);
        ozl = cat8(so.l, say.l);
      }
      tr_put(xr + 0 * 512, lane, dob);
      tr_put(xr + 1 * 512, lane, su.h);
      tr_put(xr + 2 * 512, lane, su.l);
      tr_put(xr + 3 * 512, lane, sdy.h);
      tr_put(xr + 4 * 512, lane, sdy.l);
      tr_put(xr + 5 * 512, lane, say.h);
      tr_put(xr + 6 * 512, lane, say.l);
      tr_put(xr + 7 * 512, lane, sau.h);
      tr_put(xr + 8 * 512, lane, sau.l);
      wave_fence();
      const bf16x4 dOr = tr_get(xr + 0 * 512, n, grp);
      const bf16x4 Urh = tr_get(xr + 1 * 512, n, grp), Url = tr_get(xr + 2 * 512, n, grp);
      const bf16x4 dYrh = tr_get(xr + 3 * 512, n, grp), dYrl = tr_get(xr + 4 * 512, n, grp);
      const bf16x4 aYrh = tr_get(xr + 5 * 512, n, grp), aYrl = tr_get(xr + 6 * 512, n, grp);
      const bf16x4 aUrh = tr_get(xr + 7 * 512, n, grp), aUrl = tr_get(xr + 8 * 512, n, grp);
      wave_fence();
      dPp = mma32b(cat8(dOr, dOr), cat8(Urh, Url), dPp);
      dAp = mma32b(cat8(dYrh, dYrl), cat8(Urh, Urh), dAp);
      dAp = mma32b_lo(cat8(dYrh, dYrl), Url, dAp);
      ayuh = cat8(aYrh, aUrh);
      ayul = cat8(aYrl, aUrl);
      dO8 = cat8(dOr, dOr);
    }

    // ---- cross-wave reduction
    // (row sums over the slice's 16 columns land in lane n = 15)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pB[i] = rowsum16(pB[i]);
      pG[i] = rowsum16(pG[i]);
      pW[i] = rowsum16(pW[i]);
    }
    hdh = rowsum16(hdh);
    {
      const int hb = __builtin_bit_cast(int, hdh);
      hdh = __builtin_bit_cast(float, __builtin_amdgcn_readlane(hb, 15)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(hb, 31)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(hb, 47)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(hb, 63));
    }
    // dq partials over this wave's slice: dO H^T, through row fragments of H
    // (SQ 32-row blocks of d_k per LDS round trip)
    constexpr int SQ = L::XT / 4, SK = L::XT / 8;
    static_assert(NS % SQ == 0 && NS % SK == 0, "whole rounds of transposes");
    f32x4 dQp[NT];
#pragma unroll
    for (int r = 0; r < NT; ++r) dQp[r] = zero4();
    if (act) {
#pragma unroll
      for (int s0 = 0; s0 < NS; s0 += SQ) {
#pragma unroll
        for (int s = s0; s < s0 + SQ; ++s) {
          char* const x4 = xr + 4 * (s - s0) * 512;
          tr_put(x4 + 0 * 512, lane, first4(Hh[s]));
          tr_put(x4 + 1 * 512, lane, first4(Hl[s]));
          tr_put(x4 + 2 * 512, lane, second4(Hh[s]));
          tr_put(x4 + 3 * 512, lane, second4(Hl[s]));
        }
        wave_fence();
#pragma unroll
        for (int s = s0; s < s0 + SQ; ++s) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            char* const x4 = xr + 4 * (s - s0) * 512;
            const bf16x4 hrh = tr_get(x4 + (2 * e) * 512, n, grp);
            const bf16x4 hrl = tr_get(x4 + (2 * e + 1) * 512, n, grp);
            dQp[2 * s + e] = mma32b(dO8, cat8(hrh, hrl), dQp[2 * s + e]);
          }
        }
        wave_fence();
      }
    }
    __syncthreads();                       // every wave is done with its transposition tiles
#pragma unroll
    for (int r = 0; r < NT; ++r) red[(w * NT + r) * 64 + lane] = dQp[r];
    rs[(w * 2 + 0) * 64 + lane] = dPp;
    rs[(w * 2 + 1) * 64 + lane] = dAp;
    if (n == 15) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rw[(w * 3 + 0) * 16 + 4 * grp + i] = pB[i];
        rw[(w * 3 + 1) * 16 + 4 * grp + i] = pG[i];
        rw[(w * 3 + 2) * 16 + 4 * grp + i] = pW[i];
      }
    }
    if (lane == 0) sHdH[w] = hdh;
    __syncthreads();
    // wave w < NT owns 16-row block w of d_k for dq and dk
    f32x4 dQa = zero4(), dKa = zero4();
    if (w < NT) {
      for (int v = 0; v < 8; ++v) dQa += red[(v * NT + w) * 64 + lane];
      // dq = diag(gamma) dO H^T + ...: the row scale after the sum over slices
#pragma unroll
      for (int i = 0; i < 4; ++i) dQa[i] *= sc[32 + 4 * grp + i];
    }
    const int t = (tid >> 4) & 15, jj = tid & 15;      // (token, token) view, threads < 256
    float dPacc = 0.f, dAacc = 0.f;
    if (tid < 256) {
      for (int v = 0; v < 8; ++v) {
        dPacc += rs[(v * 2 + 0) * 64 + 16 * (t >> 2) + jj][t & 3];
        dAacc -= rs[(v * 2 + 1) * 64 + 16 * (t >> 2) + jj][t & 3];
      }
    }
    __syncthreads();                       // the dq partials are read
    // dk partials over this wave's slice: aY H^T + aU dH'^T
    f32x4 dKp[NT];
#pragma unroll
    for (int r = 0; r < NT; ++r) dKp[r] = zero4();
    if (act) {
#pragma unroll
      for (int s0 = 0; s0 < NS; s0 += SK) {
#pragma unroll
        for (int s = s0; s < s0 + SK; ++s) {
          char* const x8 = xr + 8 * (s - s0) * 512;
          tr_put(x8 + 0 * 512, lane, first4(Hh[s]));
          tr_put(x8 + 1 * 512, lane, first4(Hl[s]));
          tr_put(x8 + 2 * 512, lane, first4(Dh[s]));
          tr_put(x8 + 3 * 512, lane, first4(Dl[s]));
          tr_put(x8 + 4 * 512, lane, second4(Hh[s]));
          tr_put(x8 + 5 * 512, lane, second4(Hl[s]));
          tr_put(x8 + 6 * 512, lane, second4(Dh[s]));
          tr_put(x8 + 7 * 512, lane, second4(Dl[s]));
        }
        wave_fence();
#pragma unroll
        for (int s = s0; s < s0 + SK; ++s) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            char* const x8 = xr + 8 * (s - s0) * 512;
            const int r = 2 * s + e;
            const bf16x4 hrh = tr_get(x8 + (4 * e + 0) * 512, n, grp);
            const bf16x4 hrl = tr_get(x8 + (4 * e + 1) * 512, n, grp);
            const bf16x4 drh = tr_get(x8 + (4 * e + 2) * 512, n, grp);
            const bf16x4 drl = tr_get(x8 + (4 * e + 3) * 512, n, grp);
            // aY H^T + aU D^T as [aY | aU] [H ; D], split by split: hi.hi,
            // lo.hi, hi.lo
            const bf16x8 hdh = cat8(hrh, drh);
            dKp[r] = mma32b(ayuh, hdh, dKp[r]);
            dKp[r] = mma32b(ayul, hdh, dKp[r]);
            dKp[r] = mma32b(ayuh, cat8(hrl, drl), dKp[r]);
          }
        }
        wave_fence();
      }
    }
    __syncthreads();                       // every wave is done with its transposition tiles
#pragma unroll
    for (int r = 0; r < NT; ++r) red[(w * NT + r) * 64 + lane] = dKp[r];
    const float* pm = reinterpret_cast<const float*>(sm + L::PM + j * 1088);
    const float* ek = reinterpret_cast<const float*>(sm + L::EK + j * 1024);
    if (tid < 256) {
      const int i = jj;
      const float e = i <= t ? __expf(sc[t] - sc[i]) : 0.f;
      const float dP = i <= t ? dPacc : 0.f;
      const float dA = i < t ? dAacc : 0.f;
      const float ekk = ek[16 * t + i];
      sPE[t][i] = dP * e;
      sM[t][i] = dA * sc[16 + t] * e;
      sPP[t][i] = dP * pm[17 * t + i];
      sAA[t][i] = dA * sc[16 + t] * ekk;
      float rak = dA * ekk;
      rak = rowsum16(rak);               // the row's total in lane jj = 15
      if (jj == 15) {
        float sb = 0.f, sg = 0.f, sw = 0.f;
        for (int v = 0; v < 8; ++v) {
          sb += rw[(v * 3 + 0) * 16 + t];
          sg += rw[(v * 3 + 1) * 16 + t];
          sw += rw[(v * 3 + 2) * 16 + t];
        }
        sRowB[t] = sb;
        sRowG[t] = sg;
        sRowW[t] = sw;
        sRowAK[t] = rak;
      }
    }
    __syncthreads();
    if (w < NT) {
      for (int v = 0; v < 8; ++v) dKa += red[(v * NT + w) * 64 + lane];
      // in-tile terms: dQ += (dP o E) K, dK += (dP o E)^T Q + (M + M^T) K, over
      // the 16 columns of d_k block w
      f32x4 pe, pet, mm;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 4 * grp + q;
        pe[q] = sPE[n][i];
        pet[q] = sPE[i][n];
        mm[q] = sM[n][i] + sM[i][n];
      }
      const Sp4 spe = split4(pe), spet = split4(pet), smm = split4(mm);
      const bf16x4 kt = RW::tfrag(kr, w, n, grp);
      const bf16x4 qt = RW::tfrag(qr, w, n, grp);
      dQa = mma32b(cat8(spe.h, spe.l), cat8(kt, kt), dQa);
      const bf16x8 qk = cat8(qt, kt);
      dKa = mma32b(cat8(spet.h, smm.h), qk, dKa);
      dKa = mma32b(cat8(spet.l, smm.l), qk, dKa);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 16 * c + 4 * grp + i;
        if (tok < sq.T) {
          const int64_t ro = ((sq.tok0 + tok) * a.H + h) * DK + 16 * w + n;
          a.dq[ro] = dQa[i];
          a.dk[ro] = dKa[i];
        }
      }
    }
    if (tid < 256) {
      // dg_u = sum_{t >= u} dG_t (see chunk_bwd.hip): lane (u, i) takes W_i
      // (i < u) or G_i (i >= u) and column i of PP + AA over the rows t >= u
      // when i < u; a 16-lane sum then gives dg_u - gamma_C <H, dH'>.
      const int u = t, i = jj;
      float x = i < u ? sRowW[i] : sRowG[i];
#pragma unroll
      for (int t2 = 0; t2 < kT; ++t2) {
        const float y = sPP[t2][i] + sAA[t2][i];
        x += (t2 >= u && i < u) ? y : 0.f;
      }
      x = rowsum16(x);                   // the row's total in lane i = 15
      const int tk = 16 * c + u;
      if (i == 15 && tk < sq.T) {
        float hs = 0.f;
        for (int v = 0; v < 8; ++v) hs += sHdH[v];
        const float dg = gamC * hs + x;
        const int64_t idx = (sq.tok0 + tk) * a.H + h;
        a.dgate[idx] = sc[64 + u] * dg;
        a.dbeta[idx] = sRowB[u] + sRowAK[u];
      }
    }
    // dH' at the end of tile j - 1:
    //   D' = gamma_C D + Q^T diag(gamma) dO - K^T diag(beta gamma) dY
    if (act && j > 0) {
      f32x4 Dn[NT];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        Dn[2 * s] = (to_f4(first4(Dh[s])) + to_f4(first4(Dl[s]))) * gamC;
        Dn[2 * s + 1] = (to_f4(second4(Dh[s])) + to_f4(second4(Dl[s]))) * gamC;
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x4 qt = RW::tfrag(qr, t, n, grp);
        const bf16x4 kt = RW::tfrag(kr, t, n, grp);
        const bf16x8 qk = cat8(qt, kt);
        Dn[t] = mma32b(qk, ozh, Dn[t]);
        Dn[t] = mma32b(qk, ozl, Dn[t]);
      }
      split_state<NS>(Dn, Dh, Dl);
      const uint4* const hn = hp(j - 1);
#pragma unroll
      for (int t = 0; t < NT; ++t) hw8[t] = hn[t * 64 + lane];
    }
    __syncthreads();                       // the tile's shared values are consumed
  }
}

// The reverse pass over the tiles of `a`: tile records, both state chains,
// gradients.  With forward_only, the records and the forward chain only (the
// segmented form's first pass: it needs the state after the last tile, a.hTo).
template <int DK>
hipError_t launch_bwd2_t(const BwdArgs& a, hipStream_t st, bool forward_only = false) {
  const int64_t tiles = a.cu ? (int64_t)a.H * a.nslot : (int64_t)a.B * a.H * a.NT;
  const int64_t groups = a.cu ? (int64_t)a.H * a.nslotG : (int64_t)a.B * a.H * a.NG;
  const int64_t slices = (int64_t)a.B * a.H * (a.Dv / 16);
  hipLaunchKernelGGL((bwd_prep_wave_kernel<DK>), dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0, st,
                     a, tiles);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // four (or two) column slices per workgroup when the slice count allows:
  // the staged tile then serves that many chain waves; blocks [0, nblk) carry
  // the forward chain, [nblk, 2 nblk) the gradient chain
  const int spw = (a.Dv / 16) % 4 == 0 ? 4 : (a.Dv / 16) % 2 == 0 ? 2 : 1;
  const int nblk = (int)(slices / spw);
  const unsigned grid = (unsigned)(forward_only ? nblk : 2 * nblk);
  if ((e = launch_bwd_bf16_states(&a, sizeof a, DK, spw, grid, nblk, st)) != hipSuccess || forward_only) return e;
  hipLaunchKernelGGL((bwd2_grad_kernel<DK>), dim3((unsigned)groups), dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace

bool chunk_bwd_bf16_path(int Dk, int Dv, int fp32) {
  return !fp32 && (Dk == 64 || Dk == 128) && Dv % 16 == 0 && Dv >= 16 && Dv <= 128;
}

// Workspace of the bf16 path: the per-tile records, then H words at every
// group start and D words at every group end.
long long chunk_bwd_bf16_workspace_bytes(int B, int T, int H, int Dk, int Dv) {
  const long long nt = (T + kT - 1) / kT;
  const long long tiles = (long long)B * H * nt;
  const long long groups = (long long)B * H * ((nt + kGS - 1) / kGS);
  return tiles * (BRec::FLOATS * 4LL) + groups * (kHPG + 1LL) * Dk * Dv * 4LL;
}

long long chunk_bwd_bf16_varlen_workspace_bytes(int T, int nseq, int H, int Dk, int Dv) {
  const long long tiles = (long long)H * (T / kT + nseq + 1);
  const long long groups = (long long)H * (T / (kT * kGS) + nseq + 1);
  return tiles * (BRec::FLOATS * 4LL) + groups * (kHPG + 1LL) * Dk * Dv * 4LL;
}

// Arguments of one reverse pass (batched, or packed when cu is set), with the
// workspace laid out as the records, then the start-state words, then the
// state-gradient words.
static BwdArgs bwd_args(const void* q, const void* k, const void* v, const void* dout,
                        const float* gate, int gate_logit, float G, const float* beta,
                        const float* h0, const float* dhT, float* dq, float* dk, float* dv,
                        float* dgate, float* dbeta, float* dh0, const int* cu, int B, int T,
                        int H, int Dk, int Dv, void* ws) {
  const int NT = (T + kT - 1) / kT;
  const int nslot = cu ? T / kT + B + 1 : 0;
  const int64_t tiles = cu ? (int64_t)H * nslot : (int64_t)B * H * NT;
  const int NG = (NT + kGS - 1) / kGS;
  const int nslotG = cu ? T / (kT * kGS) + B + 1 : 0;
  const int64_t groups = cu ? (int64_t)H * nslotG : (int64_t)B * H * NG;
  char* w = static_cast<char*>(ws);
  BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.dout = dout;
  a.gate = gate; a.beta = beta; a.h0 = h0; a.dhT = dhT;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dgate = dgate; a.dbeta = dbeta; a.dh0 = dh0;
  a.rec = reinterpret_cast<float*>(w);
  a.hw = reinterpret_cast<unsigned*>(w + tiles * BRec::FLOATS * 4);
  a.dw = a.hw + groups * (int64_t)kHPG * Dk * Dv;
  a.gate_logit = gate_logit; a.G = G;
  a.B = B; a.T = T; a.H = H; a.Dv = Dv; a.NT = NT;
  a.cu = cu; a.nslot = nslot;
  a.NG = NG; a.nslotG = nslotG;
  a.hTo = nullptr;
  return a;
}

hipError_t launch_chunk_bwd_bf16(const void* q, const void* k, const void* v, const void* dout,
                                 const float* gate, int gate_logit, float G, const float* beta,
                                 const float* h0, const float* dhT, float* dq, float* dk,
                                 float* dv, float* dgate, float* dbeta, float* dh0, const int* cu,
                                 int B, int T, int H, int Dk, int Dv, void* ws, hipStream_t st) {
  const BwdArgs a = bwd_args(q, k, v, dout, gate, gate_logit, G, beta, h0, dhT, dq, dk, dv, dgate,
                             dbeta, dh0, cu, B, T, H, Dk, Dv, ws);
  return Dk == 128 ? launch_bwd2_t<128>(a, st) : launch_bwd2_t<64>(a, st);
}

// Segmented form (batched only): per sequence, segments of L tokens (a
// multiple of kT * kGS, so that every tile, group and stored state falls where
// it falls in one pass over the whole sequence).  Workspace: one segment's
// reverse-pass workspace (B = 1, T = L), then float32 [H, Dk, Dv] states at
// the start of segments 1 .. S-1, then two [H, Dk, Dv] state-gradient buffers.
static long long seg_area_bytes(int L, int H, int Dk, int Dv) {
  return (chunk_bwd_bf16_workspace_bytes(1, L, H, Dk, Dv) + 255) / 256 * 256;
}

long long chunk_bwd_bf16_segmented_workspace_bytes(int T, int H, int Dk, int Dv, int L) {
  const long long S = (T + L - 1) / L;
  const long long st = (long long)H * Dk * Dv * 4;
  return seg_area_bytes(std::min(L, T), H, Dk, Dv) + (S > 1 ? S - 1 : 0) * st + 2 * st;
}

hipError_t launch_chunk_bwd_bf16_segmented(const void* q, const void* k, const void* v,
                                           const void* dout, const float* gate, int gate_logit,
                                           float G, const float* beta, const float* h0,
                                           const float* dhT, float* dq, float* dk, float* dv,
                                           float* dgate, float* dbeta, float* dh0, int B, int T,
                                           int H, int Dk, int Dv, int L, void* ws,
                                           hipStream_t st) {
  const int S = (T + L - 1) / L;
  const int64_t nst = (int64_t)H * Dk * Dv;
  char* const w = static_cast<char*>(ws);
  float* const hs = reinterpret_cast<float*>(w + seg_area_bytes(std::min(L, T), H, Dk, Dv));
  float* const dc[2] = {hs + (S > 1 ? S - 1 : 0) * nst, hs + (S > 1 ? S : 1) * nst};
  const __bf16* qb = static_cast<const __bf16*>(q);
  const __bf16* kb = static_cast<const __bf16*>(k);
  const __bf16* vb = static_cast<const __bf16*>(v);
  const __bf16* ob = static_cast<const __bf16*>(dout);
  auto run = [&](const BwdArgs& a, bool forward_only) {
    return Dk == 128 ? launch_bwd2_t<128>(a, st, forward_only)
                     : launch_bwd2_t<64>(a, st, forward_only);
  };
  for (int b = 0; b < B; ++b) {
    // segment s of sequence b: tokens [t0, t0 + Ls), its start state and the
    // gradient of its end state
    auto seg = [&](int s, const float* hin, const float* din, float* dout0) {
      const int64_t t0 = (int64_t)b * T + (int64_t)s * L;
      const int Ls = std::min(L, T - s * L);
      return bwd_args(qb + t0 * H * Dk, kb + t0 * H * Dk, vb + t0 * H * Dv, ob + t0 * H * Dv,
                      gate + t0 * H, gate_logit, G, beta + t0 * H, hin, din,
                      dq + t0 * H * Dk, dk + t0 * H * Dk, dv + t0 * H * Dv, dgate + t0 * H,
                      dbeta + t0 * H, dout0, nullptr, 1, Ls, H, Dk, Dv, ws);
    };
    const float* h0b = h0 ? h0 + b * nst : nullptr;
    auto start = [&](int s) { return s == 0 ? h0b : hs + (int64_t)(s - 1) * nst; };
    // pass 1: the state at every segment start, carried forward
    for (int s = 0; s + 1 < S; ++s) {
      BwdArgs a = seg(s, start(s), nullptr, nullptr);
      a.hTo = hs + (int64_t)s * nst;
      const hipError_t e = run(a, true);
      if (e != hipSuccess) return e;
    }
    // pass 2: the segments backwards, the state gradient carried backwards
    for (int s = S - 1; s >= 0; --s) {
      const float* din = s == S - 1 ? (dhT ? dhT + b * nst : nullptr) : dc[(s + 1) & 1];
      float* dout0 = s == 0 ? (dh0 ? dh0 + b * nst : nullptr) : dc[s & 1];
      const hipError_t e = run(seg(s, start(s), din, dout0), false);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace la
