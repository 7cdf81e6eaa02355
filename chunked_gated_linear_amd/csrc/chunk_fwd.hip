// chunk_fwd.hip -- chunked forward pass of gated delta-rule linear attention.
//
// The sequence is cut into 16-token tiles ("Deep Dive: The Next Generation of
// Ultra-Long Context Sparse MoE LLMs", sec. 3.2).  Inside a tile every token
// interaction is a matrix product on the matrix cores -- the diagonal block
// K K^T / Q K^T and the "historical state -> current token" block Q H, K H
// ("Core Technologies Behind Ultra-Long-Context Sparse MoE Large Models",
// sec. 2.1 and 2.3) -- and the state is carried from tile to tile ("How
// Trillion-Scale Sparse MoE Models Achieve Million-Token Long Context",
// sec. 3.1).
//
// Algebra of one tile (derived from the recurrence; h = S^T, d_k x d_v).  Let
// H be the state entering the tile, G_t the running sum of g inside the tile,
// gamma_t = exp(G_t), delta_t = exp(G_15 - G_t), gamma_C = exp(G_15).  Then
//     A[t][s] = beta_t exp(G_t - G_s) k_t.k_s        (s < t)
//     T       = (I + A)^-1,   Tb = T diag(beta)      (unit lower triangular)
//     P[t][s] = exp(G_t - G_s) q_t.k_s               (s <= t)
//     U       = Tb (V - diag(gamma) K H)             (16 x d_v)
//     O       = diag(gamma) Q H + P U
//     H'      = gamma_C H + K^T diag(delta) U
// Only exponentials of non-positive numbers are ever formed, so no value above
// 1 appears; with the bounded gate (g in [-5, 0]) the in-tile factors stay in
// [exp(-80), 1].  The decay is applied elementwise to the matrix-core results,
// so the diagonal tiles need no special path.
//
// Work split.  One workgroup per (b, h, 16-column slice of d_v); it streams the
// tiles of its sequence in order.  Wave 0 ("chain") owns the fp32 state slice
// H (d_k x 16) in registers and runs the serial part: K H, Q H, the tile solve
// product Tb(.), P U and the rank-16 state update, all on MFMA.  Waves 1..NP
// ("producers") prepare the H-independent parts of upcoming tiles: loads,
// the gate and in-tile cumulative sum, K K^T and K Q^T on MFMA, the decay
// masks, the 16 x 16 triangular solve, and K^T fragments (K transposed by an
// MFMA against the identity).  They hand them over through LDS, double
// buffered by epochs of NP tiles; one workgroup barrier per epoch.  Global
// loads for tile c are issued one epoch before the tile is prepared.
//
// Blocks are numbered so that all d_v slices of one head share an XCD (and its
// L2): the hardware deals workgroups to the 8 XCDs round robin.
//
// The same kernel serves packed sequences (device offsets: each workgroup
// takes its sequence's start and length from them; an empty sequence only
// copies h0 to hT) and raw inputs (the producers L2-normalise each token's q
// and k rows as they load them and take beta = sigmoid of the given logit).
#include "la_device.h"
#include "la_launch.h"

namespace la {

template <typename E, int DK, int NP>
struct Cfg {
  static constexpr int NT = DK / 16;   // 16-row tiles of the state slice
  static constexpr int NS = DK / 32;   // 32-deep contraction blocks
  static constexpr int EB = Elt<E>::kBytes;
  // One prepared tile ("record") in LDS, every field lane-contiguous.
  static constexpr int KF = 0;                        // NS x 64 lanes x 8 elts
  static constexpr int QF = KF + NS * 64 * 8 * EB;    // NS x 64 x 8
  static constexpr int KT = QF + NS * 64 * 8 * EB;    // NT x 64 x 4
  static constexpr int VF = KT + NT * 64 * 4 * EB;    // 64 x 4
  static constexpr int PF = VF + 64 * 4 * EB;         // 64 x 4
  static constexpr int TB = PF + 64 * 4 * EB;         // 16 x 16 row-major
  static constexpr int GM = TB + 256 * EB;            // gamma[16]   f32
  static constexpr int DL = GM + 64;                  // delta[16]   f32
  static constexpr int GC = DL + 64;                  // gamma_C     f32 (x4)
  static constexpr int REC = GC + 16;
  // Producer scratch: A (16 x 16 f32) and beta[16].
  static constexpr int SA = 0;
  static constexpr int SB = 1024;
  static constexpr int SCR = 1024 + 64;
  static constexpr int LDS = 2 * NP * REC + NP * SCR;
  static_assert(REC % 16 == 0 && SCR % 16 == 0, "LDS alignment");
};

// Map the flat block index to (head, d_v slice) so that the NV slices of a head
// land on the same XCD: inside each group of 8 heads, block = slice * 8 + head%8.
__device__ inline void map_block(int n, int NH, int NV, int& head, int& vt) {
  const int per = 8 * NV;
  const int full = NH / 8;
  const int a = n / per;
  if (a < full) {
    const int loc = n - a * per;
    head = 8 * a + (loc & 7);
    vt = loc >> 3;
  } else {
    const int loc = n - full * per;
    const int r = NH - 8 * full;
    head = 8 * full + loc % r;
    vt = loc / r;
  }
}

template <typename E, int DK>
struct Raw {  // producer-side registers for one tile
  typename Elt<E>::F32 kf[DK / 32];
  typename Elt<E>::F32 qf[DK / 32];
  E vv[4];
  float gx, bt;
};

template <typename E, int DK, int NP>
__global__ __launch_bounds__(64 * (NP + 1)) void chunk_fwd_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ gate, int gate_logit, float G,
    const float* __restrict__ beta, const float* h0, E* __restrict__ o, float* hT,
    int B, int TA, int H, int DV, const int* __restrict__ cu, int raw,
    const float* __restrict__ gsc, const float* __restrict__ gbi) {
  using C = Cfg<E, DK, NP>;
  using X = Elt<E>;
  using F16 = typename X::F16;
  using F32 = typename X::F32;
  constexpr int NT = C::NT, NS = C::NS;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  const int NV = DV / 16;
  int head, vt;
  map_block(blockIdx.x, B * H, NV, head, vt);
  const int b = head / H, h = head % H;
  // affine gate pre-activation (logit mode): logit = gsc[h] * x + gbi[h]
  const float gsc_h = gsc ? gsc[h] : 1.f, gbi_h = gbi ? gbi[h] : 0.f;
  const int v0 = vt * 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, grp = lane >> 4;
  // sequence b: T tokens from token tok0 of the token axis -- B sequences of
  // TA tokens (cu == NULL), or tokens [cu[b], cu[b+1]) of one packed sequence
  // of TA tokens (offsets clamped to [0, TA] and made non-decreasing)
  int T;
  int64_t tok0;
  if (cu) {
    const int tb = min(max(cu[b], 0), TA);
    T = min(max(cu[b + 1], tb), TA) - tb;
    tok0 = tb;
  } else {
    T = TA;
    tok0 = (int64_t)b * TA;
  }
  const int NC = (T + 15) >> 4;
  const int NE = (NC + NP - 1) / NP;

  // element offsets of token t of the sequence, head h
  auto rowk = [&](int t) -> int64_t { return (tok0 + t) * H + h; };
  auto rec_of = [&](int ep, int j) -> char* { return smem + ((ep & 1) * NP + j) * C::REC; };

  if (wave == 0) {
    // ------------------------------------------------------------ chain wave
    f32x4 Hacc[NT];
    const int64_t sbase = ((int64_t)b * H + h) * DK * DV;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Hacc[t][i] = h0 ? h0[sbase + (int64_t)(16 * t + 4 * grp + i) * DV + v0 + n] : 0.f;
    }
    F32 Hb[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) Hb[s] = X::from_acc2(Hacc[2 * s], Hacc[2 * s + 1]);
    // this lane's output element of token 4*grp in the sequence; tokens are
    // ostride elements apart
    const int64_t ostride = (int64_t)H * DV;
    E* const orow = o + rowk(4 * grp) * DV + v0 + n;
    __syncthreads();  // epoch 0 prepared

    for (int ep = 0; ep < NE; ++ep) {
      for (int j = 0; j < NP; ++j) {
        const int c = ep * NP + j;
        if (c >= NC) break;
        const char* rec = rec_of(ep, j);
        f32x4 R = zero4(), QH = zero4();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const F32 kf = reinterpret_cast<const F32*>(rec + C::KF)[s * 64 + lane];
          const F32 qf = reinterpret_cast<const F32*>(rec + C::QF)[s * 64 + lane];
          R = X::mma32(kf, Hb[s], R);
          QH = X::mma32(qf, Hb[s], QH);
        }
        const f32x4 gam = reinterpret_cast<const f32x4*>(rec + C::GM)[grp];
        const f32x4 del = reinterpret_cast<const f32x4*>(rec + C::DL)[grp];
        const float gC = *reinterpret_cast<const float*>(rec + C::GC);
        const F16 vf = reinterpret_cast<const F16*>(rec + C::VF)[lane];
        const F16 tb = *reinterpret_cast<const F16*>(rec + C::TB + (n * 16 + 4 * grp) * C::EB);
        const F16 pf = reinterpret_cast<const F16*>(rec + C::PF)[lane];
        f32x4 Y;
#pragma unroll
        for (int i = 0; i < 4; ++i) Y[i] = X::to_f(vf.v[i]) - gam[i] * R[i];
        const f32x4 U = X::mma16(tb, X::from_acc(Y), zero4());
        f32x4 O;
#pragma unroll
        for (int i = 0; i < 4; ++i) O[i] = gam[i] * QH[i];
        O = X::mma16(pf, X::from_acc(U), O);
        E* oc = orow + (int64_t)(16 * c) * ostride;
        if (16 * c + 16 <= T) {
#pragma unroll
          for (int i = 0; i < 4; ++i) oc[i * ostride] = X::from_f(O[i]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * c + 4 * grp + i < T) oc[i * ostride] = X::from_f(O[i]);
        }
        f32x4 Up;
#pragma unroll
        for (int i = 0; i < 4; ++i) Up[i] = del[i] * U[i];
        const F16 upb = X::from_acc(Up);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const F16 kt = reinterpret_cast<const F16*>(rec + C::KT)[t * 64 + lane];
          Hacc[t] = Hacc[t] * gC;
          Hacc[t] = X::mma16(kt, upb, Hacc[t]);
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) Hb[s] = X::from_acc2(Hacc[2 * s], Hacc[2 * s + 1]);
      }
      __syncthreads();  // this epoch consumed, next epoch prepared
    }
    if (hT) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          hT[sbase + (int64_t)(16 * t + 4 * grp + i) * DV + v0 + n] = Hacc[t][i];
      }
    }
    return;
  }

  // -------------------------------------------------------------- producers
  const int p = wave - 1;
  char* scr = smem + 2 * NP * C::REC + p * C::SCR;
  float* sA = reinterpret_cast<float*>(scr + C::SA);
  float* sB = reinterpret_cast<float*>(scr + C::SB);

  // Issue the global loads of tile c into r.  Rows past the end are read from
  // the last valid row (always in bounds) and zeroed later in produce(), so no
  // loaded value is consumed here and the loads stay in flight for an epoch.
  // Loads are issued unconditionally (tile index clamped to the last tile) so
  // the number of loads in flight is the same on every path and the compiler
  // can wait for exactly the older set.
  auto load = [&](Raw<E, DK>& r, int c) {
    if (NC == 0) return;          // an empty sequence loads nothing
    c = min(c, NC - 1);
    const int t = min(16 * c + n, T - 1);
    const int64_t base = rowk(t) * DK;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if constexpr (sizeof(E) == 2) {
        const bf16x4 k0 = *reinterpret_cast<const bf16x4*>(k + base + 32 * s + 4 * grp);
        const bf16x4 k1 = *reinterpret_cast<const bf16x4*>(k + base + 32 * s + 16 + 4 * grp);
        const bf16x4 q0 = *reinterpret_cast<const bf16x4*>(q + base + 32 * s + 4 * grp);
        const bf16x4 q1 = *reinterpret_cast<const bf16x4*>(q + base + 32 * s + 16 + 4 * grp);
        r.kf[s].v = bf16x8{k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
        r.qf[s].v = bf16x8{q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
      } else {
        r.kf[s].lo = *reinterpret_cast<const f32x4*>(k + base + 32 * s + 4 * grp);
        r.kf[s].hi = *reinterpret_cast<const f32x4*>(k + base + 32 * s + 16 + 4 * grp);
        r.qf[s].lo = *reinterpret_cast<const f32x4*>(q + base + 32 * s + 4 * grp);
        r.qf[s].hi = *reinterpret_cast<const f32x4*>(q + base + 32 * s + 16 + 4 * grp);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r.vv[i] = v[rowk(min(16 * c + 4 * grp + i, T - 1)) * DV + v0 + n];
    r.gx = gate[rowk(t)];
    r.bt = beta[rowk(t)];
  };

  auto produce = [&](const Raw<E, DK>& r, int c) {
    if (c >= NC) return;
    char* rec = rec_of(c / NP, c % NP);
    // padding tokens past T: q = k = v = 0, g = 0, beta = 0 (an identity step)
    const bool ok = 16 * c + n < T;
    const float g = ok ? (gate_logit ? bounded_gate(fmaf(gsc_h, r.gx, gbi_h), G) : r.gx) : 0.f;
    // raw inputs: beta from its logit
    const float bt = ok ? (raw ? sigmoid_f(r.bt) : r.bt) : 0.f;
    F32 kf[NS], qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      kf[s] = r.kf[s];
      qf[s] = r.qf[s];
      if (!ok) {
        kf[s] = F32{};
        qf[s] = F32{};
      }
    }
    if (raw) {
      // raw inputs: q and k L2-normalised per token (a zero vector stays
      // zero); lanes (n, grp = 0..3) together hold all d_k channels of token n
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sk += kf[s].lo[i] * kf[s].lo[i] + kf[s].hi[i] * kf[s].hi[i];
          sq += qf[s].lo[i] * qf[s].lo[i] + qf[s].hi[i] * qf[s].hi[i];
        }
      }
      sk += __shfl_xor(sk, 16);
      sk += __shfl_xor(sk, 32);
      sq += __shfl_xor(sq, 16);
      sq += __shfl_xor(sq, 32);
      const float ik = sk > 0.f ? 1.f / sqrtf(sk) : 0.f;
      const float iq = sq > 0.f ? 1.f / sqrtf(sq) : 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        kf[s].lo *= ik;
        kf[s].hi *= ik;
        qf[s].lo *= iq;
        qf[s].hi *= iq;
      }
    }
    const float Gi = scan16(g, n);              // G_n, inclusive
    const float Gtot = __shfl(Gi, 15, 16);      // G_15 (padding adds 0)
    if (grp == 0) {
      reinterpret_cast<float*>(rec + C::GM)[n] = __expf(Gi);
      reinterpret_cast<float*>(rec + C::DL)[n] = __expf(Gtot - Gi);
      if (n == 0) *reinterpret_cast<float*>(rec + C::GC) = __expf(Gtot);
      sB[n] = bt;
    }
    float Gr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) Gr[i] = __shfl(Gi, 4 * grp + i);

    // K K^T and K Q^T: lane (n, grp) reg i holds row (4grp+i) column n, which
    // by symmetry / by construction is entry [n][4grp+i] of K K^T / of Q K^T.
    f32x4 skk = zero4(), sqk = zero4();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      skk = X::mma32(kf[s], kf[s], skk);
      sqk = X::mma32(kf[s], qf[s], sqk);
    }
    f32x4 arow, prow;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s_ = 4 * grp + i;
      const float d = __expf(fminf(Gi - Gr[i], 0.f));   // exp(G_n - G_s), s <= n
      arow[i] = s_ < n ? bt * d * skk[i] : 0.f;
      prow[i] = s_ <= n ? d * sqk[i] : 0.f;
    }
    reinterpret_cast<f32x4*>(sA)[n * 4 + grp] = arow;          // A[n][4grp..4grp+3]
    reinterpret_cast<F16*>(rec + C::PF)[lane] = X::from_acc(prow);

    // K^T fragments: (K restricted to 16 columns) x I puts K[4grp+i][16t+n] in
    // lane (n, grp) reg i -- the A fragment of K^T for state tile t.
    f32x4 idv;
#pragma unroll
    for (int j = 0; j < 4; ++j) idv[j] = (4 * grp + j == n) ? 1.f : 0.f;
    const F16 ident = X::from_acc(idv);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const f32x4 kt = X::mma16(X::half(kf[t >> 1], t & 1), ident, zero4());
      reinterpret_cast<F16*>(rec + C::KT)[t * 64 + lane] = X::from_acc(kt);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      reinterpret_cast<F32*>(rec + C::KF)[s * 64 + lane] = kf[s];
      reinterpret_cast<F32*>(rec + C::QF)[s * 64 + lane] = qf[s];
    }
    F16 vf;
#pragma unroll
    for (int i = 0; i < 4; ++i) vf.v[i] = (16 * c + 4 * grp + i < T) ? r.vv[i] : X::from_f(0.f);
    reinterpret_cast<F16*>(rec + C::VF)[lane] = vf;

    // LDS traffic of one wave is performed in order; the wave barrier keeps the
    // compiler from moving the reads of A / beta above the writes.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // T = (I + A)^-1, row n per lane: from T (I + A) = I,
    //   T[n][s] = delta_ns - sum_{r > s} T[n][r] A[r][s];
    // once x[r] is final (all rows above r done), subtract its contribution.
    float x[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) x[s] = (s == n) ? 1.f : 0.f;
#pragma unroll
    for (int rr = 15; rr >= 1; --rr) {
      float arr[16];
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const f32x4 a4 = reinterpret_cast<const f32x4*>(sA)[rr * 4 + c4];
        arr[4 * c4 + 0] = a4[0]; arr[4 * c4 + 1] = a4[1];
        arr[4 * c4 + 2] = a4[2]; arr[4 * c4 + 3] = a4[3];
      }
      const float xr = x[rr];
#pragma unroll
      for (int s = 0; s < rr; ++s) x[s] -= xr * arr[s];
    }
    if (grp == 0) {
      E row[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) row[s] = X::from_f(x[s] * sB[s]);
#pragma unroll
      for (int s = 0; s < 16; s += 4) {
        F16 f;
        f.v[0] = row[s]; f.v[1] = row[s + 1]; f.v[2] = row[s + 2]; f.v[3] = row[s + 3];
        *reinterpret_cast<F16*>(rec + C::TB + (n * 16 + s) * C::EB) = f;
      }
    }
    // the next tile's writes to A / beta must not pass this tile's reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // Two register sets, alternating by epoch: while tile (ep+1)*NP + p is
  // prepared from one set, the loads for tile (ep+2)*NP + p fill the other.
  // The loop is unrolled by two so each set keeps its own registers.
  Raw<E, DK> ra, rb;
  load(ra, p);
  produce(ra, p);               // epoch 0
  load(ra, NP + p);             // epoch 1, prepared during epoch 0
  __syncthreads();
  for (int ep = 0; ep < NE; ep += 2) {
    load(rb, (ep + 2) * NP + p);
    produce(ra, (ep + 1) * NP + p);
    __syncthreads();
    if (ep + 1 < NE) {
      load(ra, (ep + 3) * NP + p);
      produce(rb, (ep + 2) * NP + p);
      __syncthreads();
    }
  }
}

// B sequences of T tokens (cu == NULL), or B packed sequences with device
// offsets cu in one sequence of T tokens.
template <typename E, int DK, int NP>
static hipError_t launch_t(const void* q, const void* k, const void* v, const float* gate,
                           int gate_logit, float G, const float* beta, const float* h0,
                           void* o, float* hT, int B, int T, int H, int Dv, const int* cu,
                           int raw, hipStream_t st, const float* gsc, const float* gbi) {
  const int blocks = B * H * (Dv / 16);
  hipLaunchKernelGGL((chunk_fwd_kernel<E, DK, NP>), dim3(blocks), dim3(64 * (NP + 1)), 0, st,
                     (const E*)q, (const E*)k, (const E*)v, gate, gate_logit, G, beta, h0,
                     (E*)o, hT, B, T, H, Dv, cu, raw, gsc, gbi);
  return hipGetLastError();
}

hipError_t launch_chunk_fwd(const void* q, const void* k, const void* v, const float* gate,
                            int gate_logit, float G, const float* beta, const float* h0,
                            void* o, float* hT, int B, int T, int H, int Dk, int Dv, int raw,
                            hipStream_t st, const float* gsc, const float* gbi) {
  return launch_chunk_fwd_varlen(q, k, v, gate, gate_logit, G, beta, h0, o, hT, nullptr, B, T, H,
                                 Dk, Dv, raw, st, gsc, gbi);
}

hipError_t launch_chunk_fwd_varlen(const void* q, const void* k, const void* v,
                                   const float* gate, int gate_logit, float G,
                                   const float* beta, const float* h0, void* o, float* hT,
                                   const int* cu, int B, int T, int H, int Dk, int Dv, int raw,
                                   hipStream_t st, const float* gsc, const float* gbi) {
  if (Dk == 64)
    return launch_t<float, 64, 2>(q, k, v, gate, gate_logit, G, beta, h0, o, hT, B, T, H, Dv, cu,
                                  raw, st, gsc, gbi);
  if (Dk == 128)
    return launch_t<float, 128, 2>(q, k, v, gate, gate_logit, G, beta, h0, o, hT, B, T, H, Dv, cu,
                                   raw, st, gsc, gbi);
  return hipErrorInvalidValue;
}

}  // namespace la
