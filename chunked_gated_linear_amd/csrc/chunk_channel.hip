// chunk_channel.hip -- chunked forward pass with a per-channel bounded gate:
// one log-decay per key channel, g_t in [-G, 0]^{d_k}.
//
// Recurrence (h = S^T, d_k x d_v; D_t = diag(exp(g_t)) acts on the key side of
// the old state, then the delta-rule erase and write act on the decayed state):
//     d_t = D_t h_{t-1},  h_t = d_t - beta_t k_t (k_t^T d_t) + beta_t k_t v_t^T,
//     o_t = h_t^T q_t.
// With one decay per channel the cumulative decay no longer factors out of the
// token dot products, so inside a 16-token tile it has to enter the matrix-core
// operands, and the reciprocal of the cumulative decay appears.  The pages
// bound the log-decay so that this reciprocal stays finite in a 16-token tile
// ("Core Technologies Behind Ultra-Long-Context Sparse MoE Large Models",
// sec. 2.1 and 2.3; "How Trillion-Scale Sparse MoE Models Achieve Million-Token
// Long Context", sec. 3.1 and 3.2: at most exp(16 G) = exp(80)).
//
// Algebra of one tile (derived from the recurrence).  H is the state entering
// the tile, G_t[c] the in-tile running sum of g over tokens (a vector over
// channels), Gam_t = exp(G_t), Gam_C = Gam_15.  With u_t = beta_t (v_t - d_t^T k_t):
//     A[t][s] = beta_t (k_t o Gam_t) . (k_s / Gam_s)         (s < t)
//     P[t][s] = (q_t o Gam_t) . (k_s / Gam_s)                (s <= t)
//     U  = (I + A)^-1 diag(beta) (V - (K o Gam) H)
//     O  = (Q o Gam) H + P U
//     H' = diag(Gam_C) H + (K o (Gam_C / Gam))^T U
// The state-facing operands K o Gam, Q o Gam and K o Gam_C/Gam are at most 1
// in size.  For A and P the factors are taken relative to the tile's middle
// token m = 7 instead of its start: (k_t o exp(G_t - G_m)) . (k_s o exp(G_m - G_s))
// is the same number, and every operand then stays within exp(+-8 G) (exp(+-40)
// at G = 5) instead of reaching exp(80), so no product comes near the float
// overflow or the subnormal range.
//
// Arithmetic is fp32 throughout (inputs in bf16 convert exactly); the matrix
// products run on the fp32 MFMA (16x16x4).  Work split as in the fp32 scalar
// path: one workgroup per (b, h, 16-column slice of d_v); wave 0 ("chain")
// owns the fp32 state slice in registers and runs the serial part, waves
// 1..NP ("producers") prepare upcoming tiles -- loads, the gate, the
// per-channel in-tile running sums, the scaled operands, A and P on MFMA, the
// 16 x 16 solve -- and hand them over through LDS, double-buffered by epochs
// of NP tiles.
#include "la_device.h"
#include "la_launch.h"

namespace la {
namespace {

template <int DK, int NP>
struct ChCfg {
  static constexpr int NT = DK / 16;   // 16-row tiles of the state slice
  static constexpr int NS = DK / 32;   // 32-deep contraction blocks
  // One prepared tile in LDS (fp32), every field lane-contiguous.
  static constexpr int KF = 0;                       // K o Gam:  NS x 64 lanes x 8
  static constexpr int QF = KF + NS * 64 * 8 * 4;    // Q o Gam:  NS x 64 x 8
  static constexpr int KT = QF + NS * 64 * 8 * 4;    // (K o Gam_C/Gam)^T: NT x 64 x 4
  static constexpr int VF = KT + NT * 64 * 4 * 4;    // V slice: 64 x 4
  static constexpr int PF = VF + 64 * 4 * 4;         // P: 64 x 4
  static constexpr int TB = PF + 64 * 4 * 4;         // (I + A)^-1 diag(beta), 16 x 16
  static constexpr int GC = TB + 256 * 4;            // Gam_C[DK]
  static constexpr int REC = GC + DK * 4;
  // Producer scratch: A (16 x 16) and beta[16].
  static constexpr int SA = 0;
  static constexpr int SB = 1024;
  static constexpr int SCR = 1024 + 64;
  static constexpr int LDS = 2 * NP * REC + NP * SCR;
  static_assert(REC % 16 == 0 && SCR % 16 == 0, "LDS alignment");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Flat block index -> (head, d_v slice), the NV slices of a head on one XCD
// (workgroups are dealt to the 8 XCDs round robin).
__device__ inline void ch_map_block(int n, int NH, int NV, int& head, int& vt) {
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

// Producer registers for one tile: the lane's 8 * NS channels of its token's
// k and q (in the input type), the same channels of the gate, four v values.
template <typename E, int DK>
struct ChRaw {
  typename Elt<E>::F32 kf[DK / 32];
  typename Elt<E>::F32 qf[DK / 32];
  f32x4 glo[DK / 32], ghi[DK / 32];
  E vv[4];
  float bt;
};

// 8 elements of a 32-deep fragment as fp32 (lo = j 0..3, hi = j 4..7).
__device__ inline Elt<float>::F32 to_f32(const Elt<float>::F32& a) { return a; }
__device__ inline Elt<float>::F32 to_f32(const Elt<__bf16>::F32& a) {
  Elt<float>::F32 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r.lo[j] = (float)a.v[j];
    r.hi[j] = (float)a.v[4 + j];
  }
  return r;
}

template <typename E, int DK, int NP>
__global__ __launch_bounds__(64 * (NP + 1)) void chunk_fwd_channel_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ gate, int gate_logit, float G,
    const float* __restrict__ beta, const float* h0, E* __restrict__ o, float* hT,
    int B, int T, int H, int DV) {
  using C = ChCfg<DK, NP>;
  using X = Elt<float>;
  using F16 = X::F16;
  using F32 = X::F32;
  constexpr int NT = C::NT, NS = C::NS;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  const int NV = DV / 16;
  int head, vt;
  ch_map_block(blockIdx.x, B * H, NV, head, vt);
  const int b = head / H, h = head % H;
  const int v0 = vt * 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, grp = lane >> 4;
  const int NC = (T + 15) >> 4;
  const int NE = (NC + NP - 1) / NP;

  auto rowk = [&](int t) -> int64_t { return ((int64_t)b * T + t) * H + h; };
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
    const int64_t ostride = (int64_t)H * DV;
    E* const orow = o + rowk(4 * grp) * DV + v0 + n;
    __syncthreads();  // epoch 0 prepared
    for (int ep = 0; ep < NE; ++ep) {
      for (int j = 0; j < NP; ++j) {
        const int c = ep * NP + j;
        if (c >= NC) break;
        const char* rec = rec_of(ep, j);
        // R = (K o Gam) H and (Q o Gam) H, contraction over d_k
        f32x4 R = zero4(), QH = zero4();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const F32 hb = X::from_acc2(Hacc[2 * s], Hacc[2 * s + 1]);
          const F32 kf = reinterpret_cast<const F32*>(rec + C::KF)[s * 64 + lane];
          const F32 qf = reinterpret_cast<const F32*>(rec + C::QF)[s * 64 + lane];
          R = X::mma32(kf, hb, R);
          QH = X::mma32(qf, hb, QH);
        }
        const F16 vf = reinterpret_cast<const F16*>(rec + C::VF)[lane];
        const F16 tb = *reinterpret_cast<const F16*>(rec + C::TB + (n * 16 + 4 * grp) * 4);
        const F16 pf = reinterpret_cast<const F16*>(rec + C::PF)[lane];
        f32x4 Y;
#pragma unroll
        for (int i = 0; i < 4; ++i) Y[i] = vf.v[i] - R[i];
        const f32x4 U = X::mma16(tb, X::from_acc(Y), zero4());
        const f32x4 O = X::mma16(pf, X::from_acc(U), QH);
        E* oc = orow + (int64_t)(16 * c) * ostride;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * c + 4 * grp + i < T) oc[i * ostride] = Elt<E>::from_f(O[i]);
        const F16 ub = X::from_acc(U);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const f32x4 gc = reinterpret_cast<const f32x4*>(rec + C::GC)[4 * t + grp];
          const F16 kt = reinterpret_cast<const F16*>(rec + C::KT)[t * 64 + lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) Hacc[t][i] *= gc[i];   // row 16t + 4grp + i
          Hacc[t] = X::mma16(kt, ub, Hacc[t]);
        }
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

  // Global loads of tile c (index clamped to the last tile, rows past the end
  // read from the last valid row and zeroed in produce()), issued one epoch
  // before the tile is prepared.
  auto load = [&](ChRaw<E, DK>& r, int c) {
    c = min(c, NC - 1);
    const int t = min(16 * c + n, T - 1);
    const int64_t base = rowk(t) * DK;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c0 = 32 * s + 4 * grp, c1 = c0 + 16;
      if constexpr (sizeof(E) == 2) {
        const bf16x4 k0 = *reinterpret_cast<const bf16x4*>(k + base + c0);
        const bf16x4 k1 = *reinterpret_cast<const bf16x4*>(k + base + c1);
        const bf16x4 q0 = *reinterpret_cast<const bf16x4*>(q + base + c0);
        const bf16x4 q1 = *reinterpret_cast<const bf16x4*>(q + base + c1);
        r.kf[s].v = bf16x8{k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
        r.qf[s].v = bf16x8{q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
      } else {
        r.kf[s].lo = *reinterpret_cast<const f32x4*>(k + base + c0);
        r.kf[s].hi = *reinterpret_cast<const f32x4*>(k + base + c1);
        r.qf[s].lo = *reinterpret_cast<const f32x4*>(q + base + c0);
        r.qf[s].hi = *reinterpret_cast<const f32x4*>(q + base + c1);
      }
      r.glo[s] = *reinterpret_cast<const f32x4*>(gate + base + c0);
      r.ghi[s] = *reinterpret_cast<const f32x4*>(gate + base + c1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r.vv[i] = v[rowk(min(16 * c + 4 * grp + i, T - 1)) * DV + v0 + n];
    r.bt = beta[rowk(t)];
  };

  auto produce = [&](const ChRaw<E, DK>& r, int c) {
    if (c >= NC) return;
    char* rec = rec_of(c / NP, c % NP);
    // padding tokens past T: q = k = v = 0, g = 0, beta = 0 (an identity step)
    const bool ok = 16 * c + n < T;
    const float bt = ok ? r.bt : 0.f;
    // per lane: 8 channels per 32-deep block s (j < 4: 32s + 4grp + j,
    // j >= 4: 32s + 16 + 4grp + j - 4), token t = n
    float vkg[NS][8], vqg[NS][8], vkd[NS][8], vkm[NS][8], vqm[NS][8], vki[NS][8];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const F32 k32 = to_f32(r.kf[s]), q32 = to_f32(r.qf[s]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = j < 4 ? r.glo[s][j] : r.ghi[s][j - 4];
        const float g = ok ? (gate_logit ? bounded_gate(x, G) : x) : 0.f;
        const float Gt = scan16(g, n);                  // G_t[c], t = n
        const float Gm = __shfl(Gt, 7, 16);             // G at the middle token
        const float Gl = __shfl(Gt, 15, 16);            // G at the last token
        const float kv = ok ? (j < 4 ? k32.lo[j] : k32.hi[j - 4]) : 0.f;
        const float qv = ok ? (j < 4 ? q32.lo[j] : q32.hi[j - 4]) : 0.f;
        const float e_start = __expf(Gt);               // Gam_t            (<= 1)
        const float e_end = __expf(Gl - Gt);            // Gam_C / Gam_t    (<= 1)
        const float e_mid = __expf(Gt - Gm);            // Gam_t / Gam_m
        const float e_imid = __expf(Gm - Gt);           // Gam_m / Gam_t
        vkg[s][j] = kv * e_start;
        vqg[s][j] = qv * e_start;
        vkd[s][j] = kv * e_end;
        vkm[s][j] = kv * e_mid;
        vqm[s][j] = qv * e_mid;
        vki[s][j] = kv * e_imid;
        if (n == 0) {   // Gam_C of this channel
          const int ch = 32 * s + (j < 4 ? 4 * grp + j : 16 + 4 * grp + j - 4);
          reinterpret_cast<float*>(rec + C::GC)[ch] = __expf(Gl);
        }
      }
    }
    auto pack = [](const float (&a)[8]) {
      F32 f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f.lo[j] = a[j];
        f.hi[j] = a[4 + j];
      }
      return f;
    };
    F32 kg[NS], qg[NS], kd[NS], km[NS], qm[NS], ki[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      kg[s] = pack(vkg[s]);
      qg[s] = pack(vqg[s]);
      kd[s] = pack(vkd[s]);
      km[s] = pack(vkm[s]);
      qm[s] = pack(vqm[s]);
      ki[s] = pack(vki[s]);
    }
    if (grp == 0) sB[n] = bt;

    // A and P: lane (n, grp) register i gets entry [4grp+i][n] of
    // (K / Gam_m-scaled) x (K or Q scaled), i.e. row n, column s = 4grp+i of
    // A (before beta) and of P.
    f32x4 sa = zero4(), sp = zero4();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      sa = X::mma32(ki[s], km[s], sa);
      sp = X::mma32(ki[s], qm[s], sp);
    }
    f32x4 arow, prow;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s_ = 4 * grp + i;
      arow[i] = s_ < n ? bt * sa[i] : 0.f;
      prow[i] = s_ <= n ? sp[i] : 0.f;
    }
    reinterpret_cast<f32x4*>(sA)[n * 4 + grp] = arow;          // A[n][4grp..4grp+3]
    reinterpret_cast<F16*>(rec + C::PF)[lane] = X::from_acc(prow);

    // (K o Gam_C/Gam)^T fragments: the 16-column block t of that matrix times
    // the identity puts entry [4grp+i][16t+n] in lane (n, grp) register i.
    f32x4 idv;
#pragma unroll
    for (int j = 0; j < 4; ++j) idv[j] = (4 * grp + j == n) ? 1.f : 0.f;
    const F16 ident = X::from_acc(idv);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const f32x4 kt = X::mma16(X::half(kd[t >> 1], t & 1), ident, zero4());
      reinterpret_cast<F16*>(rec + C::KT)[t * 64 + lane] = X::from_acc(kt);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      reinterpret_cast<F32*>(rec + C::KF)[s * 64 + lane] = kg[s];
      reinterpret_cast<F32*>(rec + C::QF)[s * 64 + lane] = qg[s];
    }
    F16 vf;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vf.v[i] = (16 * c + 4 * grp + i < T) ? Elt<E>::to_f(r.vv[i]) : 0.f;
    reinterpret_cast<F16*>(rec + C::VF)[lane] = vf;

    // this wave's LDS writes (A, beta) before its reads of them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // (I + A)^-1, row n per lane: T[n][s] = delta_ns - sum_{r > s} T[n][r] A[r][s],
    // eliminating from the bottom row up.
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
#pragma unroll
      for (int s = 0; s < 16; s += 4) {
        const f32x4 row{x[s] * sB[s], x[s + 1] * sB[s + 1], x[s + 2] * sB[s + 2],
                        x[s + 3] * sB[s + 3]};
        *reinterpret_cast<f32x4*>(rec + C::TB + (n * 16 + s) * 4) = row;
      }
    }
    // the next tile's writes to A / beta must not pass this tile's reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // Two register sets alternating by epoch: while tile (ep+1)*NP + p is
  // prepared from one, the loads for tile (ep+2)*NP + p fill the other.
  ChRaw<E, DK> ra, rb;
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

template <typename E, int DK, int NP>
hipError_t launch_ch(const void* q, const void* k, const void* v, const float* gate,
                     int gate_logit, float G, const float* beta, const float* h0, void* o,
                     float* hT, int B, int T, int H, int Dv, hipStream_t st) {
  const int blocks = B * H * (Dv / 16);
  hipLaunchKernelGGL((chunk_fwd_channel_kernel<E, DK, NP>), dim3(blocks), dim3(64 * (NP + 1)),
                     0, st, (const E*)q, (const E*)k, (const E*)v, gate, gate_logit, G, beta,
                     h0, (E*)o, hT, B, T, H, Dv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_fwd_channel(const void* q, const void* k, const void* v,
                                    const float* gate, int gate_logit, float G,
                                    const float* beta, const float* h0, void* o, float* hT,
                                    int B, int T, int H, int Dk, int Dv, int fp32,
                                    hipStream_t st) {
  if (fp32) {
    if (Dk == 64) return launch_ch<float, 64, 2>(q, k, v, gate, gate_logit, G, beta, h0, o, hT, B, T, H, Dv, st);
    if (Dk == 128) return launch_ch<float, 128, 2>(q, k, v, gate, gate_logit, G, beta, h0, o, hT, B, T, H, Dv, st);
  } else {
    if (Dk == 64) return launch_ch<__bf16, 64, 2>(q, k, v, gate, gate_logit, G, beta, h0, o, hT, B, T, H, Dv, st);
    if (Dk == 128) return launch_ch<__bf16, 128, 2>(q, k, v, gate, gate_logit, G, beta, h0, o, hT, B, T, H, Dv, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace la
