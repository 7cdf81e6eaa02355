// chunk_fwd2.hip -- bf16 chunked forward pass, two 16-token tiles per step of
// the state recurrence.
//
// Same method and algebra as chunk_fwd.hip (16-token tiles whose diagonal and
// "historical state -> current token" blocks are matrix-core products; "Deep
// Dive: The Next Generation of Ultra-Long Context Sparse MoE LLMs", sec. 3.2;
// "Core Technologies Behind Ultra-Long-Context Sparse MoE Large Models", sec.
// 2.1), but the state H is carried across pairs of tiles (32 tokens, tiles a
// and b).  With G the running sum of g over the pair, gamma = exp(G),
// delta_p = exp(G_31 - G_p), Gamma = exp(G_31):
//     A   = [[A00, 0], [A10, A11]],  A[t][s] = beta_t exp(G_t - G_s) k_t.k_s (s < t)
//     T   = (I + A)^-1 = [[T00, 0], [T10, T11]],  T10 = -T11 A10 T00
//     Tb  = T diag(beta),  P[t][s] = exp(G_t - G_s) q_t.k_s (s <= t)
//     U   = Tb (V - diag(gamma) K H)
//     O   = diag(gamma) Q H + P U
//     H'  = Gamma H + K^T diag(delta) U
// T00 and T11 are solved in fp32 by forward substitution, T10 with fp32 MFMA;
// only exponentials of non-positive numbers appear.  Carrying H per pair of
// tiles halves the per-token cost of rescaling and converting the state, and
// the state update becomes a full 32-deep MFMA.
//
// Precision: the small in-tile operands Tb, P and U are split into bf16 hi + lo
// parts, contracted as [X_hi | X_lo] . [Y ; Y] in one 32-deep MFMA (the same
// issue cost as a 16-deep product).
//
// Work split: one workgroup of 6 waves per (b, h, 16 columns of d_v):
//   wave 0  "chain"     the fp32 state slice in registers; per pair: K H, U,
//                       the state update (19 MFMAs), then hands H (bf16) and U
//                       to the output wave through LDS;
//   wave 1  "output"    Q H and P U on MFMA and the bf16 output stores; it
//                       reads q straight from global memory (one epoch ahead)
//                       and follows the chain pair by pair through an LDS flag;
//   waves 2-5 "producers" each prepare one pair per epoch (4 pairs = 128 tokens)
//                       into an LDS record, double buffered by epoch: loads,
//                       gate, in-pair cumulative sum, K K^T and K Q^T on MFMA,
//                       decay masks, the triangular solves, hi/lo splits.
// One workgroup barrier per epoch.  K^T for the state update is read straight
// from the K fragments with the gfx950 transposing LDS read.
//
// State row order.  Accumulator tile t = 2s + h of the state holds, in lane
// (n, grp) register i, row rho = 32 s + 8 grp + 4 h + i of the d_k x 16 slice.
// With that order every 32-deep fragment of K or Q is 8 consecutive elements
// of a row (one 16-byte load) and two accumulator tiles are directly the
// 32-deep B fragment of H.
#include "la_device.h"
#include "la_launch.h"

namespace la {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

template <int DK>
struct Cfg2 {
  static constexpr int NP = 4;                 // producers = pairs per epoch
  static constexpr int NW = NP + 2;            // waves per workgroup
  static constexpr int NT = DK / 16, NS = DK / 32;
  // record of one pair of tiles (byte offsets; every field lane-contiguous)
  static constexpr int KF = 0;                          // [2][NS][64] x 16 B (swizzled)
  static constexpr int VF = KF + 2 * NS * 64 * 16;      // [2][64] x 8 B
  static constexpr int TB0 = VF + 2 * 64 * 8;           // [64] x 16 B  [Tb00 hi | Tb00 lo]
  static constexpr int TB1H = TB0 + 64 * 16;            //              [Tb10 hi | Tb11 hi]
  static constexpr int TB1L = TB1H + 64 * 16;           //              [Tb10 lo | Tb11 lo]
  static constexpr int PF0 = TB1L + 64 * 16;            //              [P00 hi  | P00 lo]
  static constexpr int PF1H = PF0 + 64 * 16;            //              [P10 hi  | P11 hi]
  static constexpr int PF1L = PF1H + 64 * 16;           //              [P10 lo  | P11 lo]
  static constexpr int GM = PF1L + 64 * 16;             // gamma[32]  f32
  static constexpr int DL = GM + 128;                   // delta[32]  f32
  static constexpr int GC = DL + 128;                   // Gamma      f32 (x4)
  static constexpr int REC = GC + 16;
  // chain -> output hand-over, one slot per pair of an epoch
  static constexpr int OB_H = 0;                        // [NS][64] x 16 B  H (bf16)
  static constexpr int OB_U = NS * 64 * 16;             // [2][64] x 16 B   U_a, U_b (f32)
  static constexpr int OB = OB_U + 2 * 64 * 16;
  // producer scratch: A00 (then T00), A11 (then T11), beta[32], G[32]
  static constexpr int SA0 = 0, SA1 = 1024, SB = 2048, SG = 2048 + 128;
  static constexpr int SCR = SG + 128;
  static constexpr int OFF_OB = 2 * NP * REC;
  static constexpr int OFF_SCR = OFF_OB + NP * OB;
  static constexpr int OFF_FLAG = OFF_SCR + NP * SCR;
  static constexpr int LDS = OFF_FLAG + 16 * NP;
  static_assert(REC % 16 == 0 && SCR % 16 == 0 && OB % 16 == 0, "LDS alignment");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// K fragment slot inside a tile's block: (s, grp, m) -> s*64 + grp*16 + (m ^ 4grp).
// The XOR keeps the transposing reads of the state update free of bank
// conflicts; ordinary fragment reads stay lane-contiguous.
__device__ inline int kslot(int s, int grp, int m) { return s * 64 + grp * 16 + (m ^ (4 * grp)); }

__device__ inline bf16x4 hi4(f32x4 x) {
  return bf16x4{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
}
__device__ inline bf16x4 lo4(f32x4 x, bf16x4 h) {
  return bf16x4{(__bf16)(x[0] - (float)h[0]), (__bf16)(x[1] - (float)h[1]),
                (__bf16)(x[2] - (float)h[2]), (__bf16)(x[3] - (float)h[3])};
}
__device__ inline bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ inline f32x4 mma32b(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Inclusive prefix sum over each row of 16 lanes with DPP row shifts (lanes
// shifted in from outside the row contribute 0).
__device__ inline float scan16_dpp(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, false));
  return x;
}

template <int DK>
struct Raw2 {      // producer registers for one pair of tiles (x = 0: tile a, 1: tile b)
  bf16x8 kf[2][DK / 32];
  bf16x8 qf[2][DK / 32];
  __bf16 vv[2][4];
  float gx[2], bt[2];
};

__device__ inline void map_block2(int n, int NH, int NV, int& head, int& vt) {
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

// Wave-local ordering of LDS traffic (a wave's LDS operations execute in
// order; this keeps the compiler from reordering across the point).
__device__ inline void wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bound on the output wave's wait for one pair (each poll sleeps ~64 cycles):
// far above any real wait, it only guarantees that the wave always exits.
constexpr int kSpinLimit = 1 << 22;

template <int DK>
__global__ __launch_bounds__(64 * Cfg2<DK>::NW) void chunk_fwd2_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const float* __restrict__ gate, int gate_logit, float G,
    const float* __restrict__ beta, const float* h0, __bf16* __restrict__ o, float* hT,
    int B, int T, int H, int DV) {
  using C = Cfg2<DK>;
  using F = Elt<float>;
  constexpr int NT = C::NT, NS = C::NS, NP = C::NP;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  const int NV = DV / 16;
  int head, vt;
  map_block2(blockIdx.x, B * H, NV, head, vt);
  const int b = head / H, h = head % H;
  const int v0 = vt * 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, grp = lane >> 4;
  const int NSC = (T + 31) >> 5;                 // pairs of tiles
  const int NE = (NSC + NP - 1) / NP;            // epochs

  auto rec_of = [&](int ep, int j) -> char* { return smem + ((ep & 1) * NP + j) * C::REC; };
  auto ob_of = [&](int j) -> char* { return smem + C::OFF_OB + j * C::OB; };
  int* const flags = reinterpret_cast<int*>(smem + C::OFF_FLAG);
  // Row offsets fit in 32 bits (checked on the host: T * H * max(Dk, Dv) < 2^31).
  const int64_t tok0 = (int64_t)b * T * H + h;   // token (b, 0, h)

  if (threadIdx.x < NP) flags[threadIdx.x * 4] = 0;

  if (wave == 0) {
    // ------------------------------------------------------------ chain wave
    f32x4 Hacc[NT];
    const int64_t sbase = ((int64_t)b * H + h) * DK * DV;
    auto srow = [&](int t, int i) { return 32 * (t >> 1) + 8 * grp + 4 * (t & 1) + i; };
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Hacc[t][i] = h0 ? h0[sbase + (int64_t)srow(t, i) * DV + v0 + n] : 0.f;
    bf16x8 Hb[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) Hb[s] = cat8(hi4(Hacc[2 * s]), hi4(Hacc[2 * s + 1]));
    // transposing-read lane offset: lane (j, grp) points at K[4 grp + j/4][rho chunk j%4]
    const int trl = ((n & 3) * 16 + ((4 * grp + (n >> 2)) ^ (4 * (n & 3)))) * 16;
    __syncthreads();  // epoch 0 prepared

    struct Ops { bf16x8 ka[NS], kb[NS]; f32x4 ga, gb, da, db; float Gam; bf16x4 va, vb;
                 bf16x8 tb0, tb1h, tb1l; };
    auto fetch = [&](const char* rec, Ops& x) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        x.ka[s] = reinterpret_cast<const bf16x8*>(rec + C::KF)[kslot(s, grp, n)];
        x.kb[s] = reinterpret_cast<const bf16x8*>(rec + C::KF + NS * 1024)[kslot(s, grp, n)];
      }
      x.ga = reinterpret_cast<const f32x4*>(rec + C::GM)[grp];
      x.gb = reinterpret_cast<const f32x4*>(rec + C::GM)[4 + grp];
      x.da = reinterpret_cast<const f32x4*>(rec + C::DL)[grp];
      x.db = reinterpret_cast<const f32x4*>(rec + C::DL)[4 + grp];
      x.Gam = *reinterpret_cast<const float*>(rec + C::GC);
      x.va = reinterpret_cast<const bf16x4*>(rec + C::VF)[lane];
      x.vb = reinterpret_cast<const bf16x4*>(rec + C::VF)[64 + lane];
      x.tb0 = reinterpret_cast<const bf16x8*>(rec + C::TB0)[lane];
      x.tb1h = reinterpret_cast<const bf16x8*>(rec + C::TB1H)[lane];
      x.tb1l = reinterpret_cast<const bf16x8*>(rec + C::TB1L)[lane];
    };

    for (int ep = 0; ep < NE; ++ep) {
      Ops cur;
      fetch(rec_of(ep, 0), cur);
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const int c = ep * NP + j;
        if (c >= NSC) break;
        char* rec = rec_of(ep, j);
        Ops nxt;
        if (j + 1 < NP) fetch(rec_of(ep, j + 1), nxt);   // one pair ahead
        // hand H (bf16) to the output wave before it changes
        char* ob = ob_of(j);
#pragma unroll
        for (int s = 0; s < NS; ++s) reinterpret_cast<bf16x8*>(ob + C::OB_H)[s * 64 + lane] = Hb[s];
        f32x4 Ra = zero4(), Rb = zero4();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          Ra = mma32b(cur.ka[s], Hb[s], Ra);
          Rb = mma32b(cur.kb[s], Hb[s], Rb);
        }
        f32x4 Ya, Yb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Ya[i] = (float)cur.va[i] - cur.ga[i] * Ra[i];
          Yb[i] = (float)cur.vb[i] - cur.gb[i] * Rb[i];
        }
        const bf16x4 ya = hi4(Ya), yb = hi4(Yb);
        // U_a = Tb00 Y_a ; U_b = Tb10 Y_a + Tb11 Y_b   (Tb in hi + lo parts)
        const f32x4 Ua = mma32b(cur.tb0, cat8(ya, ya), zero4());
        f32x4 Ub = mma32b(cur.tb1h, cat8(ya, yb), zero4());
        Ub = mma32b(cur.tb1l, cat8(ya, yb), Ub);
        reinterpret_cast<f32x4*>(ob + C::OB_U)[lane] = Ua;
        reinterpret_cast<f32x4*>(ob + C::OB_U)[64 + lane] = Ub;
        // publish the pair to the output wave
        __hip_atomic_store(&flags[j * 4], c + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        // H' = Gamma H + K^T diag(delta) U, 32-deep over both tiles
        f32x4 Upa, Upb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Upa[i] = cur.da[i] * Ua[i];
          Upb[i] = cur.db[i] * Ub[i];
        }
        const bf16x8 up = cat8(hi4(Upa), hi4(Upb));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int off = (t >> 1) * 1024 + trl + 8 * (t & 1);
          const s16x4_t ta = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(smem + (rec - smem) + C::KF + off));
          const s16x4_t tb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(smem + (rec - smem) + C::KF + NS * 1024 + off));
          const bf16x8 kt = cat8(__builtin_bit_cast(bf16x4, ta), __builtin_bit_cast(bf16x4, tb));
          Hacc[t] = Hacc[t] * cur.Gam;
          Hacc[t] = mma32b(kt, up, Hacc[t]);
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) Hb[s] = cat8(hi4(Hacc[2 * s]), hi4(Hacc[2 * s + 1]));
        if (j + 1 < NP) cur = nxt;
      }
      __syncthreads();  // this epoch consumed (chain and output), next epoch prepared
    }
    if (hT) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          hT[sbase + (int64_t)srow(t, i) * DV + v0 + n] = Hacc[t][i];
    }
    return;
  }

  if (wave == 1) {
    // ----------------------------------------------------------- output wave
    // q fragments are read straight from global memory (the producers touched
    // the same lines an epoch earlier), one pair ahead, two register sets.
    const __bf16* const qb0 = q + tok0 * DK + 8 * grp;
    __bf16* const orow = o + (tok0 + (int64_t)(4 * grp) * H) * DV + v0 + n;
    const int ostride = H * DV;
    bf16x8 qs[2][2][NS];
    auto loadq = [&](bf16x8 (&qq)[2][NS], int c) {
      c = min(c, NSC - 1);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int t = min(32 * c + 16 * x + n, T - 1);
#pragma unroll
        for (int s = 0; s < NS; ++s)
          qq[x][s] = *reinterpret_cast<const bf16x8*>(qb0 + t * H * DK + 32 * s);
      }
    };
    auto pair = [&](const bf16x8 (&qq)[2][NS], int ep, int j) {
      const int c = ep * NP + j;
      const char* rec = rec_of(ep, j);
      const char* ob = ob_of(j);
      for (int spin = 0; spin < kSpinLimit; ++spin) {
        if (__hip_atomic_load(&flags[j * 4], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == c + 1)
          break;
        __builtin_amdgcn_s_sleep(1);
      }
      f32x4 Qa = zero4(), Qb = zero4();
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 hb = reinterpret_cast<const bf16x8*>(ob + C::OB_H)[s * 64 + lane];
        Qa = mma32b(qq[0][s], hb, Qa);
        Qb = mma32b(qq[1][s], hb, Qb);
      }
      const f32x4 Ua = reinterpret_cast<const f32x4*>(ob + C::OB_U)[lane];
      const f32x4 Ub = reinterpret_cast<const f32x4*>(ob + C::OB_U)[64 + lane];
      const bf16x4 uah = hi4(Ua), ubh = hi4(Ub);
      const bf16x4 ual = lo4(Ua, uah), ubl = lo4(Ub, ubh);
      const f32x4 ga = reinterpret_cast<const f32x4*>(rec + C::GM)[grp];
      const f32x4 gb = reinterpret_cast<const f32x4*>(rec + C::GM)[4 + grp];
      const bf16x8 pf0 = reinterpret_cast<const bf16x8*>(rec + C::PF0)[lane];
      const bf16x8 pf1h = reinterpret_cast<const bf16x8*>(rec + C::PF1H)[lane];
      const bf16x8 pf1l = reinterpret_cast<const bf16x8*>(rec + C::PF1L)[lane];
      f32x4 Oa, Ob;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Oa[i] = ga[i] * Qa[i];
        Ob[i] = gb[i] * Qb[i];
      }
      // O_a += P00 U_a ; O_b += P10 U_a + P11 U_b  (P and U in hi + lo parts)
      Oa = mma32b(pf0, cat8(uah, uah), Oa);
      Oa = mma32b(pf0, cat8(ual, bf16x4{}), Oa);
      Ob = mma32b(pf1h, cat8(uah, ubh), Ob);
      Ob = mma32b(pf1l, cat8(uah, ubh), Ob);
      Ob = mma32b(pf1h, cat8(ual, ubl), Ob);
      __bf16* oc = orow + (int64_t)(32 * c) * ostride;
      if (32 * c + 32 <= T) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          oc[i * ostride] = (__bf16)Oa[i];
          oc[(16 + i) * ostride] = (__bf16)Ob[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (32 * c + 4 * grp + i < T) oc[i * ostride] = (__bf16)Oa[i];
          if (32 * c + 16 + 4 * grp + i < T) oc[(16 + i) * ostride] = (__bf16)Ob[i];
        }
      }
    };
    static_assert(NP % 2 == 0, "pair parity selects the q register set");
    loadq(qs[0], 0);
    __syncthreads();  // epoch 0 prepared
    for (int ep = 0; ep < NE; ++ep) {
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const int c = ep * NP + j;
        loadq(qs[(j + 1) & 1], c + 1);
        if (c < NSC) pair(qs[j & 1], ep, j);
      }
      __syncthreads();
    }
    return;
  }

  // -------------------------------------------------------------- producers
  const int p = wave - 2;
  char* scr = smem + C::OFF_SCR + p * C::SCR;
  float* sA0 = reinterpret_cast<float*>(scr + C::SA0);   // A00, then T00
  float* sA1 = reinterpret_cast<float*>(scr + C::SA1);   // A11, then T11
  float* sB = reinterpret_cast<float*>(scr + C::SB);
  float* sG = reinterpret_cast<float*>(scr + C::SG);

  // Global loads of pair c into r (pair index clamped, rows clamped to T-1 so
  // every address is valid and the number of loads never varies, whichever
  // branch issues them).  Padding rows
  // need no masking of q, k or v: with beta = 0 and g = 0 their rows of T are
  // unit vectors, so their U rows -- and every contribution they make to O or
  // to the state -- are exactly zero.
  const __bf16* const kb0 = k + tok0 * DK + 8 * grp;
  const __bf16* const qb0 = q + tok0 * DK + 8 * grp;
  const __bf16* const vb0 = v + tok0 * DV + v0 + n;
  const float* const gb0 = gate + tok0;
  const float* const bb0 = beta + tok0;
  auto load = [&](Raw2<DK>& r, int c) {
    c = min(c, NSC - 1);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int t = min(32 * c + 16 * x + n, T - 1);
      const int ok = t * H * DK;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        r.kf[x][s] = *reinterpret_cast<const bf16x8*>(kb0 + ok + 32 * s);
        r.qf[x][s] = *reinterpret_cast<const bf16x8*>(qb0 + ok + 32 * s);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        r.vv[x][i] = vb0[min(32 * c + 16 * x + 4 * grp + i, T - 1) * H * DV];
      r.gx[x] = gb0[t * H];
      r.bt[x] = bb0[t * H];
    }
  };

  auto produce = [&](Raw2<DK>& r, int c) {
    if (c >= NSC) return;
    char* rec = rec_of(c / NP, c % NP);
    const int t0 = 32 * c;
    const bool oka = t0 + n < T, okb = t0 + 16 + n < T;
    // padding tokens past T: g = 0, beta = 0 (an identity step)
    const float gav = oka ? (gate_logit ? bounded_gate(r.gx[0], G) : r.gx[0]) : 0.f;
    const float gbv = okb ? (gate_logit ? bounded_gate(r.gx[1], G) : r.gx[1]) : 0.f;
    const float ba = oka ? r.bt[0] : 0.f, bb = okb ? r.bt[1] : 0.f;
    const float Ga = scan16_dpp(gav);
    const float Ga15 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, Ga), 15));
    const float Gb = Ga15 + scan16_dpp(gbv);
    const float Gb15 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, Gb), 15));
    if (grp == 0) {
      float* gm = reinterpret_cast<float*>(rec + C::GM);
      float* dl = reinterpret_cast<float*>(rec + C::DL);
      gm[n] = __expf(Ga);
      gm[16 + n] = __expf(Gb);
      dl[n] = __expf(Gb15 - Ga);
      dl[16 + n] = __expf(Gb15 - Gb);
      if (n == 0) *reinterpret_cast<float*>(rec + C::GC) = __expf(Gb15);
      sB[n] = ba;
      sB[16 + n] = bb;
      sG[n] = Ga;
      sG[16 + n] = Gb;
    }
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      bf16x4 vf;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vf[i] = (t0 + 16 * x + 4 * grp + i < T) ? r.vv[x][i] : (__bf16)0.f;
      reinterpret_cast<bf16x4*>(rec + C::VF)[x * 64 + lane] = vf;
    }
    const bf16x8* ka = r.kf[0];
    const bf16x8* kb = r.kf[1];
    const bf16x8* qa = r.qf[0];
    const bf16x8* qb = r.qf[1];
    // lane (n, grp) reg i of each product holds block entry [n][4 grp + i]
    f32x4 s00 = zero4(), s11 = zero4(), s10 = zero4();
    f32x4 p00 = zero4(), p11 = zero4(), p10 = zero4();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      s00 = mma32b(ka[s], ka[s], s00);
      s11 = mma32b(kb[s], kb[s], s11);
      s10 = mma32b(ka[s], kb[s], s10);     // [n][s] = k_b,n . k_a,s
      p00 = mma32b(ka[s], qa[s], p00);     // [n][s] = q_a,n . k_a,s
      p11 = mma32b(kb[s], qb[s], p11);
      p10 = mma32b(ka[s], qb[s], p10);     // [n][s] = q_b,n . k_a,s
    }
    // K fragments for the chain (after this the registers of r are dead)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      reinterpret_cast<bf16x8*>(rec + C::KF)[kslot(s, grp, n)] = ka[s];
      reinterpret_cast<bf16x8*>(rec + C::KF + NS * 1024)[kslot(s, grp, n)] = kb[s];
    }
    wave_fence();
    const f32x4 Gca = reinterpret_cast<const f32x4*>(sG)[grp];       // G_a at the 4 columns
    const f32x4 Gcb = reinterpret_cast<const f32x4*>(sG)[4 + grp];   // G_b at the 4 columns
    f32x4 a00, a11, a10, pp00, pp11, pp10;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sc = 4 * grp + i;
      const float d00 = __expf(fminf(Ga - Gca[i], 0.f));
      const float d11 = __expf(fminf(Gb - Gcb[i], 0.f));
      const float d10 = __expf(fminf(Gb - Gca[i], 0.f));
      a00[i] = sc < n ? ba * d00 * s00[i] : 0.f;
      a11[i] = sc < n ? bb * d11 * s11[i] : 0.f;
      a10[i] = bb * d10 * s10[i];
      pp00[i] = sc <= n ? d00 * p00[i] : 0.f;
      pp11[i] = sc <= n ? d11 * p11[i] : 0.f;
      pp10[i] = d10 * p10[i];
    }
    reinterpret_cast<f32x4*>(sA0)[n * 4 + grp] = a00;
    reinterpret_cast<f32x4*>(sA1)[n * 4 + grp] = a11;
    {
      const bf16x4 h00 = hi4(pp00), h10 = hi4(pp10), h11 = hi4(pp11);
      reinterpret_cast<bf16x8*>(rec + C::PF0)[lane] = cat8(h00, lo4(pp00, h00));
      reinterpret_cast<bf16x8*>(rec + C::PF1H)[lane] = cat8(h10, h11);
      reinterpret_cast<bf16x8*>(rec + C::PF1L)[lane] = cat8(lo4(pp10, h10), lo4(pp11, h11));
    }
    wave_fence();

    // T00 (lane groups 0, 1) and T11 (groups 2, 3), row n per lane:
    // T[n][s] = delta_ns - sum_{r > s} T[n][r] A[r][s]; rows of A are read one
    // step ahead of their use.  The rows of T then overwrite A.
    {
      // x holds row n of T below the diagonal (it starts at 0; the unit
      // diagonal enters as x[n] = 1 when step rr reaches n).
      f32x4* Ab = reinterpret_cast<f32x4*>(grp < 2 ? sA0 : sA1);
      float x[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) x[s] = 0.f;
      f32x4 cur[4], nxt[4];
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) cur[c4] = Ab[15 * 4 + c4];
#pragma unroll
      for (int rr = 15; rr >= 1; --rr) {
        if (rr > 1) {
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) nxt[c4] = Ab[(rr - 1) * 4 + c4];
        }
        const float xr = (rr == n) ? 1.f : x[rr];
#pragma unroll
        for (int s = 0; s < rr; ++s) x[s] -= xr * cur[s >> 2][s & 3];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) cur[c4] = nxt[c4];
      }
      wave_fence();   // every lane has read all rows of A before T overwrites it
      if ((grp & 1) == 0) {
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          f32x4 row;
#pragma unroll
          for (int e = 0; e < 4; ++e) row[e] = (4 * c4 + e == n) ? 1.f : x[4 * c4 + e];
          Ab[n * 4 + c4] = row;
        }
      }
    }
    wave_fence();
    const float* sT0 = sA0;
    const float* sT1 = sA1;

    // M = A10 T00 (fp32 MFMA): A = A10 rows (registers), B = T00 columns.
    f32x4 t00c;
#pragma unroll
    for (int j = 0; j < 4; ++j) t00c[j] = sT0[(4 * grp + j) * 16 + n];
    const f32x4 M = F::mma16(F::F16{a10}, F::F16{t00c}, zero4());   // lane: M[4grp+i][n]
    // (T11 M)^T = M^T T11^T: the accumulator of M is the A fragment of M^T;
    // T11 rows give the B fragment of T11^T.  Lane (n, grp) reg i of the result
    // is (T11 M)[n][4 grp + i] = -T10[n][4 grp + i].
    const f32x4 t11r = reinterpret_cast<const f32x4*>(sT1)[n * 4 + grp];
    const f32x4 TM = F::mma16(F::F16{M}, F::F16{t11r}, zero4());
    const f32x4 t00r = reinterpret_cast<const f32x4*>(sT0)[n * 4 + grp];
    const f32x4 bea = reinterpret_cast<const f32x4*>(sB)[grp];
    const f32x4 beb = reinterpret_cast<const f32x4*>(sB)[4 + grp];
    f32x4 tb00, tb10, tb11;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tb00[i] = t00r[i] * bea[i];
      tb10[i] = -TM[i] * bea[i];
      tb11[i] = t11r[i] * beb[i];
    }
    {
      const bf16x4 h00 = hi4(tb00), h10 = hi4(tb10), h11 = hi4(tb11);
      reinterpret_cast<bf16x8*>(rec + C::TB0)[lane] = cat8(h00, lo4(tb00, h00));
      reinterpret_cast<bf16x8*>(rec + C::TB1H)[lane] = cat8(h10, h11);
      reinterpret_cast<bf16x8*>(rec + C::TB1L)[lane] = cat8(lo4(tb10, h10), lo4(tb11, h11));
    }
    // Loads of this producer's pair in the next epoch.  Issued last, so no
    // wait in this pair's work queues behind them; they land while the wave
    // waits at the barrier.
    load(r, c + NP);
    wave_fence();   // the next pair's scratch writes must not pass these reads
  };

  // One register set: produce(c) issues the loads of pair c + NP itself.
  Raw2<DK> ra;
  load(ra, p);
  produce(ra, p);               // epoch 0 (loads pair NP + p for epoch 1)
  __syncthreads();
  for (int ep = 0; ep < NE; ++ep) {
    produce(ra, (ep + 1) * NP + p);
    __syncthreads();
  }
}

template <int DK>
static hipError_t launch2_t(const void* q, const void* k, const void* v, const float* gate,
                            int gate_logit, float G, const float* beta, const float* h0,
                            void* o, float* hT, int B, int T, int H, int Dv, hipStream_t st) {
  const int blocks = B * H * (Dv / 16);
  hipLaunchKernelGGL((chunk_fwd2_kernel<DK>), dim3(blocks), dim3(64 * Cfg2<DK>::NW), 0, st,
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, gate, gate_logit, G,
                     beta, h0, (__bf16*)o, hT, B, T, H, Dv);
  return hipGetLastError();
}

hipError_t launch_chunk_fwd_pair(const void* q, const void* k, const void* v, const float* gate,
                                 int gate_logit, float G, const float* beta, const float* h0,
                                 void* o, float* hT, int B, int T, int H, int Dk, int Dv,
                                 hipStream_t st) {
  if (Dk == 64) return launch2_t<64>(q, k, v, gate, gate_logit, G, beta, h0, o, hT, B, T, H, Dv, st);
  if (Dk == 128) return launch2_t<128>(q, k, v, gate, gate_logit, G, beta, h0, o, hT, B, T, H, Dv, st);
  return hipErrorInvalidValue;
}

}  // namespace la
