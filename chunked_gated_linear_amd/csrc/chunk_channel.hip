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
// The state and every accumulation are fp32.  fp32 inputs run every product
// on the fp32 MFMA (16x16x4).  bf16 inputs run A, P, the solve, T Y and P U in
// fp32 too, and the state products (K o Gam) H, (Q o Gam) H and the update on
// the bf16 MFMA: the state as a bf16 copy, U as bf16 high and low parts.
// Two launches:
//   chunk_channel_prep_kernel  one wave per (sequence, head, tile), all in
//       parallel: the gate, the per-channel in-tile running sums (DPP row
//       scans), the scaled operands, A and P on MFMA, the 16 x 16 solve; the
//       tile's record (everything that does not depend on the state) goes to
//       the workspace once per head;
//   chunk_fwd_channel_kernel   one workgroup per (sequence, head, 16-column
//       slice of d_v): wave 0 ("chain") owns the fp32 state slice in
//       registers and runs the serial part; waves 1..NP ("loaders") copy the
//       records and the slice's v values into LDS, double-buffered by epochs
//       of NP = 2 tiles, their global loads issued two epochs before the
//       chain reads them; the chain forms the outputs (for bf16 in 78 KB of
//       LDS, so that two workgroups share a compute unit).
// bf16 inputs with fewer workgroups than two per compute unit (a few long
// sequences) take the 32-token pair path of chunk_channel_pair.hip instead.
#include "la_device.h"
#include "la_launch.h"

namespace la {
namespace {

// One tile's record (bytes), in the workspace and in LDS; every field is
// lane-contiguous in the order the chain wave reads it.  The workspace copy
// stops at VF: the v values belong to a column slice and are loaded per slice.
// EB is the byte size of the state-facing operands: 4 (fp32 fragments for the
// fp32 MFMA) for fp32 inputs, 2 (bf16 fragments for the bf16 MFMA) for bf16
// inputs; (K o Gam_C/Gam)^T takes 16 bytes per lane and state tile either way
// (4 fp32, or 4 bf16 tokens twice, the A side of a hi/lo product).
template <int DK, int EB>
struct ChRec {
  static constexpr int NT = DK / 16;   // 16-row tiles of the state slice
  static constexpr int NS = DK / 32;   // 32-deep contraction blocks
  static constexpr int KF = 0;                       // K o Gam:  NS x 64 lanes x 8
  static constexpr int QF = KF + NS * 64 * 8 * EB;   // Q o Gam:  NS x 64 x 8
  static constexpr int KT = QF + NS * 64 * 8 * EB;   // (K o Gam_C/Gam)^T: NT x 64 x 16 B
  static constexpr int PF = KT + NT * 64 * 16;       // P: 64 x 4 f32
  static constexpr int TB = PF + 64 * 4 * 4;         // (I + A)^-1 diag(beta), 16 x 16
  static constexpr int GC = TB + 256 * 4;            // Gam_C[DK]
  static constexpr int VF = GC + DK * 4;             // V slice: 64 x 4 (LDS only)
  static constexpr int GLOBAL = VF;                  // bytes per tile in the workspace
  static constexpr int LDS = VF + 64 * 4 * 4;        // bytes per tile in LDS
  static constexpr int CHUNKS = GLOBAL / 16;         // 16-byte pieces of a record
  static_assert(GLOBAL % 16 == 0 && LDS % 16 == 0, "alignment");
};

// Producer scratch per wave (LDS): A (16 x 16) and beta[16].
constexpr int kScrA = 0, kScrB = 1024, kScr = 1024 + 64;
// Per-wave LDS of the preparation kernel: the scratch above, then the staged
// transposed key block (at most 8 tiles x 64 lanes x 16 bytes) and Gam_C (at
// most 128 floats, kGcs bytes into the staging area).
constexpr int kGcs = 8 * 64 * 16;
constexpr int kKts = kScr, kPrepWave = kScr + kGcs + 128 * 4;

// Records of two epochs of NP tiles.
template <typename E, int DK, int NP>
struct ChCfg {
  static constexpr int LDS = 2 * NP * ChRec<DK, sizeof(E)>::LDS;
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Inclusive prefix sum over the 16 lanes of each row (DPP row shifts by 1, 2,
// 4, 8; lanes whose source falls outside the row add 0): no LDS traffic.
__device__ inline float row_scan16(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, false));
  return x;
}

// Lane L of each 16-lane row broadcast to the whole row (DPP row_newbcast).
template <int L>
__device__ inline float row_bcast(float x) {
  static_assert(L >= 0 && L < 16, "lane within a row");
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + L, 0xf, 0xf, false));
}

// Registers for preparing one tile: the lane's 8 * NS channels of its token's
// k and q (in the input type), the same channels of the gate, beta.
template <typename E, int DK>
struct ChRaw {
  typename Elt<E>::F32 kf[DK / 32];
  typename Elt<E>::F32 qf[DK / 32];
  f32x4 glo[DK / 32], ghi[DK / 32];
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

// Loads of tile c of a sequence of T tokens whose token t is row
// (tok0 + t) * H + h of the arrays (token rows past the end read the last
// valid row; prep_tile zeroes them).
template <typename E, int DK>
__device__ inline void load_tile(ChRaw<E, DK>& r, const E* __restrict__ q,
                                 const E* __restrict__ k, const float* __restrict__ gate,
                                 const float* __restrict__ beta, int64_t tok0, int h, int c,
                                 int T, int H, int n, int grp) {
  constexpr int NS = DK / 32;
  const int t = min(16 * c + n, T - 1);
  const int64_t row = (tok0 + t) * H + h;
  const int64_t base = row * DK;
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
  r.bt = beta[row];
}

// Prepare tile c into the record at `rec` (sA, sB: this wave's LDS scratch).
template <typename E, int DK>
// The transposed key block (NT x 64 lanes x 16 bytes) and Gam_C are assembled
// in `kts`, this wave's LDS staging area, and copied to the record as whole
// 16-byte fragments.
__device__ inline void prep_tile(const ChRaw<E, DK>& r, int c, int T, char* __restrict__ rec,
                                 float* sA, float* sB, char* kts, int gate_logit, float G, int n,
                                 int grp, int lane) {
  using R = ChRec<DK, sizeof(E)>;
  using X = Elt<float>;
  using F16 = X::F16;
  using F32 = X::F32;
  constexpr int NS = R::NS;
    // padding tokens past T: q = k = v = 0, g = 0, beta = 0 (an identity step)
    const bool ok = 16 * c + n < T;
    const float bt = ok ? r.bt : 0.f;
    if (grp == 0) sB[n] = bt;
    // One 32-deep channel block s at a time (8 channels per lane: j < 4 is
    // channel 32s + 4grp + j, j >= 4 is 32s + 16 + 4grp + j - 4; token t = n):
    // the per-channel running sums, the scaled operands, their share of A and
    // P (lane (n, grp) register i ends with entry [n][4grp+i], i.e. row n,
    // column s = 4grp+i, of A before beta and of P), and the record fields.
    f32x4 sa = zero4(), sp = zero4();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const F32 k32 = to_f32(r.kf[s]), q32 = to_f32(r.qf[s]);
      float vkg[8], vqg[8], vkm[8], vqm[8], vki[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = j < 4 ? r.glo[s][j] : r.ghi[s][j - 4];
        // log mode: clamped to [-G, 0], so that the in-tile factors stay
        // within exp(+-8 G) whatever the caller passes
        const float g = ok ? (gate_logit ? bounded_gate(x, G) : fminf(fmaxf(x, -G), 0.f)) : 0.f;
        const float Gt = row_scan16(g);                 // G_t[c], t = n
        const float Gm = row_bcast<7>(Gt);              // G at the middle token
        const float Gl = row_bcast<15>(Gt);             // G at the last token
        const float kv = ok ? (j < 4 ? k32.lo[j] : k32.hi[j - 4]) : 0.f;
        const float qv = ok ? (j < 4 ? q32.lo[j] : q32.hi[j - 4]) : 0.f;
        const float e_start = __expf(Gt);               // Gam_t            (<= 1)
        const float e_last = row_bcast<15>(e_start);    // Gam_C = exp(G at the last token)
        const float e_end = __expf(Gl - Gt);            // Gam_C / Gam_t    (<= 1)
        const float e_mid = __expf(Gt - Gm);            // Gam_t / Gam_m
        const float e_imid = __expf(Gm - Gt);           // Gam_m / Gam_t
        vkg[j] = kv * e_start;
        vqg[j] = qv * e_start;
        vkm[j] = kv * e_mid;
        vqm[j] = qv * e_mid;
        vki[j] = kv * e_imid;
        const int ch = 32 * s + (j < 4 ? 4 * grp + j : 16 + 4 * grp + j - 4);
        // (K o Gam_C/Gam)^T in the chain's A-fragment order: for state tile
        // ch / 16, lane (ch % 16, n / 4) register n % 4
        const int kt_lane = (ch >> 4) * 64 + (n >> 2) * 16 + (ch & 15);
        if constexpr (sizeof(E) == 4) {
          reinterpret_cast<float*>(kts)[kt_lane * 4 + (n & 3)] = kv * e_end;
        } else {   // token n in registers n % 4 and 4 + n % 4 of its lane
          const __bf16 kd = (__bf16)(kv * e_end);
          reinterpret_cast<__bf16*>(kts)[kt_lane * 8 + (n & 3)] = kd;
          reinterpret_cast<__bf16*>(kts)[kt_lane * 8 + 4 + (n & 3)] = kd;
        }
        if (n == 0) reinterpret_cast<float*>(kts + kGcs)[ch] = e_last;
      }
      F32 kg, qg, km, qm, ki;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kg.lo[j] = vkg[j]; kg.hi[j] = vkg[4 + j];
        qg.lo[j] = vqg[j]; qg.hi[j] = vqg[4 + j];
        km.lo[j] = vkm[j]; km.hi[j] = vkm[4 + j];
        qm.lo[j] = vqm[j]; qm.hi[j] = vqm[4 + j];
        ki.lo[j] = vki[j]; ki.hi[j] = vki[4 + j];
      }
      if constexpr (sizeof(E) == 4) {
        reinterpret_cast<F32*>(rec + R::KF)[s * 64 + lane] = kg;
        reinterpret_cast<F32*>(rec + R::QF)[s * 64 + lane] = qg;
      } else {
        Elt<__bf16>::F32 kb, qb;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          kb.v[j] = (__bf16)vkg[j];
          qb.v[j] = (__bf16)vqg[j];
        }
        reinterpret_cast<Elt<__bf16>::F32*>(rec + R::KF)[s * 64 + lane] = kb;
        reinterpret_cast<Elt<__bf16>::F32*>(rec + R::QF)[s * 64 + lane] = qb;
      }
      sa = X::mma32(ki, km, sa);
      sp = X::mma32(ki, qm, sp);
    }
    f32x4 arow, prow;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s_ = 4 * grp + i;
      arow[i] = s_ < n ? bt * sa[i] : 0.f;
      prow[i] = s_ <= n ? sp[i] : 0.f;
    }
    reinterpret_cast<f32x4*>(sA)[n * 4 + grp] = arow;          // A[n][4grp..4grp+3]
    reinterpret_cast<F16*>(rec + R::PF)[lane] = X::from_acc(prow);
    // this wave's LDS writes (A, beta, the staged key block) before its reads
    // of them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int t = 0; t < R::NT; ++t)
      reinterpret_cast<f32x4*>(rec + R::KT)[t * 64 + lane] =
          reinterpret_cast<const f32x4*>(kts)[t * 64 + lane];
    if (lane < DK / 4)
      reinterpret_cast<f32x4*>(rec + R::GC)[lane] =
          reinterpret_cast<const f32x4*>(kts + kGcs)[lane];

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
        *reinterpret_cast<f32x4*>(rec + R::TB + (n * 16 + s) * 4) = row;
      }
    }
}

static inline int channel_varlen_slots(int T, int nseq) { return T / 16 + nseq + 1; }

// Packed sequences: sequence s is tokens [cu[s], cu[s+1]) of one packed
// sequence of TB tokens (offsets clamped to [0, TB] so that any values stay
// memory-safe); its tile c has workspace record slot(s, c) = floor(cu[s] / 16)
// + s + c of nslot per head (slots of different sequences do not overlap for
// non-decreasing offsets, and nslot = TB / 16 + nseq + 1 covers them all).
__device__ inline int ch_seq_begin(const int* cu, int s, int TB) { return min(max(cu[s], 0), TB); }
__device__ inline int ch_seq_end(const int* cu, int s, int TB) {
  return min(max(cu[s + 1], ch_seq_begin(cu, s, TB)), TB);
}

// ------------------------------------------------------------- prep kernel
// Batched (cu == nullptr): job = (b H + h) NC + c.  Packed: job = h nslot +
// slot, the sequence found by binary search over the offsets, unused slots
// skipped.
template <typename E, int DK>
__global__ __launch_bounds__(256) void chunk_channel_prep_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const float* __restrict__ gate,
    int gate_logit, float G, const float* __restrict__ beta, char* __restrict__ ws, int B,
    int T, int H, const int* __restrict__ cu, int nslot) {
  __shared__ __attribute__((aligned(16))) char smem[4 * kPrepWave];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, grp = lane >> 4;
  float* sA = reinterpret_cast<float*>(smem + wave * kPrepWave + kScrA);
  float* sB = reinterpret_cast<float*>(smem + wave * kPrepWave + kScrB);
  char* kts = smem + wave * kPrepWave + kKts;
  const int NC = (T + 15) >> 4;
  const int64_t jobs = cu ? (int64_t)H * nslot : (int64_t)B * H * NC;
  for (int64_t job = (int64_t)blockIdx.x * 4 + wave; job < jobs; job += (int64_t)gridDim.x * 4) {
    int c, h, Ts;
    int64_t tok0;
    if (cu) {
      h = (int)(job / nslot);
      const int slot = (int)(job - (int64_t)h * nslot);
      int lo = 0, hi = B - 1;                    // the last s with slot(s, 0) <= slot
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ch_seq_begin(cu, mid, T) / 16 + mid <= slot) lo = mid;
        else hi = mid - 1;
      }
      const int tb = ch_seq_begin(cu, lo, T);
      Ts = ch_seq_end(cu, lo, T) - tb;
      c = slot - (tb / 16 + lo);
      if (c < 0 || c >= ((Ts + 15) >> 4)) continue;   // a slot no tile uses
      tok0 = tb;
    } else {
      c = (int)(job % NC);
      const int64_t bh = job / NC;
      h = (int)(bh % H);
      tok0 = (bh / H) * (int64_t)T;
      Ts = T;
    }
    ChRaw<E, DK> r;
    load_tile<E, DK>(r, q, k, gate, beta, tok0, h, c, Ts, H, n, grp);
    prep_tile<E, DK>(r, c, Ts, ws + job * ChRec<DK, sizeof(E)>::GLOBAL, sA, sB, kts, gate_logit,
                     G, n, grp, lane);
    // the next job's writes to A / beta must not pass this job's reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

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

// A loader's registers for one tile: its share of the record (16-byte pieces
// lane, lane + 64, ...) and the slice's four v values.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
template <typename E, int DK>
struct ChCopy {
  static constexpr int PIECES = (ChRec<DK, sizeof(E)>::CHUNKS + 63) / 64;
  u32x4 piece[PIECES];
  E vv[4];
};

// ------------------------------------------------------------ chain kernel
template <typename E, int DK, int NP>
__global__ __launch_bounds__(64 * (NP + 1)) void chunk_fwd_channel_kernel(
    const E* __restrict__ v, const char* __restrict__ ws, const float* h0,
    E* __restrict__ o, float* hT, int B, int TA, int H, int DV, const int* __restrict__ cu,
    int nslot) {
  using R = ChRec<DK, sizeof(E)>;
  using C = ChCfg<E, DK, NP>;
  using X = Elt<float>;
  using F16 = X::F16;
  using F32 = X::F32;
  constexpr int NT = R::NT, NS = R::NS;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  const int NV = DV / 16;
  int head, vt;
  ch_map_block(blockIdx.x, B * H, NV, head, vt);
  const int b = head / H, h = head % H;
  const int v0 = vt * 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, grp = lane >> 4;
  // this sequence: T tokens whose token t is row (tok0 + t) * H + h, tile c's
  // record at recs + c * GLOBAL
  int T;
  int64_t tok0, rec0;
  if (cu) {
    const int tb = ch_seq_begin(cu, b, TA);
    T = ch_seq_end(cu, b, TA) - tb;
    tok0 = tb;
    rec0 = (int64_t)h * nslot + tb / 16 + b;
  } else {
    T = TA;
    tok0 = (int64_t)b * TA;
    rec0 = ((int64_t)b * H + h) * ((TA + 15) >> 4);
  }
  const int NC = (T + 15) >> 4;
  const int NE = (NC + NP - 1) / NP;

  auto rowk = [&](int t) -> int64_t { return (tok0 + t) * H + h; };
  auto rec_of = [&](int ep, int j) -> char* { return smem + ((ep & 1) * NP + j) * R::LDS; };
  const int64_t ostride = (int64_t)H * DV;
  E* const orow = o + rowk(4 * grp) * DV + v0 + n;   // token 4 grp of the tile, column v0 + n

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
    __syncthreads();  // epoch 0 loaded
    for (int ep = 0; ep < NE; ++ep) {
      for (int j = 0; j < NP; ++j) {
        const int c = ep * NP + j;
        if (c >= NC) break;
        const char* rec = rec_of(ep, j);
        if constexpr (sizeof(E) == 4) {
          // R = (K o Gam) H and (Q o Gam) H, contraction over d_k, then
          // U = T (V - R), H' = diag(Gam_C) H + (K o Gam_C/Gam)^T U: fp32 MFMA
          f32x4 Rk = zero4(), QH = zero4();
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            const F32 hb = X::from_acc2(Hacc[2 * s], Hacc[2 * s + 1]);
            const F32 kf = reinterpret_cast<const F32*>(rec + R::KF)[s * 64 + lane];
            const F32 qf = reinterpret_cast<const F32*>(rec + R::QF)[s * 64 + lane];
            Rk = X::mma32(kf, hb, Rk);
            QH = X::mma32(qf, hb, QH);
          }
          const F16 vf = reinterpret_cast<const F16*>(rec + R::VF)[lane];
          const F16 tb = *reinterpret_cast<const F16*>(rec + R::TB + (n * 16 + 4 * grp) * 4);
          const F16 pf = reinterpret_cast<const F16*>(rec + R::PF)[lane];
          f32x4 Y;
#pragma unroll
          for (int i = 0; i < 4; ++i) Y[i] = vf.v[i] - Rk[i];
          const f32x4 U = X::mma16(tb, X::from_acc(Y), zero4());
          const F16 ub = X::from_acc(U);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const f32x4 gc = reinterpret_cast<const f32x4*>(rec + R::GC)[4 * t + grp];
            const F16 kt = reinterpret_cast<const F16*>(rec + R::KT)[t * 64 + lane];
#pragma unroll
            for (int i = 0; i < 4; ++i) Hacc[t][i] *= gc[i];   // row 16t + 4grp + i
            Hacc[t] = X::mma16(kt, ub, Hacc[t]);
          }
          const f32x4 O = X::mma16(pf, X::from_acc(U), QH);
          E* oc = orow + (int64_t)(16 * c) * ostride;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * c + 4 * grp + i < T) oc[i * ostride] = Elt<E>::from_f(O[i]);
        } else {
          // bf16 MFMA on the bf16 operands and a bf16 copy of the state.  Every
          // operand of the chain R -> U -> H' is requested from LDS at once, in
          // order of first use, so that no read waits inside it.
          using XB = Elt<__bf16>;
          XB::F32 kf[NS], kt[NT];
          f32x4 gc[NT];
#pragma unroll
          for (int s = 0; s < NS; ++s) kf[s] = reinterpret_cast<const XB::F32*>(rec + R::KF)[s * 64 + lane];
          const F16 vf = reinterpret_cast<const F16*>(rec + R::VF)[lane];
          const F16 tb = *reinterpret_cast<const F16*>(rec + R::TB + (n * 16 + 4 * grp) * 4);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            kt[t] = reinterpret_cast<const XB::F32*>(rec + R::KT)[t * 64 + lane];
            gc[t] = reinterpret_cast<const f32x4*>(rec + R::GC)[4 * t + grp];
          }
          __builtin_amdgcn_sched_barrier(0);
          // R = (K o Gam) H
          XB::F32 hb[NS];
          f32x4 Rk = zero4();
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            hb[s] = XB::from_acc2(Hacc[2 * s], Hacc[2 * s + 1]);
            Rk = XB::mma32(kf[s], hb[s], Rk);
          }
          f32x4 Y;
#pragma unroll
          for (int i = 0; i < 4; ++i) Y[i] = vf.v[i] - Rk[i];
          const f32x4 U = X::mma16(tb, X::from_acc(Y), zero4());
          // H' = diag(Gam_C) H + (K o Gam_C/Gam)^T (U_hi + U_lo): U split into
          // bf16 high and low parts, one 32-deep bf16 MFMA per state tile
          XB::F32 ub;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const __bf16 hi = (__bf16)U[i];
            ub.v[i] = hi;
            ub.v[4 + i] = (__bf16)(U[i] - (float)hi);
          }
#pragma unroll
          for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) Hacc[t][i] *= gc[t][i];   // row 16t + 4grp + i
            Hacc[t] = XB::mma32(kt[t], ub, Hacc[t]);
          }
          // the output after the state update: O = (Q o Gam) H + P U
          f32x4 QH = zero4();
#pragma unroll
          for (int s2 = 0; s2 < NS; ++s2)
            QH = XB::mma32(reinterpret_cast<const XB::F32*>(rec + R::QF)[s2 * 64 + lane], hb[s2], QH);
          const F16 pf = reinterpret_cast<const F16*>(rec + R::PF)[lane];
          const f32x4 O = X::mma16(pf, X::from_acc(U), QH);
          E* oc = orow + (int64_t)(16 * c) * ostride;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * c + 4 * grp + i < T) oc[i * ostride] = Elt<E>::from_f(O[i]);
        }
      }
      __syncthreads();  // this epoch consumed, next epoch loaded
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

  // ---------------------------------------------------------------- loaders
  const int p = wave - 1;
  const char* recs = ws + rec0 * R::GLOBAL;
  // Global loads of tile c (clamped to the last tile, so every path issues
  // the same number of loads and the compiler can wait for the older set; an
  // empty sequence loads nothing).
  auto load = [&](ChCopy<E, DK>& r, int c) {
    if (NC == 0) return;
    c = min(c, NC - 1);
    const u32x4* src = reinterpret_cast<const u32x4*>(recs + (int64_t)c * R::GLOBAL);
#pragma unroll
    for (int i = 0; i < ChCopy<E, DK>::PIECES; ++i) {
      const int x = i * 64 + lane;
      r.piece[i] = src[x < R::CHUNKS ? x : R::CHUNKS - 1];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r.vv[i] = v[rowk(min(16 * c + 4 * grp + i, T - 1)) * DV + v0 + n];
  };
  auto store = [&](const ChCopy<E, DK>& r, int c) {
    if (c >= NC) return;
    char* rec = rec_of(c / NP, c % NP);
    u32x4* dst = reinterpret_cast<u32x4*>(rec);
#pragma unroll
    for (int i = 0; i < ChCopy<E, DK>::PIECES; ++i) {
      const int x = i * 64 + lane;
      if (x < R::CHUNKS) dst[x] = r.piece[i];
    }
    F16 vf;   // v past the end of the sequence is 0 (padding tokens)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vf.v[i] = (16 * c + 4 * grp + i < T) ? Elt<E>::to_f(r.vv[i]) : 0.f;
    reinterpret_cast<F16*>(rec + R::VF)[lane] = vf;
  };

  // Two register sets alternating by epoch: while tile (ep+1)*NP + p is
  // stored from one, the loads for tile (ep+2)*NP + p fill the other.
  // (Loads issued two epochs ahead, from a third set, measured no faster.)
  ChCopy<E, DK> ra, rb;
  load(ra, p);
  store(ra, p);                 // epoch 0
  load(ra, NP + p);             // epoch 1, stored during epoch 0
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


// B sequences of T tokens (cu == nullptr), or B packed sequences with device
// offsets cu in one sequence of T tokens.
template <typename E, int DK, int NP>
hipError_t launch_ch(const void* q, const void* k, const void* v, const float* gate,
                     int gate_logit, float G, const float* beta, const float* h0, void* o,
                     float* hT, int B, int T, int H, int Dv, const int* cu, void* ws,
                     hipStream_t st) {
  const int NC = (T + 15) / 16;
  const int nslot = channel_varlen_slots(T, B);
  const int64_t jobs = cu ? (int64_t)H * nslot : (int64_t)B * H * NC;
  const int prep_blocks = (int)((jobs + 3) / 4 < 4096 ? (jobs + 3) / 4 : 4096);
  if (prep_blocks > 0) {
    hipLaunchKernelGGL((chunk_channel_prep_kernel<E, DK>), dim3(prep_blocks), dim3(256), 0, st,
                       (const E*)q, (const E*)k, gate, gate_logit, G, beta, (char*)ws, B, T, H,
                       cu, nslot);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int blocks = B * H * (Dv / 16);
  hipLaunchKernelGGL((chunk_fwd_channel_kernel<E, DK, NP>), dim3(blocks), dim3(64 * (NP + 1)),
                     0, st, (const E*)v, (const char*)ws, h0, (E*)o, hT, B, T, H, Dv, cu, nslot);
  return hipGetLastError();
}

// ------------------------------------------------------------ decode step
// One new token per (b, h) with a per-channel decay a = exp(g) (d_k values),
// state updated in place.  With d = diag(a) h:
//     u  = beta (v - h^T (a o k)),   h' = diag(a) h + k u^T,
//     o  = h'^T q = h^T (a o q) + (k . q) u
// so h is read once and written once, as in the scalar-gate decode step.
// Layout as there: a persistent grid of 1024-thread workgroups walks the
// (b, h) list; thread (rg, c4) holds columns 4 c4 .. 4 c4 + 3 of rows rg,
// rg + RG, ... as float4; the state is streamed with non-temporal accesses.
constexpr int kDecThreads = 1024;

template <typename E, int DK, int DV>
__global__ __launch_bounds__(kDecThreads) void decode_channel_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ gate, int gate_logit, float G,
    const float* __restrict__ beta, float* __restrict__ S, E* __restrict__ o, int BH) {
  constexpr int NC4 = DV / 4;
  constexpr int RG = kDecThreads / NC4;
  constexpr int RPT = DK / RG;
  static_assert(RG * NC4 == kDecThreads && RPT * RG == DK, "decode tiling");
  __shared__ float sk[DK], sa[DK], ska[DK], sqa[DK];
  __shared__ f32x4 pa[RG][NC4], pb[RG][NC4];
  __shared__ float su[DV];
  __shared__ float skq;
  const int tid = threadIdx.x;
  const int c4 = tid % NC4, rg = tid / NC4;
  for (int64_t bh = blockIdx.x; bh < BH; bh += gridDim.x) {
    const float bt = beta[bh];
    if (tid < DK) {
      const float gx = gate[bh * DK + tid];
      const float a = __expf(gate_logit ? bounded_gate(gx, G) : fminf(fmaxf(gx, -G), 0.f));
      const float kv = Elt<E>::to_f(k[bh * DK + tid]);
      sk[tid] = kv;
      sa[tid] = a;
      ska[tid] = a * kv;
      sqa[tid] = a * Elt<E>::to_f(q[bh * DK + tid]);
    }
    f32x4* Sh = reinterpret_cast<f32x4*>(S + bh * DK * DV);
    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = __builtin_nontemporal_load(Sh + (rg + RG * i) * NC4 + c4);
    __syncthreads();
    f32x4 pk = zero4(), pq = zero4();
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      pk += ska[rg + RG * i] * s[i];
      pq += sqa[rg + RG * i] * s[i];
    }
    pa[rg][c4] = pk;
    pb[rg][c4] = pq;
    if (tid < 64) {  // k . q, one wave, fixed order
      float p = 0.f;
      for (int d = tid; d < DK; d += 64) p += sk[d] * Elt<E>::to_f(q[bh * DK + d]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
      if (tid == 0) skq = p;
    }
    __syncthreads();
    if (tid < DV) {
      const int cq = tid >> 2, cr = tid & 3;
      float hk = 0.f, hq = 0.f;
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        hk += pa[r][cq][cr];
        hq += pb[r][cq][cr];
      }
      const float u = bt * (Elt<E>::to_f(v[bh * DV + tid]) - hk);
      su[tid] = u;
      o[bh * DV + tid] = Elt<E>::from_f(hq + skq * u);
    }
    __syncthreads();
    const f32x4 u4 = reinterpret_cast<const f32x4*>(su)[c4];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = rg + RG * i;
      __builtin_nontemporal_store(sa[row] * s[i] + sk[row] * u4, Sh + row * NC4 + c4);
    }
    __syncthreads();   // the shared buffers are reused by the next (b, h)
  }
}

template <typename E, int DK, int DV>
hipError_t launch_dec_ch(const void* q, const void* k, const void* v, const float* gate,
                         int gate_logit, float G, const float* beta, float* S, void* o, int BH,
                         hipStream_t st) {
  const int cap = 4 * device_cus();
  const int grid = BH < cap ? BH : cap;
  hipLaunchKernelGGL((decode_channel_kernel<E, DK, DV>), dim3(grid), dim3(kDecThreads), 0, st,
                     (const E*)q, (const E*)k, (const E*)v, gate, gate_logit, G, beta, S, (E*)o,
                     BH);
  return hipGetLastError();
}

}  // namespace

// bf16 inputs take either the 16-token path or the 32-token pair path
// (chunk_channel_pair.hip), chosen at launch from the workgroup count: the
// workspace covers both.
long long chunk_channel_workspace_bytes(int B, int T, int H, int Dk, int Dv, int fp32) {
  const long long nc = (T + 15) / 16;
  const long long rec = fp32 ? (Dk == 64 ? ChRec<64, 4>::GLOBAL : ChRec<128, 4>::GLOBAL)
                             : (Dk == 64 ? ChRec<64, 2>::GLOBAL : ChRec<128, 2>::GLOBAL);
  const long long one = (long long)B * H * nc * rec;
  if (fp32) return one;
  const long long pair = chunk_channel_pair_workspace_bytes(B, T, H, Dk, Dv);
  return one > pair ? one : pair;
}

hipError_t launch_chunk_fwd_channel(const void* q, const void* k, const void* v,
                                    const float* gate, int gate_logit, float G,
                                    const float* beta, const float* h0, void* o, float* hT,
                                    int B, int T, int H, int Dk, int Dv, int fp32, void* ws,
                                    hipStream_t st) {
  return launch_chunk_fwd_channel_varlen(q, k, v, gate, gate_logit, G, beta, h0, o, hT, nullptr,
                                         B, T, H, Dk, Dv, fp32, ws, st);
}

hipError_t launch_chunk_fwd_channel_varlen(const void* q, const void* k, const void* v,
                                           const float* gate, int gate_logit, float G,
                                           const float* beta, const float* h0, void* o,
                                           float* hT, const int* cu, int B, int T, int H, int Dk,
                                           int Dv, int fp32, void* ws, hipStream_t st) {
// Tiles per epoch (= loader waves) and who forms the outputs.  fp32: two, the
// chain (the fp32 records take 110 KB).  bf16 with fewer workgroups than two
// per compute unit (a few long sequences): the 32-token pair path (144 KB,
// one workgroup per unit, each as fast as it can go).  bf16 with more (many
// sequences or heads): two tiles, the chain (78 KB: two workgroups share a
// unit).
#define LA_CH(E, DK, NP) \
  return launch_ch<E, DK, NP>(q, k, v, gate, gate_logit, G, beta, h0, o, hT, B, T, H, Dv, \
                                    cu, ws, st)
  if (fp32) {
    if (Dk == 64) LA_CH(float, 64, 2);
    if (Dk == 128) LA_CH(float, 128, 2);
  } else {
    const bool dense = (int64_t)B * H * (Dv / 16) >= 2 * (int64_t)device_cus();
    if (!dense)
      return launch_chunk_fwd_channel_pair(q, k, v, gate, gate_logit, G, beta, h0, o, hT, B, T,
                                           H, Dk, Dv, cu, ws, st);
    if (Dk == 64) LA_CH(__bf16, 64, 2);
    if (Dk == 128) LA_CH(__bf16, 128, 2);
  }
#undef LA_CH
  return hipErrorInvalidValue;
}

long long chunk_channel_varlen_workspace_bytes(int T, int nseq, int H, int Dk, int fp32) {
  const long long rec = fp32 ? (Dk == 64 ? ChRec<64, 4>::GLOBAL : ChRec<128, 4>::GLOBAL)
                             : (Dk == 64 ? ChRec<64, 2>::GLOBAL : ChRec<128, 2>::GLOBAL);
  const long long one = (long long)H * channel_varlen_slots(T, nseq) * rec;
  if (fp32) return one;
  const long long pair = chunk_channel_pair_varlen_workspace_bytes(T, nseq, H, Dk);
  return one > pair ? one : pair;
}

hipError_t launch_decode_channel(const void* q, const void* k, const void* v,
                                 const float* gate, int gate_logit, float G, const float* beta,
                                 float* S, void* o, int BH, int Dk, int Dv, int fp32,
                                 hipStream_t st) {
#define LA_DECC(E, DK, DV) \
  if (Dk == DK && Dv == DV) return launch_dec_ch<E, DK, DV>(q, k, v, gate, gate_logit, G, beta, S, o, BH, st);
  if (fp32) {
    LA_DECC(float, 64, 64) LA_DECC(float, 64, 128) LA_DECC(float, 128, 64) LA_DECC(float, 128, 128)
  } else {
    LA_DECC(__bf16, 64, 64) LA_DECC(__bf16, 64, 128) LA_DECC(__bf16, 128, 64) LA_DECC(__bf16, 128, 128)
  }
#undef LA_DECC
  return hipErrorInvalidValue;
}

}  // namespace la
