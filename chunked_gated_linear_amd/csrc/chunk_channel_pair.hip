// chunk_channel_pair.hip -- the per-channel forward pass for bf16 inputs,
// with the state carried across pairs of 16-token tiles (32 tokens).
//
// Same recurrence and tile algebra as chunk_channel.hip (the decay acts on the
// key side of the old state, then the delta-rule erase and write; inside a
// tile the cumulative per-channel decay Gam_t = exp(G_t) enters the matrix-core
// operands, and the reciprocal of the cumulative decay appears -- the case the
// pages bound the log-decay for: "Core Technologies Behind Ultra-Long-Context
// Sparse MoE Large Models", sec. 2.1 and 2.3; "How Trillion-Scale Sparse MoE
// Models Achieve Million-Token Long Context", sec. 3.1 and 3.2).  Here the
// state steps over a pair of tiles a (tokens 0..15) and b (16..31) at once,
// with G_t the running sum over the pair:
//     A = [[A00, 0], [A10, A11]],  A[t][s] = beta_t (k_t o Gam_t) . (k_s / Gam_s)  (s < t)
//     P = [[P00, 0], [P10, P11]],  P[t][s] = (q_t o Gam_t) . (k_s / Gam_s)       (s <= t)
//     U  = (I + A)^-1 diag(beta) (V - (K o Gam) H)
//     O  = (Q o Gam) H + P U
//     H' = diag(Gam_31) H + (K o (Gam_31 / Gam))^T U
// (I + A)^-1 is blockwise: T00 and T11 are the tiles' 16 x 16 inverses and
// T10 = -T11 A10 T00.  Operand ranges: the state-facing operands K o Gam,
// Q o Gam and K o Gam_31/Gam are at most 1.  For the diagonal blocks the
// factors are taken about each tile's middle token (token 7, token 23), so
// every operand stays within exp(+-8 G) as in the single-tile form; for the
// cross blocks A10 and P10 (t in b, s in a) about the boundary token 15:
// (k_t o exp(G_t - G_15)) . (k_s o exp(G_15 - G_s)), both factors at most 1.
// So no operand comes near the float overflow or the subnormal range at any G.
//
// Precision: A, P, the solves and T10 in fp32 (fp32 MFMA 16x16x4); the
// record's operators T diag(beta) and P in bf16 hi + lo parts; the state is
// fp32 in registers, its bf16 copy feeds (K o Gam) H and (Q o Gam) H; the
// state update takes U rounded to bf16 (one part), the output U in hi + lo.
//
// Two launches:
//   chunk_channel_prep_pair_kernel   one wave per (sequence, head, pair), all
//       in parallel: the pair's record (everything that does not depend on the
//       state, 31,232 bytes at d_k = 128) into the workspace;
//   chunk_fwd_channel_pair_kernel    one workgroup per (sequence, head,
//       16-column slice of d_v): a chain wave (the fp32 state slice in
//       registers, serial over pairs), an output wave (one pair behind: O
//       from the chain's bf16 state and U) and NL loader waves (direct-to-LDS
//       loads of the records and the slice's v into a ring, two pairs ahead).
//       The d_v slices of a head run on one XCD and share its L2: the
//       records come from HBM once per head.
#include "la_device.h"
#include "la_launch.h"

namespace la {
namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

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
__device__ inline void wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
template <int N>
__device__ inline void wait_vmcnt() {
  constexpr int n = N > 63 ? 63 : N;
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }
__device__ inline void wg_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
__device__ inline void lds_dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}

// Inclusive prefix sum over the 16 lanes of each row, and lane L of each row
// broadcast to the row (DPP row shifts / row_newbcast; no LDS traffic).
__device__ inline float row_scan16(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, false));
  return x;
}
template <int L>
__device__ inline float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + L, 0xf, 0xf, false));
}

// The record of one pair (bytes); every fragment field is 64 lanes x 16 B in
// lane order.  The workspace copy stops at VF; the v values of the slice are
// loaded per slice.
template <int DK>
struct CpRec {
  static constexpr int NT = DK / 16, NS = DK / 32;
  static constexpr int WF = 0;                      // W = Tb (K o Gam): [tile][NS] A fragments, bf16
  static constexpr int QF = WF + 2 * NS * 1024;     // Q o Gam: [tile][NS]
  static constexpr int KT = QF + 2 * NS * 1024;     // (K o Gam_31/Gam)^T: [NT], 32 tokens deep
  static constexpr int TB0 = KT + NT * 1024;        // [Tb00 hi | Tb00 lo]
  static constexpr int TB1H = TB0 + 1024;           // [Tb10 hi | Tb11 hi]
  static constexpr int TB1L = TB1H + 1024;          // [Tb10 lo | Tb11 lo]
  static constexpr int PF0 = TB1L + 1024;           // [P00 hi  | P00 lo]
  static constexpr int PF1H = PF0 + 1024;           // [P10 hi  | P11 hi]
  static constexpr int PF1L = PF1H + 1024;          // [P10 lo  | P11 lo]
  static constexpr int GC = PF1L + 1024;            // Gam_31[DK] f32
  static constexpr int GLOBAL = GC + DK * 4;        // bytes per pair in the workspace
  static constexpr int PIECES = (GLOBAL + 1023) / 1024;   // 1 KB direct-to-LDS loads of a record
  // [32 tokens][16 columns] bf16 (LDS only), after the padding that the last,
  // partial record piece fills
  static constexpr int VF = PIECES * 1024;
  static constexpr int LDS = VF + 1024;
  static constexpr int LOADS = PIECES + 1;          // loads per pair and wave
  static_assert(GLOBAL % 16 == 0, "alignment");
};

// ------------------------------------------------------------- prep kernel
constexpr int kCpWaves = 4;
// per wave: A00 (then T00), A11 (then T11), beta[32], the staged transposed
// blocks (K o Gam_31/Gam)^T and (K o Gam)^T (NT x 1 KB each) and Gam_31 (DK
// floats)
constexpr int kCpA0 = 0, kCpA1 = 1024, kCpB = 2048, kCpKt = 2176;
template <int DK>
struct CpPrep {
  static constexpr int KFT = kCpKt + (DK / 16) * 1024;
  static constexpr int GC = KFT + (DK / 16) * 1024;
  static constexpr int WAVE = GC + DK * 4;
  static constexpr int LDS = kCpWaves * WAVE;
};

__device__ inline int cp_seq_begin(const int* cu, int s, int TB) { return min(max(cu[s], 0), TB); }
__device__ inline int cp_seq_end(const int* cu, int s, int TB) {
  return min(max(cu[s + 1], cp_seq_begin(cu, s, TB)), TB);
}

// Arguments of one pass over tokens [0, T) of each sequence.  Batched (cu ==
// nullptr): B sequences whose token t is row (b TB + t) H + h of the arrays
// (the pointers may be advanced to a later token of every sequence; TB is the
// full sequence length), records [sequence, head, pair].  Packed: B = nseq
// sequences at device offsets cu in one sequence of T tokens, records at
// slot(s, p) = floor(cu[s] / 32) + s + p of nslot per head.
struct CpArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const float* gate;
  int gate_logit;
  float G;
  const float* beta;
  char* ws;
  const float* h0;
  __bf16* o;
  float* hT;
  int B, T, TB, H, DV;
  const int* cu;
  int nslot;
};

// Jobs first, first + step, ... of the (sequence, head, pair) records, one
// wave each, with scratch `scr` (CpPrep::WAVE bytes of LDS).  Batched: job =
// (b H + h) NPR + p.  Packed: job = h nslot + slot, the sequence found by
// binary search over the offsets (unused slots skipped).
template <int DK>
__device__ __forceinline__ void cp_prep_jobs(char* scr, int64_t first, int64_t step,
                                             const CpArgs& a) {
  using R = CpRec<DK>;
  using PL = CpPrep<DK>;
  using F = Elt<float>;
  constexpr int NS = R::NS, NT = R::NT;
  const __bf16* __restrict__ const q = a.q;
  const __bf16* __restrict__ const k = a.k;
  const float* __restrict__ const gate = a.gate;
  const float* __restrict__ const beta = a.beta;
  char* __restrict__ const ws = a.ws;
  const int* __restrict__ const cu = a.cu;
  const int gate_logit = a.gate_logit, B = a.B, T = a.T, H = a.H, nslot = a.nslot;
  const float G = a.G;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, grp = lane >> 4;
  float* sA0 = reinterpret_cast<float*>(scr + kCpA0);
  float* sA1 = reinterpret_cast<float*>(scr + kCpA1);
  float* sB = reinterpret_cast<float*>(scr + kCpB);
  char* kts = scr + kCpKt;
  char* kfts = scr + PL::KFT;
  float* sgc = reinterpret_cast<float*>(scr + PL::GC);
  const int NPR = (T + 31) >> 5;
  const int64_t jobs = cu ? (int64_t)H * nslot : (int64_t)B * H * NPR;
  // Job j's rows: token n of tile x (0: a, 1: b) is row[x] of the arrays, ok[x]
  // whether it lies inside the sequence (rows past the end read the last
  // valid row and are zeroed); returns the first job at or after j that has
  // a pair (jobs if none).
  auto find = [&](int64_t j, bool* ok, int64_t* row) -> int64_t {
    for (; j < jobs; j += step) {
      int c, h, Ts;
      int64_t tok0;
      if (cu) {
        h = (int)(j / nslot);
        const int slot = (int)(j - (int64_t)h * nslot);
        int lo = 0, hi = B - 1;                  // the last s with slot(s, 0) <= slot
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (cp_seq_begin(cu, mid, T) / 32 + mid <= slot) lo = mid;
          else hi = mid - 1;
        }
        const int tb = cp_seq_begin(cu, lo, T);
        Ts = cp_seq_end(cu, lo, T) - tb;
        c = slot - (tb / 32 + lo);
        if (c < 0 || c >= ((Ts + 31) >> 5)) continue;   // a slot no pair uses
        tok0 = tb;
      } else {
        c = (int)(j % NPR);
        const int64_t bh = j / NPR;
        h = (int)(bh % H);
        tok0 = (bh / H) * (int64_t)a.TB;
        Ts = T;
      }
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        ok[x] = 32 * c + 16 * x + n < Ts;
        row[x] = (tok0 + min(32 * c + 16 * x + n, Ts - 1)) * H + h;
      }
      return j;
    }
    return jobs;
  };
  // One 32-deep channel block s of a job's k, q and gate: lane (n, grp)
  // register j is channel 32 s + 16 (j >> 2) + 4 grp + (j & 3) of token n of
  // each tile.
  struct Raw { bf16x4 k0, k1, q0, q1; f32x4 g0, g1; };
  auto load_block = [&](int s, const int64_t* row, Raw* r) {
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int64_t base = row[x] * DK + 32 * s + 4 * grp;
      r[x].k0 = *reinterpret_cast<const bf16x4*>(k + base);
      r[x].k1 = *reinterpret_cast<const bf16x4*>(k + base + 16);
      r[x].q0 = *reinterpret_cast<const bf16x4*>(q + base);
      r[x].q1 = *reinterpret_cast<const bf16x4*>(q + base + 16);
      r[x].g0 = *reinterpret_cast<const f32x4*>(gate + base);
      r[x].g1 = *reinterpret_cast<const f32x4*>(gate + base + 16);
    }
  };
  // The loads of block s + 1 are issued before block s is worked on, so
  // that a job waits for memory about once rather than once per block.
  bool ok[2];
  int64_t row[2];
  for (int64_t job = find(first, ok, row); job < jobs; job = find(job + step, ok, row)) {
    char* wr = ws + job * R::GLOBAL;
    const float ba = ok[0] ? beta[row[0]] : 0.f, bb = ok[1] ? beta[row[1]] : 0.f;
    if (grp == 0) {
      sB[n] = ba;
      sB[16 + n] = bb;
    }
    f32x4 s00 = zero4(), s11 = zero4(), s10 = zero4();
    f32x4 p00 = zero4(), p11 = zero4(), p10 = zero4();
    Raw raw[NS][2];
    load_block(0, row, raw[0]);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s + 1 < NS) load_block(s + 1, row, raw[s + 1]);
      float kv[2][8], qv[2][8], gv[2][8];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const bf16x4 k0 = raw[s][x].k0, k1 = raw[s][x].k1, q0 = raw[s][x].q0, q1 = raw[s][x].q1;
        const f32x4 g0 = raw[s][x].g0, g1 = raw[s][x].g1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kv[x][j] = ok[x] ? (float)k0[j] : 0.f;
          kv[x][4 + j] = ok[x] ? (float)k1[j] : 0.f;
          qv[x][j] = ok[x] ? (float)q0[j] : 0.f;
          qv[x][4 + j] = ok[x] ? (float)q1[j] : 0.f;
          // log mode: clamped to [-G, 0], so that the in-tile factors stay
          // within exp(+-8 G) whatever the caller passes
          const float x0 = g0[j], x1 = g1[j];
          gv[x][j] = ok[x] ? (gate_logit ? bounded_gate(x0, G) : fminf(fmaxf(x0, -G), 0.f)) : 0.f;
          gv[x][4 + j] = ok[x] ? (gate_logit ? bounded_gate(x1, G) : fminf(fmaxf(x1, -G), 0.f)) : 0.f;
        }
      }
      F::F32 kia, kma, qma, kib, kmb, qmb, kxa, kxb, qxb;
      bf16x8 kfa, kfb, qfa, qfb;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float Ga = row_scan16(gv[0][j]);          // running sum, tile a token n
        const float Ga15 = row_bcast<15>(Ga);
        const float Gam = row_bcast<7>(Ga);
        const float Gb = Ga15 + row_scan16(gv[1][j]);   // running sum over the pair, token 16 + n
        const float Gb31 = row_bcast<15>(Gb);
        const float Gbm = row_bcast<7>(Gb);
        const float ka = kv[0][j], kb = kv[1][j], qa = qv[0][j], qb = qv[1][j];
        // state-facing operands (at most 1)
        const float ea = __expf(Ga), eb = __expf(Gb);
        kfa[j] = (__bf16)(ka * ea);
        kfb[j] = (__bf16)(kb * eb);
        qfa[j] = (__bf16)(qa * ea);
        qfb[j] = (__bf16)(qb * eb);
        const int ch = 32 * s + 16 * (j >> 2) + 4 * grp + (j & 3);
        // (K o Gam_31/Gam)^T in the chain's A-fragment order: state tile
        // ch / 16, lane (ch % 16, n / 4), register n % 4 (tile a) or 4 + n % 4
        // (tile b)
        const int kl = (ch >> 4) * 64 + (n >> 2) * 16 + (ch & 15);
        reinterpret_cast<__bf16*>(kts)[kl * 8 + (n & 3)] = (__bf16)(ka * __expf(Gb31 - Ga));
        reinterpret_cast<__bf16*>(kts)[kl * 8 + 4 + (n & 3)] = (__bf16)(kb * __expf(Gb31 - Gb));
        // (K o Gam)^T in the same order, the A side of W^T = (K o Gam)^T Tb^T
        reinterpret_cast<__bf16*>(kfts)[kl * 8 + (n & 3)] = kfa[j];
        reinterpret_cast<__bf16*>(kfts)[kl * 8 + 4 + (n & 3)] = kfb[j];
        if (n == 0) sgc[ch] = __expf(Gb31);
        // diagonal blocks: factors about the tile's middle token
        const float ema = __expf(Ga - Gam), emb = __expf(Gb - Gbm);
        const float ima = __expf(Gam - Ga), imb = __expf(Gbm - Gb);
        // cross block: factors about the boundary token 15 (both <= 1)
        const float exa = __expf(Ga15 - Ga), exb = __expf(Gb - Ga15);
        if (j < 4) {
          kia.lo[j] = ka * ima; kma.lo[j] = ka * ema; qma.lo[j] = qa * ema;
          kib.lo[j] = kb * imb; kmb.lo[j] = kb * emb; qmb.lo[j] = qb * emb;
          kxa.lo[j] = ka * exa; kxb.lo[j] = kb * exb; qxb.lo[j] = qb * exb;
        } else {
          kia.hi[j - 4] = ka * ima; kma.hi[j - 4] = ka * ema; qma.hi[j - 4] = qa * ema;
          kib.hi[j - 4] = kb * imb; kmb.hi[j - 4] = kb * emb; qmb.hi[j - 4] = qb * emb;
          kxa.hi[j - 4] = ka * exa; kxb.hi[j - 4] = kb * exb; qxb.hi[j - 4] = qb * exb;
        }
      }
      reinterpret_cast<bf16x8*>(wr + R::QF)[(0 * NS + s) * 64 + lane] = qfa;
      reinterpret_cast<bf16x8*>(wr + R::QF)[(1 * NS + s) * 64 + lane] = qfb;
      // lane (n, grp) reg i of each product: block entry [n][4 grp + i]
      // (row n of A before beta, or of P; A_op rows are the column tokens)
      s00 = F::mma32(kia, kma, s00);
      p00 = F::mma32(kia, qma, p00);
      s11 = F::mma32(kib, kmb, s11);
      p11 = F::mma32(kib, qmb, p11);
      s10 = F::mma32(kxa, kxb, s10);
      p10 = F::mma32(kxa, qxb, p10);
    }
    f32x4 a00, a11, a10, pp00, pp11, pp10;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int sc = 4 * grp + i;
      a00[i] = sc < n ? ba * s00[i] : 0.f;
      a11[i] = sc < n ? bb * s11[i] : 0.f;
      a10[i] = bb * s10[i];
      pp00[i] = sc <= n ? p00[i] : 0.f;
      pp11[i] = sc <= n ? p11[i] : 0.f;
      pp10[i] = p10[i];
    }
    reinterpret_cast<f32x4*>(sA0)[n * 4 + grp] = a00;
    reinterpret_cast<f32x4*>(sA1)[n * 4 + grp] = a11;
    {
      const bf16x4 h00 = hi4(pp00), h10 = hi4(pp10), h11 = hi4(pp11);
      reinterpret_cast<bf16x8*>(wr + R::PF0)[lane] = cat8(h00, lo4(pp00, h00));
      reinterpret_cast<bf16x8*>(wr + R::PF1H)[lane] = cat8(h10, h11);
      reinterpret_cast<bf16x8*>(wr + R::PF1L)[lane] = cat8(lo4(pp10, h10), lo4(pp11, h11));
    }
    wave_fence();   // A, beta, the staged key block and Gam_31 written
#pragma unroll
    for (int t = 0; t < NT; ++t)
      reinterpret_cast<f32x4*>(wr + R::KT)[t * 64 + lane] =
          reinterpret_cast<const f32x4*>(kts)[t * 64 + lane];
    if (lane < DK / 4)
      reinterpret_cast<f32x4*>(wr + R::GC)[lane] = reinterpret_cast<const f32x4*>(sgc)[lane];

    // T00 (lane groups 0, 1) and T11 (groups 2, 3), row n per lane:
    // T[n][s] = delta_ns - sum_{r > s} T[n][r] A[r][s], from the bottom row up.
    {
      f32x4* Ab = reinterpret_cast<f32x4*>(grp < 2 ? sA0 : sA1);
      float xr_[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) xr_[s] = 0.f;
#pragma unroll
      for (int rr = 15; rr >= 1; --rr) {
        f32x4 arow[4];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) arow[c4] = Ab[rr * 4 + c4];
        const float xr = (rr == n) ? 1.f : xr_[rr];
#pragma unroll
        for (int s = 0; s < rr; ++s) xr_[s] -= xr * arow[s >> 2][s & 3];
      }
      wave_fence();   // every lane has read all rows of A before T overwrites it
      if ((grp & 1) == 0) {
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          f32x4 r4;
#pragma unroll
          for (int e = 0; e < 4; ++e) r4[e] = (4 * c4 + e == n) ? 1.f : xr_[4 * c4 + e];
          Ab[n * 4 + c4] = r4;
        }
      }
    }
    wave_fence();
    // M = A10 T00 (A10 rows in registers, T00 columns), then (T11 M)^T: lane
    // (n, grp) reg i of TM is (T11 M)[n][4 grp + i] = -T10[n][4 grp + i].
    f32x4 t00c;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) t00c[jj] = sA0[(4 * grp + jj) * 16 + n];
    const f32x4 M = F::mma16(F::F16{a10}, F::F16{t00c}, zero4());
    const f32x4 t11r = reinterpret_cast<const f32x4*>(sA1)[n * 4 + grp];
    const f32x4 TM = F::mma16(F::F16{M}, F::F16{t11r}, zero4());
    const f32x4 t00r = reinterpret_cast<const f32x4*>(sA0)[n * 4 + grp];
    const f32x4 bea = reinterpret_cast<const f32x4*>(sB)[grp];
    const f32x4 beb = reinterpret_cast<const f32x4*>(sB)[4 + grp];
    f32x4 tb00, tb10, tb11;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tb00[i] = t00r[i] * bea[i];
      tb10[i] = -TM[i] * bea[i];
      tb11[i] = t11r[i] * beb[i];
    }
    const bf16x4 h00 = hi4(tb00), h10 = hi4(tb10), h11 = hi4(tb11);
    const bf16x4 l00 = lo4(tb00, h00), l10 = lo4(tb10, h10), l11 = lo4(tb11, h11);
    reinterpret_cast<bf16x8*>(wr + R::TB0)[lane] = cat8(h00, l00);
    reinterpret_cast<bf16x8*>(wr + R::TB1H)[lane] = cat8(h10, h11);
    reinterpret_cast<bf16x8*>(wr + R::TB1L)[lane] = cat8(l10, l11);
    // W = Tb (K o Gam) in the chain's A-fragment order, as W^T = (K o Gam)^T
    // Tb^T over the pair's 32 tokens: the A side is the staged (K o Gam)^T of
    // a 16-channel tile, the B side row n of Tb in hi and lo parts (the rows
    // of tile a have no tile-b columns); lane (n, grp) register i of tile x
    // ends with W[n][16 x + 4 grp + i].
    {
      const bf16x4 z4 = {};
      const bf16x8 bah = cat8(h00, z4), bal = cat8(l00, z4);
      const bf16x8 bbh = cat8(h10, h11), bbl = cat8(l10, l11);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        f32x4 da[2], db[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bf16x8 a = reinterpret_cast<const bf16x8*>(kfts)[(2 * s + u) * 64 + lane];
          da[u] = mma32b(a, bal, mma32b(a, bah, zero4()));
          db[u] = mma32b(a, bbl, mma32b(a, bbh, zero4()));
        }
        reinterpret_cast<bf16x8*>(wr + R::WF)[s * 64 + lane] = cat8(hi4(da[0]), hi4(da[1]));
        reinterpret_cast<bf16x8*>(wr + R::WF)[(NS + s) * 64 + lane] = cat8(hi4(db[0]), hi4(db[1]));
      }
    }
    wave_fence();   // the next job's writes to this wave's scratch must not pass these reads
  }
}

template <int DK>
__global__ __launch_bounds__(64 * kCpWaves) void chunk_channel_prep_pair_kernel(CpArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[CpPrep<DK>::LDS];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  cp_prep_jobs<DK>(smem + wave * CpPrep<DK>::WAVE, (int64_t)blockIdx.x * kCpWaves + wave,
                   (int64_t)gridDim.x * kCpWaves, a);
}

// ------------------------------------------------------------ state kernel
// Waves: chain 0, output 1, loaders 2 .. NL + 1.  A wave's direct-to-LDS
// loads move about 8 bytes per cycle however many are in flight, so the 32 KB
// of a pair's records are split over NL loader waves, PL loads each (a loader
// whose share is short repeats the pair's last load, so that every loader
// issues the same count).
template <int DK, int NL>
struct CpCfg {
  using R = CpRec<DK>;
  static constexpr int WAVES = NL + 2;
  static constexpr int PL = (R::LOADS + NL - 1) / NL;      // loads per pair and loader wave
  static constexpr int NT = DK / 16, NS = DK / 32;
  // chain -> output hand-over, double buffered by pair parity: the bf16 state
  // the pair started from, and U_a, U_b (f32)
  static constexpr int OB_H = 0;
  static constexpr int OB_U = NS * 1024;
  static constexpr int OB = OB_U + 2048;
  static constexpr int OFF_REC = 2 * OB;
  static constexpr int NBUF = (160 * 1024 - OFF_REC - 256) / R::LDS < 6
                                  ? (160 * 1024 - OFF_REC - 256) / R::LDS : 6;
  static constexpr int OFF_PF = OFF_REC + NBUF * R::LDS;   // landing slot of the L2 prefetch
  static constexpr int PF_AHEAD = 8;                       // pairs the L2 prefetch runs ahead
  static constexpr int LDS = OFF_PF + 256;
  static_assert(NBUF >= 4, "ring of at least four records");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert((NBUF - 3) * (PL + 1) <= 63, "vmcnt range");
};

__device__ inline void cp_map_block(int n, int NH, int NV, int& head, int& vt) {
  // block n serves head 8 a + n % 8: the d_v slices of a head share one XCD
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

template <int DK, int NL, bool ROT>
__device__ __forceinline__ void cp_state_body(char* smem, int blk, const CpArgs& a) {
  using R = CpRec<DK>;
  using C = CpCfg<DK, NL>;
  constexpr int NT = C::NT, NS = C::NS, NBUF = C::NBUF;
  const __bf16* __restrict__ const v = a.v;
  const char* __restrict__ const ws = a.ws;
  const float* const h0 = a.h0;
  __bf16* __restrict__ const o = a.o;
  float* const hT = a.hT;
  const int* __restrict__ const cu = a.cu;
  const int B = a.B, TA = a.T, H = a.H, DV = a.DV, nslot = a.nslot;
  const int NV = DV / 16;
  int head, vt;
  cp_map_block(blk, B * H, NV, head, vt);
  const int b = head / H, h = head % H;
  const int v0 = vt * 16;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, grp = lane >> 4;
  int T;
  int64_t tok0;             // token 0 of the sequence on the token axis
  const char* wsh;          // record of pair 0
  if (cu) {
    const int tb = cp_seq_begin(cu, b, TA);
    T = cp_seq_end(cu, b, TA) - tb;
    tok0 = tb;
    wsh = ws + ((int64_t)h * nslot + tb / 32 + b) * R::GLOBAL;
  } else {
    T = TA;
    tok0 = (int64_t)b * a.TB;
    wsh = ws + (int64_t)head * ((TA + 31) >> 5) * R::GLOBAL;
  }
  const int NPR = (T + 31) >> 5;
  const int64_t sbase = ((int64_t)b * H + h) * DK * DV;
  if (NPR == 0) {
    // an empty packed sequence: hT = h0 (zeros without h0), by the chain wave
    if (wave == 0 && hT) {
      for (int r = 0; r < DK; r += 4)
        hT[sbase + (int64_t)(r + grp) * DV + v0 + n] =
            h0 ? h0[sbase + (int64_t)(r + grp) * DV + v0 + n] : 0.f;
    }
    return;
  }
  auto rec_of = [&](int c) -> char* {
    int rb = __builtin_amdgcn_readfirstlane(C::OFF_REC + (c % NBUF) * R::LDS);
    asm volatile("" : "+s"(rb));
    return smem + rb;
  };
  // Barriers: one before pair 0, one after each pair c = 0 .. NPR-1 and one
  // more that lets the output wave finish the last pair: NPR + 2 in all,
  // executed by every wave.

  if (wave >= 2) {
    // ----------------------------------------------------------- loaders
    // Ring of NBUF records; pair c lives in record c % NBUF.  During pair c
    // the chain reads record c and the output wave record c - 1, so the
    // record of pair c - 2 is free for pair c + NBUF - 2; pair c + 1 must have
    // landed by the barrier that ends pair c.  Loader l moves the 1 KB pieces
    // l, l + NL, ... of each pair (piece PIECES is the slice's v), starting
    // at a different one in each d_v slice so that the slices of a head do
    // not ask the same L2 lines at once.  Pair indices are clamped so that
    // every load is valid and the load count never varies.
    const int l = wave - 2;
    const int m0 = ROT ? vt % C::PL : 0;
    // L2 prefetch: one 4-byte load per 128-byte line of the record PF_AHEAD
    // pairs ahead, the lines split over the NV slices and NL loaders of the
    // head (the slices run on one XCD and share its L2), so that the loads
    // into LDS hit L2 instead of waiting for HBM.
    constexpr int nlines = (R::GLOBAL + 127) / 128;
    const int pf_line = min(vt * NL + l + NV * NL * lane, nlines - 1);
    lds_void* const junk = (lds_void*)(smem + C::OFF_PF);
    auto issue = [&](int c) {
      __builtin_amdgcn_global_load_lds(wsh + (int64_t)min(c + C::PF_AHEAD, NPR - 1) * R::GLOBAL + pf_line * 128,
                                       junk, 4, 0, 0);
      c = min(c, NPR - 1);
      char* rec = rec_of(c);
      const char* src = wsh + (int64_t)c * R::GLOBAL;
#pragma unroll
      for (int mm = 0; mm < C::PL; ++mm) {
        int m = mm + m0;
        m = m >= C::PL ? m - C::PL : m;
        const int i = min(l + NL * m, R::LOADS - 1);
        if (i < R::PIECES) {
          // the last record piece may be partial: its lanes past the end
          // re-read the record's last 16 bytes into the slot's padding
          const int off = min(1024 * i + 16 * lane, R::GLOBAL - 16);
          lds_dma16(src + off, rec + 1024 * i);
        } else {
          // v of the slice: lane L fetches 8 columns (half L % 2) of token L / 2
          const int t = min(32 * c + (lane >> 1), T - 1);
          lds_dma16(v + ((tok0 + t) * H + h) * DV + v0 + 8 * (lane & 1), rec + R::VF);
        }
      }
    };
    // Loads complete in order, so with kAhead loads allowed in flight every
    // pair but the NBUF - 3 issued last has landed.
    constexpr int kAhead = (NBUF - 3) * (C::PL + 1);
#pragma unroll 1
    for (int c = 0; c < NBUF - 2; ++c) issue(c);
    wait_vmcnt<kAhead>();                          // pair 0 landed
    wg_barrier();
#pragma unroll 1
    for (int c = 0; c <= NPR; ++c) {
      issue(c + NBUF - 2);                         // into the record of pair c - 2
      wait_vmcnt<kAhead>();                        // pair c + 1 landed
      wg_barrier();
    }
    wait_vmcnt<0>();
    return;
  }

  if (wave == 0) {
    // ------------------------------------------------------------ chain wave
    f32x4 Hacc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Hacc[t][i] = h0 ? h0[sbase + (int64_t)(16 * t + 4 * grp + i) * DV + v0 + n] : 0.f;
    }
    bf16x8 Hb[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) Hb[s] = cat8(hi4(Hacc[2 * s]), hi4(Hacc[2 * s + 1]));
    const int o_v = R::VF + 8 * lane;               // V, transposing read
    // With W = Tb (K o Gam), U = Tb V - W H: Tb V does not depend on the
    // state, and W H of pair c + 1 is formed 32 state rows at a time as the
    // update of pair c produces them.  TV and WH hold Tb V and W H of the
    // pair that comes next, kt and gc the operands of its state update
    // (read one pair ahead, so that the update never waits for LDS).
    f32x4 TVa, TVb, WHa, WHb;
    bf16x8 kt[NT];
    f32x4 gc[NT];
    auto next_pair = [&](const char* rec, char* ob, auto&& update) {
      // phase 0: the pair's reads, in the order they are needed
      // V in accumulator layout: lane (n, grp) receives V[4 grp + r][n]
      const bf16x4 va = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(rec + o_v)));
      const bf16x4 vb = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(rec + o_v + 512)));
      const bf16x8 tb0 = reinterpret_cast<const bf16x8*>(rec + R::TB0)[lane];
      const bf16x8 tb1h = reinterpret_cast<const bf16x8*>(rec + R::TB1H)[lane];
      const bf16x8 tb1l = reinterpret_cast<const bf16x8*>(rec + R::TB1L)[lane];
      bf16x8 wf[2 * NS];
#pragma unroll
      for (int s = 0; s < 2 * NS; ++s) wf[s] = reinterpret_cast<const bf16x8*>(rec + R::WF)[s * 64 + lane];
      __builtin_amdgcn_sched_barrier(0);
      // phase 1: the update of state tiles 0 .. 3 (operands in registers)
      update(0);
      update(1);
      __builtin_amdgcn_sched_barrier(0);
      WHa = zero4();
      WHb = zero4();
      // phases 2 .. NS + 1: rows 32 s .. 32 s + 31 of the new state to the
      // output wave and into W H, the update of tiles 2 s + 4, 2 s + 5, Tb V
      // once its operands are in, and the reads of the update operands of the
      // pair (a tile's registers are free once it is updated)
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        Hb[s] = cat8(hi4(Hacc[2 * s]), hi4(Hacc[2 * s + 1]));
        *reinterpret_cast<bf16x8*>(ob + C::OB_H + s * 1024) = Hb[s];
        WHa = mma32b(wf[s], Hb[s], WHa);
        WHb = mma32b(wf[NS + s], Hb[s], WHb);
        if (s + 2 < NS) update(s + 2);
        if (s == 1) {
          // Tb V (Tb in hi + lo parts, V exact)
          TVa = mma32b(tb0, cat8(va, va), zero4());
          TVb = mma32b(tb1h, cat8(va, vb), zero4());
          TVb = mma32b(tb1l, cat8(va, vb), TVb);
        }
        // tiles 0 .. 2 s + 5 are updated by now: read tiles 4 s .. 4 s + 3
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int t = 4 * s + u;
          if (t < NT) {
            kt[t] = reinterpret_cast<const bf16x8*>(rec + R::KT)[t * 64 + lane];
            gc[t] = *reinterpret_cast<const f32x4*>(rec + R::GC + (16 * t + 4 * grp) * 4);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    wg_barrier();                                   // pair 0 landed
    next_pair(rec_of(0), smem + 16 * lane, [&](int) {});
#pragma unroll 1
    for (int c = 0; c < NPR; ++c) {
      char* ob = smem + (c & 1) * C::OB + 16 * lane;
      const f32x4 Ua = TVa - WHa, Ub = TVb - WHb;
      *reinterpret_cast<f32x4*>(ob + C::OB_U) = Ua;
      *reinterpret_cast<f32x4*>(ob + C::OB_U + 1024) = Ub;
      const bf16x8 ub = cat8(hi4(Ua), hi4(Ub));
      // End of the pair for the other waves once U is handed over: the
      // record of pair c stays in place until the barrier that ends pair
      // c + 1, and that of pair c + 1 has landed at this one.
      wait_lgkm0();
      __builtin_amdgcn_sched_barrier(0);
      wg_barrier();
      // H' = diag(Gam_31) H + (K o Gam_31/Gam)^T U, 32 tokens deep, with W H
      // and Tb V of pair c + 1 alongside
      next_pair(rec_of(min(c + 1, NPR - 1)), smem + ((c + 1) & 1) * C::OB + 16 * lane, [&](int s) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int t = 2 * s + u;
#pragma unroll
          for (int i = 0; i < 4; ++i) Hacc[t][i] *= gc[t][i];   // row 16t + 4grp + i
          Hacc[t] = mma32b(kt[t], ub, Hacc[t]);
        }
      });
    }
    wg_barrier();                  // the output wave's last pair
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

  // -------------------------------------------------------------- output wave
  // Pair c after the barrier that ends the chain's pair c:
  //   O_a^T = H^T (Q_a o Gam)^T + U_a^T P00^T
  //   O_b^T = H^T (Q_b o Gam)^T + U_a^T P10^T + U_b^T P11^T
  // formed transposed so that lane (n, grp) ends with columns 4 grp .. 4 grp
  // + 3 of token n (one 8-byte store per tile).
  {
    __bf16* const orow = o + ((tok0 + n) * H + h) * DV + v0 + 4 * grp;
    const int64_t ostride = (int64_t)H * DV;
    wg_barrier();    // before pair 0
    wg_barrier();    // after the chain's pair 0
#pragma unroll 1
    for (int c = 0; c < NPR; ++c) {
      const char* rec = rec_of(c);
      const char* ob = smem + (c & 1) * C::OB + 16 * lane;
      f32x4 Oa = zero4(), Ob = zero4();
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 hb = *reinterpret_cast<const bf16x8*>(ob + C::OB_H + s * 1024);
        Oa = mma32b(hb, reinterpret_cast<const bf16x8*>(rec + R::QF)[s * 64 + lane], Oa);
        Ob = mma32b(hb, reinterpret_cast<const bf16x8*>(rec + R::QF)[(NS + s) * 64 + lane], Ob);
      }
      const f32x4 Ua = *reinterpret_cast<const f32x4*>(ob + C::OB_U);
      const f32x4 Ub = *reinterpret_cast<const f32x4*>(ob + C::OB_U + 1024);
      const bf16x8 pf0 = reinterpret_cast<const bf16x8*>(rec + R::PF0)[lane];
      const bf16x8 pf1h = reinterpret_cast<const bf16x8*>(rec + R::PF1H)[lane];
      const bf16x8 pf1l = reinterpret_cast<const bf16x8*>(rec + R::PF1L)[lane];
      wait_lgkm0();   // hand-over read: the chain may overwrite it after the next barrier
      const bf16x4 uah = hi4(Ua), ubh = hi4(Ub);
      const bf16x4 ual = lo4(Ua, uah), ubl = lo4(Ub, ubh);
      // O_a += P00 U_a ; O_b += P10 U_a + P11 U_b  (P and U in hi + lo parts)
      Oa = mma32b(cat8(uah, uah), pf0, Oa);
      Oa = mma32b(cat8(ual, bf16x4{}), pf0, Oa);
      Ob = mma32b(cat8(uah, ubh), pf1h, Ob);
      Ob = mma32b(cat8(uah, ubh), pf1l, Ob);
      Ob = mma32b(cat8(ual, ubl), pf1h, Ob);
      __bf16* oc = orow + (int64_t)(32 * c) * ostride;
      if (32 * c + n < T) *reinterpret_cast<bf16x4*>(oc) = hi4(Oa);
      if (32 * c + 16 + n < T) *reinterpret_cast<bf16x4*>(oc + 16 * ostride) = hi4(Ob);
      wg_barrier();
    }
  }
}

// Blocks [0, nstate) carry the state over one stretch of the sequences (a
// d_v slice each); any blocks after them prepare the records of the next
// stretch (every wave a job at a time) on the compute units the state blocks
// leave idle.  The two share no data within a launch.
template <int DK, int NL, bool ROT>
__global__ __launch_bounds__(64 * (NL + 2)) void chunk_fwd_channel_pair_kernel(
    CpArgs sa, CpArgs pa, int nstate) {
  using C = CpCfg<DK, NL>;
  static_assert(C::WAVES * CpPrep<DK>::WAVE <= C::LDS, "the prep blocks use the same LDS");
  __shared__ __attribute__((aligned(256))) char smem[C::LDS];
  if ((int)blockIdx.x < nstate) {
    cp_state_body<DK, NL, ROT>(smem, blockIdx.x, sa);
  } else {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    cp_prep_jobs<DK>(smem + wave * CpPrep<DK>::WAVE,
                     (int64_t)((int)blockIdx.x - nstate) * C::WAVES + wave,
                     (int64_t)((int)gridDim.x - nstate) * C::WAVES, pa);
  }
}

// Long batched sequences are cut into stretches of whole pairs: the records
// of stretch 0 are prepared alone, then launch s carries the state over
// stretch s while its extra blocks prepare stretch s + 1.  The fp32 state
// passes from one stretch to the next through the workspace (read and
// written in place by the workgroup that owns each slice), so the results are
// those of one pass.  Sequences of kCpStretchPairs pairs or more may be cut
// (the workspace then holds the carried state); stretches have at least
// kCpMinStretchPairs pairs, and there are at most kCpMaxStretches.
constexpr int kCpStretchPairs = 512;
constexpr int kCpMinStretchPairs = 128;
constexpr int kCpMaxStretches = 16;

template <int DK>
hipError_t launch_cp_t(const void* q, const void* k, const void* v, const float* gate,
                       int gate_logit, float G, const float* beta, const float* h0, void* o,
                       float* hT, int B, int T, int H, int Dv, const int* cu, void* ws,
                       hipStream_t st) {
  // four loader waves, each moving about 8 bytes per cycle into LDS (six
  // measured no faster: the chain sets the pace)
  constexpr int NL = 4;
  using C = CpCfg<DK, NL>;
  const int NPR = (T + 31) / 32;
  const int nslot = T / 32 + B + 1;
  const int nstate = B * H * (Dv / 16);
  const int cus = device_cus();
  int S = 1;
  if (!cu && NPR >= kCpStretchPairs && 2 * nstate <= cus)
    S = min(kCpMaxStretches, NPR / kCpMinStretchPairs);
  char* const wsb = static_cast<char*>(ws);
  float* const carry = reinterpret_cast<float*>(wsb + (int64_t)B * H * NPR * CpRec<DK>::GLOBAL);
  auto stretch = [&](int s) {
    const int p0 = (int)((int64_t)NPR * s / S), p1 = (int)((int64_t)NPR * (s + 1) / S);
    const int64_t t0 = cu ? 0 : 32 * (int64_t)p0;
    const int Ts = cu ? T : min(32 * p1, T) - 32 * p0;
    CpArgs a{(const __bf16*)q + t0 * H * DK, (const __bf16*)k + t0 * H * DK,
             (const __bf16*)v + t0 * H * Dv, gate + t0 * H * DK, gate_logit, G, beta + t0 * H,
             wsb + (int64_t)B * H * p0 * CpRec<DK>::GLOBAL, s == 0 ? h0 : carry,
             (__bf16*)o + t0 * H * Dv, s == S - 1 ? hT : carry, B, Ts, T, H, Dv, cu, nslot};
    return a;
  };
  auto jobs = [&](const CpArgs& a) {
    return cu ? (int64_t)H * nslot : (int64_t)B * H * ((a.T + 31) / 32);
  };
  {
    const CpArgs a = stretch(0);
    const int64_t pb = (jobs(a) + kCpWaves - 1) / kCpWaves;
    const int prep_blocks = (int)(pb < 4096 ? pb : 4096);
    if (prep_blocks > 0) {
      hipLaunchKernelGGL((chunk_channel_prep_pair_kernel<DK>), dim3(prep_blocks),
                         dim3(64 * kCpWaves), 0, st, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  for (int s = 0; s < S; ++s) {
    const CpArgs sa = stretch(s);
    CpArgs pa{};
    int resident = 0;
    if (s + 1 < S) {
      pa = stretch(s + 1);
      const int64_t need = (jobs(pa) + C::WAVES - 1) / C::WAVES;
      resident = (int)min((int64_t)(cus - nstate), need);
      if (resident < 1) resident = 1;
    }
    hipLaunchKernelGGL((chunk_fwd_channel_pair_kernel<DK, NL, true>), dim3(nstate + resident),
                       dim3(64 * C::WAVES), 0, st, sa, pa, nstate);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

static long long cp_record_bytes(int Dk) {
  return Dk == 64 ? CpRec<64>::GLOBAL : CpRec<128>::GLOBAL;
}

long long chunk_channel_pair_workspace_bytes(int B, int T, int H, int Dk, int Dv) {
  const long long npr = (T + 31) / 32;
  long long n = (long long)B * H * npr * cp_record_bytes(Dk);
  if (npr >= kCpStretchPairs) n += (long long)B * H * Dk * Dv * 4;   // the carried state
  return n;
}

long long chunk_channel_pair_varlen_workspace_bytes(int T, int nseq, int H, int Dk) {
  return (long long)H * (T / 32 + nseq + 1) * cp_record_bytes(Dk);
}

hipError_t launch_chunk_fwd_channel_pair(const void* q, const void* k, const void* v,
                                         const float* gate, int gate_logit, float G,
                                         const float* beta, const float* h0, void* o, float* hT,
                                         int B, int T, int H, int Dk, int Dv, const int* cu,
                                         void* ws, hipStream_t st) {
  if (Dk == 64) return launch_cp_t<64>(q, k, v, gate, gate_logit, G, beta, h0, o, hT, B, T, H, Dv, cu, ws, st);
  if (Dk == 128) return launch_cp_t<128>(q, k, v, gate, gate_logit, G, beta, h0, o, hT, B, T, H, Dv, cu, ws, st);
  return hipErrorInvalidValue;
}

}  // namespace la
